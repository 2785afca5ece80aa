// CoWindow Attention backward, bf16, head dim 128, for gfx950.
//
// Gradients of the same masked softmax attention the forward computes (the pages state
// that the pattern supports training forward and backward — beyondmarketintelligence.com
// post, second paragraph; "CoWindow Attention" abstract), recomputed from the saved
// logsumexp:
//   P = exp(scale q.k - LSE), Delta_i = dO_i . O_i, dP = dO V^T, dS = P (dP - Delta)
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO
// Three kernels, no atomics (deterministic):
//   delta  : Delta per (row, query head), and an fp16 copy of Q scaled per row by a
//            power of two;
//   dq     : one work item per (KV head, q-block of 128 / G tokens), walking the row list
//            of visible 128-key blocks: S^T, dP^T, dS^T on MFMA, dQ^T += K^T dS^T with
//            K^T read by ds_read_b64_tr_b16 from the row-major LDS tile;
//   dkdv   : one work item per (KV head, 128-key block), walking the column list of
//            visible q-blocks; each of the 4 waves keeps 32 keys of K and V in registers
//            and accumulates dK, dV for them over all G query heads of the KV head:
//            S = Q K^T and dP = dO V^T on MFMA, then dV += P^T dO and dK += dS^T Q with
//            P (bf16) and dS (fp16) packed from the accumulator registers as A operands
//            and dO, Q read transposed from LDS; Q, K and dS enter the S and dK products
//            in fp16 (exact power-of-two scalings undone through per-row constants).
// Rows of a q-block are token-major (row r = token * G + head-in-group); rows beyond
// G * Bq or Lq carry LSE = +inf and Delta = 0 so that they contribute nothing.

#include <type_traits>

#include "cowa.h"
#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 128;
constexpr int ROWS = kBwdRows;  // 128 query rows per q-block
constexpr int BK = kBwdBk;      // 128 keys per k-block

// Returns x unchanged, but the value is taken at this point of the program: computations
// that use the result cannot be hoisted above it (it pins VALU work to its pipeline slot).
__device__ __forceinline__ float pin(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void pin_out(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_out(float& x) { asm volatile("" : "+v"(x)); }

// ------------------------------------------------------------------------ Delta
// Per row (token, query head): Delta = dO . O, and the fp16 copy of q that the dK
// product reads, q / 2^e with max |q| / 2^e in [1, 2) (2^e stored beside Delta).  Sixteen
// lanes per row, 8 elements each.
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, t, hq) flat
  const int li = threadIdx.x & 15;
  const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
  float acc = 0.f, qm = 0.f;
  u32x4 qw = {0u, 0u, 0u, 0u};
  if (row < nrows) {
    const u32x4 ow = *(const u32x4*)((const __bf16*)a.o + row * D + 8 * li);
    const u32x4 dw = *(const u32x4*)((const __bf16*)a.dout + row * D + 8 * li);
    qw = *(const u32x4*)((const __bf16*)a.q + row * D + 8 * li);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(ow[k] << 16), __uint_as_float(dw[k] << 16), acc);
      acc = fmaf(__uint_as_float(ow[k] & 0xffff0000u), __uint_as_float(dw[k] & 0xffff0000u), acc);
      qm = fmaxf(qm, fmaxf(fabsf(__uint_as_float(qw[k] << 16)), fabsf(__uint_as_float(qw[k] & 0xffff0000u))));
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    acc += __shfl_xor(acc, m, 16);
    qm = fmaxf(qm, __shfl_xor(qm, m, 16));
  }
  if (row < nrows) {
    const int qe = pow2_exponent(qm);
    u32x4 hw;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      hw[k] = pack_f16x2(__builtin_amdgcn_ldexpf(__uint_as_float(qw[k] << 16), -qe),
                         __builtin_amdgcn_ldexpf(__uint_as_float(qw[k] & 0xffff0000u), -qe));
    *(u32x4*)((uint16_t*)a.q16 + row * D + 8 * li) = hw;
    if (li == 0) {
      const int hq = (int)(row % a.Hq);
      const int64_t bt = row / a.Hq;
      const int t = (int)(bt % a.Lq);
      const int b = (int)(bt / a.Lq);
      const int64_t o = ((int64_t)b * a.Hq + hq) * a.Lq + t;
      a.delta[o] = acc;
      a.qscale[o] = __builtin_amdgcn_ldexpf(1.f, qe);
    }
  }
}

template <int V>
using IC = std::integral_constant<int, V>;

// S and dP products with the accumulator in VGPRs (the VALU reads each element as soon as
// it is final, without an AGPR read) and the B operand in AGPRs (the lane's register-
// resident fragment: K or V in the dK/dV kernel, Q or dO in the dQ kernel).  The "0"
// forms start from a zero accumulator; their output is early-clobber, so it never shares
// registers with the operands.
__device__ __forceinline__ void mfma_f16_va(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_f16_va0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_bf16_va(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_bf16_va0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}

// ------------------------------------------------------------------------ dQ
// One work item = (KV head, q-block of 128 rows), 4 waves x 32 rows; each lane owns one
// query row (column of the transposed products) and keeps its Q and dO fragments in
// AGPRs (the B operands of S^T and dP^T, whose accumulators are VGPRs).  The item walks
// its row list as 64-key tiles t (two per listed 128-key
// block).  Iteration t is one block of 48 MFMAs, the dQ^T += K^T dS^T products of tile
// t-1 (16) then S^T = K Q^T and dP^T = V dO^T of tile t+1 (32), with the VALU work of
// tile t (P, dS and their bf16 packing) spread between them by scheduling fences.  K
// and V tiles are copied straight into LDS two tiles ahead: four K buffers (tiles t-1,
// t+1 read, t+2 arriving) and two V buffers (t+1 read, t+2 arriving), each its own
// array, indexed at compile time (the tile loop is unrolled by 4), so the compiler can
// tell the reads from the copies in flight.
constexpr int QBK = 64;          // keys per tile
constexpr int QTL = QBK * D;     // elements per K or V tile (16 KB)

__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16384))) __bf16 sK0[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sK1[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sK2[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sK3[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sV0[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sV1[QTL];
  auto kbuf = [&](auto c) -> __bf16* {
    constexpr int i = decltype(c)::value & 3;
    if constexpr (i == 0) return sK0;
    else if constexpr (i == 1) return sK1;
    else if constexpr (i == 2) return sK2;
    else return sK3;
  };
  auto vbuf = [&](auto c) -> __bf16* {
    if constexpr ((decltype(c)::value & 1) == 0) return sV0;
    else return sV1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: copy targets form on the SALU
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int item = load_uniform(a.row_order, blockIdx.x);
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int G = a.G, Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;
  const __bf16* dO = (const __bf16*)a.dout;

  // Key rows past Lk are outside the copies' range: their LDS keeps what it held.  Cleared
  // once here, it only ever holds zeros or earlier finite rows, which the mask hides.
#pragma unroll
  for (int i = 0; i < QTL / (256 * 8); ++i) {
    const int o = 8 * (tid + 256 * i);
    store16(sK0 + o, zero_bf16x8());
    store16(sK1 + o, zero_bf16x8());
    store16(sK2 + o, zero_bf16x8());
    store16(sK3 + o, zero_bf16x8());
    store16(sV0 + o, zero_bf16x8());
    store16(sV1 + o, zero_bf16x8());
  }
  __syncthreads();  // cleared before any copy lands

  // this lane's query row
  const int r = wave * 32 + n;
  const int rt = r / G;
  const int t = qb * Bq + rt;
  const int hq = h * G + (r - rt * G);
  const bool rvalid = (rt < Bq) && (t < a.Lq);
  const int p = t + off;
  float lse2 = INFINITY, dlt = 0.f;
  bf16x8 qf[8], df[8];
  if (rvalid) {
    lse2 = a.lse[((int64_t)b * a.Hq + hq) * a.Lq + t] * kLog2e;
    dlt = a.delta[((int64_t)b * a.Hq + hq) * a.Lq + t];
    const int64_t ro = (((int64_t)b * a.Lq + t) * a.Hq + hq) * D + 8 * h2;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      qf[dd] = load16(Q + ro + 16 * dd);
      df[dd] = load16(dO + ro + 16 * dd);
    }
  } else {
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) qf[dd] = df[dd] = zero_bf16x8();
  }
  // held in AGPRs as the B operands of the S, dP products: the VGPRs hold those products'
  // accumulators
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) asm volatile("" : "+a"(qf[dd]), "+a"(df[dd]));
  if (lse2 == -INFINITY) lse2 = INFINITY;  // a row with no visible key has P = 0

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // LDS offsets (elements) inside a tile, as in the dK/dV kernel: operand reads of key row
  // 32 k2 + n, columns 16 dd + 8 h2 (base XOR dd << 4); transposed reads of key rows
  // 16 (2 k2 + hf) + vrow (+8), columns 32 db + vcol (base XOR db << 5).
  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);
  int ofs_a0 = lds_swz(n, 8 * h2);
  int ofs_t0[2] = {lds_swz(vrow, vcol), lds_swz(vrow + 8, vcol)};
  auto ofs_a = [&](int k2, int dd) { return 4096 * k2 + (ofs_a0 ^ (dd << 4)); };
  auto ofs_t = [&](int k2, int hf, int pp, int db) { return 2048 * (2 * k2 + hf) + (ofs_t0[pp] ^ (db << 5)); };

  // Copies of a tile: wave w fills key rows 16 w .. 16 w + 15, 4 rows per copy; lane L of
  // copy u fills row kr = 16 w + 4 u + L / 16, physical chunk L % 16 (logical chunk
  // (L % 16) ^ lds_sw(kr)).  voff[u]: its byte offset from the tile's first key.
  const int HkvD = a.Hkv * D;
  uint32_t voff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int kr = 16 * wave + 4 * u + (lane >> 4);
    voff[u] = 2u * (uint32_t)(kr * HkvD + h * D + 8 * ((lane & 15) ^ lds_sw(kr)));
  }

  const int e0 = load_uniform(a.row_ptr, item);
  const int n_ent = load_uniform(a.row_ptr, item + 1) - e0;
  const int ntile = 2 * n_ent;
  // first key of tile tt, and its entry; tiles past the list get an empty copy range
  auto tile_j0 = [&](int ent, int tt) { return (ent >> 1) * BK + (tt & 1) * QBK; };
  __amdgpu_buffer_rsrc_t rk, rv;
  // the batch's K / V base and byte count are formed once; per tile only the offset
  const int64_t kv_bytes = (int64_t)a.Lk * HkvD * 2;
  const char* const kbase = (const char*)(K + (int64_t)b * a.Lk * HkvD);
  const char* const vbase = (const char*)(V + (int64_t)b * a.Lk * HkvD);
  auto prepare_copy = [&](int ent, int tt, bool real) {
    const int64_t off = (int64_t)tile_j0(ent, tt) * (HkvD * 2);
    rk = tile_rsrc(kbase, kv_bytes, off, real);
    rv = tile_rsrc(vbase, kv_bytes, off, real);
  };
  auto copy = [&](int i, __bf16* kd, __bf16* vd) {  // copy i of 8 (u = i / 2, K then V)
    const int u = i >> 1;
    buf2lds((i & 1) ? rv : rk, voff[u], ((i & 1) ? vd : kd) + (16 * wave + 4 * u) * D);
  };
  // masked element: S = -inf where the key is hidden from the row
  auto mask = [&](f32x16 (&s)[2], int j0) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + 32 * k2 + 8 * (i >> 2) + 4 * h2 + (i & 3);
        s[k2][i] = (rvalid & visible(p, j, a.Lk, a.win.sink, a.win.near_w, band)) ? s[k2][i] : -INFINITY;
      }
  };

  if (n_ent > 0) {
    // entries of tiles t, t+1, t+2 (two tiles per entry).  The entry after them is
    // fetched by a vector load (a scalar load would share its wait counter with the LDS
    // operand reads) through a resource over this item's entries, so a fetch past the end
    // reads 0 (only ever used for tiles that are not copied), and taken two tiles later.
    const __amdgpu_buffer_rsrc_t r_ent = make_rsrc(a.row_ent + e0, (int64_t)n_ent * 4);
    int ent[3];
    ent[0] = load_uniform(a.row_ent, e0);
    ent[1] = ent[0];
    ent[2] = n_ent > 1 ? load_uniform(a.row_ent, e0 + 1) : ent[0];
    int ent_next = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * 2, 0);

    // prologue: tiles 0 and 1 resident; S, dP of tile 0
    prepare_copy(ent[0], 0, true);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy(i, sK0, sV0);
    prepare_copy(ent[1], 1, ntile > 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy(i, sK1, sV1);
    wait_loads_and_barrier();

    f32x16 sA[2], dA[2], sB[2], dB[2];  // S^T, dP^T of two consecutive tiles (2 key blocks)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      mfma_bf16_va0(sA[k2], load16(sK0 + ofs_a(k2, 0)), qf[0]);
      mfma_bf16_va0(dA[k2], load16(sV0 + ofs_a(k2, 0)), df[0]);
#pragma unroll
      for (int dd = 1; dd < 8; ++dd) {
        mfma_bf16_va(sA[k2], load16(sK0 + ofs_a(k2, dd)), qf[dd]);
        mfma_bf16_va(dA[k2], load16(sV0 + ofs_a(k2, dd)), df[dd]);
      }
    }
    uint32_t dsp[2][2][4];  // packed dS^T of the previous tile: [k2][hf] bf16x8 as 4 words
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < 4; ++w) dsp[k2][hf][w] = 0u;

    // One iteration for tile tt (tt % 4 = TC at compile time).  cur: S, dP of tile tt;
    // nxt: S, dP of tile tt + 1 (computed here).
    auto iteration = [&](auto tcc, const int tt, f32x16 (&cs)[2], f32x16 (&cd)[2], f32x16 (&ns)[2],
                         f32x16 (&nd)[2]) {
      constexpr int TC = decltype(tcc)::value;
      wait_loads_and_barrier();  // tile tt + 1 resident; every wave done with tile tt - 1
      // copies of tile tt + 2 (K into the buffer of tile tt - 2, V into that of tile tt)
      prepare_copy(ent[2], tt + 2, tt + 2 < ntile);
      __bf16* kd = kbuf(IC<(TC + 2) & 3>{});
      __bf16* vd = vbuf(IC<TC & 1>{});
      if (ent[0] & 1) mask(cs, tile_j0(ent[0], tt));
      const __bf16* kq = kbuf(IC<(TC + 3) & 3>{});  // K of tile tt - 1 (dQ)
      const __bf16* kn = kbuf(IC<(TC + 1) & 3>{});  // K of tile tt + 1 (S)
      const __bf16* vn = vbuf(IC<(TC + 1) & 1>{});  // V of tile tt + 1 (dP)
      float pr[2][16], dsv[2][16];
      uint32_t npk[2][2][4];
      // operands: transposed K of tile tt - 1 for the first 16 MFMAs, K / V rows of tile
      // tt + 1 for the other 32, each read kLead MFMAs ahead
      constexpr int kLead = 4;
      bf16x8 opA[48];
      auto load_op = [&](int x) {
        if (x < 16) {
          const int k2 = x >> 3, hf = (x >> 2) & 1, db = x & 3;
          opA[x] = join(lds_read_tr4(kq + ofs_t(k2, hf, 0, db)), lds_read_tr4(kq + ofs_t(k2, hf, 1, db)));
        } else {  // four chains (k2, S / dP) in rotation
          const int y = x - 16, k2 = y & 1, dd = y >> 2;
          opA[x] = load16((((y >> 1) & 1) ? vn : kn) + ofs_a(k2, dd));
        }
      };
#pragma unroll
      for (int x = 0; x < kLead; ++x) load_op(x);
      float csv[2], cdv[2];  // S, dP elements taken one step before use
      csv[0] = pin(cs[0][0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < 48; ++x) {
        if (x + kLead < 48) load_op(x + kLead);
        if (x < 16) {
          const int k2 = x >> 3, hf = (x >> 2) & 1, db = x & 3;
          const u32x4 w = {dsp[k2][hf][0], dsp[k2][hf][1], dsp[k2][hf][2], dsp[k2][hf][3]};
          acc[db] = mfma32x32x16(opA[x], __builtin_bit_cast(bf16x8, w), acc[db]);
        } else {
          // accumulators in VGPRs, each chain starting from zero (dd = 0)
          const int y = x - 16, k2 = y & 1, dd = y >> 2;
          if ((y >> 1) & 1) {
            if (dd == 0) mfma_bf16_va0(nd[k2], opA[x], df[0]);
            else mfma_bf16_va(nd[k2], opA[x], df[dd]);
          } else {
            if (dd == 0) mfma_bf16_va0(ns[k2], opA[x], qf[0]);
            else mfma_bf16_va(ns[k2], opA[x], qf[dd]);
          }
        }
        if (x >= 4 && x < 12) copy(x - 4, kd, vd);
        __builtin_amdgcn_sched_barrier(0);
        // VALU of tile tt: element e = x (0..31) gets P in step x, dS in step x + 4; pairs
        // are packed to bf16 in steps 32..47.  Inputs are taken (pin) one step before use
        // and results fenced (pin_out) one step after they are made: a read right at a pin
        // or a fence right after an exp costs a wait state each.
        if (x < 32) pr[x >> 4][x & 15] = __builtin_amdgcn_exp2f(fmaf(csv[x & 1], a.scale_log2, -lse2));
        if (x + 1 < 32) csv[(x + 1) & 1] = pin(cs[(x + 1) >> 4][(x + 1) & 15]);
        if (x >= 1 && x <= 32) pin_out(pr[(x - 1) >> 4][(x - 1) & 15]);
        if (x >= 4 && x < 36) {
          const int e = x - 4, k2 = e >> 4, i = e & 15;
          dsv[k2][i] = pr[k2][i] * (cdv[e & 1] - dlt);
        }
        if (x >= 3 && x < 35) {
          const int e = x - 3;
          cdv[e & 1] = pin(cd[e >> 4][e & 15]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // dS pair q (elements 2 q, 2 q + 1) packed to bf16 at step 2 q + 7, after this
        // step's own VALU work (its second element was fenced at the end of the previous
        // step: a read right after the fence would cost a wait state), and fenced in turn
        // a step later; pair q sits in word q % 4 of half (q / 4) % 2 of block q / 8
        if (x >= 7 && x <= 37 && (x & 1)) {
          const int q = (x - 7) >> 1, k2 = q >> 3, hf = (q >> 2) & 1, w = q & 3;
          const float x0 = dsv[k2][2 * (q & 7)], x1 = dsv[k2][2 * (q & 7) + 1];
          const bf16x2 v = {(__bf16)x0, (__bf16)x1};
          npk[k2][hf][w] = __builtin_bit_cast(uint32_t, v);
        }
        if (x >= 8 && x <= 38 && (x & 1) == 0) {
          const int q = (x - 8) >> 1;
          pin_out(npk[q >> 3][(q >> 2) & 1][q & 3]);
        }
        if (x >= 5 && x <= 36) pin_out(dsv[(x - 5) >> 4][(x - 5) & 15]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int w = 0; w < 4; ++w) dsp[k2][hf][w] = npk[k2][hf][w];
      // advance the entry window at entry boundaries (two tiles per entry)
      if (tt & 1) {
        ent[0] = ent[2];
        ent[1] = ent[2];
        ent[2] = __builtin_amdgcn_readfirstlane(ent_next);
        const int en = ((tt + 1) >> 1) + 2;  // entry of tile tt + 5
        ent_next = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * en, 0);
      } else {
        ent[0] = ent[1];
      }
    };
    int tt = 0;
    for (; tt + 4 <= ntile; tt += 4) {
      iteration(IC<0>{}, tt, sA, dA, sB, dB);
      iteration(IC<1>{}, tt + 1, sB, dB, sA, dA);
      iteration(IC<2>{}, tt + 2, sA, dA, sB, dB);
      iteration(IC<3>{}, tt + 3, sB, dB, sA, dA);
    }
    if (tt < ntile) {  // ntile is even: two more tiles
      iteration(IC<0>{}, tt, sA, dA, sB, dB);
      iteration(IC<1>{}, tt + 1, sB, dB, sA, dA);
    }
    // dQ of the last tile (its K sits in buffer (ntile - 1) % 4)
    __builtin_amdgcn_s_waitcnt(0x0f70);
    const int lastc = (ntile - 1) & 3;
    const __bf16* kl = lastc == 0 ? sK0 : lastc == 1 ? sK1 : lastc == 2 ? sK2 : sK3;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int k2 = x >> 3, hf = (x >> 2) & 1, db = x & 3;
      const bf16x8 ka = join(lds_read_tr4(kl + ofs_t(k2, hf, 0, db)), lds_read_tr4(kl + ofs_t(k2, hf, 1, db)));
      const u32x4 w = {dsp[k2][hf][0], dsp[k2][hf][1], dsp[k2][hf][2], dsp[k2][hf][3]};
      acc[db] = mfma32x32x16(ka, __builtin_bit_cast(bf16x8, w), acc[db]);
    }
  }

  if (rvalid) {
    __bf16* dq = (__bf16*)a.dq + (((int64_t)b * a.Lq + t) * a.Hq + hq) * D + 4 * h2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const bf16x4 v = to_bf16x4(acc[db][4 * q4] * a.scale, acc[db][4 * q4 + 1] * a.scale,
                                   acc[db][4 * q4 + 2] * a.scale, acc[db][4 * q4 + 3] * a.scale);
        *(u32x2*)(dq + 32 * db + 8 * q4) = __builtin_bit_cast(u32x2, v);
      }
  }
}

// ------------------------------------------------------------------------ dK, dV
// Software pipeline over the 32-row blocks g of the item's column list (4 per q-block).
// Step g: phase 1 issues S and dP of block g + 1 (16 MFMAs) with dS of block g and the
// packing of P and dS of block g between them; phase 2 issues dV and dK of block g (16
// MFMAs) with P of block g + 1 between them.  Scheduling fences keep each piece of VALU
// work in its slot, so the matrix core and the VALU run at the same time.  The Q and dO
// tiles of a q-block are double-buffered in LDS and filled by direct global->LDS copies
// issued one q-block ahead.
//
// dK is formed in fp16: dS and Q are each rounded once to fp16 (10-bit mantissa), which
// keeps dK well inside the bf16 tolerance (a single bf16 rounding of dS is not enough:
// dK sums the products of many rows whose dS nearly cancel).  Q comes from the fp16
// copy the Delta kernel writes, each row divided by 2^e_r (its max |q| then in [1, 2)),
// so the copy is exact; S = Q K^T then also runs in fp16, with K divided by 2^e_K per
// work item.  The scales come back through per-row constants:
//   P = exp2(S16 c_r - LSE_r log2 e)   with c_r = scale log2(e) 2^(e_r + e_K),
//   dS16 = 2^e_r dS = P (2^e_r dP - 2^e_r Delta_r),   so dS16^T Q16 = dS^T Q.
constexpr int QTILE = ROWS * D;  // one q-block of Q (or dO) in LDS

// (x0, x1) -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1) {
  const bf16x2 h = {(__bf16)x0, (__bf16)x1};
  return __builtin_bit_cast(uint32_t, h);
}

// bf16 x -> fp16 bits of x / 2^e (exact while |x| / 2^e is in the fp16 normal range).
__device__ __forceinline__ bf16x8 bf16_to_f16_scaled(const bf16x8& x, int e) {
  const u32x4 w = __builtin_bit_cast(u32x4, x);
  u32x4 h;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    h[q] = pack_f16x2(__builtin_amdgcn_ldexpf(__uint_as_float(w[q] << 16), -e),
                      __builtin_amdgcn_ldexpf(__uint_as_float(w[q] & 0xffff0000u), -e));
  return __builtin_bit_cast(bf16x8, h);
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  // Q (fp16 copy) and dO of a q-block, [Q, dO][rows] with swizzled 256-byte rows
  // (lds_swz); dO sits at a fixed distance from Q, so one address serves both.  Two
  // separate arrays (not one indexed by the buffer): every read names the array it reads,
  // so the compiler can tell it apart from the copies in flight into the other one and
  // does not wait for them.
  __shared__ __attribute__((aligned(1024))) __bf16 sQD0[2 * QTILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sQD1[2 * QTILE];
  // per-row constants of a q-block: [LSE log2 e, c_r, 2^e_r, 2^e_r Delta][rows]
  __shared__ __attribute__((aligned(16))) float sLT0[4 * ROWS];
  __shared__ __attribute__((aligned(16))) float sLT1[4 * ROWS];
  __shared__ int sRt[ROWS];  // row -> token in the q-block
  __shared__ float sKmax[4];  // max |k| of each wave's keys
  auto tiles = [&](auto bufc) -> __bf16* {
    if constexpr (decltype(bufc)::value == 0) return sQD0;
    else return sQD1;
  };
  auto lts = [&](auto bufc) -> float* {
    if constexpr (decltype(bufc)::value == 0) return sLT0;
    else return sLT1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: copy targets form on the SALU
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int item = load_uniform(a.col_order, blockIdx.x);
  const int b = blockIdx.y;
  const int h = item / a.nkb;
  const int kb = item - h * a.nkb;
  const int G = a.G, Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const uint16_t* Q16 = (const uint16_t*)a.q16;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;
  const __bf16* dO = (const __bf16*)a.dout;

  if (tid < ROWS) sRt[tid] = tid / G;
  // Rows of the last q-block past Lq are outside the copies' range: their LDS keeps what
  // it held.  Cleared once here, it only ever holds zeros or earlier finite rows, which
  // the row's LSE of +inf turns into P = 0.
#pragma unroll
  for (int i = 0; i < 2 * QTILE / (256 * 8); ++i) {
    store16(sQD0 + 8 * (tid + 256 * i), zero_bf16x8());
    store16(sQD1 + 8 * (tid + 256 * i), zero_bf16x8());
  }
  __syncthreads();  // cleared before any copy lands

  // this lane's key (column of S and dP)
  const int j = kb * BK + wave * 32 + n;
  const bool kvalid = j < a.Lk;
  bf16x8 kf[8], vf[8];
  {
    const int64_t ko = (((int64_t)b * a.Lk + (kvalid ? j : 0)) * a.Hkv + h) * D + 8 * h2;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      kf[dd] = kvalid ? load16(K + ko + 16 * dd) : zero_bf16x8();
      vf[dd] = kvalid ? load16(V + ko + 16 * dd) : zero_bf16x8();
      // held in AGPRs (MFMA reads its A/B operands from either file): leaves the VGPRs
      // to the pipeline's temporaries
      asm volatile("" : "+a"(vf[dd]));
    }
  }

  f32x16 accK[4], accV[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) accK[db][i] = accV[db][i] = 0.f;

  // Per-lane LDS offsets inside a 32-row block (the swizzle depends on row % 16 only, so
  // row block rb adds 32 rb rows and half hf adds 16 rows to these):
  //   operand reads (S, dP): row n, columns 16 dd + 8 h2;
  //   transposed reads (dV, dK): rows vrow (+8), columns 32 db + vcol.
  // Under the XOR swizzle the element offset for dd (resp. db) is the dd = 0 (db = 0)
  // offset with bits 4-6 (5-6) XORed by dd (db), so three registers hold them all.
  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);
  int ofs_a0 = lds_swz(n, 8 * h2);
  int ofs_t0[2] = {lds_swz(vrow, vcol), lds_swz(vrow + 8, vcol)};
  auto ofs_a = [&](int dd) { return ofs_a0 ^ (dd << 4); };
  auto ofs_t = [&](int p, int db) { return ofs_t0[p] ^ (db << 5); };

  // Direct copies: wave w fills rows 32 w .. 32 w + 31 of a tile, 4 rows per copy; lane L
  // of copy u fills row r = 32 w + 4 u + L / 16, physical chunk L % 16, i.e. logical chunk
  // (L % 16) ^ lds_sw(r) of that row.  voff_u[u] is that chunk's byte offset from the
  // q-block's first token: token tk = r / G (rows past the q-block take its last token;
  // their LSE is +inf) times Hq * D, plus the head's columns.
  const int HqD = a.Hq * D;
  uint32_t voff_u[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = wave * 32 + 4 * u + (lane >> 4);
    int rt = r / G, g = r - rt * G;
    if (rt >= Bq) {
      rt = Bq - 1;
      g = 0;
    }
    voff_u[u] = 2u * (uint32_t)(rt * HqD + (h * G + g) * D + 8 * ((lane & 15) ^ lds_sw(r)));
  }
  // Row constants staging: thread tid < ROWS owns row tid of the next q-block.  The raw
  // loaded values are only touched when stored to LDS (after the wait that precedes the
  // q-block's first use), so the loads do not stall the wave when they are issued.
  const int my_rt = tid / G, my_g = tid - my_rt * G;
  float plse = 0.f, pdel = 0.f, pqs = 1.f, ck = a.scale_log2;
  bool pvalid = false;
  // LSE, Delta and Q row scales of this KV head's G query heads, [G, Lq] each
  const int64_t lt_base = ((int64_t)b * a.Hq + h * G) * a.Lq;
  const __amdgpu_buffer_rsrc_t r_lse = make_rsrc(a.lse + lt_base, (int64_t)G * a.Lq * 4);
  const __amdgpu_buffer_rsrc_t r_del = make_rsrc(a.delta + lt_base, (int64_t)G * a.Lq * 4);
  const __amdgpu_buffer_rsrc_t r_qs = make_rsrc(a.qscale + lt_base, (int64_t)G * a.Lq * 4);

  const int e0 = load_uniform(a.col_ptr, item);
  const int n_ent = load_uniform(a.col_ptr, item + 1) - e0;

  // Copies of q-block qb's Q and dO rows: prepare_entry builds the two buffer resources
  // (scalar; the range ends at token Lq, so rows past Lq read zeros; an empty range when
  // there is no next q-block, so the copies then touch no memory) and loads the row
  // constants into registers; copy(i) issues copy i of 16 (u = i / 2, Q then dO) into
  // buffer bufc, so the copies can be spread over MFMA slots.
  __amdgpu_buffer_rsrc_t rq_n, rd_n;
  const int64_t qd_bytes = (int64_t)a.Lq * HqD * 2;
  const char* const qbase = (const char*)(Q16 + (int64_t)b * a.Lq * HqD);
  const char* const dobase = (const char*)(dO + (int64_t)b * a.Lq * HqD);
  auto prepare_entry = [&](int qb, bool real) {
    const int t0 = qb * Bq;
    const int64_t off = (int64_t)t0 * (HqD * 2);
    rq_n = tile_rsrc(qbase, qd_bytes, off, real);
    rd_n = tile_rsrc(dobase, qd_bytes, off, real);
    if (tid < ROWS) {
      pvalid = my_rt < Bq && t0 + my_rt < a.Lq;
      // rows past Lq read row Lq - 1 (in bounds; discarded by pvalid)
      const uint32_t vo = 4u * (uint32_t)(my_g * a.Lq + min(t0 + my_rt, a.Lq - 1));
      plse = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_lse, vo, 0, 0));
      pdel = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_del, vo, 0, 0));
      pqs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_qs, vo, 0, 0));
    }
  };
  auto copy = [&](int i, auto bufc) {
    __bf16* dst = tiles(bufc) + wave * 32 * D + 4 * (i >> 1) * D + ((i & 1) ? QTILE : 0);
    buf2lds((i & 1) ? rd_n : rq_n, voff_u[i >> 1], dst);
  };
  // Rows with no token or no visible key: LSE +inf (P = 0), c_r > 0 (so that a masked
  // S = -inf still gives P = 0), and 0 for the dS scale and Delta.  ck = scale log2(e)
  // 2^e_K.
  auto store_lse = [&](auto bufc) {
    if (tid < ROWS) {
      float* lt = lts(bufc);
      lt[tid] = (pvalid && plse != -INFINITY) ? plse * kLog2e : INFINITY;
      lt[ROWS + tid] = pvalid ? ck * pqs : ck;
      lt[2 * ROWS + tid] = pvalid ? pqs : 0.f;
      lt[3 * ROWS + tid] = pvalid ? pdel * pqs : 0.f;
    }
  };
  // boundary q-block: the window predicate per element (S = -inf where hidden)
  auto mask = [&](f32x16& s, int rb, int qb) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int rr = 32 * rb + 8 * i4 + 4 * h2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = qb * Bq + sRt[rr + i];
        const bool vis = kvalid & visible(t + off, j, a.Lk, a.win.sink, a.win.near_w, band);
        s[4 * i4 + i] = vis ? s[4 * i4 + i] : -INFINITY;
      }
    }
  };

  // Carried from one step to the next: P of the block in fp32, dP as the MFMA left it,
  // and the first group of the block's dS constants (2^e_r, 2^e_r Delta), read early so
  // the next step's first slot does not wait for LDS.
  struct Carry {
    float pr[16];
    f32x16 dp;
    f32x4 f0, t0;
  };
  auto as_bf16x8 = [](const uint32_t (&w)[4]) { return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]}); };

  if (n_ent > 0) {
    // The list is walked cyclically from its first q-block at or after the one holding
    // token (kb | 31) Bk.  The work items an XCD runs together are about 32 neighbouring
    // k-blocks of one head, whose lists are near-translates of each other and all hold
    // that q-block: started there, they read the same Q / dO tiles at the same time (one
    // L2 fill serves all of them) instead of ranges shifted by Bk tokens per k-block.
    int rot = 0;
    {
      const int qa = max(0, ((kb | 31) * BK - off) / Bq);
      int lo = 0, hi = n_ent;  // first index whose q-block is >= qa (the list ascends)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((load_uniform(a.col_ent, e0 + mid) >> 1) < qa) lo = mid + 1;
        else hi = mid;
      }
      rot = lo < n_ent ? lo : 0;
    }
    auto ent_index = [&](int e) {  // list index of walk position e (e < 2 n_ent)
      const int i = e + rot;
      return i >= n_ent ? i - n_ent : i;
    };
    int ent_c = load_uniform(a.col_ent, e0 + rot);  // entry of the current q-block
    // entry of the next q-block, fetched one q-block before it is needed by a vector load
    // (a scalar load would share its wait counter with the LDS operand reads) through a
    // resource over this item's entries (a fetch past the end reads 0 and is not used)
    const __amdgpu_buffer_rsrc_t r_ent = make_rsrc(a.col_ent + e0, (int64_t)n_ent * 4);
    int ent_ahead = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * ent_index(1), 0);
    int ent_n = ent_c;
    prepare_entry(ent_c >> 1, true);
#pragma unroll
    for (int i = 0; i < 16; ++i) copy(i, IC<0>{});
    // K of the work item in fp16, divided by 2^e_K (max |k| over its 128 keys then in
    // [1, 2)): each wave's max goes through LDS
    {
      float km = 0.f;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const u32x4 w = __builtin_bit_cast(u32x4, kf[dd]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          km = fmaxf(km, fmaxf(fabsf(__uint_as_float(w[q] << 16)), fabsf(__uint_as_float(w[q] & 0xffff0000u))));
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) km = fmaxf(km, __shfl_xor(km, m));
      if (lane == 0) sKmax[wave] = km;
    }
    wait_loads_and_barrier();
    {
      const int ek = pow2_exponent(fmaxf(fmaxf(sKmax[0], sKmax[1]), fmaxf(sKmax[2], sKmax[3])));
      ck = a.scale_log2 * __builtin_amdgcn_ldexpf(1.f, ek);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        kf[dd] = bf16_to_f16_scaled(kf[dd], ek);
        asm volatile("" : "+a"(kf[dd]));
      }
    }
    store_lse(IC<0>{});
    __syncthreads();

    Carry wA, wB;
    // Q and dO operands (dd = 0, 1) of the S, dP products a step issues first, read during
    // the previous step's phase 2 so that its first MFMAs do not wait for LDS (possible
    // whenever those rows are resident then: not for the step that follows row block 2,
    // whose rows come from the q-block still being copied)
    bf16x8 pfq[2], pfd[2];
#pragma unroll
    for (int dd = 0; dd < 2; ++dd) {
      pfq[dd] = load16(sQD0 + 4096 + ofs_a(dd));
      pfd[dd] = load16(sQD0 + 4096 + QTILE + ofs_a(dd));
    }
    {  // prologue: S, dP and P of block 0
      f32x16 s;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = wA.dp[i] = 0.f;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        s = mfma32x32x16_f16(load16(sQD0 + ofs_a(dd)), kf[dd], s);
        wA.dp = mfma32x32x16(load16(sQD0 + QTILE + ofs_a(dd)), vf[dd], wA.dp);
      }
      if (ent_c & 1) mask(s, 0, ent_c >> 1);
      const float* lt = sLT0 + 4 * h2;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 l4 = *(const f32x4*)(lt + 8 * i4);
        const f32x4 c4 = *(const f32x4*)(lt + ROWS + 8 * i4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wA.pr[4 * i4 + i] = __builtin_amdgcn_exp2f(fmaf(s[4 * i4 + i], c4[i], -l4[i]));
      }
      wA.f0 = *(const f32x4*)(lt + 2 * ROWS);
      wA.t0 = *(const f32x4*)(lt + 3 * ROWS);
    }

    // One pipeline step for row block RB of the q-block in buffer BUF (both compile-time).
    // After the item's last block the "next" block is the resident other buffer's first
    // block: computed and discarded, so the step has no branches inside its interleaved
    // parts.
    auto step = [&](auto rbc, auto bufc, const int e, Carry& cur, Carry& nxt) {
      constexpr int RB = decltype(rbc)::value;
      constexpr int BUF = decltype(bufc)::value;
      constexpr int RB1 = (RB + 1) & 3;
      constexpr int BUF1 = RB == 3 ? BUF ^ 1 : BUF;
      const bool more = e + 1 < n_ent;  // a next q-block exists
      // the dK, dV accumulators stay in AGPRs across steps (else the allocator parks them
      // in VGPRs over part of the loop and copies them back and forth)
#pragma unroll
      for (int db = 0; db < 4; ++db) asm volatile("" : "+a"(accK[db]), "+a"(accV[db]));
      if constexpr (RB == 0) {
        // every wave is done with q-block e - 1: its buffer takes q-block e + 1, copied
        // during the phase-2 MFMAs of this step and the next
        __syncthreads();
        const int ea = __builtin_amdgcn_readfirstlane(ent_ahead);
        if (more) ent_n = ea;
        prepare_entry(ent_n >> 1, more);
        ent_ahead = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * ent_index(e + 2), 0);
      }
      const int ent_g1 = RB == 3 ? ent_n : ent_c;  // entry of the next block
      if constexpr (RB == 3) {
        if (more) {  // q-block e + 1 resident
          __builtin_amdgcn_s_waitcnt(0x0f70);
          store_lse(IC<BUF ^ 1>{});
          __syncthreads();
        }
      }

      // ---- phase 1: S, dP of the next block; dS of block g, packing of P and dS
      const __bf16* tg = tiles(bufc) + 4096 * RB;         // Q rows of block g (dO: + QTILE)
      const __bf16* t1 = tiles(IC<BUF1>{}) + 4096 * RB1;  // Q rows of the next block
      const float* lg = lts(bufc) + 32 * RB + 4 * h2;     // row constants of block g
      const float* lt = lts(IC<BUF1>{}) + 32 * RB1 + 4 * h2;  // and of the next block
      // operands of the next block's S, dP: four dd steps in flight, dd + 4 read when dd's
      // pair of MFMAs has been issued
      bf16x8 qa[8], da[8];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        if (RB != 3 && dd < 2) {
          qa[dd] = pfq[dd];
          da[dd] = pfd[dd];
        } else {
          qa[dd] = load16(t1 + ofs_a(dd));
          da[dd] = load16(t1 + QTILE + ofs_a(dd));
        }
      }
      bf16x8 dt[2][4], qt[2][4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dt[0][db] = join(lds_read_tr4(tg + QTILE + ofs_t(0, db)), lds_read_tr4(tg + QTILE + ofs_t(1, db)));
        qt[0][db] = join(lds_read_tr4(tg + ofs_t(0, db)), lds_read_tr4(tg + ofs_t(1, db)));
      }
      f32x16 sn;
      f32x4 f4[4], t4[4], l4[4], c4[4];
      f4[0] = cur.f0;
      t4[0] = cur.t0;
      float ds[16], prv[3], dpv[3];
      uint32_t wpa[2][4], wds[2][4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        prv[e] = pin(cur.pr[e]);
        dpv[e] = pin(cur.dp[e]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int dd = x >> 1;
        if (x == 0) mfma_f16_va0(sn, qa[0], kf[0]);
        else if (x == 1) mfma_bf16_va0(nxt.dp, da[0], vf[0]);
        else if (x & 1) mfma_bf16_va(nxt.dp, da[dd], vf[dd]);
        else mfma_f16_va(sn, qa[dd], kf[dd]);
        if ((x & 1) && dd + 4 < 8) {
          qa[dd + 4] = load16(t1 + ofs_a(dd + 4));
          da[dd + 4] = load16(t1 + QTILE + ofs_a(dd + 4));
        }
        // dS constants of groups 1..3, four slots before their first use; P constants of
        // the next block's group 0, for phase 2
        if ((x & 3) == 0 && x < 12) {
          const int i4 = (x >> 2) + 1;
          f4[i4] = *(const f32x4*)(lg + 2 * ROWS + 8 * i4);
          t4[i4] = *(const f32x4*)(lg + 3 * ROWS + 8 * i4);
        }
        if (x == 12) {
          l4[0] = *(const f32x4*)lt;
          c4[0] = *(const f32x4*)(lt + ROWS);
        }
        __builtin_amdgcn_sched_barrier(0);
        // P pair q at slot 2 q + 1, from the two pinned values (fenced at the next slot),
        // ahead of the slot's dS
        if (x & 1) {
          const int q = x >> 1;
          wpa[q >> 2][q & 3] = pack_bf16x2(prv[(x - 1) % 3], prv[x % 3]);
        } else if (x >= 2) {
          const int q = (x - 2) >> 1;
          pin_out(wpa[q >> 2][q & 3]);
        }
        // dS element x; inputs are taken (pin) two slots before and the result fenced
        // (pin_out) one slot after, so nothing waits on a result in its own slot.  A VALU
        // read of a pinned value right after the asm statement costs a wait state, and a
        // product written as asm does not count as one: hence two slots, not one.
        ds[x] = prv[x % 3] * fmaf(dpv[x % 3], f4[x >> 2][x & 3], -t4[x >> 2][x & 3]);
        if (x + 2 < 16) {
          prv[(x + 2) % 3] = pin(cur.pr[x + 2]);
          dpv[(x + 2) % 3] = pin(cur.dp[x + 2]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // dS pair q at slot 2 q + 3, after this slot's dS element (its second element was
        // fenced at the end of the previous slot), fenced in turn at the next slot
        if ((x & 1) && x >= 3) {
          const int q = (x - 3) >> 1;
          wds[q >> 2][q & 3] = pack_f16x2(ds[2 * q], ds[2 * q + 1]);
        }
        if ((x & 1) == 0 && x >= 4) {
          const int q = (x - 4) >> 1;
          pin_out(wds[q >> 2][q & 3]);
        }
        if (x >= 1) pin_out(ds[x - 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin_out(ds[15]);
      pin_out(wpa[1][3]);
      pin_out(wds[1][2]);
      wds[1][3] = pack_f16x2(ds[14], ds[15]);
      if (ent_g1 & 1) mask(sn, RB1, ent_g1 >> 1);

      // ---- phase 2: dV, dK of block g, interleaved with P of the next block
      const bf16x8 pa[2] = {as_bf16x8(wpa[0]), as_bf16x8(wpa[1])};
      const bf16x8 sa[2] = {as_bf16x8(wds[0]), as_bf16x8(wds[1])};
      float snv[2];
      snv[0] = pin(sn[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        // MFMA x: half hf = x / 8; dV (x even) and dK (x odd) for db = (x % 8) / 2
        const int hf = x >> 3, db = (x & 7) >> 1;
        if (x & 1) accK[db] = mfma32x32x16_f16(sa[hf], qt[hf][db], accK[db]);
        else accV[db] = mfma32x32x16(pa[hf], dt[hf][db], accV[db]);
        // transposed operands of half 1, each read right after its half-0 register is last
        // used: dO^T (db) after MFMA 2 db, read at 2 db + 1; Q^T (db) after MFMA 2 db + 1,
        // read at 2 db + 2
        if (x < 8 && (x & 1)) {
          const int db1 = x >> 1;
          dt[1][db1] = join(lds_read_tr4(tg + 2048 + QTILE + ofs_t(0, db1)), lds_read_tr4(tg + 2048 + QTILE + ofs_t(1, db1)));
        }
        if (x >= 2 && x <= 8 && (x & 1) == 0) {
          const int db1 = (x - 2) >> 1;
          qt[1][db1] = join(lds_read_tr4(tg + 2048 + ofs_t(0, db1)), lds_read_tr4(tg + 2048 + ofs_t(1, db1)));
        }
        // copies of the next q-block: 8 in each of the first two steps, one every 2 MFMAs
        if constexpr (RB < 2)
          if (x & 1) copy(8 * RB + (x >> 1), IC<BUF ^ 1>{});
        // P constants of groups 1..3, four slots ahead; the next step's first dS constants
        if ((x & 3) == 0 && x < 12) {
          const int i4 = (x >> 2) + 1;
          l4[i4] = *(const f32x4*)(lt + 8 * i4);
          c4[i4] = *(const f32x4*)(lt + ROWS + 8 * i4);
        }
        if (x == 12) {
          nxt.f0 = *(const f32x4*)(lt + 2 * ROWS);
          nxt.t0 = *(const f32x4*)(lt + 3 * ROWS);
        }
        // the next step's first operands (rows of block g + 2)
        if constexpr (RB != 2) {
          constexpr int RBn = (RB + 1) & 3, BUFn = RB == 3 ? BUF ^ 1 : BUF;
          constexpr int RB1n = (RBn + 1) & 3, BUF1n = RBn == 3 ? BUFn ^ 1 : BUFn;
          const __bf16* t1n = tiles(IC<BUF1n>{}) + 4096 * RB1n;
          if (x == 13 || x == 14) {
            const int dd = x - 13;
            pfq[dd] = load16(t1n + ofs_a(dd));
            pfd[dd] = load16(t1n + QTILE + ofs_a(dd));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        nxt.pr[x] = __builtin_amdgcn_exp2f(fmaf(snv[x & 1], c4[x >> 2][x & 3], -l4[x >> 2][x & 3]));
        if (x + 1 < 16) snv[(x + 1) & 1] = pin(sn[x + 1]);
        if (x >= 1) pin_out(nxt.pr[x - 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin_out(nxt.pr[15]);
      if constexpr (RB == 3) ent_c = ent_n;
    };
    auto entry = [&](auto bufc, const int e) {
      step(IC<0>{}, bufc, e, wA, wB);
      step(IC<1>{}, bufc, e, wB, wA);
      step(IC<2>{}, bufc, e, wA, wB);
      step(IC<3>{}, bufc, e, wB, wA);
    };
    // q-blocks alternate between the two buffers
    for (int e = 0; e < n_ent; e += 2) {
      entry(IC<0>{}, e);
      if (e + 1 < n_ent) entry(IC<1>{}, e + 1);
    }
    // the last q-block's steps issued copies with an empty range: let them retire before
    // the work group's LDS can be handed on
    __builtin_amdgcn_s_waitcnt(0x0f70);
  }

  // element i of accK[db] / accV[db]: key 32 wave + 8 (i / 4) + 4 h2 + i % 4, dim 32 db + n
  __bf16* dK = (__bf16*)a.dk;
  __bf16* dV = (__bf16*)a.dv;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int jj = kb * BK + wave * 32 + 8 * (i >> 2) + 4 * h2 + (i & 3);
      if (jj < a.Lk) {
        const int64_t o = (((int64_t)b * a.Lk + jj) * a.Hkv + h) * D + 32 * db + n;
        dK[o] = (__bf16)(accK[db][i] * a.scale);
        dV[o] = (__bf16)accV[db][i];
      }
    }
}

}  // namespace

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, int stages, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (stages & COWA_BWD_DELTA) {
    const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((nrows + 15) / 16)), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (stages & COWA_BWD_DQ) {
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(a.Hkv * a.nqb, a.B), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (stages & COWA_BWD_DKDV) {
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(a.Hkv * a.nkb, a.B), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return err;
}

}  // namespace cowa
