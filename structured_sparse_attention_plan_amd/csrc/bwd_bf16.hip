// CoWindow Attention backward, bf16, head dim 128, for gfx950.
//
// Gradients of the same masked softmax attention the forward computes (the pages state
// that the pattern supports training forward and backward — beyondmarketintelligence.com
// post, second paragraph; "CoWindow Attention" abstract), recomputed from the saved
// logsumexp:
//   P = exp(scale q.k - LSE), Delta_i = dO_i . O_i, dP = dO V^T, dS = P (dP - Delta)
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO
// Three kernels, deterministic (the only atomics take two maxima):
//   delta  : Delta per (row, query head), and an fp16 copy of Q scaled per row by a
//            power of two;
//   dq     : one work item per (KV head, q-block of 128 / G tokens), walking the row list
//            of visible 128-key blocks: S^T, dP^T on MFMA, dS^T on the VALU,
//            dQ^T += K^T dS^T with K^T read by ds_read_b64_tr_b16 from the row-major LDS
//            tile; two work groups per CU;
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
// Per row (token, query head): Delta = dO . O (with O's rounding residual when the forward
// kept it), and the fp16 copies of q and dO that the products read, each row divided by
// the power of two that puts its max |x| in [1, 2) (2^e for q, 2^f for dO; e is stored as
// the scale 2^e and f as the exponent).  Sixteen lanes per row, 8 elements each.
//
// The same launch takes the launch-wide maxima the fp16 products need for their range
// (kept as unsigned integers: the bit patterns of non-negative floats and biased
// exponents order like the values), each atomic issued only when a wave's value exceeds
// the recorded one, so few reach the one L2 line:
//   [0] |dO_i| 2^e_i and [1] |Delta_i| 2^e_i (|.| the Euclidean norm over D): with |v_j|,
//       |dS_ij| 2^e_i = P_ij |dO_i . v_j - Delta_i| 2^e_i <= |dO_i| 2^e_i |v_j| + |Delta_i| 2^e_i;
//   [2] max f_i over rows with dO != 0 (the common scale of the dV product);
//   [3] max |k| (the scale of the fp16 copy of K) and [4] max |v_j|^2, from extra work
//       groups over the rows of K and V.
// bwd_clear_kernel zeroes them first.
__global__ __launch_bounds__(64) void bwd_clear_kernel(float* maxima) {
  if (threadIdx.x < 8) maxima[threadIdx.x] = 0.f;
}

__device__ __forceinline__ void max_u32(unsigned* g, unsigned v) {
  if (v > __atomic_load_n(g, __ATOMIC_RELAXED)) atomicMax(g, v);
}

// bf16 row chunk (8 values) -> fp16 bits of x / 2^e (exact while x / 2^e stays normal)
__device__ __forceinline__ u32x4 f16_scaled(const u32x4& w, int e) {
  u32x4 h;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    h[k] = pack_f16x2(__builtin_amdgcn_ldexpf(__uint_as_float(w[k] << 16), -e),
                      __builtin_amdgcn_ldexpf(__uint_as_float(w[k] & 0xffff0000u), -e));
  return h;
}

__device__ __forceinline__ float absmax8(const u32x4& w) {
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[k] << 16)), fabsf(__uint_as_float(w[k] & 0xffff0000u))));
  return m;
}

__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int li = threadIdx.x & 15;
  const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
  const int64_t qgroups = (nrows + 15) / 16;
  unsigned* g = (unsigned*)a.maxima;
  if ((int64_t)blockIdx.x >= qgroups) {
    // rows of K and V (b, j, h): max |k| and max |v_j|^2
    const int64_t row = ((int64_t)blockIdx.x - qgroups) * 16 + (threadIdx.x >> 4);
    float km = 0.f, vn = 0.f;
    if (row < (int64_t)a.B * a.Lk * a.Hkv) {
      const u32x4 kw = *(const u32x4*)((const __bf16*)a.k + row * D + 8 * li);
      const u32x4 vw = *(const u32x4*)((const __bf16*)a.v + row * D + 8 * li);
      km = absmax8(kw);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v0 = __uint_as_float(vw[k] << 16), v1 = __uint_as_float(vw[k] & 0xffff0000u);
        vn = fmaf(v0, v0, fmaf(v1, v1, vn));
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) vn += __shfl_xor(vn, m, 16);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      km = fmaxf(km, __shfl_xor(km, m));
      vn = fmaxf(vn, __shfl_xor(vn, m));
    }
    if ((threadIdx.x & 63) == 0) {
      max_u32(g + 3, __float_as_uint(km));
      max_u32(g + 4, __float_as_uint(vn));
    }
    return;
  }
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, t, hq) flat
  float acc = 0.f, qm = 0.f, dm = 0.f, dn = 0.f;
  u32x4 qw = {0u, 0u, 0u, 0u}, dw = {0u, 0u, 0u, 0u};
  if (row < nrows) {
    const u32x4 ow = *(const u32x4*)((const __bf16*)a.o + row * D + 8 * li);
    dw = *(const u32x4*)((const __bf16*)a.dout + row * D + 8 * li);
    qw = *(const u32x4*)((const __bf16*)a.q + row * D + 8 * li);
    u32x4 lw = {0u, 0u, 0u, 0u};
    if (a.o_lo) lw = *(const u32x4*)((const __bf16*)a.o_lo + row * D + 8 * li);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float d0 = __uint_as_float(dw[k] << 16), d1 = __uint_as_float(dw[k] & 0xffff0000u);
      const float o0 = __uint_as_float(ow[k] << 16) + __uint_as_float(lw[k] << 16);
      const float o1 = __uint_as_float(ow[k] & 0xffff0000u) + __uint_as_float(lw[k] & 0xffff0000u);
      acc = fmaf(o0, d0, acc);
      acc = fmaf(o1, d1, acc);
      dn = fmaf(d0, d0, fmaf(d1, d1, dn));
    }
    qm = absmax8(qw);
    dm = absmax8(dw);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    acc += __shfl_xor(acc, m, 16);
    dn += __shfl_xor(dn, m, 16);
    qm = fmaxf(qm, __shfl_xor(qm, m, 16));
    dm = fmaxf(dm, __shfl_xor(dm, m, 16));
  }
  const int qe = pow2_exponent(qm);
  const int fe = pow2_exponent(dm);
  float bn = 0.f, bd = 0.f;  // |dO| 2^e, |Delta| 2^e of this lane's row
  unsigned fb = 0u;          // f + kExpBias of a row with dO != 0, else 0
  if (row < nrows) {
    bn = __builtin_amdgcn_ldexpf(sqrtf(dn), qe);
    bd = __builtin_amdgcn_ldexpf(fabsf(acc), qe);
    fb = dm > 0.f ? (unsigned)(fe + kExpBias) : 0u;
    *(u32x4*)((uint16_t*)a.q16 + row * D + 8 * li) = f16_scaled(qw, qe);
    *(u32x4*)((uint16_t*)a.do16 + row * D + 8 * li) = f16_scaled(dw, fe);
    if (li == 0) {
      const int hq = (int)(row % a.Hq);
      const int64_t bt = row / a.Hq;
      const int t = (int)(bt % a.Lq);
      const int b = (int)(bt / a.Lq);
      const int64_t o = ((int64_t)b * a.Hq + hq) * a.Lq + t;
      a.delta[o] = acc;
      a.qscale[o] = __builtin_amdgcn_ldexpf(1.f, qe);
      a.doexp[o] = (float)fe;
    }
  }
#pragma unroll
  for (int m = 16; m < 64; m <<= 1) {
    bn = fmaxf(bn, __shfl_xor(bn, m));
    bd = fmaxf(bd, __shfl_xor(bd, m));
    fb = max(fb, (unsigned)__shfl_xor((int)fb, m));
  }
  if ((threadIdx.x & 63) == 0) {
    max_u32(g, __float_as_uint(bn));
    max_u32(g + 1, __float_as_uint(bd));
    max_u32(g + 2, fb);
  }
}

// The fp16 copy of K read by the dQ kernel: K / 2^gK with max |k| / 2^gK in [1, 2) over
// the launch (one scale, so the dQ product needs no per-key factor).
__global__ __launch_bounds__(256) void bwd_k16_kernel(BwdArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int li = threadIdx.x & 15;
  if (row >= (int64_t)a.B * a.Lk * a.Hkv) return;
  const int ge = pow2_exponent(a.maxima[3]);
  const u32x4 kw = *(const u32x4*)((const __bf16*)a.k + row * D + 8 * li);
  *(u32x4*)((uint16_t*)a.k16 + row * D + 8 * li) = f16_scaled(kw, ge);
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

// clears the 8 queue heads of one launch (see claim_item)
__global__ __launch_bounds__(64) void bwd_queue_clear_kernel(int32_t* heads) {
  if (threadIdx.x < 8) heads[threadIdx.x] = 0;
}

// ------------------------------------------------------------------------ dQ
constexpr int QBK = 64;          // keys per tile
constexpr int QTL = QBK * D;     // elements per K or V tile (16 KB)

// One work item = (KV head, q-block of 128 rows), 4 waves x 32 rows; each lane owns one
// query row (column of the transposed products) and keeps its Q (fp16) and dO fragments
// in AGPRs as the B operands of S^T and dP^T, whose accumulators are VGPRs.  The item
// walks its row list as 64-key tiles (two per listed 128-key block).  Sized for two work
// groups per CU (64 KB of LDS, at most 256 registers per wave), so each SIMD holds two
// waves and interleaves one wave's MFMAs with the other's VALU work and LDS reads; the
// compiler schedules the products (a hand-pipelined one-wave-per-SIMD version with 96 KB
// of LDS took about 2.5% longer).  Per tile t (K(t), V(t) resident in buffer t % 2, the
// direct copies of tile t + 1 in flight into the other): for each 32-key half, S^T = K Q^T
// (fp16) and dP^T = V dO^T (bf16), then P and dS on the VALU, then dQ^T += K^T dS^T (fp16)
// with K^T read by ds_read_b64_tr_b16 from the row-major tile.
// MALA (the backward of cowa_mala_fwd with its tile decisions held fixed): dP is taken as
// 0 on the 64-key tiles the forward skipped for the row's forward q-block (a.mala_mask),
// so dS = -P Delta there.
template <bool MALA>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16384))) __bf16 sK0[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sK1[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sV0[QTL];
  __shared__ __attribute__((aligned(16384))) __bf16 sV1[QTL];
  auto kbuf = [&](auto c) -> __bf16* {
    if constexpr ((decltype(c)::value & 1) == 0) return sK0;
    else return sK1;
  };
  auto vbuf = [&](auto c) -> __bf16* {
    if constexpr ((decltype(c)::value & 1) == 0) return sV0;
    else return sV1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h2 = lane >> 5;
  __shared__ int sItem;
  const int item = take_item(a.row_order, a.Hkv * a.nqb, a.queues, &sItem);
  if (item < 0) return;
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int G = a.G, Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const uint16_t* Q16 = (const uint16_t*)a.q16;
  const uint16_t* K16 = (const uint16_t*)a.k16;
  const __bf16* V = (const __bf16*)a.v;
  const __bf16* dO = (const __bf16*)a.dout;

  // key rows past Lk keep what LDS held: cleared once, they only hold zeros or earlier
  // finite rows, which the mask hides
#pragma unroll
  for (int i = 0; i < QTL / (256 * 8); ++i) {
    const int o = 8 * (tid + 256 * i);
    store16(sK0 + o, zero_bf16x8());
    store16(sK1 + o, zero_bf16x8());
    store16(sV0 + o, zero_bf16x8());
    store16(sV1 + o, zero_bf16x8());
  }
  __syncthreads();

  // this lane's query row and its constants (as in bwd_dq_kernel)
  const int r = wave * 32 + n;
  const int rt = r / G;
  const int t = qb * Bq + rt;
  const int hq = h * G + (r - rt * G);
  const bool rvalid = (rt < Bq) && (t < a.Lq);
  const int p = t + off;
  const int gk = pow2_exponent(a.maxima[3]);
  float lse2 = INFINITY, dlt = 0.f, crow = __builtin_amdgcn_ldexpf(a.scale_log2, gk), fq = 1.f, tq = 0.f;
  float dq_out = 0.f;
  bf16x8 qf[8], df[8];
  if (rvalid) {
    const int64_t ri = ((int64_t)b * a.Hq + hq) * a.Lq + t;
    lse2 = a.lse[ri] * kLog2e;
    dlt = a.delta[ri];
    crow *= a.qscale[ri];
    const int64_t ro = (((int64_t)b * a.Lq + t) * a.Hq + hq) * D + 8 * h2;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      qf[dd] = load16(Q16 + ro + 16 * dd);
      df[dd] = load16(dO + ro + 16 * dd);
    }
  } else {
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) qf[dd] = df[dd] = zero_bf16x8();
  }
  {
    float dn = 0.f;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const u32x4 w = __builtin_bit_cast(u32x4, df[dd]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d0 = __uint_as_float(w[q] << 16), d1 = __uint_as_float(w[q] & 0xffff0000u);
        dn = fmaf(d0, d0, fmaf(d1, d1, dn));
      }
    }
    dn += __shfl_xor(dn, 32);
    const float bound = sqrtf(dn) * sqrtf(a.maxima[4]) + fabsf(dlt);
    const int se = bound > 0.f ? min(100, max(-100, 13 - pow2_exponent(bound))) : 0;
    fq = __builtin_amdgcn_ldexpf(1.f, se);
    tq = dlt * fq;
    dq_out = __builtin_amdgcn_ldexpf(a.scale, gk - se);
  }
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) asm volatile("" : "+a"(qf[dd]), "+a"(df[dd]));
  if (lse2 == -INFINITY) lse2 = INFINITY;

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);
  const int ofs_a0 = lds_swz(n, 8 * h2);
  const int ofs_t0[2] = {lds_swz(vrow, vcol), lds_swz(vrow + 8, vcol)};
  auto ofs_a = [&](int k2, int dd) { return 4096 * k2 + (ofs_a0 ^ (dd << 4)); };
  auto ofs_t = [&](int k2, int hf, int pp, int db) { return 2048 * (2 * k2 + hf) + (ofs_t0[pp] ^ (db << 5)); };

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
  auto tile_j0 = [&](int ent, int tt) { return (ent >> 1) * BK + (tt & 1) * QBK; };
  const int64_t kv_bytes = (int64_t)a.Lk * HkvD * 2;
  const char* const kbase = (const char*)(K16 + (int64_t)b * a.Lk * HkvD);
  const char* const vbase = (const char*)(V + (int64_t)b * a.Lk * HkvD);
  auto copy_tile = [&](int ent, int tt, __bf16* kd, __bf16* vd) {
    const int64_t o = (int64_t)tile_j0(ent, tt) * (HkvD * 2);
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, kv_bytes, o, true);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase, kv_bytes, o, true);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      buf2lds(rk, voff[u], kd + (16 * wave + 4 * u) * D);
      buf2lds(rv, voff[u], vd + (16 * wave + 4 * u) * D);
    }
  };

  if (n_ent > 0) {
    const __amdgpu_buffer_rsrc_t r_ent = make_rsrc(a.row_ent + e0, (int64_t)n_ent * 4);
    int ent_cur = load_uniform(a.row_ent, e0);  // entry of tile tt
    int ent_nxt = ent_cur;                      // entry of tile tt + 1
    int ent_ahead = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * 1, 0);  // of tile 2
    copy_tile(ent_cur, 0, sK0, sV0);
    // MALA: this row's keep flags by 64-key block (of its forward q-block), the one of
    // tile tt + 1 fetched during tile tt
    const uint8_t* mrow = nullptr;
    int flag_cur = 1, flag_nxt = 1;
    if constexpr (MALA) {
      mrow = a.mala_mask + ((int64_t)h * a.mala_nqb + (rvalid ? t / a.mala_bq : 0)) * a.mala_nkb;
      flag_cur = mrow[min(tile_j0(ent_cur, 0) / QBK, a.mala_nkb - 1)];
    }

    auto tile = [&](auto bufc, const int tt) {
      constexpr int BUF = decltype(bufc)::value;
      wait_loads_and_barrier();  // tile tt resident; every wave is done with tile tt - 1
      const int64_t o_n = (int64_t)tile_j0(ent_nxt, tt + 1) * (HkvD * 2);
      const __amdgpu_buffer_rsrc_t rk_n = tile_rsrc(kbase, kv_bytes, o_n, tt + 1 < ntile);
      const __amdgpu_buffer_rsrc_t rv_n = tile_rsrc(vbase, kv_bytes, o_n, tt + 1 < ntile);
      __bf16* const kd_n = kbuf(IC<BUF ^ 1>{});
      __bf16* const vd_n = vbuf(IC<BUF ^ 1>{});
      if constexpr (MALA) {
        // (a last half past Lk holds no key: any flag serves, the clamp keeps it in bounds)
        if (tt + 1 < ntile) flag_nxt = mrow[min(tile_j0(ent_nxt, tt + 1) / QBK, a.mala_nkb - 1)];
      }
      const __bf16* kt = kbuf(IC<BUF>{});
      const __bf16* vt = vbuf(IC<BUF>{});
      const int j0 = tile_j0(ent_cur, tt);
      const bool partial = ent_cur & 1;
      // MALA: the dP factor of the dS constant is 0 on a skipped tile.  The products
      // themselves all run: the VALU reads each result only after the products that
      // follow it in this interleaved order, and leaving some out would remove that
      // distance.
      const float fqt = MALA ? (flag_cur ? fq : 0.f) : fq;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        // the K and V operands are read two steps ahead of their products (a ring of
        // three), in an order the fences hold: read just before its product, each one
        // would wait for the LDS latency with the matrix core idle
        f32x16 sv, dv;
        bf16x8 ka[3], va[3];
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
          ka[dd] = load16(kt + ofs_a(k2, dd));
          va[dd] = load16(vt + ofs_a(k2, dd));
        }
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          __builtin_amdgcn_sched_barrier(0);
          if (dd + 2 < 8) {
            ka[(dd + 2) % 3] = load16(kt + ofs_a(k2, dd + 2));
            va[(dd + 2) % 3] = load16(vt + ofs_a(k2, dd + 2));
          }
          if (k2 == 0 && (dd & 1) == 0) {
            const int u = dd >> 1;
            buf2lds(rk_n, voff[u], kd_n + (16 * wave + 4 * u) * D);
            buf2lds(rv_n, voff[u], vd_n + (16 * wave + 4 * u) * D);
          }
          if (dd == 0) {
            mfma_f16_va0(sv, ka[0], qf[0]);
            mfma_bf16_va0(dv, va[0], df[0]);
          } else {
            mfma_f16_va(sv, ka[dd % 3], qf[dd]);
            mfma_bf16_va(dv, va[dd % 3], df[dd]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (partial) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = j0 + 32 * k2 + 8 * (i >> 2) + 4 * h2 + (i & 3);
            sv[i] = (rvalid & visible(p, j, a.Lk, a.win.sink, a.win.near_w, band)) ? sv[i] : -INFINITY;
          }
        }
        uint32_t w[2][4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i0 = 8 * hf + 2 * q;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[i0], crow, -lse2));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[i0 + 1], crow, -lse2));
            w[hf][q] = pack_f16x2(p0 * fmaf(dv[i0], fqt, -tq), p1 * fmaf(dv[i0 + 1], fqt, -tq));
          }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const bf16x8 dsb = __builtin_bit_cast(bf16x8, u32x4{w[hf][0], w[hf][1], w[hf][2], w[hf][3]});
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x8 ka = join(lds_read_tr4(kt + ofs_t(k2, hf, 0, db)), lds_read_tr4(kt + ofs_t(k2, hf, 1, db)));
            acc[db] = mfma32x32x16_f16(ka, dsb, acc[db]);
          }
        }
      }
      // advance the entries (tiles 2 e and 2 e + 1 share entry e): after an even tile the
      // next tile's successor starts a new entry, fetched two tiles ago; after an odd tile
      // it shares the next tile's entry
      ent_cur = ent_nxt;
      flag_cur = flag_nxt;
      if ((tt & 1) == 0) {
        ent_nxt = __builtin_amdgcn_readfirstlane(ent_ahead);
        ent_ahead = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * ((tt >> 1) + 2), 0);
      } else {
        ent_nxt = ent_cur;
      }
    };
    for (int tt = 0; tt < ntile; tt += 2) {
      tile(IC<0>{}, tt);
      tile(IC<1>{}, tt + 1);  // ntile is even
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
  }

  if (rvalid) {
    __bf16* dq = (__bf16*)a.dq + (((int64_t)b * a.Lq + t) * a.Hq + hq) * D + 4 * h2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const bf16x4 v = to_bf16x4(acc[db][4 * q4] * dq_out, acc[db][4 * q4 + 1] * dq_out,
                                   acc[db][4 * q4 + 2] * dq_out, acc[db][4 * q4 + 3] * dq_out);
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

// MALA (the backward of cowa_mala_fwd with its tile decisions held fixed): for the rows
// whose forward tile of this wave's 64 keys was skipped, dP and the P of the dV product
// are taken as 0 (a mask factor per row and key half, staged with the row constants and
// folded into the dS constant f), so dS = -P Delta there and dV gets nothing.
template <bool MALA>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  // row constants per q-block: 4 (CoWA) or 7 (MALA: f and the mask factor per key half)
  constexpr int NLT = MALA ? 7 : 4;
  // Q (fp16 copy) and dO of a q-block, [Q, dO][rows] with swizzled 256-byte rows
  // (lds_swz); dO sits at a fixed distance from Q, so one address serves both.  Two
  // separate arrays (not one indexed by the buffer): every read names the array it reads,
  // so the compiler can tell it apart from the copies in flight into the other one and
  // does not wait for them.
  __shared__ __attribute__((aligned(1024))) __bf16 sQD0[2 * QTILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sQD1[2 * QTILE];
  // per-row constants of a q-block: [LSE log2 e, c_r, 2^e_r, 2^e_r Delta][rows]
  __shared__ __attribute__((aligned(16))) float sLT0[NLT * ROWS];
  __shared__ __attribute__((aligned(16))) float sLT1[NLT * ROWS];
  __shared__ int sRt[ROWS];  // row -> token in the q-block
  __shared__ float sKmax[4];  // max |k| of each wave's keys
  __shared__ float sVmax[4];  // max over each wave's keys of |v_j|^2
  __shared__ float sVabs[4];  // max |v| of each wave's keys
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
  __shared__ int sItem;
  const int item = take_item(a.col_order, a.Hkv * a.nkb, a.queues ? a.queues + 8 : nullptr, &sItem);
  if (item < 0) return;
  const int b = blockIdx.y;
  const int h = item / a.nkb;
  const int kb = item - h * a.nkb;
  const int G = a.G, Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const uint16_t* Q16 = (const uint16_t*)a.q16;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;
  const uint16_t* dO16 = (const uint16_t*)a.do16;

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
  float plse = 0.f, pdel = 0.f, pqs = 1.f, pdx = 0.f, ck = a.scale_log2;
  int pm0 = 1, pm1 = 1;  // MALA: keep flags of the row's forward tiles of the two key halves
  // the dS constant f of this wave's key half, and (MALA) its mask factor, in the row table
  const int f_off = (MALA && wave >= 2) ? 4 * ROWS : 2 * ROWS;
  const int m_off = (wave >= 2) ? 6 * ROWS : 5 * ROWS;
  // dS range scale of this item (2^sc, see below) and the dK output factor scale 2^-sc;
  // the exponent eV of the item's fp16 V; the dV product's common exponent F
  float dsc = 1.f, dk_out = a.scale;
  int ev = 0;
  const unsigned fbias = ((const unsigned*)a.maxima)[2];
  const int fcommon = fbias ? (int)fbias - kExpBias : 0;
  bool pvalid = false;
  // LSE, Delta and Q row scales of this KV head's G query heads, [G, Lq] each
  const int64_t lt_base = ((int64_t)b * a.Hq + h * G) * a.Lq;
  const __amdgpu_buffer_rsrc_t r_lse = make_rsrc(a.lse + lt_base, (int64_t)G * a.Lq * 4);
  const __amdgpu_buffer_rsrc_t r_del = make_rsrc(a.delta + lt_base, (int64_t)G * a.Lq * 4);
  const __amdgpu_buffer_rsrc_t r_qs = make_rsrc(a.qscale + lt_base, (int64_t)G * a.Lq * 4);
  const __amdgpu_buffer_rsrc_t r_dx = make_rsrc(a.doexp + lt_base, (int64_t)G * a.Lq * 4);

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
  const char* const dobase = (const char*)(dO16 + (int64_t)b * a.Lq * HqD);
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
      pdx = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_dx, vo, 0, 0));
      if constexpr (MALA) {
        const int tok = min(t0 + my_rt, a.Lq - 1);
        const uint8_t* mr = a.mala_mask + ((int64_t)h * a.mala_nqb + tok / a.mala_bq) * a.mala_nkb;
        pm0 = 2 * kb < a.mala_nkb ? mr[2 * kb] : 0;
        pm1 = 2 * kb + 1 < a.mala_nkb ? mr[2 * kb + 1] : 0;
      }
    }
  };
  auto copy = [&](int i, auto bufc) {
    __bf16* dst = tiles(bufc) + wave * 32 * D + 4 * (i >> 1) * D + ((i & 1) ? QTILE : 0);
    buf2lds((i & 1) ? rd_n : rq_n, voff_u[i >> 1], dst);
  };
  // Rows with no token or no visible key: LSE +inf (P = 0), c_r > 0 (so that a masked
  // S = -inf still gives P = 0), and 0 for the dS scale and Delta.  ck = scale log2(e)
  // 2^e_K.
  //
  // The dV and dP products take dO in fp16 (row r divided by 2^f_r, f_r from doexp) and V
  // in fp16 (divided by 2^eV per item), so dP16 = dP 2^-(f_r + eV), and P enters dV as
  // P16 = P 2^e_r' with e_r' = min(f_r - F, 0) (F the largest f_r: P16 <= 1), which the
  // exp2 takes through its LSE term.  Then dV = 2^F sum P16 dO16, and
  //   dS 2^(e_r + sc) = P16 (dP16 2^(f_r + eV - e_r') - Delta 2^-e_r') 2^(e_r + sc),
  // so the two dS constants become f = 2^(e_r + sc + f_r + eV - e_r'), t = Delta 2^(e_r + sc - e_r').
  auto store_lse = [&](auto bufc) {
    if (tid < ROWS) {
      float* lt = lts(bufc);
      const int fr = (int)pdx;
      const int er = min(fr - fcommon, 0);
      lt[tid] = (pvalid && plse != -INFINITY) ? plse * kLog2e - (float)er : INFINITY;
      lt[ROWS + tid] = pvalid ? ck * pqs : ck;
      const float fv = pvalid ? __builtin_amdgcn_ldexpf(pqs * dsc, fr + ev - er) : 0.f;
      if constexpr (MALA) {
        const float m0 = pm0 ? 1.f : 0.f, m1 = pm1 ? 1.f : 0.f;
        lt[2 * ROWS + tid] = fv * m0;
        lt[4 * ROWS + tid] = fv * m1;
        lt[5 * ROWS + tid] = m0;
        lt[6 * ROWS + tid] = m1;
      } else {
        lt[2 * ROWS + tid] = fv;
      }
      lt[3 * ROWS + tid] = pvalid ? __builtin_amdgcn_ldexpf(pdel * (pqs * dsc), -er) : 0.f;
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
      float km = 0.f, vm = 0.f;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        km = fmaxf(km, absmax8(__builtin_bit_cast(u32x4, kf[dd])));
        vm = fmaxf(vm, absmax8(__builtin_bit_cast(u32x4, vf[dd])));
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        km = fmaxf(km, __shfl_xor(km, m));
        vm = fmaxf(vm, __shfl_xor(vm, m));
      }
      if (lane == 0) {
        sKmax[wave] = km;
        sVabs[wave] = vm;
      }
      // |v_j|^2 of this lane's key (the two lane halves hold 64 dimensions each), max
      // over the wave's 32 keys
      float vn = 0.f;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const u32x4 w = __builtin_bit_cast(u32x4, vf[dd]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = __uint_as_float(w[q] << 16), v1 = __uint_as_float(w[q] & 0xffff0000u);
          vn = fmaf(v0, v0, fmaf(v1, v1, vn));
        }
      }
      vn += __shfl_xor(vn, 32);
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) vn = fmaxf(vn, __shfl_xor(vn, m));
      if (lane == 0) sVmax[wave] = vn;
    }
    wait_loads_and_barrier();
    {
      const int ek = pow2_exponent(fmaxf(fmaxf(sKmax[0], sKmax[1]), fmaxf(sKmax[2], sKmax[3])));
      ck = a.scale_log2 * __builtin_amdgcn_ldexpf(1.f, ek);
      ev = pow2_exponent(fmaxf(fmaxf(sVabs[0], sVabs[1]), fmaxf(sVabs[2], sVabs[3])));
      // dS enters the dK product as dS 2^e_r 2^sc in fp16, with 2^sc chosen per item so
      // that the bound |dO_i| 2^e_r |v|max + |Delta_i| 2^e_r (launch-wide row maxima from
      // the Delta kernel, |v|max over this item's keys) is below 2^14, four times inside
      // the fp16 range; dK is multiplied by 2^-sc at the end.  The scale is a power of
      // two, so it changes no value beyond the fp16 rounding it protects.
      const float vmax = sqrtf(fmaxf(fmaxf(sVmax[0], sVmax[1]), fmaxf(sVmax[2], sVmax[3])));
      const float bound = a.maxima[0] * vmax + a.maxima[1];
      const int sc = bound > 0.f ? min(100, max(-100, 13 - pow2_exponent(bound))) : 0;
      dsc = __builtin_amdgcn_ldexpf(1.f, sc);
      dk_out = a.scale * __builtin_amdgcn_ldexpf(1.f, -sc);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        kf[dd] = bf16_to_f16_scaled(kf[dd], ek);
        vf[dd] = bf16_to_f16_scaled(vf[dd], ev);
        asm volatile("" : "+a"(kf[dd]), "+a"(vf[dd]));
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
        wA.dp = mfma32x32x16_f16(load16(sQD0 + QTILE + ofs_a(dd)), vf[dd], wA.dp);
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
      wA.f0 = *(const f32x4*)(lt + f_off);
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
      f32x16 sn;
      f32x4 f4[4], t4[4], l4[4], c4[4];
      f4[0] = cur.f0;
      t4[0] = cur.t0;
      f32x4 mk[4];  // MALA: mask factors of block g's rows for this wave's key half
      if constexpr (MALA) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) mk[i4] = *(const f32x4*)(lg + m_off + 8 * i4);
      }
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
        else if (x == 1) mfma_f16_va0(nxt.dp, da[0], vf[0]);
        else if (x & 1) mfma_f16_va(nxt.dp, da[dd], vf[dd]);
        else mfma_f16_va(sn, qa[dd], kf[dd]);
        if ((x & 1) && dd + 4 < 8) {
          qa[dd + 4] = load16(t1 + ofs_a(dd + 4));
          da[dd + 4] = load16(t1 + QTILE + ofs_a(dd + 4));
        }
        // copies of the next q-block: 8 in each of the first two steps, one every 2 MFMAs
        // (here rather than beside the phase-2 products, whose slots carry the transposed
        // reads)
        if constexpr (RB < 2)
          if (x & 1) copy(8 * RB + (x >> 1), IC<BUF ^ 1>{});
        // transposed operands of half 0 for phase 2 (dO^T at slot 4 db, Q^T at 4 db + 2),
        // one pair every other slot: issued together before the first product they made
        // a burst of 20 LDS reads, more than the wait counter tracks, and the first
        // product waited for ten of them
        if ((x & 1) == 0) {
          const int db = x >> 2;
          if ((x & 2) == 0) dt[0][db] = join(lds_read_tr4(tg + QTILE + ofs_t(0, db)), lds_read_tr4(tg + QTILE + ofs_t(1, db)));
          else qt[0][db] = join(lds_read_tr4(tg + ofs_t(0, db)), lds_read_tr4(tg + ofs_t(1, db)));
        }
        // dS constants of groups 1..3, four slots before their first use; P constants of
        // the next block's group 0, for phase 2
        if ((x & 3) == 0 && x < 12) {
          const int i4 = (x >> 2) + 1;
          f4[i4] = *(const f32x4*)(lg + f_off + 8 * i4);
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
          if constexpr (MALA)
            wpa[q >> 2][q & 3] = pack_f16x2(prv[(x - 1) % 3] * mk[(x - 1) >> 2][(x - 1) & 3],
                                            prv[x % 3] * mk[x >> 2][x & 3]);
          else
            wpa[q >> 2][q & 3] = pack_f16x2(prv[(x - 1) % 3], prv[x % 3]);
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
        else accV[db] = mfma32x32x16_f16(pa[hf], dt[hf][db], accV[db]);
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
        // P constants of groups 1..3, four slots ahead; the next step's first dS constants
        if ((x & 3) == 0 && x < 12) {
          const int i4 = (x >> 2) + 1;
          l4[i4] = *(const f32x4*)(lt + 8 * i4);
          c4[i4] = *(const f32x4*)(lt + ROWS + 8 * i4);
        }
        if (x == 12) {
          nxt.f0 = *(const f32x4*)(lt + f_off);
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

  const float dv_out = __builtin_amdgcn_ldexpf(1.f, fcommon);
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
        dK[o] = (__bf16)(accK[db][i] * dk_out);
        dV[o] = (__bf16)(accV[db][i] * dv_out);
      }
    }
}

// MALA: the forward's keep flags (one per entry of its row lists) as a dense mask
// [Hkv * nqb_f, nkb64]: one work group per forward row item scatters its entries (the
// forward's k-blocks are the 64-key blocks); unlisted tiles see no key and stay 0.
__global__ __launch_bounds__(256) void mala_mask_clear_kernel(uint8_t* m, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) m[i] = 0;
}
__global__ __launch_bounds__(256) void mala_mask_kernel(MalaMaskArgs a) {
  const int item = blockIdx.x;
  const int e0 = a.row_ptr[item], e1 = a.row_ptr[item + 1];
  for (int e = e0 + (int)threadIdx.x; e < e1; e += 256)
    a.mask[(int64_t)item * a.nkb + (a.row_ent[e] >> 1)] = a.kept[e] ? 1 : 0;
}

}  // namespace

hipError_t launch_mala_mask(const MalaMaskArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_items * a.nkb;
  hipLaunchKernelGGL(mala_mask_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.mask, n);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mala_mask_kernel, dim3(a.n_items), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, int stages, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (stages & COWA_BWD_DELTA) {
    const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
    const int64_t nkv = (int64_t)a.B * a.Lk * a.Hkv;
    hipLaunchKernelGGL(bwd_clear_kernel, dim3(1), dim3(64), 0, s, a.maxima);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((nrows + 15) / 16 + (nkv + 15) / 16)), dim3(256),
                       0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_k16_kernel, dim3((unsigned)((nkv + 15) / 16)), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // grid: every item, plus spare work groups when the queues are in use
  auto grid = [&](int n) { return dim3((unsigned)(a.queues ? n + n / 16 + 8 : n), a.B); };
  if (stages & COWA_BWD_DQ) {
    if (a.queues) {
      hipLaunchKernelGGL(bwd_queue_clear_kernel, dim3(1), dim3(64), 0, s, a.queues);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (a.mala_mask) hipLaunchKernelGGL(bwd_dq_kernel<true>, grid(a.Hkv * a.nqb), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(bwd_dq_kernel<false>, grid(a.Hkv * a.nqb), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (stages & COWA_BWD_DKDV) {
    if (a.queues) {
      hipLaunchKernelGGL(bwd_queue_clear_kernel, dim3(1), dim3(64), 0, s, a.queues + 8);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (a.mala_mask) hipLaunchKernelGGL(bwd_dkdv_kernel<true>, grid(a.Hkv * a.nkb), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(bwd_dkdv_kernel<false>, grid(a.Hkv * a.nkb), dim3(256), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return err;
}

}  // namespace cowa
