// CoWindow Attention forward, bf16 in/out, head dim 128, for gfx950.
//
// One work item = (KV head h, q-block of Bq = 256 / G tokens): the query rows of the G
// query heads that share KV head h (slinene.github.io ai-papers-daily page, method key
// point 3: windows follow the KV head, so one K/V tile read from HBM serves all G query
// heads).  Rows are token-major (row r = token * G + head-in-group), so the item's Q is
// one strided run of G * 256 bytes per token.  Four waves own 64 rows each, as two
// 32-column blocks of v_mfma_f32_32x32x16_bf16.
//
// The item walks the planner's row list of visible 64-key blocks (masked blocks are
// never touched).  Three products run as a software pipeline, one block t per loop
// iteration of 64 MFMA slots:
//   [A] S(t+1)^T = K(t+1) Q^T on the even slots: K (A operand, one key row per lane) and
//       Q^T (B operand) from LDS, so each lane owns one query row (column) and 16 of every
//       32 keys.  Its accumulators are VGPRs: the softmax reads them as plain VALU
//       operands (reading accumulation registers while the matrix core runs costs several
//       cycles per value);
//   [B] online softmax of S(t) in base 2 (scale * log2 e folded into one FMA), one
//       element per slot beside the MFMAs; a boundary (PARTIAL) block is masked first
//       (each row's visible keys as one run where they form one, else the window
//       predicate per element);
//   [C] O^T += V(t-1)^T P(t-1)^T on the odd slots: P^T goes from the softmax registers
//       straight into the B operand (no LDS round trip) and V^T is read from the
//       row-major LDS tile with ds_read_b64_tr_b16, two 4-key runs per operand matching
//       the accumulator layout.  O stays in the accumulation registers.
// Reference: the result O / l does not depend on the value m subtracted before exp2, so
// no running max is kept.  The first tile sets m to its column max; later tiles keep it
// unless a column's sum over the tile leaves [2^-32, 2^32] (the low bound only while
// the column has no mass yet), when the tile's column max replaces it and O, l follow.
// With P <= 2^32 and at most 2^31 keys, O and l stay finite in fp32.
//
// Memory pipeline: K and V are double-buffered in LDS and filled by direct buffer->LDS
// copies (no staging registers), spread over the MFMA slots: K(t+2) and V(t) are copied
// during block t and waited for at the next block's single barrier.  LDS rows are 256
// bytes with the 16-byte chunks XOR-swizzled by a function of the row, so both the
// row-wise operand reads and the transposed V reads are free of bank conflicts, and the
// addresses of one lane differ only in the XOR of the chunk bits.
// Output: O / l in bf16 and LSE = ln 2 * (m + log2 l) in fp32; optionally the part of
// the fp32 O that the bf16 rounding drops (O - bf16(O), rounded to bf16), from which the
// backward forms Delta = dO . O to about 16 significant bits.
//
// MFMA lane layouts of v_mfma_f32_32x32x16_bf16 (n = lane % 32, h2 = lane / 32):
//   A (32 x 16): A[n][8 h2 + e]   B (16 x 32): B[8 h2 + e][n]
//   C (32 x 32): element i of 16 is C[8 (i / 4) + 4 h2 + i % 4][n]

#include <type_traits>

#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 128;
constexpr int WAVES = 4;
constexpr int ROWS = kFwdRows;       // 256 rows per item
constexpr int WROWS = ROWS / WAVES;  // 64 rows per wave
constexpr int CB = WROWS / 32;       // 2 column blocks of 32 per wave
constexpr int BK = kFwdBk;           // 64 keys per tile
constexpr int KB2 = BK / 32;         // 2 key blocks of 32
constexpr int TILE = BK * D;         // elements per K or V tile

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<B>), f(IC<B+1>), ..., f(IC<E-1>): straight-line code with a compile-time index,
// whatever the size of the body
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

// LDS tiles: 256-byte rows with XOR-swizzled 16-byte chunks (lds_sw / lds_swz).
__device__ __forceinline__ int sw(int r) { return lds_sw(r); }
__device__ __forceinline__ int swz(int r, int e) { return lds_swz(r, e); }

// x * alpha for a value held in an accumulation register, done in place: read to a VGPR,
// multiply, write back.  Only used on the rare rescale path, long after the MFMA that
// last wrote the register (a whole tile of LDS reads and MFMAs lies in between).
__device__ __forceinline__ float agpr_scale(float x, float alpha) {
  float t;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(x));
  t *= alpha;
  float r;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(r) : "v"(t));
  return r;
}

// Fences a result at this point of the program: it must be complete here, so its
// computation stays in the slot that produced it.
__device__ __forceinline__ void pin_out(bf16x8& x) { asm volatile("" : "+v"(x)); }

// S products with their accumulators in VGPRs: the softmax reads S with plain VALU
// operands (a read of an accumulation register costs several cycles while the matrix
// core runs).  Every S accumulator is read by the VALU a block after its last product,
// and each chain has three other products between dependent steps, so these need no
// wait states beyond what the matrix core itself enforces; their LDS operands carry the
// compiler's usual waits.
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// the same with the B operand in AGPRs (the Q^T fragments, resident for the whole item)
__device__ __forceinline__ void mfma_va(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_va0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}


// MODE 0: the CoWA forward.  MODE 1: scoring only (no PV): LSE over every visible key,
// and per tile and row the log2 of the row's probability numerator in the tile (the
// tile's row sum in the reference then in use, plus that reference), from which
// mala_decide_kernel finds each tile's largest row mass once the LSE is known.
// MODE 2: the MALA pass over the kept tiles only, given that LSE: P = exp(scale s - LSE)
// exactly normalised, O = sum of the kept P V (no division), LSE left as it is.
template <int MODE>
__global__ __launch_bounds__(256, 1) void fwd_bf16_d128_kernel(FwdArgs a) {
  // K and V double buffers, one array per buffer: the tile parity is known at compile
  // time in each of the two unrolled iterations, so every read names the array it reads
  // and the compiler can tell it from the copies in flight into the other one.  They
  // come first in LDS, so that every operand address of the loop is a per-lane base plus
  // an offset that fits the 16-bit offset field of the LDS reads.
  __shared__ __attribute__((aligned(16384))) __bf16 sK0[TILE];
  __shared__ __attribute__((aligned(16384))) __bf16 sK1[TILE];
  __shared__ __attribute__((aligned(16384))) __bf16 sV0[TILE];
  __shared__ __attribute__((aligned(16384))) __bf16 sV1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sQ[ROWS * D];
  auto kbuf = [&](auto c) __attribute__((always_inline)) -> __bf16* {
    if constexpr ((decltype(c)::value & 1) == 0) return sK0;
    else return sK1;
  };
  auto vbuf = [&](auto c) __attribute__((always_inline)) -> __bf16* {
    if constexpr ((decltype(c)::value & 1) == 0) return sV0;
    else return sV1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int n = lane & 31;
  const int h2 = lane >> 5;
  __shared__ int sItem;
  const int item = take_item(a.row_order, a.n_items, a.queues, &sItem);
  if (item < 0) return;
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int G = a.G;
  const int Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;

  // Key rows past Lk are outside the copies' range and keep what LDS held: cleared once
  // here, they only ever hold zeros or earlier finite rows (their scores are masked).
#pragma unroll
  for (int i = 0; i < TILE / (256 * 8); ++i) {
    store16(sK0 + 8 * (tid + 256 * i), zero_bf16x8());
    store16(sK1 + 8 * (tid + 256 * i), zero_bf16x8());
    store16(sV0 + 8 * (tid + 256 * i), zero_bf16x8());
    store16(sV1 + 8 * (tid + 256 * i), zero_bf16x8());
  }
  __syncthreads();

  int tok[CB], hq[CB];
  bool rvalid[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int r = wave * WROWS + c * 32 + n;
    const int rt = r / G;
    tok[c] = qb * Bq + rt;
    hq[c] = h * G + (r - rt * G);
    rvalid[c] = (rt < Bq) && (tok[c] < a.Lq);
  }

  // ---- direct loads.  Lane L of a 1 KB copy fills row r = 4 * blk + L / 16, physical
  // chunk L % 16, so it fetches logical chunk (L % 16) ^ sw(r) of that row.
  const int lrow = lane >> 4;
  const int lchunk = lane & 15;
  {  // this wave's 64 query rows (rows past the q-block or Lq read a valid row; unused)
    __bf16* dst = sQ + wave * WROWS * D;
#pragma unroll
    for (int u = 0; u < WROWS / 4; ++u) {
      const int r = wave * WROWS + 4 * u + lrow;
      const int rt = r / G;
      int t = qb * Bq + rt;
      int g = r - rt * G;
      if (rt >= Bq || t >= a.Lq) {
        t = min(qb * Bq, a.Lq - 1);
        g = 0;
      }
      const int c = lchunk ^ sw(r);
      g2lds(Q + (((int64_t)b * a.Lq + t) * a.Hq + h * G + g) * D + 8 * c, dst + 4 * u * D);
    }
  }
  // K / V tile copies: wave w fills rows 16 w .. 16 w + 15, 4 rows per copy; lane L of
  // copy u fills row r = 16 w + 4 u + L / 16 at physical chunk L % 16.  voff[u] is the
  // byte offset of its source chunk from the tile's first key.  A tile is read through a
  // buffer resource ending at key Lk (keys past Lk read nothing; they are masked), or
  // with an empty range when the tile does not exist, so the copies need no branches and
  // can be spread over the MFMA slots of the interleaved block.
  const int HkvD = a.Hkv * D;
  uint32_t voff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * wave + 4 * u + lrow;
    voff[u] = 2u * (uint32_t)(r * HkvD + h * D + 8 * (lchunk ^ sw(r)));
  }
  // The batch's base is formed once per item; per tile only the offset and the tile's
  // row count remain on the scalar unit.
  const int tile_bytes = BK * HkvD * 2;
  const char* const kbase = (const char*)(K + (int64_t)b * a.Lk * HkvD);
  const char* const vbase = (const char*)(V + (int64_t)b * a.Lk * HkvD);
  // resource over the BK rows of tile ent (fewer at the end of the sequence, none when
  // !real): the copies only read inside their tile, so the range needs no 64-bit
  // arithmetic beyond the tile's base
  const int row_bytes = HkvD * 2;
  auto tile_copy_rsrc = [&](const char* base, int ent, bool real) __attribute__((always_inline)) {
    const int kb = ent >> 1;
    const int rows = min(a.Lk - kb * BK, BK);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kb * tile_bytes), (short)0,
                                             real ? rows * row_bytes : 0, 0x00020000);
  };
  auto copy_tile = [&](__amdgpu_buffer_rsrc_t r, int u, __bf16* dst) __attribute__((always_inline)) {
    buf2lds(r, voff[u], dst + (16 * wave + 4 * u) * D);
  };

  f32x16 acc[CB][4];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][db][i] = 0.f;
  // m: the reference subtracted from the scaled scores (base 2) before exp2, per column;
  // l: this lane's share of the column's row sum in that reference
  float m[CB], l[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    m[c] = 0.f;
    l[c] = 0.f;
  }

  const int e0 = a.row_ptr[item];
  // MALA pass: the item's kept entries, compacted at the same offsets
  const int nt = MODE == 2 ? a.mala_counts[(int64_t)b * a.n_items + item] : a.row_ptr[item + 1] - e0;
  const int32_t* const ents = MODE == 2 ? a.mala_ents + (int64_t)b * a.mala_nnz : a.row_ent;
  // LDS addressing.  With the chunk swizzle, the operand addresses of one lane differ
  // only by an XOR of the chunk bits, so each is one XOR away from a per-lane base:
  //   K / Q rows n of a tile at dd: kofs0 ^ (dd << 5) bytes (+ 8192 for key / row block 1);
  //   V^T operand (k2, hf, db), first and second run of 4 rows:
  //     vofs0 ^ (db << 6) and (vofs0 ^ (db << 6) ^ 32) + 2048, + 4096 (2 k2 + hf) bytes,
  // where 16-lane group gg covers d columns 16 (gg & 1) .. +15 of a 32-column block and
  // key run 4 (gg >> 1) (+8).
  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);
  const uint32_t kofs0 = 2u * (uint32_t)swz(n, 8 * h2);
  const uint32_t qofs0 = kofs0 + 2u * (uint32_t)(wave * WROWS * D);
  const uint32_t vofs0 = 2u * (uint32_t)swz(vrow, vcol);
  auto at = [](const __bf16* base, uint32_t byte_ofs) __attribute__((always_inline)) {
    return (const __bf16*)((const char*)base + byte_ofs);
  };

  // The Q^T operands of this wave's rows (B operands of every S product), read once from
  // the Q tile after its copies land and kept in AGPRs: the products then read only K
  // from LDS.
  bf16x8 qa[CB][D / 16];
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int dd = 0; dd < D / 16; ++dd) {
        qa[c][dd] = load16(at(sQ, (qofs0 ^ (dd << 5)) + 8192 * c));
        asm volatile("" : "+a"(qa[c][dd]));
      }
  };
  auto scores = [&](f32x16 (&s)[KB2][CB]) __attribute__((always_inline)) {  // S of tile 0
    const __bf16* kt = sK0;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
#pragma unroll
      for (int k2 = 0; k2 < KB2; ++k2) {
        const bf16x8 kf = load16(at(kt, (kofs0 ^ (dd << 5)) + 8192 * k2));
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          if (dd == 0) mfma_va0(s[k2][c], kf, qa[c][dd]);
          else mfma_va(s[k2][c], kf, qa[c][dd]);
        }
      }
    }
  };

  // Loop-invariant operand bases: kb[dd] for the K rows at step dd, vb[db][0 / 1] for the
  // first and second run of 4 rows of the V^T operand at column block db.  The loop
  // re-takes (pins) them at the top of every iteration, so each read is one of these
  // registers plus an immediate offset (key block, row group, buffer) and the loop does
  // no address arithmetic.
  uint32_t kb[D / 16], vb[4][2];
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) kb[dd] = kofs0 ^ (uint32_t)(dd << 5);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    vb[db][0] = vofs0 ^ (uint32_t)(db << 6);
    vb[db][1] = (vb[db][0] ^ 32u) + 2048u;
  }
  // tr-read of the V^T operand for (k2, hf, db) from a V tile
  auto vfrag = [&](const __bf16* vt, int k2, int hf, int db) __attribute__((always_inline)) {
    const uint32_t rows = 4096u * (uint32_t)(2 * k2 + hf);
    return join(lds_read_tr4(at(vt, vb[db][0] + rows)), lds_read_tr4(at(vt, vb[db][1] + rows)));
  };

  // Boundary tile, both row blocks: each row's visible keys of the tile as a 64-bit mask
  // over the key offsets jc (key (ent >> 1) BK + 4 h2 + jc; the lane's 32 elements sit at
  // the offsets of kLaneKeys), from the row's single run where its visible keys form one
  // (visible_run, almost every boundary tile of the CoWA windows), else from the window
  // predicate key by key in a loop (narrow windows or gaps); then one select per element,
  // skipped when every row sees the whole tile.  One copy of the select code serves both
  // cases, which keeps the kernel's code small enough for the instruction cache.  Rows
  // without a token (past Lq in the last q-block, which makes every tile of that q-block a
  // boundary tile) see every key: their results are never stored, and masking them
  // entirely would leave their column sums at 0 and send every one of those tiles through
  // the reference move.
  constexpr uint64_t kLaneKeys = 0x0F0F0F0F0F0F0F0Full;  // jc = 32 k2 + 8 (i / 4) + i % 4
  auto mask_tile = [&](f32x16 (&v)[KB2][CB], int ent) __attribute__((always_inline)) {
    if (ent & 1) {
      const int jbase = (ent >> 1) * BK + 4 * h2;
      uint64_t bits[CB];
      bool whole = true;
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        int lo, hi;
        const int p = tok[c] + off;
        const bool one = visible_run(p, jbase, a.Lk, a.win.sink, a.win.near_w, band, lo, hi);
        if (!rvalid[c]) {
          bits[c] = ~0ull;
        } else if (one) {  // keys lo .. hi (none when lo > hi)
          bits[c] = lo > hi ? 0ull : ((hi >= 63 ? ~0ull : (2ull << hi) - 1ull) & ~((1ull << lo) - 1ull));
        } else {
          uint64_t m = 0;
#pragma unroll 1
          for (int jc = 0; jc < BK - 4; ++jc)
            m |= (uint64_t)visible(p, jbase + jc, a.Lk, a.win.sink, a.win.near_w, band) << jc;
          bits[c] = m;
        }
        whole &= (bits[c] & kLaneKeys) == kLaneKeys;
      }
      if (__builtin_amdgcn_ballot_w64(!whole) != 0) {
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int jc = 32 * k2 + 8 * (i >> 2) + (i & 3);
              const float x = v[k2][c][i];
              v[k2][c][i] = ((bits[c] >> jc) & 1ull) ? x : -INFINITY;
            }
      }
    }
  };

  // Reference check.  The softmax is exact for any reference, so P(t) is computed with
  // the current one and the reference only moves when a column's sum over the tile
  // leaves the safe range: above 2^32 (a P near overflow), or below 2^-32 while the
  // column has no mass yet (its first visible keys all far below the reference).  Then
  // the tile's column max becomes the reference and the column's P(t) is recomputed; O
  // and l follow by alpha once O holds the previous tiles.  P <= 2^32 with at most 2^31
  // keys keeps O and l finite in fp32.
  constexpr float kSumHi = 4294967296.0f, kSumLo = 1.0f / 4294967296.0f;
  // the value of the same column in the other half of the wave
  auto swap_halves = [&](float x) __attribute__((always_inline)) {
    const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(h2 == 0 ? sw2[1] : sw2[0]);
  };
  // recompute row block c of P(t) from its scores with reference mr; returns its sum
  auto softmax_rows = [&](const f32x16 (&sc)[KB2][CB], bf16x8 (&pfc)[KB2][CB][2], int c, float mr)
      __attribute__((always_inline)) {
    float sum = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = __builtin_amdgcn_exp2f(fmaf((sc[k2][c][8 * hf + e]), a.scale_log2, -mr));
          sum += pb[e];
        }
        pfc[k2][c][hf] = join(to_bf16x4(pb[0], pb[1], pb[2], pb[3]), to_bf16x4(pb[4], pb[5], pb[6], pb[7]));
      }
    return sum;
  };

  // probabilities x0, x1 rounded to bf16 as one register (two keys of a PV operand)
  auto bf16_pair = [&](float x0, float x1) __attribute__((always_inline)) {
    const bf16x2 h = {(__bf16)x0, (__bf16)x1};
    return __builtin_bit_cast(uint32_t, h);
  };

  // List entries of tiles t .. t+2 are kept in scalar registers; entry t+3 is fetched
  // during iteration t with a vector load (through a resource over this item's entries,
  // so a fetch past the end reads 0) and taken at the top of iteration t+1.  A scalar
  // load would share its wait counter with the LDS operand reads, whose first wait would
  // then also wait for it.
  int ent0 = 0, ent1 = 0, ent2 = 0;
  const __amdgpu_buffer_rsrc_t r_ent = make_rsrc(ents + e0, (int64_t)nt * 4);
  int ent_next = 0;  // entry t+3 in flight (VGPR)

  // Iteration t (parity PAR = t % 2) is one block of 64 MFMA slots:
  //   even slots: S(t+1) = K(t+1) Q^T, four products per 16-wide slice of d;
  //   odd slots:  O^T += V(t-1)^T P(t-1)^T;
  //   VALU, one softmax element of S(t) per slot, read from its accumulator one slot
  //   ahead (row block 0 in slots 0-31, row block 1 in slots 32-63).
  // After the block O holds every tile up to t-1: the reference check runs on the column
  // sums of P(t) (rarely moving a reference and rescaling O), and l takes the sums.
  // Registers: S(t) and S(t+1) take two sets of accumulators (128) beside O (128), all
  // of the accumulation registers; P(t-1) and P(t) alternate the same way.
  // LDS: K(t+1) and V(t-1) are read; K(t+2) and V(t) are copied in meanwhile, into the
  // buffers of K(t) and V(t-2), which every wave finished with in iteration t-1.
  f32x16 sx[2][KB2][CB];
  bf16x8 pf[2][KB2][CB][2];
  auto iteration = [&](auto parity, int t) __attribute__((always_inline)) {
    constexpr int PAR = decltype(parity)::value;
    f32x16(&sc)[KB2][CB] = sx[PAR];      // S(t)
    f32x16(&sn)[KB2][CB] = sx[PAR ^ 1];  // S(t+1)
    bf16x8(&pfc)[KB2][CB][2] = pf[PAR];
    const bf16x8(&pfp)[KB2][CB][2] = pf[PAR ^ 1];
    wait_loads_and_barrier();  // K(t+1), V(t-1) resident; every wave is done with t-1
    const __amdgpu_buffer_rsrc_t rk = tile_copy_rsrc(kbase, ent2, t + 2 < nt);
    const __amdgpu_buffer_rsrc_t rv = tile_copy_rsrc(vbase, ent0, true);
    __bf16* const kdst = kbuf(IC<PAR>{});          // K(t+2)
    __bf16* const vdst = vbuf(IC<PAR>{});          // V(t)
    const __bf16* const kt = kbuf(IC<PAR ^ 1>{});  // K(t+1)
    const __bf16* const vt = vbuf(IC<PAR ^ 1>{});  // V(t-1)
    const int ent3 = __builtin_amdgcn_readfirstlane(ent_next);  // loaded in iteration t-1
    ent_next = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * (t + 4), 0);
    const int ent_t = ent0;  // tile t
    ent0 = ent1;
    ent1 = ent2;
    ent2 = ent3;

    // S(t+1) operands by step dd (four MFMAs, (k2, c)): the K rows of both key blocks at
    // dd (the Q^T columns are resident); step dd + 1 is read during step dd
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) asm volatile("" : "+v"(kb[dd]));
#pragma unroll
    for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(vb[db][0]), "+v"(vb[db][1]));
    bf16x8 kq[2][2];
    auto load_step = [&](int dd, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
      dst[0] = load16(at(kt, kb[dd]));
      dst[1] = load16(at(kt, kb[dd] + 8192u));
    };
    load_step(0, kq[0]);
    bf16x8 vf[3];
    if constexpr (MODE == 0) {
      vf[0] = vfrag(vt, 0, 0, 0);
      vf[1] = vfrag(vt, 0, 0, 1);
    }
    mask_tile(sc, ent_t);

    float sum[CB] = {0.f, 0.f};
    float pb[8];
    uint32_t pw[4];
    // element p of the tile's P into the row sum and, as the second of a pair, into its
    // bf16 PV operand (complete after every eighth element)
    auto fold = [&](auto pi) __attribute__((always_inline)) {
      constexpr int p = decltype(pi)::value, pc = p >> 5, pe = p & 31;
      sum[pc] += pb[p & 7];
      if constexpr (MODE == 1) return;  // scoring only: no PV operand
      if constexpr ((p & 1) == 1) pw[(p & 7) >> 1] = bf16_pair(pb[(p - 1) & 7], pb[p & 7]);
      if constexpr ((p & 7) == 7) {
        bf16x8& dst = pfc[pe >> 4][pc][(pe >> 3) & 1];
        dst = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        pin_out(dst);
      }
    };
    // the block of 64 slots, with (PV = 1) or without (PV = 0) the O^T += V^T P^T products
    auto slots = [&](auto pvc) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pvc)::value != 0;
    if constexpr (PV && MODE == 2) {
      vf[0] = vfrag(vt, 0, 0, 0);
      vf[1] = vfrag(vt, 0, 0, 1);
    }
    float xin = (sc[0][0][0]);
    float xin1 = MODE == 1 ? (sc[0][0][1]) : 0.f;  // scoring: the second element of a slot
    static_for<0, 64>([&](auto slot) __attribute__((always_inline)) {
      constexpr int s = decltype(slot)::value;
      // scoring (MODE 1, no PV products): the odd slots hold nothing; each even slot takes
      // the softmax of elements s and s + 1 beside its product, and the K copies
      if constexpr (MODE == 1 && (s & 1) == 1) return;
      if constexpr ((s & 1) == 0) {
        // MFMA k = s / 2 covers dd = k / 4, (k2, c) = k % 4
        constexpr int k = s >> 1, dd = k >> 2, k2 = (k >> 1) & 1, c = k & 1;
        if constexpr ((k & 3) == 0 && dd + 1 < D / 16) load_step(dd + 1, kq[(dd + 1) & 1]);
        // the first product of an accumulator (dd = 0) starts from zero
        if constexpr (dd == 0) mfma_va0(sn[k2][c], kq[dd & 1][k2], qa[c][dd]);
        else mfma_va(sn[k2][c], kq[dd & 1][k2], qa[c][dd]);
      } else if constexpr (PV) {
        // MFMA k = s / 2 covers operand group g = k / 2 ((k2, hf) = g / 4, db = g % 4)
        // and row block c = k % 2; the V^T operand of group g + 2 is read at the first
        // MFMA of group g
        constexpr int k = s >> 1, g = k >> 1, c = k & 1;
        constexpr int k2 = g >> 3, hf = (g >> 2) & 1, db = g & 3;
        if constexpr (c == 0 && g + 2 < 16) {
          constexpr int g2 = g + 2;
          vf[g2 % 3] = vfrag(vt, g2 >> 3, (g2 >> 2) & 1, g2 & 3);
        }
        acc[c][db] = mfma32x32x16(vf[g % 3], pfp[k2][c][hf], acc[c][db]);
      }
      // the tile copies, one every 4 slots in the first half of the block (slots 3, 7, ..,
      // 31): landing early, they are done by the next barrier (one every 8 slots over the
      // whole block took 2% longer); scoring: one every 8 slots
      if constexpr (MODE == 1 ? (s & 7) == 4 : ((s & 3) == 3 && s < 32)) {
        constexpr int u = MODE == 1 ? (s >> 3) : (s >> 2);  // 0..7: K(t+2) copies, then V(t) copies
        if constexpr (u < 4) copy_tile(rk, u, kdst);
        else if constexpr (MODE != 1) copy_tile(rv, u - 4, vdst);  // scoring reads no V
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        // softmax element s: row block s / 32, element e = s % 32 (key block e / 16,
        // accumulator element e % 16), its input taken one slot ahead.  Element s - 2
        // joins the fp32 row sum (it sets LSE, which the backward reuses) and, when it
        // completes a pair, the pair is rounded to bf16 into its PV operand: one add and
        // half a conversion per slot, in the order of additions of a plain running sum.
        // Two slots (not one) after its exponential: a product written as an asm
        // statement does not count as a wait state, and a VALU read of a transcendental
        // result needs one.
        constexpr int c = s >> 5;
        if constexpr (MODE == 1) {
          // elements s, s + 1 (one row block: s is even), their inputs taken a slot ahead;
          // the previous slot's two elements join the row sum
          const float x0 = xin, x1 = xin1;
          if constexpr (s + 2 < 64) {
            xin = (sc[((s + 2) >> 4) & 1][(s + 2) >> 5][(s + 2) & 15]);
            xin1 = (sc[((s + 3) >> 4) & 1][(s + 3) >> 5][(s + 3) & 15]);
          }
          if constexpr (s >= 2) {
            fold(IC<s - 2>{});
            fold(IC<s - 1>{});
          }
          pb[s & 7] = __builtin_amdgcn_exp2f(fmaf(x0, a.scale_log2, -m[c]));
          pb[(s + 1) & 7] = __builtin_amdgcn_exp2f(fmaf(x1, a.scale_log2, -m[c]));
        } else {
          const float x = xin;
          if constexpr (s + 1 < 64) xin = (sc[((s + 1) >> 4) & 1][(s + 1) >> 5][(s + 1) & 15]);
          if constexpr (s >= 2) fold(IC<s - 2>{});
          pb[s & 7] = __builtin_amdgcn_exp2f(fmaf(x, a.scale_log2, -m[c]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    };
    if constexpr (MODE == 1) slots(IC<0>{});
    else slots(IC<1>{});
    fold(IC<62>{});
    fold(IC<63>{});

    if constexpr (MODE == 2) return;  // P normalised by the given LSE: no reference to move

    // reference check on the column sums (both lane halves).  A column's sum exceeds
    // 2^32 only if one of its halves exceeds 2^31, and its l is 0 only if both halves'
    // are, so when every lane passes the test on its own half no column can fail the
    // exact test, and the exact test (two lane swaps per row block) is skipped.
    float alpha[CB] = {1.f, 1.f};
    bool near_edge = false;
#pragma unroll
    for (int c = 0; c < CB; ++c) near_edge |= (sum[c] > 0.5f * kSumHi) | ((l[c] == 0.f) & (sum[c] < kSumLo));
    if (__builtin_amdgcn_ballot_w64(near_edge) != 0) {
      bool redo[CB];
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float cs = sum[c] + swap_halves(sum[c]);
        const float cl = l[c] + swap_halves(l[c]);
        redo[c] = (cs > kSumHi) | ((cl == 0.f) & (cs < kSumLo));
      }
      if (__builtin_amdgcn_ballot_w64(redo[0] | redo[1]) != 0) {
        // rare: the tile's column max becomes the reference of the columns that need one
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          float mx = -INFINITY;
#pragma unroll
          for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, (sc[k2][c][i]));
          const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          const float mt = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * a.scale_log2;
          const bool mv = redo[c] & (mt > -INFINITY);
          alpha[c] = mv ? __builtin_amdgcn_exp2f(m[c] - mt) : 1.f;
          m[c] = mv ? mt : m[c];
          if (__builtin_amdgcn_ballot_w64(mv) != 0) {
            const float s2 = softmax_rows(sc, pfc, c, m[c]);
            sum[c] = mv ? s2 : sum[c];
          }
        }
        // O holds tiles up to t-1 in the previous references: take it to the new ones
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[c][db][i] = agpr_scale(acc[c][db][i], alpha[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) l[c] = l[c] * alpha[c] + sum[c];  // fp32 row sums set LSE
    if constexpr (MODE == 1) {
      // the tile's row numerators in log2 (both lane halves of a column, in the reference
      // the sums were taken in); rows without a token get -inf
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float cs = sum[c] + swap_halves(sum[c]);
        const float lm = (rvalid[c] & (cs > 0.f)) ? log2f(cs) + m[c] : -INFINITY;
        if (h2 == 0)
          a.mala_mass[(((int64_t)b * a.mala_nnz + e0 + t) * ROWS) + wave * WROWS + c * 32 + n] = lm;
      }
    }
  };

  // O^T += V(t)^T P(t)^T for the last tile, alone
  auto last_pv = [&](auto parity) __attribute__((always_inline)) {
    constexpr int PAR = decltype(parity)::value;
    const __bf16* const vt = vbuf(IC<PAR>{});
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const bf16x8 vf = vfrag(vt, g >> 3, (g >> 2) & 1, g & 3);
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[c][g & 3] = mfma32x32x16(vf, pf[PAR][g >> 3][c][(g >> 2) & 1], acc[c][g & 3]);
    }
  };

  if (nt > 0) {
    ent0 = load_uniform(ents, e0);
    ent1 = nt > 1 ? load_uniform(ents, e0 + 1) : 0;
    ent2 = nt > 2 ? load_uniform(ents, e0 + 2) : 0;
    ent_next = __builtin_amdgcn_raw_buffer_load_b32(r_ent, 0, 4 * 3, 0);
    {
      const __amdgpu_buffer_rsrc_t rk0 = tile_copy_rsrc(kbase, ent0, true);
      const __amdgpu_buffer_rsrc_t rk1 = tile_copy_rsrc(kbase, ent1, nt > 1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        copy_tile(rk0, u, sK0);
        copy_tile(rk1, u, sK1);
      }
    }
    // P(-1) = 0: the first iteration's PV stage adds nothing
#pragma unroll
    for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) pf[1][k2][c][hf] = zero_bf16x8();
    wait_loads_and_barrier();
    // S(0), masked, sets the first reference: its column max (exact P = 1 for the
    // column's top key, so a column that sees one key reproduces its V row), or 0 for a
    // column with no visible key in tile 0.  MALA: the reference is the given LSE (P
    // exactly normalised; +inf for rows without a token or a visible key: P = 0)
    load_q();
    scores(sx[0]);
    mask_tile(sx[0], ent0);
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      if constexpr (MODE == 2) {
        const float lv = rvalid[c] ? a.lse[((int64_t)b * a.Hq + hq[c]) * a.Lq + tok[c]] : -INFINITY;
        m[c] = lv == -INFINITY ? INFINITY : lv * kLog2e;
      } else {
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 32; ++e) mx = fmaxf(mx, sx[0][e >> 4][c][e & 15]);
        const float mt = fmaxf(mx, swap_halves(mx)) * a.scale_log2;
        m[c] = mt > -INFINITY ? mt : 0.f;
      }
    }
    for (int t = 0; t < nt; t += 2) {
      iteration(IC<0>{}, t);
      if (t + 1 < nt) iteration(IC<1>{}, t + 1);
    }
    wait_loads_and_barrier();  // V(nt-1) resident
    if constexpr (MODE != 1) {
      if ((nt - 1) & 1) last_pv(IC<1>{});
      else last_pv(IC<0>{});
    }
  }

  // ---- finalize: l summed over the two lane halves of a column (MALA: P was normalised,
  // O is the plain sum; scoring writes only LSE).  O, and its rounding residual, leave
  // through this wave's 64 rows of the Q tile (free once its last product has read them;
  // an item without tiles waits here for its Q copies): each lane puts its runs of 4 dims
  // of row n into LDS (chunk-swizzled rows), then each store writes four whole 256-byte
  // rows (a row is one (token, head), and the G heads of a token are adjacent in O)
  // instead of 8 bytes in each of 32 rows.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  // The lane's coordinates and rows are formed again here (from the lane count, not the
  // work-item id) rather than carried across the tile loop, which uses every register.
  // Item row r = token * G + head; token r / G by a multiply-shift (exact for r < 256,
  // G <= 256).
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int n_e = lane_e & 31, h2_e = lane_e >> 5;
  const uint32_t ginv = (65536u + (uint32_t)G - 1u) / (uint32_t)G;
  float inv[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const float lt = l[c] + __shfl_xor(l[c], 32);
    inv[c] = MODE == 2 ? 1.f : lt > 0.f ? 1.f / lt : 0.f;
    const int r = wave * WROWS + c * 32 + n_e;
    const int rt = (int)(((uint32_t)r * ginv) >> 16);
    const int t = qb * Bq + rt;
    if (MODE != 2 && rt < Bq && t < a.Lq && h2_e == 0)  // MALA's kept-tile pass keeps the given LSE
      a.lse[((int64_t)b * a.Hq + h * G + (r - rt * G)) * a.Lq + t] = lt > 0.f ? (m[c] + log2f(lt)) * kLn2 : -INFINITY;
  }
  if constexpr (MODE != 1) {
    __bf16* const so = sQ + wave * WROWS * D;
    // lo = false: O / l rounded to bf16; true: what that rounding dropped, rounded to bf16
    auto put = [&](bool lo) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[c][db][4 * q4 + e] * inv[c];
            const bf16x4 v = to_bf16x4(x[0], x[1], x[2], x[3]);
            const bf16x4 w = lo ? to_bf16x4(x[0] - (float)v[0], x[1] - (float)v[1], x[2] - (float)v[2],
                                            x[3] - (float)v[3])
                                : v;
            *(u32x2*)(so + swz(c * 32 + n_e, 32 * db + 8 * q4 + 4 * h2_e)) = __builtin_bit_cast(u32x2, w);
          }
    };
    // copy u: lane L sends logical chunk L % 16 of local row 4 u + L / 16
    auto drain = [&](__bf16* dst) __attribute__((always_inline)) {
      // all of the wave's LDS reads first, then the stores (a read inside each store's
      // row condition waited for its own LDS latency, 16 times over)
      u32x4 wv[WROWS / 4];
#pragma unroll
      for (int u = 0; u < WROWS / 4; ++u) {
        const int rl = 4 * u + (lane_e >> 4), ch = lane_e & 15;
        wv[u] = *(const u32x4*)(so + rl * D + 8 * (ch ^ sw(rl)));
      }
#pragma unroll
      for (int u = 0; u < WROWS / 4; ++u) {
        const int rl = 4 * u + (lane_e >> 4), ch = lane_e & 15;
        const u32x4 w = wv[u];
        const int r = wave * WROWS + rl;
        const int rt = (int)(((uint32_t)r * ginv) >> 16);
        const int t = qb * Bq + rt;
        if (rt < Bq && t < a.Lq)
          *(u32x4*)(dst + (((int64_t)b * a.Lq + t) * a.Hq + h * G + (r - rt * G)) * D + 8 * ch) = w;
      }
    };
    put(false);
    drain((__bf16*)a.o);
    if (a.o_lo) {
      put(true);
      drain((__bf16*)a.o_lo);
    }
  }
}

// MALA decisions, one work group per (item, sequence): thread r owns row r of the item
// (its LSE from the scoring pass); a tile is kept when its largest row mass
// 2^(numerator - LSE) reaches tau.  Tiles go 16 at a time (16 independent loads per
// thread, one barrier); thread 0 writes the decisions and the kept entries in list order.
constexpr int DEC_TILES = 16;
__global__ __launch_bounds__(ROWS) void mala_decide_kernel(FwdArgs a) {
  __shared__ float smax[DEC_TILES][WAVES];
  const int item = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = item / a.nqb, qb = item - h * a.nqb;
  const int e0 = a.row_ptr[item], nt = a.row_ptr[item + 1] - e0;
  const int rt = tid / a.G, g = tid - rt * a.G, t = qb * a.Bq + rt;
  const bool valid = (rt < a.Bq) & (t < a.Lq);
  const float lv = valid ? a.lse[((int64_t)b * a.Hq + h * a.G + g) * a.Lq + t] : -INFINITY;
  const float lse2 = lv * kLog2e;
  const float* mass = a.mala_mass + ((int64_t)b * a.mala_nnz + e0) * ROWS + tid;
  int32_t* const ents = a.mala_ents + (int64_t)b * a.mala_nnz + e0;
  int cnt = 0;
  for (int i0 = 0; i0 < nt; i0 += DEC_TILES) {
    float x[DEC_TILES];
#pragma unroll
    for (int j = 0; j < DEC_TILES; ++j) {
      const float lm = i0 + j < nt ? mass[(int64_t)(i0 + j) * ROWS] : -INFINITY;
      x[j] = (lv > -INFINITY && lm > -INFINITY) ? exp2f(lm - lse2) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < DEC_TILES; ++j) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) x[j] = fmaxf(x[j], __shfl_xor(x[j], off));
      if (lane == 0) smax[j][wave] = x[j];
    }
    __syncthreads();
    if (tid == 0) {
      for (int j = 0; j < DEC_TILES && i0 + j < nt; ++j) {
        float mx = smax[j][0];
        for (int w = 1; w < WAVES; ++w) mx = fmaxf(mx, smax[j][w]);
        const bool keep = mx >= a.mala_tau;
        if (a.kept && b == 0) a.kept[e0 + i0 + j] = keep ? 1 : 0;
        if (keep) ents[cnt++] = a.row_ent[e0 + i0 + j];
      }
    }
    __syncthreads();  // smax is rewritten by the next group
  }
  if (tid == 0) a.mala_counts[(int64_t)b * a.n_items + item] = cnt;
}

}  // namespace

// clears the 8 queue heads of one launch (see claim_item)
__global__ __launch_bounds__(64) void fwd_queue_clear_kernel(int32_t* heads) {
  if (threadIdx.x < 8) heads[threadIdx.x] = 0;
}

hipError_t launch_fwd_bf16_d128(const FwdArgs& a, hipStream_t s) {
  // with the queues, spare work groups let fast XCDs take over positions of slow ones
  dim3 grid(a.queues ? a.n_items + a.n_items / 16 + 8 : a.n_items, a.B);
  if (a.queues) {
    hipLaunchKernelGGL(fwd_queue_clear_kernel, dim3(1), dim3(64), 0, s, a.queues);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(fwd_bf16_d128_kernel<0>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mala_fwd_bf16_d128(const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.n_items, a.B);
  hipLaunchKernelGGL(fwd_bf16_d128_kernel<1>, grid, dim3(256), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mala_decide_kernel, grid, dim3(ROWS), 0, s, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(fwd_bf16_d128_kernel<2>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cowa
