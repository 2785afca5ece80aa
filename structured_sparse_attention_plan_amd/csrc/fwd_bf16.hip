// CoWindow Attention forward, bf16 in/out, head dim 128, for gfx950.
//
// One work item = (KV head h, q-block of Bq = 256 / G tokens): the query rows of the G
// query heads that share KV head h (slinene.github.io ai-papers-daily page, method key
// point 3: windows follow the KV head, so one K/V tile read from HBM serves all G query
// heads).  Rows are token-major (row r = token * G + head-in-group), so the item's Q is
// one strided run of G * 256 bytes per token.  Four waves own 64 rows each, as two
// 32-column blocks of v_mfma_f32_32x32x16_bf16.
//
// Per visible k-block (64 keys, from the planner's row list; masked blocks are never
// touched):
//   1. the 256 threads stage K and V (64 x 128 bf16 each, row-major) in LDS; the next
//      block's global loads are issued before this block's math;
//   2. S^T = K Q^T: K from LDS (A operand, one key row per lane), Q^T from LDS (B
//      operand; each wave stages its own 64 rows once per item), so each lane owns one
//      query row (column) and 16 of every 32 keys;
//   3. boundary (PARTIAL) blocks apply the window predicate element by element; FULL
//      blocks skip it;
//   4. online softmax in base 2 (scale * log2 e folded into one FMA), the row max taken
//      across the two lane halves of a column; the running max only moves when a row's
//      tile max exceeds it by more than 8 (log2 units): exact, because O / l does not
//      depend on the reference, and P stays <= 256;
//   5. O^T += V^T P^T: P^T goes from the C-layout accumulator straight into the B
//      operand (no LDS round trip) and V^T is read from the row-major LDS tile with
//      ds_read_b64_tr_b16, two 4-key runs per operand matching the accumulator layout.
// Output: O / l in bf16 and LSE = ln 2 * (m + log2 l) in fp32.
//
// MFMA lane layouts of v_mfma_f32_32x32x16_bf16 (n = lane % 32, h2 = lane / 32):
//   A (32 x 16): A[n][8 h2 + e]   B (16 x 32): B[8 h2 + e][n]
//   C (32 x 32): element i of 16 is C[8 (i / 4) + 4 h2 + i % 4][n]

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
constexpr int PITCH = D + 16;        // LDS row pitch in elements (288 bytes)
constexpr float kRescaleThreshold = 8.0f;

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

__global__ __launch_bounds__(256, 1) void fwd_bf16_d128_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 sQ[ROWS * PITCH];
  __shared__ __attribute__((aligned(16))) __bf16 sK[BK * PITCH];
  __shared__ __attribute__((aligned(16))) __bf16 sV[BK * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int item = a.row_order[blockIdx.x];
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

  // ---- this wave's 64 query rows -> LDS
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
  __bf16* sQw = sQ + wave * WROWS * PITCH;
#pragma unroll 4
  for (int u = 0; u < WROWS * 16 / 64; ++u) {
    const int id = lane + 64 * u;
    const int row = id >> 4, cc = id & 15;
    const int r = wave * WROWS + row;
    const int rt = r / G;
    const int t = qb * Bq + rt;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (rt < Bq && t < a.Lq)
      v = *(const u32x4*)(Q + (((int64_t)b * a.Lq + t) * a.Hq + h * G + (r - rt * G)) * D + 8 * cc);
    *(u32x4*)(sQw + row * PITCH + 8 * cc) = v;
  }

  f32x16 acc[CB][4];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][db][i] = 0.f;
  float m[CB], l[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    m[c] = -INFINITY;
    l[c] = 0.f;
  }

  // ---- K/V staging: thread tid moves 16-byte chunks tid + 256 u (u < 4): row id / 16,
  // column chunk id % 16
  const int e0 = a.row_ptr[item], e1 = a.row_ptr[item + 1];
  u32x4 pk[4], pv[4];
  auto fetch = [&](int e) {
    const int kb = a.row_ent[e] >> 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = tid + 256 * u;
      const int row = id >> 4, cc = id & 15;
      const int j = kb * BK + row;
      if (j < a.Lk) {
        const int64_t o = (((int64_t)b * a.Lk + j) * a.Hkv + h) * D + 8 * cc;
        pk[u] = *(const u32x4*)(K + o);
        pv[u] = *(const u32x4*)(V + o);
      } else {
        pk[u] = u32x4{0, 0, 0, 0};
        pv[u] = u32x4{0, 0, 0, 0};
      }
    }
  };
  if (e0 < e1) fetch(e0);

  // tr-read addressing for the V^T operand: 16-lane group gg covers d columns
  // 16 (gg & 1) .. +15 of a 32-column block and key run 4 (gg >> 1) (+8)
  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);

  // A rescale of the output accumulators (rare: only when a row's tile max exceeds its
  // reference by more than the threshold) reads, scales and writes each accumulator
  // register in place (agpr_scale), so the accumulators stay resident in AGPRs; scaling
  // them with ordinary VALU code makes the compiler copy all 128 of them every tile.
  f32x16 s[KB2][CB];
  float mt[CB];
  int e = e0;
  auto stage_and_scores = [&](int ee) {
    const int ent = a.row_ent[ee];
    const int kb = ent >> 1;
    const bool partial = ent & 1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = tid + 256 * u;
      const int row = id >> 4, cc = id & 15;
      *(u32x4*)(sK + row * PITCH + 8 * cc) = pk[u];
      *(u32x4*)(sV + row * PITCH + 8 * cc) = pv[u];
    }
    __syncthreads();
    if (ee + 1 < e1) fetch(ee + 1);

    // ---- S^T = K Q^T
#pragma unroll
    for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[k2][c][i] = 0.f;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      bf16x8 qf[CB];
#pragma unroll
      for (int c = 0; c < CB; ++c) qf[c] = load16(sQw + (c * 32 + n) * PITCH + 16 * dd + 8 * h2);
#pragma unroll
      for (int k2 = 0; k2 < KB2; ++k2) {
        const bf16x8 kf = load16(sK + (32 * k2 + n) * PITCH + 16 * dd + 8 * h2);
#pragma unroll
        for (int c = 0; c < CB; ++c) s[k2][c] = mfma32x32x16(kf, qf[c], s[k2][c]);
      }
    }

    // ---- mask boundary tiles (branch-free per element)
    if (partial) {
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int p = tok[c] + off;
#pragma unroll
        for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = kb * BK + 32 * k2 + 8 * (i >> 2) + 4 * h2 + (i & 3);
            const bool vis = rvalid[c] & visible(p, j, a.Lk, a.win.sink, a.win.near_w, band);
            s[k2][c][i] = vis ? s[k2][c][i] : -INFINITY;
          }
      }
    }

    // ---- tile max per row, across the two lane halves of a column
    bool need = false;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      float x = s[0][c][0];
#pragma unroll
      for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
        for (int i = 0; i < 16; ++i) x = fmaxf(x, s[k2][c][i]);
      x = fmaxf(x, __shfl_xor(x, 32));
      mt[c] = x * a.scale_log2;
      need |= mt[c] > m[c] + kRescaleThreshold;
    }
    return __builtin_amdgcn_ballot_w64(need) != 0;
  };

  // P = exp2(scale log2e S - m) as bf16 B operands, row sums into l, then O^T += V^T P^T.
  // pf[k2][c][hf] holds keys 32 k2 + 16 hf + {4 h2 .. +3, 8 + 4 h2 .. +3}, i.e.
  // accumulator elements 8 hf .. 8 hf + 7.
  auto accumulate = [&]() {
    bf16x8 pf[KB2][CB][2];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const float ref = (m[c] == -INFINITY) ? 0.f : m[c];
      float sum = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float p[8];
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) {
            p[e2] = __builtin_amdgcn_exp2f(fmaf(s[k2][c][8 * hf + e2], a.scale_log2, -ref));
            sum += p[e2];
          }
          pf[k2][c][hf] = join(to_bf16x4(p[0], p[1], p[2], p[3]), to_bf16x4(p[4], p[5], p[6], p[7]));
        }
      l[c] += sum;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int k2 = 0; k2 < KB2; ++k2) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const __bf16* vp = sV + (32 * k2 + 16 * hf + vrow) * PITCH + 32 * db + vcol;
          const bf16x8 vf = join(lds_read_tr4(vp), lds_read_tr4(vp + 8 * PITCH));
#pragma unroll
          for (int c = 0; c < CB; ++c) acc[c][db] = mfma32x32x16(vf, pf[k2][c][hf], acc[c][db]);
        }
      }
    }
  };

  for (; e < e1; ++e) {
    if (stage_and_scores(e)) {
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float mn = fmaxf(m[c], mt[c]);
        const float alpha = (m[c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[c] - mn);
        m[c] = mn;
        l[c] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[c][db][i] = agpr_scale(acc[c][db][i], alpha);
      }
    }
    accumulate();
  }

  // ---- finalize: l summed over the two lane halves of a column
  __bf16* O = (__bf16*)a.o;
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    float lt = l[c] + __shfl_xor(l[c], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (rvalid[c]) {
      __bf16* op = O + (((int64_t)b * a.Lq + tok[c]) * a.Hq + hq[c]) * D + 4 * h2;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const bf16x4 v = to_bf16x4(acc[c][db][4 * q4] * inv, acc[c][db][4 * q4 + 1] * inv,
                                     acc[c][db][4 * q4 + 2] * inv, acc[c][db][4 * q4 + 3] * inv);
          *(u32x2*)(op + 32 * db + 8 * q4) = __builtin_bit_cast(u32x2, v);
        }
      if (h2 == 0)
        a.lse[((int64_t)b * a.Hq + hq[c]) * a.Lq + tok[c]] =
            lt > 0.f ? (m[c] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16_d128(const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.n_items, a.B);
  hipLaunchKernelGGL(fwd_bf16_d128_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cowa
