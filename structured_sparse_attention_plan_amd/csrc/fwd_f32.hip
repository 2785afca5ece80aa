// CoWindow Attention forward in fp32, head dim 64 (the small latency-bound workload), on
// the matrix cores (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation).
//
// One work group per (KV head h, q-block of BQ = 8 tokens), the G <= 4 query heads that
// share KV head h together (they read the same K/V tiles; the pages tie the windows to
// the KV head: slinene.github.io ai-papers-daily page, method key point 3).  Its rows
// (token-major, r = token * G + head) are one or two blocks of 16 MFMA columns.  Each of
// the 4 waves takes 16 keys of every 64-key tile in the planner's row list, keeps its own
// running max, sum and O over them (base-2 online softmax), and the waves' states are
// merged at the end through LDS.  Per tile and wave:
//   S^T = K Q^T: K (A operand, one key per lane) and Q^T (B operand) in registers, the
//     16 k-steps pairing dims 16 g + kc of lane group g (any pairing of the contracted
//     index serves, so each lane loads 16 consecutive dims of its row with 16-byte loads);
//   O^T += V^T P^T: P^T straight from the score registers (lane group g holds keys
//     4 g .. 4 g + 3 of its row, so k-step kc pairs key 4 g + kc), V^T with lane n taking
//     dims 4 n .. 4 n + 3 of a key row, so D-block db of the product holds dims 4 m + db.
// K and V of the next tile are loaded into registers while the current one is computed.
//
// MFMA lane layouts of v_mfma_f32_16x16x4_f32 (n = lane % 16, g = lane / 16):
//   A (16 x 4): A[n][g]   B (4 x 16): B[g][n]   C (16 x 16): element i is C[4 g + i][n]

#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 64;
constexpr int BQ = kF32Bq;  // tokens per q-block
constexpr int BK = kF32Bk;  // keys per tile
constexpr int WAVES = 4;    // 16 keys of every tile each


__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// RB: blocks of 16 rows (1 for G <= 2, 2 for G = 3, 4)
template <int RB>
__global__ __launch_bounds__(256) void fwd_f32_d64_kernel(FwdArgs a) {
  constexpr int ROWS = 16 * RB;
  __shared__ float sm[WAVES][ROWS];
  __shared__ float sl[WAVES][ROWS];
  __shared__ __attribute__((aligned(16))) float so[WAVES][ROWS][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int item = a.row_order[blockIdx.x];
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int G = a.G;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);
  const float c2 = a.scale_log2;

  const float* Q = (const float*)a.q;
  const float* K = (const float*)a.k;
  const float* V = (const float*)a.v;

  // Q^T operands of row n of each block: Q[row][16 g + kc], kc = 0..15
  float qf[RB][16];
  int tok[RB];
  bool rvalid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 16 * rb + n;
    const int rt = r / G;
    tok[rb] = qb * BQ + rt;
    rvalid[rb] = rt < BQ && tok[rb] < a.Lq;
    const float* qp = Q + (((int64_t)b * a.Lq + (rvalid[rb] ? tok[rb] : 0)) * a.Hq + h * G +
                           (rvalid[rb] ? r - rt * G : 0)) * D + 16 * g;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4 x = rvalid[rb] ? *(const f32x4*)(qp + 4 * v) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[rb][4 * v + e] = x[e];
    }
  }

  float m[RB], l[RB];
  f32x4 acc[RB][4];  // O^T: element i of acc[rb][db] is dim 16 g + 4 i + db of row n
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K of key 16 wave + n of a tile (dims 16 g .. + 15) and V of keys 16 wave + 4 g + kc
  // (dims 4 n .. + 3); keys past Lk read key Lk - 1 (their tiles are boundary tiles, and
  // the mask hides them)
  f32x4 kq[2][4], vq[2][4];
  auto fetch = [&](int ent, f32x4 (&kd)[4], f32x4 (&vd)[4]) {
    const int j0 = (ent >> 1) * BK + 16 * wave;
    const int jk = min(j0 + n, a.Lk - 1);
    const float* kp = K + (((int64_t)b * a.Lk + jk) * a.Hkv + h) * D + 16 * g;
#pragma unroll
    for (int v = 0; v < 4; ++v) kd[v] = *(const f32x4*)(kp + 4 * v);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int jv = min(j0 + 4 * g + kc, a.Lk - 1);
      vd[kc] = *(const f32x4*)(V + (((int64_t)b * a.Lk + jv) * a.Hkv + h) * D + 4 * n);
    }
  };

  auto tile = [&](int ent, const f32x4 (&kd)[4], const f32x4 (&vd)[4]) {
    const int j0 = (ent >> 1) * BK + 16 * wave + 4 * g;  // key of element 0 of this lane
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 16; ++kc) s = mfma_f32(kd[kc >> 2][kc & 3], qf[rb][kc], s);
      // element i: key j0 + i of row n
      if (ent & 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = rvalid[rb] & visible(tok[rb] + off, j0 + i, a.Lk, a.win.sink, a.win.near_w, band);
          s[i] = vis ? s[i] : -INFINITY;
        }
      }
      // the row's max over the wave's 16 keys (the four lane groups), then the update
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m[rb], mx * c2);
      const float alpha = (m[rb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[rb] - mn);
      m[rb] = mn;
      // no visible key yet (mn = -inf): probabilities 0 through a reference of 0
      const float mref = mn == -INFINITY ? 0.f : mn;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mref));
      l[rb] = l[rb] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4 o = acc[rb][db] * alpha;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) o = mfma_f32(vd[kc][db], p[kc], o);
        acc[rb][db] = o;
      }
    }
  };

  const int e0 = a.row_ptr[item], e1 = a.row_ptr[item + 1];
  if (e0 < e1) {
    int ent = a.row_ent[e0];
    fetch(ent, kq[0], vq[0]);
    for (int e = e0; e < e1; e += 2) {
      int ent1 = 0;
      if (e + 1 < e1) {
        ent1 = a.row_ent[e + 1];
        fetch(ent1, kq[1], vq[1]);
      }
      tile(ent, kq[0], vq[0]);
      if (e + 1 < e1) {
        if (e + 2 < e1) {
          ent = a.row_ent[e + 2];
          fetch(ent, kq[0], vq[0]);
        }
        tile(ent1, kq[1], vq[1]);
      }
    }
  }

  // merge the four waves: each row's sum over its lane groups, then max, rescaled sums
  // and outputs over the waves
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = l[rb] + __shfl_xor(l[rb], 16);
    lt += __shfl_xor(lt, 32);
    if (g == 0) {
      sm[wave][16 * rb + n] = m[rb];
      sl[wave][16 * rb + n] = lt;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 o = {acc[rb][0][i], acc[rb][1][i], acc[rb][2][i], acc[rb][3][i]};
      *(f32x4*)&so[wave][16 * rb + n][16 * g + 4 * i] = o;
    }
  }
  __syncthreads();
  for (int x = tid; x < ROWS * D; x += 256) {
    const int r = x / D, d = x - r * D;
    const int rt = r / G;
    const int t = qb * BQ + rt;
    if (rt >= BQ || t >= a.Lq) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm[w][r]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float wt = sm[w][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[w][r] - M);
        L += wt * sl[w][r];
        o += wt * so[w][r][d];
      }
    }
    const int hq = h * G + (r - rt * G);
    ((float*)a.o)[(((int64_t)b * a.Lq + t) * a.Hq + hq) * D + d] = L > 0.f ? o / L : 0.f;
    if (d == 0) a.lse[((int64_t)b * a.Hq + hq) * a.Lq + t] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_f32_d64(const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.n_items, a.B);
  if (a.G <= 2) hipLaunchKernelGGL(fwd_f32_d64_kernel<1>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fwd_f32_d64_kernel<2>, grid, dim3(256), 0, s, a);  // G <= 4 (checked by the C API)
  return hipGetLastError();
}

}  // namespace cowa
