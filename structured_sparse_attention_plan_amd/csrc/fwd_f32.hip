// CoWindow Attention forward in fp32, head dim 64 (the small latency-bound workload).
//
// One work group per (KV head h, q-block of 64 tokens): 64 * G threads (G <= 4), one row
// each (the G query heads that share KV head h read the same K/V tiles; the pages tie
// the windows to the KV head — slinene.github.io ai-papers-daily page, method key
// point 3).  For every visible 64-key block in the planner's row list, K and V are
// staged in LDS and each thread computes its 64 scores with fp32 FMAs (all threads read
// the same LDS word, a broadcast), masks PARTIAL blocks with the window predicate,
// updates its running max / sum (base-2 online softmax) and accumulates P V.

#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 64;
constexpr int BQ = kF32Bq;
constexpr int BK = kF32Bk;

__global__ __launch_bounds__(256) void fwd_f32_d64_kernel(FwdArgs a) {
  __shared__ float sK[BK][D + 1];
  __shared__ float sV[BK][D];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int item = a.row_order[blockIdx.x];
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int gi = tid / BQ;  // head within the group
  const int t = qb * BQ + (tid - gi * BQ);
  const int hq = h * a.G + gi;
  const bool valid = t < a.Lq;
  const int p = t + (a.Lk - a.Lq);
  const HeadBand band = head_band(a.win, h);

  const float* Q = (const float*)a.q;
  const float* K = (const float*)a.k;
  const float* V = (const float*)a.v;

  float q[D], o[D];
  const float* qp = Q + (((int64_t)b * a.Lq + (valid ? t : 0)) * a.Hq + hq) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int e0 = a.row_ptr[item], e1 = a.row_ptr[item + 1];
  for (int e = e0; e < e1; ++e) {
    const int ent = a.row_ent[e];
    const int kb = ent >> 1;
    const bool partial = ent & 1;
    __syncthreads();
    for (int x = tid; x < BK * D; x += nthr) {
      const int r = x / D, d = x - r * D;
      const int j = kb * BK + r;
      const int64_t o_ = (((int64_t)b * a.Lk + j) * a.Hkv + h) * D + d;
      sK[r][d] = j < a.Lk ? K[o_] : 0.f;
      sV[r][d] = j < a.Lk ? V[o_] : 0.f;
    }
    __syncthreads();

    float s[BK];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < BK; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], sK[r][d], acc);
      const int j = kb * BK + r;
      if (partial && !(valid && visible(p, j, a.Lk, a.win.sink, a.win.near_w, band))) acc = -INFINITY;
      s[r] = acc * a.scale_log2;
      mt = fmaxf(mt, s[r]);
    }
    const float mn = fmaxf(m, mt);
    if (mn == -INFINITY) continue;  // nothing visible yet for this row
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int r = 0; r < BK; ++r) {
      const float pr = exp2f(s[r] - mn);
      l += pr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(pr, sV[r][d], o[d]);
    }
  }

  if (valid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = (float*)a.o + (((int64_t)b * a.Lq + t) * a.Hq + hq) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
    a.lse[((int64_t)b * a.Hq + hq) * a.Lq + t] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_f32_d64(const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.n_items, a.B);
  hipLaunchKernelGGL(fwd_f32_d64_kernel, grid, dim3(BQ * a.G), 0, s, a);
  return hipGetLastError();
}

}  // namespace cowa
