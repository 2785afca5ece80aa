// CoWindow Attention forward in fp32, head dim 64 (the small latency-bound workload).
//
// One work group per (KV head h, q-block of BQ = 8 tokens), the G query heads that
// share KV head h together (they read the same K/V tiles; the pages tie the windows to
// the KV head — slinene.github.io ai-papers-daily page, method key point 3).  Each row
// is served by SUB = 16 neighbouring lanes, lane ks taking keys ks, ks + 16, ks + 32 and
// ks + 48 of every 64-key tile: the small workload spreads over the whole chip (at 1024
// tokens, 256 work groups of 256 threads) and each lane's chain of dependent FMAs per
// tile is short.  For every visible tile in the planner's row list K and V are staged in
// LDS (the 16 lanes of a row read 16 different key rows, one per bank group); each lane
// computes its 4 scores with fp32 FMAs, masks PARTIAL tiles with the window predicate,
// and keeps its own running max, sum and P V over its keys (base-2 online softmax).  At
// the end the 16 lanes of a row merge their states (max, then each sum and output
// rescaled to it and added).

#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 64;
constexpr int BQ = kF32Bq;
constexpr int BK = kF32Bk;
constexpr int SUB = 16;           // lanes per row
constexpr int KPL = BK / SUB;     // keys per lane and tile
constexpr int LDK = D + 4;        // padded LDS row (floats): 16-byte aligned, banks spread

// GQ: the group size (query heads per KV head), which sets the thread count
template <int GQ>
__global__ __launch_bounds__(BQ * GQ * SUB) void fwd_f32_d64_kernel(FwdArgs a) {
  constexpr int NTHR = BQ * GQ * SUB;
  __shared__ __attribute__((aligned(16))) float sK[BK * LDK];
  __shared__ __attribute__((aligned(16))) float sV[BK * LDK];

  const int tid = threadIdx.x;
  const int item = a.row_order[blockIdx.x];
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int row = tid / SUB, ks = tid - row * SUB;
  const int gi = row / BQ;  // head within the group
  const int t = qb * BQ + (row - gi * BQ);
  const int hq = h * a.G + gi;
  const bool valid = t < a.Lq;
  const int p = t + (a.Lk - a.Lq);
  const HeadBand band = head_band(a.win, h);

  const float* Q = (const float*)a.q;
  const float* K = (const float*)a.k;
  const float* V = (const float*)a.v;

  float4 q[D / 4], o[D / 4];
  const float4* qp = (const float4*)(Q + (((int64_t)b * a.Lq + (valid ? t : 0)) * a.Hq + hq) * D);
#pragma unroll
  for (int d4 = 0; d4 < D / 4; ++d4) {
    q[d4] = valid ? qp[d4] : make_float4(0.f, 0.f, 0.f, 0.f);
    o[d4] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -INFINITY, l = 0.f;

  // Tile staging: thread tid moves the 16-byte chunks x = tid + NTHR c (x < 1024) of the
  // tile's K and V.  The next tile's chunks are loaded into registers while the current
  // one is computed.
  constexpr int NCH = BK * D / 4, NC = (NCH + NTHR - 1) / NTHR;
  float4 pk[NC], pv[NC];
  auto fetch = [&](int ent) {
    const int kb = ent >> 1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int x = tid + NTHR * c;
      if (x < NCH) {
        const int r = x / (D / 4), d4 = x - r * (D / 4);
        const int j = kb * BK + r;
        // a valid row in any case; keys past Lk are stored as zeros
        const int64_t o_ = (((int64_t)b * a.Lk + (j < a.Lk ? j : 0)) * a.Hkv + h) * D + 4 * d4;
        pk[c] = *(const float4*)(K + o_);
        pv[c] = *(const float4*)(V + o_);
        if (j >= a.Lk) pk[c] = pv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int x = tid + NTHR * c;
      if (x < NCH) {
        const int r = x / (D / 4), d4 = x - r * (D / 4);
        *(float4*)(sK + r * LDK + 4 * d4) = pk[c];
        *(float4*)(sV + r * LDK + 4 * d4) = pv[c];
      }
    }
  };

  const int e0 = a.row_ptr[item], e1 = a.row_ptr[item + 1];
  if (e0 < e1) fetch(a.row_ent[e0]);
  for (int e = e0; e < e1; ++e) {
    const int ent = a.row_ent[e];
    const int kb = ent >> 1;
    const bool partial = ent & 1;
    __syncthreads();  // every lane is done with the previous tile
    stage();
    __syncthreads();
    if (e + 1 < e1) fetch(a.row_ent[e + 1]);

    float s[KPL];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const int r = SUB * u + ks;
      const float4* kr = (const float4*)(sK + r * LDK);
      float acc = 0.f;
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 kv = kr[d4];
        acc = fmaf(q[d4].x, kv.x, acc);
        acc = fmaf(q[d4].y, kv.y, acc);
        acc = fmaf(q[d4].z, kv.z, acc);
        acc = fmaf(q[d4].w, kv.w, acc);
      }
      const int j = kb * BK + r;
      if (partial && !(valid && visible(p, j, a.Lk, a.win.sink, a.win.near_w, band))) acc = -INFINITY;
      s[u] = acc * a.scale_log2;
      mt = fmaxf(mt, s[u]);
    }
    const float mn = fmaxf(m, mt);
    if (mn == -INFINITY) continue;  // nothing visible yet for this lane's keys
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) {
      o[d4].x *= alpha;
      o[d4].y *= alpha;
      o[d4].z *= alpha;
      o[d4].w *= alpha;
    }
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const float pr = exp2f(s[u] - mn);
      l += pr;
      const float4* vr = (const float4*)(sV + (SUB * u + ks) * LDK);
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 vv = vr[d4];
        o[d4].x = fmaf(pr, vv.x, o[d4].x);
        o[d4].y = fmaf(pr, vv.y, o[d4].y);
        o[d4].z = fmaf(pr, vv.z, o[d4].z);
        o[d4].w = fmaf(pr, vv.w, o[d4].w);
      }
    }
  }

  // merge the row's 16 lane states: the common max, then sums and outputs rescaled to
  // it (a lane that saw nothing has m = -inf and contributes 0)
  float mr = m;
#pragma unroll
  for (int x = 1; x < SUB; x <<= 1) mr = fmaxf(mr, __shfl_xor(mr, x));
  const float f = (m == -INFINITY) ? 0.f : exp2f(m - mr);
  l *= f;
#pragma unroll
  for (int x = 1; x < SUB; x <<= 1) l += __shfl_xor(l, x);
#pragma unroll
  for (int d4 = 0; d4 < D / 4; ++d4) {
    float4 y = o[d4];
    y.x *= f;
    y.y *= f;
    y.z *= f;
    y.w *= f;
#pragma unroll
    for (int x = 1; x < SUB; x <<= 1) {
      y.x += __shfl_xor(y.x, x);
      y.y += __shfl_xor(y.y, x);
      y.z += __shfl_xor(y.z, x);
      y.w += __shfl_xor(y.w, x);
    }
    o[d4] = y;
  }

  if (valid) {
    // lane ks writes the row's columns 4 ks .. 4 ks + 3
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float4* op = (float4*)((float*)a.o + (((int64_t)b * a.Lq + t) * a.Hq + hq) * D);
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4)
      if (d4 == ks) op[d4] = make_float4(o[d4].x * inv, o[d4].y * inv, o[d4].z * inv, o[d4].w * inv);
    if (ks == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Lq + t] = l > 0.f ? (mr + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_f32_d64(const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.n_items, a.B);
  switch (a.G) {  // G <= 4 (checked by the C API)
    case 1: hipLaunchKernelGGL(fwd_f32_d64_kernel<1>, grid, dim3(BQ * 1 * SUB), 0, s, a); break;
    case 2: hipLaunchKernelGGL(fwd_f32_d64_kernel<2>, grid, dim3(BQ * 2 * SUB), 0, s, a); break;
    case 3: hipLaunchKernelGGL(fwd_f32_d64_kernel<3>, grid, dim3(BQ * 3 * SUB), 0, s, a); break;
    default: hipLaunchKernelGGL(fwd_f32_d64_kernel<4>, grid, dim3(BQ * 4 * SUB), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace cowa
