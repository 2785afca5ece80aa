// CoWindow Attention decode, bf16 KV cache, head dim 128, for gfx950.
//
// One new query token per sequence sits at key position Lk - 1; its bottom-right
// distance to key j is Lk - 1 - j, the same definition the forward uses
// (slinene.github.io ai-papers-daily page, method key point 2).  Each KV head reads
// only the k-blocks in its row of the planner's lists (sink, its own long-range band,
// near window), so HBM traffic is the visible part of the cache only (same page,
// practical note 3 and method key point 3).
//
// Split-KV: work group (split s, KV head h, sequence b) streams a contiguous share of
// the head's visible blocks.  Inside the group, 16 slots of 16 lanes each take one key
// at a time; a lane holds 8 of the 128 dims (16-byte loads, so a slot reads one 256-byte
// K or V row), and the G query heads of the KV head share every K/V read.  Scores are
// reduced across the 16 lanes of a slot with DPP moves; the online softmax runs per slot,
// four keys at a time.  The 16 slots are merged through LDS into one partial (max, sum, o[128]) per
// query head and split; a second kernel merges the splits (log-sum-exp) into O and LSE.

#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 128;
constexpr int BK = kDecBk;
constexpr int SLOTS = 16;

__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

// Sum over the 16 lanes of a row (lanes 16 r .. 16 r + 15), left in every lane of the
// row, with DPP moves (no LDS): pairs by quad permutes (lane ^ 1, lane ^ 2), then the
// half-row mirror pairs the two quads of each 8 lanes and the row mirror the two halves.
// Each step adds the same two values in both lanes of a pair, so all 16 lanes end with
// the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_pair(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum16(float x) {
  x = dpp_pair<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_pair<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_pair<0x141>(x);  // row_half_mirror
  x = dpp_pair<0x140>(x);  // row_mirror
  return x;
}

// Visible 64-key blocks of one query at position p of a sequence of Lb keys (Lb >= 1):
// the prefix sink [0, sink), the near window (p - near, p] and the head's band
// (p - hi, p - lo], each taken to blocks, sorted and merged into at most three disjoint
// ascending runs [ba, bb) (the list the planner gives a one-row q-block).
struct BlockRuns {
  int ba[3], bb[3];
  int n;      // runs
  int total;  // blocks over all runs
};
__device__ __forceinline__ BlockRuns visible_block_runs(int p, int Lb, int sink, int near_w, HeadBand band) {
  int ra[3], rb[3], n = 0;
  if (sink > 0) {
    ra[n] = 0;
    rb[n] = min(sink, Lb);
    ++n;
  }
  if (near_w > 0) {
    ra[n] = max(0, p - near_w + 1);
    rb[n] = p + 1;
    ++n;
  }
  if (band.hi > band.lo && p >= band.lo) {
    ra[n] = max(0, p - band.hi + 1);  // hi clamped to int32 max: dense bands start at 0
    rb[n] = p - band.lo + 1;
    ++n;
  }
  int ba[3], bb[3];
  for (int k = 0; k < n; ++k) {
    ba[k] = ra[k] / kDecBk;
    bb[k] = (rb[k] - 1) / kDecBk + 1;
  }
  // sort three runs by start, then merge overlapping or adjacent ones
  for (int x = 0; x < n; ++x)
    for (int y = x + 1; y < n; ++y)
      if (ba[y] < ba[x]) {
        const int t0 = ba[x], t1 = bb[x];
        ba[x] = ba[y];
        bb[x] = bb[y];
        ba[y] = t0;
        bb[y] = t1;
      }
  BlockRuns r;
  r.n = 0;
  r.total = 0;
  for (int k = 0; k < n; ++k) {
    if (r.n > 0 && ba[k] <= r.bb[r.n - 1]) {
      r.bb[r.n - 1] = max(r.bb[r.n - 1], bb[k]);
    } else {
      r.ba[r.n] = ba[k];
      r.bb[r.n] = bb[k];
      ++r.n;
    }
  }
  for (int k = 0; k < r.n; ++k) r.total += r.bb[k] - r.ba[k];
  return r;
}

// Block of run position e (0 <= e < total), runs in ascending order.
__device__ __forceinline__ int run_block(const BlockRuns& r, int e) {
  int kb = r.ba[0] + e;
  if (r.n > 1 && e >= r.bb[0] - r.ba[0]) {
    e -= r.bb[0] - r.ba[0];
    kb = r.ba[1] + e;
    if (r.n > 2 && e >= r.bb[1] - r.ba[1]) kb = r.ba[2] + (e - (r.bb[1] - r.ba[1]));
  }
  return kb;
}

template <int G, bool VAR>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ float sm[SLOTS][G];
  __shared__ float sl[SLOTS][G];
  __shared__ float so[SLOTS][G][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int slot = tid >> 4;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const HeadBand band = head_band(a.win, h);
  // the sequence's length: the cache capacity, or its own length in varlen mode (clamped
  // to [0, Lk]; a sequence of length 0 sees nothing)
  const int Lb = VAR ? min(max(a.seqlens[b], 0), a.Lk) : a.Lk;
  const int p = Lb - 1;

  // query rows of the G heads, 8 dims per lane, as fp32
  float q[G][8];
  const __bf16* Qb = (const __bf16*)a.q + ((int64_t)b * a.Hq + h * G) * D + 8 * li;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) unpack8(*(const u32x4*)(Qb + gi * D), q[gi]);

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -INFINITY;
    l[gi] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[gi][x] = 0.f;
  }

  // this split's share of the head's visible blocks: entries [s0, s1) of the plan's row
  // list, or of the runs derived from the sequence's length
  BlockRuns runs;
  int e0, e1;
  if constexpr (VAR) {
    runs = Lb > 0 ? visible_block_runs(p, Lb, a.win.sink, a.win.near_w, band) : BlockRuns{{0, 0, 0}, {0, 0, 0}, 0, 0};
    e0 = 0;
    e1 = runs.total;
  } else {
    e0 = a.row_ptr[h];
    e1 = a.row_ptr[h + 1];
  }
  const int chunk = (e1 - e0 + a.nsplit - 1) / a.nsplit;
  const int s0 = e0 + split * chunk;
  const int s1 = min(e1, s0 + chunk);
  const __bf16* Kb = (const __bf16*)a.k + ((int64_t)b * a.Lk * a.Hkv + h) * D + 8 * li;
  const __bf16* Vb = (const __bf16*)a.v + ((int64_t)b * a.Lk * a.Hkv + h) * D + 8 * li;
  const int64_t rstride = (int64_t)a.Hkv * D;

  for (int e = s0; e < s1; ++e) {
    // varlen: every block takes the per-key check (no FULL/PARTIAL flags without a plan)
    const int ent = VAR ? (run_block(runs, e) << 1) | 1 : a.row_ent[e];
    const int kb = ent >> 1;
    const bool partial = ent & 1;
    u32x4 kw[4], vw[4];
    bool ok[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int j = kb * BK + rr * SLOTS + slot;
      ok[rr] = j < Lb;
      const int jj = ok[rr] ? j : 0;
      kw[rr] = *(const u32x4*)(Kb + jj * rstride);
      vw[rr] = *(const u32x4*)(Vb + jj * rstride);
      if (partial) ok[rr] = ok[rr] && visible(p, j, Lb, a.win.sink, a.win.near_w, band);
    }
    float s[4][G];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float kx[8];
      unpack8(kw[rr], kx);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc = fmaf(q[gi][x], kx[x], acc);
        acc = sum16(acc);
        s[rr][gi] = ok[rr] ? acc * a.scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float mt = fmaxf(fmaxf(s[0][gi], s[1][gi]), fmaxf(s[2][gi], s[3][gi]));
      const float mn = fmaxf(m[gi], mt);
      if (mn == -INFINITY) continue;
      const float alpha = (m[gi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[gi] - mn);
      m[gi] = mn;
      l[gi] *= alpha;
#pragma unroll
      for (int x = 0; x < 8; ++x) o[gi][x] *= alpha;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float vx[8];
      unpack8(vw[rr], vx);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float pr = (m[gi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[rr][gi] - m[gi]);
        l[gi] += pr;
#pragma unroll
        for (int x = 0; x < 8; ++x) o[gi][x] = fmaf(pr, vx[x], o[gi][x]);
      }
    }
  }

  // ---- merge the 16 slots
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    if (li == 0) {
      sm[slot][gi] = m[gi];
      sl[slot][gi] = l[gi];
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) so[slot][gi][8 * li + x] = o[gi][x];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int gi = x / D, d = x - gi * D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) M = fmaxf(M, sm[k][gi]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const float w = (sm[k][gi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[k][gi] - M);
        L += w * sl[k][gi];
        acc += w * so[k][gi][d];
      }
    }
    const int64_t row = ((int64_t)b * a.Hq + h * G + gi) * a.nsplit + split;
    a.part[row * D + d] = acc;
    if (d == 0) {
      a.part_ml[2 * row] = M;
      a.part_ml[2 * row + 1] = L;
    }
  }
}

// One work group per (sequence, query head): lane s of the first wave reads split s's
// (max, sum), the weights exp2(m_s - M) go through LDS, and thread d merges dim d.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float w[64];
  __shared__ float tot[2];
  const int bh = blockIdx.x;  // b * Hq + hq
  const int d = threadIdx.x;
  const int64_t base = (int64_t)bh * a.nsplit;
  if (d < 64) {
    const bool in = d < a.nsplit;
    const float ms = in ? a.part_ml[2 * (base + d)] : -INFINITY;
    const float ls = in ? a.part_ml[2 * (base + d) + 1] : 0.f;
    float M = ms;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    const float wt = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    float L = wt * ls;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) L += __shfl_xor(L, x);
    w[d] = wt;
    if (d == 0) {
      tot[0] = M;
      tot[1] = L;
    }
  }
  __syncthreads();
  const float M = tot[0], L = tot[1];
  float acc = 0.f;
  for (int s = 0; s < a.nsplit; ++s) acc += w[s] * a.part[(base + s) * D + d];
  const float out = L > 0.f ? acc / L : 0.f;
  ((__bf16*)a.o)[(int64_t)bh * D + d] = (__bf16)out;
  if (a.lse && d == 0) a.lse[bh] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  if (a.seqlens)
    hipLaunchKernelGGL((decode_split_kernel<G, true>), dim3(a.nsplit, a.Hkv, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<G, false>), dim3(a.nsplit, a.Hkv, a.B), dim3(256), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 5: return launch_g<5>(a, s);
    case 8: return launch_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supports_group(int G) { return G == 1 || G == 2 || G == 4 || G == 5 || G == 8; }

}  // namespace cowa
