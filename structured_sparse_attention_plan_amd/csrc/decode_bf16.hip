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
#include "wcache.h"

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

// MODE: 0 full caches with the planner's row list; 1 full caches, each sequence's
// visible blocks derived from its length (varlen); 2 window-only caches (wcache.h), blocks
// derived from the length as in mode 1, each key read from its head's slot.
template <int G, int MODE>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr bool VAR = MODE != 0;
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

  // query rows of the G heads, 8 dims per lane, as fp32, times scale log2(e): the scores
  // come out in base-2 units
  float q[G][8];
  const __bf16* Qb = (const __bf16*)a.q + ((int64_t)b * a.Hq + h * G) * D + 8 * li;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    unpack8(*(const u32x4*)(Qb + gi * D), q[gi]);
#pragma unroll
    for (int x = 0; x < 8; ++x) q[gi][x] *= a.scale_log2;
  }

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
    runs = Lb > 0 ? visible_block_runs(p, Lb, a.win.sink, a.win.near_w, band)
                   : BlockRuns{0, 0, 0, 0, 0, 0, 0};
    e0 = 0;
    e1 = runs.total;
  } else {
    e0 = a.row_ptr[h];
    e1 = a.row_ptr[h + 1];
  }
  // Every list is spread over all nsplit splits (ceil(n / nsplit) blocks each), so a
  // short list (a short sequence, a head whose band lies before the sequence start) keeps
  // as many loads in flight as a long one.  (A split size fixed per launch, which left
  // short lists on fewer splits, took 6% longer for 16 sequences of 64K-125K at 128K
  // capacity and the same for full caches.)  Planned and plan-free decodes of the same
  // query split alike (equal results, bit for bit).
  const int chunk = (e1 - e0 + a.nsplit - 1) / a.nsplit;
  const int s0 = e0 + split * chunk;
  const int s1 = min(e1, s0 + chunk);
  // full caches: row j of head h at [b, j, h]; window caches: head h's slot of j in
  // [b, wslots, D], the ring offset of a block's first key taken once per block
  WinRing ring{0, 0};
  int64_t hbase = 0;
  if constexpr (MODE == 2) {
    ring = wcache_ring(a.cwin, h, a.Lk);
    hbase = wcache_offset(a.cwin, h, a.Lk);
  }
  const int rs = (int)ring.sink_slots, rr_ = (int)ring.ring;
  const __bf16* Kb = MODE == 2 ? (const __bf16*)a.k + ((int64_t)b * a.wslots + hbase) * D + 8 * li
                               : (const __bf16*)a.k + ((int64_t)b * a.Lk * a.Hkv + h) * D + 8 * li;
  const __bf16* Vb = MODE == 2 ? (const __bf16*)a.v + ((int64_t)b * a.wslots + hbase) * D + 8 * li
                               : (const __bf16*)a.v + ((int64_t)b * a.Lk * a.Hkv + h) * D + 8 * li;
  const int64_t rstride = MODE == 2 ? (int64_t)D : (int64_t)a.Hkv * D;

  for (int e = s0; e < s1; ++e) {
    // varlen: every block takes the per-key check (no FULL/PARTIAL flags without a plan)
    const int ent = VAR ? (run_block(runs, e) << 1) | 1 : a.row_ent[e];
    const int kb = ent >> 1;
    const bool partial = ent & 1;
    u32x4 kw[4], vw[4];
    bool ok[4];
    // window caches: a block past the sink with a ring of at least a block maps onto one
    // or two runs of the ring: slot rs + m0 + offset, less the ring once it wraps
    const int kb0 = __builtin_amdgcn_readfirstlane(kb) * BK;
    const bool ring_fast = MODE == 2 && rr_ >= BK && kb0 >= rs;
    const int m0 = ring_fast ? kb0 % rr_ : 0;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int off_in = rr * SLOTS + slot;
      const int j = kb * BK + off_in;
      ok[rr] = j < Lb;
      int jj = ok[rr] ? j : 0;
      if constexpr (MODE == 2) {
        if (ring_fast) {
          const int m = m0 + off_in;
          jj = rs + (m >= rr_ ? m - rr_ : m);
        } else {
          // slot of key j: j inside the sink, else sink + (j mod ring); keys a head never
          // sees (no ring) read slot 0 and are masked below
          jj = (jj < rs) ? jj : (rr_ > 0 ? rs + jj % rr_ : 0);
        }
        if (!ok[rr]) jj = 0;
      }
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
        s[rr][gi] = ok[rr] ? acc : -INFINITY;
      }
    }
    // running max per (slot, head): O and l are rescaled only in blocks where some
    // lane's max rises (after the first few blocks, rarely); a max of -inf (no visible key
    // yet) gives probabilities of 0 through a reference of 0
    bool rises = false;
    float mnew[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float mt = fmaxf(fmaxf(s[0][gi], s[1][gi]), fmaxf(s[2][gi], s[3][gi]));
      mnew[gi] = fmaxf(m[gi], mt);
      rises |= mnew[gi] > m[gi];
    }
    if (__builtin_amdgcn_ballot_w64(rises) != 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float alpha = (m[gi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[gi] - mnew[gi]);
        const bool up = mnew[gi] > m[gi];
        m[gi] = mnew[gi];
        l[gi] = up ? l[gi] * alpha : l[gi];
#pragma unroll
        for (int x = 0; x < 8; ++x) o[gi][x] = up ? o[gi][x] * alpha : o[gi][x];
      }
    }
    float mref[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) mref[gi] = m[gi] == -INFINITY ? 0.f : m[gi];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float vx[8];
      unpack8(vw[rr], vx);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float pr = __builtin_amdgcn_exp2f(s[rr][gi] - mref[gi]);
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
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  if (a.window_mode)
    hipLaunchKernelGGL((decode_split_kernel<G, 2>), grid, dim3(256), 0, s, a);
  else if (a.seqlens)
    hipLaunchKernelGGL((decode_split_kernel<G, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<G, 0>), grid, dim3(256), 0, s, a);
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
    case 3: return launch_g<3>(a, s);
    case 4: return launch_g<4>(a, s);
    case 5: return launch_g<5>(a, s);
    case 6: return launch_g<6>(a, s);
    case 7: return launch_g<7>(a, s);
    case 8: return launch_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// every group size up to 8 (the query rows of a KV head live in registers: G x 16 each)
bool decode_supports_group(int G) { return G >= 1 && G <= 8; }

// ---------------------------------------------------------------------- window cache append
// Row (b, t, h) of the new tokens (position pos0[b] + t) goes to head h's slot.  Of the
// chunk's positions that share a ring slot only the last one is written (the others are
// R_h or more behind the chunk's newest token, so head h never sees them again), which
// keeps the writes of one launch disjoint.  Sixteen lanes per 256-byte row.
namespace {
__global__ __launch_bounds__(256) void wcache_append_kernel(WcacheAppendArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int li = threadIdx.x & 15;
  if (row >= (int64_t)a.B * a.T * a.Hkv) return;
  const int h = (int)(row % a.Hkv);
  const int64_t bt = row / a.Hkv;
  const int t = (int)(bt % a.T);
  const int b = (int)(bt / a.T);
  const int64_t p0 = a.pos0[b];
  const int64_t j = p0 + t;
  if (j < 0 || j >= a.Lmax) return;
  const WinRing r = wcache_ring(a.cwin, h, a.Lmax);
  const bool keep = j < r.sink_slots || (r.ring > 0 && j >= p0 + a.T - r.ring);
  if (!keep) return;
  const int64_t dst = ((int64_t)b * a.wslots + wcache_offset(a.cwin, h, a.Lmax) + wcache_slot(r, j)) * D + 8 * li;
  const int64_t src = row * D + 8 * li;
  *(u32x4*)((__bf16*)a.k + dst) = *(const u32x4*)((const __bf16*)a.k_new + src);
  *(u32x4*)((__bf16*)a.v + dst) = *(const u32x4*)((const __bf16*)a.v_new + src);
}
}  // namespace

hipError_t launch_wcache_append(const WcacheAppendArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.T * a.Hkv;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(wcache_append_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cowa
