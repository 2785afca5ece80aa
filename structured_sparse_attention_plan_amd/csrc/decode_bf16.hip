// CoWindow Attention decode, bf16 KV cache, head dim 128, for gfx950.
//
// One new query token per sequence sits at key position Lk - 1; its bottom-right
// distance to key j is Lk - 1 - j, the same definition the forward uses
// (slinene.github.io ai-papers-daily page, method key point 2).  Each KV head reads
// only the k-blocks in its row of the planner's lists (sink, its own long-range band,
// near window), so HBM traffic is the visible part of the cache only (same page,
// practical note 3 and method key point 3).
//
// Split-KV: one wave per (split s, KV head h, sequence b) streams a contiguous share of
// the head's visible 64-key blocks.  The G <= 8 query rows of the KV head are the 16
// columns of v_mfma_f32_16x16x32_bf16 products (columns past G hold zeros and are never
// written), so the matrix cores take the dot products and the VALU only the softmax:
//   S^T = K Q^T: K (A operand, one key per lane and 8 dims) is loaded from HBM straight
//     into registers one block ahead; Q^T (B operand) stays in registers;
//   O^T += V^T P^T: P^T goes from the softmax registers into the B operand and V^T is
//     read with ds_read_b64_tr_b16 from a row-major V tile that direct buffer->LDS copies
//     fill one block ahead (two buffers).
// The softmax keeps a running max per query row (the four lane groups of a row share it
// through two cross-lane maxima per block); O and l are rescaled only in blocks where a
// row's max rises.  The wave's partial (max, sum, O) per query head goes to the
// workspace, and a second kernel merges the splits (log-sum-exp) into O and LSE.
//
// MFMA lane layouts of v_mfma_f32_16x16x32_bf16 (n = lane % 16, g = lane / 16):
//   A (16 x 32): A[n][8 g + e]   B (32 x 16): B[8 g + e][n]   C (16 x 16): C[4 g + i][n]

#include <type_traits>

#include "device_common.h"
#include "wcache.h"

namespace cowa {
namespace {

constexpr int D = 128;
constexpr int BK = kDecBk;      // 64 keys per block
constexpr int TILE = BK * D;    // elements of one V tile

template <int V>
using IC = std::integral_constant<int, V>;

// MODE: 0 full caches with the planner's row list; 1 full caches, each sequence's
// visible blocks derived from its length (varlen); 2 window-only caches (wcache.h), blocks
// derived from the length as in mode 1, each key read from its head's slot.
template <int MODE>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  constexpr bool VAR = MODE != 0;
  // V tiles of blocks e (even e: sV0) and e + 1, rows of 256 bytes with XOR-swizzled
  // 16-byte chunks (lds_swz); one array per buffer, so that the compiler tells the reads
  // of one from the copies in flight into the other
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[TILE];
  auto vbuf = [&](auto c) -> __bf16* {
    if constexpr (decltype(c)::value == 0) return sV0;
    else return sV1;
  };

  const int lane = threadIdx.x;
  const int n = lane & 15;  // query row (B / C column) or key (A row) of the lane
  const int g = lane >> 4;  // lane group
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.G;
  const HeadBand band = head_band(a.win, h);
  // the sequence's length: the cache capacity, or its own length in varlen mode (clamped
  // to [0, Lk]; a sequence of length 0 sees nothing)
  const int Lb = VAR ? min(max(a.seqlens[b], 0), a.Lk) : a.Lk;
  const int p = Lb - 1;
  const float c2 = a.scale_log2;  // scores to base-2 units (scale > 0)

  // Q^T operands, k-chunk kc = dims 32 kc .. 32 kc + 31: row n's dims 32 kc + 8 g .. + 7
  bf16x8 qf[4];
  {
    const __bf16* qr = (const __bf16*)a.q + ((int64_t)b * a.Hq + h * G + (n < G ? n : 0)) * D + 8 * g;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qf[kc] = n < G ? load16(qr + 32 * kc) : zero_bf16x8();
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
    e0 = load_uniform(a.row_ptr, h);
    e1 = load_uniform(a.row_ptr, h + 1);
  }
  // Every list is spread over all nsplit splits (ceil(n / nsplit) blocks each), so a
  // short list (a short sequence, a head whose band lies before the sequence start) keeps
  // as many loads in flight as a long one.  Planned and plan-free decodes of the same
  // query split alike (equal results, bit for bit).
  const int chunk = (e1 - e0 + a.nsplit - 1) / a.nsplit;
  const int s0 = e0 + split * chunk;
  const int s1 = min(e1, s0 + chunk);
  auto entry = [&](int e) -> int {  // (block << 1) | partial; plan-free blocks are checked
    if constexpr (VAR) return (run_block(runs, e) << 1) | 1;
    else return load_uniform(a.row_ent, e);
  };

  // Addressing.  Full caches: key j of head h at row (b Lk + j) Hkv + h; a block's loads go
  // through a resource from its first key's row over its keys below Lb (the rest read
  // zeros), at byte offset r Hkv 256 for key r of the block.  Window caches: head h's
  // slots of sequence b, key j at slot(j), a resource over the head's slots.
  //   K loads: lane (n, g) of load (kq, kc) reads key 16 kq + n, dims 32 kc + 8 g .. + 7;
  //   V copies: lane L of copy u fills tile row r = 4 u + L / 16 at physical chunk L % 16,
  //     i.e. logical chunk (L % 16) ^ lds_sw(r) of that key's row.
  const int rowb = MODE == 2 ? D * 2 : a.Hkv * D * 2;  // bytes between consecutive keys
  WinRing ring{0, 0};
  int64_t hbase = 0;
  if constexpr (MODE == 2) {
    ring = wcache_ring(a.cwin, h, a.Lk);
    hbase = wcache_offset(a.cwin, h, a.Lk);
  }
  const int rs = (int)ring.sink_slots, rr_ = (int)ring.ring;
  const char* const kseq = MODE == 2 ? (const char*)a.k + ((int64_t)b * a.wslots + hbase) * (D * 2)
                                     : (const char*)a.k + ((int64_t)b * a.Lk * a.Hkv + h) * (D * 2);
  const char* const vseq = MODE == 2 ? (const char*)a.v + ((int64_t)b * a.wslots + hbase) * (D * 2)
                                     : (const char*)a.v + ((int64_t)b * a.Lk * a.Hkv + h) * (D * 2);
  // per-lane offsets inside a block (full caches: fixed; window caches: per block)
  uint32_t vk[4], vv[16];
  auto block_offsets = [&](int kb) {
    if constexpr (MODE == 2) {
      // slot of key j = kb BK + r: a block past the sink with a ring of at least a block
      // maps onto one or two runs of the ring (slot rs + m0 + r, less the ring once it
      // wraps); otherwise j inside the sink, else sink + (j mod ring); keys past Lb or
      // that the head never holds read slot 0 (masked)
      const int kb0 = kb * BK;
      const bool fast = rr_ >= BK && kb0 >= rs;
      const int m0 = fast ? kb0 % rr_ : 0;
      auto slot = [&](int r) {
        const int j = kb0 + r;
        int sl;
        if (fast) {
          const int m = m0 + r;
          sl = rs + (m >= rr_ ? m - rr_ : m);
        } else {
          sl = (j < rs) ? j : (rr_ > 0 ? rs + j % rr_ : 0);
        }
        return j < Lb ? sl : 0;
      };
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) vk[kq] = (uint32_t)slot(16 * kq + n) * (D * 2) + 16u * g;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int r = 4 * u + (lane >> 4);
        vv[u] = (uint32_t)slot(r) * (D * 2) + 16u * (uint32_t)((lane & 15) ^ lds_sw(r));
      }
    } else {
      (void)kb;
    }
  };
  if constexpr (MODE != 2) {
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) vk[kq] = (uint32_t)(16 * kq + n) * rowb + 16u * g;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = 4 * u + (lane >> 4);
      vv[u] = (uint32_t)r * rowb + 16u * (uint32_t)((lane & 15) ^ lds_sw(r));
    }
  }
  auto block_rsrc = [&](const char* base, int kb) {
    if constexpr (MODE == 2) {
      return make_rsrc(base, (int64_t)(rs + rr_) * (D * 2));
    } else {
      const int rows = min(Lb - kb * BK, BK);
      return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kb * BK * rowb), (short)0,
                                               rows * rowb, 0x00020000);
    }
  };
  bf16x8 kf[2][4][4];  // K of blocks e (even e: [0]) and e + 1: [kq][kc]
  auto issue_block = [&](int ent, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int kb = ent >> 1;
    block_offsets(kb);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vseq, kb);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kseq, kb);
    __bf16* const dst = vbuf(IC<BUF>{});
#pragma unroll
    for (int u = 0; u < 16; ++u) buf2lds(rv, vv[u], dst + 4 * u * D);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        kf[BUF][kq][kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, vk[kq] + 64 * kc, 0, 0));
  };

  // V^T operand reads: lane (j, g) gives the address of row 32 cc + 16 hf + 4 g + j / 4,
  // dims 16 db + 4 (j % 4) .. + 3 and receives 4 keys of dim 16 db + j; under the swizzle
  // the offset for db is the db = 0 one XOR db << 4
  const int vt0 = lds_swz(4 * g + (n >> 2), 4 * (n & 3));
  auto vfrag = [&](const __bf16* vt, int cc, int db) {
    const int o = (vt0 ^ (db << 4)) + 32 * cc * D;
    return join(lds_read_tr4(vt + o), lds_read_tr4(vt + o + 16 * D));
  };

  f32x4 acc[8];  // O^T: element i of acc[db] is dim 16 db + 4 g + i of row n
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // row n's max (base 2) and this lane's share of its sum

  auto step = [&](auto bufc, int e, int ent) {
    constexpr int BUF = decltype(bufc)::value;
    // block e + 1 into the other buffers while block e is computed
    const bool more = e + 1 < s1;
    __builtin_amdgcn_sched_barrier(0);
    if (more) issue_block(entry(e + 1), IC<BUF ^ 1>{});
    __builtin_amdgcn_sched_barrier(0);
    // block e resident: its 16 copies and 16 loads were issued before the 32 of block e + 1
    if (more) __builtin_amdgcn_s_waitcnt(0x8f70);  // vmcnt(32)
    else __builtin_amdgcn_s_waitcnt(0x0f70);       // vmcnt(0)

    const int kb = ent >> 1;
    f32x4 s[4];  // S^T: element i of s[kq] is key 16 kq + 4 g + i of row n
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      s[kq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) s[kq] = mfma16x16x32(kf[BUF][kq][kc], qf[kc], s[kq]);
    }
    // boundary block (every plan-free block is checked): the row's visible keys of the
    // block as one run where they form one, else the window predicate per key
    if (ent & 1) {
      int lo = 0, hi = BK - 1;
      const bool one = visible_run(p, kb * BK, Lb, a.win.sink, a.win.near_w, band, lo, hi);
      if (!(one && lo == 0 && hi == BK - 1)) {
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jc = 16 * kq + 4 * g + i;
            const bool vis = one ? (jc >= lo) & (jc <= hi)
                                 : visible(p, kb * BK + jc, Lb, a.win.sink, a.win.near_w, band);
            s[kq][i] = vis ? s[kq][i] : -INFINITY;
          }
      }
    }
    // running max of the row (base 2): the lane's 16 keys, then the four lane groups
    float mx = -INFINITY;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kq][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * c2;
    if (__builtin_amdgcn_ballot_w64(mt > m) != 0) {
      const bool up = mt > m;
      const float alpha = (m == -INFINITY || !up) ? (up ? 0.f : 1.f) : __builtin_amdgcn_exp2f(m - mt);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
      m = up ? mt : m;
    }
    // a max of -inf (no visible key yet) gives probabilities of 0 through a reference of 0
    const float mref = m == -INFINITY ? 0.f : m;
    bf16x8 pb[2];  // P^T operands of key chunks cc: keys 32 cc + 4 g + 0..3, then + 16
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[kq][i], c2, -mref));
        l += pr;
        pb[kq >> 1][4 * (kq & 1) + i] = (__bf16)pr;
      }
    const __bf16* const vt = vbuf(IC<BUF>{});
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] = mfma16x16x32(vfrag(vt, cc, db), pb[cc], acc[db]);
  };

  if (s0 < s1) {
    int ent = entry(s0);
    issue_block(ent, IC<0>{});
    for (int e = s0; e < s1; e += 2) {
      step(IC<0>{}, e, ent);
      if (e + 1 < s1) {
        ent = entry(e + 1);
        step(IC<1>{}, e + 1, ent);
        if (e + 2 < s1) ent = entry(e + 2);
      }
    }
  }

  // the row's sum over the four lane groups; lane (n, g) writes dims 16 db + 4 g .. + 3
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (n < G) {
    const int64_t row = ((int64_t)b * a.Hq + h * G + n) * a.nsplit + split;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(a.part + row * D + 16 * db + 4 * g) = acc[db];
    if (g == 0) {
      a.part_ml[2 * row] = m;
      a.part_ml[2 * row + 1] = l;
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

}  // namespace

hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t s) {
  if (!decode_supports_group(a.G)) return hipErrorInvalidValue;
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  if (a.window_mode)
    hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(64), 0, s, a);
  else if (a.seqlens)
    hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_split_kernel<0>, grid, dim3(64), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

// every group size up to 8 (the query rows of a KV head are columns of 16-wide products)
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
