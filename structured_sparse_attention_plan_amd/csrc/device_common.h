// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers, LDS
// transpose loads and the window predicate.
//
// MFMA lane layouts (v_mfma_f32_16x16x32_bf16, wave64), with i = lane % 16, g = lane / 16:
//   A (16 x 32): lane holds A[i][8g .. 8g+7]          (8 bf16)
//   B (32 x 16): lane holds B[8g .. 8g+7][i]          (8 bf16)
//   C (16 x 16): lane holds C[4g .. 4g+3][i]          (4 fp32)
// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address of 4
// consecutive bf16 at row r0 + j/4, column c0 + 4 (j%4) of a row-major matrix M; lane i
// then receives M[r0 .. r0+3][c0 + i].  Two such loads give one A/B operand whose 8
// contracted values come from two runs of 4 rows, which is exactly how a C-layout
// accumulator tile maps onto the contracted index of the next product.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace cowa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The fp16 product of the same shape and lane layout; a and b are 16-bit containers
// that hold fp16 bit patterns (LDS reads and packed registers share one type).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x16 mfma32x32x16_f16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                c, 0, 0, 0);
}

// (x0, x1) -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float x0, float x1) {
  const f16x2 h = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, h);
}

// floor(log2 |x|) of a normal fp32 x (x >= 0 here, the max of absolute values); 0 for
// zero and subnormals.  Dividing by 2^e then puts x in [1, 2).
__device__ __forceinline__ int pow2_exponent(float x) {
  const int eb = (int)((__float_as_uint(x) >> 23) & 255u);
  return eb == 0 ? 0 : eb - 127;
}

// Transposed LDS load (see the header comment).  `p` points into __shared__ memory.
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  const lds_i16x4* lp = (const lds_i16x4*)(__attribute__((address_space(3))) const void*)(p);
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lp);
  return __builtin_bit_cast(bf16x4, v);
}

// LDS tiles of 128 bf16 columns use 256-byte rows (every row starts at bank 0) with the
// 16-byte chunks of row r permuted by XOR with lds_sw(r), which is conflict-free for both
// read patterns of the kernels (64 banks of 4 bytes; 16 lanes per cycle for 16-byte
// reads, 32 lanes per cycle for 8-byte reads):
//   * 16-byte operand reads, one chunk of 16 consecutive rows: lds_sw takes 16 distinct
//     values on any 16 consecutive rows;
//   * ds_read_b64_tr_b16, 4 aligned rows x 4 aligned chunks: bits 2-3 of lds_sw(r) are
//     r % 4 and bits 0-1 depend only on r / 4, so the 16 (row, chunk) pairs land on 16
//     distinct chunks.
__device__ __forceinline__ int lds_sw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Element offset of (row r, column e) in such a tile.
__device__ __forceinline__ int lds_swz(int r, int e) {
  return r * 128 + ((((e >> 3) ^ lds_sw(r)) & 15) << 3) + (e & 7);
}

// Read-only plan data with a wave-uniform index, read through the constant address space
// so that it becomes a scalar load (tracked apart from the vector-memory counter that the
// direct LDS copies use).
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// A pointer the compiler can prove wave-uniform (held in scalar registers), so that
// uniform + 32-bit per-lane offset addressing uses the scalar-base form of the load.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource over [base, base + bytes): loads through it take a 32-bit per-lane
// byte offset (plus a scalar one) and return zeros past `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : bytes < 0x7fffffff ? (int)bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr((const char*)base), (short)0, n,
                                           0x00020000);
}

// Resource over [base + off, base + total) (empty when !real): per copy tile only the
// offset product and a 64-bit add and subtract run on the scalar unit, the base and
// total being formed once per work item.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int64_t total, int64_t off,
                                                           bool real) {
  const int64_t left = total - off;
  const int n = (!real || left <= 0) ? 0 : left < 0x7fffffff ? (int)left : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), (short)0, n, 0x00020000);
}

// One 1 KB direct buffer->LDS copy per wave: lane L moves the 16 bytes at byte offset
// voff of the resource to lds + 16 L (lds is wave-uniform).
__device__ __forceinline__ void buf2lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, __bf16* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)voff, 0, 0, 0);
}

// One 1 KB direct global->LDS copy per wave: lane L moves the 16 bytes at src (its own
// address) to lds + 16 L (lds is wave-uniform).
__device__ __forceinline__ void g2lds(const void* src, __bf16* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait for every outstanding vector-memory load of this wave (direct LDS copies
// included), then the work-group barrier.
__device__ __forceinline__ void wait_loads_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 load16(const void* p) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)p);
}

__device__ __forceinline__ void store16(void* p, const bf16x8& v) {
  *(u32x4*)p = __builtin_bit_cast(u32x4, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  r[2] = (__bf16)c;
  r[3] = (__bf16)d;
  return r;
}

// Window of KV head h as distances [lo, hi); hi clamped to int32.
struct HeadBand {
  int32_t lo, hi;
};

// (host and device: the CPU test suite checks visible_run against visible)
__host__ __device__ __forceinline__ HeadBand head_band(const DevWindow& w, int h) {
  int64_t lo = (int64_t)w.band_lo0 + (int64_t)h * w.band_step;
  int64_t hi = lo + w.band_w;
  const int64_t cap = 0x7fffffff;
  return {(int32_t)(lo < cap ? lo : cap), (int32_t)(hi < cap ? hi : cap)};
}

// Key j (< Lk) visible to the query at key position p under a head's window.
__host__ __device__ __forceinline__ bool visible(int p, int j, int Lk, int sink, int near_w, HeadBand b) {
  const int d = p - j;
  return (j < Lk) & (d >= 0) & ((j < sink) | (d < near_w) | ((d >= b.lo) & (d < b.hi)));
}

// The visible keys of one query row inside a boundary tile, as one run: with
// jc = j - jbase (jbase the tile's first key, plus any fixed lane offset), key j is
// visible iff lo <= jc <= hi, for jc in [0, 63].  The window's three parts (sink, band,
// near window) and the causal and Lk limits give at most three runs; when they join
// into one (or none) this returns true, and false when the row sees two or more
// separate runs in the tile (narrow windows or gaps), where the caller tests keys one by
// one.  The parts in ascending order of their first key: sink [0, S1], band [B0, B1],
// near window [N0, R] (the band lies at distances >= near, so it never starts after
// the near window).
__host__ __device__ __forceinline__ bool visible_run(int p, int jbase, int Lk, int sink, int near_w, HeadBand b,
                                            int& lo, int& hi) {
  const int P = p - jbase;                            // d >= 0  <=>  jc <= P
  const int R = min(min(P, Lk - 1 - jbase), 63);      // last key the row may see
  const int Pc = max(P, -1);                          // (R < 0 already when P < 0)
  const int S1 = min(sink - 1 - jbase, R);
  const int B0 = max(Pc - b.hi + 1, 0), B1 = min(Pc - b.lo, R);
  const int N0 = max(Pc - near_w + 1, 0);
  int l = 64, e = -1;  // the union so far: [l, e], empty while e < l
  bool one = true;
  if (S1 >= 0) {
    l = 0;
    e = S1;
  }
  if (B0 <= B1) {
    one &= (e < l) | (B0 <= e + 1);
    l = min(l, B0);
    e = max(e, B1);
  }
  if (N0 <= R) {
    one &= (e < l) | (N0 <= e + 1);
    l = min(l, N0);
    e = max(e, R);
  }
  lo = l;
  hi = e;
  return one;
}


// Visible 64-key blocks of one query at position p of a sequence of Lb >= 1 keys, as at
// most three disjoint ascending runs of blocks [a, b) (the list the planner gives a
// one-row q-block): the prefix sink [0, sink), the head's band of distances [lo, hi) and
// the near window of distances [0, near), each taken to blocks, sorted by first block and
// merged where they overlap or touch.  Slots are fixed (an empty one has a = b = kNoRun)
// and every index is a constant, so the runs stay in registers.
struct BlockRuns {
  int a0, b0, a1, b1, a2, b2;
  int total;  // blocks over the three runs
};
constexpr int kNoRun = 0x3fffffff;

__host__ __device__ __forceinline__ void sort_run_pair(int& a, int& b, int& c, int& d) {
  if (c < a) {
    const int t = a, u = b;
    a = c;
    b = d;
    c = t;
    d = u;
  }
}

__host__ __device__ __forceinline__ BlockRuns visible_block_runs(int p, int Lb, int sink, int near_w, HeadBand band) {
  constexpr int BK = kDecBk;
  BlockRuns r{kNoRun, kNoRun, kNoRun, kNoRun, kNoRun, kNoRun, 0};
  if (sink > 0) {
    r.a0 = 0;
    r.b0 = (min(sink, Lb) - 1) / BK + 1;
  }
  if (near_w > 0) {
    r.a1 = max(0, p - near_w + 1) / BK;
    r.b1 = p / BK + 1;
  }
  if (band.hi > band.lo && p >= band.lo) {
    r.a2 = max(0, p - band.hi + 1) / BK;  // hi clamped to int32 max: dense bands start at 0
    r.b2 = (p - band.lo) / BK + 1;
  }
  sort_run_pair(r.a0, r.b0, r.a1, r.b1);
  sort_run_pair(r.a1, r.b1, r.a2, r.b2);
  sort_run_pair(r.a0, r.b0, r.a1, r.b1);
  // run 1 joins run 0 when it starts at or before run 0's end (both empty: nothing moves)
  if (r.a1 <= r.b0) {
    r.b0 = max(r.b0, r.b1);
    r.a1 = r.b1 = kNoRun;
  }
  // run 2 can only meet the last non-empty run before it (runs 0 and 1 are disjoint
  // when 1 is not empty, and 2 starts no earlier than 1)
  if (r.a1 != kNoRun) {
    if (r.a2 <= r.b1) {
      r.b1 = max(r.b1, r.b2);
      r.a2 = r.b2 = kNoRun;
    }
  } else if (r.a2 <= r.b0) {
    r.b0 = max(r.b0, r.b2);
    r.a2 = r.b2 = kNoRun;
  }
  r.total = (r.b0 - r.a0) + (r.b1 - r.a1) + (r.b2 - r.a2);
  return r;
}

// Block of run position e (0 <= e < total), runs in ascending order.
__host__ __device__ __forceinline__ int run_block(const BlockRuns& r, int e) {
  const int n0 = r.b0 - r.a0, n1 = r.b1 - r.a1;
  return e < n0 ? r.a0 + e : (e < n0 + n1 ? r.a1 + (e - n0) : r.a2 + (e - n0 - n1));
}

// Work queues.
// With `queues` set (one sequence), a work group does not take item order[blockIdx.x]:
// thread 0 takes the next unclaimed position of its own XCD's queue (the launch order's
// positions x, x + 8, ... that round-robin dispatch would give XCD x, in that order) by an
// atomic add on the queue's head, and when that queue is used up the next position of
// another XCD's queue.  XCDs of one chip run the same work up to 3% apart, so a fixed
// deal ends with the slowest; with the queues a fast XCD's work groups take over positions
// a slow one has not reached (the grid has n / 16 + 8 spare work groups for that; a work
// group that finds every queue used up exits).  Each work group makes at most 8 attempts,
// and every position is taken exactly once.  Returns -1 when no position is left.
__device__ __forceinline__ int claim_item(const int32_t* order, int n, int32_t* heads) {
  // XCC_ID hardware register: bits 3:0 hold the XCD of this work group
  const int x = (int)__builtin_amdgcn_s_getreg((31 << 11) | 20) & 7;
  for (int k = 0; k < 8; ++k) {
    const int q = (x + k) & 7;
    const int len = (n - q + 7) / 8;  // positions q, q + 8, ... below n
    if (len <= 0) continue;
    const int i = atomicAdd(heads + q, 1);
    if (i < len) return order[q + 8 * i];
  }
  return -1;
}

// The item of this work group (every thread; one barrier): from the queues when the launch
// has them, else the fixed position blockIdx.x of the launch order.
__device__ __forceinline__ int take_item(const int32_t* order, int n, int32_t* heads, int* slot) {
  if (!heads) return load_uniform(order, blockIdx.x);
  if (threadIdx.x == 0) *slot = claim_item(order, n, heads);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot);
}

}  // namespace cowa
