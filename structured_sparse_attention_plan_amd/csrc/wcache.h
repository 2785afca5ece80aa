// Layout of the window-only decode cache, shared by the host layer and the kernels.
//
// A decode query at position p under KV head h sees the prefix sink (keys j < sink) and
// the keys at distance p - j in the near window [0, near) or in the head's band
// [lo_h, hi_h) (slinene.github.io ai-papers-daily page, method key points 1-2).  Distances
// only grow as the sequence advances, so a key j >= sink that is R_h = max(near, hi_h)
// or more positions behind the newest token is never seen by head h again; a key closer
// than that can still be (now, or once the band reaches it).  Each head therefore holds
// the sink keys and a ring of the last R_h positions (each rank holds only the cache its
// window can still reach: same page, practical note 3):
//   slot(j) = j                  for j < S_h (the sink)
//           = S_h + (j mod R_h)  otherwise
// with S_h = min(sink, Lmax), and the whole history (R_h = Lmax, S_h = 0) when the ring
// would reach back to the sink anyway.  Appending position j overwrites position j - R_h,
// which is then R_h behind the newest token.  Heads are laid out one after the other:
// head h's slots start at the sum of the capacities S + R of the heads before it.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cowa.h"

namespace cowa {

struct WinRing {
  int64_t sink_slots;  // S_h
  int64_t ring;        // R_h (0: no ring, only the sink is ever visible)
};

__host__ __device__ inline WinRing wcache_ring(const cowa_window& w, int h, int64_t Lmax) {
  int64_t reach;  // one past the largest distance at which head h sees a key
  if (w.band_mode == COWA_BAND_DENSE) {
    reach = Lmax;
  } else {
    const int64_t slot = (w.band_mode == COWA_BAND_COMPLEMENTARY) ? h : 0;
    const int64_t hi = (int64_t)w.near_w + w.gap + (slot + 1) * (int64_t)w.lr;
    reach = w.lr > 0 ? (hi > w.near_w ? hi : (int64_t)w.near_w) : (int64_t)w.near_w;
  }
  if (reach > Lmax) reach = Lmax;
  const int64_t sink = w.sink < Lmax ? (int64_t)w.sink : Lmax;
  if (reach + sink >= Lmax) return {0, Lmax};  // the ring holds every position
  return {sink, reach};
}

// First slot of head h (h = Hkv: slots per sequence).
__host__ __device__ inline int64_t wcache_offset(const cowa_window& w, int h, int64_t Lmax) {
  int64_t o = 0;
  for (int x = 0; x < h; ++x) {
    const WinRing r = wcache_ring(w, x, Lmax);
    o += r.sink_slots + r.ring;
  }
  return o;
}

// Slot of position j, or -1 when head h never sees it (no ring and j past the sink).
__host__ __device__ inline int64_t wcache_slot(const WinRing& r, int64_t j) {
  if (j < r.sink_slots) return j;
  return r.ring > 0 ? r.sink_slots + (j % r.ring) : -1;
}

}  // namespace cowa
