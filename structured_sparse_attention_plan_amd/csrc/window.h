// Window convention shared by the planner, the host layer and the kernels.
//
// KV head h (global index) owns the long-range band [lo, hi) of bottom-right causal
// distances (slinene.github.io ai-papers-daily page, method key points 1-2): the bands
// start after the near window and a gap, have equal width lr, and are laid out in head
// order (complementary mode); duplicated mode gives every head the first band, dense
// mode widens each band to every larger distance.
#pragma once

#include <cstdint>

#include "cowa.h"

namespace cowa {

constexpr int64_t kUnbounded = INT64_MAX / 4;

struct Band {
  int64_t lo, hi;  // hi == kUnbounded: no upper edge
  bool unbounded() const { return hi >= kUnbounded; }
  int64_t width() const { return hi > lo ? hi - lo : 0; }
};

inline bool window_valid(const cowa_window& w) {
  return w.sink >= 0 && w.near_w >= 0 && w.gap >= 0 && w.lr >= 0 &&
         w.band_mode >= COWA_BAND_COMPLEMENTARY && w.band_mode <= COWA_BAND_DENSE;
}

inline Band band_of(const cowa_window& w, int32_t h) {
  const int64_t start = (int64_t)w.near_w + w.gap;
  if (w.band_mode == COWA_BAND_DENSE) return {start, kUnbounded};
  const int64_t slot = (w.band_mode == COWA_BAND_COMPLEMENTARY) ? h : 0;
  const int64_t lo = start + slot * (int64_t)w.lr;
  return {lo, lo + w.lr};
}

}  // namespace cowa
