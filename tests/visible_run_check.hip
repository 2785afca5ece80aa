// Host check of the kernels' run test for boundary tiles: for random windows, heads,
// sequence lengths, query positions and tiles, wherever visible_run reports a single
// run it must equal the per-key window predicate on every key of the tile, and wherever
// it reports more than one run the predicate must indeed show two separate runs.  Then
// the plan-free decode's block runs (visible_block_runs / run_block): for random windows
// and sequence lengths, the blocks they list, in order, must be exactly the ascending
// 64-key blocks that hold a key visible to the sequence's last position.
// Built with hipcc and run on the host by tests/test_visible_run.py (no GPU needed).
#include <cstdio>
#include <random>

#include "device_common.h"

using namespace cowa;

int main() {
  std::mt19937 rng(20261203);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  long tiles = 0, single = 0, several = 0;
  for (int it = 0; it < 400000; ++it) {
    // small and large windows, narrow bands, gaps; the three band modes
    const int scale = uni(0, 2) == 0 ? 8 : 600;
    DevWindow w;
    w.sink = uni(0, 2) == 0 ? 0 : uni(0, scale);
    w.near_w = uni(0, scale);
    const int gap = uni(0, 3) == 0 ? uni(0, scale) : 0;
    const int lr = uni(0, scale);
    const int mode = uni(0, 2);  // complementary, duplicated, dense
    w.band_lo0 = w.near_w + gap;
    w.band_step = mode == 0 ? lr : 0;
    w.band_w = mode == 2 ? 0x3fffffff : lr;
    const HeadBand b = head_band(w, uni(0, 7));
    const int Lk = uni(1, 5000);
    const int kb = uni(0, (Lk - 1) / 64);
    const int jbase = 64 * kb + 4 * uni(0, 1);  // the lane offset 4 h2
    // query position: anywhere (negative: a query before the keys), or so that the tile
    // meets the diagonal, the near window's end or an edge of the band
    int p = uni(-130, Lk + 130);
    const int edge = uni(0, 7);
    if (edge == 1) p = jbase + uni(-70, 70);
    if (edge == 2) p = jbase + w.near_w + uni(-70, 70);
    if (edge == 3 && b.lo < (1 << 20)) p = jbase + b.lo + uni(-70, 70);
    if (edge == 4 && b.hi < (1 << 20)) p = jbase + b.hi + uni(-70, 70);
    int lo = 0, hi = 0;
    const bool one = visible_run(p, jbase, Lk, w.sink, w.near_w, b, lo, hi);
    bool vis[64];
    int runs = 0;
    for (int jc = 0; jc < 64; ++jc) {
      vis[jc] = visible(p, jbase + jc, Lk, w.sink, w.near_w, b);
      if (vis[jc] && (jc == 0 || !vis[jc - 1])) ++runs;
    }
    ++tiles;
    if (one) {
      ++single;
      for (int jc = 0; jc < 64; ++jc) {
        if (vis[jc] != (lo <= jc && jc <= hi)) {
          std::printf("mismatch: sink %d near %d lo0 %d step %d w %d band [%d, %d) Lk %d p %d jbase %d "
                      "jc %d run [%d, %d] visible %d\n",
                      w.sink, w.near_w, w.band_lo0, w.band_step, w.band_w, b.lo, b.hi, Lk, p, jbase, jc,
                      lo, hi, (int)vis[jc]);
          return 1;
        }
      }
    } else {
      ++several;
      if (runs < 2) {
        std::printf("reported several runs, predicate shows %d: sink %d near %d band [%d, %d) Lk %d p %d "
                    "jbase %d\n", runs, w.sink, w.near_w, b.lo, b.hi, Lk, p, jbase);
        return 1;
      }
    }
  }
  std::printf("%ld tiles: %ld as one run (checked key by key), %ld with several runs\n", tiles, single,
              several);

  long seqs = 0, blocks = 0, multi = 0;
  static bool want[5000 / 64 + 2];
  for (int it = 0; it < 60000; ++it) {
    const int scale = uni(0, 2) == 0 ? 70 : 900;
    DevWindow w;
    w.sink = uni(0, 2) == 0 ? 0 : uni(0, scale);
    w.near_w = uni(0, 4) == 0 ? 0 : uni(1, scale);
    const int gap = uni(0, 3) == 0 ? uni(0, scale) : 0;
    const int lr = uni(0, scale);
    const int mode = uni(0, 2);
    w.band_lo0 = w.near_w + gap;
    w.band_step = mode == 0 ? lr : 0;
    w.band_w = mode == 2 ? 0x3fffffff : lr;
    const HeadBand b = head_band(w, uni(0, 7));
    const int Lb = uni(0, 3) == 0 ? uni(1, 200) : uni(1, 5000);
    const int p = Lb - 1;
    const int nkb = (Lb + 63) / 64;
    int nwant = 0;
    for (int kb = 0; kb < nkb; ++kb) {
      want[kb] = false;
      for (int j = 64 * kb; j < 64 * kb + 64 && j < Lb; ++j) want[kb] |= visible(p, j, Lb, w.sink, w.near_w, b);
      nwant += want[kb];
    }
    const BlockRuns r = visible_block_runs(p, Lb, w.sink, w.near_w, b);
    ++seqs;
    multi += (r.a1 != kNoRun);
    if (r.total != nwant) {
      std::printf("block runs: %d blocks listed, %d visible: sink %d near %d band [%d, %d) Lb %d\n", r.total,
                  nwant, w.sink, w.near_w, b.lo, b.hi, Lb);
      return 1;
    }
    int prev = -1;
    for (int e = 0; e < r.total; ++e) {
      const int kb = run_block(r, e);
      if (kb <= prev || kb >= nkb || !want[kb]) {
        std::printf("block runs: entry %d is block %d (previous %d): sink %d near %d band [%d, %d) Lb %d\n", e,
                    kb, prev, w.sink, w.near_w, b.lo, b.hi, Lb);
        return 1;
      }
      prev = kb;
      ++blocks;
    }
  }
  std::printf("%ld sequences: %ld blocks listed in order (%ld with more than one run)\n", seqs, blocks, multi);
  return 0;
}
