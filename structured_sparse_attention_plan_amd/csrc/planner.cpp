// Block-visibility planner for CoWindow Attention.
//
// The traversal of the operator visits only KV blocks that hold visible keys
// (slinene.github.io ai-papers-daily page, "CoWindow Attention: Full Causal Coverage Is
// a Collective Property", method key point 3).  For a block of consecutive query rows
// every window — prefix sink, near diagonal and the head's long-range band (method key
// point 1) — is a key interval whose end points move by one per row, so the keys a
// q-block can see are the union of at most three intervals.  The planner turns those
// into k-block ranges and emits them, so its work is proportional to the number of
// visible tiles: masked tiles are never enumerated.
//
// Host-only code: no device memory, no HIP calls.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "cowa.h"
#include "window.h"

namespace {

struct Range {  // half-open [a, b)
  int64_t a, b;
};

// Keys any row of [p0, p1] (positions p = i + Lk - Lq) can see, as up to three
// half-open key intervals (empty ones dropped).
int block_key_ranges(const cowa::Band& band, int64_t sink, int64_t near_w, int64_t p0,
                     int64_t p1, Range out[3]) {
  int n = 0;
  // prefix sink: keys [0, sink) that are causal for some row
  if (sink > 0 && p1 >= 0) out[n++] = {0, std::min<int64_t>(sink, p1 + 1)};
  // near diagonal: distances [0, near) -> keys (p - near, p]
  if (near_w > 0 && p1 >= 0) out[n++] = {std::max<int64_t>(0, p0 - near_w + 1), p1 + 1};
  // long-range band: distances [lo, hi) -> keys (p - hi, p - lo]; rows with p < lo see none
  if (band.width() > 0 && p1 >= band.lo) {
    int64_t pf = std::max<int64_t>(p0, band.lo);
    int64_t a = band.unbounded() ? 0 : std::max<int64_t>(0, pf - band.hi + 1);
    out[n++] = {a, p1 - band.lo + 1};
  }
  return n;
}

// Number of keys a single row at position p sees (union of its three intervals).
int64_t row_visible(const cowa::Band& band, int64_t sink, int64_t near_w, int64_t p) {
  Range r[3];
  int n = block_key_ranges(band, sink, near_w, p, p, r);
  std::sort(r, r + n, [](const Range& x, const Range& y) { return x.a < y.a; });
  int64_t total = 0, end = 0;
  for (int k = 0; k < n; ++k) {
    int64_t a = std::max(r[k].a, end);
    if (r[k].b > a) {
      total += r[k].b - a;
      end = r[k].b;
    }
  }
  return total;
}

// True iff every (row, key) of rows [p0, p1] x keys [j0, j1] (inclusive) is visible.
// Keys below `sink` are visible iff causal; for the others visibility depends only on
// the distance d = p - j, and the tile covers every d in [p0 - j1, p1 - j0'].
bool tile_full(const cowa::Band& band, int64_t sink, int64_t near_w, int64_t p0, int64_t p1,
               int64_t j0, int64_t j1) {
  if (j0 < sink) {  // sink part [j0, min(j1, sink - 1)]
    int64_t js = std::min<int64_t>(j1, sink - 1);
    if (p0 - js < 0) return false;
  }
  int64_t jr = std::max<int64_t>(j0, sink);
  if (jr > j1) return true;
  int64_t dlo = p0 - j1, dhi = p1 - jr;
  if (dlo < 0) return false;
  if (dhi < near_w) return true;
  if (band.width() > 0) {
    bool below_hi = band.unbounded() || dhi < band.hi;
    if (dlo >= band.lo && below_hi) return true;
    // near window and band touch or overlap: one run [0, hi)
    if (band.lo <= near_w && below_hi) return true;
  }
  return false;
}

}  // namespace

extern "C" int cowa_window_make(int32_t Lmax, int32_t Hkv, int32_t sink, int32_t near_w,
                                int32_t gap, int32_t band_mode, cowa_window* out) {
  if (!out || Hkv < 1 || Lmax < 0 || sink < 0 || near_w < 0 || gap < 0) return COWA_ERR_INVALID_ARG;
  if (band_mode < COWA_BAND_COMPLEMENTARY || band_mode > COWA_BAND_DENSE) return COWA_ERR_INVALID_ARG;
  int64_t rest = (int64_t)Lmax - near_w - gap;
  out->sink = sink;
  out->near_w = near_w;
  out->gap = gap;
  out->lr = rest > 0 ? (int32_t)((rest + Hkv - 1) / Hkv) : 0;
  out->band_mode = band_mode;
  return COWA_OK;
}

extern "C" int cowa_plan_blocks(int32_t Lq, int32_t Lk, int32_t Hkv, int32_t Bq, int32_t Bk,
                                const cowa_window* win, cowa_plan_info* info, int32_t* row_ptr,
                                int32_t* row_ent, int32_t* col_ptr, int32_t* col_ent,
                                int32_t* row_order, int32_t* col_order) {
  if (!win || !info) return COWA_ERR_INVALID_ARG;
  if (Lq < 1 || Lk < 1 || Hkv < 1 || Bq < 1 || Bk < 1) return COWA_ERR_INVALID_ARG;
  if (!cowa::window_valid(*win)) return COWA_ERR_INVALID_ARG;
  const bool want = row_ptr || row_ent || col_ptr || col_ent || row_order || col_order;
  if (want && !(row_ptr && row_ent && col_ptr && col_ent && row_order && col_order))
    return COWA_ERR_INVALID_ARG;

  const int64_t off = (int64_t)Lk - Lq;
  const int32_t nqb = (Lq + Bq - 1) / Bq, nkb = (Lk + Bk - 1) / Bk;
  const int64_t sink = win->sink, near_w = win->near_w;

  // Pass 1: per row item, the merged k-block ranges; counts and edges.
  std::vector<int32_t> row_cnt((size_t)Hkv * nqb, 0);
  int64_t nnz = 0, n_partial = 0, edges = 0, visited = 0;
  std::vector<int32_t> ents;  // only filled when the caller wants the lists
  std::vector<int32_t> col_cnt(want ? (size_t)Hkv * nkb : 0, 0);
  if (want) row_ptr[0] = 0;

  for (int32_t h = 0; h < Hkv; ++h) {
    const cowa::Band band = cowa::band_of(*win, h);
    for (int64_t i = 0; i < Lq; ++i) edges += row_visible(band, sink, near_w, i + off);
    for (int32_t qb = 0; qb < nqb; ++qb) {
      const int64_t r0 = (int64_t)qb * Bq, r1 = std::min<int64_t>(Lq, r0 + Bq) - 1;
      const bool rows_whole = (r0 + Bq) <= Lq;
      const int64_t p0 = r0 + off, p1 = r1 + off;
      Range kr[3];
      int n = block_key_ranges(band, sink, near_w, p0, p1, kr);
      // key ranges -> k-block ranges, merged in ascending order
      Range br[3];
      for (int k = 0; k < n; ++k) {
        int64_t a = std::max<int64_t>(0, kr[k].a), b = std::min<int64_t>(Lk, kr[k].b);
        br[k] = (b > a) ? Range{a / Bk, (b - 1) / Bk + 1} : Range{0, 0};
      }
      std::sort(br, br + n, [](const Range& x, const Range& y) { return x.a < y.a; });
      int64_t end = 0;
      int32_t cnt = 0;
      for (int k = 0; k < n; ++k) {
        for (int64_t kb = std::max(br[k].a, end); kb < br[k].b; ++kb) {
          ++visited;
          const int64_t j0 = kb * Bk, j1 = std::min<int64_t>(Lk, j0 + Bk) - 1;
          const bool keys_whole = (j0 + Bk) <= Lk;
          const bool full = rows_whole && keys_whole && tile_full(band, sink, near_w, p0, p1, j0, j1);
          n_partial += full ? 0 : 1;
          ++cnt;
          if (want) {
            ents.push_back((int32_t)((kb << 1) | (full ? 0 : 1)));
            ++col_cnt[(size_t)h * nkb + kb];
          }
        }
        end = std::max(end, br[k].b);
      }
      row_cnt[(size_t)h * nqb + qb] = cnt;
      nnz += cnt;
      if (nnz > INT32_MAX) return COWA_ERR_UNSUPPORTED;
      if (want) row_ptr[(size_t)h * nqb + qb + 1] = (int32_t)nnz;
    }
  }

  info->Lq = Lq;
  info->Lk = Lk;
  info->Hkv = Hkv;
  info->Bq = Bq;
  info->Bk = Bk;
  info->nqb = nqb;
  info->nkb = nkb;
  info->nnz = nnz;
  info->n_partial = n_partial;
  info->visited = visited;
  info->edges = edges;
  if (!want) return COWA_OK;

  std::memcpy(row_ent, ents.data(), sizeof(int32_t) * (size_t)nnz);

  // Column lists: transpose, keeping q-blocks ascending within a column.
  col_ptr[0] = 0;
  for (size_t c = 0; c < col_cnt.size(); ++c) col_ptr[c + 1] = col_ptr[c] + col_cnt[c];
  std::vector<int32_t> fill(col_ptr, col_ptr + col_cnt.size());
  for (int32_t h = 0; h < Hkv; ++h)
    for (int32_t qb = 0; qb < nqb; ++qb) {
      const size_t it = (size_t)h * nqb + qb;
      for (int32_t e = row_ptr[it]; e < row_ptr[it + 1]; ++e) {
        const int32_t kb = COWA_ENT_BLOCK(row_ent[e]);
        col_ent[fill[(size_t)h * nkb + kb]++] = (qb << 1) | COWA_ENT_PARTIAL(row_ent[e]);
      }
    }

  // Launch orders.  Work groups are dispatched in launch order, round-robin over the 8
  // XCDs (work group b runs on XCD b % 8), and each XCD has its own L2 and its own queue:
  // its CUs take its work groups in order, so the launch ends when the XCD with the most
  // work ends, and every XCD holds the same number of items (one position in eight).
  //  1. Heavy items first: an item whose list is more than twice the mean length (the
  //     columns holding the prefix sink are seen by every row) goes first, longest first,
  //     so that it does not start late and run alone at the end of the launch.
  //  2. The rest in parts: every head's blocks are cut into contiguous parts of at least
  //     16 blocks (at most 64 parts per head; shorter parts only where an XCD's share is
  //     under 64 items), and the parts are dealt longest first, each to the
  //     XCD with the least work so far that still has room for it (a part that fits
  //     nowhere whole is split into consecutive pieces for the XCDs with the most room).  Work is estimated as the list length
  //     plus 4 entries of per-item start-up.  An XCD runs its parts in the order it was
  //     dealt them, each part's blocks in ascending order, so the items it runs together
  //     are neighbouring blocks of one head, which read the same K/V (or Q/dO) tiles from
  //     its L2; with parts this small every XCD's estimated work ends within about one
  //     part of the others' (with 8 equal-count parts per head, one per XCD, the XCDs'
  //     work differed by up to 2.5% at 131072 tokens and 4% at 32768).
  auto xcd_order = [&](int32_t nblk, const int32_t* ptr, int32_t* order) {
    constexpr int X = 8;
    constexpr int64_t kStartup = 4;
    const int64_t nitem = (int64_t)Hkv * nblk;
    const double mean = (double)ptr[nitem] / (double)nitem;
    auto work = [&](int64_t it) { return (int64_t)(ptr[it + 1] - ptr[it]) + kStartup; };
    std::vector<int32_t> heavy;
    for (int64_t it = 0; it < nitem; ++it)
      if (ptr[it + 1] - ptr[it] > 2.0 * mean) heavy.push_back((int32_t)it);
    std::stable_sort(heavy.begin(), heavy.end(), [&](int32_t x, int32_t y) {
      return ptr[x + 1] - ptr[x] > ptr[y + 1] - ptr[y];
    });
    std::vector<char> is_heavy((size_t)nitem, 0);
    for (int32_t it : heavy) is_heavy[it] = 1;
    const int64_t nh = (int64_t)heavy.size();
    for (int64_t p = 0; p < nh; ++p) order[p] = heavy[p];
    // positions left to each XCD, and its work so far
    int64_t room[X], load[X] = {};
    for (int x = 0; x < X; ++x) room[x] = (nitem - x + X - 1) / X;
    for (int64_t p = 0; p < nh; ++p) {
      --room[p % X];
      load[p % X] += work(heavy[p]);
    }
    // parts: [lo, hi) of one head's blocks, heavy items left out when dealt
    struct Part {
      int64_t lo, hi, work;
    };
    // part length: at least 16 blocks (64 parts per head at most), and at most a quarter
    // of an XCD's share, so that parts fit whole
    const int64_t share = nitem / X;
    const int64_t plen = std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(16, nblk / 64), share / 4));
    const int32_t K = (int32_t)std::max<int64_t>(1, nblk / plen);
    std::vector<Part> parts;
    for (int32_t hh = 0; hh < Hkv; ++hh)
      for (int32_t k = 0; k < K; ++k) {
        Part pt{hh * (int64_t)nblk + (int64_t)k * nblk / K, hh * (int64_t)nblk + (int64_t)(k + 1) * nblk / K, 0};
        for (int64_t it = pt.lo; it < pt.hi; ++it)
          if (!is_heavy[it]) pt.work += work(it);
        parts.push_back(pt);
      }
    std::stable_sort(parts.begin(), parts.end(), [](const Part& a, const Part& b) { return a.work > b.work; });
    std::vector<std::vector<int32_t>> stream(X);
    auto least_loaded = [&](int64_t need) {
      int best = -1;
      for (int x = 0; x < X; ++x)
        if (room[x] >= need && (best < 0 || load[x] < load[best])) best = x;
      return best;
    };
    std::vector<int32_t> its;
    auto deal = [&](int x, size_t from, size_t to) {
      for (size_t i = from; i < to; ++i) {
        stream[x].push_back(its[i]);
        --room[x];
        load[x] += work(its[i]);
      }
    };
    for (const Part& pt : parts) {
      its.clear();
      for (int64_t it = pt.lo; it < pt.hi; ++it)
        if (!is_heavy[it]) its.push_back((int32_t)it);
      const int x = least_loaded((int64_t)its.size());
      if (x >= 0) {
        deal(x, 0, its.size());
        continue;
      }
      // no XCD has room for the whole part: consecutive pieces to the XCDs with the most
      // room left
      for (size_t i = 0; i < its.size();) {
        int xm = 0;
        for (int xx = 1; xx < X; ++xx)
          if (room[xx] > room[xm]) xm = xx;
        const size_t take = std::min<size_t>((size_t)room[xm], its.size() - i);
        deal(xm, i, i + take);
        i += take;
      }
    }
    // XCD x's items go to its positions p = x, x + 8, ... after the heavy items
    for (int x = 0; x < X; ++x) {
      int64_t p = nh + ((x - nh) % X + X) % X;
      for (int32_t it : stream[x]) {
        order[p] = it;
        p += X;
      }
    }
  };
  xcd_order(nqb, row_ptr, row_order);
  xcd_order(nkb, col_ptr, col_order);
  return COWA_OK;
}
