// Launch interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cowa.h"

namespace cowa {

// Window of one problem as the kernels read it: per KV head h the band is
// [band_lo0 + h * band_step, band_lo0 + h * band_step + band_w) of distances
// (band_step = 0 for duplicated bands; band_w = INT32_MAX/2 for dense mode).
struct DevWindow {
  int32_t sink, near_w;
  int32_t band_lo0, band_step, band_w;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* o_lo;  // bf16 rounding residual of O (may be null)
  float* lse;
  const int32_t* row_ptr;
  const int32_t* row_ent;
  const int32_t* row_order;
  int32_t B, Lq, Lk, Hq, Hkv, G;
  int32_t nqb, nkb, n_items;  // n_items = Hkv * nqb
  int32_t Bq, Bk;    // tokens per q-block, keys per k-block
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  DevWindow win;
  float mala_tau;    // MALA: keep a tile when some row's probability mass in it is >= tau
  int32_t* kept;     // MALA: per row-list entry, 1 if the tile's PV was done (may be null)
  // MALA workspace: per (sequence, row-list entry, row of the item) the log2 of the row's
  // probability numerator in the tile (scoring pass), the kept entries of each item
  // (compacted in list order) and their count per (sequence, item)
  float* mala_mass;        // [B, nnz, kFwdRows]
  int32_t* mala_ents;      // [B, nnz]
  int32_t* mala_counts;    // [B, n_items]
  // workspace (one sequence only, else null): the 8 per-XCD queue heads of the launch,
  // cleared by the launch before it starts
  int32_t* queues;
  int32_t mala_nnz;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* o_lo;  // bf16 rounding residual of O (may be null)
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // workspace [B, Hq, Lq]: Delta = dO . O per row
  float* qscale;  // workspace [B, Hq, Lq]: 2^e with max |q| / 2^e in [1, 2) per row
  float* doexp;   // workspace [B, Hq, Lq]: f with max |dO| / 2^f in [1, 2) per row (0 if dO = 0)
  void* q16;      // workspace [B, Lq, Hq, D] fp16: q / qscale per row
  void* do16;     // workspace [B, Lq, Hq, D] fp16: dO / 2^doexp per row
  void* k16;      // workspace [B, Lk, Hkv, D] fp16: K / 2^gK, one gK per launch
  // workspace: launch-wide maxima (bit patterns of non-negative floats, or biased
  // exponents, compared as unsigned): [0] |dO_i| qscale_i, [1] |Delta_i| qscale_i,
  // [2] doexp + kExpBias over rows with dO != 0, [3] max |k|, [4] max |v_j|^2
  float* maxima;
  const int32_t* row_ptr;
  const int32_t* row_ent;
  const int32_t* row_order;
  const int32_t* col_ptr;
  const int32_t* col_ent;
  const int32_t* col_order;
  int32_t B, Lq, Lk, Hq, Hkv, G;
  int32_t nqb, nkb;
  int32_t Bq, Bk;
  float scale, scale_log2;
  DevWindow win;
  // MALA backward: keep flags [Hkv, mala_nqb, mala_nkb] by (KV head, forward q-block of
  // mala_bq tokens, 64-key block); null for the CoWA backward
  const uint8_t* mala_mask;
  int32_t mala_bq, mala_nqb, mala_nkb;
  // workspace (one sequence only, else null): per-XCD queue heads of the dQ launch [0, 8)
  // and of the dK/dV launch [8, 16); each launch clears its own before it starts
  int32_t* queues;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;        // may be null
  float* part;       // workspace: [B, Hq, nsplit, D] partial outputs
  float* part_ml;    // workspace: [B, Hq, nsplit, 2] (max in log2 units, sum)
  const int32_t* row_ptr;
  const int32_t* row_ent;
  const int32_t* seqlens;  // varlen / window-cache decode: [B] cache lengths (no plan); else null
  int32_t B, Lk, Hq, Hkv, G;
  int32_t Bk, nsplit;
  float scale_log2;
  DevWindow win;
  // window-only cache (wcache.h): k, v are [B, wslots, D]; null window_mode: full caches
  int32_t window_mode;
  int64_t wslots;
  cowa_window cwin;
};

struct WcacheAppendArgs {
  void* k;  // window caches [B, wslots, D]
  void* v;
  const void* k_new;  // [B, T, Hkv, D]
  const void* v_new;
  const int32_t* pos0;  // [B] position of each sequence's first new token
  int32_t B, T, Hkv, Lmax;
  int64_t wslots;
  cowa_window cwin;
};

hipError_t launch_fwd_f32_d64(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16_d128(const FwdArgs& a, hipStream_t s);
hipError_t launch_mala_fwd_bf16_d128(const FwdArgs& a, hipStream_t s);  // scoring, then the gated pass
// MALA backward: the forward's per-entry keep flags scattered to a dense mask
struct MalaMaskArgs {
  uint8_t* mask;           // [n_items, nkb]
  const int32_t* row_ptr;  // the forward plan's row lists
  const int32_t* row_ent;
  const int32_t* kept;     // per forward entry
  int32_t n_items, nkb;
};
hipError_t launch_mala_mask(const MalaMaskArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16_d128(const BwdArgs& a, int stages, hipStream_t s);
hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t s);  // varlen when a.seqlens
hipError_t launch_wcache_append(const WcacheAppendArgs& a, hipStream_t s);
bool decode_supports_group(int G);

// Tile shapes of each kernel family (tokens per q-block, keys per k-block).
constexpr int kF32Bq = 8, kF32Bk = 64;
constexpr int kFwdRows = 256;  // query rows (tokens x GQA heads) per forward work item
constexpr int kFwdBk = 64;
constexpr int kBwdRows = 128;  // query rows per backward q-block
constexpr int kBwdBk = 128;
constexpr int kDecBk = 64;
constexpr int kDecSplitBlocks = 16;  // k-blocks per decode split (upper bound)
constexpr int kExpBias = 256;        // bias of exponents kept as unsigned maxima

}  // namespace cowa
