// Launch interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // workspace [B, Hq, Lq]: Delta = dO . O per row
  float* qscale;  // workspace [B, Hq, Lq]: 2^e with max |q| / 2^e in [1, 2) per row
  void* q16;      // workspace [B, Lq, Hq, D] fp16: q / qscale per row
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
  const int32_t* seqlens;  // varlen decode: [B] cache lengths (no plan); else null
  int32_t B, Lk, Hq, Hkv, G;
  int32_t Bk, nsplit;
  float scale_log2;
  DevWindow win;
};

hipError_t launch_fwd_f32_d64(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16_d128(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16_d128(const BwdArgs& a, int stages, hipStream_t s);
hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t s);  // varlen when a.seqlens
bool decode_supports_group(int G);

// Tile shapes of each kernel family (tokens per q-block, keys per k-block).
constexpr int kF32Bq = 64, kF32Bk = 64;
constexpr int kFwdRows = 256;  // query rows (tokens x GQA heads) per forward work item
constexpr int kFwdBk = 64;
constexpr int kBwdRows = 128;  // query rows per backward q-block
constexpr int kBwdBk = 128;
constexpr int kDecBk = 64;
constexpr int kDecSplitBlocks = 16;  // k-blocks per decode split (upper bound)

}  // namespace cowa
