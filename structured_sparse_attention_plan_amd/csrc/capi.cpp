// C-ABI host layer of libcowa: argument validation, tile sizes, workspace sizing and
// kernel launch.  Nothing here allocates device memory or keeps state between calls;
// every error is reported before anything is enqueued.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cowa.h"
#include "kernels.h"
#include "window.h"

namespace {

using namespace cowa;

bool same_window(const cowa_window& a, const cowa_window& b) {
  return a.sink == b.sink && a.near_w == b.near_w && a.gap == b.gap && a.lr == b.lr &&
         a.band_mode == b.band_mode;
}

DevWindow dev_window(const cowa_window& w) {
  DevWindow d;
  d.sink = w.sink;
  d.near_w = w.near_w;
  d.band_lo0 = w.near_w + w.gap;
  d.band_step = (w.band_mode == COWA_BAND_COMPLEMENTARY) ? w.lr : 0;
  d.band_w = (w.band_mode == COWA_BAND_DENSE) ? 0x3fffffff : w.lr;
  return d;
}

// Shape checks common to every op.  Lengths are capped at 2^30 so that every distance
// and band edge fits int32 on the device.
int check_problem(const cowa_problem* p) {
  if (!p) return COWA_ERR_INVALID_ARG;
  if (p->B < 1 || p->Lq < 1 || p->Lk < 1 || p->Hq < 1 || p->Hkv < 1 || p->D < 1)
    return COWA_ERR_INVALID_ARG;
  if (!(p->scale > 0.f)) return COWA_ERR_INVALID_ARG;
  if (!window_valid(p->win)) return COWA_ERR_INVALID_ARG;
  if (p->Hq % p->Hkv != 0) return COWA_ERR_UNSUPPORTED;
  if (p->B > 65535 || p->Lq > (1 << 30) || p->Lk > (1 << 30)) return COWA_ERR_UNSUPPORTED;
  if ((int64_t)p->win.near_w + p->win.gap + (int64_t)p->Hkv * p->win.lr > (1 << 30))
    return COWA_ERR_UNSUPPORTED;
  return COWA_OK;
}

int check_op_support(int op, const cowa_problem* p) {
  const int G = p->Hq / p->Hkv;
  switch (op) {
    case COWA_OP_FWD:
      if (p->dtype == COWA_DTYPE_F32) return (p->D == 64 && G <= 4) ? COWA_OK : COWA_ERR_UNSUPPORTED;
      if (p->dtype == COWA_DTYPE_BF16) return (p->D == 128 && G <= kFwdRows) ? COWA_OK : COWA_ERR_UNSUPPORTED;
      return COWA_ERR_UNSUPPORTED;
    case COWA_OP_BWD:
      return (p->dtype == COWA_DTYPE_BF16 && p->D == 128 && G <= kBwdRows) ? COWA_OK
                                                                           : COWA_ERR_UNSUPPORTED;
    case COWA_OP_DECODE:
      if (p->dtype != COWA_DTYPE_BF16 || p->D != 128 || p->Lq != 1) return COWA_ERR_UNSUPPORTED;
      return decode_supports_group(G) ? COWA_OK : COWA_ERR_UNSUPPORTED;
    default:
      return COWA_ERR_INVALID_ARG;
  }
}

void tiles_for(int op, const cowa_problem* p, int32_t* Bq, int32_t* Bk) {
  const int G = p->Hq / p->Hkv;
  switch (op) {
    case COWA_OP_FWD:
      if (p->dtype == COWA_DTYPE_F32) {
        *Bq = kF32Bq;
        *Bk = kF32Bk;
      } else {
        *Bq = kFwdRows / G;
        *Bk = kFwdBk;
      }
      return;
    case COWA_OP_BWD:
      *Bq = kBwdRows / G;
      *Bk = kBwdBk;
      return;
    default:  // decode: one query row
      *Bq = 1;
      *Bk = kDecBk;
      return;
  }
}

int check_plan(int op, const cowa_problem* p, const cowa_plan_dev* plan, bool need_cols) {
  if (!plan || !plan->row_ptr || !plan->row_ent || !plan->row_order) return COWA_ERR_INVALID_ARG;
  if (need_cols && (!plan->col_ptr || !plan->col_ent || !plan->col_order)) return COWA_ERR_INVALID_ARG;
  int32_t Bq, Bk;
  tiles_for(op, p, &Bq, &Bk);
  const cowa_plan_info& in = plan->info;
  if (in.Lq != p->Lq || in.Lk != p->Lk || in.Hkv != p->Hkv || in.Bq != Bq || in.Bk != Bk)
    return COWA_ERR_PLAN_MISMATCH;
  if (in.nqb != (p->Lq + Bq - 1) / Bq || in.nkb != (p->Lk + Bk - 1) / Bk) return COWA_ERR_PLAN_MISMATCH;
  if (!same_window(plan->win, p->win)) return COWA_ERR_PLAN_MISMATCH;
  return COWA_OK;
}

int decode_splits(const cowa_problem* p) {
  const int32_t nkb = (p->Lk + kDecBk - 1) / kDecBk;
  int64_t want = (4096 + (int64_t)p->B * p->Hkv - 1) / ((int64_t)p->B * p->Hkv);
  if (want > 64) want = 64;
  if (want > nkb) want = nkb;
  return want < 1 ? 1 : (int)want;
}

int hip_status(hipError_t e) { return e == hipSuccess ? COWA_OK : COWA_ERR_HIP; }

}  // namespace

extern "C" const char* cowa_status_string(int status) {
  switch (status) {
    case COWA_OK: return "ok";
    case COWA_ERR_INVALID_ARG: return "invalid argument";
    case COWA_ERR_UNSUPPORTED: return "unsupported problem (dtype, head dim, group size or size limit)";
    case COWA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case COWA_ERR_PLAN_MISMATCH: return "plan was built for another shape, window or tiling";
    case COWA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int cowa_tile_sizes(int op, const cowa_problem* p, int32_t* Bq, int32_t* Bk) {
  if (!Bq || !Bk) return COWA_ERR_INVALID_ARG;
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(op, p);
  if (st != COWA_OK) return st;
  tiles_for(op, p, Bq, Bk);
  return COWA_OK;
}

extern "C" int cowa_workspace_size(int op, const cowa_problem* p, size_t* bytes) {
  if (!bytes) return COWA_ERR_INVALID_ARG;
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(op, p);
  if (st != COWA_OK) return st;
  switch (op) {
    case COWA_OP_FWD:
      *bytes = 0;
      break;
    case COWA_OP_BWD: {  // Delta, the row scales of Q and the fp16 copy of Q
      const size_t rows = (size_t)p->B * p->Hq * p->Lq;
      *bytes = 2 * ((rows * sizeof(float) + 255) / 256 * 256) + rows * p->D * 2;
      break;
    }
    default: {
      const size_t rows = (size_t)p->B * p->Hq * decode_splits(p);
      const size_t part = (rows * p->D * sizeof(float) + 255) / 256 * 256;
      *bytes = part + rows * 2 * sizeof(float);
    }
  }
  return COWA_OK;
}

extern "C" int cowa_fwd(const cowa_problem* p, const cowa_plan_dev* plan, const void* q, const void* k,
                        const void* v, void* o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_FWD, p);
  if (st != COWA_OK) return st;
  if (!q || !k || !v || !o || !lse) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_FWD, p, plan, false);
  if (st != COWA_OK) return st;

  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.row_ptr = plan->row_ptr;
  a.row_ent = plan->row_ent;
  a.row_order = plan->row_order;
  a.B = p->B;
  a.Lq = p->Lq;
  a.Lk = p->Lk;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.nqb = plan->info.nqb;
  a.nkb = plan->info.nkb;
  a.n_items = p->Hkv * plan->info.nqb;
  a.Bq = plan->info.Bq;
  a.Bk = plan->info.Bk;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.44269504088896340736f;
  a.win = dev_window(p->win);
  hipStream_t s = (hipStream_t)stream;
  if (p->dtype == COWA_DTYPE_F32) return hip_status(launch_fwd_f32_d64(a, s));
  return hip_status(launch_fwd_bf16_d128(a, s));
}

extern "C" int cowa_bwd(const cowa_problem* p, const cowa_plan_dev* plan, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const void* dout, void* dq,
                        void* dk, void* dv, int stages, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_BWD, p);
  if (st != COWA_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return COWA_ERR_INVALID_ARG;
  if (stages < 1 || stages > COWA_BWD_ALL) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_BWD, p, plan, true);
  if (st != COWA_OK) return st;
  size_t need = 0;
  cowa_workspace_size(COWA_OP_BWD, p, &need);
  if (!workspace || workspace_bytes < need) return COWA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return COWA_ERR_INVALID_ARG;

  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t row_bytes = ((size_t)p->B * p->Hq * p->Lq * sizeof(float) + 255) / 256 * 256;
  a.delta = (float*)workspace;
  a.qscale = (float*)((char*)workspace + row_bytes);
  a.q16 = (char*)workspace + 2 * row_bytes;
  a.row_ptr = plan->row_ptr;
  a.row_ent = plan->row_ent;
  a.row_order = plan->row_order;
  a.col_ptr = plan->col_ptr;
  a.col_ent = plan->col_ent;
  a.col_order = plan->col_order;
  a.B = p->B;
  a.Lq = p->Lq;
  a.Lk = p->Lk;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.nqb = plan->info.nqb;
  a.nkb = plan->info.nkb;
  a.Bq = plan->info.Bq;
  a.Bk = plan->info.Bk;
  a.scale = p->scale;
  a.scale_log2 = p->scale * 1.44269504088896340736f;
  a.win = dev_window(p->win);
  return hip_status(launch_bwd_bf16_d128(a, stages, (hipStream_t)stream));
}

extern "C" int cowa_decode(const cowa_problem* p, const cowa_plan_dev* plan, const void* q,
                           const void* k_cache, const void* v_cache, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_DECODE, p);
  if (st != COWA_OK) return st;
  if (!q || !k_cache || !v_cache || !o) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_DECODE, p, plan, false);
  if (st != COWA_OK) return st;
  size_t need = 0;
  cowa_workspace_size(COWA_OP_DECODE, p, &need);
  if (!workspace || workspace_bytes < need) return COWA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return COWA_ERR_INVALID_ARG;

  DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse = lse;
  a.nsplit = decode_splits(p);
  const size_t rows = (size_t)p->B * p->Hq * a.nsplit;
  a.part = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + (rows * p->D * sizeof(float) + 255) / 256 * 256);
  a.row_ptr = plan->row_ptr;
  a.row_ent = plan->row_ent;
  a.B = p->B;
  a.Lk = p->Lk;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.Bk = plan->info.Bk;
  a.scale_log2 = p->scale * 1.44269504088896340736f;
  a.win = dev_window(p->win);
  return hip_status(launch_decode_bf16_d128(a, (hipStream_t)stream));
}

extern "C" int cowa_decode_varlen(const cowa_problem* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seqlens_k, void* o, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_DECODE, p);
  if (st != COWA_OK) return st;
  if (!q || !k_cache || !v_cache || !o || !seqlens_k) return COWA_ERR_INVALID_ARG;
  size_t need = 0;
  cowa_workspace_size(COWA_OP_DECODE, p, &need);
  if (!workspace || workspace_bytes < need) return COWA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return COWA_ERR_INVALID_ARG;

  DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse = lse;
  a.nsplit = decode_splits(p);
  const size_t rows = (size_t)p->B * p->Hq * a.nsplit;
  a.part = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + (rows * p->D * sizeof(float) + 255) / 256 * 256);
  a.seqlens = seqlens_k;
  a.B = p->B;
  a.Lk = p->Lk;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.Bk = kDecBk;
  a.scale_log2 = p->scale * 1.44269504088896340736f;
  a.win = dev_window(p->win);
  return hip_status(launch_decode_bf16_d128(a, (hipStream_t)stream));
}
