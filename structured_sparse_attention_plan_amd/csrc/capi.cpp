// C-ABI host layer of libcowa: argument validation, tile sizes, workspace sizing and
// kernel launch.  Nothing here allocates device memory or keeps state between calls;
// every error is reported before anything is enqueued.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "cowa.h"
#include "kernels.h"
#include "wcache.h"
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
    case COWA_OP_MALA_FWD:
      return (p->dtype == COWA_DTYPE_BF16 && p->D == 128 && G <= kFwdRows) ? COWA_OK
                                                                           : COWA_ERR_UNSUPPORTED;
    case COWA_OP_MALA_BWD:  // one sequence: the forward's keep flags exist for B = 1 only
      return (p->dtype == COWA_DTYPE_BF16 && p->D == 128 && G <= kBwdRows && p->B == 1)
                 ? COWA_OK
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
    case COWA_OP_MALA_FWD:
      if (p->dtype == COWA_DTYPE_F32) {
        *Bq = kF32Bq;
        *Bk = kF32Bk;
      } else {
        *Bq = kFwdRows / G;
        *Bk = kFwdBk;
      }
      return;
    case COWA_OP_BWD:
    case COWA_OP_MALA_BWD:
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

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Byte offsets of the backward workspace: three fp32 arrays per (query head, row) (Delta,
// the row scales of Q, the row exponents of dO), 256 bytes of launch-wide maxima, then
// the fp16 copies of Q and dO ([B, Lq, Hq, D]) and of K ([B, Lk, Hkv, D]).
struct BwdLayout {
  size_t delta, qscale, doexp, maxima, q16, do16, k16, total;
};
BwdLayout bwd_layout(const cowa_problem* p) {
  const size_t rows = (size_t)p->B * p->Hq * p->Lq;
  const size_t rowf = round256(rows * sizeof(float));
  const size_t rowh = round256(rows * p->D * 2);
  BwdLayout l;
  l.delta = 0;
  l.qscale = rowf;
  l.doexp = 2 * rowf;
  l.maxima = 3 * rowf;
  l.q16 = l.maxima + 256;
  l.do16 = l.q16 + rowh;
  l.k16 = l.do16 + rowh;
  l.total = l.k16 + round256((size_t)p->B * p->Lk * p->Hkv * p->D * 2);
  return l;
}

// MALA forward workspace: per (sequence, forward entry, row) the scoring pass's log2 row
// numerator (fp32), the kept entries per (sequence, entry) and their counts per
// (sequence, item).
struct MalaFwdLayout {
  size_t mass, ents, counts, total;
};
MalaFwdLayout mala_fwd_layout(const cowa_problem* p, int64_t nnz, int64_t n_items) {
  MalaFwdLayout l;
  l.mass = 0;
  l.ents = round256((size_t)p->B * (size_t)nnz * kFwdRows * sizeof(float));
  l.counts = l.ents + round256((size_t)p->B * (size_t)nnz * sizeof(int32_t));
  l.total = l.counts + round256((size_t)p->B * (size_t)n_items * sizeof(int32_t));
  return l;
}

// MALA backward: the forward's tiling (Bq_f tokens, 64 keys) and the byte mask of its
// keep flags [Hkv, nqb_f, nkb_f] after the backward workspace.
struct MalaTiles {
  int32_t bq, nqb, nkb;
  size_t mask_bytes;
};
MalaTiles mala_tiles(const cowa_problem* p) {
  MalaTiles t;
  tiles_for(COWA_OP_FWD, p, &t.bq, &t.nkb);
  t.nkb = (p->Lk + kFwdBk - 1) / kFwdBk;
  t.nqb = (p->Lq + t.bq - 1) / t.bq;
  t.mask_bytes = round256((size_t)p->Hkv * t.nqb * t.nkb);
  return t;
}

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
    case COWA_OP_FWD:  // bf16: the optional per-XCD work queue heads (cowa_fwd)
      *bytes = p->dtype == COWA_DTYPE_BF16 ? 256 : 0;
      break;
    case COWA_OP_BWD:
      *bytes = bwd_layout(p).total;
      break;
    case COWA_OP_MALA_BWD:
      *bytes = bwd_layout(p).total + mala_tiles(p).mask_bytes;
      break;
    case COWA_OP_MALA_FWD: {  // the number of visible forward tiles, from the planner's count
      int32_t Bq, Bk;
      tiles_for(COWA_OP_FWD, p, &Bq, &Bk);
      cowa_plan_info info{};
      st = cowa_plan_blocks(p->Lq, p->Lk, p->Hkv, Bq, Bk, &p->win, &info, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr);
      if (st != COWA_OK) return st;
      *bytes = mala_fwd_layout(p, info.nnz, (int64_t)p->Hkv * info.nqb).total;
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
                        const void* v, void* o, float* lse, void* o_lo, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_FWD, p);
  if (st != COWA_OK) return st;
  if (!q || !k || !v || !o || !lse) return COWA_ERR_INVALID_ARG;
  if (o_lo && p->dtype != COWA_DTYPE_BF16) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_FWD, p, plan, false);
  if (st != COWA_OK) return st;

  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o_lo = o_lo;
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
  // the optional workspace holds the launch's per-XCD work queue heads (one sequence)
  if (p->dtype == COWA_DTYPE_BF16 && p->B == 1 && workspace && workspace_bytes >= 256 &&
      ((uintptr_t)workspace & 255) == 0)
    a.queues = (int32_t*)workspace;
  hipStream_t s = (hipStream_t)stream;
  if (p->dtype == COWA_DTYPE_F32) return hip_status(launch_fwd_f32_d64(a, s));
  return hip_status(launch_fwd_bf16_d128(a, s));
}

extern "C" int cowa_mala_fwd(const cowa_problem* p, const cowa_plan_dev* plan, float tau, const void* q,
                             const void* k, const void* v, void* o, float* lse, void* o_lo,
                             int32_t* kept, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_MALA_FWD, p);
  if (st != COWA_OK) return st;
  if (!q || !k || !v || !o || !lse || !(tau >= 0.f)) return COWA_ERR_INVALID_ARG;
  if (kept && p->B != 1) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_FWD, p, plan, false);
  if (st != COWA_OK) return st;
  const MalaFwdLayout wl = mala_fwd_layout(p, plan->info.nnz, (int64_t)p->Hkv * plan->info.nqb);
  if (!workspace || workspace_bytes < wl.total) return COWA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return COWA_ERR_INVALID_ARG;
  if (plan->info.nnz > INT32_MAX) return COWA_ERR_UNSUPPORTED;
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
  a.o_lo = o_lo;
  a.mala_tau = tau;
  a.kept = kept;
  char* const ws = (char*)workspace;
  a.mala_mass = (float*)(ws + wl.mass);
  a.mala_ents = (int32_t*)(ws + wl.ents);
  a.mala_counts = (int32_t*)(ws + wl.counts);
  a.mala_nnz = (int32_t)plan->info.nnz;
  return hip_status(launch_mala_fwd_bf16_d128(a, (hipStream_t)stream));
}

namespace {
// The backward's arguments (everything but the MALA fields) after the checks passed.
BwdArgs bwd_args(const cowa_problem* p, const cowa_plan_dev* plan, const void* q, const void* k,
                 const void* v, const void* o, const void* o_lo, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* workspace) {
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o_lo = o_lo;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const BwdLayout wl = bwd_layout(p);
  char* const ws = (char*)workspace;
  a.delta = (float*)(ws + wl.delta);
  a.qscale = (float*)(ws + wl.qscale);
  a.doexp = (float*)(ws + wl.doexp);
  a.maxima = (float*)(ws + wl.maxima);
  // per-XCD work queues of the dQ and dK/dV launches, in the unused half of the maxima
  // block (one sequence: the launch orders cover one sequence's items)
  a.queues = p->B == 1 ? (int32_t*)(ws + wl.maxima + 128) : nullptr;
  a.q16 = ws + wl.q16;
  a.do16 = ws + wl.do16;
  a.k16 = ws + wl.k16;
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
  return a;
}
}  // namespace

extern "C" int cowa_bwd(const cowa_problem* p, const cowa_plan_dev* plan, const void* q, const void* k,
                        const void* v, const void* o, const void* o_lo, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int stages, void* workspace,
                        size_t workspace_bytes, void* stream) {
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
  const BwdArgs a = bwd_args(p, plan, q, k, v, o, o_lo, lse, dout, dq, dk, dv, workspace);
  return hip_status(launch_bwd_bf16_d128(a, stages, (hipStream_t)stream));
}

extern "C" int cowa_mala_bwd(const cowa_problem* p, const cowa_plan_dev* fwd_plan,
                             const cowa_plan_dev* plan, const int32_t* kept, const void* q,
                             const void* k, const void* v, const void* o, const void* o_lo,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_MALA_BWD, p);
  if (st != COWA_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !kept) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_FWD, p, fwd_plan, false);
  if (st != COWA_OK) return st;
  st = check_plan(COWA_OP_MALA_BWD, p, plan, true);
  if (st != COWA_OK) return st;
  size_t need = 0;
  cowa_workspace_size(COWA_OP_MALA_BWD, p, &need);
  if (!workspace || workspace_bytes < need) return COWA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return COWA_ERR_INVALID_ARG;
  BwdArgs a = bwd_args(p, plan, q, k, v, o, o_lo, lse, dout, dq, dk, dv, workspace);
  const MalaTiles mt = mala_tiles(p);
  MalaMaskArgs m{};
  m.mask = (uint8_t*)workspace + bwd_layout(p).total;
  m.row_ptr = fwd_plan->row_ptr;
  m.row_ent = fwd_plan->row_ent;
  m.kept = kept;
  m.n_items = p->Hkv * mt.nqb;
  m.nkb = mt.nkb;
  hipStream_t s = (hipStream_t)stream;
  st = hip_status(launch_mala_mask(m, s));
  if (st != COWA_OK) return st;
  a.mala_mask = m.mask;
  a.mala_bq = mt.bq;
  a.mala_nqb = mt.nqb;
  a.mala_nkb = mt.nkb;
  return hip_status(launch_bwd_bf16_d128(a, COWA_BWD_ALL, s));
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

// ---------------------------------------------------------------------- window-only cache
extern "C" int cowa_wcache_layout(const cowa_window* win, int32_t Hkv, int32_t Lmax, int64_t* head_offset,
                                  int64_t* slots) {
  if (!win || !slots || Hkv < 1 || Lmax < 1 || !window_valid(*win)) return COWA_ERR_INVALID_ARG;
  if (Lmax > (1 << 30)) return COWA_ERR_UNSUPPORTED;
  if (head_offset)
    for (int h = 0; h <= Hkv; ++h) head_offset[h] = wcache_offset(*win, h, Lmax);
  *slots = wcache_offset(*win, Hkv, Lmax);
  return COWA_OK;
}

namespace {
int check_wcache(const cowa_wcache* c) {
  if (!c || !c->k || !c->v) return COWA_ERR_INVALID_ARG;
  if (c->B < 1 || c->Hkv < 1 || c->Lmax < 1 || !window_valid(c->win)) return COWA_ERR_INVALID_ARG;
  if (c->D != 128 || c->B > 65535 || c->Lmax > (1 << 30)) return COWA_ERR_UNSUPPORTED;
  return COWA_OK;
}
}  // namespace

extern "C" int cowa_wcache_append(const cowa_wcache* c, const void* k_new, const void* v_new, int32_t T,
                                  const int32_t* pos0, void* stream) {
  int st = check_wcache(c);
  if (st != COWA_OK) return st;
  if (!k_new || !v_new || !pos0 || T < 0) return COWA_ERR_INVALID_ARG;
  WcacheAppendArgs a{};
  a.k = c->k;
  a.v = c->v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos0 = pos0;
  a.B = c->B;
  a.T = T;
  a.Hkv = c->Hkv;
  a.Lmax = c->Lmax;
  a.wslots = wcache_offset(c->win, c->Hkv, c->Lmax);
  a.cwin = c->win;
  return hip_status(launch_wcache_append(a, (hipStream_t)stream));
}

extern "C" int cowa_wcache_decode(const cowa_problem* p, const cowa_wcache* c, const void* q,
                                  const int32_t* seqlens, void* o, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_DECODE, p);
  if (st != COWA_OK) return st;
  st = check_wcache(c);
  if (st != COWA_OK) return st;
  if (c->B != p->B || c->Hkv != p->Hkv || c->D != p->D || c->Lmax != p->Lk || !same_window(c->win, p->win))
    return COWA_ERR_INVALID_ARG;
  if (!q || !seqlens || !o) return COWA_ERR_INVALID_ARG;
  // the kernel addresses one head's slots with 32-bit byte offsets
  for (int h = 0; h < c->Hkv; ++h) {
    const WinRing r = wcache_ring(c->win, h, c->Lmax);
    if ((r.sink_slots + r.ring) * c->D * 2 > 0x7fffffff) return COWA_ERR_UNSUPPORTED;
  }
  size_t need = 0;
  cowa_workspace_size(COWA_OP_DECODE, p, &need);
  if (!workspace || workspace_bytes < need) return COWA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return COWA_ERR_INVALID_ARG;

  DecodeArgs a{};
  a.q = q;
  a.k = c->k;
  a.v = c->v;
  a.o = o;
  a.lse = lse;
  a.nsplit = decode_splits(p);
  const size_t rows = (size_t)p->B * p->Hq * a.nsplit;
  a.part = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + (rows * p->D * sizeof(float) + 255) / 256 * 256);
  a.seqlens = seqlens;
  a.B = p->B;
  a.Lk = p->Lk;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.Bk = kDecBk;
  a.scale_log2 = p->scale * 1.44269504088896340736f;
  a.win = dev_window(p->win);
  a.window_mode = 1;
  a.wslots = wcache_offset(c->win, c->Hkv, c->Lmax);
  a.cwin = c->win;
  return hip_status(launch_decode_bf16_d128(a, (hipStream_t)stream));
}

// ---------------------------------------------------------------------- no-allocation decode
// The decode's split partials in a file-scope device array instead of a caller workspace.
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// comes from hipGetSymbolAddress, once per device with that device current, and only that
// address is ever handed to a kernel.
namespace {

constexpr size_t kScratchBytes = COWA_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first call made on
// the device), or null with *err set.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int cowa_decode_noalloc(const cowa_problem* p, const cowa_plan_dev* plan, const void* q,
                                   const void* k_cache, const void* v_cache, void* o, float* lse,
                                   void* stream) {
  int st = check_problem(p);
  if (st != COWA_OK) return st;
  st = check_op_support(COWA_OP_DECODE, p);
  if (st != COWA_OK) return st;
  if (!q || !k_cache || !v_cache || !o) return COWA_ERR_INVALID_ARG;
  st = check_plan(COWA_OP_DECODE, p, plan, false);
  if (st != COWA_OK) return st;
  size_t need = 0;
  cowa_workspace_size(COWA_OP_DECODE, p, &need);
  if (need > kScratchBytes) return COWA_ERR_WORKSPACE_TOO_SMALL;
  hipError_t err;
  void* ws = scratch_on_current_device(&err);
  if (!ws) return COWA_ERR_HIP;
  return cowa_decode(p, plan, q, k_cache, v_cache, o, lse, ws, kScratchBytes, stream);
}
