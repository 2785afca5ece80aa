/*
 * cowa.h — C ABI of libcowa: CoWindow Attention (CoWA) on AMD Instinct MI355X (gfx950).
 *
 * What the operator computes.  CoWA is causal grouped-query attention in which every
 * KV head sees a shared prefix-sink window, a shared near-diagonal window and a
 * long-range band of its own; the bands of the KV heads are complementary, so their
 * union covers the whole causal history ("CoWindow Attention: Full Causal Coverage Is
 * a Collective Property", abstract; page crimsonlingua.com, second paragraph).  The
 * window is described by the quadruple (sink width, near width, gap, long-range
 * width) on bottom-right-aligned causal distance, one definition for training,
 * prefill and decoding (slinene.github.io ai-papers-daily page, method key point 2).
 * Execution skips the invisible KV blocks by walking lists of visible blocks
 * (same page, method key point 3).
 *
 * Window convention (the readings this library fixes; the pages give no formula):
 *   query row i in [0, Lq), key j in [0, Lk), bottom-right distance
 *       d(i, j) = i + (Lk - Lq) - j                       causal iff d >= 0
 *   KV head h (global index) owns the band [lo_h, hi_h) of distances with
 *       lo_h = near_w + gap + s_h * lr,  hi_h = lo_h + lr
 *       s_h  = h (COWA_BAND_COMPLEMENTARY), 0 (COWA_BAND_DUPLICATED)
 *       COWA_BAND_DENSE: lo_h = near_w + gap, hi_h = +infinity
 *   key j is visible to query row i under KV head h iff
 *       d >= 0  and  ( j < sink  or  d < near_w  or  lo_h <= d < hi_h )
 *   The complementary width is lr = ceil((Lmax - near_w - gap) / Hkv), so that the
 *   Hkv bands tile the distances [near_w + gap, Lmax) (cowa_window_make).
 *   Query head q reads KV head q / (Hq / Hkv) (contiguous GQA groups).
 *
 * Tensor layout (all row-major, contiguous, "BSHD"):
 *   Q, O, dO, dQ : [B, Lq, Hq, D]      K, V, dK, dV : [B, Lk, Hkv, D]
 *   LSE, Delta   : [B, Hq, Lq] fp32, natural-log logsumexp of scale * q.k over the
 *                  visible keys.
 *
 * Ownership: the caller owns every host and device buffer; the library allocates no
 * device memory and keeps no state between calls.  Device work is enqueued on the
 * hipStream_t passed as `void* stream` (NULL = the null stream) and is asynchronous:
 * a fault during a kernel surfaces at the caller's next synchronisation.  Functions
 * never throw; they return a cowa_status.  Arguments are validated before anything is
 * launched, so an error status means no device work was enqueued.
 */
#ifndef COWA_H_
#define COWA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
typedef enum cowa_status {
  COWA_OK = 0,
  COWA_ERR_INVALID_ARG = -1,        /* a NULL pointer, a negative size, ... */
  COWA_ERR_UNSUPPORTED = -2,        /* a (dtype, D, Hq/Hkv) the kernels do not cover */
  COWA_ERR_WORKSPACE_TOO_SMALL = -3,
  COWA_ERR_PLAN_MISMATCH = -4,      /* plan built for another shape, window or tiling */
  COWA_ERR_HIP = -5                 /* a HIP runtime call failed (launch error) */
} cowa_status;

/* Human-readable text of a status code (static storage; never NULL). */
const char* cowa_status_string(int status);

/* ---------------------------------------------------------------- window */
enum { COWA_BAND_COMPLEMENTARY = 0, COWA_BAND_DUPLICATED = 1, COWA_BAND_DENSE = 2 };

/* The window quadruple (sink width, near width, gap, long-range width) plus the band
 * assignment mode.  All widths are in tokens and must be >= 0. */
typedef struct cowa_window {
  int32_t sink;      /* keys j < sink are visible (subject to causality)          */
  int32_t near_w;    /* distances 0 <= d < near_w are visible                       */
  int32_t gap;       /* distances [near_w, near_w + gap) belong to no band          */
  int32_t lr;        /* long-range band width                                        */
  int32_t band_mode; /* COWA_BAND_*                                                  */
} cowa_window;

/* Fill *out with the window whose Hkv bands split the distances
 * [near_w + gap, Lmax) into Hkv equal widths lr = ceil((Lmax - near_w - gap) / Hkv)
 * (clamped at 0).  band_mode is stored as given.  Errors: INVALID_ARG on a NULL out,
 * Hkv < 1, or a negative width or length. */
int cowa_window_make(int32_t Lmax, int32_t Hkv, int32_t sink, int32_t near_w, int32_t gap,
                     int32_t band_mode, cowa_window* out);

/* ---------------------------------------------------------------- planner */
/* Shape and counts of a block-visibility plan. */
typedef struct cowa_plan_info {
  int32_t Lq, Lk, Hkv, Bq, Bk;  /* what the plan was built for                     */
  int32_t nqb, nkb;             /* ceil(Lq / Bq), ceil(Lk / Bk)                     */
  int64_t nnz;                  /* visible (q-block, k-block, KV head) tiles        */
  int64_t n_partial;            /* of which PARTIAL (not every element visible)     */
  int64_t visited;              /* tiles the enumerator touched; equals nnz          */
  int64_t edges;                /* visible (query row, key, KV head) triples         */
} cowa_plan_info;

/* Tile entry encoding used by every list: (block_index << 1) | partial_flag. */
#define COWA_ENT_BLOCK(e) ((int32_t)(e) >> 1)
#define COWA_ENT_PARTIAL(e) ((int32_t)(e) & 1)

/* Block-visibility planner (slinene.github.io ai-papers-daily page, method key point 3:
 * the traversal visits only visible KV blocks).  For every KV head h and q-block qb it
 * lists the k-blocks holding at least one visible (row, key) pair, ascending, each
 * flagged PARTIAL unless every one of its Bq x Bk elements lies inside [0,Lq) x [0,Lk)
 * and is visible (a FULL tile needs no masking at all).  It works from the
 * at most three key intervals (sink, band, near) of each query row, so masked tiles are
 * never touched: `visited` counts the tiles it emitted.
 *
 * Outputs (host memory, caller-allocated; pass all NULL to get only *info):
 *   row_ptr   [Hkv * nqb + 1]  CSR offsets, item id = h * nqb + qb
 *   row_ent   [nnz]            k-block entries per row item, ascending k-block
 *   col_ptr   [Hkv * nkb + 1]  CSR offsets, item id = h * nkb + kb
 *   col_ent   [nnz]            q-block entries per column item, ascending q-block
 *   row_order [Hkv * nqb]      row item ids in launch order (a permutation)
 *   col_order [Hkv * nkb]      column item ids in launch order (a permutation)
 * The launch orders are built for MI355X's 8 XCDs, whose L2 caches are separate and to
 * which work groups are dealt round-robin.  Items whose list is longer than twice the
 * mean (the columns that hold the prefix sink) come first, longest first, so none starts
 * late; after them, the items dealt to one XCD are contiguous blocks of one KV head at a
 * time, so concurrently running items share K/V (or Q/dO) tiles.
 * The arrays must be either all NULL or all non-NULL.  Every list (within an item) is
 * sorted ascending; entries use COWA_ENT_BLOCK / COWA_ENT_PARTIAL.
 * Errors: INVALID_ARG for NULL info/window, a non-positive size or a negative width;
 * UNSUPPORTED when nnz would exceed INT32_MAX. */
int cowa_plan_blocks(int32_t Lq, int32_t Lk, int32_t Hkv, int32_t Bq, int32_t Bk,
                     const cowa_window* win, cowa_plan_info* info,
                     int32_t* row_ptr, int32_t* row_ent, int32_t* col_ptr, int32_t* col_ent,
                     int32_t* row_order, int32_t* col_order);

/* A plan resident in device memory (the caller copies the host arrays of
 * cowa_plan_blocks into device buffers and fills this struct).  info and win must be
 * the values the plan was built with; they are checked against the problem. */
typedef struct cowa_plan_dev {
  cowa_plan_info info;
  cowa_window win;
  const int32_t* row_ptr;
  const int32_t* row_ent;
  const int32_t* col_ptr;
  const int32_t* col_ent;
  const int32_t* row_order;
  const int32_t* col_order;
} cowa_plan_dev;

/* ---------------------------------------------------------------- problem */
enum { COWA_DTYPE_BF16 = 0, COWA_DTYPE_F32 = 1 };
enum { COWA_OP_FWD = 0, COWA_OP_BWD = 1, COWA_OP_DECODE = 2 };

typedef struct cowa_problem {
  int32_t B, Lq, Lk, Hq, Hkv, D;
  int32_t dtype;      /* COWA_DTYPE_*                                               */
  float scale;        /* softmax scale applied to q.k (the usual 1/sqrt(D))         */
  cowa_window win;
} cowa_problem;

/* Tile sizes (Bq, Bk) the kernels of `op` use for this problem; plans passed to that
 * op must be built with them.  Errors: INVALID_ARG, UNSUPPORTED. */
int cowa_tile_sizes(int op, const cowa_problem* p, int32_t* Bq, int32_t* Bk);

/* Bytes of device workspace `op` needs for problem p (0 if none).  The backward keeps
 * Delta and a power-of-two scale per (query head, row) in fp32 and an fp16 copy of Q
 * (B * Lq * Hq * D * 2 bytes); the decode keeps its split partials. */
int cowa_workspace_size(int op, const cowa_problem* p, size_t* bytes);

/* Forward (the operator of the abstract; training forward and prefill).  For every
 * query head and row: O = softmax(scale * q K^T restricted to visible keys) V, and
 * LSE = log of the softmax denominator (natural log, including the scale).
 * Supported: dtype BF16 with D = 128 (bf16 in/out, fp32 accumulation) and dtype F32
 * with D = 64; Hq % Hkv == 0.  q,k,v,o are device pointers of `dtype`; lse is fp32.
 * A row with no visible key (only possible with near_w = 0) gets O = 0, LSE = -inf.
 * Errors: INVALID_ARG, UNSUPPORTED, PLAN_MISMATCH (plan tiling must be
 * cowa_tile_sizes(COWA_OP_FWD)), HIP. */
int cowa_fwd(const cowa_problem* p, const cowa_plan_dev* plan,
             const void* q, const void* k, const void* v, void* o, float* lse,
             void* workspace, size_t workspace_bytes, void* stream);

/* Backward from the saved LSE (training backward; same pattern as the forward):
 *   Delta_i = dO_i . O_i,  P = exp(scale q.k - LSE),  dS = P (dO.v - Delta)
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO   (dK, dV summed over the
 *   query heads of each KV head).
 * `stages` selects the kernels to run (COWA_BWD_ALL for the whole backward): DELTA
 * writes Delta, the row scales of Q and the fp16 copy of Q into the workspace; DQ and
 * DKDV read them from there, so a caller that runs them separately (for example on two
 * streams) must run DELTA first on the same workspace.  dK is formed from dS and Q in
 * fp16: each row of Q is divided by a power of two that puts its max |q| in [1, 2),
 * which copies every entry of at least 2^-14 times the row's max exactly, and dS is
 * scaled by the same power; the result stays finite while |dS| times the row's max |q|
 * stays below 2^15.  dQ is written by DQ, dK and dV by DKDV; no output is accumulated
 * into.
 * Supported: dtype BF16, D = 128.  All tensors bf16 except lse (fp32).  The plan must
 * hold both row and column lists at cowa_tile_sizes(COWA_OP_BWD).  workspace must be
 * at least cowa_workspace_size(COWA_OP_BWD) bytes, 256-byte aligned.
 * Errors: INVALID_ARG (also for stages outside 1..7), UNSUPPORTED,
 * WORKSPACE_TOO_SMALL, PLAN_MISMATCH, HIP. */
enum { COWA_BWD_DELTA = 1, COWA_BWD_DQ = 2, COWA_BWD_DKDV = 4, COWA_BWD_ALL = 7 };
int cowa_bwd(const cowa_problem* p, const cowa_plan_dev* plan,
             const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int stages,
             void* workspace, size_t workspace_bytes, void* stream);

/* Decode: one new query token per sequence (p->Lq == 1) over a KV cache of p->Lk
 * positions that already holds the new token's K/V; the query sits at position Lk-1,
 * so the bottom-right distance is d = Lk - 1 - j, the same definition as the forward.
 * Each KV head reads only its visible blocks.  q/o: [B, 1, Hq, D] bf16;
 * k_cache/v_cache: [B, Lk, Hkv, D] bf16; lse: [B, Hq] fp32 or NULL.
 * Supported: dtype BF16, D = 128.  workspace: cowa_workspace_size(COWA_OP_DECODE).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, PLAN_MISMATCH, HIP. */
int cowa_decode(const cowa_problem* p, const cowa_plan_dev* plan,
                const void* q, const void* k_cache, const void* v_cache,
                void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Decode over caches of different lengths: a batch of sequences at different positions,
 * each under the same bottom-right distance as the forward (slinene.github.io
 * ai-papers-daily page, method key point 2).
 * k_cache/v_cache hold p->Lk positions per sequence (the capacity); sequence b uses the
 * first seqlens_k[b] of them, including its new token's K/V, and its query sits at
 * position seqlens_k[b] - 1, so d = seqlens_k[b] - 1 - j.  The window is p->win for every
 * sequence.  No plan: each work group derives its sequence's visible 64-key blocks (prefix
 * sink, near window, the head's band) from the length and checks every key.
 * seqlens_k: device int32 [B], read by the kernel; values are clamped to [0, Lk], and a
 * sequence of length 0 gets O = 0, LSE = -inf.  q/o/lse as in cowa_decode; workspace:
 * cowa_workspace_size(COWA_OP_DECODE).  With every length equal to Lk the result is
 * cowa_decode's.  Errors: INVALID_ARG (also for NULL seqlens_k), UNSUPPORTED,
 * WORKSPACE_TOO_SMALL, HIP. */
int cowa_decode_varlen(const cowa_problem* p, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* seqlens_k, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* COWA_H_ */
