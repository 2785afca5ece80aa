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
enum { COWA_OP_FWD = 0, COWA_OP_BWD = 1, COWA_OP_DECODE = 2, COWA_OP_MALA_BWD = 3, COWA_OP_MALA_FWD = 4 };

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
 * three fp32 values per (query head, row) (Delta, the power-of-two scales of Q and dO),
 * 256 bytes of launch-wide maxima (with the dQ and dK/dV launches' per-XCD work queue
 * heads for one sequence), fp16 copies of Q and dO (2 * B * Lq * Hq * D * 2 bytes) and
 * of K (B * Lk * Hkv * D * 2 bytes); the decode keeps its split partials; the bf16
 * forward takes 256 bytes for its optional work queue heads.
 * COWA_OP_MALA_FWD needs 1 KB per visible forward tile and sequence plus the kept lists
 * (cowa_mala_fwd); COWA_OP_MALA_BWD adds one byte per forward tile (Hkv * ceil(Lq / Bq_f) * ceil(Lk / 64),
 * Bq_f the forward's tile height, rounded up to 256) to the backward's workspace. */
int cowa_workspace_size(int op, const cowa_problem* p, size_t* bytes);

/* Forward (the operator of the abstract, used for training and for prefill: "CoWindow
 * Attention" abstract; beyondmarketintelligence.com post, second paragraph).  For every
 * query head and row: O = softmax(scale * q K^T restricted to visible keys) V, and
 * LSE = log of the softmax denominator (natural log, including the scale).
 * Supported: dtype BF16 with D = 128 (bf16 in/out, fp32 accumulation) and dtype F32
 * with D = 64; Hq % Hkv == 0.  q,k,v,o are device pointers of `dtype`; lse is fp32.
 * o_lo (bf16 only, may be NULL): receives O - bf16(O) rounded to bf16, the part of the
 * fp32 result that the bf16 O drops, in O's layout.  A training caller keeps it with O
 * and LSE and passes it to cowa_bwd, which then forms Delta = dO . O from O to about 16
 * significant bits instead of 8.
 * A row with no visible key (only possible with near_w = 0, or with Lq > Lk for the
 * first Lq - Lk rows) gets O = 0, LSE = -inf.
 * workspace (optional, bf16): with at least cowa_workspace_size(COWA_OP_FWD) bytes (256),
 * 256-byte aligned, and B = 1, it holds the launch's per-XCD work queue heads: each work
 * group takes the next item of its XCD's part of the launch order, or of another XCD's
 * part once its own is done, so XCDs that run slower take fewer items; NULL (or a smaller
 * or unaligned one) keeps the fixed order.  The results are the same either way; calls
 * that share a workspace must not overlap.
 * Errors: INVALID_ARG (also for o_lo with dtype F32), UNSUPPORTED, PLAN_MISMATCH (plan
 * tiling must be cowa_tile_sizes(COWA_OP_FWD)), HIP. */
int cowa_fwd(const cowa_problem* p, const cowa_plan_dev* plan,
             const void* q, const void* k, const void* v, void* o, float* lse, void* o_lo,
             void* workspace, size_t workspace_bytes, void* stream);

/* MALA forward (MassAlloc Attention, the companion operator the pages describe beside
 * CoWA: beyondmarketintelligence.com post, second paragraph and takeaway; crimsonlingua.com
 * news item, fifth paragraph): the QK scoring stays full, and the softmax's own
 * statistics decide whether the rest of a tile's work is done.  Readings fixed here: a
 * tile is (KV head, q-block of the forward's tiling, k-block); it is kept when some row
 * of the tile puts at least `tau` of its probability mass P = exp(scale q.k - LSE) there;
 * O = sum over kept tiles of P V, the denominator staying the full one.  A scoring pass
 * scores every visible key, writes the exact LSE and keeps each tile's row sums; the
 * decisions follow from them and the LSE; a last pass runs the kept tiles only
 * (scores and PV products).  tau = 0 keeps every tile (exact attention); a
 * row loses at most its dropped mass times max |v| per dimension.  The window is the
 * visibility the scoring covers (COWA_BAND_DENSE: full causal scoring, as the pages
 * describe MALA; the CoWA windows give MALA on top of CoWA).
 * q,k,v,o bf16 as in cowa_fwd, D = 128; lse fp32 [B, Hq, Lq] (written: the full LSE);
 * o_lo (may be NULL): O's bf16 rounding residual, as in cowa_fwd, for cowa_mala_bwd.
 * kept (may be NULL; B = 1 only): int32 per entry of the plan's row lists, set to 1 where
 * the tile's PV was done and 0 where it was skipped.  The plan is a forward plan
 * (cowa_tile_sizes(COWA_OP_FWD)).  workspace: cowa_workspace_size(COWA_OP_MALA_FWD) bytes
 * (per sequence, 1 KB per visible forward tile for the row sums and 4 bytes per tile and
 * per item for the kept lists), 256-byte aligned.  Errors: INVALID_ARG (also for tau < 0
 * or NaN, and kept with B > 1), UNSUPPORTED (not BF16 / D = 128), WORKSPACE_TOO_SMALL,
 * PLAN_MISMATCH, HIP. */
int cowa_mala_fwd(const cowa_problem* p, const cowa_plan_dev* plan, float tau,
                  const void* q, const void* k, const void* v, void* o, float* lse,
                  void* o_lo, int32_t* kept, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Backward from the saved LSE: the pattern serves training forward and backward alike
 * (beyondmarketintelligence.com post, second paragraph; "CoWindow Attention" abstract),
 * with the gradients of the same masked softmax attention:
 *   Delta_i = dO_i . O_i,  P = exp(scale q.k - LSE),  dS = P (dO.v - Delta)
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO   (dK, dV summed over the
 *   query heads of each KV head).
 * o_lo: the residual cowa_fwd wrote (may be NULL: Delta then uses the bf16 O alone).
 * `stages` selects the kernels to run (COWA_BWD_ALL for the whole backward): DELTA
 * writes Delta, the scales and fp16 copies of Q, dO and K and the launch-wide maxima into
 * the workspace; DQ and DKDV read them from there, so a caller that runs them separately
 * (for example on two streams) must run DELTA first on the same workspace.
 * Precision: every product runs on MFMA with fp32 accumulation.  S, dP, dV and dK take
 * fp16 operands: Q and dO rows and K (per launch in the dQ kernel, per 128-key block in
 * the dK/dV kernel) and V (per 128-key block) are divided by powers of two that put their
 * largest magnitude in [1, 2), which copies every bf16 value of at least 2^-14 of that
 * largest magnitude exactly; P enters dV and dQ's dS and dK's dS enter their products
 * rounded once to fp16 (11 significant bits), each scaled by a power of two chosen from
 * launch-wide bounds (|dO_i| |v_j| + |Delta_i| for dS) so that it stays below 2^14.  The
 * scales are undone exactly at the end.  A row whose dO is much smaller than the largest
 * dO row of the launch (by more than about 2^10) contributes its smallest probabilities
 * to dV at reduced (subnormal fp16) precision.  Inputs whose magnitudes lie within
 * 2^-60 .. 2^60 keep every scale inside the fp32 range.
 * dQ is written by DQ, dK and dV by DKDV; no output is accumulated into.
 * Supported: dtype BF16, D = 128.  All tensors bf16 except lse (fp32).  The plan must
 * hold both row and column lists at cowa_tile_sizes(COWA_OP_BWD).  workspace must be
 * at least cowa_workspace_size(COWA_OP_BWD) bytes, 256-byte aligned.
 * Errors: INVALID_ARG (also for stages outside 1..7), UNSUPPORTED,
 * WORKSPACE_TOO_SMALL, PLAN_MISMATCH, HIP. */
enum { COWA_BWD_DELTA = 1, COWA_BWD_DQ = 2, COWA_BWD_DKDV = 4, COWA_BWD_ALL = 7 };
int cowa_bwd(const cowa_problem* p, const cowa_plan_dev* plan,
             const void* q, const void* k, const void* v, const void* o, const void* o_lo,
             const float* lse, const void* dout, void* dq, void* dk, void* dv, int stages,
             void* workspace, size_t workspace_bytes, void* stream);

/* MALA backward: the gradients of cowa_mala_fwd's output with its tile decisions held
 * fixed (the decision is a threshold test, piecewise constant in the inputs; the pages
 * describe MALA as a drop-in operator for training and inference alike:
 * beyondmarketintelligence.com post, second paragraph).  With P = exp(scale q.k - LSE)
 * over every visible key (the full scoring) and m = 1 on kept tiles, 0 on skipped ones:
 *   Delta_i = dO_i . O_i,  dP = m (dO.v),  dS = P (dP - Delta)
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = (m P)^T dO,
 * so skipped tiles give dV nothing and pass dS = -P Delta to dQ and dK through the
 * denominator.  tau = 0 (every tile kept) is exactly cowa_bwd.
 * kept: the int32 flags cowa_mala_fwd wrote for fwd_plan's row lists (device); o, o_lo
 * and lse: its outputs (o_lo may be NULL: Delta then uses the bf16 O alone).  fwd_plan: the forward plan the forward ran with
 * (cowa_tile_sizes(COWA_OP_FWD)); plan: a backward plan with row and column lists
 * (cowa_tile_sizes(COWA_OP_MALA_BWD), the same as COWA_OP_BWD).  Precision and ranges as
 * cowa_bwd.  Runs all three stages.  workspace: cowa_workspace_size(COWA_OP_MALA_BWD),
 * 256-byte aligned.
 * Supported: dtype BF16, D = 128, B = 1.  Errors: INVALID_ARG (also for kept NULL),
 * UNSUPPORTED, WORKSPACE_TOO_SMALL, PLAN_MISMATCH (either plan), HIP. */
int cowa_mala_bwd(const cowa_problem* p, const cowa_plan_dev* fwd_plan, const cowa_plan_dev* plan,
                  const int32_t* kept, const void* q, const void* k, const void* v,
                  const void* o, const void* o_lo, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Decode: one new query token per sequence (p->Lq == 1) over a KV cache of p->Lk
 * positions that already holds the new token's K/V; the query sits at position Lk-1,
 * so the bottom-right distance is d = Lk - 1 - j, the same definition as the forward
 * (one distance for training, prefill and decoding: slinene.github.io ai-papers-daily
 * page, method key point 2; each KV head reads only its window's blocks: same page,
 * method key point 3).
 * Each KV head reads only its visible blocks.  q/o: [B, 1, Hq, D] bf16;
 * k_cache/v_cache: [B, Lk, Hkv, D] bf16; lse: [B, Hq] fp32 or NULL.
 * Supported: dtype BF16, D = 128, Hq / Hkv from 1 to 8.  workspace:
 * cowa_workspace_size(COWA_OP_DECODE).
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

/* ---------------------------------------------------------------- window-only cache
 * Each rank needs only the KV cache of its own window (slinene.github.io ai-papers-daily
 * page, practical note 3).  Under the bottom-right distance a decode query at position p
 * sees, under KV head h, the prefix sink and the keys at distance p - j in the near window
 * or in the head's band; distances only grow as tokens are appended, so a key (past the
 * sink) that is R_h = max(near_w, hi_h) or more positions behind the newest token is never
 * seen by head h again, while a nearer one is seen now or once the band reaches it (for
 * h > 0 that includes the keys between the near window and the band).  The cache of head
 * h therefore holds the sink and a ring of the last R_h positions:
 *   slot(j) = j                 for j < min(sink, Lmax)
 *           = sink + (j mod R_h) otherwise
 * (R_h = Lmax and no separate sink when sink + R_h >= Lmax: the whole history).  hi_h is
 * the band's upper distance (Lmax in dense mode).  Heads follow one another in the slot
 * dimension; per sequence the caches take cowa_wcache_layout's `slots` rows of D values.
 * At 131072 positions (sink 128, near 4096, 8 bands of 15872) head 0 holds 20096 rows
 * and head 7 all 131072: 605056 rows for the 8 heads against 1048576 for full caches. */
typedef struct cowa_wcache {
  int32_t B, Hkv, D;  /* sequences, KV heads, head dim (128)                          */
  int32_t Lmax;       /* positions the cache serves (the window's Lmax)               */
  cowa_window win;
  void* k;            /* device [B, slots, D] bf16                                     */
  void* v;            /* device [B, slots, D] bf16                                     */
} cowa_wcache;

/* Slots per sequence (*slots) and, if head_offset is not NULL, the first slot of each
 * head (head_offset[h], h = 0..Hkv; head_offset[Hkv] = *slots).
 * Errors: INVALID_ARG (NULL win/slots, Hkv < 1, Lmax < 1, bad window), UNSUPPORTED
 * (Lmax > 2^30). */
int cowa_wcache_layout(const cowa_window* win, int32_t Hkv, int32_t Lmax, int64_t* head_offset,
                       int64_t* slots);

/* Append T tokens per sequence: k_new/v_new [B, T, Hkv, D] bf16 hold the K/V rows of
 * positions pos0[b] .. pos0[b] + T - 1 of sequence b (pos0: device int32 [B]).  Each head
 * stores the positions it can still see; of the positions of one chunk that share a ring
 * slot only the last is written, so T may exceed the ring (a whole prefill in one call).
 * Positions must be appended in order, each once; positions outside [0, Lmax) are
 * ignored.  Errors: INVALID_ARG, UNSUPPORTED (D != 128), HIP. */
int cowa_wcache_append(const cowa_wcache* c, const void* k_new, const void* v_new, int32_t T,
                       const int32_t* pos0, void* stream);

/* Decode over window-only caches: as cowa_decode_varlen (sequence b has length
 * seqlens[b], its query at position seqlens[b] - 1, clamped to [0, Lmax]) with each key
 * read from its head's slot; the same blocks in the same order, so the result equals
 * cowa_decode_varlen's over full caches holding the same rows, bit for bit.  p->Lk must
 * be c->Lmax, and p's B, Hkv, D and window those of c.  workspace:
 * cowa_workspace_size(COWA_OP_DECODE, p).  Errors: INVALID_ARG, UNSUPPORTED (also when a
 * head holds more than (2^31 - 1) / (2 D) slots: 8388607 at D = 128, the kernel's 32-bit
 * offsets), WORKSPACE_TOO_SMALL, HIP. */
int cowa_wcache_decode(const cowa_problem* p, const cowa_wcache* c, const void* q,
                       const int32_t* seqlens, void* o, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Decode without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, checks and results as cowa_decode (bit-identical outputs), but the split
 * partials live in a library-owned device array of COWA_DECODE_SCRATCH_BYTES bytes per
 * GPU, which each GPU the library runs on holds until the process ends; its address is
 * looked up (hipGetSymbolAddress) on the first call made on a device, with that device
 * current, which must be the device of `stream`.  Nothing is allocated and nothing needs
 * to start at zero: every partial is written before it is read.  All calls on one GPU
 * share its array, so calls that overlap in time on one GPU (different streams, or
 * different host threads) race; calls on one stream are ordered and safe.
 * Errors: as cowa_decode, and WORKSPACE_TOO_SMALL (before any device work) when
 * cowa_workspace_size(COWA_OP_DECODE, p) exceeds COWA_DECODE_SCRATCH_BYTES (it is about
 * B * Hq * 32 * 520 bytes at 131072 cache positions: B * Hq up to about 1000); HIP when
 * the address lookup fails. */
#define COWA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int cowa_decode_noalloc(const cowa_problem* p, const cowa_plan_dev* plan,
                        const void* q, const void* k_cache, const void* v_cache,
                        void* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* COWA_H_ */
