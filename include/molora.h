/*
 * molora.h — C ABI of the MI355X (gfx950) per-token adapter-routing library.
 *
 * The method (MoLoRA pages, "MoLoRA: Composable Specialization via Per-Token
 * Adapter Routing"; the technical figures and tables are on the
 * thelatestinai.com page): every token is routed to one adapter by its
 * vocabulary range, or to k adapters by a learned top-k gate (Table 1,
 * "Routing decision"); the routed (token, adapter) pairs are counted per
 * adapter, turned into offsets ("pointer arrays") and grouped by adapter
 * (Table 1 rows "Histogram computation", "Pointer arrays"; Figure 2 right);
 * grouped LoRA shrink x·A_e (d_in -> r) and expand h·B_e (r -> d_out) run
 * over adapters held at fixed GPU addresses (Figure 4, hot set; Table 10 for
 * the shapes A (K, d, r) and B (K, r, d)); the gate-weighted deltas, scaled by
 * the LoRA factor alpha/r, are added into the base output y (Figure 2 left:
 * weighted sum).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to memory of the current
 *    HIP device, 16-byte aligned.  "host" pointers are read during the call.
 *  - The caller owns every buffer.  The library owns only the host-side
 *    molora_hotset descriptor.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Except
 *    for molora_hotset_init / molora_hotset_destroy, every call only
 *    enqueues work on `stream`: it never synchronises the host and never
 *    reads device memory from the host, so the calls can be captured into a
 *    HIP graph.
 *  - Return value: MOLORA_OK, or an error code.  Argument errors are detected
 *    on the host before anything is enqueued; molora_last_error() then holds
 *    a message (thread-local).  MOLORA_EHIP reports a HIP runtime error.
 *  - N = 0 (no tokens) is a successful no-op.
 *  - Data-dependent conditions are not errors: a token id outside every
 *    vocabulary range, or an adapter index outside [0, K), marks the pair
 *    "unrouted"; such pairs are left out of counts/offsets/perm and add no
 *    delta.
 *  - bf16 means the 16-bit bfloat16 format (upper half of an IEEE fp32).
 */
#ifndef MOLORA_H
#define MOLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOLORA_OK = 0,
  MOLORA_EINVAL = 1,  /* null/misaligned pointer, bad shape or count */
  MOLORA_ENOTSUP = 2, /* shape outside the supported set (see each call) */
  MOLORA_ENOSPC = 3,  /* slab or workspace smaller than required */
  MOLORA_EHIP = 4     /* HIP runtime or launch error */
};

enum { MOLORA_LAYOUT_DIRECT = 0, MOLORA_LAYOUT_INDIRECT = 1 };
enum { MOLORA_PATH_AUTO = 0, MOLORA_PATH_GROUPED = 1, MOLORA_PATH_SKINNY = 2, MOLORA_PATH_TILE = 3,
       MOLORA_PATH_BLOCK = 4, MOLORA_PATH_GROUPED_FIXED = 5 };
enum { MOLORA_BF16 = 0, MOLORA_F32 = 1 };

/* Limits of this build. */
#define MOLORA_MAX_ADAPTERS 64 /* K (hot-set capacity per target) */
#define MOLORA_MAX_RANK 64     /* r */
#define MOLORA_MAX_TOPK 8      /* k */
#define MOLORA_ROUTER_HIDDEN 64 /* H of the router MLP d -> H -> K */

/* Message for the last non-OK return on this thread ("" if none). */
const char *molora_last_error(void);

/* ------------------------------------------------------------------------
 * Hot set (thelatestinai.com, Figure 4: adapters pre-allocated on the GPU at
 * fixed addresses so that the step can be captured in a graph; Table 2:
 * direct versus indirect memory layout).
 *
 * One hot set holds K adapters of rank r for each of n_targets projections
 * (e.g. the 7 LoRA targets of one transformer layer).  Target t has input
 * width d_in and output width d_out; its user-facing weights are
 *   A: bf16 [K][d_in][r]   row-major (Table 10: A has shape (K, d, r))
 *   B: bf16 [K][r][d_out]  row-major (Table 10: B has shape (K, r, d))
 * molora_hotset_init copies them into the caller's slab in the library's
 * internal layout (transposed, rank padded to a multiple of 16) and records
 * their addresses in the descriptor.  The slab must stay allocated and must
 * not move until molora_hotset_destroy: graphs captured over molora_apply
 * embed its addresses.
 *   layout = MOLORA_LAYOUT_DIRECT:   adapter e of target t lives at
 *            base_t + e * stride_t; kernels compute the address.
 *   layout = MOLORA_LAYOUT_INDIRECT: adapters are placed at permuted slots of
 *            the slab and kernels load their addresses from a per-target
 *            pointer table held in the slab (same arithmetic, one extra
 *            dependent load).
 * Supported: 1 <= K <= 64, 1 <= r <= 64, d_in and d_out multiples of 128,
 * 1 <= n_targets <= 16.
 * ------------------------------------------------------------------------ */
typedef struct molora_hotset molora_hotset;

typedef struct {
  int d_in;      /* input width of the projection */
  int d_out;     /* output width of the projection */
  const void *A; /* device, bf16 [K][d_in][r]; read only during init */
  const void *B; /* device, bf16 [K][r][d_out]; read only during init */
} molora_target;

/* Bytes of slab that molora_hotset_init needs (host arithmetic only). */
int molora_hotset_bytes(int K, int r, int n_targets, const molora_target *targets,
                        int layout, size_t *bytes);

/* Build a hot set.  `scale` is the LoRA factor alpha/r applied to every delta.
 * Synchronous: enqueues the relayout on `stream` and waits for it.  Must not
 * be called while `stream` is being captured.  On success *out owns a new
 * descriptor. */
int molora_hotset_init(molora_hotset **out, int K, int r, float scale, int n_targets,
                       const molora_target *targets, int layout, void *slab,
                       size_t slab_bytes, void *stream);

/* Page one adapter into its hot-set slot (thelatestinai.com, Figure 4 and
 * Table 4: the paging baseline copies adapters from host memory on demand,
 * the hot set keeps them resident at fixed addresses; Figures 7 and 8 compare
 * the two under different access patterns).  Writes adapter e of target
 * `target` into the slot molora_hotset_init gave it, in the same internal
 * layout and bit for bit what init writes for the same weights; the slot's
 * address does not change, so graphs captured over molora_apply stay valid.
 *   A  device bf16 [d_in][r]  row-major (adapter e's A; read by the kernels)
 *   B  device bf16 [r][d_out] row-major (adapter e's B; read by the kernels)
 * Asynchronous: enqueues two copy kernels on `stream` and returns; A and B
 * must stay valid until they have run.  Nothing is synchronised, so the call
 * may be captured in a graph.  Kernels on other streams that read adapter e
 * while the load runs race with it: order them through `stream`.
 * Errors (nothing enqueued): NULL hs, A or B, target or e out of range, or a
 * pointer not 2-byte aligned -> MOLORA_EINVAL; a launch failure -> MOLORA_EHIP. */
int molora_hotset_load(molora_hotset *hs, int target, int e, const void *A, const void *B,
                       void *stream);

/* Free the descriptor (not the slab).  NULL is accepted. */
int molora_hotset_destroy(molora_hotset *hs);

/* ------------------------------------------------------------------------
 * Vocabulary routing R_vocab(v) (thelatestinai.com, Table 1).
 *   ids    device int32 [N]: token ids
 *   bounds host int32 [K+1], non-decreasing: adapter e owns the half-open
 *          id range [bounds[e], bounds[e+1])
 *   idx    device int32 [N] out: adapter of each token, -1 if the id lies
 *          outside [bounds[0], bounds[K])
 *   w      device fp32 [N] out: gate weight, 1 for routed tokens, 0 else
 * 1 <= K <= 64.
 * ------------------------------------------------------------------------ */
int molora_route_vocab(const int32_t *ids, int N, const int32_t *bounds, int K,
                       int32_t *idx, float *w, void *stream);

/* ------------------------------------------------------------------------
 * Learned top-k routing TopK(g_theta(x)) (thelatestinai.com, Table 1 with the
 * routing cost O(64d + 64K), read as the MLP d -> 64 -> K; Figure 2: top-k
 * adapters combined by a weighted sum).
 *   Router mode (W1 != NULL):
 *     x      device bf16 [N][d]
 *     W1     device bf16 [64][d]   (nn.Linear layout: [out][in])
 *     b1     device fp32 [64] or NULL
 *     W2     device bf16 [K][64]
 *     b2     device fp32 [K] or NULL
 *     logits device fp32 [N][K] out: ReLU(x W1^T + b1) W2^T + b2, fp32
 *            accumulation of the bf16 products
 *   Logits mode (W1 == NULL; x, b1, W2, b2 ignored):
 *     logits device fp32 [N][K] in: precomputed gate logits
 *   Selection, both modes:
 *     idx    device int32 [N][k] out: the k largest logits; equal logits are
 *            taken in ascending adapter index; a token's k slots are stored
 *            in ascending adapter index
 *     w      device fp32 [N][k] out: softmax over the k selected logits
 *     flags  device uint8 [N] out or NULL: 1 when k < K and the k-th largest
 *            logit exceeds the (k+1)-th by less than 1e-4 (a near tie)
 *   ws       NULL, or a device workspace (256-byte aligned, no initial
 *            contents) of molora_route_topk_workspace() bytes.  In router
 *            mode with d <= 4096 it holds the first layer's sums over eighths
 *            of d, computed in a launch of its own that reads W1 once per 128
 *            tokens; the selection launch then adds them in the order the
 *            one-launch path uses, so every output is the same bit for bit
 *            with or without it.  Ignored in logits mode and for larger d.
 *            Calls that share a workspace must not run concurrently.
 *   ws_bytes its size
 * Supported: 1 <= K <= 64, 1 <= k <= min(K, 8); router mode needs
 * d a multiple of 128.  Errors: a workspace smaller than required ->
 * MOLORA_ENOSPC.
 * ------------------------------------------------------------------------ */
int molora_route_topk_workspace(int N, int d, size_t *bytes);
int molora_route_topk(const void *x, int N, int d, const void *W1, const float *b1,
                      const void *W2, const float *b2, float *logits, int K, int k,
                      int32_t *idx, float *w, uint8_t *flags, void *ws, size_t ws_bytes,
                      void *stream);

/* ------------------------------------------------------------------------
 * Dispatch: histogram, offsets and grouping permutation (thelatestinai.com,
 * Table 1 rows "Histogram computation" and "Pointer arrays"; Figure 2 right:
 * tokens grouped by their selected adapter).
 *   idx     device int32 [N*k]: adapter of pair p = t*k + s
 *   w       device fp32  [N*k]: gate weight of pair p
 *   counts  device int32 [K] out: routed pairs per adapter
 *   offsets device int32 [K+1] out: exclusive prefix sum of counts;
 *           offsets[K] = number of routed pairs (N*k when all are routed)
 *   perm    device int32 [N*k] out: perm[q] = pair id at grouped position q
 *           (entries q >= offsets[K] are left untouched); inside adapter e's
 *           segment [offsets[e], offsets[e+1]) the pair ids ascend, so the
 *           result is unique and deterministic
 *   perm_w  device fp32 [N*k] out: perm_w[q] = w[perm[q]]
 *   inv     device int32 [N*k] out or NULL: inv[p] = q with perm[q] = p, or
 *           -1 for an unrouted pair
 *   ws      device workspace of at least molora_dispatch_workspace() bytes
 *           (may be NULL when that size is 0; no initial contents needed).
 *           Up to 8192 pairs one launch sorts them (size 0): one workgroup, or
 *           above 4096 pairs with K <= 16 a workgroup per 1024 pairs, each
 *           counting all pairs; above 8192 the sort runs as two launches over
 *           workgroups of 1024 pairs each (of ceil(N*k / 128) rounded up to a
 *           multiple of 1024 above 131072 pairs) and the workspace holds their
 *           per-adapter counts (4*K bytes each).
 *           Calls that share a workspace must not run concurrently.
 * Supported: 1 <= K <= 64, 1 <= k <= 8, N*k < 2^31.
 * ------------------------------------------------------------------------ */
int molora_dispatch_workspace(int N, int k, int K, size_t *bytes);
int molora_dispatch(const int32_t *idx, const float *w, int N, int k, int K,
                    int32_t *counts, int32_t *offsets, int32_t *perm, float *perm_w,
                    int32_t *inv, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Apply: grouped LoRA shrink/expand with the gate-weighted, alpha/r-scaled
 * scatter-add (thelatestinai.com, Figure 2: per-token weighted sum computed by
 * a grouped GEMM over tokens grouped by adapter; Table 10 shapes).
 * For every routed pair q of the dispatch (token t = perm[q] / k, adapter e
 * = the segment holding q):
 *     y[t] = y0[t] + sum_q perm_w[q] * scale * (x[t] A_e) B_e
 * Tokens with no routed pair get y[t] = y0[t].
 *   hs, target  hot set and the projection index inside it
 *   x       device bf16 [N][d_in]
 *   y0      device [N][d_out] base output, dtype y0_dtype (MOLORA_BF16 or
 *           MOLORA_F32); may be the same buffer as y (in place)
 *   y       device [N][d_out] out, dtype y_dtype
 *   offsets, perm, perm_w, inv: the outputs of molora_dispatch for this
 *           routing (all four required)
 *   path    MOLORA_PATH_AUTO (small hot sets, K * r_pad <= 64: _BLOCK from
 *           192 pairs at k > 1, else _GROUPED; at k == 1 _BLOCK from 4096 tokens;
 *           otherwise r <= 32: for k == 1 _TILE when N >= 1024 and K <= 4, else
 *           _GROUPED; for k > 1 _TILE when K <= 16 and N*k >= 192, else
 *           _GROUPED; r > 32: _GROUPED from 1024 pairs, else _SKINNY;
 *           molora_apply_path reports the choice),
 *           _GROUPED (MFMA tiles of grouped rows of one adapter: 16 rows for
 *           k == 1 and r <= 32; otherwise passes over tiles of up to 64 rows,
 *           each adapter segment cut on the device from the offsets into tiles
 *           of balanced height so no tile spans two adapters (thelatestinai.com,
 *           Table 9, adaptive tiling), every tile run as one workgroup per
 *           512-wide slice of d_in (shrink) and of d_out (expand); for k > 1
 *           (k*K <= 64) each pass applies two routed pairs of a token (keyed by
 *           their adapter pair) once N >= 32 K (K + 1), else one routed pair of
 *           every token, the sum carried in fp32 between passes),
 *           _GROUPED_FIXED (the same passes with fixed 64-row tiles per
 *           segment, also for k == 1 and r <= 32: Table 9's fixed tiling, the
 *           comparator of the adaptive one),
 *           _SKINNY (the grouped shrink split over d_in, for small batches;
 *           with 2 <= k <= 4, N <= 1024 and K * r_pad <= 1024 one expand
 *           launch over 32-column slices adds each token's routed pairs in
 *           registers: no rank passes and no fp32 carry), or
 *           _TILE (8 consecutive tokens per workgroup, every adapter the tile
 *           uses applied in turn; needs K <= 16), or
 *           _BLOCK (64 consecutive tokens per block, two launches: the shrink
 *           split over workgroups by 512-wide slices of d_in, writing partial
 *           sums to the workspace, then the expand split by 512-wide slices of
 *           d_out; needs K <= 16)
 *   ws      device workspace of at least molora_apply_workspace() bytes for
 *           the same N, k, y_dtype and path (no initial contents needed; for
 *           k > 1 on the grouped path with a bf16 y it holds an fp32 [N][d_out]
 *           buffer); calls that share a workspace must not run concurrently
 * Accumulation is fp32; the shrink result h stays fp32 and enters the
 * expand as a bf16 hi/lo pair, so bf16 rounding happens only at the store
 * of y when y_dtype is MOLORA_BF16 (round to nearest even).
 * ------------------------------------------------------------------------ */
int molora_apply_workspace(const molora_hotset *hs, int target, int N, int k, int y_dtype,
                           int path, size_t *bytes);
/* The path molora_apply runs for these arguments: `path` itself, or for MOLORA_PATH_AUTO the
 * rule's choice (host arithmetic only, nothing enqueued).  Errors as molora_apply_workspace. */
int molora_apply_path(const molora_hotset *hs, int target, int N, int k, int path, int *resolved);
int molora_apply(const molora_hotset *hs, int target, const void *x, const void *y0,
                 int y0_dtype, void *y, int y_dtype, int N, int k, const int32_t *offsets,
                 const int32_t *perm, const float *perm_w, const int32_t *inv, int path,
                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Several projections sharing one routing (thelatestinai.com, Table 10: the
 * adapter targets of a layer, q/k/v/o/gate/up/down, all follow the token's
 * routing decision): the apply of molora_apply for n <= 8 distinct targets,
 * with one launch per phase for all of them on the skinny path (the rank
 * sort of k > 1 done once, or at decode sizes one expand launch for every
 * target) and on the block path; the grouped and tile paths apply the
 * targets in turn.
 *   targets host int [n]: hot-set target of each projection (distinct)
 *   x, y0, y host arrays [n] of device pointers, as in molora_apply for
 *           targets[i] (y[i] distinct; y0[i] may equal y[i]); one y0_dtype
 *           and one y_dtype for all
 *   N, k, offsets, perm, perm_w, inv, path: as in molora_apply (shared);
 *           AUTO as in molora_apply, except that for n > 1 small hot sets
 *           (K * r_pad <= 64) take _BLOCK from 192 pairs and _BLOCK replaces
 *           _TILE when k > 1
 *   ws      device workspace of at least molora_apply_multi_workspace()
 *           bytes, 256-byte aligned (no initial contents needed)
 * Results equal n molora_apply calls on the resolved path bit for bit.  Errors as molora_apply;
 * MOLORA_ENOTSUP for n outside [1, 8].
 * ------------------------------------------------------------------------ */
int molora_apply_multi_workspace(const molora_hotset *hs, int n, const int *targets, int N,
                                 int k, int y_dtype, int path, size_t *bytes);
int molora_apply_multi(const molora_hotset *hs, int n, const int *targets,
                       const void *const *x, const void *const *y0, int y0_dtype,
                       void *const *y, int y_dtype, int N, int k, const int32_t *offsets,
                       const int32_t *perm, const float *perm_w, const int32_t *inv, int path,
                       void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Dispatch and a multi-target apply in one call (thelatestinai.com, Table 1
 * rows "Histogram computation", "Pointer arrays" and the grouped apply;
 * Table 10: every target of a layer follows the token's routing): equals
 * molora_dispatch(idx, w) followed by molora_apply_multi on its outputs, bit
 * for bit, in fewer launches.  For hot sets whose adapters' 512-wide slices
 * fit in LDS together (K * r_pad <= 64) on the block path, with at most 8192
 * pairs, the block shrink reads each token's adapters and weights from idx
 * and w directly and its launch also runs the dispatch: two launches in all.
 * Otherwise the dispatch runs first.
 *   targets, x, y0, y0_dtype, y, y_dtype, N, k, path: as molora_apply_multi
 *   idx, w   device int32 / fp32 [N*k]: the routing, as molora_dispatch
 *   counts, offsets, perm, perm_w, inv: molora_dispatch's outputs (all
 *            required here)
 *   ws       device workspace of molora_dispatch_apply_multi_workspace()
 *            bytes, 256-byte aligned (no initial contents needed)
 * Errors as molora_dispatch and molora_apply_multi.
 * ------------------------------------------------------------------------ */
int molora_dispatch_apply_multi_workspace(const molora_hotset *hs, int n, const int *targets,
                                          int N, int k, int y_dtype, int path, size_t *bytes);
int molora_dispatch_apply_multi(const molora_hotset *hs, int n, const int *targets,
                                const void *const *x, const void *const *y0, int y0_dtype,
                                void *const *y, int y_dtype, int N, int k, const int32_t *idx,
                                const float *w, int32_t *counts, int32_t *offsets, int32_t *perm,
                                float *perm_w, int32_t *inv, int path, void *ws, size_t ws_bytes,
                                void *stream);

/* ------------------------------------------------------------------------
 * The whole vocabulary-routed step (thelatestinai.com, Table 1: routing
 * decision, histogram, pointer arrays and grouped dispatch; Figure 2:
 * per-token weighted sum; Table 4 "Per-token + Graph": the step in as few
 * launches as possible).  Equivalent to molora_route_vocab, molora_dispatch
 * and molora_apply with k = 1, producing bit-identical idx, w, counts,
 * offsets, perm, perm_w and inv, and y as below.
 *   With a workspace (ws != NULL): two launches over 512-wide slices; the
 *   first routes 64-token blocks from their ids and writes each token's
 *   partial x A_e per d_in slice (its own adapter only), the second sums the
 *   partials in slice order and writes y per output slice; y equals
 *   MOLORA_PATH_BLOCK's bit for bit.  Up to 4096 tokens these two launches
 *   also write the dispatch outputs (no other launch); above that, route and
 *   a chip-wide dispatch run first as launches of their own.
 *   Without a workspace (ws == NULL): up to 4096 tokens one launch of the
 *   8-token tile apply (MOLORA_PATH_TILE's arithmetic) that also routes and
 *   writes the dispatch outputs; above that route, a one-workgroup dispatch
 *   and the tile apply as three launches.
 *   hs, target    hot set with K = hs->K adapters (K <= 16) and the projection
 *   ids, bounds   as molora_route_vocab (bounds: host int32 [K+1])
 *   x, y0, y      as molora_apply (y0 may equal y)
 *   idx, w        device [N] out, as molora_route_vocab
 *   counts..inv   device out, as molora_dispatch with k = 1 (inv required)
 *   ws            NULL, or a device workspace of at least
 *                 molora_step_workspace() bytes for the same hot set, target
 *                 and N, 256-byte aligned, owned by the caller (no initial
 *                 contents needed): the chip-wide dispatch's counts (above
 *                 4096 tokens), then the fp32 partial sums
 *                 [ceil(N/64)][ceil(d_in/512)][64][r_pad].  Calls that share
 *                 a workspace must not run concurrently.
 * Errors: K > 16 -> MOLORA_ENOTSUP; a workspace smaller than required or
 * misaligned -> MOLORA_ENOSPC; NULL or misaligned buffers -> MOLORA_EINVAL;
 * nothing is enqueued on any error.
 * ------------------------------------------------------------------------ */
int molora_step_workspace(const molora_hotset *hs, int target, int N, size_t *bytes);
int molora_step_vocab(const molora_hotset *hs, int target, const int32_t *ids, int N,
                      const int32_t *bounds, const void *x, const void *y0, int y0_dtype,
                      void *y, int y_dtype, int32_t *idx, float *w, int32_t *counts,
                      int32_t *offsets, int32_t *perm, float *perm_w, int32_t *inv,
                      void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * molora_step_vocab with a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments minus ws / ws_bytes, the same
 * launches and bit-identical results.  The workspace is a scratch array of
 * MOLORA_NOALLOC_SCRATCH_BYTES compiled into the library, one per GPU, held
 * until the process ends; its address on the current device is looked up
 * once (in molora_hotset_init, else on the first call on that device).  The
 * call allocates nothing.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (several streams, several host threads) race
 * and must be serialised by the caller.  The array needs no initial
 * contents; it keeps the last call's partial sums.
 * Errors: a step whose molora_step_workspace() exceeds the array ->
 * MOLORA_ENOSPC (nothing enqueued); otherwise as molora_step_vocab.
 * ------------------------------------------------------------------------ */
#define MOLORA_NOALLOC_SCRATCH_BYTES (8u << 20)
int molora_step_vocab_noalloc(const molora_hotset *hs, int target, const int32_t *ids, int N,
                              const int32_t *bounds, const void *x, const void *y0,
                              int y0_dtype, void *y, int y_dtype, int32_t *idx, float *w,
                              int32_t *counts, int32_t *offsets, int32_t *perm, float *perm_w,
                              int32_t *inv, void *stream);

/* ------------------------------------------------------------------------
 * Per-sequence comparator metadata (thelatestinai.com, Table 3: per-sequence
 * routing needs K passes for a K-modality batch; the abstract: work K*N
 * versus N).  From a k = 1 routing idx [N], builds K one-hot dispatches: pass e
 * routes every token to adapter e with weight 1 if idx[t] == e, else 0, so
 * K molora_apply calls (in place, y0 == y after the first) reproduce the
 * per-token result with K*N adapter applications.
 *   offsets device int32 [K][K+1] out;  perm device int32 [N] out (identity);
 *   perm_w  device fp32 [K][N] out.
 * ------------------------------------------------------------------------ */
int molora_seqpass_meta(const int32_t *idx, int N, int K, int32_t *offsets, int32_t *perm,
                        float *perm_w, void *stream);

/* ------------------------------------------------------------------------
 * Backward of the routed LoRA (thelatestinai.com, Figure 2: the grouping by
 * selected adapter serves the gradients too, read backwards; Table 13: the
 * adapters and the router are trained from the loss, without routing labels).
 *
 * molora_hotset_init_transposed builds the transposed twin of a hot set: the
 * same arguments as molora_hotset_init (the same targets, A and B in their
 * forward layouts), but target t of the result maps d_out -> d_in with
 * adapter e = (B_e^T, A_e^T).  molora_apply on it computes
 * y0 + sum w * scale * (x B_e^T) A_e^T, which with x = dL/dy is the adapters'
 * part of dL/dx.  molora_hotset_bytes of the forward targets sizes its slab
 * (the same bytes); molora_hotset_load on the twin takes A and B in their
 * forward layouts as well.  Errors as molora_hotset_init.
 *
 * molora_backward, for one target of a forward hot set `hs` and its twin
 * `hs_t` (same K, r, scale), with the forward's routing (offsets, perm,
 * perm_w, inv of molora_dispatch, as given to molora_apply) and gy = dL/dy:
 *   x    device bf16 [N][d_in]   the forward's input
 *   gy   device bf16 [N][d_out]  dL/dy
 *   dx0  device [N][d_in] (dx0_dtype), the rest of dL/dx (e.g. the base
 *        layer's); dx = dx0 + sum over the token's pairs of
 *        w * scale * (gy B_e^T) A_e^T, written in dx_dtype (bf16 or fp32;
 *        dx may equal dx0 when the dtypes agree).  dx NULL: skipped.
 *   dA   device fp32 [K][d_in][r] out or NULL: sum over adapter e's pairs of
 *        outer(x_t, w * scale * gy_t B_e^T); an adapter without pairs gets 0
 *   dB   device fp32 [K][r][d_out] out or NULL: sum over e's pairs of
 *        outer(w * scale * x_t A_e, gy_t)
 *   dw   device fp32 [N*k] out or NULL: dL/dw of pair p = t*k + s, i.e.
 *        scale * (x_t A_e) . (gy_t B_e^T); 0 for unrouted pairs.  Feed it to
 *        molora_route_topk_backward (below) for the router's gradient.
 *   ws   device workspace of molora_backward_workspace() bytes, 256-byte
 *        aligned, no initial contents (NULL allowed only when N = 0 and dA,
 *        dB are NULL).  Calls sharing it must not overlap.
 * Products are bf16 x bf16 with fp32 accumulation; the per-pair vectors
 * w*scale*h and w*scale*g enter the weight gradients as bf16 hi + lo pairs
 * (about fp32 accuracy).  Sums over pairs run in a fixed order: results are
 * deterministic.  Asynchronous on `stream`, no allocation, capturable.
 * Errors (nothing enqueued): mismatched hot sets, shapes or dtypes, NULL or
 * misaligned required pointers -> MOLORA_EINVAL / MOLORA_ENOTSUP; a short
 * workspace -> MOLORA_ENOSPC.
 * ------------------------------------------------------------------------ */
int molora_hotset_init_transposed(molora_hotset **out, int K, int r, float scale, int n_targets,
                                  const molora_target *targets, int layout, void *slab,
                                  size_t slab_bytes, void *stream);
int molora_backward_workspace(const molora_hotset *hs, const molora_hotset *hs_t, int target,
                              int N, int k, int dx_dtype, size_t *bytes);
int molora_backward(const molora_hotset *hs, const molora_hotset *hs_t, int target,
                    const void *x, const void *gy, const void *dx0, int dx0_dtype, void *dx,
                    int dx_dtype, int N, int k, const int32_t *offsets, const int32_t *perm,
                    const float *perm_w, const int32_t *inv, float *dA, float *dB, float *dw,
                    void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Router gradient (thelatestinai.com, Table 1 TopK(g_theta(x)) with the MLP
 * d -> 64 -> K; Figure 2's weighted sum; Table 13: the router learns from
 * the loss without labels).
 *
 * molora_route_topk_backward: dL/dlogits through the softmax over the k
 * selected logits, the selection held fixed (it is piecewise constant):
 *   idx, w  device int32 / fp32 [N][k]: molora_route_topk's outputs
 *   dw      device fp32 [N][k]: dL/dw (molora_backward's dw of every target,
 *           summed by the caller when several targets share the routing)
 *   dlogits device fp32 [N][K] out: slot j's logit gets
 *           w_j (dw_j - sum_i w_i dw_i); unselected logits get 0.
 *   Slots whose idx lies outside [0, K) receive nothing.
 *
 * molora_router_backward: the MLP's gradients given dlogits, for the
 * router of molora_route_topk (W1 bf16 [64][d] and W2 bf16 [K][64] in
 * nn.Linear layout, b1 fp32 [64] or NULL; b2 does not enter).  The
 * pre-activation x W1^T + b1 is recomputed with the forward's own kernel
 * code, so the ReLU's mask (derivative 1 where the pre-activation is > 0)
 * is the forward's fp32 decision.
 *   dW1 fp32 [64][d], db1 fp32 [64], dW2 fp32 [K][64], db2 fp32 [K]: out or
 *       NULL (sums over the N tokens; zeros when N = 0)
 *   dx  fp32 [N][d] out or NULL: dx0 + dL/d(pre-activation) W1, dx0 fp32
 *       [N][d] or NULL (= 0); dx may equal dx0
 *   ws  device workspace of molora_router_backward_workspace() bytes,
 *       256-byte aligned, no initial contents.
 * dW1 comes from the same MFMA weight-gradient reduction as molora_backward's
 * dA (fixed order); dW2, db1, db2 from per-64-token partial sums added in
 * block order; dx on the vector ALU.  Deterministic, asynchronous,
 * capturable, no allocation.  Supported: 1 <= K <= 64, d a multiple of 128.
 * Errors (nothing enqueued): shapes -> MOLORA_ENOTSUP; NULL or misaligned
 * required pointers, every output NULL -> MOLORA_EINVAL; short workspace ->
 * MOLORA_ENOSPC.
 * ------------------------------------------------------------------------ */
int molora_route_topk_backward(const int32_t *idx, const float *w, const float *dw, int N, int K,
                               int k, float *dlogits, void *stream);
int molora_router_backward_workspace(int N, int d, int K, size_t *bytes);
int molora_router_backward(const void *x, int N, int d, const void *W1, const float *b1,
                           const void *W2, int K, const float *dlogits, float *dW1, float *db1,
                           float *dW2, float *db2, const float *dx0, float *dx, void *ws,
                           size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Synthetic decoder with per-token LoRA (thelatestinai.com, Table 7: an
 * end-to-end transformer, d = 1024/2048/4096, L = 2/4, whose per-token pass is
 * compared with a per-sequence simulation of one forward pass per adapter;
 * Table 8: an interleaved two-modality batch, d = 2048, L = 4, K = 2).  The
 * pages fix only d, L, K and the batch; this layer is a plain pre-norm
 * decoder:
 *   x += o(attn(rmsnorm1(x)));   x += down(silu(gate(h)) * up(h)), h = rmsnorm2(x)
 * RMSNorm with a learned weight and eps 1e-6; causal softmax attention inside
 * each sequence, heads of width 128 (d / 128 heads), scores scaled by
 * 1/sqrt(128), no positional encoding; no biases.  Each of the seven
 * projections q, k, v, o, gate, up, down is base + per-token LoRA: the base
 * product (rocBLAS, bf16 operands, fp32 accumulation, stored bf16) then the
 * grouped per-token delta of molora_apply added in place, all projections
 * sharing one routing (offsets, perm, perm_w, inv of molora_dispatch for the
 * N = n_seq * seq_len tokens, token t of sequence b being row b * seq_len + t).
 * Activations are stored bf16 between kernels.
 *   layer.norm1, norm2  device bf16 [d]
 *   layer.W[7]          device bf16, nn.Linear layout [out][in]: q, k, v, o
 *                       [d][d]; gate, up [f][d]; down [d][f]
 *   layer.lora          a forward hot set of exactly these 7 targets (in that
 *                       order and those shapes), or NULL: no adapters on that
 *                       layer.  Every LoRA layer has the same K.
 *   x_in, x_out         device bf16 [N][d] (x_out may equal x_in)
 *   ws                  molora_xf_workspace() bytes, 256-byte aligned, no
 *                       initial contents (activations, scores, the applies'
 *                       workspace and rocBLAS's; the first call on a device
 *                       creates that device's rocBLAS handle).
 * Supported: d, f multiples of 128; 1 <= k <= 8.  Asynchronous on `stream`.
 * Errors (nothing enqueued): shapes -> MOLORA_ENOTSUP; NULL, misaligned or
 * mismatched arguments -> MOLORA_EINVAL; short workspace -> MOLORA_ENOSPC; a
 * failed launch or GEMM -> MOLORA_EHIP.
 * ------------------------------------------------------------------------ */
typedef struct {
  const void *norm1, *norm2;
  const void *W[7];
  const molora_hotset *lora;
} molora_xf_layer;
int molora_xf_workspace(int d, int f, int n_layers, const molora_xf_layer *layers, int n_seq,
                        int seq_len, int k, size_t *bytes);
int molora_xf_forward(int d, int f, int n_layers, const molora_xf_layer *layers, int n_seq,
                      int seq_len, const void *x_in, void *x_out, int k, const int32_t *offsets,
                      const int32_t *perm, const float *perm_w, const int32_t *inv, void *ws,
                      size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOLORA_H */
