/*
 * moe.h - C ABI of the MI355X (gfx950) forward pass of one mixture-of-experts
 * FFN layer on one GPU's share of experts.
 *
 * The layer (pages: "Expert Parallelism (MoE)", section "MoE Layer Structure";
 * "Expert Parallelism (EP)", section "Key math / How it works"):
 *   route    - a router Linear d -> E scores every token, softmax turns the
 *              logits into probabilities, the top-k experts are selected;
 *   dispatch - each selected (token, slot) is moved to its expert; on one GPU
 *              this is a permutation into expert-contiguous rows, with an
 *              optional capacity cap that drops overflowing selections
 *              ("Top-K Routing and Capacity Factor");
 *   experts  - each expert applies Linear(d -> ffn) -> GELU -> Linear(ffn -> d);
 *   combine  - Y[t] = sum over the kept selections of routing weight times the
 *              expert output, written back at the token's own position.
 * The router also emits the load statistics of the auxiliary balancing loss
 * L_aux = alpha * sum_i f_i * P_i ("Load Balancing: The Auxiliary Loss").
 *
 * Conventions for every entry point
 *  - Buffer pointers are DEVICE pointers on the current HIP device, allocated
 *    and owned by the caller, row-major and densely packed.  The library never
 *    allocates, frees or keeps device memory (except the fixed static scratch
 *    of moe_dispatch_noalloc, part of the loaded library), and keeps no state
 *    between calls except a thread-local copy of the last error message.
 *  - Work is enqueued on `stream` (NULL = the default stream) and is
 *    asynchronous: a call returns before the GPU has finished and never
 *    synchronises.  Counts that the GPU computes (rows per expert, drops) never
 *    come back to the host inside a call: grids are sized from bounds and read
 *    the actual counts on the device.  A call enqueues kernel launches only
 *    (no memset or copy nodes), so it may be captured into a HIP graph and
 *    replayed, with the same buffers (moe_forward_overlap also records and
 *    waits on the caller's events between its two streams).
 *  - Errors: arguments are validated before anything is enqueued; an invalid
 *    call returns a non-zero status, enqueues nothing and leaves every output
 *    untouched.  MOE_ERR_HIP reports a launch failure (moe_last_error() has the
 *    HIP message); faults inside a kernel surface at the caller's next
 *    synchronisation, as with any asynchronous HIP work.
 *  - Workspaces (`ws`, `ws_bytes`) are caller-provided device scratch of at
 *    least the size the matching *_workspace_size function returns.  Their
 *    first 256 bytes hold arrival counters (the single-launch router's): they
 *    must be zero before the first call on a workspace (allocate it zeroed or
 *    clear it once), and every call leaves them zero when its work completes.
 *    The rest needs no initialisation and is undefined afterwards.  Calls
 *    that share one workspace must be ordered on one stream.
 *  - dtype: MOE_BF16 (bfloat16) or MOE_F32 for activations, expert weights and
 *    expert biases.  The router weight and bias, routing weights and load
 *    statistics are always float32.  Integer outputs are int32.
 *  - Weights use the nn.Linear layout [out, in], stacked along a leading expert
 *    dimension, so one GPU's share of experts is a contiguous slice.
 *  - Sizes: 1 <= k <= min(E, 32), E <= 1024, d and ffn multiples of 8.  T = 0
 *    is valid and writes only the small outputs (zero counts and statistics).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* a size, pointer or range is invalid           */
    MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement  */
    MOE_ERR_WORKSPACE = 3,   /* ws is NULL or smaller than required           */
    MOE_ERR_HIP = 4          /* a HIP runtime call or launch failed           */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Version of this ABI (bumped on any incompatible change). */
int moe_abi_version(void);
/* Static description of a status code. */
const char *moe_status_string(moe_status_t s);
/* Message of the last failed call on this thread ("" if none). */
const char *moe_last_error(void);

/* Largest number of dispatched rows any routing can produce: T*k without a
 * cap, min(T*k, E_loc*C) with capacity C = floor(T*capacity_factor/E).
 * num_local_experts = 0 means E.  Returns -1 on invalid sizes. */
int64_t moe_max_rows(int64_t T, int E, int k, float capacity_factor, int num_local_experts);

/* ------------------------------------------------------------------------ *
 * moe_route - router Linear, softmax, top-k and load statistics.
 *
 * "MoE Layer Structure": the router is a Linear d -> E producing per-token
 * expert ids; the top-k experts of each token are activated, and the routing
 * weight of an expert multiplies its output in Y.  Computed here:
 *   logits[t,e] = sum_i x[t,i] * w_router[e,i] + b_router[e]  (fp32 accumulate)
 *   p[t,:]      = softmax(logits[t,:]) over all E experts
 *   topk_idx[t,j], j = 0..k-1: experts by score descending, ties to the lower
 *                 id; score[t,e] = logits[t,e] (+ sel_bias[e] when given)
 *   topk_w[t,j] = p[t, topk_idx[t,j]]  (full-softmax probability, not
 *                 renormalised over the selected experts)
 * sel_bias ("Expert Parallelism (EP)", "Key math / How it works", load
 * balancing: DeepSeek-V3 balances with a bias adjustment instead of the
 * auxiliary loss) is a per-expert bias on the selection only: the weights,
 * P and L_aux come from the unbiased softmax.  How the bias is updated
 * between steps is not part of this call.
 * "Load Balancing: The Auxiliary Loss":
 *   expert_count[e] = number of (t, j) with topk_idx[t,j] = e (before any cap)
 *   f[e] = expert_count[e] / T,  P[e] = (1/T) sum_t p[t,e]
 *   l_aux[0] = alpha * sum_e f[e] * P[e]     (alpha: 0.01 is the usual value)
 * The reductions over tokens run in a fixed order: results are bitwise
 * reproducible run to run.  With bf16 activations and E <= 64 the whole call
 * is one kernel launch: the blocks' partial statistics are summed in a fixed
 * order, in groups of blocks and then over the groups, by the last blocks to
 * finish, using the workspace's arrival counters.
 *
 * x [T,d] (dtype), w_router [E,d] f32, b_router [E] f32 or NULL (zero bias),
 * sel_bias [E] f32 or NULL (plain top-k).
 * topk_idx [T,k] i32 and topk_w [T,k] f32 are required; expert_count [E],
 * f [E], P [E], l_aux [1] may each be NULL (not written).
 * ws: moe_route_workspace_size(T, d, E) bytes.
 * Errors: INVALID_ARG for T < 0, d < 1, E < 1, k < 1, k > E, NULL x, w_router,
 * topk_idx or topk_w; UNSUPPORTED for E > 1024, k > 32, d % 8 != 0,
 * d > 2^21; WORKSPACE for a small ws.
 * ------------------------------------------------------------------------ */
size_t moe_route_workspace_size(int64_t T, int d, int E);
moe_status_t moe_route(const void *x, moe_dtype_t dtype, const float *w_router,
                       const float *b_router, const float *sel_bias, int64_t T, int d, int E, int k,
                       float alpha,
                       int32_t *topk_idx, float *topk_w, int32_t *expert_count, float *f,
                       float *P, float *l_aux, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_dispatch - capacity, token dropping and the expert-contiguous permutation.
 *
 * "Top-K Routing and Capacity Factor": capacity = (tokens per batch /
 * N_experts) * capacity_factor; selections that would push an expert over it
 * are dropped and their routing weight is zeroed.  "Key math / How it works":
 * dispatch moves each token to the owner of its expert; on one GPU that is a
 * permutation into expert-contiguous rows of this GPU's share of experts
 * [expert_begin, expert_begin + num_local_experts).
 *
 *   C = floor(T * capacity_factor / E) when capacity_factor > 0, else no cap.
 *   Selections are taken in token order (t ascending, then slot j).  A
 *   selection of a non-local expert (or an id outside [0, E)) is remote.  A
 *   local selection is kept while its expert has fewer than C earlier
 *   selections, otherwise dropped.
 *   kept_count[l]  = kept selections of local expert l
 *   seg_offsets    = exclusive scan of kept_count ([E_loc + 1], last = rows)
 *   slot_row[t,j]  = seg_offsets[l] + (rank of the selection among the kept
 *                    selections of its expert), -1 dropped, -2 remote
 *   row_src[row]   = t*k + j of the selection placed in that row
 *   x_perm[row,:]  = x[t,:]        (skipped when x_perm is NULL)
 *   n_dropped[0]   = local selections dropped by the cap
 * Rows are ordered by (local expert, token): the result is unique and
 * bitwise reproducible.
 *
 * x [T,d] (dtype; may be NULL when x_perm is NULL or T = 0), topk_idx [T,k]
 * i32, seg_offsets [E_loc+1], kept_count [E_loc], slot_row [T,k], row_src
 * [max_rows], x_perm [max_rows, d] or NULL, n_dropped [1] or NULL (with
 * T = 0 only seg_offsets, kept_count and n_dropped are written, all zero).
 * max_rows must be >= moe_max_rows(T, E, k, capacity_factor, num_local_experts).
 * num_local_experts = 0 means the whole layer (expert_begin must then be 0).
 * ws: moe_dispatch_workspace_size(T, k, E_loc) bytes.
 * Errors: INVALID_ARG for bad sizes, a local range outside [0, E), a small
 * max_rows, or NULL required pointers; UNSUPPORTED for E > 1024, k > 32,
 * d % 8 != 0; WORKSPACE for a small ws.
 * ------------------------------------------------------------------------ */
size_t moe_dispatch_workspace_size(int64_t T, int k, int num_local_experts);
moe_status_t moe_dispatch(const void *x, moe_dtype_t dtype, const int32_t *topk_idx, int64_t T,
                          int d, int E, int k, float capacity_factor, int expert_begin,
                          int num_local_experts, int32_t *seg_offsets, int32_t *kept_count,
                          int32_t *slot_row, int32_t *row_src, void *x_perm, int64_t max_rows,
                          int32_t *n_dropped, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_dispatch_noalloc - moe_dispatch for callers that cannot allocate device
 * memory or hand over a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Same arguments, results and errors as moe_dispatch, without ws/ws_bytes:
 * the planner's scratch lives in a static device buffer of the library
 * (moe_dispatch_noalloc_scratch_bytes() bytes, 64 KiB, one per device, held
 * until the process ends).  The call allocates nothing and calls no
 * allocating routine.  Sizes whose scratch need (moe_dispatch_workspace_size)
 * exceeds the buffer return MOE_ERR_UNSUPPORTED (the planner keeps it within
 * 64 KiB for every supported size).  Every call on a device shares that
 * device's buffer: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.
 * ------------------------------------------------------------------------ */
size_t moe_dispatch_noalloc_scratch_bytes(void);
moe_status_t moe_dispatch_noalloc(const void *x, moe_dtype_t dtype, const int32_t *topk_idx, int64_t T, int d,
                                  int E, int k, float capacity_factor, int expert_begin, int num_local_experts,
                                  int32_t *seg_offsets, int32_t *kept_count, int32_t *slot_row,
                                  int32_t *row_src, void *x_perm, int64_t max_rows, int32_t *n_dropped,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_grouped_gemm - one Linear layer of every expert over its row segment.
 *
 * The expert GEMMs of "Key math / How it works", one Linear of the expert
 * FFN of "MoE Layer Structure".  For each segment s (rows seg_offsets[s] ..
 * seg_offsets[s+1] - 1 of a):
 *   out[r, n] = act( sum_k a[r, k] * w[s, n, k] + bias[s, n] )
 * with act = identity (activation 0) or GELU 0.5*u*(1 + erf(u/sqrt 2))
 * (activation 1; erf to within 1.5e-7).  Accumulation is fp32; bf16 outputs
 * are rounded to nearest even.  Rows outside every segment are not written.
 *
 * a [max_rows, K], w [num_segments, N, K], bias [num_segments, N] or NULL,
 * out [max_rows, N], all in dtype.  seg_offsets [num_segments + 1] on the
 * device, non-decreasing; offsets are clamped to [0, max_rows].
 * seg_offsets = NULL means one segment covering rows 0 .. max_rows - 1.
 * ws (optional, may be NULL): device scratch of at least
 * moe_grouped_gemm_workspace_size() bytes.  With it, the tiles of a last,
 * partly filled round are split along K over the idle compute units and
 * their fp32 partial sums are added in a fixed order (results stay bitwise
 * reproducible); without it every tile runs whole.
 * Errors: INVALID_ARG for sizes < 1 (max_rows = 0 is a no-op), NULL a, w or
 * out, misaligned buffers; UNSUPPORTED for N or K not a multiple of 8,
 * N or K above 2^21, activation not 0 or 1, more than 1024 segments.
 * ------------------------------------------------------------------------ */
size_t moe_grouped_gemm_workspace_size(void);
moe_status_t moe_grouped_gemm(const void *a, const int32_t *seg_offsets, int num_segments,
                              int64_t max_rows, int N, int K, moe_dtype_t dtype, const void *w,
                              const void *bias, int activation, void *out, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_expert_ffn - the expert FFN of "MoE Layer Structure" on every segment:
 *   h      = GELU(x_perm . w1[s]^T + b1[s])     [rows, ffn]
 *   y_perm = h . w2[s]^T + b2[s]                [rows, d]
 * x_perm [max_rows, d], w1 [S, ffn, d], b1 [S, ffn] or NULL, w2 [S, d, ffn],
 * b2 [S, d] or NULL, h [max_rows, ffn] (scratch, written), y_perm
 * [max_rows, d]; S = num_segments.  seg_offsets and ws as in
 * moe_grouped_gemm (the two layers share ws one after the other).
 * Errors: as moe_grouped_gemm, for both layers.
 * ------------------------------------------------------------------------ */
moe_status_t moe_expert_ffn(const void *x_perm, const int32_t *seg_offsets, int num_segments,
                            int64_t max_rows, int d, int ffn, moe_dtype_t dtype, const void *w1,
                            const void *b1, const void *w2, const void *b2, void *h, void *y_perm,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_combine - the weighted sum of "MoE Layer Structure", back at each
 * token's own position ("Key math / How it works": combine sends outputs back
 * to each token's home position):
 *   y[t,:] = sum_{j : 0 <= slot_row[t,j] < max_rows} topk_w[t,j] * y_perm[slot_row[t,j], :]
 *            (+ y_shared[t,:])
 * summed in fp32 in slot order j = 0..k-1, the shared term last.  Dropped and
 * remote selections (slot_row < 0) contribute nothing, so a token with no kept
 * selection gets 0 (or y_shared).
 * y_perm [max_rows, d], slot_row [T,k], topk_w [T,k] f32, y_shared [T,d] or
 * NULL, y [T,d]; activations in dtype.
 * Errors: INVALID_ARG for bad sizes or NULL required pointers; UNSUPPORTED for
 * k > 32 or d % 8 != 0.
 * ------------------------------------------------------------------------ */
moe_status_t moe_combine(const void *y_perm, int64_t max_rows, const int32_t *slot_row,
                         const float *topk_w, const void *y_shared, int64_t T, int d, int k,
                         moe_dtype_t dtype, void *y, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_forward - the whole layer: route, dispatch, expert FFN (plus the shared
 * expert when present), combine; enqueued on one stream with no host
 * synchronisation.
 *
 * The shared expert ("Expert Parallelism (EP)", "Key math / How it works":
 * DeepSeek-V3's 256 routed + 1 shared experts; "Production MoE Models":
 * shared experts for non-routed computation) runs on every token with weight
 * 1 and is added in the combine.  A local share of experts
 * (expert_begin, num_local_experts) is one GPU's slice of the layer: the
 * router still scores all E experts, selections of other GPUs' experts are
 * left out of this GPU's dispatch and output, and the statistics cover all E.
 * ------------------------------------------------------------------------ */
typedef struct {
    int64_t T;               /* tokens                                        */
    int32_t d, E, k, ffn;    /* hidden, experts scored, selected, inner size  */
    float capacity_factor;   /* <= 0: no cap                                  */
    int32_t expert_begin;    /* first local expert                            */
    int32_t num_local_experts; /* 0 = all E                                   */
    int32_t has_shared;      /* 1: weights carry a shared expert              */
    float alpha;             /* balancing weight of L_aux                     */
    moe_dtype_t dtype;
} moe_problem_t;

typedef struct {
    const float *w_router, *b_router;   /* [E,d], [E] or NULL, f32             */
    const void *w1, *b1, *w2, *b2;      /* local experts: [E_loc,ffn,d], [E_loc,ffn]|NULL,
                                           [E_loc,d,ffn], [E_loc,d]|NULL        */
    const void *ws1, *bs1, *ws2, *bs2;  /* shared expert: [ffn,d], [ffn]|NULL,
                                           [d,ffn], [d]|NULL                    */
    const float *sel_bias;              /* [E] or NULL: selection-only router bias
                                           (see moe_route)                      */
} moe_weights_t;

/* Optional outputs; every field may be NULL (then kept in the workspace). */
typedef struct {
    int32_t *topk_idx;     /* [T,k] */
    float *topk_w;         /* [T,k] */
    int32_t *expert_count; /* [E]   */
    float *f, *P, *l_aux;  /* [E], [E], [1] */
    int32_t *seg_offsets;  /* [E_loc+1] */
    int32_t *kept_count;   /* [E_loc] */
    int32_t *slot_row;     /* [T,k] */
    int32_t *row_src;      /* [moe_max_rows(...)] */
    int32_t *n_dropped;    /* [1] */
} moe_outputs_t;

size_t moe_forward_workspace_size(const moe_problem_t *p);
moe_status_t moe_forward(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                         const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_forward_overlap - moe_forward with the shared expert on a second stream
 * ("Expert Parallelism (EP)", "Key math / How it works": the shared expert's
 * work does not depend on the routing, so it can run while the routed path
 * routes and dispatches).
 *
 * side: a second stream of the same device (default priority); fork, join:
 * two caller-owned events (hipEventDisableTiming is enough), reused by every
 * call and recorded by it, so the call creates and frees nothing.  `fork` is
 * recorded on `stream` and waited for by `side`; the shared expert's two
 * GEMMs are enqueued on `side`; `join` is recorded on `side` and waited for
 * by `stream` before the combine.  Everything else is enqueued on `stream`
 * exactly as in moe_forward, and the results are bitwise identical to
 * moe_forward's.  Without a shared expert (or with side == NULL or side ==
 * stream) this is moe_forward and the events are not used.
 * If an error stops the call after work was put on `side`, `side` is still
 * joined back into `stream` before the call returns, so nothing the call
 * enqueued runs outside `stream`'s order.  Events and streams may be captured
 * into a HIP graph together with the call (fork/join edges).
 * ws: moe_forward_overlap_workspace_size(p) bytes (the shared expert gets its
 * own intermediate and split-K buffers).
 * Errors: as moe_forward, plus INVALID_ARG for a missing event when the
 * shared expert goes to `side`, and MOE_ERR_HIP if an event record or wait
 * fails.
 * ------------------------------------------------------------------------ */
typedef struct ihipEvent_t *hipEvent_t;
size_t moe_forward_overlap_workspace_size(const moe_problem_t *p);
moe_status_t moe_forward_overlap(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                                 const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t stream,
                                 hipStream_t side, hipEvent_t fork, hipEvent_t join);

/* ------------------------------------------------------------------------ *
 * moe_backward - gradients of a scalar loss L through the layer of moe_forward.
 *
 * "Load Balancing: The Auxiliary Loss": L_aux = alpha * sum_i f_i * P_i is
 * added to the task loss and backpropagated; f_i counts selections and has no
 * gradient, P_i is the mean router probability of expert i.  "MoE Layer
 * Structure": Y is the routing-weighted sum of the expert outputs, the
 * routing weight being the softmax probability of the selected expert.  Top-k
 * selection (with or without sel_bias) and capacity dropping are piecewise
 * constant: no gradient flows through them.
 *
 * Inputs: the layer (p, w, x) exactly as given to moe_forward, dy = dL/dY
 * [T,d] in the layer's dtype, g_aux = dL/dL_aux.  Routing, dispatch and the
 * first Linear are recomputed on the device with the forward's kernels, so the
 * selections and drops are those of moe_forward.
 * Outputs (float32, caller-owned, overwritten; grads->... NULL where allowed):
 *   dx [T,d] (may be NULL when T = 0), dw_router [E,d], dw1 [E_loc,ffn,d],
 *   dw2 [E_loc,d,ffn] required;
 *   dws1 [ffn,d], dws2 [d,ffn] required with a shared expert;
 *   db_router [E], db1 [E_loc,ffn], db2 [E_loc,d], dbs1 [ffn], dbs2 [d] and
 *   dlogits [T,E] (dL/d router logits) optional.
 * With a local share (num_local_experts < E) the routed terms cover this
 * GPU's experts only: dL/dp takes the dw of the local kept selections, plus
 * the auxiliary-loss term g_aux * alpha * f_e / T for every e.
 * Arithmetic: expert GEMMs on the layer's dtype with fp32 accumulation (bf16
 * operands for MOE_BF16: the GELU-backward output and the hidden activation
 * are rounded to bf16 before their GEMMs); router, softmax and every
 * reduction in fp32.  Results are bitwise reproducible run to run.
 * Every buffer is 16-byte aligned.
 * Sizes: as moe_forward; MOE_BF16 also needs d and ffn multiples of 64 and at
 * least 128, and the weight-gradient GEMMs at most 2^21 columns (about the
 * layer's kept rows plus 128 per local expert) (else MOE_ERR_UNSUPPORTED).
 * ws: moe_backward_workspace_size(p) bytes.
 * Errors: as moe_forward.
 * ------------------------------------------------------------------------ */
typedef struct {
    float *dx;                       /* [T,d]                                  */
    float *dw_router, *db_router;    /* [E,d], [E]                             */
    float *dw1, *db1, *dw2, *db2;    /* [E_loc,ffn,d], [E_loc,ffn], [E_loc,d,ffn], [E_loc,d] */
    float *dws1, *dbs1, *dws2, *dbs2; /* [ffn,d], [ffn], [d,ffn], [d]          */
    float *dlogits;                  /* [T,E]                                  */
} moe_grads_t;

size_t moe_backward_workspace_size(const moe_problem_t *p);
moe_status_t moe_backward(const moe_problem_t *p, const moe_weights_t *w, const void *x, const void *dy,
                          float g_aux, const moe_grads_t *grads, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * moe_forward_save / moe_backward_saved - the same forward and backward with
 * the first Linear's pre-activations kept in between, so that the backward
 * does not recompute that GEMM ("MoE Layer Structure": each expert is
 * Linear -> GELU -> Linear; the backward of GELU needs its input).
 *
 * moe_forward_save writes, besides everything moe_forward writes,
 *   u_saved        [moe_max_rows(...), ffn] fp32: u = W1 x + b1 of every
 *                  dispatched row, in the dispatch's row order (rows past
 *                  the kept ones are left untouched);
 *   u_shared_saved [T, ffn] fp32: the shared expert's u (NULL without one),
 * and then applies GELU to them in a separate pass; y and the outputs are
 * bitwise those of moe_forward.  ws: moe_forward_workspace_size(p) bytes.
 * moe_backward_saved takes the same arguments as moe_backward plus those two
 * buffers, which must come from moe_forward_save on the same p, w and x
 * (the routing is recomputed and is the forward's: same inputs, same
 * selections); its gradients are bitwise those of moe_backward.
 * ws: moe_backward_workspace_size(p) bytes.
 * Both buffers are caller-owned, 16-byte aligned, required when T > 0
 * (u_shared_saved only with a shared expert).  MOE_BF16 needs d a multiple
 * of 64 and at least 128 (else MOE_ERR_UNSUPPORTED), as moe_backward does.
 * Errors: as moe_forward / moe_backward, plus MOE_ERR_INVALID_ARG for a
 * missing or misaligned u buffer.
 * ------------------------------------------------------------------------ */
moe_status_t moe_forward_save(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                              const moe_outputs_t *out, float *u_saved, float *u_shared_saved, void *ws,
                              size_t ws_bytes, hipStream_t stream);
moe_status_t moe_backward_saved(const moe_problem_t *p, const moe_weights_t *w, const void *x, const void *dy,
                                float g_aux, const float *u_saved, const float *u_shared_saved,
                                const moe_grads_t *grads, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
