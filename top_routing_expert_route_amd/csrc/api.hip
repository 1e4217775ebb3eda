// Public C ABI of the MoE layer library: argument validation, workspace
// sizing and carving, and the stream-ordered orchestration of the kernels.
// Every entry point validates before anything is enqueued.
#include "common.hpp"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

namespace moe {

static thread_local char g_err[512];

moe_status_t fail(moe_status_t s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = 0; }

moe_status_t check_launch(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

} // namespace moe

using namespace moe;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int local_count(int E, int num_local_experts) { return num_local_experts > 0 ? num_local_experts : E; }

moe_status_t check_ws(void *ws, size_t ws_bytes, size_t need, const char *who)
{
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    ws ? ws_bytes : (size_t)0);
    return MOE_OK;
}

moe_status_t check_route_args(const void *x, moe_dtype_t dt, const float *w_router, int64_t T, int d, int E, int k,
                              const int32_t *topk_idx, const float *topk_w)
{
    if (dt != MOE_F32 && dt != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "route: unknown dtype %d", (int)dt);
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E)
        return fail(MOE_ERR_INVALID_ARG, "route: invalid sizes T=%lld d=%d E=%d k=%d", (long long)T, d, E, k);
    if (!w_router || (T > 0 && (!x || !topk_idx || !topk_w)))
        return fail(MOE_ERR_INVALID_ARG, "route: a required pointer is NULL");
    if (!aligned16(x) || !aligned16(w_router))
        return fail(MOE_ERR_INVALID_ARG, "route: x and w_router must be 16-byte aligned");
    if (E > 1024 || k > 32 || d % 8 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "route: needs E <= 1024, k <= 32, d %% 8 == 0 (E=%d k=%d d=%d)", E, k, d);
    if (T > (int64_t)INT32_MAX / (k > 0 ? k : 1))
        return fail(MOE_ERR_UNSUPPORTED, "route: T*k must fit int32");
    return MOE_OK;
}

moe_status_t check_dispatch_args(const void *x, moe_dtype_t dt, const int32_t *topk_idx, int64_t T, int d, int E,
                                 int k, float cf, int e0, int nle, const int32_t *seg_offsets,
                                 const int32_t *kept_count, const int32_t *slot_row, const int32_t *row_src,
                                 const void *x_perm, int64_t max_rows)
{
    if (dt != MOE_F32 && dt != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "dispatch: unknown dtype %d", (int)dt);
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E || nle < 0 || e0 < 0)
        return fail(MOE_ERR_INVALID_ARG, "dispatch: invalid sizes T=%lld d=%d E=%d k=%d", (long long)T, d, E, k);
    if (nle == 0 && e0 != 0)
        return fail(MOE_ERR_INVALID_ARG, "dispatch: num_local_experts = 0 (whole layer) needs expert_begin = 0");
    const int E_loc = local_count(E, nle);
    if ((int64_t)e0 + E_loc > E)
        return fail(MOE_ERR_INVALID_ARG, "dispatch: local experts [%d, %d) outside [0, %d)", e0, e0 + E_loc, E);
    if (!(cf == cf))
        return fail(MOE_ERR_INVALID_ARG, "dispatch: capacity_factor is NaN");
    if (!seg_offsets || !kept_count || (T > 0 && (!topk_idx || !slot_row || !row_src)))
        return fail(MOE_ERR_INVALID_ARG, "dispatch: a required pointer is NULL");
    if (x_perm && !x)
        return fail(MOE_ERR_INVALID_ARG, "dispatch: x_perm needs x");
    if (!aligned16(x) || !aligned16(x_perm))
        return fail(MOE_ERR_INVALID_ARG, "dispatch: x and x_perm must be 16-byte aligned");
    if (E > 1024 || k > 32 || d % 8 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "dispatch: needs E <= 1024, k <= 32, d %% 8 == 0");
    if (T > (int64_t)INT32_MAX / k)
        return fail(MOE_ERR_UNSUPPORTED, "dispatch: T*k must fit int32");
    const int64_t need = moe_max_rows(T, E, k, cf, nle);
    if (max_rows < need)
        return fail(MOE_ERR_INVALID_ARG, "dispatch: max_rows %lld < %lld rows the routing can produce",
                    (long long)max_rows, (long long)need);
    return MOE_OK;
}

moe_status_t check_gemm_args(const void *a, const int32_t *seg, int S, int64_t max_rows, int N, int K,
                             moe_dtype_t dt, const void *w, const void *bias, int act, const void *out,
                             const char *who)
{
    if (dt != MOE_F32 && dt != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dt);
    if (max_rows < 0 || N < 1 || K < 1 || (seg && S < 1))
        return fail(MOE_ERR_INVALID_ARG, "%s: invalid sizes rows=%lld N=%d K=%d S=%d", who, (long long)max_rows, N,
                    K, S);
    if (max_rows > 0 && (!a || !w || !out))
        return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", who);
    if (!aligned16(a) || !aligned16(w) || !aligned16(out) || !aligned16(bias))
        return fail(MOE_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", who);
    if (N % 8 != 0 || K % 8 != 0 || act < 0 || act > 1 || (seg && S > 1024))
        return fail(MOE_ERR_UNSUPPORTED, "%s: needs N, K multiples of 8, activation 0/1, <= 1024 segments", who);
    if (max_rows > (int64_t)INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "%s: rows must fit int32", who);
    return MOE_OK;
}

moe_status_t check_combine_args(const void *y_perm, int64_t max_rows, const int32_t *slot_row, const float *topk_w,
                                const void *y_shared, int64_t T, int d, int k, moe_dtype_t dt, const void *y)
{
    if (dt != MOE_F32 && dt != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "combine: unknown dtype %d", (int)dt);
    if (T < 0 || d < 1 || k < 1 || max_rows < 0)
        return fail(MOE_ERR_INVALID_ARG, "combine: invalid sizes");
    if (T > 0 && (!slot_row || !topk_w || !y || (max_rows > 0 && !y_perm)))
        return fail(MOE_ERR_INVALID_ARG, "combine: a required pointer is NULL");
    if (!aligned16(y_perm) || !aligned16(y_shared) || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "combine: buffers must be 16-byte aligned");
    if (k > 32 || d % 8 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "combine: needs k <= 32, d %% 8 == 0");
    return MOE_OK;
}

size_t elem_size(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }

// Workspace layout of moe_forward; with base == nullptr only sizes are summed.
struct ForwardWs {
    int32_t *topk_idx, *expert_count, *seg_offsets, *kept_count, *slot_row, *row_src, *n_dropped;
    float *topk_w, *f, *P, *l_aux;
    void *route_ws, *dispatch_ws, *gemm_ws, *x_perm, *h, *y_perm, *y_sh;
    void *h_sh, *gemm_ws_sh; // the shared expert's own buffers when it runs on a second stream
    size_t gemm_ws_bytes;
    size_t bytes;
};

ForwardWs carve_forward(const moe_problem_t *p, const moe_outputs_t *out, void *base, bool overlap = false)
{
    static const moe_outputs_t none = {};
    if (!out)
        out = &none;
    const int E_loc = local_count(p->E, p->num_local_experts);
    const int64_t max_rows = moe_max_rows(p->T, p->E, p->k, p->capacity_factor, p->num_local_experts);
    const size_t es = elem_size(p->dtype);
    const int64_t Tk = p->T * p->k;
    Carver cv{(char *)base, 0};
    ForwardWs w;
    w.topk_idx = out->topk_idx ? out->topk_idx : cv.take<int32_t>((size_t)Tk);
    w.topk_w = out->topk_w ? out->topk_w : cv.take<float>((size_t)Tk);
    w.expert_count = out->expert_count;
    w.f = out->f;
    w.P = out->P;
    w.l_aux = out->l_aux;
    w.route_ws = cv.take<char>(route_ws_bytes(p->T, p->d, p->E));
    w.seg_offsets = out->seg_offsets ? out->seg_offsets : cv.take<int32_t>((size_t)E_loc + 1);
    w.kept_count = out->kept_count ? out->kept_count : cv.take<int32_t>((size_t)E_loc);
    w.slot_row = out->slot_row ? out->slot_row : cv.take<int32_t>((size_t)Tk);
    w.row_src = out->row_src ? out->row_src : cv.take<int32_t>((size_t)max_rows);
    w.n_dropped = out->n_dropped;
    w.dispatch_ws = cv.take<char>(dispatch_ws_bytes(p->T, p->k, E_loc));
    w.gemm_ws_bytes = p->dtype == MOE_BF16 ? gemm_ws_bytes() : 0;
    w.gemm_ws = cv.take<char>(w.gemm_ws_bytes);
    w.x_perm = cv.take<char>((size_t)max_rows * p->d * es);
    const int64_t h_rows = p->has_shared && p->T > max_rows ? p->T : max_rows;
    w.h = cv.take<char>((size_t)h_rows * p->ffn * es);
    w.y_perm = cv.take<char>((size_t)max_rows * p->d * es);
    w.y_sh = p->has_shared ? cv.take<char>((size_t)p->T * p->d * es) : nullptr;
    const bool sep = overlap && p->has_shared;
    w.h_sh = sep ? cv.take<char>((size_t)p->T * p->ffn * es) : w.h;
    w.gemm_ws_sh = sep ? cv.take<char>(w.gemm_ws_bytes) : w.gemm_ws;
    w.bytes = cv.off;
    return w;
}

} // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(moe_status_t s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *moe_last_error(void) { return moe::g_err; }

int64_t moe_max_rows(int64_t T, int E, int k, float capacity_factor, int num_local_experts)
{
    if (T < 0 || E < 1 || k < 1 || num_local_experts < 0)
        return -1;
    const int E_loc = local_count(E, num_local_experts);
    int64_t rows = T * k;
    const int64_t C = capacity_of(T, E, capacity_factor);
    if (C >= 0 && (int64_t)E_loc * C < rows)
        rows = (int64_t)E_loc * C;
    return rows;
}

size_t moe_route_workspace_size(int64_t T, int d, int E)
{
    if (T < 0 || E < 1 || d < 1)
        return 0;
    return route_ws_bytes(T, d, E);
}

moe_status_t moe_route(const void *x, moe_dtype_t dtype, const float *w_router, const float *b_router,
                       const float *sel_bias, int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx,
                       float *topk_w, int32_t *expert_count, float *f, float *P, float *l_aux, void *ws,
                       size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_route_args(x, dtype, w_router, T, d, E, k, topk_idx, topk_w))
        return s;
    if (moe_status_t s = check_ws(ws, ws_bytes, route_ws_bytes(T, d, E), "route"))
        return s;
    return launch_route(x, dtype, w_router, b_router, sel_bias, T, d, E, k, alpha, topk_idx, topk_w, expert_count,
                        f, P, l_aux, ws, stream);
}

size_t moe_dispatch_workspace_size(int64_t T, int k, int num_local_experts)
{
    if (T < 0 || k < 1 || num_local_experts < 1)
        return 0;
    return dispatch_ws_bytes(T, k, num_local_experts);
}

moe_status_t moe_dispatch(const void *x, moe_dtype_t dtype, const int32_t *topk_idx, int64_t T, int d, int E, int k,
                          float capacity_factor, int expert_begin, int num_local_experts, int32_t *seg_offsets,
                          int32_t *kept_count, int32_t *slot_row, int32_t *row_src, void *x_perm, int64_t max_rows,
                          int32_t *n_dropped, void *ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_dispatch_args(x, dtype, topk_idx, T, d, E, k, capacity_factor, expert_begin,
                                             num_local_experts, seg_offsets, kept_count, slot_row, row_src, x_perm,
                                             max_rows))
        return s;
    const int E_loc = local_count(E, num_local_experts);
    if (moe_status_t s = check_ws(ws, ws_bytes, dispatch_ws_bytes(T, k, E_loc), "dispatch"))
        return s;
    return launch_dispatch(x, dtype, topk_idx, T, d, E, k, capacity_factor, expert_begin, E_loc, seg_offsets,
                           kept_count, slot_row, row_src, x_perm, max_rows, n_dropped, ws, stream);
}

size_t moe_grouped_gemm_workspace_size(void) { return gemm_ws_bytes(); }

moe_status_t moe_grouped_gemm(const void *a, const int32_t *seg_offsets, int num_segments, int64_t max_rows, int N,
                              int K, moe_dtype_t dtype, const void *w, const void *bias, int activation, void *out,
                              void *ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_gemm_args(a, seg_offsets, num_segments, max_rows, N, K, dtype, w, bias, activation,
                                         out, "grouped_gemm"))
        return s;
    if (!aligned16(ws))
        return fail(MOE_ERR_INVALID_ARG, "grouped_gemm: ws must be 16-byte aligned");
    return launch_grouped_gemm(a, seg_offsets, num_segments, max_rows, N, K, dtype, w, bias, activation, out, ws,
                               ws_bytes, stream);
}

moe_status_t moe_expert_ffn(const void *x_perm, const int32_t *seg_offsets, int num_segments, int64_t max_rows,
                            int d, int ffn, moe_dtype_t dtype, const void *w1, const void *b1, const void *w2,
                            const void *b2, void *h, void *y_perm, void *ws, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_gemm_args(x_perm, seg_offsets, num_segments, max_rows, ffn, d, dtype, w1, b1, 1, h,
                                         "expert_ffn (first Linear)"))
        return s;
    if (moe_status_t s = check_gemm_args(h, seg_offsets, num_segments, max_rows, d, ffn, dtype, w2, b2, 0, y_perm,
                                         "expert_ffn (second Linear)"))
        return s;
    if (!aligned16(ws))
        return fail(MOE_ERR_INVALID_ARG, "expert_ffn: ws must be 16-byte aligned");
    if (moe_status_t s = launch_grouped_gemm(x_perm, seg_offsets, num_segments, max_rows, ffn, d, dtype, w1, b1, 1,
                                             h, ws, ws_bytes, stream))
        return s;
    return launch_grouped_gemm(h, seg_offsets, num_segments, max_rows, d, ffn, dtype, w2, b2, 0, y_perm, ws, ws_bytes,
                               stream);
}

moe_status_t moe_combine(const void *y_perm, int64_t max_rows, const int32_t *slot_row, const float *topk_w,
                         const void *y_shared, int64_t T, int d, int k, moe_dtype_t dtype, void *y, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_combine_args(y_perm, max_rows, slot_row, topk_w, y_shared, T, d, k, dtype, y))
        return s;
    return launch_combine(y_perm, max_rows, slot_row, topk_w, y_shared, T, d, k, dtype, y, stream);
}

size_t moe_forward_workspace_size(const moe_problem_t *p)
{
    if (!p || p->T < 0 || p->E < 1 || p->k < 1 || p->d < 1 || p->ffn < 1 || p->num_local_experts < 0)
        return 0;
    return carve_forward(p, nullptr, nullptr).bytes;
}

} // extern "C"

namespace {

moe_status_t forward_impl(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                          const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t stream, hipStream_t side)
{
    clear_error();
    if (!p || !w)
        return fail(MOE_ERR_INVALID_ARG, "forward: problem and weights are required");
    if (p->T < 0 || p->d < 1 || p->ffn < 1 || p->E < 1 || p->k < 1)
        return fail(MOE_ERR_INVALID_ARG, "forward: invalid sizes");
    if (moe_status_t s = check_route_args(x, p->dtype, w->w_router, p->T, p->d, p->E, p->k, (const int32_t *)1,
                                          (const float *)1))
        return s;
    if (p->T > 0 && !y)
        return fail(MOE_ERR_INVALID_ARG, "forward: y is required");
    const int E_loc = local_count(p->E, p->num_local_experts);
    const int64_t max_rows = moe_max_rows(p->T, p->E, p->k, p->capacity_factor, p->num_local_experts);
    if (moe_status_t s = check_dispatch_args(x, p->dtype, (const int32_t *)1, p->T, p->d, p->E, p->k,
                                             p->capacity_factor, p->expert_begin, p->num_local_experts,
                                             (const int32_t *)1, (const int32_t *)1, (const int32_t *)1,
                                             (const int32_t *)1, nullptr, max_rows))
        return s;
    if (!w->w1 || !w->w2 || (p->has_shared && (!w->ws1 || !w->ws2)))
        return fail(MOE_ERR_INVALID_ARG, "forward: expert weights are required");
    if (moe_status_t s = check_gemm_args(x, nullptr, 1, max_rows, p->ffn, p->d, p->dtype, w->w1, w->b1, 1, y,
                                         "forward (first Linear)"))
        return s;
    if (moe_status_t s = check_gemm_args(x, nullptr, 1, max_rows, p->d, p->ffn, p->dtype, w->w2, w->b2, 0, y,
                                         "forward (second Linear)"))
        return s;
    if (p->has_shared &&
        (!aligned16(w->ws1) || !aligned16(w->ws2) || !aligned16(w->bs1) || !aligned16(w->bs2)))
        return fail(MOE_ERR_INVALID_ARG, "forward: shared expert buffers must be 16-byte aligned");
    if (!aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "forward: y must be 16-byte aligned");
    const bool overlap = side != nullptr && side != stream && p->has_shared && p->T > 0;
    const ForwardWs need = carve_forward(p, out, nullptr, side != nullptr);
    if (moe_status_t s = check_ws(ws, ws_bytes, need.bytes, "forward"))
        return s;
    const ForwardWs b = carve_forward(p, out, ws, side != nullptr);

    // The shared expert needs only x: on the side stream it runs while the
    // routed path routes, dispatches and runs its own GEMMs.
    hipEvent_t ev_start = nullptr, ev_done = nullptr;
    auto release = [&]() {
        if (ev_start)
            (void)hipEventDestroy(ev_start);
        if (ev_done)
            (void)hipEventDestroy(ev_done);
    };
    if (overlap) {
        if (hipEventCreateWithFlags(&ev_start, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&ev_done, hipEventDisableTiming) != hipSuccess) {
            release();
            return fail(MOE_ERR_HIP, "forward: cannot create events for the side stream");
        }
        if (hipEventRecord(ev_start, stream) != hipSuccess || hipStreamWaitEvent(side, ev_start, 0) != hipSuccess) {
            release();
            return fail(MOE_ERR_HIP, "forward: cannot order the side stream after the main stream");
        }
        moe_status_t s = launch_grouped_gemm(x, nullptr, 1, p->T, p->ffn, p->d, p->dtype, w->ws1, w->bs1, 1,
                                             b.h_sh, b.gemm_ws_sh, b.gemm_ws_bytes, side);
        if (!s)
            s = launch_grouped_gemm(b.h_sh, nullptr, 1, p->T, p->d, p->ffn, p->dtype, w->ws2, w->bs2, 0, b.y_sh,
                                    b.gemm_ws_sh, b.gemm_ws_bytes, side);
        if (!s && hipEventRecord(ev_done, side) != hipSuccess)
            s = fail(MOE_ERR_HIP, "forward: cannot record the side stream's completion");
        if (s) {
            release();
            return s;
        }
    }
    moe_status_t s = launch_route(x, p->dtype, w->w_router, w->b_router, w->sel_bias, p->T, p->d, p->E, p->k,
                                  p->alpha,
                                  b.topk_idx, b.topk_w, b.expert_count, b.f, b.P, b.l_aux, b.route_ws, stream);
    if (!s)
        s = launch_dispatch(x, p->dtype, b.topk_idx, p->T, p->d, p->E, p->k, p->capacity_factor, p->expert_begin,
                            E_loc, b.seg_offsets, b.kept_count, b.slot_row, b.row_src, b.x_perm, max_rows,
                            b.n_dropped, b.dispatch_ws, stream);
    if (!s && p->T > 0) {
        s = launch_grouped_gemm(b.x_perm, b.seg_offsets, E_loc, max_rows, p->ffn, p->d, p->dtype, w->w1, w->b1, 1,
                                b.h, b.gemm_ws, b.gemm_ws_bytes, stream);
        if (!s)
            s = launch_grouped_gemm(b.h, b.seg_offsets, E_loc, max_rows, p->d, p->ffn, p->dtype, w->w2, w->b2, 0,
                                    b.y_perm, b.gemm_ws, b.gemm_ws_bytes, stream);
        if (!s && p->has_shared && !overlap) {
            s = launch_grouped_gemm(x, nullptr, 1, p->T, p->ffn, p->d, p->dtype, w->ws1, w->bs1, 1, b.h, b.gemm_ws,
                                    b.gemm_ws_bytes, stream);
            if (!s)
                s = launch_grouped_gemm(b.h, nullptr, 1, p->T, p->d, p->ffn, p->dtype, w->ws2, w->bs2, 0, b.y_sh,
                                        b.gemm_ws, b.gemm_ws_bytes, stream);
        }
        if (!s && overlap && hipStreamWaitEvent(stream, ev_done, 0) != hipSuccess)
            s = fail(MOE_ERR_HIP, "forward: cannot order the combine after the side stream");
        if (!s)
            s = launch_combine(b.y_perm, max_rows, b.slot_row, b.topk_w, b.y_sh, p->T, p->d, p->k, p->dtype, y,
                               stream);
    }
    release();
    return s;
}

} // namespace

extern "C" moe_status_t moe_forward(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                                    const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return forward_impl(p, w, x, y, out, ws, ws_bytes, stream, nullptr);
}

extern "C" size_t moe_forward_overlap_workspace_size(const moe_problem_t *p)
{
    if (!p || p->T < 0 || p->E < 1 || p->k < 1 || p->d < 1 || p->ffn < 1 || p->num_local_experts < 0)
        return 0;
    return carve_forward(p, nullptr, nullptr, true).bytes;
}

extern "C" moe_status_t moe_forward_overlap(const moe_problem_t *p, const moe_weights_t *w, const void *x,
                                            void *y, const moe_outputs_t *out, void *ws, size_t ws_bytes,
                                            hipStream_t stream, hipStream_t side)
{
    return forward_impl(p, w, x, y, out, ws, ws_bytes, stream, side ? side : stream);
}
