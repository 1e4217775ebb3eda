// Public C ABI of the MoE layer library: argument validation, workspace
// sizing and carving, and the stream-ordered orchestration of the kernels.
// Every entry point validates before anything is enqueued.
#include "common.hpp"

#include <mutex>
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

// Largest reduction length and output width of a GEMM: the kernels address
// a 256-row operand or output tile through one buffer record of at most 2^31
// bytes (256 x K x 4, 256 x N x 4).
constexpr int kMaxK = 1 << 21;

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
    if (E > 1024 || k > 32 || d % 8 != 0 || d > kMaxK)
        return fail(MOE_ERR_UNSUPPORTED, "route: needs E <= 1024, k <= 32, d %% 8 == 0, d <= %d (E=%d k=%d d=%d)",
                    kMaxK, E, k, d);
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
    if (T > 0 && x_perm && !x)
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
    if (K > kMaxK || N > kMaxK)
        return fail(MOE_ERR_UNSUPPORTED, "%s: N = %d, K = %d, at most %d (a 256-row tile must fit a 32-bit buffer "
                    "record)", who, N, K, kMaxK);
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
    Carver cv{(char *)base, kCtrlBytes}; // [0, kCtrlBytes): the router's arrival counters
    ForwardWs w;
    w.topk_idx = out->topk_idx ? out->topk_idx : cv.take<int32_t>((size_t)Tk);
    w.topk_w = out->topk_w ? out->topk_w : cv.take<float>((size_t)Tk);
    w.expert_count = out->expert_count;
    w.f = out->f;
    w.P = out->P;
    w.l_aux = out->l_aux;
    w.route_ws = cv.take<char>(route_ws_bytes(p->T, p->d, p->E, p->dtype));
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

// Route workspaces: the arrival counters in the control bytes, then the
// statistics' partial and group rows (and, off the single-launch path, the
// logits).
static size_t route_ws_total(int64_t T, int d, int E, moe_dtype_t dt)
{
    return T > 0 ? kCtrlBytes + route_ws_bytes(T, d, E, dt) : 0;
}

size_t moe_route_workspace_size(int64_t T, int d, int E)
{
    if (T < 0 || E < 1 || d < 1)
        return 0;
    // the fp32-activation layout is the larger of the two
    const size_t a = route_ws_total(T, d, E, MOE_F32), b = route_ws_total(T, d, E, MOE_BF16);
    return a > b ? a : b;
}

moe_status_t moe_route(const void *x, moe_dtype_t dtype, const float *w_router, const float *b_router,
                       const float *sel_bias, int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx,
                       float *topk_w, int32_t *expert_count, float *f, float *P, float *l_aux, void *ws,
                       size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_route_args(x, dtype, w_router, T, d, E, k, topk_idx, topk_w))
        return s;
    if (moe_status_t s = check_ws(ws, ws_bytes, route_ws_total(T, d, E, dtype), "route"))
        return s;
    return launch_route(x, dtype, w_router, b_router, sel_bias, T, d, E, k, alpha, topk_idx, topk_w, expert_count,
                        f, P, l_aux, nullptr, T > 0 ? (char *)ws + kCtrlBytes : nullptr, (unsigned *)ws, stream);
}

size_t moe_dispatch_workspace_size(int64_t T, int k, int num_local_experts)
{
    if (T < 0 || k < 1 || num_local_experts < 1)
        return 0;
    return kCtrlBytes + dispatch_ws_bytes(T, k, num_local_experts);
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
    if (moe_status_t s = check_ws(ws, ws_bytes, kCtrlBytes + dispatch_ws_bytes(T, k, E_loc), "dispatch"))
        return s;
    return launch_dispatch(x, dtype, topk_idx, T, d, E, k, capacity_factor, expert_begin, E_loc, seg_offsets,
                           kept_count, slot_row, row_src, x_perm, max_rows, n_dropped, (char *)ws + kCtrlBytes,
                           stream);
}

} // extern "C"

// ------------------------------------------------ dispatch without allocation
// moe_dispatch_noalloc keeps its scratch (the per-chunk expert counts of the
// dispatch planner) in this file-scope device array instead of a caller
// workspace.  Each device holds its own copy for the life of the process; its
// address on the current device is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels (the array's
// name is a host-side stand-in in host code).
namespace {

constexpr size_t kStaticScratchBytes = 64 * 1024;
constexpr int kMaxDevices = 64;

__device__ __attribute__((used)) __align__(256) int32_t scratch[kStaticScratchBytes / sizeof(int32_t)];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

moe_status_t static_scratch(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_HIP, "dispatch_noalloc: no usable current device (%d)", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_HIP, "dispatch_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

} // namespace

extern "C" {

size_t moe_dispatch_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

moe_status_t moe_dispatch_noalloc(const void *x, moe_dtype_t dtype, const int32_t *topk_idx, int64_t T, int d, int E,
                                  int k, float capacity_factor, int expert_begin, int num_local_experts,
                                  int32_t *seg_offsets, int32_t *kept_count, int32_t *slot_row, int32_t *row_src,
                                  void *x_perm, int64_t max_rows, int32_t *n_dropped, hipStream_t stream)
{
    clear_error();
    if (moe_status_t s = check_dispatch_args(x, dtype, topk_idx, T, d, E, k, capacity_factor, expert_begin,
                                             num_local_experts, seg_offsets, kept_count, slot_row, row_src, x_perm,
                                             max_rows))
        return s;
    const int E_loc = local_count(E, num_local_experts);
    const size_t need = dispatch_ws_bytes(T, k, E_loc);
    if (need > kStaticScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED, "dispatch_noalloc: needs %zu bytes of scratch, the static buffer holds %zu",
                    need, kStaticScratchBytes);
    void *ws = nullptr;
    if (moe_status_t s = static_scratch(&ws))
        return s;
    return launch_dispatch(x, dtype, topk_idx, T, d, E, k, capacity_factor, expert_begin, E_loc, seg_offsets,
                           kept_count, slot_row, row_src, x_perm, max_rows, n_dropped, ws, stream);
}

size_t moe_grouped_gemm_workspace_size(void) { return kCtrlBytes + gemm_ws_bytes(); }

// The split-K partials of an optional GEMM workspace (after its control bytes).
static void *gemm_part(void *ws, size_t ws_bytes, size_t *part_bytes)
{
    if (!ws || ws_bytes < kCtrlBytes + gemm_ws_bytes()) {
        *part_bytes = 0;
        return nullptr;
    }
    *part_bytes = ws_bytes - kCtrlBytes;
    return (char *)ws + kCtrlBytes;
}

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
    size_t pb = 0;
    void *part = gemm_part(ws, ws_bytes, &pb);
    return launch_grouped_gemm(a, seg_offsets, num_segments, max_rows, N, K, dtype, w, bias, activation, out, part, pb,
                               stream);
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
    size_t pb = 0;
    void *part = gemm_part(ws, ws_bytes, &pb);
    if (moe_status_t s = launch_grouped_gemm(x_perm, seg_offsets, num_segments, max_rows, ffn, d, dtype, w1, b1, 1,
                                             h, part, pb, stream))
        return s;
    return launch_grouped_gemm(h, seg_offsets, num_segments, max_rows, d, ffn, dtype, w2, b2, 0, y_perm, part, pb,
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

// u_save / u_sh_save (moe_forward_save): the first Linear's fp32
// pre-activations of the routed rows and of the shared expert are written
// there, and GELU runs as its own pass from them.
moe_status_t forward_impl(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                          const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t stream, hipStream_t side,
                          float *u_save = nullptr, float *u_sh_save = nullptr, hipEvent_t ev_fork = nullptr,
                          hipEvent_t ev_join = nullptr)
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
    if (overlap && (!ev_fork || !ev_join))
        return fail(MOE_ERR_INVALID_ARG, "forward_overlap: the fork and join events are required");
    const ForwardWs need = carve_forward(p, out, nullptr, side != nullptr);
    if (moe_status_t s = check_ws(ws, ws_bytes, need.bytes, "forward"))
        return s;
    const ForwardWs b = carve_forward(p, out, ws, side != nullptr);

    // The shared expert needs only x: on the side stream it runs while the
    // routed path routes, dispatches and runs its own GEMMs.  Once anything
    // is on the side stream, every return path joins it back into `stream`,
    // so that no side work is left running past the call's stream order.
    bool forked = false;
    auto join = [&](moe_status_t s) -> moe_status_t {
        if (!forked)
            return s;
        if (hipEventRecord(ev_join, side) != hipSuccess || hipStreamWaitEvent(stream, ev_join, 0) != hipSuccess) {
            if (!s)
                s = fail(MOE_ERR_HIP, "forward_overlap: cannot join the side stream");
        }
        forked = false;
        return s;
    };
    if (overlap) {
        if (hipEventRecord(ev_fork, stream) != hipSuccess || hipStreamWaitEvent(side, ev_fork, 0) != hipSuccess)
            return fail(MOE_ERR_HIP, "forward_overlap: cannot order the side stream after the main stream");
        forked = true;
        moe_status_t s = launch_grouped_gemm(x, nullptr, 1, p->T, p->ffn, p->d, p->dtype, w->ws1, w->bs1, 1,
                                             b.h_sh, b.gemm_ws_sh, b.gemm_ws_bytes, side);
        if (!s)
            s = launch_grouped_gemm(b.h_sh, nullptr, 1, p->T, p->d, p->ffn, p->dtype, w->ws2, w->bs2, 0, b.y_sh,
                                    b.gemm_ws_sh, b.gemm_ws_bytes, side);
        if (s)
            return join(s);
    }
    moe_status_t s = launch_route(x, p->dtype, w->w_router, w->b_router, w->sel_bias, p->T, p->d, p->E, p->k,
                                  p->alpha,
                                  b.topk_idx, b.topk_w, b.expert_count, b.f, b.P, b.l_aux, nullptr, b.route_ws,
                                  (unsigned *)ws, stream);
    if (!s)
        s = launch_dispatch(x, p->dtype, b.topk_idx, p->T, p->d, p->E, p->k, p->capacity_factor, p->expert_begin,
                            E_loc, b.seg_offsets, b.kept_count, b.slot_row, b.row_src, b.x_perm, max_rows,
                            b.n_dropped, b.dispatch_ws, stream);
    if (!s && p->T > 0) {
        if (u_save) {
            s = launch_grouped_gemm_f32out(b.x_perm, b.seg_offsets, E_loc, max_rows, p->ffn, p->d, p->dtype, w->w1,
                                           w->b1, u_save, b.gemm_ws, b.gemm_ws_bytes, stream);
            if (!s)
                s = launch_gelu_rows(u_save, b.seg_offsets, E_loc, max_rows, p->ffn, p->dtype, b.h, stream);
        } else {
            s = launch_grouped_gemm(b.x_perm, b.seg_offsets, E_loc, max_rows, p->ffn, p->d, p->dtype, w->w1, w->b1,
                                    1, b.h, b.gemm_ws, b.gemm_ws_bytes, stream);
        }
        if (!s)
            s = launch_grouped_gemm(b.h, b.seg_offsets, E_loc, max_rows, p->d, p->ffn, p->dtype, w->w2, w->b2, 0,
                                    b.y_perm, b.gemm_ws, b.gemm_ws_bytes, stream);
        if (!s && p->has_shared && !overlap) {
            if (u_sh_save) {
                s = launch_grouped_gemm_f32out(x, nullptr, 1, p->T, p->ffn, p->d, p->dtype, w->ws1, w->bs1, u_sh_save,
                                               b.gemm_ws, b.gemm_ws_bytes, stream);
                if (!s)
                    s = launch_gelu_rows(u_sh_save, nullptr, 1, p->T, p->ffn, p->dtype, b.h, stream);
            } else {
                s = launch_grouped_gemm(x, nullptr, 1, p->T, p->ffn, p->d, p->dtype, w->ws1, w->bs1, 1, b.h,
                                        b.gemm_ws, b.gemm_ws_bytes, stream);
            }
            if (!s)
                s = launch_grouped_gemm(b.h, nullptr, 1, p->T, p->d, p->ffn, p->dtype, w->ws2, w->bs2, 0, b.y_sh,
                                        b.gemm_ws, b.gemm_ws_bytes, stream);
        }
        if (!s && overlap)
            s = join(s); // the combine reads the shared expert's output
        if (!s)
            s = launch_combine(b.y_perm, max_rows, b.slot_row, b.topk_w, b.y_sh, p->T, p->d, p->k, p->dtype, y,
                               stream);
    }
    return join(s);
}

} // namespace

extern "C" moe_status_t moe_forward(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                                    const moe_outputs_t *out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return forward_impl(p, w, x, y, out, ws, ws_bytes, stream, nullptr);
}

extern "C" moe_status_t moe_forward_save(const moe_problem_t *p, const moe_weights_t *w, const void *x, void *y,
                                         const moe_outputs_t *out, float *u_saved, float *u_shared_saved, void *ws,
                                         size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "forward_save: problem is required");
    if (p->T > 0 && (!u_saved || (p->has_shared && !u_shared_saved)))
        return fail(MOE_ERR_INVALID_ARG, "forward_save: u_saved (and u_shared_saved with a shared expert) required");
    if (!aligned16(u_saved) || !aligned16(u_shared_saved))
        return fail(MOE_ERR_INVALID_ARG, "forward_save: u_saved and u_shared_saved must be 16-byte aligned");
    // the fp32-output first Linear runs on the 256x256 kernel only
    if (p->dtype == MOE_BF16 && (p->d % 64 != 0 || p->d < 128))
        return fail(MOE_ERR_UNSUPPORTED, "forward_save: bf16 needs d a multiple of 64, at least 128 (d=%d)", p->d);
    return forward_impl(p, w, x, y, out, ws, ws_bytes, stream, nullptr, u_saved, p->has_shared ? u_shared_saved : nullptr);
}

extern "C" size_t moe_forward_overlap_workspace_size(const moe_problem_t *p)
{
    if (!p || p->T < 0 || p->E < 1 || p->k < 1 || p->d < 1 || p->ffn < 1 || p->num_local_experts < 0)
        return 0;
    return carve_forward(p, nullptr, nullptr, true).bytes;
}

extern "C" moe_status_t moe_forward_overlap(const moe_problem_t *p, const moe_weights_t *w, const void *x,
                                            void *y, const moe_outputs_t *out, void *ws, size_t ws_bytes,
                                            hipStream_t stream, hipStream_t side, hipEvent_t fork, hipEvent_t join)
{
    return forward_impl(p, w, x, y, out, ws, ws_bytes, stream, side ? side : stream, nullptr, nullptr, fork, join);
}

// ------------------------------------------------------------------ backward
namespace {

// Workspace of moe_backward.  The shared expert runs first and writes its dx
// straight into the caller's dx; the routed experts then reuse its buffers
// (rows = max(routed rows, T); transposed weights, fp32 layers only, for
// max(E_loc, 1) experts).
struct BackwardWs {
    int32_t *topk_idx, *expert_count, *seg_offsets, *kept_count, *slot_row, *row_src, *kcol;
    float *topk_w, *f, *P, *l_aux, *probs, *dl;
    void *route_ws, *dispatch_ws, *gemm_ws, *router_ws;
    size_t gemm_ws_bytes;
    void *x_perm, *dyp, *du, *w1t, *w2t, *xT, *dyT, *duT, *gwT, *gw;
    float *u, *dh, *dx_rows, *dwpart, *colpart, *bias_part;
    int64_t Kp;
    size_t bytes;
};

// The router backward runs on the matrix cores for bf16 layers with many
// experts (its fp32 vector form costs 2 T E d FMAs twice).
bool router_on_mfma(const moe_problem_t *p)
{
    return p->dtype == MOE_BF16 && p->E >= 32 && p->E % 8 == 0 && p->d % 64 == 0;
}

// bf16 weight-gradient GEMMs on the row-major dispatched rows (no
// transposed copies), when their sizes allow.  A segment holds at most T
// rows: an expert takes each token at most once, the shared expert all T.
bool wgrad_on_rows(const moe_problem_t *p)
{
    return p->dtype == MOE_BF16 && kseg_kmajor_ok(p->T, p->d, p->ffn);
}

BackwardWs carve_backward(const moe_problem_t *p, const moe_grads_t *g, void *base)
{
    const int E_loc = local_count(p->E, p->num_local_experts);
    const int64_t max_rows = moe_max_rows(p->T, p->E, p->k, p->capacity_factor, p->num_local_experts);
    const int64_t rows = p->has_shared && p->T > max_rows ? p->T : max_rows;
    const size_t es = elem_size(p->dtype);
    const int64_t Tk = p->T * p->k;
    const int64_t kp_r = kseg_cols_bound(max_rows, E_loc), kp_s = p->has_shared ? kseg_cols_bound(p->T, 1) : 0;
    Carver cv{(char *)base, kCtrlBytes}; // [0, kCtrlBytes): the router's arrival counters
    BackwardWs w;
    w.Kp = kp_r > kp_s ? kp_r : kp_s;
    w.topk_idx = cv.take<int32_t>((size_t)Tk);
    w.topk_w = cv.take<float>((size_t)Tk);
    w.expert_count = cv.take<int32_t>((size_t)p->E);
    w.f = cv.take<float>((size_t)p->E);
    w.P = cv.take<float>((size_t)p->E);
    w.l_aux = cv.take<float>(1);
    w.probs = cv.take<float>((size_t)p->T * p->E);
    w.dl = (g && g->dlogits) ? g->dlogits : cv.take<float>((size_t)p->T * p->E);
    w.route_ws = cv.take<char>(route_ws_bytes(p->T, p->d, p->E, p->dtype));
    w.seg_offsets = cv.take<int32_t>((size_t)E_loc + 1);
    w.kept_count = cv.take<int32_t>((size_t)E_loc);
    w.slot_row = cv.take<int32_t>((size_t)Tk);
    w.row_src = cv.take<int32_t>((size_t)max_rows);
    w.kcol = cv.take<int32_t>((size_t)E_loc + 1);
    w.dispatch_ws = cv.take<char>(dispatch_ws_bytes(p->T, p->k, E_loc));
    w.gemm_ws_bytes = p->dtype == MOE_BF16 ? gemm_ws_bytes() : 0;
    w.gemm_ws = cv.take<char>(w.gemm_ws_bytes);
    {
        const size_t a = router_wgrad_ws_bytes(p->T, p->d, p->E);
        const size_t m = router_on_mfma(p) ? router_mfma_ws_bytes(p->T, p->d, p->E) : 0;
        w.router_ws = cv.take<char>(a > m ? a : m);
    }
    w.x_perm = cv.take<char>((size_t)max_rows * p->d * es);
    w.dyp = cv.take<char>((size_t)max_rows * p->d * es);
    w.du = cv.take<char>((size_t)rows * p->ffn * es);
    // transposed weights only for fp32 (bf16 GEMMs read W1, W2 K-major as stored)
    const size_t wt_bytes = p->dtype == MOE_BF16 ? 0 : (size_t)E_loc * p->ffn * p->d * es;
    w.w1t = cv.take<char>(wt_bytes);
    w.w2t = cv.take<char>(wt_bytes);
    // transposed operands of the weight-gradient GEMMs, or (on rows) gw rows
    const bool on_rows = wgrad_on_rows(p);
    w.xT = cv.take<char>(on_rows ? 0 : (size_t)p->d * w.Kp * es);
    w.dyT = cv.take<char>(on_rows ? 0 : (size_t)p->d * w.Kp * es);
    w.duT = cv.take<char>(on_rows ? 0 : (size_t)p->ffn * w.Kp * es);
    w.gwT = cv.take<char>(on_rows ? 0 : (size_t)p->ffn * w.Kp * es);
    w.gw = cv.take<char>(on_rows ? (size_t)rows * p->ffn * es : 0);
    w.u = cv.take<float>((size_t)rows * p->ffn);
    w.dh = cv.take<float>((size_t)rows * p->ffn);
    w.dx_rows = cv.take<float>((size_t)rows * p->d);
    w.dwpart = cv.take<float>((size_t)max_rows * ((p->ffn + 63) / 64));
    const int64_t maxdim = p->d > p->ffn ? p->d : p->ffn;
    w.colpart = cv.take<float>((size_t)(w.Kp / 64) * maxdim);
    w.bias_part = cv.take<float>(router_bias_ws_bytes(p->E) / sizeof(float));
    w.bytes = cv.off;
    return w;
}

// One FFN's backward (the routed experts over their dispatched rows, or the
// shared expert over all tokens with seg = row_src = wgt = NULL).
struct FfnBwd {
    const void *a_rows;            // rows of the first Linear's input: x_perm, or x
    const void *dy_rows;           // NULL: gather dy rows into b.dyp
    const int32_t *seg, *row_src;
    int S;
    int64_t rows;
    const float *wgt;              // routing weights by slot, or NULL (= 1)
    const void *w1, *b1, *w2;
    float *dw1, *db1, *dw2, *db2, *dx_rows, *dwpart;
    const float *u_saved;          // the forward's pre-activations, or NULL (recomputed)
};

moe_status_t ffn_backward(const moe_problem_t *p, const void *x, const void *dy, const FfnBwd &a,
                          const BackwardWs &b, hipStream_t st)
{
    const moe_dtype_t dt = p->dtype;
    const int d = p->d, F = p->ffn;
    // bf16: the GEMMs against W2 and W1 read them K-major as stored; fp32:
    // explicit transposes W1^T [S, d, F], W2^T [S, F, d]
    const bool kmajor = dt == MOE_BF16;
    // bf16 (sizes allowing): dW1 and dW2 from the row-major rows of x, dY, du
    // and gw; otherwise from transposed copies [D, Kp]
    const bool on_rows = wgrad_on_rows(p);
    moe_status_t s = launch_kseg_layout(a.seg, a.S, a.rows, b.kcol, st);
    if (!s && !kmajor)
        s = launch_transpose_batched(a.w1, a.S, F, d, a.seg, dt, b.w1t, st);
    if (!s && !kmajor)
        s = launch_transpose_batched(a.w2, a.S, d, F, a.seg, dt, b.w2t, st);
    const float *u = a.u_saved ? a.u_saved : b.u;
    if (!s && !a.u_saved) // u = W1 x + b1 (fp32)
        s = launch_grouped_gemm_f32out(a.a_rows, a.seg, a.S, a.rows, F, d, dt, a.w1, a.b1, b.u, b.gemm_ws,
                                       b.gemm_ws_bytes, st);
    // dY rows (row-major for dh'; transposed for dW2 unless on rows) and db2;
    // nothing to do for given dY rows on rows without db2
    if (!s && !(on_rows && a.dy_rows && !a.db2))
        s = launch_gather_t(dy, d, a.row_src, p->k, a.wgt, a.seg, a.S, a.rows, b.kcol, b.Kp, dt,
                            on_rows ? nullptr : b.dyT, a.dy_rows ? nullptr : b.dyp, a.db2 ? b.colpart : nullptr, st);
    if (!s)
        s = launch_seg_colsum(b.colpart, b.kcol, a.S, d, a.db2, st);
    const void *dyr = a.dy_rows ? a.dy_rows : b.dyp;
    if (!s) // dh' = W2^T dY
        s = kmajor ? launch_grouped_gemm_kmajor_f32out(dyr, a.seg, a.S, a.rows, F, d, a.w2, b.dh, b.gemm_ws,
                                                       b.gemm_ws_bytes, st)
                   : launch_grouped_gemm_f32out(dyr, a.seg, a.S, a.rows, F, d, dt, b.w2t, nullptr, b.dh, b.gemm_ws,
                                                b.gemm_ws_bytes, st);
    if (!s)
        s = launch_act_bwd(u, b.dh, F, a.row_src, a.wgt, a.seg, a.S, a.rows, b.kcol, b.Kp, dt, b.du,
                           on_rows ? nullptr : b.duT, on_rows ? nullptr : b.gwT, on_rows ? b.gw : nullptr, a.dwpart,
                           a.db1 ? b.colpart : nullptr, st);
    if (!s)
        s = launch_seg_colsum(b.colpart, b.kcol, a.S, F, a.db1, st);
    if (!s) // dx rows = W1^T du
        s = kmajor ? launch_grouped_gemm_kmajor_f32out(b.du, a.seg, a.S, a.rows, d, F, a.w1, a.dx_rows, b.gemm_ws,
                                                       b.gemm_ws_bytes, st)
                   : launch_grouped_gemm_f32out(b.du, a.seg, a.S, a.rows, d, F, dt, b.w1t, nullptr, a.dx_rows,
                                                b.gemm_ws, b.gemm_ws_bytes, st);
    if (on_rows) {
        if (!s) // dW2_s = sum_r dY (w g)^T : [d, F]
            s = launch_kseg_gemm_kmajor(dyr, b.gw, a.seg, a.rows, p->T, b.kcol, a.S, d, F, a.dw2, st);
        if (!s) // dW1_s = sum_r du x^T : [F, d]
            s = launch_kseg_gemm_kmajor(b.du, a.a_rows, a.seg, a.rows, p->T, b.kcol, a.S, F, d, a.dw1, st);
        return s;
    }
    if (!s) // x rows, transposed, for dW1
        s = launch_gather_t(x, d, a.row_src, p->k, nullptr, a.seg, a.S, a.rows, b.kcol, b.Kp, dt, b.xT, nullptr,
                            nullptr, st);
    if (!s) // dW2_s = sum_r dY (w g)^T : [d, F]
        s = launch_kseg_gemm(b.dyT, b.gwT, b.kcol, a.S, d, F, b.Kp, dt, a.dw2, st);
    if (!s) // dW1_s = sum_r du x^T : [F, d]
        s = launch_kseg_gemm(b.duT, b.xT, b.kcol, a.S, F, d, b.Kp, dt, a.dw1, st);
    return s;
}

} // namespace

extern "C" size_t moe_backward_workspace_size(const moe_problem_t *p)
{
    if (!p || p->T < 0 || p->E < 1 || p->k < 1 || p->d < 1 || p->ffn < 1 || p->num_local_experts < 0)
        return 0;
    return carve_backward(p, nullptr, nullptr).bytes;
}

namespace {

// moe_backward; with u_saved (and u_sh_saved) the first Linear's
// pre-activations come from moe_forward_save instead of being recomputed.
moe_status_t backward_impl(const moe_problem_t *p, const moe_weights_t *w, const void *x, const void *dy,
                           float g_aux, const moe_grads_t *g, void *ws, size_t ws_bytes, hipStream_t stream,
                           const float *u_saved, const float *u_sh_saved)
{
    clear_error();
    if (!p || !w || !g)
        return fail(MOE_ERR_INVALID_ARG, "backward: problem, weights and grads are required");
    if (p->T < 0 || p->d < 1 || p->ffn < 1 || p->E < 1 || p->k < 1)
        return fail(MOE_ERR_INVALID_ARG, "backward: invalid sizes");
    if (!(g_aux == g_aux))
        return fail(MOE_ERR_INVALID_ARG, "backward: g_aux is NaN");
    if (moe_status_t s = check_route_args(x, p->dtype, w->w_router, p->T, p->d, p->E, p->k, (const int32_t *)1,
                                          (const float *)1))
        return s;
    const int E_loc = local_count(p->E, p->num_local_experts);
    const int64_t max_rows = moe_max_rows(p->T, p->E, p->k, p->capacity_factor, p->num_local_experts);
    if (moe_status_t s = check_dispatch_args(x, p->dtype, (const int32_t *)1, p->T, p->d, p->E, p->k,
                                             p->capacity_factor, p->expert_begin, p->num_local_experts,
                                             (const int32_t *)1, (const int32_t *)1, (const int32_t *)1,
                                             (const int32_t *)1, nullptr, max_rows))
        return s;
    if (!w->w1 || !w->w2 || (p->has_shared && (!w->ws1 || !w->ws2)))
        return fail(MOE_ERR_INVALID_ARG, "backward: expert weights are required");
    if ((p->T > 0 && !g->dx) || !g->dw_router || !g->dw1 || !g->dw2 || (p->has_shared && (!g->dws1 || !g->dws2)))
        return fail(MOE_ERR_INVALID_ARG, "backward: dx, dw_router, dw1, dw2 (and dws1, dws2) are required");
    if (p->T > 0 && !dy)
        return fail(MOE_ERR_INVALID_ARG, "backward: dy is required");
    {
        const void *gp[] = {g->dx, g->dw_router, g->db_router, g->dw1, g->db1, g->dw2, g->db2,
                            g->dws1, g->dbs1, g->dws2, g->dbs2, g->dlogits};
        for (const void *q : gp)
            if (!aligned16(q))
                return fail(MOE_ERR_INVALID_ARG, "backward: gradient buffers must be 16-byte aligned");
    }
    if (moe_status_t s = check_gemm_args(x, nullptr, 1, max_rows, p->ffn, p->d, p->dtype, w->w1, w->b1, 1, g->dx,
                                         "backward (first Linear)"))
        return s;
    if (moe_status_t s = check_gemm_args(x, nullptr, 1, max_rows, p->d, p->ffn, p->dtype, w->w2, w->b2, 0, g->dx,
                                         "backward (second Linear)"))
        return s;
    if (!aligned16(dy) || (p->has_shared && (!aligned16(w->ws1) || !aligned16(w->ws2) || !aligned16(w->bs1))))
        return fail(MOE_ERR_INVALID_ARG, "backward: dy and the shared expert buffers must be 16-byte aligned");
    if (p->dtype == MOE_BF16 && (p->d % 64 != 0 || p->ffn % 64 != 0 || p->d < 128 || p->ffn < 128))
        return fail(MOE_ERR_UNSUPPORTED, "backward: bf16 needs d and ffn multiples of 64, at least 128 (d=%d ffn=%d)",
                    p->d, p->ffn);
    const BackwardWs need = carve_backward(p, g, nullptr);
    if (need.Kp > kMaxK)
        return fail(MOE_ERR_UNSUPPORTED, "backward: %lld columns in the weight-gradient GEMMs, above %d",
                    (long long)need.Kp, kMaxK);
    if (moe_status_t s = check_ws(ws, ws_bytes, need.bytes, "backward"))
        return s;
    const BackwardWs b = carve_backward(p, g, ws);
    const int64_t T = p->T;
    const int d = p->d, F = p->ffn, E = p->E;

    moe_status_t s = launch_route(x, p->dtype, w->w_router, w->b_router, w->sel_bias, T, d, E, p->k, p->alpha,
                                  b.topk_idx, b.topk_w, b.expert_count, b.f, b.P, b.l_aux, b.probs, b.route_ws,
                                  (unsigned *)ws, stream);
    if (!s)
        s = launch_dispatch(x, p->dtype, b.topk_idx, T, d, E, p->k, p->capacity_factor, p->expert_begin, E_loc,
                            b.seg_offsets, b.kept_count, b.slot_row, b.row_src, b.x_perm, max_rows, nullptr,
                            b.dispatch_ws, stream);
    if (s)
        return s;
    if (T == 0) {
        // no tokens: every weight gradient is zero
        float *z[] = {g->dw_router, g->db_router, g->dw1, g->db1, g->dw2, g->db2, g->dws1, g->dbs1, g->dws2, g->dbs2};
        const int64_t n[] = {(int64_t)E * d, E, (int64_t)E_loc * F * d, (int64_t)E_loc * F, (int64_t)E_loc * d * F,
                             (int64_t)E_loc * d, p->has_shared ? (int64_t)F * d : 0, p->has_shared ? F : 0,
                             p->has_shared ? (int64_t)d * F : 0, p->has_shared ? d : 0};
        for (int i = 0; i < 10 && !s; ++i)
            s = launch_fill_zero(z[i], n[i], stream);
        return s;
    }
    if (p->has_shared) {
        FfnBwd a = {};
        a.a_rows = x;
        a.dy_rows = dy;
        a.S = 1;
        a.rows = T;
        a.w1 = w->ws1;
        a.b1 = w->bs1;
        a.w2 = w->ws2;
        a.dw1 = g->dws1;
        a.db1 = g->dbs1;
        a.dw2 = g->dws2;
        a.db2 = g->dbs2;
        a.dx_rows = g->dx; // the routed rows and the router term are added in place
        a.u_saved = u_sh_saved;
        s = ffn_backward(p, x, dy, a, b, stream);
    }
    if (!s) {
        FfnBwd a = {};
        a.a_rows = b.x_perm;
        a.seg = b.seg_offsets;
        a.row_src = b.row_src;
        a.S = E_loc;
        a.rows = max_rows;
        a.wgt = b.topk_w;
        a.w1 = w->w1;
        a.b1 = w->b1;
        a.w2 = w->w2;
        a.dw1 = g->dw1;
        a.db1 = g->db1;
        a.dw2 = g->dw2;
        a.db2 = g->db2;
        a.dx_rows = b.dx_rows;
        a.dwpart = b.dwpart;
        a.u_saved = u_saved;
        s = ffn_backward(p, x, dy, a, b, stream);
    }
    const float c_aux = (float)((double)g_aux * (double)p->alpha / (double)T);
    float *dx_r = nullptr;
    if (!s && router_on_mfma(p)) {
        s = launch_router_bwd_mfma(b.probs, b.topk_idx, b.slot_row, b.dwpart, (F + 63) / 64, w->b2, dy, d,
                                   p->expert_begin, b.f, c_aux, T, E, p->k, x, w->w_router, b.dl, g->dw_router,
                                   g->db_router, b.bias_part, &dx_r, b.router_ws, b.gemm_ws, b.gemm_ws_bytes,
                                   stream);
    } else if (!s) {
        s = launch_router_bwd(b.probs, b.topk_idx, b.slot_row, b.dwpart, (F + 63) / 64, w->b2, dy, p->dtype, d,
                              p->expert_begin, b.f, c_aux, T, E, p->k, b.dl, stream);
        if (!s)
            s = launch_router_wgrad(x, p->dtype, b.dl, T, d, E, g->dw_router, g->db_router, b.bias_part,
                                    b.router_ws, stream);
    }
    if (!s)
        s = launch_dx_combine(b.dx_rows, b.slot_row, p->k, p->has_shared ? g->dx : nullptr, dx_r, b.dl,
                              w->w_router, T, d, E, g->dx, stream);
    return s;
}

} // namespace

extern "C" moe_status_t moe_backward(const moe_problem_t *p, const moe_weights_t *w, const void *x, const void *dy,
                                     float g_aux, const moe_grads_t *g, void *ws, size_t ws_bytes,
                                     hipStream_t stream)
{
    return backward_impl(p, w, x, dy, g_aux, g, ws, ws_bytes, stream, nullptr, nullptr);
}

extern "C" moe_status_t moe_backward_saved(const moe_problem_t *p, const moe_weights_t *w, const void *x,
                                           const void *dy, float g_aux, const float *u_saved,
                                           const float *u_shared_saved, const moe_grads_t *g, void *ws,
                                           size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "backward_saved: problem is required");
    if (p->T > 0 && (!u_saved || (p->has_shared && !u_shared_saved)))
        return fail(MOE_ERR_INVALID_ARG, "backward_saved: u_saved (and u_shared_saved with a shared expert) required");
    if (!aligned16(u_saved) || !aligned16(u_shared_saved))
        return fail(MOE_ERR_INVALID_ARG, "backward_saved: u_saved and u_shared_saved must be 16-byte aligned");
    return backward_impl(p, w, x, dy, g_aux, g, ws, ws_bytes, stream, p->T > 0 ? u_saved : nullptr,
                         p->T > 0 && p->has_shared ? u_shared_saved : nullptr);
}
