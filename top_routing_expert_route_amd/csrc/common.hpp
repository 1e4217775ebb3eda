// Shared device helpers, error state and internal launcher declarations of
// the MoE layer library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe.h"

#define MOE_ABI_VERSION 3

namespace moe {

// ---------------------------------------------------------------- errors --
moe_status_t fail(moe_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// hipGetLastError after a launch; MOE_ERR_HIP with the kernel's name on failure.
moe_status_t check_launch(const char *what);

// --------------------------------------------------------------- bfloat16 --
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// GELU in its erf form, 0.5 u (1 + erf(u / sqrt 2)).  erf comes from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (|error| <= 1.5e-7 for x >= 0):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x),
// with erf(-x) = -erf(x).  With q = erfc(|u| / sqrt 2) / 2 this gives
// GELU(u) = u - u q for u >= 0 and u q for u < 0, i.e. max(u, 0) - |u| q
// (one fused multiply-add after the max: the same rounding as either branch).
// The factor 1/2 of q is folded into the coefficients: halving every
// coefficient halves each step of the Horner chain exactly (a power-of-two
// scale commutes with rounding), so q comes out bitwise as before with one
// multiply less.
constexpr float kGeluP = 0.3275911f;
constexpr float kGeluA1 = 0.254829592f * 0.5f, kGeluA2 = -0.284496736f * 0.5f, kGeluA3 = 1.421413741f * 0.5f,
                kGeluA4 = -1.453152027f * 0.5f, kGeluA5 = 1.061405429f * 0.5f;

// max(u, 0) as one instruction (the generic maximum first quiets the input,
// a second instruction the compiler cannot drop for a value of unknown origin).
__device__ __forceinline__ float relu_f32(float u)
{
    float r;
    asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(u));
    return r;
}

// q = erfc(|u| / sqrt 2) / 2 and e = exp(-u^2 / 2)
__device__ __forceinline__ float gelu_q(float u, float &e)
{
    const float x = fabsf(u) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(kGeluP, x, 1.0f));
    float poly = fmaf(kGeluA5, t, kGeluA4);
    poly = fmaf(poly, t, kGeluA3);
    poly = fmaf(poly, t, kGeluA2);
    poly = fmaf(poly, t, kGeluA1);
    poly *= t;
    e = __expf(-x * x);
    return poly * e;
}

__device__ __forceinline__ float gelu_erf(float u)
{
    float e;
    const float q = gelu_q(u, e);
    return fmaf(-fabsf(u), q, relu_f32(u));
}

// GELU and its derivative together: with Phi the standard normal CDF and phi
// its density, GELU(u) = u Phi(u) and GELU'(u) = Phi(u) + u phi(u).  Phi
// comes from the same erf approximation as gelu_erf (bitwise the same
// GELU), phi(u) = exp(-u^2 / 2) / sqrt(2 pi) shares its exponential.
__device__ __forceinline__ void gelu_and_grad(float u, float &g, float &gp)
{
    float e;
    const float q = gelu_q(u, e); // Phi(-|u|)
    g = fmaf(-fabsf(u), q, relu_f32(u));
    const float Phi = u >= 0.f ? 1.0f - q : q;
    gp = fmaf(u, e * 0.39894228040143268f, Phi);
}

// Wave reductions without the LDS crossbar: DPP moves within rows of 16
// lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror: after the first three steps every lane holds its group of 8
// lanes' result, after the fourth its row of 16), then the four row results
// are read into scalars and combined in a fixed order.  Every lane must be
// active.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float group8_sum(float v)
{
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    return v;
}

__device__ __forceinline__ float row16_sum(float v)
{
    v = group8_sum(v);
    v += dpp_mov<0x140>(v);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = group8_sum(v);
    v += dpp_mov<0x140>(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// ------------------------------------------------------------ workspaces --
constexpr size_t kAlign = 256;
__host__ __device__ constexpr size_t align_up(size_t n, size_t a = kAlign) { return (n + a - 1) / a * a; }

struct Carver {
    char *base;
    size_t off;
    template <class T> T *take(size_t n)
    {
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off += align_up(n * sizeof(T));
        return p;
    }
};

// -------------------------------------------------- internal launchers ---
// These assume validated arguments; the public entry points validate.

// Every public workspace starts with kCtrlBytes of counters that must be zero
// before the first call on it; each call leaves them zero when it completes.
// The rest of the workspace is carved from kCtrlBytes on.
constexpr size_t kCtrlBytes = 256;

// Router workspace (after the control bytes) and launcher.  `ticket` points at
// the control bytes: the 64 arrival counters of the single-launch router
// (zero on entry, zero again when the launch completes); probs [T, E] fp32
// softmax output, or NULL.
size_t route_ws_bytes(int64_t T, int d, int E, moe_dtype_t dt);
size_t gemm_ws_bytes();
int device_cus(); // compute units of the current device (cached per thread and device)
moe_status_t launch_route(const void *x, moe_dtype_t dt, const float *w_router, const float *b_router,
                          const float *sel_bias, int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx,
                          float *topk_w,
                          int32_t *expert_count, float *f, float *P, float *l_aux, float *probs, void *ws,
                          unsigned *ticket, hipStream_t stream);

size_t dispatch_ws_bytes(int64_t T, int k, int E_loc);
int64_t capacity_of(int64_t T, int E, float capacity_factor); // -1: no cap
moe_status_t launch_dispatch(const void *x, moe_dtype_t dt, const int32_t *topk_idx, int64_t T, int d,
                             int E, int k, float capacity_factor, int e0, int E_loc, int32_t *seg_offsets,
                             int32_t *kept_count, int32_t *slot_row, int32_t *row_src, void *x_perm,
                             int64_t max_rows, int32_t *n_dropped, void *ws, hipStream_t stream);

moe_status_t launch_grouped_gemm(const void *a, const int32_t *seg_offsets, int num_segments,
                                 int64_t max_rows, int N, int K, moe_dtype_t dt, const void *w,
                                 const void *bias, int activation, void *out, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

// Router logits as a bf16 GEMM: x [T, d] against w3 [3E, d] = the hi, mid
// and lo bf16 pieces of the fp32 router weight stacked along the rows; fp32
// output [T, 3E] whose three column blocks sum to the logits.  Needs d % 64 == 0.
moe_status_t launch_router_gemm(const void *x, const void *w3, int64_t T, int d, int E, float *logits, void *ws,
                                size_t ws_bytes, hipStream_t stream);

// Forward-form grouped GEMM with an fp32 output and no activation:
// out[r, n] = sum_k a[r, k] w[s, n, k] (+ bias[s, n]).  bf16 needs K % 64 == 0.
moe_status_t launch_grouped_gemm_f32out(const void *a, const int32_t *seg_offsets, int num_segments,
                                        int64_t max_rows, int N, int K, moe_dtype_t dt, const void *w,
                                        const void *bias, float *out, void *ws, size_t ws_bytes, hipStream_t stream);

// The same with a K-major weight, w_kn [S, K, N] (N contiguous): out[r, n] =
// sum_k a[r, k] w_kn[s, k, n], no bias; bf16 only, K % 64 == 0, K >= 128,
// N % 4 == 0, K * N < 2^31.
moe_status_t launch_grouped_gemm_kmajor_f32out(const void *a, const int32_t *seg_offsets, int num_segments,
                                               int64_t max_rows, int N, int K, const void *w_kn, float *out,
                                               void *ws, size_t ws_bytes, hipStream_t stream);

// K-segmented layout of the weight-gradient GEMMs: segment s of seg (NULL =
// one segment of max_rows rows) takes max(2, ceil(rows_s / 64)) steps of 64
// columns (none if empty); kcol [S+1] = first step of each segment, kcol[S]
// the total.  kseg_cols_bound bounds 64 * kcol[S].
int64_t kseg_cols_bound(int64_t max_rows, int S);
moe_status_t launch_kseg_layout(const int32_t *seg, int S, int64_t max_rows, int32_t *kcol, hipStream_t stream);
// C [S, M, N] fp32: C_s[m, n] = sum over segment s's columns k of A[m, k] W[n, k],
// A [M, Kp], W [N, Kp] (dt; padding columns zero).  Empty segments give zeros.
moe_status_t launch_kseg_gemm(const void *A, const void *W, const int32_t *kcol, int S, int M, int N, int64_t Kp,
                              moe_dtype_t dt, float *C, hipStream_t stream);
// The same sums over the row-major rows themselves (bf16): A_rows [rows, M],
// W_rows [rows, N], segment s = rows seg[s] .. seg[s+1] (seg NULL: all rows),
// kcol from launch_kseg_layout over the same seg; no segment may hold more
// than seg_max rows.  kseg_kmajor_ok: M and N multiples of 8 and
// seg_max x max(M, N) below 2^30.
bool kseg_kmajor_ok(int64_t seg_max, int M, int N);
moe_status_t launch_kseg_gemm_kmajor(const void *A_rows, const void *W_rows, const int32_t *seg, int64_t rows,
                                     int64_t seg_max, const int32_t *kcol, int S, int M, int N, float *C,
                                     hipStream_t stream);

// h = GELU(u) (dtype dt) over the rows in use of u [rows, F] fp32 (seg[S]
// of them, or all rows when seg is NULL); F % 4 == 0.
moe_status_t launch_gelu_rows(const float *u, const int32_t *seg, int S, int64_t rows, int F, moe_dtype_t dt,
                              void *h, hipStream_t stream);

moe_status_t launch_combine(const void *y_perm, int64_t max_rows, const int32_t *slot_row,
                            const float *topk_w, const void *y_shared, int64_t T, int d, int k,
                            moe_dtype_t dt, void *y, hipStream_t stream);

// Backward-pass kernels (backward.hip); the K-segmented layout and column
// map are those of launch_kseg_layout.
moe_status_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);
// dst[b] = src[b]^T for B matrices of R x C (multiples of 8); matrix b is
// skipped when seg (may be NULL) gives segment b no rows.
moe_status_t launch_transpose_batched(const void *src, int B, int R, int C, const int32_t *seg, moe_dtype_t dt,
                                      void *dst, hipStream_t stream);
moe_status_t launch_gather_t(const void *src, int D, const int32_t *row_src, int k, const float *wgt,
                             const int32_t *seg, int S, int64_t rows, const int32_t *kcol, int64_t Kp, moe_dtype_t dt,
                             void *dstT, void *dst, float *colpart, hipStream_t stream);
moe_status_t launch_act_bwd(const float *u, const float *dh, int F, const int32_t *row_src, const float *wgt,
                            const int32_t *seg, int S, int64_t rows, const int32_t *kcol, int64_t Kp, moe_dtype_t dt,
                            void *du, void *duT, void *gwT, void *gw, float *dwpart, float *colpart,
                            hipStream_t stream);
moe_status_t launch_seg_colsum(const float *colpart, const int32_t *kcol, int S, int D, float *out,
                               hipStream_t stream);
moe_status_t launch_router_bwd(const float *probs, const int32_t *topk_idx, const int32_t *slot_row,
                               const float *dwpart, int FT, const void *b2, const void *dY, moe_dtype_t dt, int d,
                               int e0, const float *f, float c_aux, int64_t T, int E, int k, float *dl,
                               hipStream_t stream);
size_t router_wgrad_ws_bytes(int64_t T, int d, int E);
size_t router_bias_ws_bytes(int E); // bias_part of the router launchers
moe_status_t launch_router_wgrad(const void *x, moe_dtype_t dt, const float *dl, int64_t T, int d, int E,
                                 float *dw_r, float *db_r, float *bias_part, void *ws, hipStream_t stream);
// dx = kept dx rows + dx_sh (may be NULL) + the router term: dx_r if given,
// else dl . W_r on the vector units.
moe_status_t launch_dx_combine(const float *dx_rows, const int32_t *slot_row, int k, const float *dx_sh,
                               const float *dx_r, const float *dl, const float *w_r, int64_t T, int d, int E, float *dx,
                               hipStream_t stream);
// Router backward on the matrix cores (bf16 layers, E % 8 == 0, d % 64 == 0):
// dl as launch_router_bwd; dW_r = dl^T x from an exact three-piece bf16 split
// of dl (fp32-accurate), db_r (if not NULL); *dx_r = a workspace buffer
// [T, d] holding dl . W_r from two-piece splits of both operands.
size_t router_mfma_ws_bytes(int64_t T, int d, int E);
moe_status_t launch_router_bwd_mfma(const float *probs, const int32_t *topk_idx, const int32_t *slot_row,
                                    const float *dwpart, int FT, const void *b2, const void *dY, int d, int e0,
                                    const float *f, float c_aux, int64_t T, int E, int k, const void *x,
                                    const float *w_r, float *dl, float *dw_r, float *db_r, float *bias_part,
                                    float **dx_r, void *ws, void *gemm_ws, size_t gemm_ws_bytes, hipStream_t stream);

} // namespace moe
