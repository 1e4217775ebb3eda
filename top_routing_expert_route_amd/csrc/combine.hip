// Combine of the MoE layer: the routing-weighted sum of the expert outputs,
// written back at each token's own position.
//
// Pages: "Expert Parallelism (MoE)", section "MoE Layer Structure" (Y = sum
// over the selected experts of expert_output * routing_weight) and section
// "Top-K Routing and Capacity Factor" (a dropped selection's routing weight
// is zeroed); "Expert Parallelism (EP)", section "Key math / How it works"
// (combine sends the outputs back to each token's home position).
//
// One wave per token.  The wave reads its k (slot_row, weight) pairs, gathers
// the kept rows of y_perm with 16-byte loads, sums in fp32 in slot order,
// adds the shared-expert row last, and writes the token's row once.
#include "common.hpp"

namespace moe {

namespace {

template <int U>
__global__ __launch_bounds__(256) void combine_bf16(const u32x4 *__restrict__ y_perm, int64_t max_rows,
                                                    const int32_t *__restrict__ slot_row,
                                                    const float *__restrict__ topk_w,
                                                    const u32x4 *__restrict__ y_shared, int64_t T, int64_t units,
                                                    int k, u32x4 *__restrict__ y)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    for (int64_t u0 = 0; u0 < units; u0 += 64 * U) {
        float acc[U][8];
#pragma unroll
        for (int q = 0; q < U; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[q][e] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int r = slot_row[t * k + j];
            if (r < 0 || r >= max_rows)
                continue;
            const float w = topk_w[t * k + j];
            const u32x4 *src = y_perm + (int64_t)r * units;
            u32x4 v[U];
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int64_t u = u0 + q * 64 + lane;
                v[q] = u < units ? src[u] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int q = 0; q < U; ++q)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    acc[q][2 * h] = fmaf(w, bf16_bits_to_f32(v[q][h] & 0xFFFFu), acc[q][2 * h]);
                    acc[q][2 * h + 1] = fmaf(w, bf16_bits_to_f32(v[q][h] >> 16), acc[q][2 * h + 1]);
                }
        }
        if (y_shared) {
            const u32x4 *src = y_shared + t * units;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int64_t u = u0 + q * 64 + lane;
                if (u < units) {
                    const u32x4 v = src[u];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        acc[q][2 * h] += bf16_bits_to_f32(v[h] & 0xFFFFu);
                        acc[q][2 * h + 1] += bf16_bits_to_f32(v[h] >> 16);
                    }
                }
            }
        }
        u32x4 *dst = y + t * units;
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int64_t u = u0 + q * 64 + lane;
            if (u < units) {
                u32x4 o;
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    o[h] = pack_bf16x2(acc[q][2 * h], acc[q][2 * h + 1]);
                dst[u] = o;
            }
        }
    }
}

template <int U>
__global__ __launch_bounds__(256) void combine_f32(const f32x4 *__restrict__ y_perm, int64_t max_rows,
                                                   const int32_t *__restrict__ slot_row,
                                                   const float *__restrict__ topk_w,
                                                   const f32x4 *__restrict__ y_shared, int64_t T, int64_t units,
                                                   int k, f32x4 *__restrict__ y)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    for (int64_t u0 = 0; u0 < units; u0 += 64 * U) {
        f32x4 acc[U];
#pragma unroll
        for (int q = 0; q < U; ++q)
            acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int r = slot_row[t * k + j];
            if (r < 0 || r >= max_rows)
                continue;
            const float w = topk_w[t * k + j];
            const f32x4 *src = y_perm + (int64_t)r * units;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int64_t u = u0 + q * 64 + lane;
                if (u < units) {
                    const f32x4 v = src[u];
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        acc[q][h] = fmaf(w, v[h], acc[q][h]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int64_t u = u0 + q * 64 + lane;
            if (u < units) {
                f32x4 o = acc[q];
                if (y_shared) {
                    const f32x4 v = y_shared[t * units + u];
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        o[h] += v[h];
                }
                y[t * units + u] = o;
            }
        }
    }
}

// h = GELU(u) in the layer's dtype for the rows in use (the first seg[S]
// rows; all `rows` when seg is NULL), from the fp32 pre-activations u
// [rows, F] (F % 4 == 0).  The same GELU and the same rounding as the first
// GEMM's fused epilogue, so h is bitwise what that epilogue writes.
template <class T>
__global__ __launch_bounds__(256) void gelu_rows(const float *__restrict__ u, const int32_t *__restrict__ seg, int S,
                                                 int64_t rows, int F, T *__restrict__ h)
{
    const int64_t used = seg ? (int64_t)seg[S] : rows;
    const int64_t n4 = (used < rows ? used : rows) * (F / 4);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const f32x4 v = reinterpret_cast<const f32x4 *>(u)[i];
        const float g0 = gelu_erf(v[0]), g1 = gelu_erf(v[1]), g2 = gelu_erf(v[2]), g3 = gelu_erf(v[3]);
        if constexpr (sizeof(T) == 2) {
            uint2 o;
            o.x = pack_bf16x2(g0, g1);
            o.y = pack_bf16x2(g2, g3);
            reinterpret_cast<uint2 *>(h)[i] = o;
        } else {
            reinterpret_cast<f32x4 *>(h)[i] = f32x4{g0, g1, g2, g3};
        }
    }
}

} // namespace

moe_status_t launch_gelu_rows(const float *u, const int32_t *seg, int S, int64_t rows, int F, moe_dtype_t dt,
                              void *h, hipStream_t stream)
{
    const int64_t n4 = rows * (F / 4);
    if (n4 == 0)
        return MOE_OK;
    const unsigned blocks = (unsigned)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
    if (dt == MOE_BF16)
        gelu_rows<uint16_t><<<blocks, 256, 0, stream>>>(u, seg, S, rows, F, (uint16_t *)h);
    else
        gelu_rows<float><<<blocks, 256, 0, stream>>>(u, seg, S, rows, F, (float *)h);
    return check_launch("gelu_rows");
}

moe_status_t launch_combine(const void *y_perm, int64_t max_rows, const int32_t *slot_row, const float *topk_w,
                            const void *y_shared, int64_t T, int d, int k, moe_dtype_t dt, void *y,
                            hipStream_t stream)
{
    if (T == 0)
        return MOE_OK;
    const unsigned blocks = (unsigned)((T + 3) / 4);
    if (dt == MOE_BF16) {
        const int64_t units = (int64_t)d / 8;
        combine_bf16<4><<<blocks, 256, 0, stream>>>((const u32x4 *)y_perm, max_rows, slot_row, topk_w,
                                                    (const u32x4 *)y_shared, T, units, k, (u32x4 *)y);
    } else {
        const int64_t units = (int64_t)d / 4;
        combine_f32<4><<<blocks, 256, 0, stream>>>((const f32x4 *)y_perm, max_rows, slot_row, topk_w,
                                                   (const f32x4 *)y_shared, T, units, k, (f32x4 *)y);
    }
    return check_launch("combine");
}

} // namespace moe
