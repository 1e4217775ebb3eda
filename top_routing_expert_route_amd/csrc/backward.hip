// Backward pass of the MoE layer: the element-wise, permutation and router
// kernels around the grouped GEMMs (which live in gemm.hip).
//
// Pages: "Load Balancing: The Auxiliary Loss" (L_aux is added to the task
// loss and backpropagated; f counts selections and carries no gradient) and
// "MoE Layer Structure" (Y = sum of routing weight times expert output, the
// weight being the router's softmax probability).
//
// Notation, per kept selection placed in dispatched row r (token t, local
// expert s, routing weight w_r = p[t, e]):
//   u_r = W1_s x_t + b1_s,  g_r = GELU(u_r),  v_r = W2_s g_r + b2_s,
//   Y_t += w_r v_r.
// With dY = dL/dY:
//   dh'_r = W2_s^T dY_t                     (the gradient at g_r, before w_r)
//   dw_r  = dY_t . v_r = dh'_r . g_r + dY_t . b2_s
//   du_r  = w_r dh'_r * GELU'(u_r)
//   dW2_s = sum_r dY_t (w_r g_r)^T,  db2_s = sum_r w_r dY_t
//   dW1_s = sum_r du_r x_t^T,        db1_s = sum_r du_r
//   dx_t += W1_s^T du_r
// Router, softmax over E: dp[t, e] = g_aux alpha f_e / T + sum of dw_r over
// t's kept selections of e; dl[t, e] = p[t, e] (dp[t, e] - sum_e' p dp);
//   dW_r = sum_t dl_t x_t^T, db_r = sum_t dl_t, dx_t += W_r^T dl_t.
// The shared expert is the same FFN with w_r = 1 on every token.
//
// The weight-gradient GEMMs contract over dispatched rows, so their operands
// are stored transposed in the K-segmented layout (kcol): row block s of
// 64-aligned columns per segment, zero-padded.  The kernels here write those
// operands straight from the row-major data, transposing through LDS tiles
// (gather_t, act_bwd).  The weights need no transpose for bf16 layers (the
// GEMMs read them K-major); fp32 layers transpose them in registers
// (transpose_batched).
#include "common.hpp"

namespace moe {

namespace {

template <class T> struct Elt;
template <> struct Elt<float> {
    static __device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elt<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t *p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

// Rows of segment s: seg == NULL is one segment of `rows` rows.
__device__ __forceinline__ void seg_rows(const int32_t *seg, int s, int64_t rows, int64_t &lo, int64_t &hi)
{
    if (!seg) {
        lo = 0;
        hi = rows;
        return;
    }
    lo = seg[s];
    hi = seg[s + 1];
    lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
    hi = hi < lo ? lo : (hi > rows ? rows : hi);
}

// Segment owning column tile ct < kcol[S]: the largest s with kcol[s] <= ct
// (empty segments share their kcol with the next one).
__device__ __forceinline__ int seg_of_tile(const int32_t *kcol, int S, int ct)
{
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (kcol[mid] <= ct)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// 8 x 8 blocks of 16-bit values held as 8 rows of 16 bytes: out[j] element i
// = in[i] element j.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            // out[j] dword h = (in[2h] elem j, in[2h+1] elem j)
            const uint32_t lo = in[2 * h][j >> 1], hi = in[2 * h + 1][j >> 1];
            out[j][h] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
    }
}

// 4 x 4 blocks of 32-bit values.
__device__ __forceinline__ void transpose4x4(const u32x4 (&in)[4], u32x4 (&out)[4])
{
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[j][i] = in[i][j];
}

// dst[b, c, r] = src[b, r, c] for B matrices of R x C (R, C multiples of 8),
// skipping matrix b when seg says segment b has no rows.  Each lane moves a
// V x V block (V = 16 bytes / element size) with V 16-byte loads, an
// in-register transpose and V 16-byte stores; a wave covers 8V x 8V with
// 128-byte row segments on both sides.
template <int ES>
__global__ __launch_bounds__(256) void transpose_batched(const uint16_t *__restrict__ src, int R, int C,
                                                         const int32_t *__restrict__ seg,
                                                         uint16_t *__restrict__ dst)
{
    constexpr int V = 16 / ES, W = 8 * V; // wave tile edge in elements
    const int64_t b = blockIdx.z;
    if (seg && seg[b + 1] <= seg[b])
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 7, rg = lane >> 3;
    const int r0 = (blockIdx.y * 2 + (wave >> 1)) * W + rg * V;
    const int c0 = (blockIdx.x * 2 + (wave & 1)) * W + cg * V;
    if (r0 >= R || c0 >= C)
        return;
    const char *s = reinterpret_cast<const char *>(src) + (b * R * C) * ES;
    char *o = reinterpret_cast<char *>(dst) + (b * R * C) * ES;
    if (V == 8) {
        u32x4 in[8], out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            in[i] = *reinterpret_cast<const u32x4 *>(s + ((int64_t)(r0 + i) * C + c0) * ES);
        transpose8x8(in, out);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<u32x4 *>(o + ((int64_t)(c0 + j) * R + r0) * ES) = out[j];
    } else {
        u32x4 in[4], out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            in[i] = *reinterpret_cast<const u32x4 *>(s + ((int64_t)(r0 + i) * C + c0) * ES);
        transpose4x4(in, out);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4 *>(o + ((int64_t)(c0 + j) * R + r0) * ES) = out[j];
    }
}

// Gather of token rows into the K-segmented layout.  Column 64 kcol[s] + i
// holds row r = lo_s + i of segment s (token t = row_src[r] / k, or r when
// row_src is NULL); columns past the segment's rows are zero.  D % 8 == 0.
//   dstT[f, col]     = src[t, f]                      (if dstT)
//   dst[r, f]        = src[t, f]                      (if dst)
//   colpart[ct, f]   = sum over the tile's rows of wgt[row_src[r]] src[t, f]
//                      (wgt NULL: weight 1)           (if colpart)
// A wave takes a 64-row column tile x 64 features, each lane an 8 x 8 block
// (rows 8 rg.., features 8 cg..): 16-byte loads and stores on both sides,
// the column sums a fixed shuffle tree.  Grid (ceil(D / 256), strided over
// the column tiles).
template <class T> __device__ __forceinline__ void load8(const T *p, float (&v)[8]);
template <> __device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float (&v)[8])
{
    const u32x4 q = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        v[2 * h] = bf16_bits_to_f32(q[h] & 0xFFFFu);
        v[2 * h + 1] = bf16_bits_to_f32(q[h] >> 16);
    }
}
template <> __device__ __forceinline__ void load8<float>(const float *p, float (&v)[8])
{
    const f32x4 a = reinterpret_cast<const f32x4 *>(p)[0], b = reinterpret_cast<const f32x4 *>(p)[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[j + 4] = b[j];
    }
}

template <class T> __device__ __forceinline__ void store8(T *p, const float (&v)[8]);
template <> __device__ __forceinline__ void store8<uint16_t>(uint16_t *p, const float (&v)[8])
{
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 4; ++h)
        o[h] = pack_bf16x2(v[2 * h], v[2 * h + 1]);
    *reinterpret_cast<u32x4 *>(p) = o;
}
template <> __device__ __forceinline__ void store8<float>(float *p, const float (&v)[8])
{
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <class T> __device__ __forceinline__ void store4v(T *p, const float (&v)[4]);
template <> __device__ __forceinline__ void store4v<uint16_t>(uint16_t *p, const float (&v)[4])
{
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2 *>(p) = o;
}
template <> __device__ __forceinline__ void store4v<float>(float *p, const float (&v)[4])
{
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

template <class T>
__global__ __launch_bounds__(256) void gather_t(const T *__restrict__ src, int D, const int32_t *__restrict__ row_src,
                                                int k, const float *__restrict__ wgt, const int32_t *__restrict__ seg,
                                                int S, int64_t rows, const int32_t *__restrict__ kcol, int64_t Kp,
                                                T *__restrict__ dstT, T *__restrict__ dst, float *__restrict__ colpart)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 7, rg = lane >> 3;
    const int ft = blockIdx.x * 4 + wave;
    if (ft * 64 >= D)
        return; // whole wave; there is no barrier below
    const int f0 = ft * 64 + cg * 8;
    const bool fv = f0 < D; // lanes past D take part in the shuffles with zeros
    const int total = kcol[S];
    for (int ct = blockIdx.y; ct < total; ct += gridDim.y) {
        const int s = seg_of_tile(kcol, S, ct);
        int64_t lo, hi;
        seg_rows(seg, s, rows, lo, hi);
        const int64_t r0 = lo + (int64_t)(ct - kcol[s]) * 64 + rg * 8;
        float v[8][8], w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + i;
            const bool ok = r < hi;
            int64_t tok = 0;
            w[i] = 0.f;
            if (ok) {
                const int64_t slot = row_src ? (int64_t)row_src[r] : r;
                tok = row_src ? slot / k : slot;
                w[i] = wgt ? wgt[slot] : 1.f;
            }
            if (ok && fv) {
                load8<T>(src + tok * D + f0, v[i]);
                if (dst)
                    store8<T>(dst + r * D + f0, v[i]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[i][j] = 0.f;
            }
        }
        if (colpart) {
            float cs[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    a = fmaf(w[i], v[i][j], a);
                a += __shfl_xor(a, 8, 64);
                a += __shfl_xor(a, 16, 64);
                a += __shfl_xor(a, 32, 64);
                cs[j] = a;
            }
            if (rg == 0 && fv)
                store8<float>(colpart + (int64_t)ct * D + f0, cs);
        }
        if (!dstT)
            continue;
        const int64_t col = (int64_t)ct * 64 + rg * 8;
#pragma unroll
        for (int j = 0; j < 8 && fv; ++j) {
            float c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                c[i] = v[i][j];
            store8<T>(dstT + (int64_t)(f0 + j) * Kp + col, c);
        }
    }
}

// GELU backward over the K-segmented rows (same row/column map as gather_t),
// from u = W1 x + b1 and dh' (both fp32 [rows, F], F % 4 == 0):
//   du[r, q]  = w_r dh'[r, q] GELU'(u[r, q])        (row-major, T)
//   gw[r, q]  = w_r GELU(u[r, q])                    (row-major, if gw)
//   duT[q, col] = du[r, q],  gwT[q, col] = gw[r, q]  (zero padding; if duT)
//   dwpart[r, qt] = sum_{q in feature tile qt} dh'[r, q] GELU(u[r, q])   (if dwpart)
//   colpart[ct, q] = sum over the tile's rows of du[r, q]               (if colpart)
// w_r = wgt[row_src[r]] (1 when wgt is NULL).  A block takes one 64-row
// column tile x 64 features.  Thread (wave w, lane l) holds a 4 x 4 block:
// features 4 (l % 16).., rows 16 (l / 16) + 4 w..; one load instruction of a
// wave reads 4 rows of 256 contiguous bytes.  du goes out row-major from
// registers; duT and gwT go through LDS ([feature][row], rows padded to a
// 16-byte multiple) and out as 16-byte row pieces of the transposed arrays.
// Row sums over the 16 lanes of a row are DPP trees, column sums add the
// thread's rows, the wave's four row groups and then the waves in order.
// Grid (FT = ceil(F / 64), strided over the column tiles).
template <class T>
__global__ __launch_bounds__(256) void act_bwd(const float *__restrict__ u, const float *__restrict__ dh, int F,
                                               int FT, const int32_t *__restrict__ row_src,
                                               const float *__restrict__ wgt, const int32_t *__restrict__ seg, int S,
                                               int64_t rows, const int32_t *__restrict__ kcol, int64_t Kp,
                                               T *__restrict__ du, T *__restrict__ duT, T *__restrict__ gwT,
                                               T *__restrict__ gw, float *__restrict__ dwpart,
                                               float *__restrict__ colpart)
{
    constexpr int ES = (int)sizeof(T);
    constexpr int LS = 64 + 16 / ES;            // LDS row (one feature) of 64 rows, padded
    constexpr int VPC = 16 / ES;                // elements per 16-byte piece
    constexpr int LPR = 64 / VPC;               // lanes per transposed row (feature)
    constexpr int FPP = 256 / LPR;              // features per pass of the block
    __shared__ __attribute__((aligned(16))) T sdu[64 * LS];
    __shared__ __attribute__((aligned(16))) T sgw[64 * LS];
    __shared__ float red[4][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, rq = lane >> 4;
    const int qt = blockIdx.x;
    const int fl = 4 * c;                       // first feature of the thread within the tile
    const int q = qt * 64 + fl;
    const bool qv = q < F;                      // F % 4 == 0: all four features or none
    const int rl = 16 * rq + 4 * wave;          // first row of the thread within the tile
    const int total = kcol[S];
    for (int ct = blockIdx.y; ct < total; ct += gridDim.y) {
        const int s = seg_of_tile(kcol, S, ct);
        int64_t lo, hi;
        seg_rows(seg, s, rows, lo, hi);
        const int64_t rt = lo + (int64_t)(ct - kcol[s]) * 64; // tile's first row
        f32x4 uu[4], hh[4];
        float w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = rt + rl + i;
            const bool ok = r < hi && qv;
            uu[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            hh[i] = uu[i];
            if (ok) {
                uu[i] = *reinterpret_cast<const f32x4 *>(u + r * F + q);
                hh[i] = *reinterpret_cast<const f32x4 *>(dh + r * F + q);
            }
            w[i] = ok ? (wgt ? wgt[row_src ? row_src[r] : r] : 1.f) : 0.f;
        }
        float vdu[4][4], vgw[4][4], rs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = rt + rl + i;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float g, gp;
                gelu_and_grad(uu[i][j], g, gp);
                vdu[i][j] = w[i] * hh[i][j] * gp; // zero outside the segment (w = 0)
                vgw[i][j] = w[i] * g;
                acc = fmaf(hh[i][j], g, acc);
            }
            rs[i] = acc;
            if (r < hi && qv) {
                store4v<T>(du + r * F + q, vdu[i]);
                if (gw)
                    store4v<T>(gw + r * F + q, vgw[i]);
            }
        }
        // transposed through LDS: feature fl + j, rows rl .. rl + 3
        __syncthreads(); // the previous tile's LDS reads are done
#pragma unroll
        for (int j = 0; j < 4 && duT; ++j) {
            const float a4[4] = {vdu[0][j], vdu[1][j], vdu[2][j], vdu[3][j]};
            const float g4[4] = {vgw[0][j], vgw[1][j], vgw[2][j], vgw[3][j]};
            store4v<T>(sdu + (fl + j) * LS + rl, a4);
            store4v<T>(sgw + (fl + j) * LS + rl, g4);
        }
        if (dwpart) {
            // row sums over the tile's 64 features: the row's 16 lanes
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = row16_sum(rs[i]);
                const int64_t r = rt + rl + i;
                if (c == 0 && r < hi)
                    dwpart[r * FT + qt] = v;
            }
        }
        if (colpart) {
            // column sums over the tile's 64 rows
            f32x4 cs;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = (vdu[0][j] + vdu[1][j]) + (vdu[2][j] + vdu[3][j]);
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                cs[j] = v;
            }
            if (rq == 0)
                *reinterpret_cast<f32x4 *>(&red[wave][fl]) = cs;
        }
        __syncthreads();
        if (colpart && threadIdx.x < 64) {
            const int f = threadIdx.x;
            const float v = (red[0][f] + red[1][f]) + (red[2][f] + red[3][f]);
            if (qt * 64 + f < F)
                colpart[(int64_t)ct * F + qt * 64 + f] = v;
        }
        // transposed rows: feature fq, a 16-byte piece of the tile's 64 columns
#pragma unroll
        for (int p = 0; p < 64 / FPP; ++p) {
            const int fq = p * FPP + threadIdx.x / LPR;
            const int piece = threadIdx.x % LPR;
            if (duT && qt * 64 + fq < F) {
                const int64_t at = (int64_t)(qt * 64 + fq) * Kp + (int64_t)ct * 64 + piece * VPC;
                *reinterpret_cast<u32x4 *>(duT + at) = *reinterpret_cast<const u32x4 *>(sdu + fq * LS + piece * VPC);
                *reinterpret_cast<u32x4 *>(gwT + at) = *reinterpret_cast<const u32x4 *>(sgw + fq * LS + piece * VPC);
            }
        }
    }
}

// out[s, f] = sum of colpart[ct, f] over segment s's column tiles (0 for an
// empty segment).  Block = 64 features x 16 waves: wave w sums the tiles
// c = kcol[s] + w + 16 i in order (256-byte rows), then the 16 partials are
// added in wave order.  Grid (ceil(D / 64), S).
__global__ __launch_bounds__(1024) void seg_colsum(const float *__restrict__ colpart, const int32_t *__restrict__ kcol,
                                                   int D, float *__restrict__ out)
{
    __shared__ float red[16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = blockIdx.y;
    const int f = blockIdx.x * 64 + lane;
    float a = 0.f;
    if (f < D)
        for (int c = kcol[s] + wave; c < kcol[s + 1]; c += 16)
            a += colpart[(int64_t)c * D + f];
    red[wave][lane] = a;
    __syncthreads();
    if (wave == 0 && f < D) {
        float t = 0.f;
        for (int w = 0; w < 16; ++w)
            t += red[w][lane];
        out[(int64_t)s * D + f] = t;
    }
}

constexpr int kMaxFastK = 8;

// dl as two bf16 pieces, laid out (hi, hi, lo) for the dl . W_r GEMM.
__device__ __forceinline__ void store_dl2(uint16_t *row, int e, int E64, float v)
{
    const uint16_t hi = f32_to_bf16_bits(v);
    const uint16_t lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
    row[e] = hi;
    row[E64 + e] = hi;
    row[2 * E64 + e] = lo;
}

// dp and the softmax backward of one token when lane j holds selection j
// (general k): the pairs are broadcast with shuffles.
__device__ void slow_router_tail(const float *pt, const float *f, float c_aux, int E, int k, int my_e, float my_dw,
                                 int lane, float *dlt, uint16_t *dl2t, int E64)
{
    float sd = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
        const int eb = pass == 1 && dl2t ? E64 : E;
        for (int b = 0; b < eb; b += 64) {
            const int e = b + lane;
            float dp = e < E ? c_aux * f[e] : 0.f;
            for (int j = 0; j < k; ++j) {
                const int ej = __shfl(my_e, j, 64);
                const float dj = __shfl(my_dw, j, 64);
                if (ej == e)
                    dp += dj;
            }
            if (pass == 0) {
                if (e < E)
                    sd = fmaf(pt[e], dp, sd);
            } else {
                const float v = e < E ? pt[e] * (dp - sd) : 0.f;
                if (e < E)
                    dlt[e] = v;
                if (dl2t && e < E64)
                    store_dl2(dl2t, e, E64, v);
            }
        }
        if (pass == 0)
            sd = wave_sum(sd);
    }
}

// Router backward, one wave per token: dw of every kept selection, then
//   dp[e] = c_aux f[e] + sum_{kept j with topk_idx = e} dw_j   (c_aux = g_aux alpha / T)
//   dl[t, e] = p[t, e] (dp[e] - sum_e' p[t, e'] dp[e']).
// dw_j = sum_qt dwpart[r, qt] (+ dY_t . b2[e - e0]).
template <class T>
__global__ __launch_bounds__(256) void router_bwd(const float *__restrict__ probs, const int32_t *__restrict__ topk_idx,
                                                  const int32_t *__restrict__ slot_row,
                                                  const float *__restrict__ dwpart, int FT, const T *__restrict__ b2,
                                                  const T *__restrict__ dY, int d, int e0,
                                                  const float *__restrict__ f, float c_aux, int64_t Ttok, int E, int k,
                                                  float *__restrict__ dl, uint16_t *__restrict__ dl2, int E64)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= Ttok)
        return; // wave-uniform; the block has no barrier
    // (expert or -1 unless kept, dw) of selection j, held uniformly
    int se[kMaxFastK];
    float sw[kMaxFastK];
    const bool fast = !b2 && k <= kMaxFastK && FT <= 8 * kMaxFastK;
    if (fast) {
        // 8 lanes per selection sum its row of partials; one DPP tree per group
        const int j = lane >> 3, sub = lane & 7;
        int e = -1;
        float a = 0.f;
        if (j < k) {
            const int r = slot_row[t * k + j];
            if (r >= 0) {
                e = topk_idx[t * k + j];
                for (int qt = sub; qt < FT; qt += 8)
                    a += dwpart[(int64_t)r * FT + qt];
            }
        }
        a = group8_sum(a);
#pragma unroll
        for (int jj = 0; jj < kMaxFastK; ++jj) {
            se[jj] = jj < k ? __builtin_amdgcn_readlane(e, 8 * jj) : -1;
            sw[jj] = jj < k ? lane_value(a, 8 * jj) : 0.f;
        }
    } else {
        // lane j keeps selection j: its expert (-1 unless kept) and dw
        int my_e = -1;
        float my_dw = 0.f;
        for (int j = 0; j < k; ++j) {
            const int64_t slot = t * k + j;
            const int r = slot_row[slot];
            const int e = topk_idx[slot];
            float a = 0.f;
            if (r >= 0) {
                for (int qt = lane; qt < FT; qt += 64)
                    a += dwpart[(int64_t)r * FT + qt];
                if (b2) {
                    const T *brow = b2 + (int64_t)(e - e0) * d;
                    for (int o = lane; o < d; o += 64)
                        a = fmaf(Elt<T>::ld(dY, t * d + o), Elt<T>::ld(brow, o), a);
                }
            }
            a = wave_sum(a);
            if (lane == j) {
                my_e = r >= 0 ? e : -1;
                my_dw = a;
            }
        }
        slow_router_tail(probs + t * E, f, c_aux, E, k, my_e, my_dw, lane, dl + t * E, dl2 ? dl2 + t * 3 * (int64_t)E64 : nullptr, E64);
        return;
    }
    const float *pt = probs + t * E;
    float sd = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
        const int eb = pass == 1 && dl2 ? E64 : E;
        for (int b = 0; b < eb; b += 64) {
            const int e = b + lane;
            float dp = e < E ? c_aux * f[e] : 0.f;
#pragma unroll
            for (int jj = 0; jj < kMaxFastK; ++jj)
                if (se[jj] == e)
                    dp += sw[jj];
            if (pass == 0) {
                if (e < E)
                    sd = fmaf(pt[e], dp, sd);
            } else {
                const float v = e < E ? pt[e] * (dp - sd) : 0.f;
                if (e < E)
                    dl[t * E + e] = v;
                if (dl2 && e < E64)
                    store_dl2(dl2 + t * (3 * (int64_t)E64), e, E64, v);
            }
        }
        if (pass == 0)
            sd = wave_sum(sd);
    }
}

// w2p[i, p E64 + e] = piece p of W_r[e, i] in the order (hi, lo, hi), the
// counterpart of router_bwd's (hi, hi, lo) rows: the GEMM sums
// dl_hi w_hi + dl_hi w_lo + dl_lo w_hi.  Zero for e >= E.
__global__ __launch_bounds__(256) void router_weight_pieces_t(const float *__restrict__ wr, int E, int d, int E64,
                                                              uint16_t *__restrict__ w2p)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)d * E64)
        return;
    const int i = (int)(q / E64), e = (int)(q % E64);
    const float v = e < E ? wr[(int64_t)e * d + i] : 0.f;
    const uint16_t hi = f32_to_bf16_bits(v);
    const uint16_t lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
    uint16_t *row = w2p + (int64_t)i * 3 * E64;
    row[e] = hi;
    row[E64 + e] = lo;
    row[2 * E64 + e] = hi;
}

// T equal token ranges: seg[s] = T s / S.
__global__ __launch_bounds__(64) void linear_segments(int32_t *__restrict__ seg, int S, int64_t T)
{
    for (int s = threadIdx.x; s <= S; s += 64)
        seg[s] = (int32_t)(T * s / S);
}

// Exact three-piece split of dl in the K-segmented layout of tokens:
// dlT3[p E + e, col] = piece p of dl[t, e] (hi, mid, lo: hi and mid are
// truncations, hi + mid + lo == dl), t the column's token; zero padding.
// E % 8 == 0.  A wave takes 64 tokens x 64 experts, a lane 8 x 8.
__device__ __forceinline__ float trunc_to_bf16(float v) { return __uint_as_float(__float_as_uint(v) & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void dl_pieces_t(const float *__restrict__ dl, int E, const int32_t *__restrict__ seg,
                                                   int S, int64_t T, const int32_t *__restrict__ kcol, int64_t Kp,
                                                   uint16_t *__restrict__ dlT3)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 7, rg = lane >> 3;
    const int et = blockIdx.x * 4 + wave;
    if (et * 64 >= E)
        return;
    const int e0 = et * 64 + cg * 8;
    if (e0 >= E)
        return; // no shuffles below
    const int total = kcol[S];
    for (int ct = blockIdx.y; ct < total; ct += gridDim.y) {
        const int s = seg_of_tile(kcol, S, ct);
        int64_t lo, hi;
        seg_rows(seg, s, T, lo, hi);
        const int64_t r0 = lo + (int64_t)(ct - kcol[s]) * 64 + rg * 8;
        float v[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (r0 + i < hi) {
                load8<float>(dl + (r0 + i) * E + e0, v[i]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[i][j] = 0.f;
            }
        }
        const int64_t col = (int64_t)ct * 64 + rg * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float ph[8], pm[8], pl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = v[i][j];
                ph[i] = trunc_to_bf16(x);
                const float r1 = x - ph[i];
                pm[i] = trunc_to_bf16(r1);
                pl[i] = r1 - pm[i];
            }
            store8<uint16_t>(dlT3 + (int64_t)(e0 + j) * Kp + col, ph);
            store8<uint16_t>(dlT3 + (int64_t)(E + e0 + j) * Kp + col, pm);
            store8<uint16_t>(dlT3 + (int64_t)(2 * E + e0 + j) * Kp + col, pl);
        }
    }
}

// dW_r[e, i] = sum over token ranges c of (hi + (mid + lo)) partials.
__global__ __launch_bounds__(256) void router_wgrad_pieces_reduce(const float *__restrict__ part, int nc, int E, int d,
                                                                  float *__restrict__ out)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)E * d;
    if (q >= n)
        return;
    float a = 0.f;
    for (int c = 0; c < nc; ++c) {
        const float *pc = part + (int64_t)c * 3 * n;
        a += pc[q] + (pc[n + q] + pc[2 * n + q]);
    }
    out[q] = a;
}

// Router weight gradient, first level: part[c, e, i] = sum over token chunk
// c of dl[t, e] x[t, i], for EG experts of group blockIdx.z.
// Grid (ceil(d / 256), chunks, ceil(E / EG)).
template <class T, int EG>
__global__ __launch_bounds__(256) void router_wgrad_part(const T *__restrict__ x, const float *__restrict__ dl,
                                                         int64_t Ttok, int d, int E, int64_t tc,
                                                         float *__restrict__ part)
{
    __shared__ float s_dl[64][EG];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y;
    const int eg0 = blockIdx.z * EG;
    float acc[EG];
#pragma unroll
    for (int e = 0; e < EG; ++e)
        acc[e] = 0.f;
    const int64_t t0 = (int64_t)c * tc, t1 = t0 + tc < Ttok ? t0 + tc : Ttok;
    for (int64_t tb = t0; tb < t1; tb += 64) {
        __syncthreads();
        for (int q = threadIdx.x; q < 64 * EG; q += 256) {
            const int tt = q / EG, e = q % EG;
            const int64_t t = tb + tt;
            s_dl[tt][e] = (t < t1 && eg0 + e < E) ? dl[t * E + eg0 + e] : 0.f;
        }
        __syncthreads();
        const int n = (int)(t1 - tb < 64 ? t1 - tb : 64);
        if (i < d) {
            for (int tt = 0; tt < n; ++tt) {
                const float xv = Elt<T>::ld(x, (tb + tt) * d + i);
#pragma unroll
                for (int e = 0; e < EG; ++e)
                    acc[e] = fmaf(s_dl[tt][e], xv, acc[e]);
            }
        }
    }
    if (i < d) {
#pragma unroll
        for (int e = 0; e < EG; ++e)
            if (eg0 + e < E)
                part[((int64_t)c * E + eg0 + e) * d + i] = acc[e];
    }
}

// dW_r[e, i] = sum_c part[c, e, i] in chunk order.
__global__ __launch_bounds__(256) void router_wgrad_reduce(const float *__restrict__ part, int nchunk, int64_t n,
                                                           float *__restrict__ out)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n)
        return;
    float a = 0.f;
    for (int c = 0; c < nchunk; ++c)
        a += part[(int64_t)c * n + q];
    out[q] = a;
}

// db_r = column sums of dl [T, E].  First level: part[c, e] = sum of dl[t, e]
// over token chunk c; a block takes 64 experts (a wave reads 256 contiguous
// bytes per token) and 4 token lanes (t = t0 + j, t0 + j + 4, ...) whose
// sums are added in lane order.  Second level: the same shape over the
// chunk partials.  Grids (chunks, ceil(E / 64)) and ceil(E / 64).
__global__ __launch_bounds__(256) void router_bias_part(const float *__restrict__ dl, int64_t Ttok, int E, int64_t tc,
                                                        float *__restrict__ part)
{
    __shared__ float red[4][64];
    const int el = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int e = blockIdx.y * 64 + el;
    const int64_t t0 = (int64_t)blockIdx.x * tc, t1 = t0 + tc < Ttok ? t0 + tc : Ttok;
    float a = 0.f;
    if (e < E)
        for (int64_t t = t0 + j; t < t1; t += 4)
            a += dl[t * E + e];
    red[j][el] = a;
    __syncthreads();
    if (j == 0 && e < E)
        part[(int64_t)blockIdx.x * E + e] = ((red[0][el] + red[1][el]) + red[2][el]) + red[3][el];
}

__global__ __launch_bounds__(256) void router_bias_reduce(const float *__restrict__ part, int nch, int E,
                                                          float *__restrict__ db)
{
    __shared__ float red[4][64];
    const int el = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + el;
    float a = 0.f;
    if (e < E)
        for (int c = j; c < nch; c += 4)
            a += part[(int64_t)c * E + e];
    red[j][el] = a;
    __syncthreads();
    if (j == 0 && e < E)
        db[e] = ((red[0][el] + red[1][el]) + red[2][el]) + red[3][el];
}

// dx[t, i] = sum_e dl[t, e] W_r[e, i] (skipped when E = 0) + sum over t's
// kept selections of dx_rows[slot_row, i] + dx_sh[t, i] + dx_r[t, i] (each
// optional).  dx_sh may be dx itself (accumulation in place: each element is
// read and written by the same thread).  Block = TB tokens x 1024 columns,
// 4 columns per thread (d % 4 == 0).
template <int TB>
__global__ __launch_bounds__(256) void dx_combine(const float *__restrict__ dx_rows,
                                                  const int32_t *__restrict__ slot_row, int k, const float *dx_sh,
                                                  const float *__restrict__ dx_r, const float *__restrict__ dl,
                                                  const float *__restrict__ w_r, int64_t Ttok, int d, int E,
                                                  float *dx)
{
    __shared__ float s_dl[TB][64];
    const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
    const int64_t t0 = (int64_t)blockIdx.y * TB;
    f32x4 acc[TB];
#pragma unroll
    for (int q = 0; q < TB; ++q)
        acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int eb = 0; eb < E; eb += 64) {
        const int ne = E - eb < 64 ? E - eb : 64;
        __syncthreads();
        for (int q = threadIdx.x; q < TB * 64; q += 256) {
            const int tq = q / 64, e = q % 64;
            s_dl[tq][e] = (t0 + tq < Ttok && e < ne) ? dl[(t0 + tq) * E + eb + e] : 0.f;
        }
        __syncthreads();
        if (i < d) {
            for (int e = 0; e < ne; ++e) {
                const f32x4 wv = *reinterpret_cast<const f32x4 *>(w_r + (int64_t)(eb + e) * d + i);
#pragma unroll
                for (int q = 0; q < TB; ++q) {
                    const float c = s_dl[q][e];
                    acc[q][0] = fmaf(c, wv[0], acc[q][0]);
                    acc[q][1] = fmaf(c, wv[1], acc[q][1]);
                    acc[q][2] = fmaf(c, wv[2], acc[q][2]);
                    acc[q][3] = fmaf(c, wv[3], acc[q][3]);
                }
            }
        }
    }
    if (i >= d)
        return;
#pragma unroll
    for (int q = 0; q < TB; ++q) {
        const int64_t t = t0 + q;
        if (t >= Ttok)
            break;
        f32x4 v = acc[q];
        for (int j = 0; j < k; ++j) {
            const int r = slot_row[t * k + j];
            if (r >= 0)
                v += *reinterpret_cast<const f32x4 *>(dx_rows + (int64_t)r * d + i);
        }
        if (dx_sh)
            v += *reinterpret_cast<const f32x4 *>(dx_sh + t * d + i);
        if (dx_r)
            v += *reinterpret_cast<const f32x4 *>(dx_r + t * d + i);
        *reinterpret_cast<f32x4 *>(dx + t * d + i) = v;
    }
}

__global__ __launch_bounds__(256) void fill_zero(float *__restrict__ p, int64_t n)
{
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (int64_t)gridDim.x * 256)
        p[q] = 0.f;
}

unsigned strided_grid(int64_t n, int64_t cap) { return (unsigned)(n < 1 ? 1 : (n < cap ? n : cap)); }

constexpr int kBiasChunks = 256; // token chunks of the router bias gradient

} // namespace

moe_status_t launch_fill_zero(float *p, int64_t n, hipStream_t stream)
{
    if (!p || n <= 0)
        return MOE_OK;
    fill_zero<<<strided_grid((n + 255) / 256, 4096), 256, 0, stream>>>(p, n);
    return check_launch("fill_zero");
}

moe_status_t launch_transpose_batched(const void *src, int B, int R, int C, const int32_t *seg, moe_dtype_t dt,
                                      void *dst, hipStream_t stream)
{
    const int W = dt == MOE_BF16 ? 64 : 32; // wave tile; a block is 2 x 2 waves
    const dim3 g((unsigned)((C + 2 * W - 1) / (2 * W)), (unsigned)((R + 2 * W - 1) / (2 * W)), (unsigned)B);
    if (dt == MOE_BF16)
        transpose_batched<2><<<g, 256, 0, stream>>>((const uint16_t *)src, R, C, seg, (uint16_t *)dst);
    else
        transpose_batched<4><<<g, 256, 0, stream>>>((const uint16_t *)src, R, C, seg, (uint16_t *)dst);
    return check_launch("transpose_batched");
}

moe_status_t launch_gather_t(const void *src, int D, const int32_t *row_src, int k, const float *wgt,
                             const int32_t *seg, int S, int64_t rows, const int32_t *kcol, int64_t Kp, moe_dtype_t dt,
                             void *dstT, void *dst, float *colpart, hipStream_t stream)
{
    const int64_t ctiles = Kp / 64;
    const int fx = (D + 255) / 256;
    const dim3 g((unsigned)fx, strided_grid(ctiles, (4096 + fx - 1) / fx));
    if (dt == MOE_BF16)
        gather_t<uint16_t><<<g, 256, 0, stream>>>((const uint16_t *)src, D, row_src, k, wgt, seg, S, rows, kcol, Kp,
                                                  (uint16_t *)dstT, (uint16_t *)dst, colpart);
    else
        gather_t<float><<<g, 256, 0, stream>>>((const float *)src, D, row_src, k, wgt, seg, S, rows, kcol, Kp,
                                               (float *)dstT, (float *)dst, colpart);
    return check_launch("gather_t");
}

moe_status_t launch_act_bwd(const float *u, const float *dh, int F, const int32_t *row_src, const float *wgt,
                            const int32_t *seg, int S, int64_t rows, const int32_t *kcol, int64_t Kp, moe_dtype_t dt,
                            void *du, void *duT, void *gwT, void *gw, float *dwpart, float *colpart,
                            hipStream_t stream)
{
    const int64_t ctiles = Kp / 64;
    const int FT = (F + 63) / 64;
    const dim3 g((unsigned)FT, strided_grid(ctiles, (32768 + FT - 1) / FT));
    if (dt == MOE_BF16)
        act_bwd<uint16_t><<<g, 256, 0, stream>>>(u, dh, F, FT, row_src, wgt, seg, S, rows, kcol, Kp, (uint16_t *)du,
                                                 (uint16_t *)duT, (uint16_t *)gwT, (uint16_t *)gw, dwpart, colpart);
    else
        act_bwd<float><<<g, 256, 0, stream>>>(u, dh, F, FT, row_src, wgt, seg, S, rows, kcol, Kp, (float *)du,
                                              (float *)duT, (float *)gwT, (float *)gw, dwpart, colpart);
    return check_launch("act_bwd");
}

moe_status_t launch_seg_colsum(const float *colpart, const int32_t *kcol, int S, int D, float *out,
                               hipStream_t stream)
{
    if (!out)
        return MOE_OK;
    seg_colsum<<<dim3((unsigned)((D + 63) / 64), (unsigned)S), 1024, 0, stream>>>(colpart, kcol, D, out);
    return check_launch("seg_colsum");
}

size_t router_bias_ws_bytes(int E) { return align_up((size_t)kBiasChunks * E * sizeof(float)); }

// db_r[e] = sum_t dl[t, e]: chunk partials, then their sum in chunk order.
static moe_status_t launch_router_bias_grad(const float *dl, int64_t T, int E, float *part, float *db_r,
                                            hipStream_t stream)
{
    const int64_t most = (T + 63) / 64;
    const int nch = (int)(most < kBiasChunks ? (most < 1 ? 1 : most) : kBiasChunks);
    const int64_t tc = (T + nch - 1) / nch;
    router_bias_part<<<dim3((unsigned)nch, (unsigned)((E + 63) / 64)), 256, 0, stream>>>(dl, T, E, tc, part);
    if (moe_status_t s = check_launch("router_bias_part"))
        return s;
    router_bias_reduce<<<(unsigned)((E + 63) / 64), 256, 0, stream>>>(part, nch, E, db_r);
    return check_launch("router_bias_reduce");
}

moe_status_t launch_router_bwd(const float *probs, const int32_t *topk_idx, const int32_t *slot_row,
                               const float *dwpart, int FT, const void *b2, const void *dY, moe_dtype_t dt, int d,
                               int e0, const float *f, float c_aux, int64_t T, int E, int k, float *dl,
                               hipStream_t stream)
{
    const unsigned g = (unsigned)((T + 3) / 4);
    if (dt == MOE_BF16)
        router_bwd<uint16_t><<<g, 256, 0, stream>>>(probs, topk_idx, slot_row, dwpart, FT, (const uint16_t *)b2,
                                                    (const uint16_t *)dY, d, e0, f, c_aux, T, E, k, dl,
                                                    nullptr, 0);
    else
        router_bwd<float><<<g, 256, 0, stream>>>(probs, topk_idx, slot_row, dwpart, FT, (const float *)b2,
                                                 (const float *)dY, d, e0, f, c_aux, T, E, k, dl,
                                                 nullptr, 0);
    return check_launch("router_bwd");
}

// Chunks of the router weight-gradient partials: about 2048 blocks in all,
// at least 64 tokens per chunk.
static int router_chunks(int64_t T, int d, int E)
{
    const int64_t cx = (d + 255) / 256, cz = E <= 8 ? 1 : (E <= 16 ? 1 : (E + 31) / 32);
    int64_t n = 2048 / (cx * cz);
    const int64_t most = (T + 63) / 64;
    n = n < 1 ? 1 : (n > most ? most : n);
    return (int)n;
}

size_t router_wgrad_ws_bytes(int64_t T, int d, int E)
{
    return align_up((size_t)router_chunks(T, d, E) * E * d * sizeof(float));
}

moe_status_t launch_router_wgrad(const void *x, moe_dtype_t dt, const float *dl, int64_t T, int d, int E,
                                 float *dw_r, float *db_r, float *bias_part, void *ws, hipStream_t stream)
{
    const int nch = router_chunks(T, d, E);
    const int64_t tc = (T + nch - 1) / nch;
    float *part = (float *)ws;
    const unsigned cx = (unsigned)((d + 255) / 256);
#define MOE_WGRAD(EG)                                                                                               \
    do {                                                                                                            \
        const dim3 g(cx, (unsigned)nch, (unsigned)((E + EG - 1) / EG));                                             \
        if (dt == MOE_BF16)                                                                                         \
            router_wgrad_part<uint16_t, EG><<<g, 256, 0, stream>>>((const uint16_t *)x, dl, T, d, E, tc, part);     \
        else                                                                                                        \
            router_wgrad_part<float, EG><<<g, 256, 0, stream>>>((const float *)x, dl, T, d, E, tc, part);           \
    } while (0)
    if (E <= 8)
        MOE_WGRAD(8);
    else if (E <= 16)
        MOE_WGRAD(16);
    else
        MOE_WGRAD(32);
#undef MOE_WGRAD
    if (moe_status_t s = check_launch("router_wgrad_part"))
        return s;
    const int64_t n = (int64_t)E * d;
    router_wgrad_reduce<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(part, nch, n, dw_r);
    if (moe_status_t s = check_launch("router_wgrad_reduce"))
        return s;
    if (db_r)
        return launch_router_bias_grad(dl, T, E, bias_part, db_r, stream);
    return MOE_OK;
}

moe_status_t launch_dx_combine(const float *dx_rows, const int32_t *slot_row, int k, const float *dx_sh,
                               const float *dx_r, const float *dl, const float *w_r, int64_t T, int d, int E, float *dx,
                               hipStream_t stream)
{
    constexpr int TB = 16;
    const dim3 g((unsigned)((d + 1023) / 1024), (unsigned)((T + TB - 1) / TB));
    // with the router term precomputed (dx_r), the dl . W_r loop is skipped
    dx_combine<TB><<<g, 256, 0, stream>>>(dx_rows, slot_row, k, dx_sh, dx_r, dl, w_r, T, d, dx_r ? 0 : E, dx);
    return check_launch("dx_combine");
}

int router_mfma_chunks(int64_t T, int d, int E)
{
    const int64_t tiles = ((3 * (int64_t)E + 255) / 256) * ((d + 255) / 256);
    int64_t n = (384 + tiles - 1) / tiles;
    const int64_t most = T / 512 > 1 ? T / 512 : 1;
    n = n < 1 ? 1 : (n > most ? most : n);
    return (int)n;
}

size_t router_mfma_ws_bytes(int64_t T, int d, int E)
{
    const int E64 = (E + 63) / 64 * 64;
    const int nc = router_mfma_chunks(T, d, E);
    const int64_t Kp = kseg_cols_bound(T, nc);
    return align_up((size_t)T * 3 * E64 * 2) + align_up((size_t)d * 3 * E64 * 2) + align_up((size_t)T * d * 4) +
           2 * align_up((size_t)(nc + 1) * 4) + align_up((size_t)d * Kp * 2) + align_up((size_t)3 * E * Kp * 2) +
           align_up((size_t)nc * 3 * E * d * 4);
}

moe_status_t launch_router_bwd_mfma(const float *probs, const int32_t *topk_idx, const int32_t *slot_row,
                                    const float *dwpart, int FT, const void *b2, const void *dY, int d, int e0,
                                    const float *f, float c_aux, int64_t T, int E, int k, const void *x,
                                    const float *w_r, float *dl, float *dw_r, float *db_r, float *bias_part,
                                    float **dx_r, void *ws, void *gemm_ws, size_t gemm_ws_bytes, hipStream_t stream)
{
    const int E64 = (E + 63) / 64 * 64;
    const int nc = router_mfma_chunks(T, d, E);
    const int64_t Kp = kseg_cols_bound(T, nc);
    Carver cv{(char *)ws, 0};
    uint16_t *dl2 = cv.take<uint16_t>((size_t)T * 3 * E64);
    uint16_t *w2p = cv.take<uint16_t>((size_t)d * 3 * E64);
    float *dxr = cv.take<float>((size_t)T * d);
    int32_t *seg = cv.take<int32_t>((size_t)nc + 1);
    int32_t *kcol = cv.take<int32_t>((size_t)nc + 1);
    uint16_t *xT = cv.take<uint16_t>((size_t)d * Kp);
    uint16_t *dlT3 = cv.take<uint16_t>((size_t)3 * E * Kp);
    float *part = cv.take<float>((size_t)nc * 3 * E * d);

    router_bwd<uint16_t><<<(unsigned)((T + 3) / 4), 256, 0, stream>>>(
        probs, topk_idx, slot_row, dwpart, FT, (const uint16_t *)b2, (const uint16_t *)dY, d, e0, f, c_aux, T, E, k,
        dl, dl2, E64);
    if (moe_status_t s = check_launch("router_bwd"))
        return s;
    // dx router term: [dl_hi | dl_hi | dl_lo] . [w_hi | w_lo | w_hi]^T
    const int64_t nw = (int64_t)d * E64;
    router_weight_pieces_t<<<(unsigned)((nw + 255) / 256), 256, 0, stream>>>(w_r, E, d, E64, w2p);
    if (moe_status_t s = check_launch("router_weight_pieces_t"))
        return s;
    if (moe_status_t s = launch_grouped_gemm_f32out(dl2, nullptr, 1, T, d, 3 * E64, MOE_BF16, w2p, nullptr, dxr,
                                                    gemm_ws, gemm_ws_bytes, stream))
        return s;
    // dW_r = sum over token ranges of dlT3 . x^T (exact pieces of dl)
    linear_segments<<<1, 64, 0, stream>>>(seg, nc, T);
    if (moe_status_t s = check_launch("linear_segments"))
        return s;
    if (moe_status_t s = launch_kseg_layout(seg, nc, T, kcol, stream))
        return s;
    if (moe_status_t s = launch_gather_t(x, d, nullptr, 1, nullptr, seg, nc, T, kcol, Kp, MOE_BF16, xT, nullptr,
                                         nullptr, stream))
        return s;
    {
        const int ex = (E + 255) / 256;
        const dim3 g((unsigned)ex, strided_grid(Kp / 64, (4096 + ex - 1) / ex));
        dl_pieces_t<<<g, 256, 0, stream>>>(dl, E, seg, nc, T, kcol, Kp, dlT3);
        if (moe_status_t s = check_launch("dl_pieces_t"))
            return s;
    }
    if (moe_status_t s = launch_kseg_gemm(dlT3, xT, kcol, nc, 3 * E, d, Kp, MOE_BF16, part, stream))
        return s;
    const int64_t n = (int64_t)E * d;
    router_wgrad_pieces_reduce<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(part, nc, E, d, dw_r);
    if (moe_status_t s = check_launch("router_wgrad_pieces_reduce"))
        return s;
    if (db_r)
        if (moe_status_t s = launch_router_bias_grad(dl, T, E, bias_part, db_r, stream))
            return s;
    *dx_r = dxr;
    return MOE_OK;
}

} // namespace moe
