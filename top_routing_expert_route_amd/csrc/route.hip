// Router of the MoE layer: logits = x . W_r^T (+ b_r), softmax over the E
// experts, top-k selection and the load statistics f, P, L_aux.
//
// Pages: "Expert Parallelism (MoE)", section "MoE Layer Structure" (router
// Linear d -> N_experts, top-K experts per token, routing weight in Y) and
// section "Load Balancing: The Auxiliary Loss" (f_i, P_i, L_aux = alpha *
// sum f_i P_i).  Optional selection-only bias ("Expert Parallelism (EP)",
// "Key math / How it works", load balancing: DeepSeek-V3's auxiliary-loss-
// free bias adjustment): a per-expert bias added to the logits for the top-k
// choice only; routing weights, P and L_aux use the unbiased softmax.
//
// Kernels
//  route_fused_small  bf16 activations, E <= 64: logits (split-bf16 MFMAs, see
//                     below), softmax, top-k and block partials in one pass.
//  route_split_weight + grouped GEMM
//                     bf16 activations, E > 64: the fp32 router weight is split
//                     exactly into three bf16 pieces (hi + mid + lo = w), stacked
//                     as 3E rows; each piece times a bf16 activation is exact in
//                     fp32, so the bf16 GEMM (fp32 accumulate, fp32 output) gives
//                     three partial logits per expert, summed by route_select.
//  route_logits_mfma  the same split for d % 64 != 0, 64x64 blocks, the four
//                     waves of a block split K and sum in LDS in a fixed order.
//  route_logits_f32   fp32 activations: one thread per (token, expert) fp32
//                     dot product (the small fp32 workloads).
//  route_select       one wave per token: softmax, top-k by (logit desc, id
//                     asc), routing weights, and per-block partial sums of the
//                     probabilities and selection counts.
//  route_reduce_partials / route_finalize
//                     fixed-order sums of the partials (chunks of rows, then
//                     the chunk sums in one block) -> counts, f, P and L_aux
//                     (bitwise reproducible).
#include "common.hpp"

#include <math.h>

namespace moe {

namespace {

constexpr int kSelTokensPerWave = 4;
constexpr int kSelTokensPerBlock = 4 * kSelTokensPerWave;

__device__ __forceinline__ float trunc_bf16(float v) { return __uint_as_float(__float_as_uint(v) & 0xFFFF0000u); }

__device__ __forceinline__ __bf16 bits_bf16(float v)
{
    return __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(v) >> 16));
}

// ET expert tiles and TT token tiles of 16 per block; 4 waves split K.
template <int ET, int TT>
__global__ __launch_bounds__(256) void route_logits_mfma(const uint16_t *__restrict__ x,
                                                         const float *__restrict__ wr, int64_t T, int d,
                                                         int E, float *__restrict__ logits)
{
    constexpr int EB = 16 * ET, TB = 16 * TT;
    __shared__ float red[3][ET * TT * 256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    const int e_base = blockIdx.y * EB;

    // K range of this wave, in steps of 32.
    const int kw = ((d + 3) / 4 + 31) / 32 * 32;
    const int kbeg = wave * kw;
    const int kend = min(d, kbeg + kw);

    f32x4 acc[ET][TT];
#pragma unroll
    for (int a = 0; a < ET; ++a)
#pragma unroll
        for (int b = 0; b < TT; ++b)
            acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int koff = (lane >> 4) * 8;

    for (int k = kbeg; k < kend; k += 32) {
        const int kk = k + koff;
        const bool kval = kk < kend;
        bf16x8 xb[TT];
#pragma unroll
        for (int b = 0; b < TT; ++b) {
            const int64_t t = t0 + b * 16 + r16;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (kval && t < T)
                v = *reinterpret_cast<const u32x4 *>(x + t * d + kk);
            xb[b] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int a = 0; a < ET; ++a) {
            const int e = e_base + a * 16 + r16;
            float wv[8];
            if (kval && e < E) {
                const f32x4 *p = reinterpret_cast<const f32x4 *>(wr + (int64_t)e * d + kk);
                f32x4 w0 = p[0], w1 = p[1];
                wv[0] = w0[0]; wv[1] = w0[1]; wv[2] = w0[2]; wv[3] = w0[3];
                wv[4] = w1[0]; wv[5] = w1[1]; wv[6] = w1[2]; wv[7] = w1[3];
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    wv[q] = 0.f;
            }
            bf16x8 hi, mid, lo;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float h = trunc_bf16(wv[q]);
                const float r1 = wv[q] - h;          // exact
                const float m = trunc_bf16(r1);
                const float r2 = r1 - m;             // exact, <= 8 significant bits
                hi[q] = bits_bf16(h);
                mid[q] = bits_bf16(m);
                lo[q] = bits_bf16(r2);
            }
#pragma unroll
            for (int b = 0; b < TT; ++b) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xb[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, xb[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xb[b], acc[a][b], 0, 0, 0);
            }
        }
    }

    // 16x16 MFMA output: lane holds rows (experts) 4*(lane/16)+v, column
    // (token) lane%16.  Waves 1..3 park their partial tiles; wave 0 adds them
    // in wave order and stores.
    if (wave > 0) {
#pragma unroll
        for (int a = 0; a < ET; ++a)
#pragma unroll
            for (int b = 0; b < TT; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[wave - 1][((a * TT + b) * 4 + v) * 64 + lane] = acc[a][b][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int a = 0; a < ET; ++a)
#pragma unroll
            for (int b = 0; b < TT; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int slot = ((a * TT + b) * 4 + v) * 64 + lane;
                    float s = acc[a][b][v];
                    s += red[0][slot];
                    s += red[1][slot];
                    s += red[2][slot];
                    const int e = e_base + a * 16 + 4 * (lane >> 4) + v;
                    const int64_t t = t0 + b * 16 + (lane & 15);
                    if (e < E && t < T)
                        logits[t * E + e] = s;
                }
    }
}

// Fused router for E <= 64 with bf16 activations: one block scores TB = 16*TT
// tokens against all experts (16*ET >= E) with the split-bf16 MFMAs (the four
// waves split K, U K-steps of loads in flight per wave), parks the logits in
// LDS, then one thread per token does softmax and top-k, and the block
// writes its partial sums of the probabilities and selection counts.
template <int ET, int TT, int U, int NW>
__global__ __launch_bounds__(64 * NW) void route_fused_small(const uint16_t *__restrict__ x,
                                                         const float *__restrict__ wr,
                                                         const float *__restrict__ bias,
                                                         const float *__restrict__ sel, int64_t T, int d, int E,
                                                         int k, int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_w, float *__restrict__ part_p,
                                                         int32_t *__restrict__ part_c, float *__restrict__ probs)
{
    constexpr int EB = 16 * ET, TB = 16 * TT;
    constexpr int LS = EB + 1; // padded LDS row of one token's logits
    __shared__ float red[NW - 1][ET * TT * 256];
    __shared__ float lg[TB * LS];
    __shared__ int cnt[EB];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    const int kw = ((d + NW - 1) / NW + 31) / 32 * 32;
    const int kbeg = wave * kw;
    const int kend = min(d, kbeg + kw);
    const int r16 = lane & 15;
    const int koff = (lane >> 4) * 8;
    if (threadIdx.x < EB)
        cnt[threadIdx.x] = 0;

    f32x4 acc[ET][TT];
#pragma unroll
    for (int a = 0; a < ET; ++a)
#pragma unroll
        for (int b = 0; b < TT; ++b)
            acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = kbeg; k0 < kend; k0 += 32 * U) {
        u32x4 xv[U][TT];
        f32x4 wv[U][ET][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * 32 + koff;
            const bool kval = kk < kend;
#pragma unroll
            for (int b = 0; b < TT; ++b) {
                const int64_t t = t0 + b * 16 + r16;
                xv[u][b] = (kval && t < T) ? *reinterpret_cast<const u32x4 *>(x + t * d + kk) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int a = 0; a < ET; ++a) {
                const int e = a * 16 + r16;
                if (kval && e < E) {
                    const f32x4 *p = reinterpret_cast<const f32x4 *>(wr + (int64_t)e * d + kk);
                    wv[u][a][0] = p[0];
                    wv[u][a][1] = p[1];
                } else {
                    wv[u][a][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    wv[u][a][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int a = 0; a < ET; ++a) {
                bf16x8 hi, mid, lo;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float w = wv[u][a][q >> 2][q & 3];
                    const float h = trunc_bf16(w);
                    const float r1 = w - h;
                    const float m = trunc_bf16(r1);
                    hi[q] = bits_bf16(h);
                    mid[q] = bits_bf16(m);
                    lo[q] = bits_bf16(r1 - m);
                }
#pragma unroll
                for (int b = 0; b < TT; ++b) {
                    const bf16x8 xb = __builtin_bit_cast(bf16x8, xv[u][b]);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xb, acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, xb, acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xb, acc[a][b], 0, 0, 0);
                }
            }
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int a = 0; a < ET; ++a)
#pragma unroll
            for (int b = 0; b < TT; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[wave - 1][((a * TT + b) * 4 + v) * 64 + lane] = acc[a][b][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int a = 0; a < ET; ++a)
#pragma unroll
            for (int b = 0; b < TT; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int slot = ((a * TT + b) * 4 + v) * 64 + lane;
                    float sum = acc[a][b][v];
#pragma unroll
                    for (int q = 0; q < NW - 1; ++q)
                        sum += red[q][slot];
                    const int e = a * 16 + 4 * (lane >> 4) + v;
                    const int tl = b * 16 + (lane & 15);
                    lg[tl * LS + e] = sum;
                }
    }
    __syncthreads();

    // One thread per token: softmax over E, top-k by (logit desc, id asc).
    const int tl = threadIdx.x;
    const int64_t t = t0 + tl;
    if (tl < TB && t < T) {
        float *row = lg + tl * LS;
        float m = -INFINITY;
        for (int e = 0; e < E; ++e) {
            const float l = row[e] + (bias ? bias[e] : 0.f);
            row[e] = l;
            m = fmaxf(m, l);
        }
        float sum = 0.f;
        for (int e = 0; e < E; ++e)
            sum += expf(row[e] - m);
        const float inv = 1.0f / sum;
        // selection score: the logit, plus the selection-only bias if given
        uint64_t taken = 0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            float bv = 0.f;
            for (int e = 0; e < E; ++e) {
                if ((taken >> e) & 1ull)
                    continue;
                const float sc = sel ? row[e] + sel[e] : row[e];
                if (best < 0 || sc > bv) {
                    best = e;
                    bv = sc;
                }
            }
            taken |= 1ull << best;
            topk_idx[t * k + j] = best;
            topk_w[t * k + j] = expf(row[best] - m) * inv;
            atomicAdd(&cnt[best], 1);
        }
        for (int e = 0; e < E; ++e)
            row[e] = expf(row[e] - m) * inv;
    } else if (tl < TB) {
        float *row = lg + tl * LS;
        for (int e = 0; e < E; ++e)
            row[e] = 0.f;
    }
    __syncthreads();
    if (probs) {
        for (int q = threadIdx.x; q < TB * E; q += 64 * NW) {
            const int tq = q / E, e = q - tq * E;
            if (t0 + tq < T)
                probs[(t0 + tq) * E + e] = lg[tq * LS + e];
        }
    }
    // Block partials: probabilities summed in token order.
    if (threadIdx.x < E) {
        const int e = threadIdx.x;
        float ps = 0.f;
        for (int q = 0; q < TB; ++q)
            ps += lg[q * LS + e];
        part_p[(int64_t)blockIdx.x * E + e] = ps;
        part_c[(int64_t)blockIdx.x * E + e] = cnt[e];
    }
}

// w3[p*E + e, i] = bf16 piece p of w_router[e, i]: hi = w truncated to bf16,
// mid = (w - hi) truncated, lo = w - hi - mid (exact: at most 8 significant
// bits remain); hi + mid + lo = w.  n = E * d.
__global__ __launch_bounds__(256) void route_split_weight(const float *__restrict__ wr, int64_t n,
                                                          uint16_t *__restrict__ w3)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float w = wr[i];
    const float h = trunc_bf16(w);
    const float r1 = w - h;
    const float m = trunc_bf16(r1);
    const float l = r1 - m;
    w3[i] = (uint16_t)(__float_as_uint(h) >> 16);
    w3[n + i] = (uint16_t)(__float_as_uint(m) >> 16);
    w3[2 * n + i] = (uint16_t)(__float_as_uint(l) >> 16);
}

__global__ __launch_bounds__(256) void route_logits_f32(const float *__restrict__ x, const float *__restrict__ wr,
                                                        int64_t T, int d, int E, float *__restrict__ logits)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * E)
        return;
    const int64_t t = i / E;
    const int e = (int)(i % E);
    const f32x4 *xr = reinterpret_cast<const f32x4 *>(x + t * d);
    const f32x4 *wv = reinterpret_cast<const f32x4 *>(wr + (int64_t)e * d);
    float s = 0.f;
    for (int q = 0; q < d / 4; ++q) {
        const f32x4 a = xr[q], b = wv[q];
        s = fmaf(a[0], b[0], s);
        s = fmaf(a[1], b[1], s);
        s = fmaf(a[2], b[2], s);
        s = fmaf(a[3], b[3], s);
    }
    logits[i] = s;
}

// EPL = experts held per lane (ceil(E / 64)).  pieces = 3: row t of
// `logits` holds three column blocks of E (hi, mid, lo router pieces) whose
// sum (mid + lo) + hi is the logit; pieces = 1: plain [T, E] logits.
template <int EPL>
__global__ __launch_bounds__(256) void route_select(const float *__restrict__ logits, int pieces,
                                                    const float *__restrict__ bias, const float *__restrict__ sel,
                                                    int64_t T, int E, int k,
                                                    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                                                    float *__restrict__ part_p, int32_t *__restrict__ part_c,
                                                    float *__restrict__ probs)
{
    __shared__ float sp[4][EPL * 64];
    __shared__ int sc[4][EPL * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    float pacc[EPL];
    int cacc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        pacc[i] = 0.f;
        cacc[i] = 0;
    }

    const int64_t tw0 = ((int64_t)blockIdx.x * 4 + wave) * kSelTokensPerWave;
    for (int q = 0; q < kSelTokensPerWave; ++q) {
        const int64_t t = tw0 + q;
        if (t >= T)
            break;
        float l[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            l[i] = -INFINITY;
            if (e < E) {
                const float *row = logits + t * (int64_t)(pieces * E);
                const float v = pieces == 3 ? row[e] + (row[E + e] + row[2 * E + e]) : row[e];
                l[i] = v + (bias ? bias[e] : 0.f);
            }
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            m = fmaxf(m, l[i]);
        m = wave_max(m);
        float ex[EPL];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            ex[i] = (lane + 64 * i < E) ? expf(l[i] - m) : 0.f;
            s += ex[i];
        }
        s = wave_sum(s);
        const float inv_s = 1.0f / s;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            pacc[i] += ex[i] * inv_s;
        if (probs) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (lane + 64 * i < E)
                    probs[t * E + lane + 64 * i] = ex[i] * inv_s;
        }

        // top-k: k rounds of a wave arg-max on (score desc, id asc); the
        // score is the logit, plus the selection-only bias if given
        float sv[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            sv[i] = (sel && e < E) ? l[i] + sel[e] : l[i];
        }
        // each round: the largest untaken score (wave max), then the lowest
        // expert id holding it (ballots; expert lane + 64 i, so slot order
        // is id order)
        uint32_t taken = 0;
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (e < E && !((taken >> i) & 1u))
                    bv = fmaxf(bv, sv[i]);
            }
            const float m = wave_max(bv);
            int bi = -1, first = -1;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const bool free_e = lane + 64 * i < E && !((taken >> i) & 1u);
                const uint64_t hit = __ballot(free_e && sv[i] == m);
                const uint64_t any = __ballot(free_e);
                if (bi < 0 && hit != 0ull)
                    bi = (int)__builtin_ctzll(hit) + 64 * i;
                if (first < 0 && any != 0ull)
                    first = (int)__builtin_ctzll(any) + 64 * i;
            }
            if (bi < 0)
                bi = first; // only NaN scores left: the lowest untaken id
            if ((bi & 63) == lane) {
                const int slot = bi >> 6;
#pragma unroll
                for (int i = 0; i < EPL; ++i)
                    if (i == slot) {
                        taken |= 1u << i;
                        cacc[i] += 1;
                        topk_idx[t * k + j] = bi;
                        topk_w[t * k + j] = ex[i] * inv_s;
                    }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        sp[wave][lane + 64 * i] = pacc[i];
        sc[wave][lane + 64 * i] = cacc[i];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        float p = sp[0][e];
        p += sp[1][e];
        p += sp[2][e];
        p += sp[3][e];
        part_p[(int64_t)blockIdx.x * E + e] = p;
        part_c[(int64_t)blockIdx.x * E + e] = sc[0][e] + sc[1][e] + sc[2][e] + sc[3][e];
    }
}

// First level of the partial-sum reduction: chunk c (one block) sums rows
// [c R, (c+1) R) of the per-block partials, in row order, for every expert.
constexpr int kFinRows = 32;

__global__ __launch_bounds__(256) void route_reduce_partials(const float *__restrict__ part_p,
                                                             const int32_t *__restrict__ part_c, int nblk, int E,
                                                             double *__restrict__ fin_p, long long *__restrict__ fin_c)
{
    const int c = blockIdx.x;
    const int r0 = c * kFinRows, r1 = min(nblk, r0 + kFinRows);
    for (int e = threadIdx.x; e < E; e += 256) {
        double ps = 0.0;
        long long cs = 0;
        for (int r = r0; r < r1; ++r) {
            ps += (double)part_p[(int64_t)r * E + e];
            cs += part_c[(int64_t)r * E + e];
        }
        fin_p[(int64_t)c * E + e] = ps;
        fin_c[(int64_t)c * E + e] = cs;
    }
}

// One block of 1024 threads; G threads per expert sum the chunk sums in a
// fixed strided order, then the G partial sums are added in order.  DIRECT:
// the rows are the per-block partials themselves (few blocks: one launch
// instead of two).
__host__ __device__ constexpr int finalize_threads_per_expert(int E)
{
    int G = 1;
    while (G * 2 * E <= 1024)
        G *= 2;
    return G;
}

template <bool DIRECT, class TP, class TC>
__global__ __launch_bounds__(1024) void route_finalize(const TP *__restrict__ fin_p, const TC *__restrict__ fin_c,
                                                       int nrows, int64_t T, int E, float alpha,
                                                       int32_t *__restrict__ expert_count, float *__restrict__ f,
                                                       float *__restrict__ P, float *__restrict__ l_aux)
{
    __shared__ double rp[1024];
    __shared__ long long rc[1024];
    __shared__ double terms[1024];
    const int G = finalize_threads_per_expert(E);
    const int tid = threadIdx.x;
    const int e = tid / G, g = tid % G;
    double ps = 0.0;
    long long cs = 0;
    if (e < E) {
        for (int b = g; b < nrows; b += G) {
            ps += (double)fin_p[(int64_t)b * E + e];
            cs += (long long)fin_c[(int64_t)b * E + e];
        }
    }
    rp[tid] = ps;
    rc[tid] = cs;
    __syncthreads();
    if (tid < E) {
        double p = 0.0;
        long long c = 0;
        for (int q = 0; q < G; ++q) {
            p += rp[tid * G + q];
            c += rc[tid * G + q];
        }
        const float fe = T > 0 ? (float)c / (float)T : 0.f;
        const float Pe = T > 0 ? (float)(p / (double)T) : 0.f;
        if (expert_count)
            expert_count[tid] = (int32_t)c;
        if (f)
            f[tid] = fe;
        if (P)
            P[tid] = Pe;
        terms[tid] = (double)fe * (double)Pe;
    }
    __syncthreads();
    if (tid == 0 && l_aux) {
        double s = 0.0;
        for (int q = 0; q < E; ++q)
            s += terms[q];
        l_aux[0] = (float)((double)alpha * s);
    }
}

} // namespace

static int fin_chunks(int nblk) { return (nblk + kFinRows - 1) / kFinRows; }

static int select_blocks(int64_t T) { return (int)((T + kSelTokensPerBlock - 1) / kSelTokensPerBlock); }

// Tokens per block of the fused small-E path.
static int fused_tb(int E) { return E <= 16 ? 16 : 32; }

static int route_blocks(int64_t T, int E, moe_dtype_t dt)
{
    if (dt == MOE_BF16 && E <= 64)
        return (int)((T + fused_tb(E) - 1) / fused_tb(E));
    return select_blocks(T);
}

// The grouped GEMM needs K % 64 == 0 and at least two K steps (d >= 128),
// and rows of whole 16-byte groups in its output (3E % 4 == 0; E % 8 == 0
// keeps the three column blocks 32-byte aligned).
static bool router_on_gemm(moe_dtype_t dt, int d, int E)
{
    return dt == MOE_BF16 && E > 64 && E % 8 == 0 && d % 64 == 0 && d >= 128;
}

size_t route_ws_bytes(int64_t T, int d, int E)
{
    // logits (two-kernel paths) + partials of the larger block count, plus the
    // split router weight and the grouped GEMM's tail partials for large E
    const int nblk = (int)((T + 15) / 16);
    const bool split = E > 64 && d % 64 == 0;
    size_t b = align_up((size_t)T * E * (split ? 3 : 1) * sizeof(float)) +
               2 * align_up((size_t)nblk * E * sizeof(float)) + 2 * align_up((size_t)fin_chunks(nblk) * E * 8);
    if (split)
        b += align_up((size_t)E * 3 * d * sizeof(uint16_t)) + align_up(gemm_ws_bytes());
    return b;
}

moe_status_t launch_route(const void *x, moe_dtype_t dt, const float *w_router, const float *b_router,
                          const float *sel_bias, int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx,
                          float *topk_w,
                          int32_t *expert_count, float *f, float *P, float *l_aux, float *probs, void *ws,
                          hipStream_t stream)
{
    const int nblk = route_blocks(T, E, dt);
    const int nblk_max = (int)((T + 15) / 16);
    Carver cv{(char *)ws, 0};
    const bool on_gemm = router_on_gemm(dt, d, E);
    const int pieces = on_gemm ? 3 : 1;
    float *logits = cv.take<float>((size_t)T * E * pieces);
    float *part_p = cv.take<float>((size_t)nblk_max * E);
    int32_t *part_c = cv.take<int32_t>((size_t)nblk_max * E);
    double *fin_p = cv.take<double>((size_t)fin_chunks(nblk_max) * E);
    long long *fin_c = cv.take<long long>((size_t)fin_chunks(nblk_max) * E);
    uint16_t *w3 = on_gemm ? cv.take<uint16_t>((size_t)E * 3 * d) : nullptr;
    void *gws = on_gemm ? cv.take<char>(gemm_ws_bytes()) : nullptr;

    if (T > 0) {
        if (dt == MOE_BF16 && E <= 64) {
            const uint16_t *xb = (const uint16_t *)x;
            const dim3 g((unsigned)nblk);
            if (E <= 16)
                route_fused_small<1, 1, 8, 8><<<g, 512, 0, stream>>>(xb, w_router, b_router, sel_bias, T, d, E, k, topk_idx,
                                                                  topk_w, part_p, part_c, probs);
            else if (E <= 32)
                route_fused_small<2, 2, 4, 8><<<g, 512, 0, stream>>>(xb, w_router, b_router, sel_bias, T, d, E, k, topk_idx,
                                                                  topk_w, part_p, part_c, probs);
            else
                route_fused_small<4, 2, 2, 8><<<g, 512, 0, stream>>>(xb, w_router, b_router, sel_bias, T, d, E, k, topk_idx,
                                                                  topk_w, part_p, part_c, probs);
            if (moe_status_t s = check_launch("route_fused_small"))
                return s;
        } else {
            if (on_gemm) {
                const int64_t n = (int64_t)E * d;
                route_split_weight<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(w_router, n, w3);
                if (moe_status_t s = check_launch("route_split_weight"))
                    return s;
                if (moe_status_t s = launch_router_gemm(x, w3, T, d, E, logits, gws, gemm_ws_bytes(), stream))
                    return s;
            } else if (dt == MOE_BF16) {
                dim3 g((unsigned)((T + 63) / 64), (unsigned)((E + 63) / 64));
                route_logits_mfma<4, 4><<<g, 256, 0, stream>>>((const uint16_t *)x, w_router, T, d, E, logits);
            } else {
                const int64_t n = T * E;
                route_logits_f32<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>((const float *)x, w_router, T, d,
                                                                                 E, logits);
            }
            if (moe_status_t s = check_launch("route_logits"))
                return s;
            const int epl = (E + 63) / 64;
            const dim3 g((unsigned)nblk);
            switch (epl) {
            case 1: route_select<1><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs); break;
            case 2: route_select<2><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs); break;
            case 3:
            case 4: route_select<4><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs); break;
            case 5: case 6: case 7: case 8:
                route_select<8><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs); break;
            default:
                route_select<16><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs); break;
            }
            if (moe_status_t s = check_launch("route_select"))
                return s;
        }
    }
    const int rows = T > 0 ? nblk : 0;
    if (rows <= 32 * finalize_threads_per_expert(E)) {
        // at most 32 partial rows per thread: sum them directly
        route_finalize<true><<<1, 1024, 0, stream>>>(part_p, part_c, rows, T, E, alpha, expert_count, f, P, l_aux);
        return check_launch("route_finalize");
    }
    const int nfin = fin_chunks(nblk);
    route_reduce_partials<<<(unsigned)nfin, 256, 0, stream>>>(part_p, part_c, nblk, E, fin_p, fin_c);
    if (moe_status_t s = check_launch("route_reduce_partials"))
        return s;
    route_finalize<false><<<1, 1024, 0, stream>>>(fin_p, fin_c, nfin, T, E, alpha, expert_count, f, P, l_aux);
    return check_launch("route_finalize");
}

} // namespace moe
