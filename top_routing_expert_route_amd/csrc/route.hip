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
//  route_fused        bf16 activations, E <= 64: logits (split-bf16 MFMAs, see
//                     the kernel), softmax, top-k, block partials and, in the
//                     last block to finish, the statistics: one launch.
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
//                     probabilities and selection counts, summed in a fixed
//                     order by the last blocks to finish (in groups of blocks,
//                     then over the groups, as in route_fused) -> counts, f, P
//                     and L_aux (bitwise reproducible).
//  route_finalize     T = 0: zero counts and statistics.
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

// ----------------------------------------------------------------------------
// Single-launch router for bf16 activations and E <= 64 experts.
//
// One block of eight waves scores TT tiles of kRouteTB = 16 tokens (TT = 1, 2
// or 4, chosen from T so that the grid still covers the chip: every block
// reads and splits the whole router weight, so fewer, larger blocks do less of
// that).  The eight waves split the hidden dimension; per 32-wide K step a
// wave runs v_mfma_f32_16x16x32_bf16 with the weight rows as the A operand (16
// experts per row tile, ET tiles) and each token tile as the B operand, the
// weight split once for all TT tiles.  The fp32 router weight is split on the fly,
// exactly, into three bf16 pieces (hi = w truncated to bf16, mid = (w - hi)
// truncated, lo = w - hi - mid, at most 8 significant bits), each product with
// a bf16 activation is exact in fp32, and the three MFMAs accumulate into the
// same fp32 tile: fp32-class logits at matrix-core rate.  Loads are raw buffer
// loads whose range check returns zeros for rows past T, experts past E and K
// past the wave's range (no branches), two chunks of CH steps in flight per
// wave, so a block keeps its whole share of x streaming while the weight
// pieces are split.
//
// The waves' partial logits are summed in wave order through LDS; softmax and
// top-k then run lane-parallel, G lanes per token (G = 8, 16, 32 or 64 >= E):
// group max and sum with butterfly shuffles (every lane of a group ends with
// the same bits), and each top-k round is a group maximum of a 64-bit key
// (order-preserving score bits, then the complement of the expert id), so the
// winner is the largest score and, on ties, the lowest id.  Each block writes
// its selection counts and its probability sums (token order) as one partial
// row (coherent agent-scope stores); the last block to arrive (an
// agent-scope ticket, counted after the block's stores completed) sums the
// partial rows in a fixed order and writes counts, f, P and L_aux, then
// resets the ticket to zero for the next call.
// ----------------------------------------------------------------------------
constexpr int kRouteWaves = 8;
constexpr int kRouteTB = 16;

template <int G> __device__ __forceinline__ float grp_max(float v)
{
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <int G> __device__ __forceinline__ float grp_sum(float v)
{
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

template <int G> __device__ __forceinline__ uint64_t grp_max_u64(uint64_t v)
{
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) {
        const uint64_t u = __shfl_xor(v, o, 64);
        v = u > v ? u : v;
    }
    return v;
}

// Unsigned key with the order of the float scores: NaN below every number,
// -0 equal to +0; 0 is left for "not a candidate".
__device__ __forceinline__ uint32_t order_key(float s)
{
    if (s != s)
        return 1u;
    const uint32_t b = __float_as_uint(s + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// Cross-block publication without cache maintenance: the partial rows are
// written and read with relaxed agent-scope atomic accesses (coherent across
// the XCDs' L2s), and each writer waits for its stores to complete before
// the block's arrival is counted, so the last block to arrive sees every
// row.  (An agent-scope fence would write back and invalidate the whole L2
// in every wave.)
template <class V> __device__ __forceinline__ void publish(V *p, V v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class V> __device__ __forceinline__ V collect(const V *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fixed-order sums of partial rows [r0, r1) (E values each): G2 threads per
// expert take rows r0 + g, r0 + g + G2, ... (four at a time, so that their
// coherent loads are in flight together) in double and int64, then thread e
// adds its G2 sums in order into sp[e], sc[e] (rp, rc: G2 x E <= blockDim.x
// entries).  With more than half as many experts as threads, each thread
// sums whole rows for experts tid, tid + blockDim.x, ... (the same order as
// G2 = 1).  Every thread sees sp and sc after the call.
template <class TP, class TC>
__device__ __forceinline__ void sum_rows(const TP *pp, const TC *pc, int64_t r0, int64_t r1, int E, double *rp, long long *rc,
                         double *sp, long long *sc)
{
    const int nt = blockDim.x, tid = threadIdx.x;
    int G2 = 1;
    while (G2 * 2 * E <= nt)
        G2 *= 2;
    if (G2 == 1) {
        for (int q = tid; q < E; q += nt) {
            double ps = 0.0;
            long long cs = 0;
            int64_t b = r0;
            for (; b + 3 < r1; b += 4) {
                TP pv[4];
                TC cv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    pv[u] = collect(pp + (b + u) * E + q);
                    cv[u] = collect(pc + (b + u) * E + q);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ps += (double)pv[u];
                    cs += (long long)cv[u];
                }
            }
            for (; b < r1; ++b) {
                ps += (double)collect(pp + b * E + q);
                cs += (long long)collect(pc + b * E + q);
            }
            sp[q] = ps;
            sc[q] = cs;
        }
        __syncthreads();
        return;
    }
    const int e = tid / G2, g = tid % G2;
    double ps = 0.0;
    long long cs = 0;
    if (e < E) {
        int64_t b = r0 + g;
        for (; b + 3 * G2 < r1; b += 4 * G2) {
            TP pv[4];
            TC cv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pv[u] = collect(pp + (b + u * G2) * E + e);
                cv[u] = collect(pc + (b + u * G2) * E + e);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ps += (double)pv[u];
                cs += (long long)cv[u];
            }
        }
        for (; b < r1; b += G2) {
            ps += (double)collect(pp + b * E + e);
            cs += (long long)collect(pc + b * E + e);
        }
    }
    if (tid < G2 * E) {
        rp[tid] = ps;
        rc[tid] = cs;
    }
    __syncthreads();
    for (int q = tid; q < E; q += nt) {
        double p = 0.0;
        long long c = 0;
        for (int i = 0; i < G2; ++i) {
            p += rp[q * G2 + i];
            c += rc[q * G2 + i];
        }
        sp[q] = p;
        sc[q] = c;
    }
    __syncthreads();
}

// True in every thread of the block whose increment of `counter` is the n-th
// (the last of n arrivals); that block also resets the counter to zero.  Call
// after the block's published stores were issued (every thread): each thread
// waits for its stores to complete before the block arrives.
__device__ __forceinline__ bool arrived_last(unsigned *counter, unsigned n, int *s_flag)
{
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); // this thread's published stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == n - 1;
        if (last)
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last ? 1 : 0;
    }
    __syncthreads();
    return *s_flag != 0;
}

// Statistics from the blocks' partial rows, in two fixed-order levels: the
// blocks form groups of gsz consecutive blocks; the last block of a group to
// arrive (counter 1 + group) sums the group's rows and publishes a group row
// (double, int64); the last group to finish (counter 0) sums the group rows
// in group order and writes counts, f, P and L_aux.  Each collecting block
// reads gsz or ngroups rows instead of one block reading every row.  With one
// group the last block sums the rows directly.  Every counter is back at zero
// when the launch completes.
__device__ __forceinline__ void finish_stats(const float *part_p, const int32_t *part_c, int gsz, double *grp_p, long long *grp_c,
                             unsigned *counters, int64_t T, int E, float alpha, int32_t *expert_count, float *f,
                             float *P, float *l_aux, double *rp, long long *rc, double *sp, long long *sc,
                             double *terms, int *s_flag)
{
    const int nb = (int)gridDim.x, tid = threadIdx.x, nt = blockDim.x;
    const int ng = (nb + gsz - 1) / gsz;
    if (ng > 1) {
        const int g = (int)blockIdx.x / gsz;
        const int r0 = g * gsz, r1 = min(nb, r0 + gsz);
        if (!arrived_last(counters + 1 + g, (unsigned)(r1 - r0), s_flag))
            return;
        sum_rows(part_p, part_c, r0, r1, E, rp, rc, sp, sc);
        for (int q = tid; q < E; q += nt) {
            publish(grp_p + (int64_t)g * E + q, sp[q]);
            publish(grp_c + (int64_t)g * E + q, sc[q]);
        }
        if (!arrived_last(counters, (unsigned)ng, s_flag))
            return;
        sum_rows(grp_p, grp_c, 0, ng, E, rp, rc, sp, sc);
    } else {
        if (!arrived_last(counters, (unsigned)nb, s_flag))
            return;
        sum_rows(part_p, part_c, 0, nb, E, rp, rc, sp, sc);
    }
    for (int q = tid; q < E; q += nt) {
        const long long c = sc[q];
        const float fe = T > 0 ? (float)c / (float)T : 0.f;
        const float Pe = T > 0 ? (float)(sp[q] / (double)T) : 0.f;
        if (expert_count)
            expert_count[q] = (int32_t)c;
        if (f)
            f[q] = fe;
        if (P)
            P[q] = Pe;
        terms[q] = (double)fe * (double)Pe;
    }
    __syncthreads();
    if (tid == 0 && l_aux) {
        double s = 0.0;
        for (int q = 0; q < E; ++q)
            s += terms[q];
        l_aux[0] = (float)((double)alpha * s);
    }
}

template <int ET, int TT, int CH, int G>
__global__ __launch_bounds__(64 * kRouteWaves) void route_fused(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    const float *__restrict__ sel, int64_t T, int d, int E, int k, float alpha, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ probs, float *__restrict__ part_p, int32_t *__restrict__ part_c,
    int gsz, double *__restrict__ grp_p, long long *__restrict__ grp_c, unsigned *__restrict__ counters,
    int32_t *__restrict__ expert_count, float *__restrict__ f, float *__restrict__ P, float *__restrict__ l_aux)
{
    constexpr int EB = 16 * ET;
    constexpr int LS = EB + 1;
    constexpr int TB = kRouteTB * TT;
    __shared__ float red[kRouteWaves][ET][4][64];
    __shared__ float lg[TB][LS];
    __shared__ int cnt[EB];
    __shared__ int s_flag;
    __shared__ double rp[64 * kRouteWaves];
    __shared__ long long rc[64 * kRouteWaves];
    __shared__ double sp[64], terms[64];
    __shared__ long long sc[64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    if (tid < EB)
        cnt[tid] = 0;

    // K range of this wave, in steps of 32
    const int kw = ((d + kRouteWaves - 1) / kRouteWaves + 31) / 32 * 32;
    const int kbeg = wave * kw;
    const int kend = min(d, kbeg + kw);
    const int nsteps = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;
    const int nch = (nsteps + CH - 1) / CH;

    // token rows of the block and the router weight as range-checked records
    const int64_t trows = min((int64_t)TB, T - t0);
    const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x + t0 * d, (uint32_t)(trows * d * 2));
    const __amdgpu_buffer_rsrc_t wrr = raw_rsrc(wr, (uint32_t)((int64_t)E * d * 4));
    const uint32_t xoff0 = (uint32_t)(n * d * 2);
    uint32_t woff0[ET];
#pragma unroll
    for (int a = 0; a < ET; ++a) {
        const int e = 16 * a + n;
        woff0[a] = e < E ? (uint32_t)(e * d * 4) : kOutOfRange;
    }

    f32x4 acc[ET][TT];
#pragma unroll
    for (int a = 0; a < ET; ++a)
#pragma unroll
        for (int u = 0; u < TT; ++u)
            acc[a][u] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Offsets are made opaque before the loads (empty asm on the register):
    // otherwise the compiler may turn the out-of-range select into divergent
    // branches around duplicated loads and drain the load counter there.
    auto load = [&](int c, u32x4 (&xv)[CH][TT], f32x4 (&wv)[CH][ET][2]) {
#pragma unroll
        for (int s = 0; s < CH; ++s) {
            const int kk = kbeg + (c * CH + s) * 32 + 8 * g;
            const bool ok = kk < kend;
#pragma unroll
            for (int u = 0; u < TT; ++u) {
                uint32_t xo = ok ? xoff0 + (uint32_t)(16 * u * d + kk) * 2u : kOutOfRange;
                asm volatile("" : "+v"(xo));
                xv[s][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 0, 0));
            }
#pragma unroll
            for (int a = 0; a < ET; ++a) {
                uint32_t o0 = (ok && woff0[a] != kOutOfRange) ? woff0[a] + (uint32_t)kk * 4u : kOutOfRange;
                uint32_t o1 = o0 == kOutOfRange ? o0 : o0 + 16u;
                asm volatile("" : "+v"(o0), "+v"(o1));
                wv[s][a][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(wrr, o0, 0, 0));
                wv[s][a][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(wrr, o1, 0, 0));
            }
        }
    };
    auto compute = [&](const u32x4 (&xv)[CH][TT], const f32x4 (&wv)[CH][ET][2]) {
#pragma unroll
        for (int s = 0; s < CH; ++s) {
#pragma unroll
            for (int a = 0; a < ET; ++a) {
                bf16x8 hi, mid, lo;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float w = wv[s][a][q >> 2][q & 3];
                    const float h = trunc_bf16(w);
                    const float r1 = w - h;           // exact
                    const float m = trunc_bf16(r1);
                    hi[q] = bits_bf16(h);
                    mid[q] = bits_bf16(m);
                    lo[q] = bits_bf16(r1 - m);        // exact, <= 8 significant bits
                }
#pragma unroll
                for (int u = 0; u < TT; ++u) {
                    const bf16x8 xb = __builtin_bit_cast(bf16x8, xv[s][u]);
                    acc[a][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xb, acc[a][u], 0, 0, 0);
                    acc[a][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, xb, acc[a][u], 0, 0, 0);
                    acc[a][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xb, acc[a][u], 0, 0, 0);
                }
            }
        }
    };

    {
        // two register chunks in flight; a chunk past the wave's range loads
        // nothing (every offset out of range) and adds zeros
        u32x4 xa[CH][TT], xb2[CH][TT];
        f32x4 wa[CH][ET][2], wb[CH][ET][2];
        load(0, xa, wa);
        for (int c = 0; c < nch; c += 2) {
            load(c + 1, xb2, wb);
            __builtin_amdgcn_sched_barrier(0); // issue the next chunk's loads before this chunk's waits
            compute(xa, wa);
            __builtin_amdgcn_sched_barrier(0);
            load(c + 2, xa, wa);
            __builtin_amdgcn_sched_barrier(0);
            compute(xb2, wb);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // partial tiles, one token tile at a time: lane holds experts 16a + 4g + v
    // of token 16u + n
#pragma unroll
    for (int u = 0; u < TT; ++u) {
#pragma unroll
        for (int a = 0; a < ET; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wave][a][v][lane] = acc[a][u][v];
        __syncthreads();
        for (int q = tid; q < ET * 256; q += 64 * kRouteWaves) {
            const int a = q >> 8, v = (q >> 6) & 3, l = q & 63;
            float sum = red[0][a][v][l];
#pragma unroll
            for (int w = 1; w < kRouteWaves; ++w)
                sum += red[w][a][v][l];
            const int e = 16 * a + 4 * (l >> 4) + v;
            if (e < E)
                lg[16 * u + (l & 15)][e] = sum + (bias ? bias[e] : 0.f);
        }
        __syncthreads();
    }

    // softmax and top-k: G lanes per token
    for (int base = 0; base < TB * G; base += 64 * kRouteWaves) {
        if ((base + wave * 64) / G >= TB)
            break; // wave-uniform: no token left for this wave
        const int idx = base + tid;
        const int tl = idx / G, e = idx % G;
        const bool ev = e < E;
        const int64_t t = t0 + tl;
        const bool tv = t < T;
        const float l = ev ? lg[tl][e] : -INFINITY;
        const float m = grp_max<G>(l);
        const float ex = ev ? expf(l - m) : 0.f;
        const float ssum = grp_sum<G>(ex);
        const float p = ex * (1.0f / ssum);
        const float sc = (ev && sel) ? l + sel[e] : l;
        const uint64_t mine = ((uint64_t)(ev ? order_key(sc) : 0u) << 32) | (uint64_t)(uint32_t)~(uint32_t)e;
        bool taken = false;
        for (int j = 0; j < k; ++j) {
            const uint64_t best = grp_max_u64<G>(taken || !ev ? 0ull : mine);
            const int be = (int)~(uint32_t)best;
            if (e == be) {
                taken = true;
                if (tv) {
                    topk_idx[t * k + j] = e;
                    topk_w[t * k + j] = p;
                    atomicAdd(&cnt[e], 1);
                }
            }
        }
        if (ev) {
            if (tv && probs)
                probs[t * E + e] = p;
            lg[tl][e] = tv ? p : 0.f;
        }
    }
    __syncthreads();

    // this block's partial row: counts, probabilities summed in token order
    for (int e = tid; e < E; e += 64 * kRouteWaves) {
        float ps = 0.f;
        for (int q = 0; q < TB; ++q)
            ps += lg[q][e];
        publish(part_p + (int64_t)blockIdx.x * E + e, ps);
        publish(part_c + (int64_t)blockIdx.x * E + e, (int32_t)cnt[e]);
    }
    finish_stats(part_p, part_c, gsz, grp_p, grp_c, counters, T, E, alpha, expert_count, f, P, l_aux, rp, rc, sp, sc,
                 terms, &s_flag);
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
                                                    float *__restrict__ probs, int gsz, double *__restrict__ grp_p,
                                                    long long *__restrict__ grp_c, unsigned *__restrict__ counters,
                                                    float alpha, int32_t *__restrict__ expert_count,
                                                    float *__restrict__ f, float *__restrict__ P,
                                                    float *__restrict__ l_aux)
{
    __shared__ float sp[4][EPL * 64];
    __shared__ int sc[4][EPL * 64];
    __shared__ double rp[256], tp[EPL * 64], terms[EPL * 64]; // statistics: E <= 64 EPL
    __shared__ long long rc[256], tc[EPL * 64];
    __shared__ int s_flag;
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
        publish(part_p + (int64_t)blockIdx.x * E + e, p);
        publish(part_c + (int64_t)blockIdx.x * E + e, sc[0][e] + sc[1][e] + sc[2][e] + sc[3][e]);
    }
    finish_stats(part_p, part_c, gsz, grp_p, grp_c, counters, T, E, alpha, expert_count, f, P, l_aux, rp, rc, tp, tc,
                 terms, &s_flag);
}

// One block of 1024 threads; G threads per expert sum the rows in a fixed
// strided order, then the G partial sums are added in order.  Used for T = 0
// (no rows: zero counts and statistics).
__host__ __device__ constexpr int finalize_threads_per_expert(int E)
{
    int G = 1;
    while (G * 2 * E <= 1024)
        G *= 2;
    return G;
}

template <class TP, class TC>
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

static int select_blocks(int64_t T) { return (int)((T + kSelTokensPerBlock - 1) / kSelTokensPerBlock); }

// Tokens per block of the fused small-E path.
// Path of the router: the single-launch kernel for bf16 activations with at
// most 64 experts, otherwise logits (split-weight grouped GEMM, MFMA or fp32
// kernel) + route_select (which also sums the statistics).
static bool route_is_fused(moe_dtype_t dt, int E) { return dt == MOE_BF16 && E <= 64; }

// Token tiles of 16 per block of the single-launch router.  Every block reads
// and splits the whole fp32 router weight, and one block fills a CU (its
// registers), so a block scores the fewest tiles that keep the grid within one
// block per CU (a second round of blocks would double the time): on 256 CUs,
// 16 tokens up to 4096, 32 up to 8192, else 64.
static int route_tt(int64_t T)
{
    const int64_t cus = device_cus();
    if (T <= cus * kRouteTB)
        return 1;
    return T <= cus * 2 * kRouteTB ? 2 : 4;
}

// Blocks per group of the single-launch router's two-level statistics: about
// sqrt(blocks), so that a group's collection and the final one are about as
// long, with at most 63 groups (the workspace's counters 1..63).  Below 8192
// partial values (blocks x E) one group: the last block's collection is short
// enough that a second arrival round would cost more than it saves.
static int route_group_size(int nblk, int E)
{
    if ((int64_t)nblk * E < 8192)
        return nblk;
    int g = (int)ceil(sqrt((double)nblk));
    if ((nblk + g - 1) / g > 63)
        g = (nblk + 62) / 63;
    return g;
}

static int route_blocks(int64_t T, int E, moe_dtype_t dt)
{
    if (route_is_fused(dt, E)) {
        const int tb = kRouteTB * route_tt(T);
        return (int)((T + tb - 1) / tb);
    }
    return select_blocks(T);
}

// The grouped GEMM needs K % 64 == 0 and at least two K steps (d >= 128),
// and rows of whole 16-byte groups in its output (3E % 4 == 0; E % 8 == 0
// keeps the three column blocks 32-byte aligned).
static bool router_on_gemm(moe_dtype_t dt, int d, int E)
{
    return dt == MOE_BF16 && E > 64 && E % 8 == 0 && d % 64 == 0 && d >= 128;
}

size_t route_ws_bytes(int64_t T, int d, int E, moe_dtype_t dt)
{
    if (T <= 0)
        return 0;
    const int nblk = route_blocks(T, E, dt);
    // per-block partial rows and per-group rows of the statistics
    const int gsz = route_group_size(nblk, E);
    const size_t stats = 2 * align_up((size_t)nblk * E * sizeof(float)) +
                         2 * align_up((size_t)((nblk + gsz - 1) / gsz) * E * 8);
    if (route_is_fused(dt, E))
        return stats;
    // plus the logits, and the split router weight and the grouped GEMM's
    // tail partials when the logits run on it
    const bool on_gemm = router_on_gemm(dt, d, E);
    size_t b = align_up((size_t)T * E * (on_gemm ? 3 : 1) * sizeof(float)) + stats;
    if (on_gemm)
        b += align_up((size_t)E * 3 * d * sizeof(uint16_t)) + align_up(gemm_ws_bytes());
    return b;
}

template <int ET, int TT, int CH, int G>
static void launch_fused1(const uint16_t *x, const float *w_router, const float *b_router, const float *sel_bias,
                          int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx, float *topk_w,
                          float *probs, float *part_p, int32_t *part_c, int gsz, double *grp_p, long long *grp_c,
                          unsigned *ticket, int32_t *expert_count, float *f, float *P, float *l_aux, int nblk,
                          hipStream_t stream)
{
    route_fused<ET, TT, CH, G><<<(unsigned)nblk, 64 * kRouteWaves, 0, stream>>>(
        x, w_router, b_router, sel_bias, T, d, E, k, alpha, topk_idx, topk_w, probs, part_p, part_c, gsz, grp_p,
        grp_c, ticket, expert_count, f, P, l_aux);
}

// K steps per register chunk: the largest power of two up to ch0 whose two
// chunks in flight (x of TT token tiles, two fp32 vectors of each of the ET
// weight tiles) and the accumulators fit the register file without spilling.
constexpr int route_ch(int ch0, int ET, int TT)
{
    const int per = 4 * TT + 4 * ET * 2;
    int ch = ch0;
    while (ch > 1 && 2 * ch * per + 4 * ET * TT > 232)
        ch /= 2;
    return ch;
}

template <int ET, int CH, int G>
static void launch_fused(int tt, const uint16_t *x, const float *w_router, const float *b_router,
                         const float *sel_bias, int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx,
                         float *topk_w, float *probs, float *part_p, int32_t *part_c, int gsz, double *grp_p,
                         long long *grp_c, unsigned *ticket, int32_t *expert_count, float *f, float *P, float *l_aux,
                         int nblk, hipStream_t stream)
{
#define MOE_F1(TT)                                                                                                  \
    launch_fused1<ET, TT, route_ch(CH, ET, TT), G>(x, w_router, b_router, sel_bias, T, d, E, k, alpha, topk_idx,    \
                                                   topk_w, probs, part_p, part_c, gsz, grp_p, grp_c, ticket,         \
                                                   expert_count, f, P, l_aux, nblk, stream)
    if (tt == 4)
        MOE_F1(4);
    else if (tt == 2)
        MOE_F1(2);
    else
        MOE_F1(1);
#undef MOE_F1
}

moe_status_t launch_route(const void *x, moe_dtype_t dt, const float *w_router, const float *b_router,
                          const float *sel_bias, int64_t T, int d, int E, int k, float alpha, int32_t *topk_idx,
                          float *topk_w,
                          int32_t *expert_count, float *f, float *P, float *l_aux, float *probs, void *ws,
                          unsigned *ticket, hipStream_t stream)
{
    if (T == 0) {
        // no tokens: zero counts and statistics
        route_finalize<float, int><<<1, 1024, 0, stream>>>((const float *)nullptr, (const int *)nullptr, 0, T, E,
                                                           alpha, expert_count, f, P, l_aux);
        return check_launch("route_finalize");
    }
    const int nblk = route_blocks(T, E, dt);
    Carver cv{(char *)ws, 0};
    if (route_is_fused(dt, E)) {
        float *part_p = cv.take<float>((size_t)nblk * E);
        int32_t *part_c = cv.take<int32_t>((size_t)nblk * E);
        const int gsz = route_group_size(nblk, E);
        const int ng = (nblk + gsz - 1) / gsz;
        double *grp_p = cv.take<double>((size_t)ng * E);
        long long *grp_c = cv.take<long long>((size_t)ng * E);
        const uint16_t *xb = (const uint16_t *)x;
#define MOE_FUSED(ET, CH, G)                                                                                         \
    launch_fused<ET, CH, G>(route_tt(T), xb, w_router, b_router, sel_bias, T, d, E, k, alpha, topk_idx, topk_w,     \
                            probs, part_p, part_c, gsz, grp_p, grp_c, ticket, expert_count, f, P, l_aux, nblk,       \
                            stream)
        if (E <= 8)
            MOE_FUSED(1, 8, 8);
        else if (E <= 16)
            MOE_FUSED(1, 8, 16);
        else if (E <= 32)
            MOE_FUSED(2, 4, 32);
        else if (E <= 48)
            MOE_FUSED(3, 2, 64);
        else
            MOE_FUSED(4, 2, 64);
#undef MOE_FUSED
        return check_launch("route_fused");
    }
    const bool on_gemm = router_on_gemm(dt, d, E);
    const int pieces = on_gemm ? 3 : 1;
    float *logits = cv.take<float>((size_t)T * E * pieces);
    float *part_p = cv.take<float>((size_t)nblk * E);
    int32_t *part_c = cv.take<int32_t>((size_t)nblk * E);
    const int gsz = route_group_size(nblk, E);
    double *grp_p = cv.take<double>((size_t)((nblk + gsz - 1) / gsz) * E);
    long long *grp_c = cv.take<long long>((size_t)((nblk + gsz - 1) / gsz) * E);
    uint16_t *w3 = on_gemm ? cv.take<uint16_t>((size_t)E * 3 * d) : nullptr;
    void *gws = on_gemm ? cv.take<char>(gemm_ws_bytes()) : nullptr;

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
        route_logits_f32<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>((const float *)x, w_router, T, d, E,
                                                                         logits);
    }
    if (moe_status_t s = check_launch("route_logits"))
        return s;
    const int epl = (E + 63) / 64;
    const dim3 g((unsigned)nblk);
#define SEL_STATS gsz, grp_p, grp_c, ticket, alpha, expert_count, f, P, l_aux
    switch (epl) {
    case 1: route_select<1><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs, SEL_STATS); break;
    case 2: route_select<2><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs, SEL_STATS); break;
    case 3:
    case 4: route_select<4><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs, SEL_STATS); break;
    case 5: case 6: case 7: case 8:
        route_select<8><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs, SEL_STATS); break;
    default:
        route_select<16><<<g, 256, 0, stream>>>(logits, pieces, b_router, sel_bias, T, E, k, topk_idx, topk_w, part_p, part_c, probs, SEL_STATS); break;
    }
#undef SEL_STATS
    return check_launch("route_select");
}

} // namespace moe
