// Grouped GEMM of the MoE layer: one Linear of every expert over its segment
// of expert-contiguous rows, with the bias and (for the first Linear) the
// exact GELU fused into the epilogue.
//
// Pages: "Expert Parallelism (MoE)", section "MoE Layer Structure" (each
// expert applies Linear(d -> 4d) -> GELU -> Linear(4d -> d)) and "Expert
// Parallelism (EP)", section "Key math / How it works" (the expert GEMMs run
// locally on the rows dispatched to this GPU).
//
// bf16 kernel (gfx950 matrix cores)
//  - out[r, n] = act(sum_k a[r, k] w[s, n, k] + b[s, n]) is computed as
//    out^T = W . A^T: the weight rows are the MFMA "A" operand and the token
//    rows the "B" operand, so each lane's accumulators hold 4 consecutive
//    output features of one row (8-byte bf16 stores).
//  - Block tile BN (features) x BM (rows), BK = 64; four waves in a 2 x 2
//    grid, each owning (BN/2) x (BM/2) as 32x32x16 bf16 MFMAs with fp32
//    accumulation.  Tiles of A and W are staged through LDS with an XOR
//    swizzle of the 16-byte chunks (row & 7) and double-buffered: the global
//    loads of step k+1 are in flight while step k computes.
//  - Persistent grid.  The tile list is derived on the device from the
//    segment offsets (no host round trip): segment s contributes
//    ceil(rows_s / BM) * (N / BN) tiles, ordered (segment, feature tile,
//    row tile) so that consecutive tiles share one weight tile.  Blocks are
//    dealt to the 8 XCDs round-robin by the hardware, so each XCD is given one
//    contiguous range of the tile list: the tiles that share weights run on
//    the same L2.
//  - Ragged tails: rows past the segment end are clamped on load and masked
//    on store; K tails are zero-filled in whole 8-element chunks.
// fp32 kernel: straightforward LDS-tiled VALU GEMM for the fp32 workloads.
#include "common.hpp"

namespace moe {

namespace {

constexpr int kBK = 64;
constexpr int kMaxSeg = 1024;
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t clamp_off(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Segment bounds with offsets clamped to [0, max_rows] and made non-decreasing.
__device__ __forceinline__ void seg_bounds(const int32_t *seg, int s, int64_t max_rows, int64_t &lo, int64_t &hi)
{
    if (!seg) {
        lo = 0;
        hi = max_rows;
        return;
    }
    lo = clamp_off(seg[s], 0, max_rows);
    hi = clamp_off(seg[s + 1], lo, max_rows);
}

// Exclusive prefix (in LDS) of the row tiles per segment; tb[S] = total.
template <int BM>
__device__ void build_tile_prefix(const int32_t *seg, int S, int64_t max_rows, int *tb)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave == 0) {
        int carry = 0;
        for (int s0 = 0; s0 < S; s0 += 64) {
            const int s = s0 + lane;
            int v = 0;
            if (s < S) {
                int64_t lo, hi;
                seg_bounds(seg, s, max_rows, lo, hi);
                v = (int)((hi - lo + BM - 1) / BM);
            }
            int inc = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(inc, o, 64);
                if (lane >= o)
                    inc += u;
            }
            if (s < S)
                tb[s] = carry + inc - v;
            carry += __shfl(inc, 63, 64);
        }
        if (lane == 0)
            tb[S] = carry;
    }
    __syncthreads();
}

// Largest s in [0, S) with tb[s] * NT <= L (tb non-decreasing, L < tb[S]*NT).
__device__ __forceinline__ int find_segment(const int *tb, int S, int NT, int64_t L)
{
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)tb[mid] * NT <= L)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

template <int BN, int BM, bool GELU>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16(const uint16_t *__restrict__ A,
                                                            const int32_t *__restrict__ seg, int S,
                                                            int64_t max_rows, const uint16_t *__restrict__ W,
                                                            const uint16_t *__restrict__ bias,
                                                            uint16_t *__restrict__ C, int N, int K)
{
    constexpr int WN = BN / 2, WM = BM / 2;
    constexpr int FN = WN / 32, FM = WM / 32;
    constexpr int LW = BN / 32, LA = BM / 32; // 16-byte loads per thread per stage
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kBK];
    __shared__ int tb[kMaxSeg + 1];

    build_tile_prefix<BM>(seg, S, max_rows, tb);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int NT = (N + BN - 1) / BN;
    const int64_t total = (int64_t)tb[S] * NT;

    // XCD-contiguous share of the tile list.
    const int xcd = blockIdx.x % kXcds;
    const int per = gridDim.x / kXcds;
    const int j = blockIdx.x / kXcds;
    const int64_t rlo = total * xcd / kXcds, rhi = total * (xcd + 1) / kXcds;

    const int lr = tid >> 3;  // row within a 32-row load group
    const int lc = tid & 7;   // 16-byte chunk within the 64-wide K slice
    const int KT = (K + kBK - 1) / kBK;

    for (int64_t L = rlo + j; L < rhi; L += per) {
        const int s = find_segment(tb, S, NT, L);
        const int mt_s = tb[s + 1] - tb[s];
        const int64_t local = L - (int64_t)tb[s] * NT;
        const int n_tile = (int)(local / mt_s);
        const int m_tile = (int)(local % mt_s);
        int64_t seg_lo, seg_hi;
        seg_bounds(seg, s, max_rows, seg_lo, seg_hi);
        const int64_t row0 = seg_lo + (int64_t)m_tile * BM;
        const int64_t row_end = min(row0 + BM, seg_hi);
        const int n0 = n_tile * BN;

        const uint16_t *wbase = W + (int64_t)s * N * K;
        const uint16_t *gw[LW];
        const uint16_t *ga[LA];
#pragma unroll
        for (int q = 0; q < LW; ++q) {
            const int n = min(n0 + q * 32 + lr, N - 1);
            gw[q] = wbase + (int64_t)n * K + lc * 8;
        }
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int64_t r = min(row0 + q * 32 + lr, row_end - 1);
            ga[q] = A + r * K + lc * 8;
        }
        const int sw_off = lr * kBK + ((lc ^ (lr & 7)) * 8);

        u32x4 rw[LW], ra[LA];
        auto gload = [&](int kt) {
            const int kk = kt * kBK + lc * 8;
            const bool ok = kk < K;
#pragma unroll
            for (int q = 0; q < LW; ++q)
                rw[q] = ok ? *reinterpret_cast<const u32x4 *>(gw[q] + kt * kBK) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < LA; ++q)
                ra[q] = ok ? *reinterpret_cast<const u32x4 *>(ga[q] + kt * kBK) : u32x4{0u, 0u, 0u, 0u};
        };
        auto lstore = [&](int buf) {
#pragma unroll
            for (int q = 0; q < LW; ++q)
                *reinterpret_cast<u32x4 *>(&sW[buf][q * 32 * kBK + sw_off]) = rw[q];
#pragma unroll
            for (int q = 0; q < LA; ++q)
                *reinterpret_cast<u32x4 *>(&sA[buf][q * 32 * kBK + sw_off]) = ra[q];
        };

        f32x16 acc[FN][FM];
#pragma unroll
        for (int a = 0; a < FN; ++a)
#pragma unroll
            for (int b = 0; b < FM; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[a][b][v] = 0.f;

        gload(0);
        lstore(0);
        __syncthreads();
        const int r32 = lane & 31, khalf = lane >> 5;
        for (int kt = 0; kt < KT; ++kt) {
            if (kt + 1 < KT)
                gload(kt + 1);
            const int buf = kt & 1;
#pragma unroll
            for (int ks = 0; ks < kBK / 16; ++ks) {
                const int ch = ks * 2 + khalf;
                bf16x8 fa[FN], fb[FM];
#pragma unroll
                for (int a = 0; a < FN; ++a) {
                    const int row = wn * WN + a * 32 + r32;
                    fa[a] = *reinterpret_cast<const bf16x8 *>(&sW[buf][row * kBK + ((ch ^ (row & 7)) * 8)]);
                }
#pragma unroll
                for (int b = 0; b < FM; ++b) {
                    const int row = wm * WM + b * 32 + r32;
                    fb[b] = *reinterpret_cast<const bf16x8 *>(&sA[buf][row * kBK + ((ch ^ (row & 7)) * 8)]);
                }
#pragma unroll
                for (int a = 0; a < FN; ++a)
#pragma unroll
                    for (int b = 0; b < FM; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
            }
            if (kt + 1 < KT)
                lstore((kt + 1) & 1);
            __syncthreads();
        }

        // Epilogue: lane holds out^T[n][m] for m = lane%32 and, for each group
        // g of 4 registers, n = 8g + 4*(lane/32) + 0..3.
        const uint16_t *bseg = bias ? bias + (int64_t)s * N : nullptr;
#pragma unroll
        for (int b = 0; b < FM; ++b) {
            const int64_t row = row0 + wm * WM + b * 32 + r32;
            if (row >= row_end)
                continue;
            uint16_t *crow = C + row * N;
#pragma unroll
            for (int a = 0; a < FN; ++a) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn * WN + a * 32 + 8 * g + 4 * khalf;
                    if (n >= N)
                        continue;
                    float v0 = acc[a][b][4 * g + 0], v1 = acc[a][b][4 * g + 1];
                    float v2 = acc[a][b][4 * g + 2], v3 = acc[a][b][4 * g + 3];
                    if (bseg) {
                        const uint2 bb = *reinterpret_cast<const uint2 *>(bseg + n);
                        v0 += bf16_bits_to_f32(bb.x & 0xFFFFu);
                        v1 += bf16_bits_to_f32(bb.x >> 16);
                        v2 += bf16_bits_to_f32(bb.y & 0xFFFFu);
                        v3 += bf16_bits_to_f32(bb.y >> 16);
                    }
                    if (GELU) {
                        v0 = gelu_erf(v0);
                        v1 = gelu_erf(v1);
                        v2 = gelu_erf(v2);
                        v3 = gelu_erf(v3);
                    }
                    uint2 o;
                    o.x = pack_bf16x2(v0, v1);
                    o.y = pack_bf16x2(v2, v3);
                    *reinterpret_cast<uint2 *>(crow + n) = o;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large-tile bf16 kernel: 256 (features) x 256 (rows) per block, four waves
// of 128 x 128 (4 x 4 MFMA 32x32x16 tiles, 256 fp32 accumulators per lane,
// held in AGPRs).
//
// Global -> LDS copies are buffer_load_dwordx4 ... lds (LDS DMA): each lane's
// 16 bytes land at M0 + 16 * lane, so a wave fills 1 KB of contiguous LDS per
// instruction and the XOR swizzle of the 16-byte chunks is applied on the
// global side.  The copies are issued as inline assembly so that the
// compiler's conservative wait-for-all-DMA before every LDS read does not
// serialise them; the kernel keeps its own vmcnt accounting: STAGES-1 K
// steps are in flight while one computes.  They have no output registers.
//
// LDS on gfx950 serves a ds_read_b128 16 lanes at a time over 64 banks
// (256 bytes): rows of BK bf16 are swizzled so that the 16 rows read by one
// group of lanes at the same logical chunk hit 16 distinct bank groups.
// Requires K % BK == 0; rows past the weight matrix or the segment end read
// as zeros (buffer range checking); row sub-tiles past the segment end skip
// their MFMAs; stores are masked.
// ---------------------------------------------------------------------------
constexpr int kL = 256; // tile edge

typedef __attribute__((address_space(3))) void lds_void;
// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;
// A scalar offset past every tile's buffer range: such a copy reads zeros.
constexpr uint32_t kOutOfRange = 0x40000000u;

template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Logical 16-byte chunk stored at physical chunk p of a row: p ^ f(row).
template <int BK> __device__ __forceinline__ int swz(int row)
{
    return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// LDS-DMA copy: 16 bytes per lane from buffer `rsrc` at voff + soff into LDS
// at m0 + 16 * lane.  Written as inline assembly so that the compiler's
// wait-count pass does not track it (it would wait for every copy before
// any LDS read); the kernel keeps the vmcnt accounting itself.  The
// instruction writes no registers.  The compiler's hazard recognizer does
// not look inside inline assembly, so the block carries its own wait states:
// the M0 write just before it needs one, and a scalar offset that a VALU op
// wrote (readfirstlane, or a reload of a spilled SGPR with v_readlane) needs
// five before a vector memory instruction may read it.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t m0)
{
    i32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r[k] = __builtin_amdgcn_readfirstlane(rsrc[k]);
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                   "{m0}"(__builtin_amdgcn_readfirstlane(m0))
                 : "memory");
}

__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
    r[2] = (int)bytes;
    r[3] = kRsrcWord3;
    return r;
}

// Values the whole wave shares, held in scalar registers (the compiler
// cannot prove that values read from LDS are uniform).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Wave grid of a 256x256 tile: WGN waves along the features and WGM along
// the rows; each wave owns (256/WGN) x (256/WGM) as FA x FB MFMA tiles of
// 32x32.  Four waves (2x2, 128x128 each, one wave per SIMD) or eight (2x4,
// 128x64 each, two waves per SIMD so that one wave's MFMAs cover the
// other's waits).
template <int WGN, int WGM> struct Grid {
    static constexpr int WGN_ = WGN, WGM_ = WGM;
    static constexpr int NW = WGN * WGM;
    static constexpr int WTN = kL / WGN, WTM = kL / WGM;
    static constexpr int FA = WTN / 32, FB = WTM / 32;
};

// One K step of a 256x256 tile: MFMAs on stage `cur` (already in LDS) while
// the LDS-DMA copies of a later K step fill the stage at LDS byte address
// `nxt`.  Each 16-wide K sub-step is cut into chunks of MFMAs plus a share of
// the LDS reads of the next sub-step; one copy is issued after each chunk, so
// the copies trickle out at the rate the address unit drains them instead of
// stalling the wave in a burst.
#ifndef MOE_GEMM_CPS
#define MOE_GEMM_CPS 0 // chunks per 16-wide sub-step; 0: one per copy
#endif
#ifndef MOE_GEMM_LEAD
#define MOE_GEMM_LEAD 8 // copies are spread over LEAD/8 of the K step
#endif
template <int BK, class G, int NBV>
__device__ __forceinline__ void k_step(const uint16_t *cur, uint32_t nxt, f32x16 (&acc)[G::FA][G::FB], i32x4 rw,
                                       i32x4 ra, uint32_t vbase, uint32_t vbase_a, uint32_t so_w, uint32_t so_a,
                                       uint32_t row_w, uint32_t row_a, int wave, int wn, int wm, int r32, int khalf,
                                       int sw)
{
    constexpr int FA = G::FA, FB = G::FB, NW = G::NW;
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NQ = kL / (NW * RPI), KS = BK / 16;
    constexpr int DPW = 2 * NQ;                                  // copies per wave per stage
    constexpr int CPS = MOE_GEMM_CPS > 0 ? MOE_GEMM_CPS : DPW / KS; // chunks per sub-step
    constexpr int NCH = KS * CPS;                                // chunks per K step
    constexpr int MPC = FA * FB / CPS;                           // MFMAs per chunk
    constexpr int RDS = FA + FB;                                 // fragment reads per sub-step
    constexpr int RPC = (RDS + CPS - 1) / CPS;
    static_assert(DPW % KS == 0 && (FA * FB) % CPS == 0, "chunking");
    const uint16_t *sW = cur;
    const uint16_t *sA = cur + kL * BK;
    bf16x8 fa[2][FA], fb[2][FB];
    auto read = [&](int ks, int buf, int r) {
        const int ch = ((ks * 2 + khalf) ^ sw) * 8;
        if (r < FA) {
            fa[buf][r] = *reinterpret_cast<const bf16x8 *>(sW + (wn * G::WTN + r * 32 + r32) * BK + ch);
        } else if (r - FA < NBV) {
            const int b = r - FA;
            fb[buf][b] = *reinterpret_cast<const bf16x8 *>(sA + (wm * G::WTM + b * 32 + r32) * BK + ch);
        }
    };
    auto dma = [&](int i) { // copy i of DPW: W rows for even i, A rows for odd i
        const int q = i >> 1;
        const uint32_t R = (uint32_t)((NW * q + wave) * RPI);
        const uint32_t so = (i & 1) ? (uint32_t)q * (uint32_t)(NW * RPI) * row_a + so_a
                                    : (uint32_t)q * (uint32_t)(NW * RPI) * row_w + so_w;
        dma16((i & 1) ? ra : rw, (i & 1) ? vbase_a : vbase, so, nxt + (uint32_t)((i & 1) * (kL * BK) + R * BK) * 2u);
    };
    if (NBV > 0) {
#pragma unroll
        for (int r = 0; r < RDS; ++r)
            read(0, 0, r);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int c = 0; c < CPS; ++c) {
            if (NBV > 0) {
#pragma unroll
                for (int i = c * MPC; i < (c + 1) * MPC; ++i) {
                    const int a = i / FB, b = i % FB;
                    if (b < NBV)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][a], fb[ks & 1][b], acc[a][b],
                                                                            0, 0, 0);
                }
                if (ks + 1 < KS) {
#pragma unroll
                    for (int r = c * RPC; r < (c + 1) * RPC && r < RDS; ++r)
                        read(ks + 1, (ks + 1) & 1, r);
                }
                if (NBV == FB) {
#pragma unroll
                    for (int m = 0; m < MPC; ++m) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (ks + 1 < KS && m < RPC && c * RPC + m < RDS)
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
            }
            // Copy j goes out after chunk (j * NCH * LEAD) / (8 * DPW).
            const int g = ks * CPS + c;
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                if ((j * NCH * MOE_GEMM_LEAD) / (8 * DPW) == g) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma(j);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
}

// Epilogue of a 256x256 tile: bias, activation and store of the rows inside
// [row0, row_end) and features < N, as bf16 (rounded to nearest even) or,
// with F32OUT, as fp32.  Accumulators are read unconditionally and only the
// stores are predicated, so no accumulator has to live outside its register.
template <bool GELU, bool BIAS, bool F32OUT>
__device__ __forceinline__ void store4(void *C, const uint16_t *__restrict__ bseg, int64_t row, bool row_ok, int n,
                                       int N, float v0, float v1, float v2, float v3)
{
    if (BIAS) {
        const uint2 bb = *reinterpret_cast<const uint2 *>(bseg + (n < N ? n : 0));
        v0 += bf16_bits_to_f32(bb.x & 0xFFFFu);
        v1 += bf16_bits_to_f32(bb.x >> 16);
        v2 += bf16_bits_to_f32(bb.y & 0xFFFFu);
        v3 += bf16_bits_to_f32(bb.y >> 16);
    }
    if (GELU) {
        v0 = gelu_erf(v0);
        v1 = gelu_erf(v1);
        v2 = gelu_erf(v2);
        v3 = gelu_erf(v3);
    }
    const bool ok = row_ok && n < N;
    const int64_t at = (ok ? row : 0) * N + (ok ? n : 0);
    if (F32OUT) {
        const f32x4 o = {v0, v1, v2, v3};
        if (ok)
            *reinterpret_cast<f32x4 *>((float *)C + at) = o;
    } else {
        uint2 o;
        o.x = pack_bf16x2(v0, v1);
        o.y = pack_bf16x2(v2, v3);
        if (ok)
            *reinterpret_cast<uint2 *>((uint16_t *)C + at) = o;
    }
}

template <class G, int NBV, bool GELU, bool BIAS, bool F32OUT>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[G::FA][G::FB], void *C,
                                           const uint16_t *__restrict__ bseg, int64_t row0, int64_t row_end, int n0,
                                           int N, int wn, int wm, int r32, int khalf)
{
#pragma unroll
    for (int b = 0; b < NBV; ++b) {
        const int64_t row = row0 + wm * G::WTM + b * 32 + r32;
        const bool row_ok = row < row_end;
#pragma unroll
        for (int a = 0; a < G::FA; ++a) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * G::WTN + a * 32 + 8 * g + 4 * khalf;
                store4<GELU, BIAS, F32OUT>(C, bseg, row, row_ok, n, N, acc[a][b][4 * g + 0], acc[a][b][4 * g + 1],
                                           acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
            }
        }
    }
}

// One 256x256 tile over K steps [kt_lo, kt_hi).  With PART the raw fp32
// accumulators go to `part` (one 256 KB slab: per wave, per register, lane
// fastest) for a later fixed-order reduction; otherwise the epilogue stores
// bf16.
template <int BK, int STAGES, class G, int NBV, bool GELU, bool BIAS, bool F32OUT, bool PART>
__device__ __forceinline__ void tile_256(const uint16_t *__restrict__ A, const uint16_t *__restrict__ wseg,
                                         const uint16_t *__restrict__ bseg, void *__restrict__ C,
                                         float *__restrict__ part, uint16_t *smem, int64_t row0, int64_t row_end,
                                         int n0, int N, int K, int Ka, int kt_lo, int kt_hi)
{
    constexpr int NW = G::NW, FA = G::FA, FB = G::FB;
    constexpr int CPR = BK / 8;            // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;          // rows filled per DMA instruction (1 KB)
    constexpr int NQ = kL / (NW * RPI);    // DMA instructions per operand per wave
    constexpr int STAGE = 2 * kL * BK;     // bf16 elements per stage (W then A)
    constexpr int PER_STAGE = 2 * NQ;      // DMA instructions per thread per stage
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WGN_, wm = wave / G::WGN_;
    const int r32 = lane & 31, khalf = lane >> 5;

    // Instruction q of this wave fills LDS rows R = (NW q + wave) * RPI ..
    // R + RPI - 1; lane -> row R + lane / CPR, physical chunk lane % CPR,
    // which holds logical chunk (lane % CPR) ^ swizzle(row).  The byte offset
    // of that row is vbase + q * NW * RPI * K * 2 (the q part is scalar).  The
    // buffer resources cover exactly the tile's valid rows: rows past the
    // weight matrix or the segment end read as zeros.
    // A's rows have Ka elements: its K offset wraps every Ka (Ka = K for a
    // plain GEMM; the router's split weight repeats the activations thrice).
    const uint32_t row_bytes = (uint32_t)K * 2u, row_a = (uint32_t)Ka * 2u;
    const int KTa = Ka / BK;
    const int lrow = lane / CPR;
    const int prow = wave * RPI + lrow;
    const int lchunk = (lane % CPR) ^ swz<BK>(prow);
    const uint32_t vbase = (uint32_t)prow * row_bytes + (uint32_t)lchunk * 16u;
    const uint32_t vbase_a = (uint32_t)prow * row_a + (uint32_t)lchunk * 16u;
    const int wrows = min(kL, N - n0);
    const int arows = (int)(row_end - row0);
    const i32x4 rw = make_rsrc(wseg + (int64_t)n0 * K, (uint32_t)wrows * row_bytes);
    const i32x4 ra = make_rsrc(A + row0 * Ka, (uint32_t)arows * row_a);
    const uint32_t lds0 = lds_addr(smem);

    f32x16 acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[a][b][v] = 0.f;

    const int sw = swz<BK>(r32);
    // Prologue: stages 0 .. STAGES-2 hold K steps kt_lo .. kt_lo+STAGES-2 (a
    // copy past kt_hi reads out of range: zeros).
    for (int p = 0; p < STAGES - 1; ++p) {
        const uint32_t dst = lds0 + (uint32_t)(p * STAGE) * 2u;
        const bool live = kt_lo + p < kt_hi;
        const uint32_t so_w = live ? (uint32_t)(kt_lo + p) * (BK * 2) : kOutOfRange;
        const uint32_t so_a = live ? (uint32_t)((kt_lo + p) % KTa) * (BK * 2) : kOutOfRange;
#pragma unroll
        for (int i = 0; i < 2 * NQ; ++i) {
            const int q = i >> 1;
            const uint32_t R = (uint32_t)((NW * q + wave) * RPI);
            const uint32_t so = (i & 1) ? (uint32_t)q * (uint32_t)(NW * RPI) * row_a + so_a
                                        : (uint32_t)q * (uint32_t)(NW * RPI) * row_bytes + so_w;
            dma16((i & 1) ? ra : rw, (i & 1) ? vbase_a : vbase, so,
                  dst + (uint32_t)((i & 1) * (kL * BK) + R * BK) * 2u);
        }
    }
    wait_vmcnt<(STAGES - 2) * PER_STAGE>();
    __syncthreads();

    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int fill = kt + STAGES - 1;
        const bool live = fill < kt_hi;
        const uint32_t so_w = live ? (uint32_t)fill * (BK * 2) : kOutOfRange;
        const uint32_t so_a = live ? (uint32_t)(fill % KTa) * (BK * 2) : kOutOfRange;
        k_step<BK, G, NBV>(smem + ((kt - kt_lo) % STAGES) * STAGE,
                           lds0 + (uint32_t)(((fill - kt_lo) % STAGES) * STAGE) * 2u, acc, rw, ra, vbase, vbase_a,
                           so_w, so_a, row_bytes, row_a, wave, wn, wm, r32, khalf, sw);
        // Stage kt+1 must have landed; the STAGES-2 stages issued after it
        // may stay in flight.
        wait_vmcnt<(STAGES - 2) * PER_STAGE>();
        __syncthreads();
    }
    wait_vmcnt<0>(); // the zero-fill copies of the last steps must land before the next tile's copies

    if (PART) {
        float *dst = part + (size_t)wave * (FA * FB * 16 * 64) + lane;
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < FB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dst[((a * FB + b) * 16 + v) * 64] = acc[a][b][v];
    } else {
        store_tile<G, NBV, GELU, BIAS, F32OUT>(acc, C, bseg, row0, row_end, n0, N, wn, wm, r32, khalf);
    }
}

// Split of the tile list over a persistent grid of G blocks.  F whole tiles
// run in full rounds (each block gets the same number); when the rest
// (`rem` tiles, at most half a round) would leave CUs idle, each of them is
// cut into `sk` K ranges, one per block, written as fp32 partials and summed
// by grouped_gemm_reduce.  Computed identically by both kernels.
struct TailPlan {
    int64_t F;   // whole tiles
    int rem;     // tail tiles split in K (0: none)
    int sk;      // K ranges per tail tile
};

__device__ __forceinline__ TailPlan plan_tail(int64_t total, int G, int KT, bool have_ws, int min_len = 1)
{
    TailPlan p{total, 0, 1};
    const int64_t R = total / G;
    const int64_t rem = total - R * G;
    if (have_ws && rem > 0 && 2 * rem <= G) {
        int sk = (int)(G / rem);
        sk = sk > 8 ? 8 : sk;
        sk = sk > KT / min_len ? KT / min_len : sk;
        if (sk >= 2) {
            p.F = R * G;
            p.rem = (int)rem;
            p.sk = sk;
        }
    }
    return p;
}

template <int BK, int STAGES, class G, bool GELU, bool BIAS, bool F32OUT, bool PART>
__device__ __forceinline__ void tile_any(int nbv, const uint16_t *A, const uint16_t *wseg, const uint16_t *bseg,
                                         void *C, float *part, uint16_t *smem, int64_t row0, int64_t row_end, int n0,
                                         int N, int K, int Ka, int kt_lo, int kt_hi)
{
#define MOE_TILE(V) tile_256<BK, STAGES, G, V, GELU, BIAS, F32OUT, PART>(A, wseg, bseg, C, part, smem, row0, row_end, \
                                                                     n0, N, K, Ka, kt_lo, kt_hi)
    if (G::FB == 4) {
        switch (nbv) {
        case 4: MOE_TILE(G::FB >= 4 ? 4 : G::FB); return;
        case 3: MOE_TILE(G::FB >= 3 ? 3 : G::FB); return;
        default: break;
        }
    }
    switch (nbv) {
    case 2: MOE_TILE(G::FB >= 2 ? 2 : G::FB); break;
    case 1: MOE_TILE(1); break;
    case 0: MOE_TILE(0); break;
    default: break;
    }
#undef MOE_TILE
}

// Location of tile L of the list: segment, rows and first feature.
struct TileLoc {
    int s;
    int64_t row0, row_end;
    int n0;
};

__device__ __forceinline__ TileLoc locate(const int *tb, const int32_t *seg, int S, int64_t max_rows, int NT,
                                          int64_t L)
{
    TileLoc t;
    t.s = find_segment(tb, S, NT, L);
    const int mt_s = tb[t.s + 1] - tb[t.s];
    const int64_t local = L - (int64_t)tb[t.s] * NT;
    const int n_tile = (int)(local / mt_s);
    const int m_tile = (int)(local % mt_s);
    int64_t seg_lo, seg_hi;
    seg_bounds(seg, t.s, max_rows, seg_lo, seg_hi);
    t.row0 = seg_lo + (int64_t)m_tile * kL;
    t.row_end = min(t.row0 + kL, seg_hi);
    t.n0 = n_tile * kL;
    return t;
}

template <class G> __device__ __forceinline__ int valid_b(const TileLoc &t, int wm)
{
    const int64_t left = t.row_end - (t.row0 + (int64_t)wm * G::WTM);
    return left <= 0 ? 0 : (left >= G::WTM ? G::FB : (int)((left + 31) / 32));
}

template <int BK, int STAGES, class G, bool GELU, bool BIAS, bool F32OUT>
__global__ __launch_bounds__(64 * G::NW, 1) void grouped_gemm_bf16_256(const uint16_t *__restrict__ A,
                                                                       const int32_t *__restrict__ seg, int S,
                                                                       int64_t max_rows,
                                                                       const uint16_t *__restrict__ W,
                                                                       const uint16_t *__restrict__ bias,
                                                                       void *__restrict__ C, int N, int K, int Ka,
                                                                       float *__restrict__ part_ws)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * 2 * kL * BK];
    __shared__ int tb[kMaxSeg + 1];
    build_tile_prefix<kL>(seg, S, max_rows, tb);

    const int wm = (threadIdx.x >> 6) / G::WGN_;
    const int NT = (N + kL - 1) / kL;
    const int KT = K / BK;
    const int64_t total = (int64_t)tb[S] * NT;
    const TailPlan plan = plan_tail(total, (int)gridDim.x, KT, part_ws != nullptr);

    // Whole tiles: an XCD-contiguous share of tiles [0, F).
    const int xcd = blockIdx.x % kXcds;
    const int per = gridDim.x / kXcds;
    const int j = blockIdx.x / kXcds;
    const int64_t rlo = plan.F * xcd / kXcds, rhi = plan.F * (xcd + 1) / kXcds;
    for (int64_t L = rlo + j; L < rhi; L += per) {
        const TileLoc t = locate(tb, seg, S, max_rows, NT, L);
        tile_any<BK, STAGES, G, GELU, BIAS, F32OUT, false>(valid_b<G>(t, wm), A, W + (int64_t)t.s * N * K,
                                                           bias ? bias + (int64_t)t.s * N : nullptr, C, nullptr, smem,
                                                           t.row0, t.row_end, t.n0, N, K, Ka, 0, KT);
        __syncthreads(); // the next tile's copies overwrite stages still read here
    }
    // Tail: one K range of one tail tile per block.
    const int u = blockIdx.x;
    if (plan.rem > 0 && u < plan.rem * plan.sk) {
        const int64_t L = plan.F + u / plan.sk;
        const int c = u % plan.sk;
        const TileLoc t = locate(tb, seg, S, max_rows, NT, L);
        const int klo = (int)((int64_t)KT * c / plan.sk), khi = (int)((int64_t)KT * (c + 1) / plan.sk);
        tile_any<BK, STAGES, G, GELU, BIAS, F32OUT, true>(valid_b<G>(t, wm), A, W + (int64_t)t.s * N * K, nullptr,
                                                          C, part_ws + (size_t)u * (kL * kL), smem, t.row0, t.row_end,
                                                          t.n0, N, K, Ka, klo, khi);
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined form of the same tiling.  Two LDS stages; within a K
// step the copies of the next stage go out during the first KS-1 sub-steps,
// the block synchronises once, before the last sub-step, and the last
// sub-step's MFMAs cover the LDS reads of the next stage's first sub-step, so
// the matrix pipe does not drain at K-step boundaries.  The last K step of a
// tile already copies the first stage of the block's next tile, so that tile
// starts without a load bubble and its copies overlap this tile's epilogue.
// ---------------------------------------------------------------------------

// Per-launch copy geometry: per-lane byte offsets (row and swizzled chunk)
// into a W and an A row, bytes per row, and K steps per A row.
struct CopyGeo {
    uint32_t vbase, vbase_a, row_w, row_a;
    int KTa;
};

// One stage's source: the tile's buffer resources and the K step's scalar
// offsets.  A fill with nothing to load uses resources of zero bytes: every
// copy is then out of range and writes zeros to LDS without touching memory
// (no branch in the K loop, and the wait counts stay uniform).
struct Fill {
    i32x4 rw, ra;
    uint32_t so_w, so_a;
};

template <int BK> __device__ __forceinline__ Fill fill_at(i32x4 rw, i32x4 ra, int kt, int KTa)
{
    Fill f;
    f.rw = rw;
    f.ra = ra;
    f.so_w = (uint32_t)kt * (BK * 2);
    f.so_a = (uint32_t)(kt % KTa) * (BK * 2);
    return f;
}

template <int BK, class G>
__device__ __forceinline__ void copy_one(const CopyGeo &cg, const Fill &f, uint32_t dst, int wave, int i)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NW = G::NW;
    const int q = i >> 1;
    const uint32_t R = (uint32_t)((NW * q + wave) * RPI);
    const uint32_t so = (i & 1) ? (uint32_t)q * (uint32_t)(NW * RPI) * cg.row_a + f.so_a
                                : (uint32_t)q * (uint32_t)(NW * RPI) * cg.row_w + f.so_w;
    dma16((i & 1) ? f.ra : f.rw, (i & 1) ? cg.vbase_a : cg.vbase, so,
          dst + (uint32_t)((i & 1) * (kL * BK) + R * BK) * 2u);
}

// This wave's copies except the newest N have landed, every wave got that
// far, and every wave's LDS reads issued so far have completed.  (Copies
// complete in issue order.)
template <int N> __device__ __forceinline__ void stage_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

#ifndef MOE_PIPE_CPS
#define MOE_PIPE_CPS 8 // chunks per 16-wide sub-step
#endif
#ifndef MOE_PIPE_RCH
#define MOE_PIPE_RCH 2 // the next sub-step's fragment reads go out in the first RCH chunks
#endif

// Fragment reads in the order the next sub-step's MFMAs first use them: the
// MFMA sequence is (a, b) = (i / FB, i % FB), so read r is A fragment a or B
// fragment b as they first appear in it.  Returns a for A, FA + b for B.
template <class G> __host__ __device__ constexpr int read_slot(int r)
{
    bool ra[G::FA] = {}, rb[G::FB] = {};
    int n = 0;
    for (int i = 0; i < G::FA * G::FB; ++i) {
        const int a = i / G::FB, b = i % G::FB;
        if (!ra[a]) {
            ra[a] = true;
            if (n++ == r)
                return a;
        }
        if (!rb[b]) {
            rb[b] = true;
            if (n++ == r)
                return G::FA + b;
        }
    }
    return -1;
}

template <int BK, class G, int NBV>
__device__ __forceinline__ void read_frag(const uint16_t *stage, int ks, bf16x8 (&fa)[G::FA], bf16x8 (&fb)[G::FB],
                                          int r, int wn, int wm, int r32, int khalf, int sw)
{
    const int ch = ((ks * 2 + khalf) ^ sw) * 8;
    if (r < G::FA) {
        fa[r] = *reinterpret_cast<const bf16x8 *>(stage + (wn * G::WTN + r * 32 + r32) * BK + ch);
    } else if (r - G::FA < NBV) {
        const int b = r - G::FA;
        fb[b] = *reinterpret_cast<const bf16x8 *>(stage + kL * BK + (wm * G::WTM + b * 32 + r32) * BK + ch);
    }
}

// One K step: MFMAs on stage `cur`; the copies of a later stage (`f`, to
// LDS byte address `fill_lds`) go out during the first KS-1 sub-steps; then
// one barrier, after which the next stage `nxt` has landed and the last
// sub-step's MFMAs cover the reads of its first sub-step.
template <int BK, int STAGES, class G, int NBV>
__device__ __forceinline__ void k_step_pipe(const uint16_t *cur, const uint16_t *nxt, uint32_t fill_lds,
                                            const Fill &f, const CopyGeo &cg, f32x16 (&acc)[G::FA][G::FB],
                                            bf16x8 (&fa)[2][G::FA], bf16x8 (&fb)[2][G::FB], int wave, int wn, int wm,
                                            int r32, int khalf, int sw)
{
    constexpr int FA = G::FA, FB = G::FB;
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NQ = kL / (G::NW * RPI), KS = BK / 16;
    constexpr int DPW = 2 * NQ;            // copies per wave per stage
    constexpr int CPS = MOE_PIPE_CPS < FA * FB ? MOE_PIPE_CPS : FA * FB; // chunks per sub-step
    constexpr int MPC = FA * FB / CPS;     // MFMAs per chunk
    constexpr int RDS = FA + FB;           // fragment reads per sub-step
    constexpr int RCH = MOE_PIPE_RCH < CPS ? MOE_PIPE_RCH : CPS;
    constexpr int RPC = (RDS + RCH - 1) / RCH; // reads per chunk in the first RCH chunks
    constexpr int NPRE = (KS - 1) * CPS;   // chunks before the barrier
    static_assert(KS >= 2 && (FA * FB) % CPS == 0, "chunking");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint16_t *src = ks + 1 < KS ? cur : nxt;
        const int kn = ks + 1 < KS ? ks + 1 : 0;
#pragma unroll
        for (int c = 0; c < CPS; ++c) {
            if (NBV > 0) {
#pragma unroll
                for (int m = 0; m < MPC; ++m) {
                    const int i = c * MPC + m;
                    const int a = i / FB, b = i % FB;
                    if (b < NBV)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][a], fb[ks & 1][b], acc[a][b],
                                                                            0, 0, 0);
#pragma unroll
                    for (int q = 0; q < RPC; ++q) {
                        const int r = c * RPC + q;
                        if (c < RCH && r < RDS && (q * MPC) / RPC == m)
                            read_frag<BK, G, NBV>(src, kn, fa[(ks + 1) & 1], fb[(ks + 1) & 1], read_slot<G>(r), wn,
                                                  wm, r32, khalf, sw);
                    }
                }
                if (NBV == FB) {
#pragma unroll
                    for (int m = 0; m < MPC; ++m) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
                        for (int q = 0; q < RPC; ++q)
                            if (c < RCH && c * RPC + q < RDS && (q * MPC) / RPC == m)
                                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
            }
            if (ks + 1 < KS) {
                const int g = ks * CPS + c;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < DPW; ++j)
                    if ((j * NPRE) / DPW == g)
                        copy_one<BK, G>(cg, f, fill_lds, wave, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (ks == KS - 2) {
            // the next stage has landed; the STAGES-2 newer ones may be in flight
            __builtin_amdgcn_sched_barrier(0);
            stage_barrier<(STAGES - 2) * DPW>();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Source of the next work item's first stages, for the last K steps of a
// tile: its resources and K range (len >= STAGES-1), or none.
struct NextSrc {
    i32x4 rw, ra;
    int kt_lo;
    bool any;
};

// One tile (or one K range of a tail tile).  On entry ring slot b holds its
// first K step (landed, behind a barrier) and the next STAGES-2 steps are in
// flight; on exit the same holds for `next` at the returned slot.
template <int BK, int STAGES, class G, int NBV, bool GELU, bool BIAS, bool F32OUT, bool PART>
__device__ __forceinline__ int tile_pipe(const uint16_t *smem, uint32_t lds0, int b, const CopyGeo &cg, i32x4 rw,
                                         i32x4 ra, int kt_lo, int kt_hi, const NextSrc &next, i32x4 null_w,
                                         i32x4 null_a, void *C, const uint16_t *bseg, float *part, int64_t row0,
                                         int64_t row_end, int n0, int N)
{
    constexpr int FA = G::FA, FB = G::FB, STAGE = 2 * kL * BK;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WGN_, wm = wave / G::WGN_;
    const int r32 = lane & 31, khalf = lane >> 5;
    const int sw = swz<BK>(r32);

    f32x16 acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int q = 0; q < FB; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[a][q][v] = 0.f;
    bf16x8 fa[2][FA], fb[2][FB];
    if (NBV > 0) {
#pragma unroll
        for (int r = 0; r < FA + FB; ++r)
            read_frag<BK, G, NBV>(smem + b * STAGE, 0, fa[0], fb[0], r, wn, wm, r32, khalf, sw);
    }
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int fs = kt + STAGES - 1; // K step to fill
        Fill f;
        if (fs < kt_hi)
            f = fill_at<BK>(rw, ra, fs, cg.KTa);
        else if (next.any)
            f = fill_at<BK>(next.rw, next.ra, next.kt_lo + (fs - kt_hi), cg.KTa);
        else
            f = fill_at<BK>(null_w, null_a, 0, cg.KTa);
        const int bn = b + 1 == STAGES ? 0 : b + 1;
        const int bf = b == 0 ? STAGES - 1 : b - 1;
        k_step_pipe<BK, STAGES, G, NBV>(smem + b * STAGE, smem + bn * STAGE, lds0 + (uint32_t)(bf * STAGE) * 2u, f,
                                        cg, acc, fa, fb, wave, wn, wm, r32, khalf, sw);
        b = bn;
    }
    if (PART) {
        float *dst = part + (size_t)wave * (FA * FB * 16 * 64) + lane;
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int q = 0; q < FB; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dst[((a * FB + q) * 16 + v) * 64] = acc[a][q][v];
    } else {
        store_tile<G, NBV, GELU, BIAS, F32OUT>(acc, C, bseg, row0, row_end, n0, N, wn, wm, r32, khalf);
    }
    return b;
}

template <int BK, int STAGES, class G, bool GELU, bool BIAS, bool F32OUT, bool PART>
__device__ __forceinline__ int tile_pipe_any(int nbv, const uint16_t *smem, uint32_t lds0, int b, const CopyGeo &cg,
                                             i32x4 rw, i32x4 ra, int kt_lo, int kt_hi, const NextSrc &next,
                                             i32x4 null_w, i32x4 null_a, void *C, const uint16_t *bseg, float *part,
                                             int64_t row0, int64_t row_end, int n0, int N)
{
#define MOE_TP(V)                                                                                                   \
    tile_pipe<BK, STAGES, G, V, GELU, BIAS, F32OUT, PART>(smem, lds0, b, cg, rw, ra, kt_lo, kt_hi, next, null_w,    \
                                                          null_a, C, bseg, part, row0, row_end, n0, N)
    if (G::FB == 4) {
        switch (nbv) {
        case 4: return MOE_TP(G::FB >= 4 ? 4 : G::FB);
        case 3: return MOE_TP(G::FB >= 3 ? 3 : G::FB);
        default: break;
        }
    }
    switch (nbv) {
    case 2: return MOE_TP(G::FB >= 2 ? 2 : G::FB);
    case 1: return MOE_TP(1);
    default: return MOE_TP(0);
    }
#undef MOE_TP
}

// Work item i of a block: its whole tiles (an XCD-contiguous share of
// [0, F), as in grouped_gemm_bf16_256), then its tail unit if it has one.
struct Work {
    TileLoc t;
    int kt_lo, kt_hi;
    int unit; // tail unit, or -1 for a whole tile
};

// Needs K / BK >= STAGES - 1 (the tail plan keeps every K range that long).
template <int BK, int STAGES, class G, bool GELU, bool BIAS, bool F32OUT>
__global__ __launch_bounds__(64 * G::NW, 1) void grouped_gemm_pipe(const uint16_t *__restrict__ A,
                                                                   const int32_t *__restrict__ seg, int S,
                                                                   int64_t max_rows, const uint16_t *__restrict__ W,
                                                                   const uint16_t *__restrict__ bias,
                                                                   void *__restrict__ C, int N, int K, int Ka,
                                                                   float *__restrict__ part_ws)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NQ = kL / (G::NW * RPI);
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * 2 * kL * BK];
    __shared__ int tb[kMaxSeg + 1];
    build_tile_prefix<kL>(seg, S, max_rows, tb);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::WGN_;
    const int NT = (N + kL - 1) / kL;
    const int KT = K / BK;
    const int64_t total = (int64_t)tb[S] * NT;
    const TailPlan plan = plan_tail(total, (int)gridDim.x, KT, part_ws != nullptr, STAGES - 1);

    const int xcd = blockIdx.x % kXcds;
    const int per = gridDim.x / kXcds;
    const int j = blockIdx.x / kXcds;
    const int64_t rlo = plan.F * xcd / kXcds, rhi = plan.F * (xcd + 1) / kXcds;
    const int64_t first = rlo + j;
    const int nw = first < rhi ? (int)((rhi - first + per - 1) / per) : 0;
    const int unit = blockIdx.x;
    const bool has_tail = plan.rem > 0 && unit < plan.rem * plan.sk;
    const int n_work = nw + (has_tail ? 1 : 0);
    if (n_work == 0)
        return;

    CopyGeo cg;
    {
        const int lrow = lane / CPR;
        const int prow = wave * RPI + lrow;
        const int lchunk = (lane % CPR) ^ swz<BK>(prow);
        cg.row_w = (uint32_t)K * 2u;
        cg.row_a = (uint32_t)Ka * 2u;
        cg.vbase = (uint32_t)prow * cg.row_w + (uint32_t)lchunk * 16u;
        cg.vbase_a = (uint32_t)prow * cg.row_a + (uint32_t)lchunk * 16u;
        cg.KTa = Ka / BK;
    }
    auto work = [&](int i) {
        Work w;
        if (i < nw) {
            w.t = locate(tb, seg, S, max_rows, NT, first + (int64_t)i * per);
            w.kt_lo = 0;
            w.kt_hi = KT;
            w.unit = -1;
        } else {
            const int c = unit % plan.sk;
            w.t = locate(tb, seg, S, max_rows, NT, plan.F + unit / plan.sk);
            w.kt_lo = (int)((int64_t)KT * c / plan.sk);
            w.kt_hi = (int)((int64_t)KT * (c + 1) / plan.sk);
            w.unit = unit;
        }
        return w;
    };
    auto src_of = [&](const Work &w, i32x4 &rw, i32x4 &ra) {
        const int wrows = min(kL, N - w.t.n0);
        const int arows = (int)(w.t.row_end - w.t.row0);
        rw = make_rsrc(W + (int64_t)w.t.s * N * K + (int64_t)w.t.n0 * K, (uint32_t)wrows * cg.row_w);
        ra = make_rsrc(A + w.t.row0 * Ka, (uint32_t)arows * cg.row_a);
    };
    const i32x4 null_w = make_rsrc(W, 0), null_a = make_rsrc(A, 0);

    const uint32_t lds0 = lds_addr(smem);
    Work w = work(0);
    i32x4 rw, ra;
    src_of(w, rw, ra);
    // Prologue: the first STAGES-1 K steps of the first work item.
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) {
        const Fill f = fill_at<BK>(rw, ra, w.kt_lo + p, cg.KTa);
#pragma unroll
        for (int i = 0; i < 2 * NQ; ++i)
            copy_one<BK, G>(cg, f, lds0 + (uint32_t)(p * 2 * kL * BK) * 2u, wave, i);
    }
    stage_barrier<(STAGES - 2) * 2 * NQ>();
    int b = 0;
    for (int i = 0; i < n_work; ++i) {
        Work wn = w;
        NextSrc next;
        next.any = i + 1 < n_work;
        next.rw = null_w;
        next.ra = null_a;
        next.kt_lo = 0;
        if (next.any) {
            wn = work(i + 1);
            src_of(wn, next.rw, next.ra);
            next.kt_lo = wn.kt_lo;
        }
        const int nbv = valid_b<G>(w.t, wm);
        if (w.unit < 0)
            b = tile_pipe_any<BK, STAGES, G, GELU, BIAS, F32OUT, false>(
                nbv, smem, lds0, b, cg, rw, ra, w.kt_lo, w.kt_hi, next, null_w, null_a, C,
                bias ? bias + (int64_t)w.t.s * N : nullptr, nullptr, w.t.row0, w.t.row_end, w.t.n0, N);
        else
            b = tile_pipe_any<BK, STAGES, G, GELU, BIAS, F32OUT, true>(
                nbv, smem, lds0, b, cg, rw, ra, w.kt_lo, w.kt_hi, next, null_w, null_a, C, nullptr,
                part_ws + (size_t)w.unit * (kL * kL), w.t.row0, w.t.row_end, w.t.n0, N);
        w = wn;
        rw = next.rw;
        ra = next.ra;
    }
}

// ---------------------------------------------------------------------------
// Register-staged form: operands marked REG go global -> VGPR two K steps
// ahead and VGPR -> LDS (ds_write) one step ahead; the others go by LDS-DMA
// one step ahead.  Two LDS stages plus the staged registers give three
// stages in flight.  Plain vector loads stream faster into the CU than LDS-DMA
// copies do, at the cost of the staging registers.
// ---------------------------------------------------------------------------

template <int BK, class G> struct Staged {
    static constexpr int DPW = 2 * (kL / (G::NW * (64 / (BK / 8))));
    u32x4 v[DPW];
};

// A stage source as plain scalars (base addresses and byte sizes of the
// tile's W and A rows); the buffer resources are formed where a copy is
// issued.  Sizes of zero make every copy out of range (zeros, no access).
struct Src2 {
    uint64_t wbase, abase;
    uint32_t wbytes, abytes;
};

struct Fill2 {
    Src2 s;
    uint32_t so_w, so_a;
};

template <int BK> __device__ __forceinline__ Fill2 fill2_at(const Src2 &s, int kt, int KTa)
{
    Fill2 f;
    f.s = s;
    f.so_w = (uint32_t)kt * (BK * 2);
    f.so_a = (uint32_t)(kt % KTa) * (BK * 2);
    return f;
}

__device__ __forceinline__ Src2 src2_of(const uint16_t *w, uint32_t wbytes, const uint16_t *a, uint32_t abytes)
{
    Src2 s;
    s.wbase = (uint64_t)uni64((int64_t)(uintptr_t)w);
    s.abase = (uint64_t)uni64((int64_t)(uintptr_t)a);
    s.wbytes = (uint32_t)uni((int)wbytes);
    s.abytes = (uint32_t)uni((int)abytes);
    return s;
}

__device__ __forceinline__ i32x4 raw_rsrc(uint64_t base, uint32_t bytes)
{
    return make_rsrc((const void *)(uintptr_t)base, bytes);
}

__device__ __forceinline__ u32x4 buf_load16(uint64_t base, uint32_t bytes, uint32_t voff, uint32_t soff)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)base, (short)0, (int)bytes, kRsrcWord3);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Order in which a K step issues its copies: LDS-DMA ones first, then the
// register loads (so a wait that leaves the register loads in flight has
// the LDS-DMA copies landed).
template <bool WREG, bool AREG, int DPW> __device__ __forceinline__ constexpr int copy_order(int n)
{
    return (WREG == AREG) ? n : (!WREG ? (n < DPW / 2 ? 2 * n : 2 * (n - DPW / 2) + 1)
                                       : (n < DPW / 2 ? 2 * n + 1 : 2 * (n - DPW / 2)));
}

// Copy i of a stage: scalar offset of its rows.
template <int BK, class G>
__device__ __forceinline__ uint32_t copy_soff(const CopyGeo &cg, const Fill2 &f, int i)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NW = G::NW;
    const int q = i >> 1;
    return (i & 1) ? (uint32_t)q * (uint32_t)(NW * RPI) * cg.row_a + f.so_a
                   : (uint32_t)q * (uint32_t)(NW * RPI) * cg.row_w + f.so_w;
}

// LDS byte offset (within a stage) of copy i's 16 bytes for this lane.
template <int BK, class G> __device__ __forceinline__ uint32_t copy_ldsoff(int wave, int lane, int i)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NW = G::NW;
    const int q = i >> 1;
    const uint32_t R = (uint32_t)((NW * q + wave) * RPI);
    return (uint32_t)((i & 1) * (kL * BK) + R * BK) * 2u + (uint32_t)lane * 16u;
}

template <bool WREG, bool AREG> __device__ __forceinline__ constexpr bool in_reg(int i)
{
    return (i & 1) ? AREG : WREG;
}

#ifndef MOE_PIPE_FA1
#define MOE_PIPE_FA1 0 // 1: single-buffered A fragments (fewer registers, exposed LDS latency)
#endif
#ifndef MOE_PIPE_WSP
#define MOE_PIPE_WSP 8 // the staged registers go to LDS over the first WSP chunks of a K step
#endif

template <int BK, class G, int NBV, bool WREG, bool AREG>
__device__ __forceinline__ void k_step_pipe2(const uint16_t *cur, uint16_t *nxt, uint32_t nxt_lds, const Fill2 &f1,
                                             const Fill2 &f2, Staged<BK, G> &stg, const CopyGeo &cg,
                                             f32x16 (&acc)[G::FA][G::FB], bf16x8 (&fa)[2][G::FA],
                                             bf16x8 (&fb)[2][G::FB], int wave, int lane, int wn, int wm, int r32,
                                             int khalf, int sw)
{
    constexpr int FA = G::FA, FB = G::FB;
    constexpr int KS = BK / 16;
    constexpr int DPW = Staged<BK, G>::DPW;
    constexpr int NDMA = (WREG ? 0 : DPW / 2) + (AREG ? 0 : DPW / 2);
    constexpr int NREG = DPW - NDMA;
    constexpr int CPS = MOE_PIPE_CPS < FA * FB ? MOE_PIPE_CPS : FA * FB;
    constexpr int MPC = FA * FB / CPS;
    constexpr int RDS = FA + FB;
    constexpr int RCH = MOE_PIPE_RCH < CPS ? MOE_PIPE_RCH : CPS;
    constexpr int RPC = (RDS + RCH - 1) / RCH;
    constexpr int NPRE = (KS - 1) * CPS;
    constexpr int WSP = MOE_PIPE_WSP < NPRE ? MOE_PIPE_WSP : NPRE; // chunks the register writes spread over
    static_assert(KS >= 2 && (FA * FB) % CPS == 0, "chunking");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint16_t *src = ks + 1 < KS ? cur : nxt;
        const int kn = ks + 1 < KS ? ks + 1 : 0;
#pragma unroll
        for (int c = 0; c < CPS; ++c) {
            if (NBV > 0) {
#pragma unroll
                for (int m = 0; m < MPC; ++m) {
                    const int i = c * MPC + m;
                    const int a = i / FB, b = i % FB;
                    if (b < NBV)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[MOE_PIPE_FA1 ? 0 : ks & 1][a],
                                                                            fb[ks & 1][b], acc[a][b], 0, 0, 0);
                    if (MOE_PIPE_FA1) {
                        // A fragment a is single-buffered: its next sub-step's
                        // value is read once its last MFMA (a, FB-1) has issued;
                        // B fragments are double-buffered and read first.
                        if (i < FB)
                            read_frag<BK, G, NBV>(src, kn, fa[0], fb[(ks + 1) & 1], FA + i, wn, wm, r32, khalf, sw);
                        if (b == FB - 1)
                            read_frag<BK, G, NBV>(src, kn, fa[0], fb[(ks + 1) & 1], a, wn, wm, r32, khalf, sw);
                    } else {
#pragma unroll
                        for (int q = 0; q < RPC; ++q) {
                            const int r = c * RPC + q;
                            if (c < RCH && r < RDS && (q * MPC) / RPC == m)
                                read_frag<BK, G, NBV>(src, kn, fa[(ks + 1) & 1], fb[(ks + 1) & 1], read_slot<G>(r),
                                                      wn, wm, r32, khalf, sw);
                        }
                    }
                }
                if (NBV == FB) {
#pragma unroll
                    for (int m = 0; m < MPC; ++m) {
                        const int i = c * MPC + m;
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (MOE_PIPE_FA1) {
                            if (i < FB)
                                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                            if (i % FB == FB - 1)
                                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        } else {
#pragma unroll
                            for (int q = 0; q < RPC; ++q)
                                if (c < RCH && c * RPC + q < RDS && (q * MPC) / RPC == m)
                                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        }
                    }
                }
            }
            if (ks + 1 < KS) {
                const int g = ks * CPS + c;
                __builtin_amdgcn_sched_barrier(0);
                if (NREG > 0) {
                    // staged registers (K step kt+1) -> the next stage, spread
                    // over the first WSP chunks; register j is reloaded only in
                    // this chunk or a later one (after its write)
#pragma unroll
                    for (int j = 0; j < DPW; ++j)
                        if (in_reg<WREG, AREG>(j) && (j * WSP) / DPW == g)
                            *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(nxt) + copy_ldsoff<BK, G>(wave, lane, j)) =
                                stg.v[j];
                }
                // copies in order: LDS-DMA ones (step kt+1) first, then the
                // register loads (step kt+2); copy n goes after chunk n*NPRE/DPW
#pragma unroll
                for (int n = 0; n < DPW; ++n) {
                    if ((n * NPRE) / DPW != g)
                        continue;
                    const int j = copy_order<WREG, AREG, DPW>(n);
                    if (!in_reg<WREG, AREG>(j)) {
                        const uint32_t so = copy_soff<BK, G>(cg, f1, j);
                        dma16((j & 1) ? raw_rsrc(f1.s.abase, f1.s.abytes) : raw_rsrc(f1.s.wbase, f1.s.wbytes),
                              (j & 1) ? cg.vbase_a : cg.vbase, so, nxt_lds + copy_ldsoff<BK, G>(wave, 0, j));
                    } else {
                        const uint32_t so = copy_soff<BK, G>(cg, f2, j);
                        stg.v[j] = (j & 1) ? buf_load16(f2.s.abase, f2.s.abytes, cg.vbase_a, so)
                                           : buf_load16(f2.s.wbase, f2.s.wbytes, cg.vbase, so);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (ks == KS - 2) {
            // the next stage is complete (its copies and register writes);
            // the register loads of the stage after it may be in flight
            __builtin_amdgcn_sched_barrier(0);
            stage_barrier<NREG>();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One tile (or one K range of a tail tile) of the register-staged kernel.
// On entry LDS stage b holds its first K step (landed, behind a barrier) and
// the staged registers hold its second; on exit the same holds for the next
// work item (sw*/sa*: own rows; nw*/na*: the next item's, sizes 0 if none).
template <int BK, class G, int NBV, bool WREG, bool AREG, bool GELU, bool BIAS, bool F32OUT, bool PART>
__device__ __forceinline__ int tile_pipe2(uint16_t *smem, uint32_t lds0, int b, const CopyGeo &cg, uint64_t swb,
                                          uint64_t sab, uint32_t sws, uint32_t sas, int kt_lo, int kt_hi,
                                          uint64_t nwb, uint64_t nab, uint32_t nws, uint32_t nas, int n_kt_lo,
                                          Staged<BK, G> &stg, void *C, const uint16_t *bseg, float *part,
                                          int64_t row0, int64_t row_end, int n0, int N)
{
    constexpr int FA = G::FA, FB = G::FB, STAGE = 2 * kL * BK;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WGN_, wm = wave / G::WGN_;
    const int r32 = lane & 31, khalf = lane >> 5;
    const int sw = swz<BK>(r32);

    f32x16 acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int q = 0; q < FB; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[a][q][v] = 0.f;
    bf16x8 fa[2][FA], fb[2][FB];
    if (NBV > 0) {
#pragma unroll
        for (int r = 0; r < FA + FB; ++r)
            read_frag<BK, G, NBV>(smem + b * STAGE, 0, fa[0], fb[0], r, wn, wm, r32, khalf, sw);
    }
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        // K steps kt+1 (LDS-DMA operands) and kt+2 (register operands): own
        // rows while inside [kt_lo, kt_hi), else the next item's first steps.
        Fill2 f1, f2;
        {
            const bool own = kt + 1 < kt_hi;
            f1.s.wbase = own ? swb : nwb;
            f1.s.abase = own ? sab : nab;
            f1.s.wbytes = own ? sws : nws;
            f1.s.abytes = own ? sas : nas;
            const int k1 = own ? kt + 1 : n_kt_lo + (kt + 1 - kt_hi);
            f1.so_w = (uint32_t)k1 * (BK * 2);
            f1.so_a = (uint32_t)(k1 % cg.KTa) * (BK * 2);
        }
        {
            const bool own = kt + 2 < kt_hi;
            f2.s.wbase = own ? swb : nwb;
            f2.s.abase = own ? sab : nab;
            f2.s.wbytes = own ? sws : nws;
            f2.s.abytes = own ? sas : nas;
            const int k2 = own ? kt + 2 : n_kt_lo + (kt + 2 - kt_hi);
            f2.so_w = (uint32_t)k2 * (BK * 2);
            f2.so_a = (uint32_t)(k2 % cg.KTa) * (BK * 2);
        }
        const int bn = b ^ 1;
        k_step_pipe2<BK, G, NBV, WREG, AREG>(smem + b * STAGE, smem + bn * STAGE, lds0 + (uint32_t)(bn * STAGE) * 2u,
                                             f1, f2, stg, cg, acc, fa, fb, wave, lane, wn, wm, r32, khalf, sw);
        b = bn;
    }
    if (PART) {
        float *dst = part + (size_t)wave * (FA * FB * 16 * 64) + lane;
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int q = 0; q < FB; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dst[((a * FB + q) * 16 + v) * 64] = acc[a][q][v];
    } else {
        store_tile<G, NBV, GELU, BIAS, F32OUT>(acc, C, bseg, row0, row_end, n0, N, wn, wm, r32, khalf);
    }
    return b;
}

template <int BK, class G, bool WREG, bool AREG, bool GELU, bool BIAS, bool F32OUT, bool PART>
__device__ __forceinline__ int tile_pipe2_any(int nbv, uint16_t *smem, uint32_t lds0, int b, const CopyGeo &cg,
                                              uint64_t swb, uint64_t sab, uint32_t sws, uint32_t sas, int kt_lo,
                                              int kt_hi, uint64_t nwb, uint64_t nab, uint32_t nws, uint32_t nas,
                                              int n_kt_lo, Staged<BK, G> &stg, void *C, const uint16_t *bseg,
                                              float *part, int64_t row0, int64_t row_end, int n0, int N)
{
#define MOE_TP2(V)                                                                                                  \
    tile_pipe2<BK, G, V, WREG, AREG, GELU, BIAS, F32OUT, PART>(smem, lds0, b, cg, swb, sab, sws, sas, kt_lo, kt_hi, \
                                                               nwb, nab, nws, nas, n_kt_lo, stg, C, bseg, part,     \
                                                               row0, row_end, n0, N)
    if (G::FB == 4) {
        switch (nbv) {
        case 4: return MOE_TP2(G::FB >= 4 ? 4 : G::FB);
        case 3: return MOE_TP2(G::FB >= 3 ? 3 : G::FB);
        default: break;
        }
    }
    switch (nbv) {
    case 2: return MOE_TP2(G::FB >= 2 ? 2 : G::FB);
    case 1: return MOE_TP2(1);
    default: return MOE_TP2(0);
    }
#undef MOE_TP2
}

// Work item i of a block: its whole tiles (an XCD-contiguous share of
// [0, F)), then its tail unit if it has one; all fields wave-uniform.
__device__ __forceinline__ Work get_work(int i, int nw, int64_t first, int per, int unit, const TailPlan &plan,
                                         const int *tb, const int32_t *seg, int S, int64_t max_rows, int NT, int KT)
{
    Work w;
    if (i < nw) {
        w.t = locate(tb, seg, S, max_rows, NT, first + (int64_t)i * per);
        w.kt_lo = 0;
        w.kt_hi = KT;
        w.unit = -1;
    } else {
        const int c = unit % plan.sk;
        w.t = locate(tb, seg, S, max_rows, NT, plan.F + unit / plan.sk);
        w.kt_lo = (int)((int64_t)KT * c / plan.sk);
        w.kt_hi = (int)((int64_t)KT * (c + 1) / plan.sk);
        w.unit = unit;
    }
    w.t.s = uni(w.t.s);
    w.t.row0 = uni64(w.t.row0);
    w.t.row_end = uni64(w.t.row_end);
    w.t.n0 = uni(w.t.n0);
    w.kt_lo = uni(w.kt_lo);
    w.kt_hi = uni(w.kt_hi);
    return w;
}

// Needs K / BK >= 2 (the tail plan keeps every K range that long).
template <int BK, class G, bool WREG, bool AREG, bool GELU, bool BIAS, bool F32OUT>
__global__ __launch_bounds__(64 * G::NW, 1) void grouped_gemm_pipe2(const uint16_t *__restrict__ A,
                                                                    const int32_t *__restrict__ seg, int S,
                                                                    int64_t max_rows, const uint16_t *__restrict__ W,
                                                                    const uint16_t *__restrict__ bias,
                                                                    void *__restrict__ C, int N, int K, int Ka,
                                                                    float *__restrict__ part_ws)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    constexpr int DPW = Staged<BK, G>::DPW;
    constexpr int NDMA = (WREG ? 0 : DPW / 2) + (AREG ? 0 : DPW / 2);
    constexpr int NREG = DPW - NDMA;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * kL * BK];
    __shared__ int tb[kMaxSeg + 1];
    build_tile_prefix<kL>(seg, S, max_rows, tb);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::WGN_;
    const int NT = (N + kL - 1) / kL;
    const int KT = K / BK;
    const int64_t total = (int64_t)tb[S] * NT;
    const TailPlan plan = plan_tail(total, (int)gridDim.x, KT, part_ws != nullptr, 2);

    const int xcd = blockIdx.x % kXcds;
    const int per = gridDim.x / kXcds;
    const int jb = blockIdx.x / kXcds;
    const int64_t rlo = plan.F * xcd / kXcds, rhi = plan.F * (xcd + 1) / kXcds;
    const int64_t first = rlo + jb;
    const int nw = first < rhi ? (int)((rhi - first + per - 1) / per) : 0;
    const int unit = blockIdx.x;
    const bool has_tail = plan.rem > 0 && unit < plan.rem * plan.sk;
    const int n_work = nw + (has_tail ? 1 : 0);
    if (n_work == 0)
        return;

    CopyGeo cg;
    {
        const int lrow = lane / CPR;
        const int prow = wave * RPI + lrow;
        const int lchunk = (lane % CPR) ^ swz<BK>(prow);
        cg.row_w = (uint32_t)K * 2u;
        cg.row_a = (uint32_t)Ka * 2u;
        cg.vbase = (uint32_t)prow * cg.row_w + (uint32_t)lchunk * 16u;
        cg.vbase_a = (uint32_t)prow * cg.row_a + (uint32_t)lchunk * 16u;
        cg.KTa = Ka / BK;
    }
    const uint32_t lds0 = lds_addr(smem);

    Work w = get_work(0, nw, first, per, unit, plan, tb, seg, S, max_rows, NT, KT);
    uint64_t swb = (uint64_t)(uintptr_t)(W + (int64_t)w.t.s * N * K + (int64_t)w.t.n0 * K);
    uint64_t sab = (uint64_t)(uintptr_t)(A + w.t.row0 * Ka);
    uint32_t sws = (uint32_t)min(kL, N - w.t.n0) * cg.row_w;
    uint32_t sas = (uint32_t)(w.t.row_end - w.t.row0) * cg.row_a;
    Staged<BK, G> stg;
    // Prologue: K step kt_lo into LDS stage 0, kt_lo+1 into the staged registers.
    {
        Fill2 f0;
        f0.s.wbase = swb;
        f0.s.abase = sab;
        f0.s.wbytes = sws;
        f0.s.abytes = sas;
        f0.so_w = (uint32_t)w.kt_lo * (BK * 2);
        f0.so_a = (uint32_t)(w.kt_lo % cg.KTa) * (BK * 2);
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const uint32_t so = copy_soff<BK, G>(cg, f0, i);
            if (in_reg<WREG, AREG>(i))
                stg.v[i] = (i & 1) ? buf_load16(sab, sas, cg.vbase_a, so) : buf_load16(swb, sws, cg.vbase, so);
            else
                dma16((i & 1) ? raw_rsrc(sab, sas) : raw_rsrc(swb, sws), (i & 1) ? cg.vbase_a : cg.vbase, so,
                      lds0 + copy_ldsoff<BK, G>(wave, 0, i));
        }
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            if (in_reg<WREG, AREG>(i))
                *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(smem) + copy_ldsoff<BK, G>(wave, lane, i)) =
                    stg.v[i];
        wait_vmcnt<0>();
        f0.so_w = (uint32_t)(w.kt_lo + 1) * (BK * 2);
        f0.so_a = (uint32_t)((w.kt_lo + 1) % cg.KTa) * (BK * 2);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            if (in_reg<WREG, AREG>(i))
                stg.v[i] = (i & 1) ? buf_load16(sab, sas, cg.vbase_a, copy_soff<BK, G>(cg, f0, i))
                                   : buf_load16(swb, sws, cg.vbase, copy_soff<BK, G>(cg, f0, i));
        stage_barrier<NREG>();
    }
    int b = 0;
    for (int i = 0; i < n_work; ++i) {
        Work wn = w;
        uint64_t nwb = swb, nab = sab;
        uint32_t nws = 0, nas = 0;
        if (i + 1 < n_work) {
            wn = get_work(i + 1, nw, first, per, unit, plan, tb, seg, S, max_rows, NT, KT);
            nwb = (uint64_t)(uintptr_t)(W + (int64_t)wn.t.s * N * K + (int64_t)wn.t.n0 * K);
            nab = (uint64_t)(uintptr_t)(A + wn.t.row0 * Ka);
            nws = (uint32_t)min(kL, N - wn.t.n0) * cg.row_w;
            nas = (uint32_t)(wn.t.row_end - wn.t.row0) * cg.row_a;
        }
        const int nbv = valid_b<G>(w.t, wm);
        if (w.unit < 0)
            b = tile_pipe2_any<BK, G, WREG, AREG, GELU, BIAS, F32OUT, false>(
                nbv, smem, lds0, b, cg, swb, sab, sws, sas, w.kt_lo, w.kt_hi, nwb, nab, nws, nas, wn.kt_lo, stg, C,
                bias ? bias + (int64_t)w.t.s * N : nullptr, nullptr, w.t.row0, w.t.row_end, w.t.n0, N);
        else
            b = tile_pipe2_any<BK, G, WREG, AREG, GELU, BIAS, F32OUT, true>(
                nbv, smem, lds0, b, cg, swb, sab, sws, sas, w.kt_lo, w.kt_hi, nwb, nab, nws, nas, wn.kt_lo, stg, C,
                nullptr, part_ws + (size_t)w.unit * (kL * kL), w.t.row0, w.t.row_end, w.t.n0, N);
        w = wn;
        swb = nwb;
        sab = nab;
        sws = nws;
        sas = nas;
    }
}

// Sums the K-range partials of each tail tile in range order and applies the
// bias, activation and bf16 store; a no-op when the GEMM had no split tail.
// Block = (tail tile, GEMM wave w); its FA waves take the feature sub-tiles
// a and loop over the row sub-tiles b.  Each lane loads its 16 accumulators
// of every K range up front (independent loads), then sums in range order.
template <class G, bool GELU, bool BIAS, bool F32OUT>
__global__ __launch_bounds__(64 * G::FA) void grouped_gemm_reduce(const int32_t *__restrict__ seg, int S,
                                                                  int64_t max_rows, const uint16_t *__restrict__ bias,
                                                                  void *__restrict__ C, int N, int K, int BKused,
                                                                  int min_len, int Gsize,
                                                                  const float *__restrict__ part_ws)
{
    __shared__ int tb[kMaxSeg + 1];
    build_tile_prefix<kL>(seg, S, max_rows, tb);
    const int NT = (N + kL - 1) / kL;
    const int64_t total = (int64_t)tb[S] * NT;
    const TailPlan plan = plan_tail(total, Gsize, K / BKused, true, min_len);
    const int tile = blockIdx.x / G::NW, wave = blockIdx.x % G::NW;
    if (plan.rem == 0 || tile >= plan.rem)
        return;
    const int lane = threadIdx.x & 63, a = threadIdx.x >> 6;
    const int wn = wave % G::WGN_, wm = wave / G::WGN_;
    const int r32 = lane & 31, khalf = lane >> 5;
    const TileLoc t = locate(tb, seg, S, max_rows, NT, plan.F + tile);
    const uint16_t *bseg = bias ? bias + (int64_t)t.s * N : nullptr;
    for (int b = 0; b < G::FB; ++b) {
        const float *src = part_ws + (size_t)tile * plan.sk * (kL * kL) +
                           (size_t)wave * (G::FA * G::FB * 16 * 64) + (size_t)((a * G::FB + b) * 16) * 64 + lane;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            v[r] = src[(size_t)r * 64];
#pragma unroll
        for (int c = 1; c < 8; ++c) {
            if (c < plan.sk) {
                float w[16];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    w[r] = src[(size_t)c * (kL * kL) + (size_t)r * 64];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    v[r] += w[r];
            }
        }
        const int64_t row = t.row0 + wm * G::WTM + b * 32 + r32;
        const bool row_ok = row < t.row_end;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = t.n0 + wn * G::WTN + a * 32 + 8 * g + 4 * khalf;
            store4<GELU, BIAS, F32OUT>(C, bseg, row, row_ok, n, N, v[4 * g], v[4 * g + 1], v[4 * g + 2],
                                       v[4 * g + 3]);
        }
    }
}

// fp32: 64 x 64 tiles, 4 x 4 per thread, K slices of 16 through LDS.
template <bool GELU>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float *__restrict__ A, const int32_t *__restrict__ seg,
                                                        int S, int64_t max_rows, const float *__restrict__ W,
                                                        const float *__restrict__ bias, float *__restrict__ C, int N,
                                                        int K)
{
    constexpr int TM = 64, TN = 64, TK = 16;
    __shared__ float sa[TK][TM + 4];
    __shared__ float sw[TK][TN + 4];
    __shared__ int tb[kMaxSeg + 1];
    build_tile_prefix<TM>(seg, S, max_rows, tb);
    const int64_t mt = blockIdx.y;
    if (mt >= tb[S])
        return;
    const int s = find_segment(tb, S, 1, mt);
    int64_t seg_lo, seg_hi;
    seg_bounds(seg, s, max_rows, seg_lo, seg_hi);
    const int64_t row0 = seg_lo + (mt - tb[s]) * TM;
    const int64_t row_end = min(row0 + TM, seg_hi);
    const int n0 = blockIdx.x * TN;
    const float *wbase = W + (int64_t)s * N * K;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
        for (int q = tid; q < TM * TK; q += 256) {
            const int r = q / TK, kk = q % TK;
            const int64_t row = min(row0 + r, row_end - 1);
            const int n = min(n0 + r, N - 1);
            sa[kk][r] = (k0 + kk < K) ? A[row * K + k0 + kk] : 0.f;
            sw[kk][r] = (k0 + kk < K) ? wbase[(int64_t)n * K + k0 + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float av[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = sa[kk][ty * 4 + i];
                wv[i] = sw[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[i][q] = fmaf(av[i], wv[q], acc[i][q]);
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + ty * 4 + i;
        if (row >= row_end)
            continue;
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx * 4 + q;
            if (n >= N)
                continue;
            float v = acc[i][q];
            if (bias)
                v += bias[(int64_t)s * N + n];
            if (GELU)
                v = gelu_erf(v);
            C[row * N + n] = v;
        }
    }
}

int device_cus()
{
    static thread_local int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 2
#endif
#ifndef MOE_GEMM_WGM
#define MOE_GEMM_WGM 4
#endif
#ifndef MOE_GEMM_PIPE
#define MOE_GEMM_PIPE 2
#endif
#ifndef MOE_PIPE_WREG
#define MOE_PIPE_WREG 1
#endif
#ifndef MOE_PIPE_AREG
#define MOE_PIPE_AREG 1
#endif
constexpr int kLargeBK = MOE_GEMM_BK, kLargeStages = MOE_GEMM_STAGES;
typedef Grid<2, MOE_GEMM_WGM> LargeGrid;

// One block per CU (a multiple of the XCD count).  With a split-K workspace
// a problem of few tiles still fills the chip (the tail plan cuts their K);
// without one, blocks beyond the tile count would only idle.
int large_grid(int64_t max_rows, int S, int N, bool split)
{
    const int64_t tiles_bound = ((max_rows + kL - 1) / kL + S) * (int64_t)((N + kL - 1) / kL);
    int64_t grid = (int64_t)device_cus();
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    const int64_t need = (tiles_bound + kXcds - 1) / kXcds * kXcds;
    if (!split && need < grid)
        grid = need;
    if (grid < kXcds)
        grid = kXcds;
    return (int)grid;
}

template <bool GELU, bool BIAS, bool F32OUT>
moe_status_t run_large(const void *a, const int32_t *seg, int S, int64_t max_rows, int N, int K, int Ka,
                       const void *w, const void *bias, void *out, float *part_ws, hipStream_t stream)
{
    typedef LargeGrid G;
    const int grid = large_grid(max_rows, S, N, part_ws != nullptr);
#if MOE_GEMM_PIPE == 2
    const int min_len = 2;
    grouped_gemm_pipe2<kLargeBK, G, MOE_PIPE_WREG, MOE_PIPE_AREG, GELU, BIAS, F32OUT>
        <<<(unsigned)grid, 64 * G::NW, 0, stream>>>((const uint16_t *)a, seg, S, max_rows, (const uint16_t *)w,
                                                     (const uint16_t *)bias, out, N, K, Ka, part_ws);
#elif MOE_GEMM_PIPE
    const int min_len = kLargeStages - 1;
    grouped_gemm_pipe<kLargeBK, kLargeStages, G, GELU, BIAS, F32OUT><<<(unsigned)grid, 64 * G::NW, 0, stream>>>(
        (const uint16_t *)a, seg, S, max_rows, (const uint16_t *)w, (const uint16_t *)bias, out, N, K, Ka, part_ws);
#else
    const int min_len = 1;
    grouped_gemm_bf16_256<kLargeBK, kLargeStages, G, GELU, BIAS, F32OUT><<<(unsigned)grid, 64 * G::NW, 0, stream>>>(
        (const uint16_t *)a, seg, S, max_rows, (const uint16_t *)w, (const uint16_t *)bias, out, N, K, Ka, part_ws);
#endif
    if (moe_status_t st = check_launch("grouped_gemm_bf16_256"))
        return st;
    if (!part_ws)
        return MOE_OK;
    grouped_gemm_reduce<G, GELU, BIAS, F32OUT><<<(unsigned)(grid / 2 * G::NW), 64 * G::FA, 0, stream>>>(
        seg, S, max_rows, (const uint16_t *)bias, out, N, K, kLargeBK, min_len, grid, part_ws);
    return check_launch("grouped_gemm_reduce");
}

moe_status_t run_bf16_256(const void *a, const int32_t *seg, int S, int64_t max_rows, int N, int K, const void *w,
                         const void *bias, int act, void *out, float *part_ws, hipStream_t stream)
{
    if (act == 1)
        return bias ? run_large<true, true, false>(a, seg, S, max_rows, N, K, K, w, bias, out, part_ws, stream)
                    : run_large<true, false, false>(a, seg, S, max_rows, N, K, K, w, bias, out, part_ws, stream);
    return bias ? run_large<false, true, false>(a, seg, S, max_rows, N, K, K, w, bias, out, part_ws, stream)
                : run_large<false, false, false>(a, seg, S, max_rows, N, K, K, w, bias, out, part_ws, stream);
}

template <int BN, int BM>
moe_status_t run_bf16(const void *a, const int32_t *seg, int S, int64_t max_rows, int N, int K, const void *w,
                      const void *bias, int act, void *out, hipStream_t stream)
{
    const int64_t tiles_bound = ((max_rows + BM - 1) / BM + S) * (int64_t)((N + BN - 1) / BN);
    int64_t grid = (int64_t)device_cus() * 2;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    const int64_t need = (tiles_bound + kXcds - 1) / kXcds * kXcds;
    if (need < grid)
        grid = need;
    if (grid < kXcds)
        grid = kXcds;
    if (act == 1)
        grouped_gemm_bf16<BN, BM, true><<<(unsigned)grid, 256, 0, stream>>>(
            (const uint16_t *)a, seg, S, max_rows, (const uint16_t *)w, (const uint16_t *)bias, (uint16_t *)out, N, K);
    else
        grouped_gemm_bf16<BN, BM, false><<<(unsigned)grid, 256, 0, stream>>>(
            (const uint16_t *)a, seg, S, max_rows, (const uint16_t *)w, (const uint16_t *)bias, (uint16_t *)out, N, K);
    return check_launch("grouped_gemm_bf16");
}

} // namespace

size_t gemm_ws_bytes()
{
    int64_t grid = (int64_t)device_cus();
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    return (size_t)grid * kL * kL * sizeof(float);
}

moe_status_t launch_grouped_gemm(const void *a, const int32_t *seg_offsets, int num_segments, int64_t max_rows,
                                 int N, int K, moe_dtype_t dt, const void *w, const void *bias, int activation,
                                 void *out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (max_rows == 0)
        return MOE_OK;
    const int S = seg_offsets ? num_segments : 1;
    if (dt == MOE_BF16) {
        if (K % 64 == 0 && K / kLargeBK >= (MOE_GEMM_PIPE == 2 ? 2 : kLargeStages - 1)) {
            float *part = (ws && ws_bytes >= gemm_ws_bytes()) ? (float *)ws : nullptr;
            return run_bf16_256(a, seg_offsets, S, max_rows, N, K, w, bias, activation, out, part, stream);
        }
        return run_bf16<128, 128>(a, seg_offsets, S, max_rows, N, K, w, bias, activation, out, stream);
    }
    const dim3 g((unsigned)((N + 63) / 64), (unsigned)((max_rows + 63) / 64 + S));
    if (activation == 1)
        grouped_gemm_f32<true><<<g, 256, 0, stream>>>((const float *)a, seg_offsets, S, max_rows, (const float *)w,
                                                       (const float *)bias, (float *)out, N, K);
    else
        grouped_gemm_f32<false><<<g, 256, 0, stream>>>((const float *)a, seg_offsets, S, max_rows, (const float *)w,
                                                        (const float *)bias, (float *)out, N, K);
    return check_launch("grouped_gemm_f32");
}

moe_status_t launch_router_gemm(const void *x, const void *w3, int64_t T, int d, int E, float *logits, void *ws,
                                size_t ws_bytes, hipStream_t stream)
{
    // logits3[T, 3E]: column p*E + e = x . (bf16 piece p of router row e)
    float *part = (ws && ws_bytes >= gemm_ws_bytes()) ? (float *)ws : nullptr;
    return run_large<false, false, true>(x, nullptr, 1, T, 3 * E, d, d, w3, nullptr, logits, part, stream);
}

} // namespace moe
