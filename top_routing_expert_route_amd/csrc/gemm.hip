// Grouped GEMM of the MoE layer: one Linear of every expert over its segment
// of expert-contiguous rows, with the bias and (for the first Linear) the
// exact GELU fused into the epilogue.
//
// Pages: "Expert Parallelism (MoE)", section "MoE Layer Structure" (each
// expert applies Linear(d -> 4d) -> GELU -> Linear(4d -> d)) and "Expert
// Parallelism (EP)", section "Key math / How it works" (the expert GEMMs run
// locally on the rows dispatched to this GPU).
//
// bf16 kernels (gfx950 matrix cores)
//  - out[r, n] = act(sum_k a[r, k] w[s, n, k] + b[s, n]) is computed as
//    out^T = W . A^T: the weight rows are the MFMA "A" operand and the token
//    rows the "B" operand, so each lane's accumulators hold 4 consecutive
//    output features of one row (8-byte bf16 stores).  32x32x16 bf16 MFMAs,
//    fp32 accumulation.
//  - Persistent grid.  The tile list is derived on the device from the
//    segment offsets (no host round trip): segment s contributes
//    ceil(rows_s / BM) * (N / BN) tiles, ordered (segment, feature tile,
//    row tile) so that consecutive tiles share one weight tile.  Blocks are
//    dealt to the 8 XCDs round-robin by the hardware, so each XCD is given one
//    contiguous range of the tile list: the tiles that share weights run on
//    the same L2.
//  - grouped_gemm_256 (K % 64 == 0, the main path): 256 x 256 tiles, eight
//    waves, register-staged three-deep operand pipeline, split-K for a short
//    last round (described at the kernel).
//  - grouped_gemm_bf16 (any K % 8 == 0): 128 x 128 tiles, four waves in a
//    2 x 2 grid; A and W staged through LDS with an XOR swizzle of the
//    16-byte chunks, double-buffered.  Rows past the segment end are clamped
//    on load and masked on store; K tails are zero-filled in 8-element chunks.
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
// Large-tile bf16 kernel: 256 (features) x 256 (rows) per block, eight waves
// in a 2 x 4 grid, each owning 128 x 64 as 4 x 2 MFMA 32x32x16 tiles (128
// fp32 accumulators per lane; two waves per SIMD, so that one wave's MFMAs
// cover the other's waits).
//
// Operand path, per K step of 64: both operand tiles (256 rows x 128 bytes
// each) go global -> VGPR (buffer loads, 16 bytes per lane) two steps ahead
// and VGPR -> LDS (ds_write_b128) one step ahead, into the LDS stage that is
// not being read.  The two LDS stages plus the staged registers keep three
// K steps in flight.  (On this access pattern plain vector loads stream into
// the CU markedly faster than LDS-DMA copies.)
//
// The block synchronises once per K step, before the last 16-wide sub-step:
// the next stage is then complete, and the last sub-step's MFMAs cover the
// LDS reads of the next stage's first sub-step, so the matrix pipe does not
// drain at step boundaries.  The last two steps of a tile already load the
// first two steps of the block's next tile: a new tile starts without a load
// bubble, and its loads overlap this tile's epilogue.
//
// LDS on gfx950 serves a ds_read_b128 16 lanes at a time over 64 banks
// (256 bytes): 16-byte chunk c of row r is stored at c ^ ((r >> 1) & 7), so
// the 16 rows read by one group of lanes at the same logical chunk hit 16
// distinct bank groups.
// Requires K % 64 == 0 and K >= 128; rows past the weight matrix or the
// segment end read as zeros (buffer range checking); row sub-tiles past the
// segment end skip their MFMAs; stores are masked.
// ---------------------------------------------------------------------------
constexpr int kL = 256; // tile edge
// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;

// Every wave got this far and every wave's LDS accesses issued so far have
// completed.  Global loads are not waited for here: the staged registers
// reach LDS through ds_writes, before which the compiler waits for the loads
// that filled them, so outstanding epilogue stores of the previous tile do
// not hold up the pipeline.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Logical 16-byte chunk stored at physical chunk p of a 64-element row.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Values the whole wave shares, held in scalar registers (the compiler
// cannot prove that values read from LDS are uniform).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave grid of a 256x256 tile: WGN waves along the features and WGM along
// the rows; each wave owns (256/WGN) x (256/WGM) as FA x FB MFMA tiles of
// 32x32.
// A K-major LDS tile holds 64 K-rows of 256 values; rows are padded to 576
// bytes so that the transposing reads of four consecutive K-rows fall on
// disjoint banks.
constexpr int kKmPitch = kL * 2 + 64;

template <int WGN, int WGM, bool WT_ = false, bool AT_ = false> struct Grid {
    static constexpr int WGN_ = WGN, WGM_ = WGM;
    // WT / AT: the weight / row operand is K-major ([K][N] or [K][M], the
    // K-segmented GEMM's dispatched rows as they are stored)
    static constexpr bool WT = WT_, AT = AT_;
    static constexpr int NW = WGN * WGM;
    static constexpr int WTN = kL / WGN, WTM = kL / WGM;
    static constexpr int FA = WTN / 32, FB = WTM / 32;
    // one LDS stage (K step of 64): the weight tile, then the row tile
    static constexpr int W_BYTES = WT ? 64 * kKmPitch : kL * 64 * 2;
    static constexpr int A_BYTES = AT ? 64 * kKmPitch : kL * 64 * 2;
    static constexpr int STAGE_ELEMS = (W_BYTES + A_BYTES) / 2;
};
typedef Grid<2, 4> LargeGrid;
typedef Grid<2, 4, true> LargeGridWT;
typedef Grid<2, 4, true, true> LargeGridKK;
constexpr int kLargeBK = 64;

// Epilogue of a 256x256 tile: bias, activation and store of the rows inside
// [row0, row_end) and features < N, as bf16 (rounded to nearest even) or,
// with F32OUT, as fp32.  Accumulators are read unconditionally and the
// stores go through a buffer record of the tile's rows: a masked lane gets
// an offset past the record and its store is dropped by the range check.
// With no branches, and the stores of every row sub-tile issued (empty ones
// are all dropped), each variant issues the same stores, so the compiler
// counts them exactly and does not drain them before the next tile's work.
// (Offsets are 32-bit: 256 x N x 4 bytes must fit, N <= 2^21.)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Output rows of one tile as a buffer record: rows [row0, row_end) of C.
struct TileOut {
    __amdgpu_buffer_rsrc_t r;
    int64_t row0;
};

template <bool F32OUT> __device__ __forceinline__ TileOut tile_out(void *C, int64_t row0, int64_t row_end, int N)
{
    constexpr uint32_t es = F32OUT ? 4u : 2u;
    TileOut rt;
    rt.row0 = row0;
    rt.r = __builtin_amdgcn_make_buffer_rsrc((char *)C + (size_t)row0 * N * es, (short)0,
                                             (int)((uint32_t)(row_end - row0) * (uint32_t)N * es), kRsrcWord3);
    return rt;
}

template <bool GELU, bool BIAS, bool F32OUT>
__device__ __forceinline__ void store4(const TileOut &rt, const uint16_t *__restrict__ bseg, int64_t row, bool row_ok,
                                       int n, int N, float v0, float v1, float v2, float v3)
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
    const uint32_t off = ok ? (uint32_t)((row - rt.row0) * N + n) * (F32OUT ? 4u : 2u) : 0x80000000u;
    if (F32OUT) {
        const f32x4 o = {v0, v1, v2, v3};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rt.r, off, 0, 0);
    } else {
        uint2 o;
        o.x = pack_bf16x2(v0, v1);
        o.y = pack_bf16x2(v2, v3);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), rt.r, off, 0, 0);
    }
}

// fp32 tile without bias or activation, through LDS: the accumulator layout
// gives each wave store 32 rows x 32 bytes, which a CU issues at a fraction
// of the rate of row-contiguous stores.  Four rounds per wave, each 32 rows x
// 64 features (8 KB of the wave's slice of the free LDS stage, 256-byte rows,
// 16-byte chunk c of row r at c ^ (r & 15)): the lanes write their
// accumulators, then read back and store 4 rows x 256 contiguous bytes per
// instruction.  The caller puts a barrier between this and the next writes
// to the stage.
template <class G, bool BIAS>
__device__ __forceinline__ void store_tile_f32_lds(const f32x16 (&acc)[G::FA][G::FB], float *C,
                                                   const uint16_t *__restrict__ bseg, char *lds, int64_t row0,
                                                   int64_t row_end, int n0, int N, int wave, int lane, int wn, int wm,
                                                   int r32, int khalf)
{
    static_assert(G::FA == 4 && G::FB == 2, "one 8 KB round per pair of A fragments and B fragment");
    const TileOut rt = tile_out<true>(C, row0, row_end, N);
    char *mine = lds + wave * 8192;
#pragma unroll
    for (int b = 0; b < G::FB; ++b) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = a2 * 8 + 2 * g + khalf;
                    const f32x16 &v = acc[2 * p + a2][b];
                    f32x4 o = {v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
                    if (BIAS) {
                        const int n = n0 + wn * G::WTN + (2 * p + a2) * 32 + 8 * g + 4 * khalf;
                        const uint2 bb = *reinterpret_cast<const uint2 *>(bseg + (n < N ? n : 0));
                        o[0] += bf16_bits_to_f32(bb.x & 0xFFFFu);
                        o[1] += bf16_bits_to_f32(bb.x >> 16);
                        o[2] += bf16_bits_to_f32(bb.y & 0xFFFFu);
                        o[3] += bf16_bits_to_f32(bb.y >> 16);
                    }
                    *reinterpret_cast<f32x4 *>(mine + r32 * 256 + ((c ^ (r32 & 15)) * 16)) = o;
                }
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int lr = 4 * q + (lane >> 4), c = lane & 15;
                const f32x4 o = *reinterpret_cast<const f32x4 *>(mine + lr * 256 + ((c ^ (lr & 15)) * 16));
                const int64_t row = row0 + wm * G::WTM + b * 32 + lr;
                const int n = n0 + wn * G::WTN + p * 64 + 4 * c;
                const bool ok = row < row_end && n < N;
                const uint32_t off = ok ? (uint32_t)((row - rt.row0) * N + n) * 4u : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rt.r, off, 0, 0);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); // reads done before the next round's writes
        }
    }
}

// bf16 tile (bias, GELU applied first) through LDS, as store_tile_f32_lds:
// two rounds per wave of 32 rows x 128 features (8-byte pieces written at
// piece c ^ 2 (r & 15) of 256-byte rows), read back and stored as 4 rows x
// 256 contiguous bytes per instruction.  N % 8 == 0.
template <class G, bool GELU, bool BIAS>
__device__ __forceinline__ void store_tile_bf16_lds(const f32x16 (&acc)[G::FA][G::FB], uint16_t *C,
                                                    const uint16_t *__restrict__ bseg, char *lds, int64_t row0,
                                                    int64_t row_end, int n0, int N, int wave, int lane, int wn,
                                                    int wm, int r32, int khalf)
{
    static_assert(G::FA == 4 && G::FB == 2, "one 8 KB round per B fragment");
    const TileOut rt = tile_out<false>(C, row0, row_end, N);
    char *mine = lds + wave * 8192;
#pragma unroll
    for (int b = 0; b < G::FB; ++b) {
#pragma unroll
        for (int a = 0; a < G::FA; ++a)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * G::WTN + a * 32 + 8 * g + 4 * khalf;
                float v0 = acc[a][b][4 * g], v1 = acc[a][b][4 * g + 1], v2 = acc[a][b][4 * g + 2],
                      v3 = acc[a][b][4 * g + 3];
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
                uint2 o;
                o.x = pack_bf16x2(v0, v1);
                o.y = pack_bf16x2(v2, v3);
                const int c8 = a * 8 + 2 * g + khalf;
                *reinterpret_cast<uint2 *>(mine + r32 * 256 + ((c8 ^ ((r32 & 15) << 1)) * 8)) = o;
            }
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int lr = 4 * q + (lane >> 4), c = lane & 15;
            const u32x4 o = *reinterpret_cast<const u32x4 *>(mine + lr * 256 + ((c ^ (lr & 15)) * 16));
            const int64_t row = row0 + wm * G::WTM + b * 32 + lr;
            const int n = n0 + wn * G::WTN + 8 * c;
            const bool ok = row < row_end && n < N;
            const uint32_t off = ok ? (uint32_t)((row - rt.row0) * N + n) * 2u : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b128(o, rt.r, off, 0, 0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); // reads done before the next round's writes
    }
}

// Split of the tile list over a persistent grid of G blocks.  F whole tiles
// run in full rounds (each block gets the same number); when the rest (`rem`
// tiles) would leave CUs idle, each of them is cut into `sk` K ranges of at
// least min_len steps (units u = sk * tile + range), written as fp32 partials
// and summed by grouped_gemm_reduce.  Block b takes units b, b + G, ...: one
// each when rem is at most half a round (sk up to 8); up to 2/3 of a round,
// for tiles of at least kTailSplit3MinKT K steps, three ranges and at most two
// units per block, so the last round takes two thirds of a tile's time
// instead of a whole one (a fuller round is not split: two units of half a
// tile gain nothing; with shorter tiles the third saved is less than the
// partials' stores and the reduce cost).  The partial workspace holds 2G
// tiles.  Computed identically by both kernels.
struct TailPlan {
    int64_t F;
    int rem;
    int sk;
};

constexpr int kTailUnitsPerBlock = 2;
constexpr int kTailSplit3MinKT = 64;

__device__ __forceinline__ TailPlan plan_tail(int64_t total, int G, int KT, bool have_ws, int min_len)
{
    TailPlan p{total, 0, 1};
    const int64_t R = total / G;
    const int64_t rem = total - R * G;
    if (!have_ws || rem == 0)
        return p;
    int sk = 0;
    if (2 * rem <= G) {
        sk = (int)(G / rem);
        sk = sk > 8 ? 8 : sk;
    } else if (3 * rem <= (int64_t)kTailUnitsPerBlock * G && KT >= kTailSplit3MinKT) {
        sk = 3;
    }
    sk = sk > KT / min_len ? KT / min_len : sk;
    if (sk >= 2) {
        p.F = R * G;
        p.rem = (int)rem;
        p.sk = sk;
    }
    return p;
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

// Row sub-tiles of wave row wm that hold rows of the tile.
template <class G> __device__ __forceinline__ int valid_b(const TileLoc &t, int wm)
{
    const int64_t left = t.row_end - (t.row0 + (int64_t)wm * G::WTM);
    return left <= 0 ? 0 : (left >= G::WTM ? G::FB : (int)((left + 31) / 32));
}

// A block's work item: a whole tile, or one K range of a tail tile.
struct Work {
    TileLoc t;
    int kt_lo, kt_hi;
    int unit; // tail unit, or -1 for a whole tile
};

// Per-launch load geometry: per-lane byte offsets (row and swizzled chunk)
// into a W and an A row, bytes per row, and K steps per A row.
struct CopyGeo {
    uint32_t vbase, vbase_a, row_w, row_a;
    int KTa;
};

// One wave's staged registers: copy i of a K step (W rows for even i, A
// rows for odd i).
template <int BK, class G> struct Staged {
    static constexpr int DPW = 2 * (kL / (G::NW * (64 / (BK / 8))));
    u32x4 v[DPW];
};

// A K step's source: base addresses and byte sizes of the tile's W and A
// rows, and the step's byte offset into them.  Sizes of zero make every load
// out of range (zeros, no memory access).
struct Fill {
    uint64_t wbase, abase;
    uint32_t wbytes, abytes;
    uint32_t so_w, so_a;
};

template <int BK, bool WT = false, bool AT = false>
__device__ __forceinline__ Fill fill_k(uint64_t wb, uint64_t ab, uint32_t ws, uint32_t as, int k, int KTa,
                                       uint32_t row_w = 0, uint32_t row_a = 0)
{
    Fill f;
    f.wbase = wb;
    f.abase = ab;
    f.wbytes = ws;
    f.abytes = as;
    f.so_w = WT ? (uint32_t)k * (uint32_t)BK * row_w : (uint32_t)k * (BK * 2);
    f.so_a = AT ? (uint32_t)k * (uint32_t)BK * row_a : (uint32_t)(k % KTa) * (BK * 2);
    return f;
}

// max(a - b, 0) for wave-uniform a and b, on the scalar unit (the compiler
// would turn the saturating difference into a vector instruction).
__device__ __forceinline__ uint32_t sat_sub_scalar(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("s_sub_u32 %0, %1, %2\n\ts_cselect_b32 %0, 0, %0" : "=&s"(r) : "s"(a), "s"(b) : "scc");
    return r;
}

// 16 bytes of a raw buffer record of `bytes` bytes at `base`, at per-lane
// byte offset voff within rows that start row_off bytes into the record,
// plus a K offset k_off inside those rows.  The row part moves the record
// itself (base + row_off, bytes - row_off, empty once row_off reaches
// bytes), so which row is read is set by the per-lane offset alone; the K
// part (smaller than one row) goes in the scalar offset.  The range check of
// a raw buffer access compares its offset with the record size and returns
// zeros without a memory access when it is not smaller, so rows past a
// segment's end or past the weight matrix read as zeros and nothing past
// the operand is touched, whether or not the scalar offset takes part in
// the check.  All record arithmetic is scalar.
__device__ __forceinline__ u32x4 buf_load16(uint64_t base, uint32_t bytes, uint32_t voff, uint32_t row_off,
                                            uint32_t k_off)
{
    row_off = (uint32_t)__builtin_amdgcn_readfirstlane((int)row_off);
    bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
    base = (uint64_t)uni64((int64_t)base);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(uintptr_t)(base + row_off), (short)0, (int)sat_sub_scalar(bytes, row_off), kRsrcWord3);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, k_off, 0));
}

// Copy i of a K step (W rows for even i, A rows for odd i).  Instruction q
// of a wave covers rows (NW q + wave) * RPI .. + RPI - 1 (RPI = 8 rows of
// 128 bytes); a K-major operand's copy moves two K-rows per instruction and
// its K step is a row offset too.
template <int BK, class G> __device__ __forceinline__ u32x4 copy_load(const CopyGeo &cg, const Fill &f, int i)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NW = G::NW;
    const uint32_t q = (uint32_t)(i >> 1);
    if (i & 1) {
        if (G::AT)
            return buf_load16(f.abase, f.abytes, cg.vbase_a, q * (uint32_t)(2 * NW) * cg.row_a + f.so_a, 0u);
        return buf_load16(f.abase, f.abytes, cg.vbase_a, q * (uint32_t)(NW * RPI) * cg.row_a, f.so_a);
    }
    if (G::WT)
        return buf_load16(f.wbase, f.wbytes, cg.vbase, q * (uint32_t)(2 * NW) * cg.row_w + f.so_w, 0u);
    return buf_load16(f.wbase, f.wbytes, cg.vbase, q * (uint32_t)(NW * RPI) * cg.row_w, f.so_w);
}

// LDS byte offset (within a stage) of copy i's 16 bytes for this lane: the
// stage holds W's 256 rows, then A's.
template <int BK, class G> __device__ __forceinline__ uint32_t copy_ldsoff(int wave, int lane, int i)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR, NW = G::NW;
    const int q = i >> 1;
    if ((G::WT && !(i & 1)) || (G::AT && (i & 1))) {
        // K-row kr of the stage's [k][n] (or [k][m]) tile (kKmPitch-byte rows),
        // 16 bytes of its 32-byte chunk c
        const int kr = 2 * (NW * q + wave) + (lane >> 5);
        const int c = (lane & 31) >> 1;
        return (uint32_t)((i & 1) * G::W_BYTES + kr * kKmPitch + c * 32 + (lane & 1) * 16);
    }
    const uint32_t R = (uint32_t)((NW * q + wave) * RPI);
    return (uint32_t)((i & 1) * G::W_BYTES) + (uint32_t)(R * BK) * 2u + (uint32_t)lane * 16u;
}

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
    if (r < G::FA && G::WT) {
        // lanes 16 g + i of a half-wave take n = base + 16 g + i, k0 .. k0 + 7
        // (k0 = 16 ks + 8 khalf) from two transposed reads of 4 K-rows each
        const int g = r32 >> 4, i = r32 & 15;
        const int kr = ks * 16 + khalf * 8 + (i >> 2);
        const int c = (wn * G::WTN + r * 32) / 16 + g;
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const char *st = reinterpret_cast<const char *>(stage);
        const int off0 = kr * kKmPitch + c * 32 + (i & 3) * 8;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + off0));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + off0 + 4 * kKmPitch));
        fa[r] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else if (r < G::FA) {
        fa[r] = *reinterpret_cast<const bf16x8 *>(stage + (wn * G::WTN + r * 32 + r32) * BK + ch);
    } else if (r - G::FA < NBV && G::AT) {
        const int b = r - G::FA;
        const int g = r32 >> 4, i = r32 & 15;
        const int kr = ks * 16 + khalf * 8 + (i >> 2);
        const int c = (wm * G::WTM + b * 32) / 16 + g;
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const char *st = reinterpret_cast<const char *>(stage) + G::W_BYTES;
        const int off0 = kr * kKmPitch + c * 32 + (i & 3) * 8;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + off0));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(st + off0 + 4 * kKmPitch));
        fb[b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else if (r - G::FA < NBV) {
        const int b = r - G::FA;
        fb[b] = *reinterpret_cast<const bf16x8 *>(stage + G::W_BYTES / 2 + (wm * G::WTM + b * 32 + r32) * BK + ch);
    }
}

// Scheduling of a K step: each 16-wide sub-step is cut into kChunks chunks
// of MFMAs; the next sub-step's fragment reads go out in the first
// kReadChunks chunks, the staged registers are written to LDS over the first
// kWriteChunks chunks of the step, and the loads of the step after next are
// spread over the chunks before the barrier.  Reads over all eight chunks
// and writes over the three sub-steps before the barrier keep the LDS
// traffic even across the step (eight waves issue 48 KB of fragment reads
// per sub-step and 64 KB of writes per step); bunching the writes into the
// first sub-step with the reads in its first quarter was 1.5-2% slower.
constexpr int kChunks = 8, kReadChunks = 8, kWriteChunks = 24;

// One K step: MFMAs on stage `cur`; the staged registers (K step kt+1) go to
// stage `nxt`, and register loads of step kt+2 (`f`) refill them; then one
// barrier, after which `nxt` is complete and the last sub-step's MFMAs cover
// the reads of its first sub-step.
template <int BK, class G, int NBV>
__device__ __forceinline__ void k_step(const uint16_t *cur, uint16_t *nxt, const Fill &f, Staged<BK, G> &stg,
                                       const CopyGeo &cg, f32x16 (&acc)[G::FA][G::FB], bf16x8 (&fa)[2][G::FA],
                                       bf16x8 (&fb)[2][G::FB], int wave, int lane, int wn, int wm, int r32, int khalf,
                                       int sw)
{
    constexpr int FA = G::FA, FB = G::FB;
    constexpr int KS = BK / 16;
    constexpr int DPW = Staged<BK, G>::DPW;
    constexpr int CPS = kChunks < FA * FB ? kChunks : FA * FB;
    constexpr int MPC = FA * FB / CPS;
    constexpr int RDS = FA + FB;
    constexpr int RCH = kReadChunks < CPS ? kReadChunks : CPS;
    constexpr int RPC = (RDS + RCH - 1) / RCH;
    constexpr int NPRE = (KS - 1) * CPS;
    constexpr int WSP = kWriteChunks < NPRE ? kWriteChunks : NPRE;
    static_assert(KS >= 2 && (FA * FB) % CPS == 0, "chunking");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        // Sub-step ks+1 comes from this stage, except after the last one:
        // then sub-step 0 of the next stage (complete: the barrier is behind).
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
                            {
                                if ((G::WT && read_slot<G>(c * RPC + q) < FA) ||
                                    (G::AT && read_slot<G>(c * RPC + q) >= FA))
                                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                                else
                                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                            }
                    }
                }
            }
            if (ks + 1 < KS) {
                const int g = ks * CPS + c;
                __builtin_amdgcn_sched_barrier(0);
                // staged register j -> nxt, then its reload (step kt+2)
#pragma unroll
                for (int j = 0; j < DPW; ++j)
                    if ((j * WSP) / DPW == g)
                        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(nxt) + copy_ldsoff<BK, G>(wave, lane, j)) =
                            stg.v[j];
#pragma unroll
                for (int j = 0; j < DPW; ++j)
                    if ((j * NPRE) / DPW == g)
                        stg.v[j] = copy_load<BK, G>(cg, f, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (ks == KS - 2) {
            // nxt complete; the register loads of step kt+2 stay in flight
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// What a block needs to find its work items: item i < nw is whole tile
// first + i * per (an XCD-contiguous share of [0, F)); item nw, if any, is
// its tail unit (one K range of a tail tile).
struct WorkCtx {
    const int *tb;
    const int32_t *seg;
    const uint16_t *A, *W;
    int64_t max_rows, first, F;
    int S, N, K, Ka, NT, KT, per, nw, unit, ustride, sk, n_work;
    bool wt; // weight operand K-major
};

// Work item i, all fields wave-uniform.
__device__ __forceinline__ Work get_work(const WorkCtx &x, int i)
{
    Work w;
    if (i < x.nw) {
        w.t = locate(x.tb, x.seg, x.S, x.max_rows, x.NT, x.first + (int64_t)i * x.per);
        w.kt_lo = 0;
        w.kt_hi = x.KT;
        w.unit = -1;
    } else {
        const int u = x.unit + (i - x.nw) * x.ustride;
        const int c = u % x.sk;
        w.t = locate(x.tb, x.seg, x.S, x.max_rows, x.NT, x.F + u / x.sk);
        w.kt_lo = (int)((int64_t)x.KT * c / x.sk);
        w.kt_hi = (int)((int64_t)x.KT * (c + 1) / x.sk);
        w.unit = u;
    }
    w.t.s = uni(w.t.s);
    w.t.row0 = uni64(w.t.row0);
    w.t.row_end = uni64(w.t.row_end);
    w.t.n0 = uni(w.t.n0);
    w.kt_lo = uni(w.kt_lo);
    w.kt_hi = uni(w.kt_hi);
    return w;
}

// Load source (W and A rows) of work item w.
struct Src {
    uint64_t wbase, abase;
    uint32_t wbytes, abytes;
};

__device__ __forceinline__ Src src_of(const WorkCtx &x, const CopyGeo &cg, const Work &w)
{
    Src s;
    s.abase = (uint64_t)(uintptr_t)(x.A + w.t.row0 * x.Ka);
    if (x.wt) {
        // K-major: from (k = 0, n = n0) to the end of the segment's [K][N] matrix
        s.wbase = (uint64_t)(uintptr_t)(x.W + (int64_t)w.t.s * x.N * x.K + w.t.n0);
        s.wbytes = (uint32_t)((int64_t)x.K * x.N - w.t.n0) * 2u;
    } else {
        s.wbase = (uint64_t)(uintptr_t)(x.W + (int64_t)w.t.s * x.N * x.K + (int64_t)w.t.n0 * x.K);
        s.wbytes = (uint32_t)min(kL, x.N - w.t.n0) * cg.row_w;
    }
    s.abytes = (uint32_t)(w.t.row_end - w.t.row0) * cg.row_a;
    return s;
}

// One tile (or one K range of a tail tile): work item i.  On entry LDS
// stage b holds its first K step (complete, behind a barrier) and the staged
// registers hold its second; on exit the same holds for item i+1 (nothing
// is loaded if there is none).  The loads switch to item i+1's rows for the
// last two K steps; its source is looked up only then, so that it does not
// occupy registers during the loop.
template <int BK, class G, int NBV, bool GELU, bool BIAS, bool F32OUT, bool PART, class X>
__device__ __forceinline__ int tile(uint16_t *smem, int b, const CopyGeo &cg, const X &x, int i, Src src,
                                    int kt_lo, int kt_hi, Staged<BK, G> &stg, void *C, const uint16_t *bseg,
                                    float *part, int64_t row0, int64_t row_end, int n0, int N)
{
    constexpr int FA = G::FA, FB = G::FB, STAGE = G::STAGE_ELEMS;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid)); // lane values are rederived per tile, not kept (spilled) across tiles
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WGN_, wm = wave / G::WGN_;
    const int r32 = lane & 31, khalf = lane >> 5;
    const int sw = swz(r32);

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
    int koff = 0; // K step of `src` loaded at step kt: kt + 2 + koff
    int kbase = G::AT ? kt_lo : 0; // K step at src's base address
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        if (kt + 2 == kt_hi) {
            // from here on, load the next item's first steps
            if (i + 1 < x.n_work) {
                const Work wn = get_work(x, i + 1);
                src = src_of(x, cg, wn);
                koff = wn.kt_lo - kt_hi;
                kbase = G::AT ? wn.kt_lo : 0;
            } else {
                src.wbytes = 0;
                src.abytes = 0;
                koff = -kt_hi;
            }
        }
        const Fill f = fill_k<BK, G::WT, G::AT>(src.wbase, src.abase, src.wbytes, src.abytes, kt + 2 + koff - kbase, cg.KTa, cg.row_w,
                                                    cg.row_a);
        const int bn = b ^ 1;
        k_step<BK, G, NBV>(smem + b * STAGE, smem + bn * STAGE, f, stg, cg, acc, fa, fb, wave, lane, wn, wm, r32,
                           khalf, sw);
        b = bn;
    }
    if (PART) {
        // only the row sub-tiles that hold rows (the reduce reads no others)
        float *dst = part + (size_t)wave * (FA * FB * 16 * 64) + lane;
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int q = 0; q < NBV; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dst[((a * FB + q) * 16 + v) * 64] = acc[a][q][v];
    } else {
        // the stage other than b (the next item's first K step) is free after
        // the loop's last barrier
        char *free_stage = reinterpret_cast<char *>(smem + (b ^ 1) * STAGE);
        if constexpr (F32OUT) {
            static_assert(!GELU, "fp32 outputs are pre-activation");
            store_tile_f32_lds<G, BIAS>(acc, (float *)C, bseg, free_stage, row0, row_end, n0, N, wave, lane, wn, wm,
                                        r32, khalf);
        } else {
            store_tile_bf16_lds<G, GELU, BIAS>(acc, (uint16_t *)C, bseg, free_stage, row0, row_end, n0, N, wave,
                                               lane, wn, wm, r32, khalf);
        }
        lds_barrier();
    }
    return b;
}

template <int BK, class G, bool GELU, bool BIAS, bool F32OUT, bool PART, class X>
__device__ __forceinline__ int tile_any(int nbv, uint16_t *smem, int b, const CopyGeo &cg, const X &x, int i,
                                        Src src, int kt_lo, int kt_hi, Staged<BK, G> &stg, void *C,
                                        const uint16_t *bseg, float *part, int64_t row0, int64_t row_end, int n0,
                                        int N)
{
#define MOE_TILE(V)                                                                                                 \
    tile<BK, G, V, GELU, BIAS, F32OUT, PART, X>(smem, b, cg, x, i, src, kt_lo, kt_hi, stg, C, bseg, part, row0,    \
                                             row_end, n0, N)
    if (G::FB == 4) {
        switch (nbv) {
        case 4: return MOE_TILE(G::FB >= 4 ? 4 : G::FB);
        case 3: return MOE_TILE(G::FB >= 3 ? 3 : G::FB);
        default: break;
        }
    }
    switch (nbv) {
    case 2: return MOE_TILE(G::FB >= 2 ? 2 : G::FB);
    case 1: return MOE_TILE(1);
    default: return MOE_TILE(0);
    }
#undef MOE_TILE
}

// Persistent grouped GEMM over 256x256 tiles.  The tile list is derived on
// the device from the segment offsets; whole tiles are dealt to the XCDs as
// contiguous ranges, and a short last round is split along K (tail units).
// A's rows have Ka elements: its K offset wraps every Ka (Ka = K for a plain
// GEMM).  Every K range is at least two steps long.
template <int BK, class G, bool GELU, bool BIAS, bool F32OUT>
__global__ __launch_bounds__(64 * G::NW, 1) void grouped_gemm_256(const uint16_t *__restrict__ A,
                                                                  const int32_t *__restrict__ seg, int S,
                                                                  int64_t max_rows, const uint16_t *__restrict__ W,
                                                                  const uint16_t *__restrict__ bias,
                                                                  void *__restrict__ C, int N, int K, int Ka,
                                                                  float *__restrict__ part_ws)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    constexpr int DPW = Staged<BK, G>::DPW;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * G::STAGE_ELEMS];
    __shared__ int tb[kMaxSeg + 1];
    build_tile_prefix<kL>(seg, S, max_rows, tb);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::WGN_;
    const int NT = (N + kL - 1) / kL;
    const int KT = K / BK;
    const int64_t total = (int64_t)tb[S] * NT;
    const TailPlan plan = plan_tail(total, (int)gridDim.x, KT, part_ws != nullptr, 2);

    WorkCtx x;
    x.tb = tb;
    x.seg = seg;
    x.A = A;
    x.W = W;
    x.max_rows = max_rows;
    x.S = S;
    x.N = N;
    x.K = K;
    x.Ka = Ka;
    x.wt = G::WT;
    x.NT = NT;
    x.KT = KT;
    x.F = plan.F;
    x.sk = plan.sk;
    const int xcd = blockIdx.x % kXcds;
    x.per = gridDim.x / kXcds;
    const int64_t rlo = plan.F * xcd / kXcds, rhi = plan.F * (xcd + 1) / kXcds;
    x.first = rlo + blockIdx.x / kXcds;
    x.nw = x.first < rhi ? (int)((rhi - x.first + x.per - 1) / x.per) : 0;
    x.unit = blockIdx.x;
    x.ustride = gridDim.x;
    const int units = plan.rem * plan.sk;
    const int ntail = x.unit < units ? (units - x.unit + x.ustride - 1) / x.ustride : 0;
    x.n_work = x.nw + ntail;
    if (x.n_work == 0)
        return;

    CopyGeo cg;
    {
        const int lrow = lane / CPR;
        const int prow = wave * RPI + lrow;
        const int lchunk = (lane % CPR) ^ swz(prow);
        cg.row_w = (uint32_t)(G::WT ? N : K) * 2u;
        cg.row_a = (uint32_t)Ka * 2u;
        // K-major weight: a copy instruction moves two 512-byte K-rows
        cg.vbase = G::WT ? (uint32_t)(2 * wave + (lane >> 5)) * cg.row_w + (uint32_t)(lane & 31) * 16u
                         : (uint32_t)prow * cg.row_w + (uint32_t)lchunk * 16u;
        cg.vbase_a = (uint32_t)prow * cg.row_a + (uint32_t)lchunk * 16u;
        cg.KTa = Ka / BK;
    }

    Staged<BK, G> stg;
    // Prologue: K step kt_lo of item 0 into LDS stage 0, kt_lo+1 into the
    // staged registers.
    {
        const Work w = get_work(x, 0);
        const Src o = src_of(x, cg, w);
        const int k0 = G::AT ? 0 : w.kt_lo; // K-major sources start at the item's first step
        const Fill f0 = fill_k<BK, G::WT, G::AT>(o.wbase, o.abase, o.wbytes, o.abytes, k0, cg.KTa, cg.row_w, cg.row_a);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            stg.v[i] = copy_load<BK, G>(cg, f0, i);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(smem) + copy_ldsoff<BK, G>(wave, lane, i)) = stg.v[i];
        const Fill f1 = fill_k<BK, G::WT, G::AT>(o.wbase, o.abase, o.wbytes, o.abytes, k0 + 1, cg.KTa, cg.row_w, cg.row_a);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            stg.v[i] = copy_load<BK, G>(cg, f1, i);
        lds_barrier();
    }
    int b = 0;
    for (int i = 0; i < x.n_work; ++i) {
        const Work w = get_work(x, i);
        const Src o = src_of(x, cg, w);
        const int nbv = valid_b<G>(w.t, wm);
        if (w.unit < 0)
            b = tile_any<BK, G, GELU, BIAS, F32OUT, false>(nbv, smem, b, cg, x, i, o, w.kt_lo, w.kt_hi, stg, C,
                                                           bias ? bias + (int64_t)w.t.s * N : nullptr, nullptr,
                                                           w.t.row0, w.t.row_end, w.t.n0, N);
        else
            b = tile_any<BK, G, GELU, BIAS, F32OUT, true>(nbv, smem, b, cg, x, i, o, w.kt_lo, w.kt_hi, stg, C,
                                                          nullptr, part_ws + (size_t)w.unit * (kL * kL), w.t.row0,
                                                          w.t.row_end, w.t.n0, N);
    }
}

// ---------------------------------------------------------------------------
// K-segmented grouped GEMM (weight gradients): for every segment s,
//   out_s[m, n] = sum_{k in segment s} A[m, k] W[n, k]      (fp32, [M, N])
// with A [M, Kp] and W [N, Kp] holding the segments' columns at 64-aligned
// offsets, zero-padded: segment s (rows_s rows of the forward) occupies
// max(2, ceil(rows_s / 64)) K steps of 64 columns, none if it is empty; kcol
// [S+1] holds the first step of each segment (kseg_layout).  Empty segments
// get no tiles (their outputs are zeroed separately).  Same tile machinery
// as grouped_gemm_256; no split-K tail.  The K-major form (Grid with WT and
// AT, bf16) reads the same sums from the row-major rows A [rows, M] and
// W [rows, N] themselves: each K step copies 64 rows of a segment into
// [k][m] and [k][n] LDS tiles, the fragments come from transposing reads,
// and rows past the segment's end read as zeros (range-checked loads), so
// the products meet the accumulators in the same order as with the
// zero-padded transposed copies.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kseg_steps(int64_t rows) { return rows <= 0 ? 0 : (int)max<int64_t>(2, (rows + 63) / 64); }

// kcol[s] = first K step of segment s, kcol[S] = total steps.  One wave.
__global__ __launch_bounds__(64) void kseg_layout(const int32_t *__restrict__ seg, int S, int64_t max_rows,
                                                  int32_t *__restrict__ kcol)
{
    const int lane = threadIdx.x;
    int carry = 0;
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int s = s0 + lane;
        int v = 0;
        if (s < S) {
            int64_t lo, hi;
            seg_bounds(seg, s, max_rows, lo, hi);
            v = kseg_steps(hi - lo);
        }
        int inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(inc, o, 64);
            if (lane >= o)
                inc += u;
        }
        if (s < S)
            kcol[s] = carry + inc - v;
        carry += __shfl(inc, 63, 64);
    }
    if (lane == 0)
        kcol[S] = carry;
}

// LDS copy of kcol and ne[s] = non-empty segments before s (ne[S] = total).
__device__ void load_kseg_prefix(const int32_t *kcol, int S, int *kb, int *ne)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave == 0) {
        int cn = 0;
        for (int s0 = 0; s0 < S; s0 += 64) {
            const int s = s0 + lane;
            int vn = 0;
            if (s < S) {
                const int a = kcol[s], b = kcol[s + 1];
                kb[s] = a;
                vn = b > a ? 1 : 0;
            }
            int in = vn;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int un = __shfl_up(in, o, 64);
                if (lane >= o)
                    in += un;
            }
            if (s < S)
                ne[s] = cn + in - vn;
            cn += __shfl(in, 63, 64);
        }
        if (lane == 0) {
            kb[S] = kcol[S];
            ne[S] = cn;
        }
    }
    __syncthreads();
}

constexpr int kKsegPanel = 4;

struct KsegCtx {
    const int *kb, *ne;
    const uint16_t *A, *W;
    const int32_t *seg; // K-major operands: dispatched rows of the segments (NULL: one of `rows`)
    int64_t rows;
    bool kmajor;        // A [rows, M] and W [rows, N] row-major instead of A [M, Kp], W [N, Kp]
    int64_t first;
    int S, M, N, Kp, MT, NT, per, nw, n_work;
    bool n_inner; // the feature tiles (W) are the smaller operand's (M > N)
};

// Work item i of the block: tile L = first + i * per of the list (non-empty
// segments ascending, then panels of the smaller operand's tiles).
__device__ __forceinline__ Work get_work(const KsegCtx &x, int i)
{
    const int64_t L = x.first + (int64_t)i * x.per;
    int per_seg = x.MT * x.NT;
    asm volatile("" : "+s"(per_seg)); // keeps the divisions' reciprocals out of the loop (no spill)
    const int q = (int)(L / per_seg); // index among the non-empty segments
    // The last segment with ne[s] <= q is the q-th non-empty one: an empty
    // segment is followed by one with the same ne, and the segments after
    // the q-th non-empty one have ne > q.
    int lo = 0, hi = x.S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (x.ne[mid] <= q)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int local = (int)(L - (int64_t)q * per_seg);
    // Panels of kKsegPanel tiles of the smaller operand: within a panel the
    // larger operand's tiles are walked, the panel's tiles fastest, so the
    // panel (about 2 MB) stays in the XCD's L2 while the 32 CUs sweep the
    // larger operand, which is read once per panel.
    int SI = x.n_inner ? x.NT : x.MT, LO = x.n_inner ? x.MT : x.NT;
    asm volatile("" : "+s"(SI), "+s"(LO));
    const int panel = local / (kKsegPanel * LO);
    const int rem = local - panel * (kKsegPanel * LO);
    const int pw = SI - panel * kKsegPanel < kKsegPanel ? SI - panel * kKsegPanel : kKsegPanel;
    const int big = rem / pw, small = panel * kKsegPanel + rem % pw;
    const int row0 = (x.n_inner ? big : small) * kL;
    const int n0 = (x.n_inner ? small : big) * kL;
    const int row_end = row0 + kL < x.M ? row0 + kL : x.M;
    Work w;
    w.t.s = uni(lo);
    w.t.n0 = uni(n0);
    w.t.row0 = uni(row0);
    w.t.row_end = uni(row_end);
    w.kt_lo = uni(x.kb[lo]);
    w.kt_hi = uni(x.kb[lo + 1]);
    w.unit = -1;
    return w;
}

// All fields wave-uniform (the buffer descriptors must be scalar).
__device__ __forceinline__ Src src_of(const KsegCtx &x, const CopyGeo &cg, const Work &w)
{
    Src s;
    const int n0 = (int)w.t.n0, row0 = (int)w.t.row0, rows = (int)(w.t.row_end - w.t.row0);
    const int nw = x.N - n0 < kL ? x.N - n0 : kL;
    if (x.kmajor) {
        // K-major: both operands start at the segment's first dispatched row;
        // rows past its end read as zeros
        int64_t lo, hi;
        seg_bounds(x.seg, w.t.s, x.rows, lo, hi);
        const int64_t n = hi - lo;
        s.wbase = (uint64_t)uni64((int64_t)(uintptr_t)(x.W + lo * x.N + n0));
        s.abase = (uint64_t)uni64((int64_t)(uintptr_t)(x.A + lo * x.M + row0));
        s.wbytes = (uint32_t)uni((int)((n * x.N - n0) * 2));
        s.abytes = (uint32_t)uni((int)((n * x.M - row0) * 2));
        return s;
    }
    s.wbase = (uint64_t)uni64((int64_t)(uintptr_t)(x.W + (int64_t)n0 * x.Kp));
    s.abase = (uint64_t)uni64((int64_t)(uintptr_t)(x.A + (int64_t)row0 * x.Kp));
    s.wbytes = (uint32_t)uni(nw * (int)cg.row_w);
    s.abytes = (uint32_t)uni(rows * (int)cg.row_a);
    return s;
}

template <int BK, class G>
__global__ __launch_bounds__(64 * G::NW, 1) void grouped_gemm_kseg(const uint16_t *__restrict__ A,
                                                                   const uint16_t *__restrict__ W,
                                                                   const int32_t *__restrict__ kcol, int S, int M,
                                                                   int N, int Kp, float *__restrict__ C,
                                                                   const int32_t *__restrict__ seg, int64_t rows)
{
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    constexpr int DPW = Staged<BK, G>::DPW;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * G::STAGE_ELEMS];
    __shared__ int kb[kMaxSeg + 1], ne[kMaxSeg + 1];
    load_kseg_prefix(kcol, S, kb, ne);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::WGN_;
    KsegCtx x;
    x.kb = kb;
    x.ne = ne;
    x.A = A;
    x.W = W;
    x.S = S;
    x.M = M;
    x.N = N;
    x.Kp = Kp;
    x.seg = seg;
    x.rows = rows;
    x.kmajor = G::AT;
    x.MT = (M + kL - 1) / kL;
    x.NT = (N + kL - 1) / kL;
    x.n_inner = M > N;
    const int64_t total = (int64_t)ne[S] * x.MT * x.NT;
    const int xcd = blockIdx.x % kXcds;
    x.per = gridDim.x / kXcds;
    const int64_t rlo = total * xcd / kXcds, rhi = total * (xcd + 1) / kXcds;
    x.first = rlo + blockIdx.x / kXcds;
    x.nw = x.first < rhi ? (int)((rhi - x.first + x.per - 1) / x.per) : 0;
    x.n_work = x.nw;
    if (x.n_work == 0)
        return;

    CopyGeo cg;
    {
        const int lrow = lane / CPR;
        const int prow = wave * RPI + lrow;
        const int lchunk = (lane % CPR) ^ swz(prow);
        if (G::AT) {
            // K-major: each wave instruction copies two 512-byte K-rows
            cg.row_w = (uint32_t)N * 2u;
            cg.row_a = (uint32_t)M * 2u;
            const uint32_t kr = (uint32_t)(2 * wave + (lane >> 5)), col = (uint32_t)(lane & 31) * 16u;
            cg.vbase = kr * cg.row_w + col;
            cg.vbase_a = kr * cg.row_a + col;
        } else {
            cg.row_w = (uint32_t)Kp * 2u;
            cg.row_a = (uint32_t)Kp * 2u;
            cg.vbase = (uint32_t)prow * cg.row_w + (uint32_t)lchunk * 16u;
            cg.vbase_a = cg.vbase;
        }
        cg.KTa = Kp / BK;
    }
    Staged<BK, G> stg;
    {
        const Work w = get_work(x, 0);
        const Src o = src_of(x, cg, w);
        const int k0 = G::AT ? 0 : w.kt_lo; // K-major sources start at the item's first step
        const Fill f0 = fill_k<BK, G::WT, G::AT>(o.wbase, o.abase, o.wbytes, o.abytes, k0, cg.KTa, cg.row_w, cg.row_a);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            stg.v[i] = copy_load<BK, G>(cg, f0, i);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(smem) + copy_ldsoff<BK, G>(wave, lane, i)) = stg.v[i];
        const Fill f1 = fill_k<BK, G::WT, G::AT>(o.wbase, o.abase, o.wbytes, o.abytes, k0 + 1, cg.KTa, cg.row_w, cg.row_a);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            stg.v[i] = copy_load<BK, G>(cg, f1, i);
        lds_barrier();
    }
    int b = 0;
    for (int i = 0; i < x.n_work; ++i) {
        const Work w = get_work(x, i);
        const Src o = src_of(x, cg, w);
        b = tile_any<BK, G, false, false, true, false>(valid_b<G>(w.t, wm), smem, b, cg, x, i, o, w.kt_lo, w.kt_hi,
                                                       stg, C + (int64_t)w.t.s * M * N, nullptr, nullptr, w.t.row0,
                                                       w.t.row_end, w.t.n0, N);
    }
}

// fp32 K-segmented GEMM: 64 x 64 output tiles of segment blockIdx.z, K
// slices of 16 through LDS; an empty segment's tile is written as zeros.
__global__ __launch_bounds__(256) void grouped_gemm_kseg_f32(const float *__restrict__ A,
                                                             const float *__restrict__ W,
                                                             const int32_t *__restrict__ kcol, int M, int N,
                                                             int64_t Kp, float *__restrict__ C)
{
    constexpr int TM = 64, TN = 64, TK = 16;
    __shared__ float sa[TK][TM + 4];
    __shared__ float sw[TK][TN + 4];
    const int s = blockIdx.z;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
    const int64_t k_lo = (int64_t)kcol[s] * 64, k_hi = (int64_t)kcol[s + 1] * 64;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    for (int64_t k0 = k_lo; k0 < k_hi; k0 += TK) {
        for (int q = tid; q < TM * TK; q += 256) {
            const int r = q / TK, kk = q % TK;
            const int m = min(m0 + r, M - 1), n = min(n0 + r, N - 1);
            sa[kk][r] = A[(int64_t)m * Kp + k0 + kk];
            sw[kk][r] = W[(int64_t)n * Kp + k0 + kk];
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
    float *out = C + (int64_t)s * M * N;
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M)
            continue;
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx * 4 + q;
            if (n < N)
                out[(int64_t)m * N + n] = acc[i][q];
        }
    }
}

// Zeroes out_s [MN] (MN % 4 == 0) of every empty segment (the bf16 path gives
// them no tiles), 16 bytes per store.
__global__ __launch_bounds__(256) void kseg_zero_empty(const int32_t *__restrict__ kcol, int64_t MN,
                                                       float *__restrict__ C)
{
    const int s = blockIdx.y;
    if (kcol[s + 1] != kcol[s])
        return;
    f32x4 *out = reinterpret_cast<f32x4 *>(C + (int64_t)s * MN);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN / 4; i += (int64_t)gridDim.x * 256)
        out[i] = z;
}

// Sums the K-range partials of each tail tile in range order and applies the
// bias, activation and bf16 store; a no-op when the GEMM had no split tail.
// Block = (tail tile, GEMM wave w), looping over the tail tiles with the
// grid's stride; its FA waves take the feature sub-tiles a and loop over the
// row sub-tiles b that hold rows (the only ones stored).  Each lane loads its
// 16 accumulators of every K range up front (independent loads), then sums in
// range order.
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
    const int wave = blockIdx.x % G::NW;
    const int lane = threadIdx.x & 63, a = threadIdx.x >> 6;
    const int wn = wave % G::WGN_, wm = wave / G::WGN_;
    const int r32 = lane & 31, khalf = lane >> 5;
    for (int tile = blockIdx.x / G::NW; tile < plan.rem; tile += gridDim.x / G::NW) {
        const TileLoc t = locate(tb, seg, S, max_rows, NT, plan.F + tile);
        const uint16_t *bseg = bias ? bias + (int64_t)t.s * N : nullptr;
        const TileOut rt = tile_out<F32OUT>(C, t.row0, t.row_end, N);
        const int nbv = valid_b<G>(t, wm);
        for (int b = 0; b < nbv; ++b) {
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
                store4<GELU, BIAS, F32OUT>(rt, bseg, row, row_ok, n, N, v[4 * g], v[4 * g + 1], v[4 * g + 2],
                                           v[4 * g + 3]);
            }
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

template <bool GELU, bool BIAS, bool F32OUT, class G = LargeGrid>
moe_status_t run_large(const void *a, const int32_t *seg, int S, int64_t max_rows, int N, int K, int Ka,
                       const void *w, const void *bias, void *out, float *part_ws, hipStream_t stream)
{
    // the epilogue stores 16 bytes per lane (4 fp32 or 8 bf16 features); rows
    // of the output must not split such a group
    if (N % (F32OUT ? 4 : 8) != 0 || K % kLargeBK != 0 || K / kLargeBK < 2 || Ka % kLargeBK != 0)
        return fail(MOE_ERR_UNSUPPORTED,
                    "grouped_gemm_256: needs N %% %d == 0, K %% 64 == 0, K >= 128 (N=%d K=%d)", F32OUT ? 4 : 8, N, K);
    const int grid = large_grid(max_rows, S, N, part_ws != nullptr);
    grouped_gemm_256<kLargeBK, G, GELU, BIAS, F32OUT><<<(unsigned)grid, 64 * G::NW, 0, stream>>>(
        (const uint16_t *)a, seg, S, max_rows, (const uint16_t *)w, (const uint16_t *)bias, out, N, K, Ka, part_ws);
    if (moe_status_t st = check_launch("grouped_gemm_256"))
        return st;
    if (!part_ws)
        return MOE_OK;
    grouped_gemm_reduce<G, GELU, BIAS, F32OUT><<<(unsigned)(grid / 2 * G::NW), 64 * G::FA, 0, stream>>>(
        seg, S, max_rows, (const uint16_t *)bias, out, N, K, kLargeBK, 2, grid, part_ws);
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

size_t gemm_ws_bytes()
{
    int64_t grid = (int64_t)device_cus();
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    return (size_t)grid * kTailUnitsPerBlock * kL * kL * sizeof(float);
}

moe_status_t launch_grouped_gemm(const void *a, const int32_t *seg_offsets, int num_segments, int64_t max_rows,
                                 int N, int K, moe_dtype_t dt, const void *w, const void *bias, int activation,
                                 void *out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (max_rows == 0)
        return MOE_OK;
    const int S = seg_offsets ? num_segments : 1;
    if (dt == MOE_BF16) {
        if (K % kLargeBK == 0 && K / kLargeBK >= 2) {
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

int64_t kseg_cols_bound(int64_t max_rows, int S)
{
    // a non-empty segment of r rows takes max(2, ceil(r / 64)) <= ceil(r / 64) + 1
    // steps, and sum_s ceil(r_s / 64) * 64 <= max_rows + 63 S
    return (max_rows + 63) / 64 * 64 + 128 * (int64_t)S;
}

moe_status_t launch_kseg_layout(const int32_t *seg, int S, int64_t max_rows, int32_t *kcol, hipStream_t stream)
{
    kseg_layout<<<1, 64, 0, stream>>>(seg, S, max_rows, kcol);
    return check_launch("kseg_layout");
}

moe_status_t launch_kseg_gemm(const void *A, const void *W, const int32_t *kcol, int S, int M, int N, int64_t Kp,
                              moe_dtype_t dt, float *C, hipStream_t stream)
{
    if (S < 1 || M < 1 || N < 1)
        return MOE_OK;
    if (dt == MOE_F32) {
        const dim3 g((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64), (unsigned)S);
        grouped_gemm_kseg_f32<<<g, 256, 0, stream>>>((const float *)A, (const float *)W, kcol, M, N, Kp, C);
        return check_launch("grouped_gemm_kseg_f32");
    }
    typedef LargeGrid G;
    if (N % 4 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm_kseg: needs N %% 4 == 0 (N=%d)", N);
    int64_t grid = (int64_t)device_cus();
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    grouped_gemm_kseg<kLargeBK, G><<<(unsigned)grid, 64 * G::NW, 0, stream>>>(
        (const uint16_t *)A, (const uint16_t *)W, kcol, S, M, N, (int)Kp, C, nullptr, 0);
    if (moe_status_t st = check_launch("grouped_gemm_kseg"))
        return st;
    const int64_t MN = (int64_t)M * N;
    const int64_t bx0 = (MN / 4 + 255) / 256, bx = bx0 < 256 ? bx0 : 256;
    kseg_zero_empty<<<dim3((unsigned)bx, (unsigned)S), 256, 0, stream>>>(kcol, MN, C);
    return check_launch("kseg_zero_empty");
}

bool kseg_kmajor_ok(int64_t seg_max, int M, int N)
{
    const int64_t w = M > N ? M : N;
    return M % 8 == 0 && N % 8 == 0 && seg_max * w * 2 < ((int64_t)1 << 31);
}

moe_status_t launch_kseg_gemm_kmajor(const void *A_rows, const void *W_rows, const int32_t *seg, int64_t rows,
                                     int64_t seg_max, const int32_t *kcol, int S, int M, int N, float *C,
                                     hipStream_t stream)
{
    if (S < 1 || M < 1 || N < 1)
        return MOE_OK;
    // each segment's operands are addressed with 32-bit byte offsets
    if (!kseg_kmajor_ok(seg_max < rows ? seg_max : rows, M, N))
        return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm_kseg (K-major): needs M, N multiples of 8 and rows per "
                                         "segment x max(M, N) below 2^30 (rows=%lld M=%d N=%d)",
                    (long long)(seg_max < rows ? seg_max : rows), M, N);
    typedef LargeGridKK G;
    int64_t grid = (int64_t)device_cus();
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    grouped_gemm_kseg<kLargeBK, G><<<(unsigned)grid, 64 * G::NW, 0, stream>>>(
        (const uint16_t *)A_rows, (const uint16_t *)W_rows, kcol, S, M, N, 0, C, seg, rows);
    if (moe_status_t st = check_launch("grouped_gemm_kseg"))
        return st;
    const int64_t MN = (int64_t)M * N;
    const int64_t bx0 = (MN / 4 + 255) / 256, bx = bx0 < 256 ? bx0 : 256;
    kseg_zero_empty<<<dim3((unsigned)bx, (unsigned)S), 256, 0, stream>>>(kcol, MN, C);
    return check_launch("kseg_zero_empty");
}

moe_status_t launch_grouped_gemm_kmajor_f32out(const void *a, const int32_t *seg_offsets, int num_segments,
                                               int64_t max_rows, int N, int K, const void *w_kn, float *out,
                                               void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (max_rows == 0)
        return MOE_OK;
    if ((int64_t)K * N > ((int64_t)1 << 31) - 1)
        return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm (K-major weight): K x N = %lld above 2^31",
                    (long long)K * N);
    const int S = seg_offsets ? num_segments : 1;
    float *part = (ws && ws_bytes >= gemm_ws_bytes()) ? (float *)ws : nullptr;
    return run_large<false, false, true, LargeGridWT>(a, seg_offsets, S, max_rows, N, K, K, w_kn, nullptr, out,
                                                      part, stream);
}

moe_status_t launch_grouped_gemm_f32out(const void *a, const int32_t *seg_offsets, int num_segments,
                                        int64_t max_rows, int N, int K, moe_dtype_t dt, const void *w,
                                        const void *bias, float *out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (max_rows == 0)
        return MOE_OK;
    const int S = seg_offsets ? num_segments : 1;
    if (dt == MOE_BF16) {
        float *part = (ws && ws_bytes >= gemm_ws_bytes()) ? (float *)ws : nullptr;
        return bias ? run_large<false, true, true>(a, seg_offsets, S, max_rows, N, K, K, w, bias, out, part, stream)
                    : run_large<false, false, true>(a, seg_offsets, S, max_rows, N, K, K, w, bias, out, part, stream);
    }
    const dim3 g((unsigned)((N + 63) / 64), (unsigned)((max_rows + 63) / 64 + S));
    grouped_gemm_f32<false><<<g, 256, 0, stream>>>((const float *)a, seg_offsets, S, max_rows, (const float *)w,
                                                    (const float *)bias, out, N, K);
    return check_launch("grouped_gemm_f32");
}

} // namespace moe
