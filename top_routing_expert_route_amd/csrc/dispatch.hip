// Dispatch of the MoE layer on one GPU: capacity cap, token dropping and the
// permutation of the kept selections into expert-contiguous rows.
//
// Pages: "Expert Parallelism (MoE)", section "Top-K Routing and Capacity
// Factor" (capacity = tokens_per_batch / N_experts * capacity_factor; the
// selections over capacity are dropped) and "Expert Parallelism (EP)",
// section "Key math / How it works" (dispatch routes each token to the owner
// of its expert - here a permutation into this GPU's expert segments).
//
// The selections t*k+j are cut into chunks of `chunk` consecutive items, one
// chunk per wave, so that the rank of a selection among the earlier
// selections of its expert is
//     (selections of that expert in earlier chunks) + (earlier in its chunk).
//  dispatch_count    per-chunk histogram of local experts (LDS atomics: exact
//                    integer counts, order-free).
//  dispatch_scan     one block: per-expert exclusive scan over chunks (two
//                    coalesced passes over the counts, segment sums scanned
//                    in LDS), capacity, kept counts,
//                    the exclusive scan of kept counts (segment offsets) and
//                    the number of dropped selections.
//  dispatch_rank     each wave walks its chunk 64 selections at a time; lanes
//                    holding the same expert find each other with 64-lane
//                    ballots over the bits of the expert id, so the rank is
//                    stable (token order) without atomics.  Writes slot_row
//                    and row_src.
//  dispatch_fused    the whole dispatch in one launch when (blocks x
//                    selections) is small: every block counts all selections
//                    itself (see the kernel).
//  dispatch_plan_small  count + scan + rank in one block of 16 waves when
//                    T*k <= 32768 and E_loc <= 256 (counts and bases in LDS),
//                    for sizes past the single-launch bound.
//  dispatch_scatter  one wave per token: the token's row of x is read once
//                    and written to each of its kept rows (16-byte accesses).
#include "common.hpp"

namespace moe {

namespace {

constexpr int kScanCap = 16384; // chunks * local experts kept small for the scan
// The single-launch dispatch reads all selections in every block: used while
// blocks x selections stays within this many reads (32 MB of L2 traffic).
constexpr int64_t kFusedReads = (int64_t)1 << 23;

__device__ __forceinline__ int local_of(int32_t e, int e0, int E_loc)
{
    const int l = e - e0;
    return (l >= 0 && l < E_loc) ? l : -1;
}

__global__ __launch_bounds__(256) void dispatch_count(const int32_t *__restrict__ topk_idx, int64_t items,
                                                      int chunk, int nchunks, int e0, int E_loc,
                                                      int32_t *__restrict__ chunk_count)
{
    extern __shared__ int hist[]; // [4][E_loc]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int *h = hist + wave * E_loc;
    for (int l = lane; l < E_loc; l += 64)
        h[l] = 0;
    __syncthreads();
    const int c = blockIdx.x * 4 + wave;
    if (c < nchunks) {
        const int64_t beg = (int64_t)c * chunk;
        const int64_t end = min(items, beg + chunk);
        for (int64_t i = beg + lane; i < end; i += 64) {
            const int l = local_of(topk_idx[i], e0, E_loc);
            if (l >= 0)
                atomicAdd(&h[l], 1);
        }
    }
    __syncthreads();
    if (c < nchunks)
        for (int l = lane; l < E_loc; l += 64)
            chunk_count[(int64_t)c * E_loc + l] = h[l];
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o)
            v += u;
    }
    return v;
}

// chunk_count [nchunks][E_loc] is turned in place into the per-chunk bases.
// The [nchunks][E_loc] counts are read row by row (consecutive threads take
// consecutive experts, so the accesses coalesce): thread (s, l) owns chunks
// [s per, (s + 1) per) of expert l, the chunk range cut into S = 1024 / E_loc
// segments.  Pass one sums the thread's chunks (eight loads in flight); the
// segment sums are scanned per expert in LDS (a wave per expert); pass two
// writes the exclusive prefixes over the thread's chunks.  Two rounds of
// independent loads instead of one dependent round per 64 chunks.
__global__ __launch_bounds__(1024) void dispatch_scan(int32_t *__restrict__ chunk_cb, int nchunks, int E_loc,
                                                      int64_t cap, int32_t *__restrict__ seg_offsets,
                                                      int32_t *__restrict__ kept_count,
                                                      int32_t *__restrict__ n_dropped)
{
    __shared__ int part[1024]; // [S][E_loc]: segment sums, then their exclusive prefixes
    __shared__ int tot[1024];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = max(1, min(nchunks, 1024 / E_loc));
    const int per = (nchunks + S - 1) / S;
    const int l = tid % E_loc, s = tid / E_loc;
    const bool act = s < S;
    const int c_lo = s * per, c_hi = min(nchunks, c_lo + per);
    if (act) {
        int sum = 0;
        for (int c0 = c_lo; c0 < c_hi; c0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = c0 + u < c_hi ? chunk_cb[(int64_t)(c0 + u) * E_loc + l] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                sum += v[u];
        }
        part[s * E_loc + l] = sum;
    }
    __syncthreads();
    for (int e = wave; e < E_loc; e += 16) {
        int carry = 0;
        for (int q0 = 0; q0 < S; q0 += 64) {
            const int q = q0 + lane;
            const int v = q < S ? part[q * E_loc + e] : 0;
            const int inc = wave_incl_scan(v, lane);
            if (q < S)
                part[q * E_loc + e] = carry + inc - v;
            carry += __shfl(inc, 63, 64);
        }
        if (lane == 0)
            tot[e] = carry;
    }
    __syncthreads();
    if (act) {
        int carry = part[s * E_loc + l];
        for (int c0 = c_lo; c0 < c_hi; c0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = c0 + u < c_hi ? chunk_cb[(int64_t)(c0 + u) * E_loc + l] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (c0 + u < c_hi)
                    chunk_cb[(int64_t)(c0 + u) * E_loc + l] = carry;
                carry += v[u];
            }
        }
    }
    if (wave == 0) {
        int carry = 0, drop = 0;
        for (int l0 = 0; l0 < E_loc; l0 += 64) {
            const int l = l0 + lane;
            int t = 0, kept = 0;
            if (l < E_loc) {
                t = tot[l];
                kept = (cap >= 0 && (int64_t)t > cap) ? (int)cap : t;
            }
            const int inc = wave_incl_scan(kept, lane);
            int dr = t - kept;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                dr += __shfl_xor(dr, o, 64);
            if (l < E_loc) {
                seg_offsets[l] = carry + inc - kept;
                kept_count[l] = kept;
            }
            carry += __shfl(inc, 63, 64);
            drop += dr;
        }
        if (lane == 0) {
            seg_offsets[E_loc] = carry;
            if (n_dropped)
                n_dropped[0] = drop;
        }
    }
}

__global__ __launch_bounds__(256) void dispatch_rank(const int32_t *__restrict__ topk_idx, int64_t items,
                                                     int chunk, int nchunks, int e0, int E_loc, int nbits,
                                                     int64_t cap, const int32_t *__restrict__ chunk_base,
                                                     const int32_t *__restrict__ seg_offsets, int64_t max_rows,
                                                     int32_t *__restrict__ slot_row, int32_t *__restrict__ row_src)
{
    extern __shared__ int run_all[]; // [4][E_loc]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * 4 + wave;
    if (c >= nchunks)
        return; // no block-wide barrier below: waves are independent
    int *run = run_all + wave * E_loc;
    for (int l = lane; l < E_loc; l += 64)
        run[l] = chunk_base[(int64_t)c * E_loc + l];
    const uint64_t below = (1ull << lane) - 1ull;
    const int64_t beg = (int64_t)c * chunk;
    const int64_t end = min(items, beg + chunk);
    for (int64_t i0 = beg; i0 < end; i0 += 64) {
        const int64_t i = i0 + lane;
        const bool valid = i < end;
        const int l = valid ? local_of(topk_idx[i], e0, E_loc) : -1;
        const bool local = l >= 0;
        uint64_t m = __ballot(local);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = local && ((l >> b) & 1);
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        if (local) {
            const int lrank = __popcll(m & below);
            const int base = run[l];
            const int64_t r = (int64_t)base + lrank;
            const bool last = (m >> lane) == 1ull;
            if (last)
                run[l] = base + __popcll(m);
            int32_t out = -1;
            if (cap < 0 || r < cap) {
                const int64_t row = (int64_t)seg_offsets[l] + r;
                if (row < max_rows) {
                    out = (int32_t)row;
                    row_src[row] = (int32_t)i;
                }
            }
            slot_row[i] = out;
        } else if (valid) {
            slot_row[i] = -2;
        }
    }
}

// count + scan + rank in one block of 16 waves for small problems (at most
// 16 chunks, E_loc <= kSmallExperts): the per-chunk counts and bases stay in
// LDS.  Same ranks, rows and counts as dispatch_count / _scan / _rank.
constexpr int kSmallExperts = 256;

__global__ __launch_bounds__(1024) void dispatch_plan_small(const int32_t *__restrict__ topk_idx, int64_t items,
                                                            int chunk, int nchunks, int e0, int E_loc, int nbits,
                                                            int64_t cap, int32_t *__restrict__ seg_offsets,
                                                            int32_t *__restrict__ kept_count,
                                                            int32_t *__restrict__ n_dropped, int64_t max_rows,
                                                            int32_t *__restrict__ slot_row,
                                                            int32_t *__restrict__ row_src)
{
    __shared__ int cb[16][kSmallExperts]; // counts, then running bases per chunk
    __shared__ int tot[kSmallExperts], seg[kSmallExperts + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int q = threadIdx.x; q < 16 * kSmallExperts; q += 1024)
        cb[q / kSmallExperts][q % kSmallExperts] = 0;
    __syncthreads();
    const int c = wave;
    const int64_t beg = (int64_t)c * chunk;
    const int64_t end = min(items, beg + chunk);
    if (c < nchunks) {
        for (int64_t i = beg + lane; i < end; i += 64) {
            const int l = local_of(topk_idx[i], e0, E_loc);
            if (l >= 0)
                atomicAdd(&cb[c][l], 1);
        }
    }
    __syncthreads();
    // exclusive scan over the chunks, per expert
    for (int l = threadIdx.x; l < E_loc; l += 1024) {
        int run = 0;
        for (int q = 0; q < nchunks; ++q) {
            const int v = cb[q][l];
            cb[q][l] = run;
            run += v;
        }
        tot[l] = run;
    }
    __syncthreads();
    if (wave == 0) {
        int carry = 0, drop = 0;
        for (int l0 = 0; l0 < E_loc; l0 += 64) {
            const int l = l0 + lane;
            int t = 0, kept = 0;
            if (l < E_loc) {
                t = tot[l];
                kept = (cap >= 0 && (int64_t)t > cap) ? (int)cap : t;
            }
            const int inc = wave_incl_scan(kept, lane);
            int dr = t - kept;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                dr += __shfl_xor(dr, o, 64);
            if (l < E_loc) {
                seg[l] = carry + inc - kept;
                seg_offsets[l] = carry + inc - kept;
                kept_count[l] = kept;
            }
            carry += __shfl(inc, 63, 64);
            drop += dr;
        }
        if (lane == 0) {
            seg[E_loc] = carry;
            seg_offsets[E_loc] = carry;
            if (n_dropped)
                n_dropped[0] = drop;
        }
    }
    __syncthreads();
    if (c >= nchunks)
        return; // no barrier below
    int *run = cb[c];
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t i0 = beg; i0 < end; i0 += 64) {
        const int64_t i = i0 + lane;
        const bool valid = i < end;
        const int l = valid ? local_of(topk_idx[i], e0, E_loc) : -1;
        const bool local = l >= 0;
        uint64_t m = __ballot(local);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = local && ((l >> b) & 1);
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        if (local) {
            const int lrank = __popcll(m & below);
            const int base = run[l];
            const int64_t r = (int64_t)base + lrank;
            const bool last = (m >> lane) == 1ull;
            if (last)
                run[l] = base + __popcll(m);
            int32_t out = -1;
            if (cap < 0 || r < cap) {
                const int64_t row = (int64_t)seg[l] + r;
                if (row < max_rows) {
                    out = (int32_t)row;
                    row_src[row] = (int32_t)i;
                }
            }
            slot_row[i] = out;
        } else if (valid) {
            slot_row[i] = -2;
        }
    }
}

// Lanes holding the same local expert id: 64-lane ballots over its bits.
__device__ __forceinline__ uint64_t match_mask(int l, bool local, int nbits)
{
    uint64_t m = __ballot(local);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = local && ((l >> b) & 1);
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Whole dispatch in one launch for small selection counts: each block of 16
// waves owns kDispTB tokens.  Every block counts all selections per local
// expert (ballot-matched groups of 64, one LDS add per expert and group) and
// those before its own tokens, derives capacity, kept counts and segment
// offsets itself (block 0 writes them), ranks its own selections in token
// order (count before the block + earlier groups of the block + lanes below
// in the group: the same rank as the multi-kernel path), writes slot_row and
// row_src, and then each wave copies its token's row of x to the token's kept
// rows.  With PREFETCH (no cap and the whole layer local: every selection is
// kept) the first piece of the row (U 16-byte vectors per lane) is loaded
// before the planning, so the row read overlaps it.  The kernel fits 64
// registers, so that two blocks share a CU when the grid has more blocks than
// CUs (a second round of blocks would double the time); the prefetch of
// eight vectors does not, and runs only when the grid fits the CUs (four
// otherwise).
constexpr int kDispTB = 16;

template <bool PREFETCH, int U>
__global__ __launch_bounds__(64 * kDispTB, (PREFETCH && U > 4) ? 1 : 8) void dispatch_fused(
    const int32_t *__restrict__ topk_idx, int64_t T, int k, int e0, int E_loc, int nbits, int64_t cap,
    const u32x4 *__restrict__ x, int64_t units, u32x4 *__restrict__ x_perm, int64_t max_rows,
    int32_t *__restrict__ seg_offsets, int32_t *__restrict__ kept_count, int32_t *__restrict__ n_dropped,
    int32_t *__restrict__ slot_row, int32_t *__restrict__ row_src)
{
    __shared__ int tot[kSmallExperts], pre[kSmallExperts], seg[kSmallExperts + 1];
    __shared__ int gc[8][kSmallExperts]; // counts of the block's own items per group of 64 (k <= 32: <= 8 groups)
    __shared__ int dst[kDispTB * 32];    // row of each own selection (-1 dropped, -2 remote)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t items = T * k;
    const int64_t t0 = (int64_t)blockIdx.x * kDispTB;
    const int64_t i0 = t0 * k, i1 = min(items, (t0 + kDispTB) * k);
    const int64_t t = t0 + wave;
    for (int q = tid; q < E_loc; q += 64 * kDispTB) {
        tot[q] = 0;
        pre[q] = 0;
    }
    // this block's own selections (group `wave` of 64), loaded with the rest
    const int ngr = (int)((i1 - i0 + 63) / 64);
    const int64_t i = i0 + (int64_t)wave * 64 + lane;
    const bool valid = wave < ngr && i < i1;
    const int own_id = valid ? topk_idx[i] : -1;
    u32x4 v[U];
    if (PREFETCH && t < T) {
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int64_t u = q * 64 + lane;
            if (u < units)
                v[q] = x[t * units + u];
        }
    }
    __syncthreads();

    // per-expert counts of all selections and of those before this block's;
    // each wave takes groups of 64, eight groups' ids loaded at once
    constexpr int kBatch = 8;
    for (int64_t b0 = (int64_t)wave * 64; b0 < items; b0 += (int64_t)64 * kDispTB * kBatch) {
        int id[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t i = b0 + (int64_t)u * 64 * kDispTB + lane;
            id[u] = i < items ? topk_idx[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t g0 = b0 + (int64_t)u * 64 * kDispTB;
            if (g0 >= items)
                break; // wave-uniform
            const int l = g0 + lane < items ? local_of(id[u], e0, E_loc) : -1;
            const bool loc = l >= 0;
            const uint64_t m = match_mask(l, loc, nbits);
            if (loc && (m >> lane) == 1ull) { // highest lane of its expert's group
                atomicAdd(&tot[l], __popcll(m));
                const int64_t below = i0 - g0;
                const uint64_t pm = below >= 64 ? ~0ull : (below <= 0 ? 0ull : ((1ull << below) - 1ull));
                const int c = __popcll(m & pm);
                if (c)
                    atomicAdd(&pre[l], c);
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        int carry = 0, drop = 0;
        for (int l0 = 0; l0 < E_loc; l0 += 64) {
            const int l = l0 + lane;
            int tl = 0, kept = 0;
            if (l < E_loc) {
                tl = tot[l];
                kept = (cap >= 0 && (int64_t)tl > cap) ? (int)cap : tl;
            }
            const int inc = wave_incl_scan(kept, lane);
            int dr = tl - kept;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                dr += __shfl_xor(dr, o, 64);
            if (l < E_loc) {
                seg[l] = carry + inc - kept;
                if (blockIdx.x == 0) {
                    seg_offsets[l] = carry + inc - kept;
                    kept_count[l] = kept;
                }
            }
            carry += __shfl(inc, 63, 64);
            drop += dr;
        }
        if (lane == 0) {
            seg[E_loc] = carry;
            if (blockIdx.x == 0) {
                seg_offsets[E_loc] = carry;
                if (n_dropped)
                    n_dropped[0] = drop;
            }
        }
    }

    // rank this block's selections: group `wave` of 64
    const int l = valid ? local_of(own_id, e0, E_loc) : -1;
    uint64_t m = 0;
    if (wave < ngr) {
        m = match_mask(l, l >= 0, nbits);
        for (int q = lane; q < E_loc; q += 64)
            gc[wave][q] = 0;
        if (l >= 0 && (m >> lane) == 1ull)
            gc[wave][l] = __popcll(m);
    }
    __syncthreads();
    if (valid) {
        int32_t out = -2;
        if (l >= 0) {
            int base = pre[l];
            for (int w2 = 0; w2 < wave; ++w2)
                base += gc[w2][l];
            const int64_t r = (int64_t)base + __popcll(m & ((1ull << lane) - 1ull));
            out = -1;
            if (cap < 0 || r < cap) {
                const int64_t row = (int64_t)seg[l] + r;
                if (row < max_rows) {
                    out = (int32_t)row;
                    row_src[row] = (int32_t)i;
                }
            }
        }
        slot_row[i] = out;
        dst[i - i0] = out;
    }
    __syncthreads();

    // scatter: wave w copies token t0 + w to its kept rows
    if (t >= T || !x_perm)
        return;
    bool any = false;
    for (int j = 0; j < k; ++j)
        any |= dst[wave * k + j] >= 0;
    if (!any)
        return;
    for (int64_t u0 = 0; u0 < units; u0 += 64 * U) {
        if (!PREFETCH || u0 > 0) {
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int64_t u = u0 + q * 64 + lane;
                if (u < units)
                    v[q] = x[t * units + u];
            }
        }
        for (int j = 0; j < k; ++j) {
            const int r = dst[wave * k + j];
            if (r < 0)
                continue;
            u32x4 *out = x_perm + (int64_t)r * units;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int64_t u = u0 + q * 64 + lane;
                if (u < units)
                    out[u] = v[q];
            }
        }
    }
}

template <int U>
__global__ __launch_bounds__(256) void dispatch_scatter(const u32x4 *__restrict__ x, const int32_t *__restrict__ slot_row,
                                                        int64_t T, int k, int64_t units, u32x4 *__restrict__ x_perm)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    bool any = false;
    for (int j = 0; j < k; ++j)
        any |= slot_row[t * k + j] >= 0;
    if (!any)
        return;
    const u32x4 *src = x + t * units;
    for (int64_t u0 = 0; u0 < units; u0 += 64 * U) {
        u32x4 v[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int64_t u = u0 + q * 64 + lane;
            if (u < units)
                v[q] = src[u];
        }
        for (int j = 0; j < k; ++j) {
            const int r = slot_row[t * k + j];
            if (r < 0)
                continue;
            u32x4 *dst = x_perm + (int64_t)r * units;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int64_t u = u0 + q * 64 + lane;
                if (u < units)
                    dst[u] = v[q];
            }
        }
    }
}

struct ChunkPlan {
    int chunk, nchunks;
};

ChunkPlan plan_chunks(int64_t items, int E_loc)
{
    int64_t chunk = 512;
    while (((items + chunk - 1) / chunk) * (int64_t)E_loc > kScanCap && chunk < (1 << 30))
        chunk *= 2;
    ChunkPlan p;
    p.chunk = (int)chunk;
    p.nchunks = (int)((items + chunk - 1) / chunk);
    return p;
}

} // namespace

int64_t capacity_of(int64_t T, int E, float capacity_factor)
{
    if (!(capacity_factor > 0.f))
        return -1;
    const double c = floor((double)T * (double)capacity_factor / (double)E);
    if (c >= (double)T)
        return T; // never binding: a token selects an expert at most once
    return (int64_t)c;
}

size_t dispatch_ws_bytes(int64_t T, int k, int E_loc)
{
    const ChunkPlan p = plan_chunks(T * k, E_loc);
    return align_up((size_t)p.nchunks * E_loc * sizeof(int32_t));
}

moe_status_t launch_dispatch(const void *x, moe_dtype_t dt, const int32_t *topk_idx, int64_t T, int d, int E,
                             int k, float capacity_factor, int e0, int E_loc, int32_t *seg_offsets,
                             int32_t *kept_count, int32_t *slot_row, int32_t *row_src, void *x_perm,
                             int64_t max_rows, int32_t *n_dropped, void *ws, hipStream_t stream)
{
    const int64_t items = T * k;
    const int64_t cap = capacity_of(T, E, capacity_factor);
    int nbits = 0;
    while ((1 << nbits) < E_loc)
        ++nbits;
    const int64_t fused_blocks = (T + kDispTB - 1) / kDispTB;
    if (items > 0 && E_loc <= kSmallExperts && k <= 32 && fused_blocks * items <= kFusedReads) {
        // one launch: every block counts all selections itself
        const int64_t units = x ? (int64_t)d * (dt == MOE_BF16 ? 2 : 4) / 16 : 0;
        const bool prefetch = x_perm && cap < 0 && E_loc == E;
        if (prefetch && fused_blocks > device_cus())
            dispatch_fused<true, 4><<<(unsigned)fused_blocks, 64 * kDispTB, 0, stream>>>(
                topk_idx, T, k, e0, E_loc, nbits, cap, (const u32x4 *)x, units, (u32x4 *)x_perm, max_rows,
                seg_offsets, kept_count, n_dropped, slot_row, row_src);
        else if (prefetch)
            dispatch_fused<true, 8><<<(unsigned)fused_blocks, 64 * kDispTB, 0, stream>>>(
                topk_idx, T, k, e0, E_loc, nbits, cap, (const u32x4 *)x, units, (u32x4 *)x_perm, max_rows,
                seg_offsets, kept_count, n_dropped, slot_row, row_src);
        else
            dispatch_fused<false, 8><<<(unsigned)fused_blocks, 64 * kDispTB, 0, stream>>>(
                topk_idx, T, k, e0, E_loc, nbits, cap, (const u32x4 *)x, units, (u32x4 *)x_perm, max_rows,
                seg_offsets, kept_count, n_dropped, slot_row, row_src);
        return check_launch("dispatch_fused");
    }
    if (items > 0 && items <= 16 * 2048 && E_loc <= kSmallExperts) {
        // one block plans the whole dispatch: 16 chunks of a multiple of 64
        const int chunk = (int)((items + 16 * 64 - 1) / (16 * 64) * 64);
        const int nch = (int)((items + chunk - 1) / chunk);
        dispatch_plan_small<<<1, 1024, 0, stream>>>(topk_idx, items, chunk, nch, e0, E_loc, nbits, cap, seg_offsets,
                                                    kept_count, n_dropped, max_rows, slot_row, row_src);
        if (moe_status_t s = check_launch("dispatch_plan_small"))
            return s;
    } else {
        const ChunkPlan p = plan_chunks(items, E_loc);
        int32_t *chunk_cb = (int32_t *)ws;
        const size_t lds = (size_t)4 * E_loc * sizeof(int);
        const unsigned blocks = (unsigned)((p.nchunks + 3) / 4);
        if (items > 0) {
            dispatch_count<<<blocks, 256, lds, stream>>>(topk_idx, items, p.chunk, p.nchunks, e0, E_loc, chunk_cb);
            if (moe_status_t s = check_launch("dispatch_count"))
                return s;
        }
        dispatch_scan<<<1, 1024, 0, stream>>>(chunk_cb, items > 0 ? p.nchunks : 0, E_loc, cap, seg_offsets,
                                              kept_count, n_dropped);
        if (moe_status_t s = check_launch("dispatch_scan"))
            return s;
        if (items == 0)
            return MOE_OK;
        dispatch_rank<<<blocks, 256, lds, stream>>>(topk_idx, items, p.chunk, p.nchunks, e0, E_loc, nbits, cap,
                                                    chunk_cb, seg_offsets, max_rows, slot_row, row_src);
        if (moe_status_t s = check_launch("dispatch_rank"))
            return s;
    }
    if (x_perm) {
        const int64_t units = (int64_t)d * (dt == MOE_BF16 ? 2 : 4) / 16;
        dispatch_scatter<8><<<(unsigned)((T + 3) / 4), 256, 0, stream>>>((const u32x4 *)x, slot_row, T, k, units,
                                                                         (u32x4 *)x_perm);
        if (moe_status_t s = check_launch("dispatch_scatter"))
            return s;
    }
    return MOE_OK;
}

} // namespace moe
