// Routing layout on gfx950: per-expert counts, exclusive offsets and stable in-order slots
// under a capacity, with drops.
//
// Definition (the dispatch-layout step of the "normal" EP APIs, awsome-distributed-ai PR
// #1238, "What changed"): pair i = t*K + j of a routed expert e takes position
// #{i' < i : id[i'] == e}; positions >= C are dropped.
//
// Design. Pairs are cut into tiles of 1024, one workgroup of 16 wavefronts per tile, one pair
// per lane, so lane order is pair order.
//  1. Each workgroup counts, per bin, the pairs of all EARLIER tiles (LDS histogram with
//     atomics; the counts do not depend on the order of the atomics). Bins are the E experts,
//     then "unrouted" (id -1) and "invalid" (any other id outside [0, E)).
//  2. Inside its tile, each wavefront finds, for every lane, the mask of lanes holding the same
//     bin with one ballot per bit of the bin number (bit-sliced match). The lane's rank is the
//     popcount of that mask below it; the lowest lane of each group writes the group size into
//     a per-wavefront histogram in LDS.
//  3. A scan over the 16 wavefronts, per bin, turns those histograms into per-wavefront bases,
//     starting from the earlier-tile count of step 1, so slot = base + rank, or -1 past C.
//  4. The last workgroup, which now holds the totals of every bin, writes count = min(total, C),
//     the exclusive scan of count (an LDS block scan), the per-rank sums and the stats.
// No workgroup waits on another and no result depends on scheduling: the outputs are
// deterministic and need no workspace.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kLayoutThreads = 1024;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kMaxBins = EP_MAX_EXPERTS + 2;

__device__ __forceinline__ int bin_of(int e, int E)
{
    return ((unsigned)e < (unsigned)E) ? e : (e == -1 ? E : E + 1);
}

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(
    const int32_t *__restrict__ idx, int TK, int E, int C, int R, int nbits,
    int32_t *__restrict__ slot, int32_t *__restrict__ count, int32_t *__restrict__ offset,
    int32_t *__restrict__ rank_count, int32_t *__restrict__ rank_offset,
    int32_t *__restrict__ stats)
{
    __shared__ int32_t base[kMaxBins];                  // earlier-tile counts, then totals
    __shared__ int32_t wcnt[kLayoutWaves][kMaxBins];    // per-wavefront counts, then bases
    __shared__ int32_t scan[EP_MAX_EXPERTS + 1];        // exclusive scan of count, then total
    __shared__ int32_t wsum[kLayoutWaves];
    __shared__ int32_t dropped_total;

    const int NB = E + 2;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int tile_begin = blockIdx.x * kLayoutThreads;

    for (int k = tid; k < NB; k += kLayoutThreads) {
        base[k] = 0;
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) wcnt[w][k] = 0;
    }
    if (tid == 0) dropped_total = 0;
    __syncthreads();

    // 1. histogram of the earlier tiles, eight independent loads in flight per lane
    {
        int p = tid;
        for (; p + 7 * kLayoutThreads < tile_begin; p += 8 * kLayoutThreads) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = idx[p + u * kLayoutThreads];
#pragma unroll
            for (int u = 0; u < 8; ++u) atomicAdd(&base[bin_of(v[u], E)], 1);
        }
        for (; p < tile_begin; p += kLayoutThreads) atomicAdd(&base[bin_of(idx[p], E)], 1);
    }

    // 2. ranks inside the wavefront by bit-sliced ballot matching
    const int p = tile_begin + tid;
    const bool in = p < TK;
    const int b = in ? bin_of(idx[p], E) : 0;
    uint64_t same = __ballot(in);
    for (int k = 0; k < nbits; ++k) {
        const bool bit = (b >> k) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lanemask_lt(lane));
    if (in && rank == 0) wcnt[wave][b] = __popcll(same);
    __syncthreads();

    // 3. per-bin scan over wavefronts, from the earlier-tile base
    for (int k = tid; k < NB; k += kLayoutThreads) {
        int run = base[k];
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) {
            const int c = wcnt[w][k];
            wcnt[w][k] = run;
            run += c;
        }
        base[k] = run;
    }
    __syncthreads();
    if (in) {
        int s = -1;
        if (b < E) {
            const int pos = wcnt[wave][b] + rank;
            s = pos < C ? pos : -1;
        }
        slot[p] = s;
    }
    if (blockIdx.x != gridDim.x - 1) return;

    // 4. last tile: totals are complete; counts, offsets, ranks and stats
    int cnt = 0, drop = 0;
    for (int e = tid; e < E; e += kLayoutThreads) {   // E <= kLayoutThreads: one expert per lane
        const int d = base[e];
        cnt = d < C ? d : C;
        drop = d - cnt;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    int wdrop = drop;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wdrop += __shfl_xor(wdrop, o);
    if (lane == kWave - 1) wsum[wave] = incl;
    if (lane == 0 && wdrop) atomicAdd(&dropped_total, wdrop);
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    const int excl = wbase + incl - cnt;
    if (tid < E) {
        count[tid] = cnt;
        offset[tid] = excl;
        scan[tid] = excl;
    }
    if (tid == 0) {
        int total = 0;
        for (int w = 0; w < kLayoutWaves; ++w) total += wsum[w];
        scan[E] = total;
    }
    __syncthreads();
    const int EL = E / R;
    for (int r = tid; r < R; r += kLayoutThreads) {
        const int lo = scan[r * EL], hi = scan[(r + 1) * EL];
        if (rank_count) rank_count[r] = hi - lo;
        if (rank_offset) rank_offset[r] = lo;
    }
    if (tid == 0) {
        stats[0] = scan[E];
        stats[1] = dropped_total;
        stats[2] = base[E];
        stats[3] = base[E + 1];
    }
}

}  // namespace

hipError_t launch_layout(const ep_shape_t &s, const int32_t *idx, int32_t *slot, int32_t *count,
                         int32_t *offset, int32_t *rank_count, int32_t *rank_offset,
                         int32_t *stats, hipStream_t stream)
{
    const int TK = s.T * s.K;
    const int tiles = TK > 0 ? (TK + kLayoutThreads - 1) / kLayoutThreads : 1;
    int nbits = 0;
    while ((1 << nbits) < s.E + 2) ++nbits;   // bins 0 .. E+1
    return launch(layout_kernel, dim3(tiles), dim3(kLayoutThreads), 0, stream, idx, TK, s.E,
                  s.C, s.R, nbits, slot, count, offset, rank_count, rank_offset, stats);
}

}  // namespace ep
