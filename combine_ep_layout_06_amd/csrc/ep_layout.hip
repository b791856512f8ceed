// Routing layout on gfx950: per-expert counts, exclusive offsets and stable in-order slots
// under a capacity, with drops.
//
// Definition (the dispatch-layout step of the "normal" EP APIs, awsome-distributed-ai PR
// #1238, "What changed"): pair i = t*K + j of a routed expert e takes position
// #{i' < i : id[i'] == e}; positions >= C are dropped.
//
// Design. Pairs are cut into tiles of 1024, one workgroup of 16 wavefronts per tile, one pair
// per lane, so lane order is pair order. Bins are the E experts, then two bins that are never
// ranked: E for invalid ids (outside [0, E) and not -1) and E+1 for unrouted ones (-1).
//  1. Each workgroup counts, per bin, the pairs of all EARLIER tiles: 16-byte id vectors, all in
//     flight at once, then one LDS atomic per id (the counts do not depend on the order of the
//     atomics).
//  2. Inside its tile, each wavefront finds, for every routed lane, the mask of lanes holding
//     the same expert with one ballot per bit of the expert number (bit-sliced match). The
//     lane's rank is the number of mask bits below it (v_mbcnt); the lowest lane of each group
//     writes the group size into a per-wavefront histogram in LDS.
//  3. A scan over the 16 wavefronts, per expert (16 lanes = one DPP row per expert), turns those
//     histograms into per-wavefront bases starting from the earlier-tile count, so
//     slot = base + rank, or -1 past C.
//  4. The last workgroup, which now holds the total of every expert, writes
//     count = min(total, C), its exclusive scan (DPP wave scans plus wave totals), the per-rank
//     sums and the stats; dropped = routed - kept.
// No workgroup waits on another and no result depends on scheduling: the outputs are
// deterministic and need no workspace. The cost is the last workgroup's pass over all earlier
// ids, which is one memory round trip plus ~T*K/1024 LDS atomics per lane.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kLayoutThreads = 1024;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kMaxBins = EP_MAX_EXPERTS + 2;
constexpr int kPrefixVec = 8;     // 16-byte id vectors in flight per lane in step 1

// Bin of an id: itself for an expert, E for an invalid id, E+1 for -1 (unrouted).
__device__ __forceinline__ int bin_of(int e, int E)
{
    return (int)min((unsigned)e, (unsigned)E) + (e == -1 ? 1 : 0);
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

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int tile_begin = blockIdx.x * kLayoutThreads;
    const bool last = blockIdx.x == gridDim.x - 1;

    // this lane's own pair, loaded first so its latency overlaps the prefix histogram
    const int p = tile_begin + tid;
    const bool in = p < TK;
    const int own = in ? idx[p] : -1;

    for (int k = tid; k < E + 2; k += kLayoutThreads) {
        base[k] = 0;
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) wcnt[w][k] = 0;
    }
    __syncthreads();

    // 1. histogram of the earlier tiles. A tile is 4 KiB of ids, so the prefix is whole 16-byte
    //    vectors; up to kPrefixVec of them per lane are in flight together. Addresses past the
    //    prefix are clamped to its last vector and their counts skipped.
    if (tile_begin > 0) {
        const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
        const int nvec = tile_begin / 4;
        for (int q0 = tid; q0 < nvec; q0 += kPrefixVec * kLayoutThreads) {
            int4 v[kPrefixVec];
#pragma unroll
            for (int u = 0; u < kPrefixVec; ++u) {
                const int q = q0 + u * kLayoutThreads;
                v[u] = idx4[q < nvec ? q : nvec - 1];
            }
#pragma unroll
            for (int u = 0; u < kPrefixVec; ++u) {
                const bool ok = q0 + u * kLayoutThreads < nvec;
                const int e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (ok) atomicAdd(&base[bin_of(e4[c], E)], 1);
            }
        }
    }

    // 2. ranks of the routed lanes inside the wavefront by bit-sliced ballot matching
    const bool routed = in && (unsigned)own < (unsigned)E;
    if (last) {                     // this tile's pairs in the two non-expert bins, for the stats
        const int unrouted = __popcll(__ballot(in && own == -1));
        const int invalid = __popcll(__ballot(in && own != -1 && !routed));
        if (lane == 0 && unrouted) atomicAdd(&base[E + 1], unrouted);
        if (lane == 0 && invalid) atomicAdd(&base[E], invalid);
    }
    uint64_t same = __ballot(routed);
    for (int k = 0; k < nbits; ++k) {
        const bool bit = (own >> k) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    const int rank = count_below(same);
    if (routed && rank == 0) wcnt[wave][own] = __popcll(same);
    __syncthreads();

    // 3. per-expert exclusive scan over the 16 wavefronts, from the earlier-tile base: the 16
    //    counts of an expert sit in one DPP row of 16 lanes
    for (int k = tid; k < E * kLayoutWaves; k += kLayoutThreads) {
        const int e = k / kLayoutWaves, w = k % kLayoutWaves;
        const int c = wcnt[w][e];
        const int incl = row16_inclusive_sum(c);
        const int b0 = base[e];
        wcnt[w][e] = b0 + incl - c;
        // the 16 lanes of an expert are in one wavefront and read b0 before this write
        if (w == kLayoutWaves - 1) base[e] = b0 + incl;
    }
    __syncthreads();
    if (in) {
        int s = -1;
        if (routed) {
            const int pos = wcnt[wave][own] + rank;
            s = pos < C ? pos : -1;
        }
        slot[p] = s;
    }
    if (!last) return;

    // 4. last tile: base[e] is the total of expert e. count = min(total, C), its exclusive
    //    scan in expert order, per-rank sums, stats. Every routed pair is kept or dropped.
    const int cnt = tid < E ? min(base[tid], C) : 0;     // E <= kLayoutThreads
    const int incl = wave_inclusive_sum(cnt);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    const int excl = wbase + incl - cnt;
    if (tid < E) {
        count[tid] = cnt;
        offset[tid] = excl;
        scan[tid] = excl;
    }
    if (tid == E - 1) scan[E] = excl + cnt;             // total kept
    __syncthreads();
    const int EL = E / R;
    for (int r = tid; r < R; r += kLayoutThreads) {
        const int lo = scan[r * EL], hi = scan[(r + 1) * EL];
        if (rank_count) rank_count[r] = hi - lo;
        if (rank_offset) rank_offset[r] = lo;
    }
    if (tid == 0) {
        const int kept = scan[E], unrouted = base[E + 1], invalid = base[E];
        stats[0] = kept;
        stats[1] = TK - unrouted - invalid - kept;
        stats[2] = unrouted;
        stats[3] = invalid;
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
    while ((1 << nbits) < s.E) ++nbits;   // expert numbers 0 .. E-1
    return launch(layout_kernel, dim3(tiles), dim3(kLayoutThreads), 0, stream, idx, TK, s.E,
                  s.C, s.R, nbits, slot, count, offset, rank_count, rank_offset, stats);
}

}  // namespace ep
