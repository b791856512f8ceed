// Routing layout of one tile of pairs, run by one workgroup of 1024 lanes (internal header).
//
// Definition (the dispatch-layout step of the "normal" EP APIs, awsome-distributed-ai PR
// #1238, "What changed"): pair i = t*K + j of a routed expert e takes position
// #{i' < i : id[i'] == e}; positions >= C are dropped.
//
// A tile is the pairs [tile_begin, tile_begin + P), P <= 1024 and a multiple of 4, one pair per
// lane so lane order is pair order. Bins are the E experts, then two bins that are never ranked:
// E for invalid ids (outside [0, E) and not -1) and E+1 for unrouted ones (-1).
//  1. The workgroup counts, per bin, the pairs of all EARLIER tiles: 16-byte id vectors, all in
//     flight at once, then one LDS atomic per id (the counts do not depend on the order of the
//     atomics).
//  2. Inside the tile, each wavefront finds, for every routed lane, the mask of lanes holding
//     the same expert with one ballot per bit of the expert number (bit-sliced match). The
//     lane's rank is the number of mask bits below it (v_mbcnt); the lowest lane of each group
//     writes the group size into a per-wavefront histogram in LDS.
//  3. A scan over the 16 wavefronts, per expert (16 lanes = one DPP row per expert), turns those
//     histograms into per-wavefront bases starting from the earlier-tile count, so
//     slot = base + rank, or -1 past C.
// The workgroup of the last tile then holds the total of every bin and finishes the layout:
//  4. count = min(total, C), its exclusive scan in expert order (DPP wave scans plus wave
//     totals), the per-rank sums and the stats; dropped = routed - kept.
// No workgroup waits on another and no result depends on scheduling: the outputs are
// deterministic and need no workspace. The cost is the pass over all earlier ids, one memory
// round trip plus ~tile_begin/1024 LDS atomics per lane.
#pragma once

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

constexpr int kTileThreads = 1024;
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kTileMaxBins = EP_MAX_EXPERTS + 2;
constexpr int kPrefixVec = 8;      // 16-byte id vectors in flight per lane in step 1

struct LayoutLds {
    int32_t base[kTileMaxBins];                 // earlier-tile counts, then running totals
    int32_t wcnt[kTileWaves][kTileMaxBins];     // per-wavefront counts, then bases
    int32_t scan[EP_MAX_EXPERTS + 1];           // exclusive scan of count, then total
    int32_t wsum[kTileWaves];
};

// Bin of an id: itself for an expert, E for an invalid id, E+1 for -1 (unrouted).
__device__ __forceinline__ int layout_bin(int e, int E)
{
    return (int)min((unsigned)e, (unsigned)E) + (e == -1 ? 1 : 0);
}

// Steps 1-3 for the tile [tile_begin, tile_begin + P). Writes slot[] for the tile's pairs and,
// if rows is not null, rows[k] = e*C + slot (or -1 for a pair that is not kept) for local pair
// k. `last` marks the workgroup that will call layout_finish. Ends with a barrier.
__device__ __forceinline__ void layout_tile(const int32_t *__restrict__ idx, int TK, int E, int C,
                                            int nbits, int tile_begin, int P, bool last,
                                            LayoutLds &L, int32_t *__restrict__ slot,
                                            int32_t *rows)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // this lane's own pair, loaded first so its latency overlaps the prefix histogram
    const int p = tile_begin + tid;
    const bool in = tid < P && p < TK;
    const int own = in ? idx[p] : -1;

    for (int k = tid; k < E + 2; k += kTileThreads) {
        L.base[k] = 0;
#pragma unroll
        for (int w = 0; w < kTileWaves; ++w) L.wcnt[w][k] = 0;
    }
    __syncthreads();

    // 1. histogram of the earlier tiles. tile_begin is a multiple of 4, so the prefix is whole
    //    16-byte vectors; up to kPrefixVec of them per lane are in flight together. Addresses
    //    past the prefix are clamped to its last vector and their counts skipped.
    if (tile_begin > 0) {
        const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
        const int nvec = tile_begin / 4;
        for (int q0 = tid; q0 < nvec; q0 += kPrefixVec * kTileThreads) {
            int4 v[kPrefixVec];
#pragma unroll
            for (int u = 0; u < kPrefixVec; ++u) {
                const int q = q0 + u * kTileThreads;
                v[u] = idx4[q < nvec ? q : nvec - 1];
            }
#pragma unroll
            for (int u = 0; u < kPrefixVec; ++u) {
                const bool ok = q0 + u * kTileThreads < nvec;
                const int e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (ok) atomicAdd(&L.base[layout_bin(e4[c], E)], 1);
            }
        }
    }

    // 2. ranks of the routed lanes inside the wavefront by bit-sliced ballot matching
    const bool routed = in && (unsigned)own < (unsigned)E;
    if (last) {                     // this tile's pairs in the two non-expert bins, for the stats
        const int unrouted = __popcll(__ballot(in && own == -1));
        const int invalid = __popcll(__ballot(in && own != -1 && !routed));
        if (lane == 0 && unrouted) atomicAdd(&L.base[E + 1], unrouted);
        if (lane == 0 && invalid) atomicAdd(&L.base[E], invalid);
    }
    uint64_t same = __ballot(routed);
    for (int k = 0; k < nbits; ++k) {
        const bool bit = (own >> k) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    const int rank = count_below(same);
    if (routed && rank == 0) L.wcnt[wave][own] = __popcll(same);
    __syncthreads();

    // 3. per-expert exclusive scan over the 16 wavefronts, from the earlier-tile base: the 16
    //    counts of an expert sit in one DPP row of 16 lanes
    for (int k = tid; k < E * kTileWaves; k += kTileThreads) {
        const int e = k / kTileWaves, w = k % kTileWaves;
        const int c = L.wcnt[w][e];
        const int incl = row16_inclusive_sum(c);
        const int b0 = L.base[e];
        L.wcnt[w][e] = b0 + incl - c;
        // the 16 lanes of an expert are in one wavefront and read b0 before this write
        if (w == kTileWaves - 1) L.base[e] = b0 + incl;
    }
    __syncthreads();
    if (in) {
        int s = -1;
        if (routed) {
            const int pos = L.wcnt[wave][own] + rank;
            s = pos < C ? pos : -1;
        }
        slot[p] = s;
        if (rows) rows[tid] = s >= 0 ? own * C + s : -1;
    }
    __syncthreads();
}

// Step 4, by the workgroup of the last tile after layout_tile: L.base[e] is the total of
// expert e, L.base[E] / L.base[E+1] the invalid / unrouted totals.
__device__ __forceinline__ void layout_finish(int TK, int E, int C, int R, LayoutLds &L,
                                              const LayoutOut &o)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int cnt = tid < E ? min(L.base[tid], C) : 0;     // E <= kTileThreads
    const int incl = wave_inclusive_sum(cnt);
    if (lane == kWave - 1) L.wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += L.wsum[w];
    const int excl = wbase + incl - cnt;
    if (tid < E) {
        o.count[tid] = cnt;
        o.offset[tid] = excl;
        L.scan[tid] = excl;
    }
    if (tid == E - 1) L.scan[E] = excl + cnt;             // total kept
    __syncthreads();
    const int EL = E / R;
    for (int r = tid; r < R; r += kTileThreads) {
        const int lo = L.scan[r * EL], hi = L.scan[(r + 1) * EL];
        if (o.rank_count) o.rank_count[r] = hi - lo;
        if (o.rank_offset) o.rank_offset[r] = lo;
    }
    if (tid == 0) {
        const int kept = L.scan[E], unrouted = L.base[E + 1], invalid = L.base[E];
        o.stats[0] = kept;
        o.stats[1] = TK - unrouted - invalid - kept;
        o.stats[2] = unrouted;
        o.stats[3] = invalid;
    }
}

// Bits needed for expert numbers 0 .. E-1.
inline int expert_bits(int E)
{
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    return nbits;
}

}  // namespace ep
