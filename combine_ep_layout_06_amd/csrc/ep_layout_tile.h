// Routing layout of one tile of pairs, run by one workgroup of 1024 lanes (internal header).
//
// Definition (the dispatch-layout step of the "normal" EP APIs, awsome-distributed-ai PR
// #1238, "What changed"): pair i = t*K + j of a routed expert e takes position
// #{i' < i : id[i'] == e}; positions >= C are dropped.
//
// A tile is the pairs [tile_begin, tile_begin + P), P <= 1024 and a multiple of 4, one pair per
// lane so lane order is pair order. Bins are the E experts, then two bins that are never ranked:
// E for invalid ids (outside [0, E) and not -1) and E+1 for unrouted ones (-1).
//  0. Every global load the layout needs is issued first, in one go: the ids of the earlier
//     tiles (16-byte vectors, up to kPrefixVec per lane) and the lane's own id, so the tile pays
//     one memory round trip before its LDS work.
//  1. The workgroup counts, per bin, the pairs of all EARLIER tiles with one LDS atomic per id
//     (the counts do not depend on the order of the atomics) into a replicated histogram: NC
//     copies of every bin, interleaved, and lane l adds into copy l % NC, so lanes that hit the
//     same bin hit different banks (on MI355X a single histogram costs ~2.3x more than
//     conflict-free atomics: random bins collide in the banks; 16 copies bring it to ~1.1x).
//  2. Inside the tile, each wavefront finds, for every routed lane, the mask of lanes holding
//     the same expert with one ballot per bit of the expert number (bit-sliced match). The
//     lane's rank is the number of mask bits below it (v_mbcnt); the lowest lane of each group
//     writes the group size into a per-wavefront histogram in LDS.
//  3. Per expert, 16 lanes (one DPP row) fold the NC copies into the earlier-tile count and
//     scan the 16 per-wavefront counts from it, so each wavefront gets its base;
//     slot = base + rank, or -1 past C.
// The workgroup of the last tile then holds the total of every bin and finishes the layout:
//  4. count = min(total, C), its exclusive scan in expert order (DPP wave scans plus wave
//     totals), the per-rank sums and the stats; dropped = routed - kept. For a packed layout the
//     scan and the rank sums are over the counts rounded up to the alignment, and the total
//     number of rows follows the offsets.
// No workgroup waits on another and no result depends on scheduling: the outputs are
// deterministic and need no workspace. The cost is the pass over all earlier ids, one memory
// round trip plus ~tile_begin/1024 conflict-free LDS atomics per lane.
//
// ALL (packed layout fused with dispatch): a pair's packed row offset[e] + slot needs every
// expert's total, so the tile also counts the ids AFTER it, into a second replicated histogram
// (each id of the batch still costs one atomic). Step 3 then yields each expert's total, and
// every workgroup scans the counts rounded up to the alignment into the packed offsets itself.
//
// CHUNKED (large batches, with a workspace): a first launch (layout_chunk_hist_kernel) writes
// the histogram of every chunk of kLayoutChunk pairs to the workspace. Step 1 then adds, per
// bin, the histograms of the chunks before the tile's chunk (lanes split over bins and chunks,
// plain loads and adds) and counts only the earlier ids of its own chunk (at most one 16-byte
// vector per lane). A workgroup's step 1 reads (T*K / kLayoutChunk) * (E + 2) words instead of
// up to T*K ids; the results are the same.
//
// LDS is the launch's dynamic shared memory, carved by layout_lds_map(E, lg_nc); its size grows
// with E (17 KB at E = 128, 140 KB at E = 1024).
#pragma once

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

constexpr int kTileThreads = 1024;
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kPrefixVec = 8;      // 16-byte id vectors per lane issued up front in step 0
constexpr int kLayoutChunk = 4096; // CHUNKED: pairs per chunk histogram (one vector per lane)
static_assert(kLayoutChunk == 4 * kTileThreads, "a chunk is one 16-byte id vector per lane");

// Chunks of kLayoutChunk pairs in a batch of TK pairs (the CHUNKED workspace holds one histogram
// of E + 2 bins per chunk).
__host__ __device__ inline int layout_chunks(int TK) { return (TK + kLayoutChunk - 1) / kLayoutChunk; }
constexpr int kHistWords = (EP_MAX_EXPERTS + 2) * 16;   // budget of the replicated histogram

// Copies per bin of the replicated histogram (a power of two, 16..64). More copies spread the
// atomics of one instruction over more banks but cost more LDS to clear and fold; 16 measured
// best on MI355X across the batch sizes here.
#ifndef EP_LAYOUT_NC
#define EP_LAYOUT_NC 16
#endif

// Word offsets of the layout's LDS arrays, from E and the histogram copies (the same on host
// and device).
struct LayoutLdsMap {
    int B;        // bins: E experts, invalid, unrouted
    int lg_nc;    // log2 of the histogram copies per bin (4, 5 or 6)
    int wcnt;     // [kTileWaves][B]: per-wavefront counts, then bases
    int hist;     // [B][NC]: replicated earlier-tile histogram
    int base;     // [B]: running totals (earlier tiles + this tile) of the experts
    int scan;     // [E + 1]: exclusive scan of count, then the total kept
    int wsum;     // [kTileWaves], then the invalid and unrouted totals
    int ksum;     // [kTileWaves]: kept counts per wavefront (differ from wsum when padded)
    int hist2;    // ALL: [B][NC] replicated histogram of the later tiles (before base)
    int tot;      // ALL: [E] totals of the experts
    int off;      // ALL: [E] packed offsets
    int words;    // total
};

// log2 of the copies for E experts: EP_LAYOUT_NC, fewer if the histogram would not fit.
inline int layout_lg_nc(int E)
{
    int lg = 4;
    while ((2 << lg) <= EP_LAYOUT_NC && lg < 6) ++lg;
    while (lg > 4 && ((E + 2) << lg) > kHistWords) --lg;
    return lg;
}

__host__ __device__ inline LayoutLdsMap layout_lds_map(int E, int lg_nc, bool all = false)
{
    LayoutLdsMap m;
    m.B = E + 2;
    m.lg_nc = lg_nc;
    const int wcnt_words = (kTileWaves * m.B + 3) & ~3;   // keep hist 16-byte aligned
    m.wcnt = 0;
    m.hist = wcnt_words;
    m.hist2 = m.hist + (m.B << m.lg_nc);                  // cleared together with hist
    m.base = m.hist2 + (all ? (m.B << m.lg_nc) : 0);
    m.scan = m.base + ((m.B + 3) & ~3);
    m.wsum = m.scan + ((E + 1 + 3) & ~3);
    m.ksum = m.wsum + kTileWaves + 2;
    m.tot = m.ksum + kTileWaves;
    m.off = m.tot + (all ? E : 0);
    m.words = m.off + (all ? E : 0);
    return m;
}

inline size_t layout_lds_bytes(int E, int lg_nc, bool all = false)
{
    return (size_t)layout_lds_map(E, lg_nc, all).words * 4;
}

// Bin of an id: itself for an expert, E for an invalid id, E+1 for -1 (unrouted).
__device__ __forceinline__ int layout_bin(int e, int E)
{
    return (int)min((unsigned)e, (unsigned)E) + (e == -1 ? 1 : 0);
}

// Sum over each row of 16 lanes, in every lane of the row (DPP butterfly: swap neighbours,
// swap pairs, mirror the half-rows, mirror the row).
__device__ __forceinline__ int row16_total(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
    return v;
}

// Step 0: the global loads of a tile, issued before anything waits on memory.
struct TileIds {
    int4 v[kPrefixVec];   // earlier-tile id vectors tid + u*1024 (clamped; see layout_tile)
    int own;              // this lane's pair, -1 past the tile or the batch
    int tail;             // ALL: one of the last TK % 4 ids if they come after the tile
};

// ALL: the vectors other than the tile's own, numbered 0 .. nb + (se - sb): the nb earlier
// ones, then vectors sb .. se of the later ones (se = TK / 4 whole vectors; the TK % 4 ids past
// them are the tails).
struct OtherVecs {
    int nb, sb, se;
    __device__ int count() const { return nb + (se - sb); }
    __device__ int phys(int v) const { return v < nb ? v : sb + (v - nb); }
};

__device__ __forceinline__ OtherVecs other_vecs(int TK, int tile_begin, int P)
{
    OtherVecs o;
    o.nb = tile_begin / 4;
    o.se = TK / 4;
    o.sb = min((tile_begin + P) / 4, o.se);     // P is a multiple of 4
    return o;
}

template <bool ALL = false, bool CHUNKED = false>
__device__ __forceinline__ TileIds layout_tile_loads(const int32_t *__restrict__ idx, int TK,
                                                     int tile_begin, int P)
{
    TileIds t;
    const int tid = threadIdx.x;
    const int p = tile_begin + tid;
    t.own = (tid < P && p < TK) ? idx[p] : -1;
    t.tail = -1;
    // a batch is issued only if some lane of the wavefront needs it: the load pipe of a CU
    // moves ~64 bytes per clock, so clamped duplicates would still cost issue time
    if constexpr (CHUNKED) {
        // the earlier vectors of the tile's own chunk: fewer than kLayoutChunk / 4 = 1024
        const int cb4 = (tile_begin / kLayoutChunk) * (kLayoutChunk / 4);
        const int nv = tile_begin / 4 - cb4;
        const int wave_q0 = __builtin_amdgcn_readfirstlane(tid & ~(kWave - 1));
        const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
#pragma unroll
        for (int u = 0; u < kPrefixVec; ++u) t.v[u] = int4{0, 0, 0, 0};
        if (wave_q0 < nv && tid < nv) t.v[0] = idx4[cb4 + tid];
    } else if constexpr (ALL) {
        const int tp = (TK / 4) * 4 + tid;      // a tail id past the tile
        if (tid < TK % 4 && tp >= tile_begin + P) t.tail = idx[tp];
        const OtherVecs ov = other_vecs(TK, tile_begin, P);
        const int nvec = ov.count();
        const int wave_q0 = __builtin_amdgcn_readfirstlane(tid & ~(kWave - 1));
        const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
#pragma unroll
        for (int u = 0; u < kPrefixVec; ++u) {
            t.v[u] = int4{0, 0, 0, 0};
            if (wave_q0 + u * kTileThreads < nvec) {
                const int q = tid + u * kTileThreads;
                t.v[u] = idx4[ov.phys(q < nvec ? q : nvec - 1)];
            }
        }
    } else {
        const int nvec = tile_begin / 4;      // tile_begin is a multiple of 4: whole vectors
        const int wave_q0 = __builtin_amdgcn_readfirstlane(tid & ~(kWave - 1));
        const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
#pragma unroll
        for (int u = 0; u < kPrefixVec; ++u) {
            t.v[u] = int4{0, 0, 0, 0};
            if (wave_q0 + u * kTileThreads < nvec) {
                const int q = tid + u * kTileThreads;
                t.v[u] = idx4[q < nvec ? q : nvec - 1];
            }
        }
    }
    return t;
}

// Steps 1-3 for the tile [tile_begin, tile_begin + P), with its loads `ids` from
// layout_tile_loads. Writes slot[] for the tile's pairs and, if rows is not null,
// rows[k] = e*C + slot (or -1 for a pair that is not kept) for local pair k. `last` marks the
// workgroup that will call layout_finish. Ends with a barrier.
// ALL: also counts the later tiles, and rows[k] = off[e] + slot, the pair's row in a packed
// buffer of rows_cap rows with each expert's count rounded up to `align` (-1 if not kept or
// past the buffer); the packed offsets are left in LDS at m.off.
template <bool ALL = false, bool CHUNKED = false>
__device__ __forceinline__ void layout_tile(const TileIds &ids, const int32_t *__restrict__ idx,
                                            int TK, int E, int C, int nbits, int tile_begin,
                                            int P, bool last, int32_t *lds,
                                            const LayoutLdsMap &m,
                                            int32_t *__restrict__ slot, int32_t *rows,
                                            int align = 1, int rows_cap = 0,
                                            const int32_t *__restrict__ chunk_hist = nullptr)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int B = m.B, NC = 1 << m.lg_nc;
    int32_t *wcnt = lds + m.wcnt, *hist = lds + m.hist, *base = lds + m.base;

    // CHUNKED: lane k = j*B + b sums bin b of the chunks j, j + J, j + 2J, ... before the
    // tile's chunk (J = kTileThreads / B chunks side by side); the first pass is loaded before
    // the LDS clear. With B > kTileThreads (E >= 1023) a few lanes take a second bin after it.
    int csum = 0;
    const int nchunk = tile_begin / kLayoutChunk;
    const int J = B <= kTileThreads ? kTileThreads / B : 1;
    if constexpr (CHUNKED) {
        if (tid < J * B) {
            const int b = tid % B;
#pragma unroll 4
            for (int cc = tid / B; cc < nchunk; cc += J) csum += chunk_hist[(size_t)cc * B + b];
        }
    }

    // zero the per-wavefront counts and the histogram copies (adjacent, 16-byte aligned)
    {
        int4 *z = reinterpret_cast<int4 *>(lds + m.wcnt);
        const int n4 = (m.base - m.wcnt) / 4;
        for (int k = tid; k < n4; k += kTileThreads) z[k] = int4{0, 0, 0, 0};
    }
    __syncthreads();

    // 1. earlier tiles into the replicated histogram. Vectors past the prefix were clamped to
    //    its last one; their counts are skipped.
    const int copy = lane & (NC - 1);
    if constexpr (CHUNKED) {
        if (csum) atomicAdd(&hist[((tid % B) << m.lg_nc) + copy], csum);
        for (int k = tid + kTileThreads; k < J * B; k += kTileThreads) {
            int sum = 0;
            for (int cc = k / B; cc < nchunk; cc += J) sum += chunk_hist[(size_t)cc * B + k % B];
            if (sum) atomicAdd(&hist[((k % B) << m.lg_nc) + copy], sum);
        }
        const int nv = tile_begin / 4 - nchunk * (kLayoutChunk / 4);
        if (tid < nv) {
            const int e4[4] = {ids.v[0].x, ids.v[0].y, ids.v[0].z, ids.v[0].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) atomicAdd(&hist[(layout_bin(e4[c], E) << m.lg_nc) + copy], 1);
        }
    } else if constexpr (ALL) {
        // every other vector: the earlier ones into hist, the later ones into the second
        // histogram, then the last TK % 4 ids if they come after the tile
        const OtherVecs ov = other_vecs(TK, tile_begin, P);
        const int nvec = ov.count();
        int32_t *hist2 = lds + m.hist2;
        if (nvec > 0) {
#pragma unroll
            for (int u = 0; u < kPrefixVec; ++u) {
                const int q = tid + u * kTileThreads;
                int32_t *h = q < ov.nb ? hist : hist2;
                const int e4[4] = {ids.v[u].x, ids.v[u].y, ids.v[u].z, ids.v[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (q < nvec) atomicAdd(&h[(layout_bin(e4[c], E) << m.lg_nc) + copy], 1);
            }
            // more than kPrefixVec*4096 other ids: the rest in further batches
            const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
            for (int q0 = tid + kPrefixVec * kTileThreads; q0 < nvec;
                 q0 += kPrefixVec * kTileThreads) {
                int4 v[kPrefixVec];
#pragma unroll
                for (int u = 0; u < kPrefixVec; ++u) {
                    const int q = q0 + u * kTileThreads;
                    v[u] = idx4[ov.phys(q < nvec ? q : nvec - 1)];
                }
#pragma unroll
                for (int u = 0; u < kPrefixVec; ++u) {
                    const int q = q0 + u * kTileThreads;
                    int32_t *h = q < ov.nb ? hist : hist2;
                    const int e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (q < nvec) atomicAdd(&h[(layout_bin(e4[c], E) << m.lg_nc) + copy], 1);
                }
            }
        }
        if (tid < TK % 4 && (TK / 4) * 4 + tid >= tile_begin + P)
            atomicAdd(&hist2[(layout_bin(ids.tail, E) << m.lg_nc) + copy], 1);
    } else {
        const int nvec = tile_begin / 4;
        if (nvec > 0) {
#pragma unroll
            for (int u = 0; u < kPrefixVec; ++u) {
                const bool ok = tid + u * kTileThreads < nvec;
                const int e4[4] = {ids.v[u].x, ids.v[u].y, ids.v[u].z, ids.v[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (ok) atomicAdd(&hist[(layout_bin(e4[c], E) << m.lg_nc) + copy], 1);
            }
            // prefixes longer than kPrefixVec*4096 ids: the rest in further batches
            const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
            for (int q0 = tid + kPrefixVec * kTileThreads; q0 < nvec;
                 q0 += kPrefixVec * kTileThreads) {
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
                        if (ok) atomicAdd(&hist[(layout_bin(e4[c], E) << m.lg_nc) + copy], 1);
                }
            }
        }
    }

    // 2. ranks of the routed lanes inside the wavefront by bit-sliced ballot matching
    const int p = tile_begin + tid;
    const bool in = tid < P && p < TK;
    const int own = ids.own;
    const bool routed = in && (unsigned)own < (unsigned)E;
    if (last) {                     // this tile's pairs in the two non-expert bins, for the stats
        const int unrouted = __popcll(__ballot(in && own == -1));
        const int invalid = __popcll(__ballot(in && own != -1 && !routed));
        if (lane == 0 && unrouted) atomicAdd(&hist[(E + 1) << m.lg_nc], unrouted);
        if (lane == 0 && invalid) atomicAdd(&hist[E << m.lg_nc], invalid);
    }
    uint64_t same = __ballot(routed);
    for (int k = 0; k < nbits; ++k) {
        const bool bit = (own >> k) & 1;
        const uint64_t mk = __ballot(bit);
        same &= bit ? mk : ~mk;
    }
    const int rank = count_below(same);
    if (routed && rank == 0) wcnt[wave * B + own] = __popcll(same);
    __syncthreads();

    // 3. per expert, one DPP row of 16 lanes: fold the NC copies (NC/16 words per lane) into
    //    the earlier-tile count b0, then the exclusive scan of the 16 wavefront counts from b0
    //    (the two non-expert bins are folded by layout_finish, which alone needs them)
    for (int k = tid; k < E * kTileWaves; k += kTileThreads) {
        const int e = k / kTileWaves, w = k % kTileWaves;
        const int32_t *h = hist + (e << m.lg_nc) + (w << (m.lg_nc - 4));
        int part;
        if (m.lg_nc == 6) {
            const int4 q = *reinterpret_cast<const int4 *>(h);
            part = (q.x + q.y) + (q.z + q.w);
        } else if (m.lg_nc == 5) {
            const int2 q = *reinterpret_cast<const int2 *>(h);
            part = q.x + q.y;
        } else {
            part = h[0];
        }
        const int b0 = row16_total(part);
        const int c = wcnt[w * B + e];
        const int incl = row16_inclusive_sum(c);
        wcnt[w * B + e] = b0 + incl - c;
        if (w == kTileWaves - 1) base[e] = b0 + incl;
        if constexpr (ALL) {            // the later tiles' count: the expert's total
            const int32_t *h2 = lds + m.hist2 + (e << m.lg_nc) + (w << (m.lg_nc - 4));
            int part2;
            if (m.lg_nc == 6) {
                const int4 q = *reinterpret_cast<const int4 *>(h2);
                part2 = (q.x + q.y) + (q.z + q.w);
            } else if (m.lg_nc == 5) {
                const int2 q = *reinterpret_cast<const int2 *>(h2);
                part2 = q.x + q.y;
            } else {
                part2 = h2[0];
            }
            const int a0 = row16_total(part2);
            if (w == kTileWaves - 1) lds[m.tot + e] = b0 + incl + a0;
        }
    }
    __syncthreads();
    if constexpr (ALL) {
        // packed offsets: exclusive scan of align_up(min(total, C), align) in expert order
        int32_t *wsum = lds + m.wsum;
        const int cnt = tid < E ? min(lds[m.tot + tid], C) : 0;   // E <= kTileThreads
        const int prow = (cnt + align - 1) / align * align;
        const int incl = wave_inclusive_sum(prow);
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int wb = 0;
        for (int w = 0; w < wave; ++w) wb += wsum[w];
        if (tid < E) lds[m.off + tid] = wb + incl - prow;
        __syncthreads();
    }
    if (in) {
        int s = -1;
        if (routed) {
            const int pos = wcnt[wave * B + own] + rank;
            s = pos < C ? pos : -1;
        }
        slot[p] = s;
        if constexpr (ALL) {
            const int r = s >= 0 ? lds[m.off + own] + s : -1;
            rows[tid] = (unsigned)r < (unsigned)rows_cap ? r : -1;
        } else {
            if (rows) rows[tid] = s >= 0 ? own * C + s : -1;
        }
    }
    __syncthreads();
}

// Step 4, by the workgroup of the last tile after layout_tile: base[e] is the total of expert
// e; the histogram copies of bins E and E+1 hold the invalid and unrouted totals. PACKED scans
// the counts rounded up to o.align instead (and writes the total rows to o.offset_end); the
// plain form is kept apart so the fused kernels carry none of that code.
template <bool PACKED>
__device__ __forceinline__ void layout_finish(int TK, int E, int C, int R, int32_t *lds,
                                              const LayoutLdsMap &m, const LayoutOut &o)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int32_t *base = lds + m.base, *hist = lds + m.hist;
    int32_t *scan = lds + m.scan, *wsum = lds + m.wsum, *ksum = lds + m.ksum;
    const int cnt = tid < E ? min(base[tid], C) : 0;     // E <= kTileThreads
    // rows the expert takes: its count, rounded up to a multiple of the alignment if packed
    const int rows = PACKED ? (cnt + o.align - 1) / o.align * o.align : cnt;
    const int incl = wave_inclusive_sum(rows);
    const int kept_incl = PACKED ? wave_inclusive_sum(cnt) : incl;
    if (lane == kWave - 1) {
        wsum[wave] = incl;
        if (PACKED) ksum[wave] = kept_incl;
    }
    if (wave == 0) {          // invalid (bin E) and unrouted (bin E+1) totals: sum of the copies
        const int NC = 1 << m.lg_nc;
        const int inv = wave_inclusive_sum(lane < NC ? hist[(E << m.lg_nc) + lane] : 0);
        const int unr = wave_inclusive_sum(lane < NC ? hist[((E + 1) << m.lg_nc) + lane] : 0);
        if (lane == kWave - 1) {
            wsum[kTileWaves] = inv;
            wsum[kTileWaves + 1] = unr;
        }
    }
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    const int excl = wbase + incl - rows;
    if (tid < E) {
        o.count[tid] = cnt;
        o.offset[tid] = excl;
        scan[tid] = excl;
    }
    if (tid == E - 1) {
        scan[E] = excl + rows;                           // total rows (= kept if not packed)
        if (PACKED) *o.offset_end = excl + rows;
    }
    __syncthreads();
    const int EL = E / R;
    for (int r = tid; r < R; r += kTileThreads) {
        const int lo = scan[r * EL], hi = scan[(r + 1) * EL];
        if (o.rank_count) o.rank_count[r] = hi - lo;
        if (o.rank_offset) o.rank_offset[r] = lo;
    }
    if (tid == 0) {
        int kept = scan[E];
        if (PACKED) {
            kept = 0;
            for (int w = 0; w < kTileWaves; ++w) kept += ksum[w];
        }
        const int invalid = wsum[kTileWaves], unrouted = wsum[kTileWaves + 1];
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
