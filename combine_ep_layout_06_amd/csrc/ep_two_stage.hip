// Two-stage, rank-deduplicated dispatch and combine on gfx950.
//
// The pages' kernel chain moves a token to each virtual rank once (dispatch_impl) and lets the
// rank expand it into its experts' rows (dispatch_copy_epilogue); on the way back each rank
// reduces per token (combine_impl) before the top-k reduction on the token's side
// (combine_reduce_epilogue) (afdEP-comm validation record, kernel_timelines). The staging
// buffer stage[R][T][row] stands in for the transport; every definition is in ep.h.
//
// Kernels:
//  * rank_layout: one workgroup of 1024 lanes per 1024 tokens, one token per lane. A token's
//    rank set is a 64-bit mask (R <= 64) built from its K ids (16-byte vectors for K = 4, 8,
//    12, 16; the ids of several earlier tokens and the lane's own are all in flight together).
//    Earlier tiles are counted per rank with one ballot per rank per 64 tokens, summed with
//    scalar adds (LDS atomics on the set bits measured no faster, and slower for few ranks);
//    the tile's own tokens are ranked with a ballot + v_mbcnt per rank and a 16-lane DPP scan
//    over the wavefronts, like the expert layout.
//  * dispatch_ranks (bf16 / FP8): the dispatch work items of ep_dispatch_item.h with the R
//    staging rows of a token in place of its K expert rows.
//  * rank_layout_dispatch (bf16 / FP8): the two above in one launch. A workgroup of 1024 lanes
//    takes a tile of at most 64 tokens, counts the earlier tokens per rank as rank_layout does
//    (every lane, 64 tokens per wavefront step), ranks its own tokens in one wavefront (ballot
//    + v_mbcnt per rank) and copies them at once, so the layout of later tiles overlaps the
//    copies of earlier ones.
//  * expand (bf16 / FP8): per kept pair, the staged row of the pair's rank is copied to the
//    pair's expert row; all of a token's row loads are issued before its stores (pairs of one
//    rank load the same row, which the second time comes from the cache).
//  * combine_ranks: a token's K expert rows are loaded once (straight-line, as in combine);
//    then for each rank, in order of its first pair, its pairs are folded in ascending j with
//    fmaf and the partial is rounded to bf16 and stored. K > 8 takes a sequential path.
//  * combine_reduce: the token's partial rows, listed in ascending rank in LDS, are gathered
//    and summed in that order in fp32, then rounded once.
#include "ep_dispatch_item.h"
#include "ep_internal.h"

#ifndef EP_TWO_STAGE_U
#define EP_TWO_STAGE_U 0        // 16-byte chunks per lane per item (0 = choose from the shape)
#endif

#ifndef EP_RANKS_FUSED_TT
#define EP_RANKS_FUSED_TT 0      // tokens per tile of the fused rank layout + stage 1
#endif
#ifndef EP_CR_NT_LOAD
#define EP_CR_NT_LOAD 1          // partial combine: non-temporal expert-row loads
#endif
#ifndef EP_CR_NT_STORE
#define EP_CR_NT_STORE 0         // partial combine: non-temporal partial-row stores
#endif
#ifndef EP_CR_U
#define EP_CR_U 0                // partial combine: chunks per lane (0 = as the other kernels)
#endif
#ifndef EP_EXPAND_NT_STORE
#define EP_EXPAND_NT_STORE 1     // expansion: non-temporal expert-row stores (see ep_fused.hip)
#endif
#ifndef EP_RED_CACHED_BYTES
#define EP_RED_CACHED_BYTES (64 << 20)  // final reduce: partial buffers up to this size are read
#endif                                  // through the caches, larger ones non-temporally
// Fused rank kernels: tile order over the XCDs (xcd_tile). At T = 4096 the FP8 one (R = 3,
// 16-token tiles) takes 12.7-13.0 us with ORDER = 1 against 13.4 us with the identity; the bf16
// one (R = 16) 23.7-23.9 us either way, 25.0 us with ORDER = 2.
#ifndef EP_RANKS_BF16_XCD_ORDER
#define EP_RANKS_BF16_XCD_ORDER 0
#endif
#ifndef EP_RANKS_FP8_XCD_ORDER
#define EP_RANKS_FP8_XCD_ORDER 1
#endif
// Fused rank kernels: the layout's id loads go out first and the first item's row loads
// after them with no branch, so the layout waits for the ids alone while the rows are in flight
// (a wavefront's loads complete in order; with the rows first, or under a branch, the compiler
// waits for all of them). From per-workgroup stamps, the layout phase of the FP8 kernel had
// taken 4.0-4.9 us, mostly the row loads, against a 3.7 us copy phase. At T = 4096: FP8 (R = 3)
// 12.4-12.5 against 12.8 us, bf16 (R = 16) 23.4-23.5 against 23.8 us. The one-stage fused
// kernels measured slower in the same arrangement (bf16 26.2-26.6 against 26.0 us with the id
// loads also branch-free, FP8 20.9 against 18.1 us) and keep theirs.
#ifndef EP_RANKS_IDS_FIRST
#define EP_RANKS_IDS_FIRST 1
#endif
#ifndef EP_RANKS_FP8_U
#define EP_RANKS_FP8_U 0         // fused FP8 rank kernel: 16-channel pieces per lane (0 = auto)
#endif

namespace ep {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStage = 256;          // staged entries per token group (tpb*K, tpb*R <= kStage)
constexpr int kRankTile = 1024;      // rank layout: tokens per workgroup, one per lane
constexpr int kRankWaves = kRankTile / kWave;
constexpr int kRankBatch = 4;        // earlier tokens per lane whose ids are loaded together

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------------------------------
// rank layout
// ------------------------------------------------------------------------------------------

// The rank of an expert, e / EL, without a division: e * M >> 20 with M = floor(2^20 / EL) + 1
// (rank_magic) is exact for 0 <= e < E <= EP_MAX_EXPERTS = 1024. (e M / 2^20 exceeds e / EL by
// less than e / 2^20, which is below 1 / EL since e EL < 2^20, so the floor is unchanged;
// EL = 1 gives e + (e >> 20) = e.) Both factors fit the 24-bit multiplier.
__host__ __device__ inline uint32_t rank_magic(int EL) { return (1u << 20) / (uint32_t)EL + 1u; }

// Bit of id e's rank if e is a valid expert (0 <= e < E), else 0. Branch-free: an invalid id's
// rank is masked before the shift.
__device__ __forceinline__ uint64_t rank_bit(int e, int E, uint32_t magic)
{
    const unsigned r = __umul24((unsigned)e, magic) >> 20;
    return (unsigned)e < (unsigned)E ? (1ull << (r & 63u)) : 0ull;
}

__device__ __forceinline__ uint64_t ranks_of(const int4 *v, int nv, int E, uint32_t magic)
{
    uint64_t m = 0;
    for (int j = 0; j < nv; ++j)
        m |= rank_bit(v[j].x, E, magic) | rank_bit(v[j].y, E, magic) |
             rank_bit(v[j].z, E, magic) | rank_bit(v[j].w, E, magic);
    return m;
}

// Rank set of token t for any K, one id at a time.
__device__ __forceinline__ uint64_t token_ranks_any(const int32_t *__restrict__ idx, int t, int K,
                                                    int E, uint32_t magic)
{
    uint64_t m = 0;
    for (int j = 0; j < K; ++j) m |= rank_bit(idx[(size_t)t * K + j], E, magic);
    return m;
}

// The 4 bits of n (n < 16) moved to the lowest bit of each byte (bit i -> bit 8i): n times
// 1 + 2^7 + 2^14 + 2^21 places four copies of n that do not overlap, the mask keeps one bit
// of each.
__device__ __forceinline__ uint32_t spread4(uint32_t n) { return __umul24(n, 0x204081u) & 0x01010101u; }

// Sum over the 64 lanes, in every lane.
__device__ __forceinline__ int wave_total(int v)
{
    return __builtin_amdgcn_readlane(wave_inclusive_sum(v), kWave - 1);
}

// Largest T for which the packed counts of rank_prefix_wave cannot overflow: a lane sees at
// most kRankBatch earlier tokens per pass of kRankBatch * kRankTile tokens, and its 8-bit
// fields hold up to 255, so 63 passes.
constexpr int kPackedRankMaxT = 63 * kRankBatch * kRankTile;

// One pass of rank_prefix_wave's loads: this lane's tokens q0 + (b0 + b) * kRankTile,
// b < kRankBatch, as KV 16-byte id vectors each; a batch is loaded only if some token of the
// wavefront in it lies before t0 (wavefront-uniform), the others read as -1 (no expert).
template <int KV>
__device__ __forceinline__ void rank_batch_loads(const int32_t *__restrict__ idx, int b0, int t0,
                                                 int K, int4 (&v)[kRankBatch][KV])
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int q0 = wave * kWave + lane;
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
#pragma unroll
        for (int j = 0; j < KV; ++j) v[b][j] = int4{-1, -1, -1, -1};
        if ((b0 + b) * kRankTile + wave * kWave < t0) {        // wavefront-uniform
            const int q = min(q0 + (b0 + b) * kRankTile, t0 - 1);
#pragma unroll
            for (int j = 0; j < KV; ++j)
                v[b][j] = reinterpret_cast<const int4 *>(idx + (size_t)q * K)[j];
        }
    }
}

// Per-rank counts of the tokens [0, t0) in this wavefront's share (tokens wave*64 + lane +
// b*kRankTile): kRankBatch tokens per lane are loaded together (16-byte id vectors when
// KV > 0). Lane r returns rank r's total.
// RQ > 0 (R <= 4 RQ and T <= kPackedRankMaxT): each lane counts its own tokens per rank in
// packed 8-bit fields, one 24-bit multiply and a mask per 4 ranks and token (spread4); one
// wave sum per rank at the end. RQ = 0: per rank and batch one ballot and a scalar popcount
// (any R <= 64).
// PRE (KV > 0): the first pass's vectors were loaded beforehand (rank_batch_loads with b0 = 0)
// and are passed in `first`.
template <int KV, int RQ, bool PRE = false>
__device__ __forceinline__ int rank_prefix_wave(const int32_t *__restrict__ idx, int t0, int K,
                                                int E, uint32_t magic, int R,
                                                const int4 (*first)[KV > 0 ? KV : 1] = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int q0 = wave * kWave + lane;
    int acc = 0;
    // RQ > 0: byte k of cnt[q] counts the lane's tokens sent to rank 4q + k
    uint32_t cnt[RQ > 0 ? RQ : 1];
#pragma unroll
    for (int q = 0; q < (RQ > 0 ? RQ : 1); ++q) cnt[q] = 0;
    for (int b0 = 0; b0 * kRankTile + wave * kWave < t0; b0 += kRankBatch) {
        uint64_t m[kRankBatch];
        if constexpr (KV > 0) {
            int4 v[kRankBatch][KV];
            if (PRE && b0 == 0) {
#pragma unroll
                for (int b = 0; b < kRankBatch; ++b)
#pragma unroll
                    for (int j = 0; j < KV; ++j) v[b][j] = first[b][j];
            } else {
                rank_batch_loads<KV>(idx, b0, t0, K, v);
            }
#pragma unroll
            for (int b = 0; b < kRankBatch; ++b)
                m[b] = q0 + (b0 + b) * kRankTile < t0 ? ranks_of(v[b], KV, E, magic) : 0;
        } else {
#pragma unroll
            for (int b = 0; b < kRankBatch; ++b) {
                const int q = q0 + (b0 + b) * kRankTile;
                m[b] = q < t0 ? token_ranks_any(idx, q, K, E, magic) : 0;
            }
        }
        if constexpr (RQ > 0) {
            // tokens past t0 have an empty mask, so every batch can be counted
#pragma unroll
            for (int q = 0; q < RQ; ++q)
#pragma unroll
                for (int b = 0; b < kRankBatch; ++b)
                    cnt[q] += spread4((uint32_t)(m[b] >> (4 * q)) & 0xFu);
        } else {
            // batches holding any of this wavefront's earlier tokens
            const int nb = min(kRankBatch, ceil_div(t0 - b0 * kRankTile - wave * kWave, kRankTile));
            for (int r = 0; r < R; ++r) {
                int c = 0;
#pragma unroll
                for (int b = 0; b < kRankBatch; ++b)
                    if (b < nb) c += __popcll(__ballot(((m[b] >> r) & 1u) != 0));
                acc = lane == r ? acc + c : acc;
            }
        }
    }
    if constexpr (RQ > 0) {
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (4 * q + k >= R) continue;       // wavefront-uniform
                const int tot = wave_total((int)((cnt[q] >> (8 * k)) & 0xFFu));
                acc = lane == 4 * q + k ? tot : acc;
            }
        }
    }
    return acc;
}

// KV > 0: K = 4*KV ids per token, read as KV 16-byte vectors; KV = 0: any K. RQ: the counting
// form of rank_prefix_wave.
template <int KV, int RQ>
__global__ __launch_bounds__(kRankTile) void rank_layout_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int R, int32_t *__restrict__ rank_slot,
    int32_t *__restrict__ rank_tokens)
{
    __shared__ int32_t wcnt[kRankWaves][EP_MAX_RANKS];   // counts, then per-wavefront bases
    __shared__ int32_t base[EP_MAX_RANKS];               // earlier-tile counts
    __shared__ int4 out16[kRankTile][4];                 // 16 ranks of each token's output row
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t magic = rank_magic(E / R);
    const int t0 = blockIdx.x * kRankTile;
    const int t = t0 + tid;

    // 1. the lane's own token and the earlier tiles (rank_prefix_wave): the own ids are loaded
    //    first and used after the prefix count, so all loads are in flight together
    uint64_t own = 0;
    int4 vo[KV > 0 ? KV : 1];
    if constexpr (KV > 0) {
        if (t < T) {
#pragma unroll
            for (int j = 0; j < KV; ++j) vo[j] = reinterpret_cast<const int4 *>(idx + (size_t)t * K)[j];
        }
    }
    const int acc = rank_prefix_wave<KV, RQ>(idx, t0, K, E, magic, R);
    if constexpr (KV > 0) own = t < T ? ranks_of(vo, KV, E, magic) : 0;
    else own = t < T ? token_ranks_any(idx, t, K, E, magic) : 0;
    if (lane < R) wcnt[wave][lane] = acc;
    __syncthreads();
    if (tid < R) {
        int sum = 0;
        for (int w = 0; w < kRankWaves; ++w) sum += wcnt[w][tid];
        base[tid] = sum;
    }
    __syncthreads();

    // 2. this tile: per wavefront, how many of its tokens go to each rank
    int own_cnt = 0;
    for (int r = 0; r < R; ++r) {
        const int c = __popcll(__ballot((own >> r) & 1));
        own_cnt = lane == r ? c : own_cnt;
    }
    if (lane < R) wcnt[wave][lane] = own_cnt;
    __syncthreads();

    // 3. per rank, the 16 wavefront counts sit in one DPP row: exclusive scan from the
    //    earlier-tile count gives each wavefront's base; the last tile writes the totals
    if (tid < R * kRankWaves) {
        const int r = tid / kRankWaves, w = tid % kRankWaves;
        const int c = wcnt[w][r];
        const int incl = row16_inclusive_sum(c);
        const int b0 = base[r];
        wcnt[w][r] = b0 + incl - c;
        if (w == kRankWaves - 1 && blockIdx.x == gridDim.x - 1) rank_tokens[r] = b0 + incl;
    }
    __syncthreads();

    // 4. the tile's rows of rank_slot, 16 ranks at a time through LDS so that consecutive lanes
    //    store consecutive 16-byte pieces (R % 4 == 0; otherwise one value per store)
    for (int r0 = 0; r0 < R; r0 += 16) {
        int v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int r = r0 + q;
            const bool sent = r < R && ((own >> r) & 1);
            const int pos = wcnt[wave][r < R ? r : 0] + count_below(__ballot(sent));
            v[q] = sent ? pos : -1;
        }
        if ((R & 3) != 0) {
            if (t < T)
                for (int q = 0; q < 16 && r0 + q < R; ++q) rank_slot[(size_t)t * R + r0 + q] = v[q];
            continue;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) out16[tid][q] = int4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        __syncthreads();
        const int nq = min(16, R - r0) / 4;               // 16-byte pieces per token in this pass
        for (int k = tid; k < kRankTile * nq; k += kRankTile) {
            const int tl = k / nq, q = k % nq;
            if (t0 + tl < T)
                *reinterpret_cast<int4 *>(rank_slot + (size_t)(t0 + tl) * R + r0 + 4 * q) =
                    out16[tl][q];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// dispatch, stage 1: one staging row per (token, rank)
// ------------------------------------------------------------------------------------------

// rows[tl*R + r] = r*T + rank_slot[t0 + tl][r], or -1 (not sent, or out of range)
__device__ __forceinline__ void stage_rank_rows(int32_t *rows, const int32_t *__restrict__ rank_slot,
                                                int t0, int nt, int R, int T)
{
    for (int k = threadIdx.x; k < nt * R; k += kThreads) {
        const int p = rank_slot[(size_t)t0 * R + k];
        rows[k] = (unsigned)p < (unsigned)T ? (k % R) * T + p : -1;
    }
}

template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kThreads) void dispatch_ranks_bf16_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ rank_slot, u32x4 *__restrict__ stage,
    int T, int H8, int R, int tpb, int nseg)
{
    __shared__ int32_t rows[kStage];
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int ntg = ceil_div(T, tpb);
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb, nt = min(tpb, T - t0);
        __syncthreads();
        stage_rank_rows(rows, rank_slot, t0, nt, R, T);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg;
            dispatch_item_bf16<KG, U, MULTI>(x, stage, rows, t0 + tl, tl, item - tl * nseg, H8, R);
        }
    }
}

template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kThreads) void dispatch_ranks_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ rank_slot,
    u32x4 *__restrict__ stage_q, float *__restrict__ stage_scale, int T, int H, int R, int tpb,
    int nseg)
{
    __shared__ int32_t rows[kStage];
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int ntg = ceil_div(T, tpb);
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb, nt = min(tpb, T - t0);
        __syncthreads();
        stage_rank_rows(rows, rank_slot, t0, nt, R, T);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg;
            dispatch_item_fp8<KG, U, MULTI>(x, stage_q, stage_scale, rows, t0 + tl, tl,
                                            item - tl * nseg, H, R);
        }
    }
}

// ------------------------------------------------------------------------------------------
// rank layout and stage 1 fused: each workgroup ranks a tile of at most 64 tokens against all
// earlier tokens, then copies (or quantises and copies) the tile's rows to their staging rows
// ------------------------------------------------------------------------------------------

// The global loads of rank_tile for KV > 0, issued before the workgroup's other loads so that
// the layout waits only for them (a wavefront's loads complete in order): wavefront 0's ids of
// the tile's own tokens (lane tl: token t0 + tl) and the first pass of earlier tokens.
template <int KV>
struct RankTileIds {
    int4 own[KV > 0 ? KV : 1];
    int4 v[kRankBatch][KV > 0 ? KV : 1];
};

template <int KV>
__device__ __forceinline__ RankTileIds<KV> rank_tile_loads(const int32_t *__restrict__ idx,
                                                           int t0, int nt, int K)
{
    RankTileIds<KV> ids;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < KV; ++j) ids.own[j] = int4{-1, -1, -1, -1};
    if (wave == 0 && lane < nt) {
#pragma unroll
        for (int j = 0; j < KV; ++j)
            ids.own[j] = reinterpret_cast<const int4 *>(idx + (size_t)(t0 + lane) * K)[j];
    }
    rank_batch_loads<KV>(idx, 0, t0, K, ids.v);
    return ids;
}

// Rank layout of the tile [t0, t0 + nt), nt <= kWave, in a workgroup of kRankTile lanes:
// rank_slot rows of the tile (coalesced, through LDS), rows[tl*R + r] = r*T + slot or -1 in
// LDS for the copies, and rank_tokens in the last workgroup. Ends with a barrier. PRE (KV > 0):
// the ids were loaded by rank_tile_loads and are passed in `pre`.
template <int KV, int RQ, bool PRE = false>
__device__ __forceinline__ void rank_tile(const int32_t *__restrict__ idx, int t0, int nt, int T,
                                          int K, int E, int R, bool last,
                                          int32_t *__restrict__ rank_slot,
                                          int32_t *__restrict__ rank_tokens, int32_t *rows,
                                          int32_t *slots, int32_t (*wcnt)[EP_MAX_RANKS],
                                          const RankTileIds<KV> *pre = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t magic = rank_magic(E / R);
    uint64_t own = 0;                  // wavefront 0, lane tl: the tile's token tl
    if (wave == 0 && lane < nt) {
        const int t = t0 + lane;
        if constexpr (KV > 0) {
            int4 v[KV];
#pragma unroll
            for (int j = 0; j < KV; ++j)
                v[j] = PRE ? pre->own[j] : reinterpret_cast<const int4 *>(idx + (size_t)t * K)[j];
            own = ranks_of(v, KV, E, magic);
        } else {
            own = token_ranks_any(idx, t, K, E, magic);
        }
    }
    const int acc = rank_prefix_wave<KV, RQ, PRE>(idx, t0, K, E, magic, R, PRE ? pre->v : nullptr);
    if (lane < R) wcnt[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        int base = 0;                  // lane r: tokens before t0 sent to rank r
        if (lane < R)
            for (int w = 0; w < kRankWaves; ++w) base += wcnt[w][lane];
        for (int r = 0; r < R; ++r) {
            const bool sent = (own >> r) & 1u;
            const uint64_t bal = __ballot(sent);
            const int b = __builtin_amdgcn_readlane(base, r);
            const int pos = b + count_below(bal);
            if (lane < nt) {
                slots[lane * R + r] = sent ? pos : -1;
                rows[lane * R + r] = sent ? r * T + pos : -1;
            }
            if (last && lane == 0) rank_tokens[r] = b + (int)__popcll(bal);
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < nt * R; k += kRankTile) rank_slot[(size_t)t0 * R + k] = slots[k];
}

template <int KV, int RQ, int KG, int U, bool MULTI>
__global__ __launch_bounds__(kRankTile, 8) void rank_layout_dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx, int32_t *__restrict__ rank_slot,
    int32_t *__restrict__ rank_tokens, u32x4 *__restrict__ stage, int T, int H8, int K, int E,
    int R, int TT, int nseg)
{
    __shared__ int32_t wcnt[kRankWaves][EP_MAX_RANKS];
    __shared__ int32_t rows[kRankTile];
    __shared__ int32_t slots[kRankTile];
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int tile = xcd_tile<EP_RANKS_BF16_XCD_ORDER>();
    const int t0 = tile * TT, nt = min(TT, T - t0);
    const int nitems = nt * nseg;
    // the ids first, then the first item's row loads (they need no slot), so that the layout
    // waits for the ids only while the rows are in flight
    constexpr bool kPre = KV > 0 && RQ > 0 && EP_RANKS_IDS_FIRST;
    RankTileIds<KV> ids;
    if constexpr (kPre) ids = rank_tile_loads<KV>(idx, t0, nt, K);
    // (issued by every wavefront, those without an item repeating the last one, so that the
    // number of loads behind the ids is the same on every path and the wait for the ids is exact)
    const int fi = min(wave, nitems - 1);
    const RowPiece<U> first = load_item_bf16<U>(x, t0 + fi / nseg, fi % nseg, H8);
    rank_tile<KV, RQ, kPre>(idx, t0, nt, T, K, E, R, tile == (int)gridDim.x - 1, rank_slot,
                            rank_tokens, rows, slots, wcnt, &ids);
    if (wave < nitems)
        store_item_bf16<KG, U, MULTI>(first, stage, rows, wave / nseg, wave % nseg, H8, R);
    for (int item = wave + kRankWaves; item < nitems; item += kRankWaves) {
        const int tl = item / nseg;
        dispatch_item_bf16<KG, U, MULTI>(x, stage, rows, t0 + tl, tl, item - tl * nseg, H8, R);
    }
}

#ifndef EP_RANKS_FP8_WAVES
#define EP_RANKS_FP8_WAVES 4     // wavefronts per SIMD the fused FP8 rank kernel is built for
#endif

template <int KV, int RQ, int KG, int U, bool MULTI>
__global__ __launch_bounds__(kRankTile, EP_RANKS_FP8_WAVES) void rank_layout_dispatch_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx, int32_t *__restrict__ rank_slot,
    int32_t *__restrict__ rank_tokens, u32x4 *__restrict__ stage_q,
    float *__restrict__ stage_scale, int T, int H, int K, int E, int R, int TT, int nseg)
{
    __shared__ int32_t wcnt[kRankWaves][EP_MAX_RANKS];
    __shared__ int32_t rows[kRankTile];
    __shared__ int32_t slots[kRankTile];
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int tile = xcd_tile<EP_RANKS_FP8_XCD_ORDER>();
    const int t0 = tile * TT, nt = min(TT, T - t0);
    const int nitems = nt * nseg;
    // the ids first, then the first item's token row (it needs no slot; cast after the
    // layout), so that the layout waits for the ids only while the row is in flight
    constexpr bool kPre = KV > 0 && RQ > 0 && EP_RANKS_IDS_FIRST;
    RankTileIds<KV> ids;
    if constexpr (kPre) ids = rank_tile_loads<KV>(idx, t0, nt, K);
    // (issued by every wavefront, those without an item repeating the last one, so that the
    // number of loads behind the ids is the same on every path and the wait for the ids is exact)
    const int fi = min(wave, nitems - 1);
    const RawPieceFp8<U> first = load_item_fp8_nobranch<U>(x, t0 + fi / nseg, fi % nseg, H);
    rank_tile<KV, RQ, kPre>(idx, t0, nt, T, K, E, R, tile == (int)gridDim.x - 1, rank_slot,
                            rank_tokens, rows, slots, wcnt, &ids);
    if (wave < nitems)
        store_item_fp8<KG, U, MULTI>(cast_item_fp8<U>(zero_past_row<U>(first)), stage_q,
                                     stage_scale, rows, wave / nseg, wave % nseg, H, R);
    for (int item = wave + kRankWaves; item < nitems; item += kRankWaves) {
        const int tl = item / nseg;
        dispatch_item_fp8<KG, U, MULTI>(x, stage_q, stage_scale, rows, t0 + tl, tl,
                                        item - tl * nseg, H, R);
    }
}

// ------------------------------------------------------------------------------------------
// per-pair staging shared by the expansion and the partial combine
// ------------------------------------------------------------------------------------------

// For the pairs of tokens [t0, t0 + nt): the staging row of the pair's rank (src), its expert
// row if kept (dst), its rank, and its weight. A pair takes part only if its id is a valid
// expert whose rank row is known; dst additionally needs a slot below C. The group's
// rank_slot rows are read into LDS first (coalesced), next to the pairs' ids and slots.
struct PairLds {
    int32_t rs[kStage];      // rank_slot rows of the group's tokens
    int32_t src[kStage];
    int32_t dst[kStage];
    int32_t rnk[kStage];
    float w[kStage];
};

__device__ __forceinline__ void stage_pairs(PairLds &L, const int32_t *__restrict__ idx,
                                            const int32_t *__restrict__ slot,
                                            const int32_t *__restrict__ rank_slot,
                                            const float *__restrict__ w, int t0, int nt, int T,
                                            int E, int C, int K, int R)
{
    for (int k = threadIdx.x; k < nt * R; k += kThreads) L.rs[k] = rank_slot[(size_t)t0 * R + k];
    int e[2], s[2];
    float wk[2];
    const int EL = E / R;
    // pairs per thread: nt*K <= kStage = 2*kThreads... loads first, then the LDS reads
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int k = threadIdx.x + u * kThreads;
        const bool in = k < nt * K;
        const size_t i = (size_t)t0 * K + (in ? k : 0);
        e[u] = in ? idx[i] : -1;
        s[u] = in ? slot[i] : -1;
        wk[u] = (in && w) ? w[i] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int k = threadIdx.x + u * kThreads;
        if (k >= nt * K) continue;
        const bool valid = (unsigned)e[u] < (unsigned)E;
        const int r = valid ? e[u] / EL : 0;
        const int p = valid ? L.rs[(k / K) * R + r] : -1;
        const bool ok = valid && (unsigned)p < (unsigned)T;
        L.rnk[k] = ok ? r : -1;
        L.src[k] = ok ? r * T + p : -1;
        L.dst[k] = ok && (unsigned)s[u] < (unsigned)C ? e[u] * C + s[u] : -1;
        L.w[k] = wk[u];
    }
}

// ------------------------------------------------------------------------------------------
// dispatch, stage 2: the rank's own expansion into its experts' rows
// ------------------------------------------------------------------------------------------

template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kThreads) void expand_bf16_kernel(
    const u32x4 *__restrict__ stage, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot, const int32_t *__restrict__ rank_slot,
    u32x4 *__restrict__ recv, int T, int H8, int E, int C, int K, int R, int tpb, int nseg)
{
    __shared__ PairLds L;
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int ntg = ceil_div(T, tpb);
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb, nt = min(tpb, T - t0);
        __syncthreads();
        stage_pairs(L, idx, slot, rank_slot, nullptr, t0, nt, T, E, C, K, R);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg, seg = item - tl * nseg;
            int cidx[U];
            bool cok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (seg * U + u) * kWave + lane;
                cok[u] = c < H8;
                cidx[u] = cok[u] ? c : H8 - 1;
            }
            const int npg = MULTI ? ceil_div(K, KG) : 1;
            for (int pg = 0; pg < npg; ++pg) {
                int d[KG];
                u32x4 v[KG][U];
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const int j = pg * KG + g;
                    const int k = tl * K + (j < K ? j : K - 1);
                    const int sr = wave_uniform(L.src[k]);
                    d[g] = j < K ? wave_uniform(L.dst[k]) : -1;
                    const u32x4 *src = stage + (size_t)(sr >= 0 ? sr : 0) * H8;
#pragma unroll
                    for (int u = 0; u < U; ++u) v[g][u] = src[cidx[u]];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    if (d[g] < 0) continue;
                    u32x4 *dst = recv + (size_t)d[g] * H8;
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (cok[u]) store16<EP_EXPAND_NT_STORE>(dst + cidx[u], v[g][u]);
                }
            }
        }
    }
}

// FP8: a lane owns 16 codes (one 16-byte chunk) of a 1024-channel segment; the first lane of
// each 8-lane group (one 128-channel block) also carries the block's scale.
template <int KG, bool MULTI>
__global__ __launch_bounds__(kThreads) void expand_fp8_kernel(
    const u32x4 *__restrict__ stage_q, const float *__restrict__ stage_scale,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ slot,
    const int32_t *__restrict__ rank_slot, u32x4 *__restrict__ recv_q,
    float *__restrict__ recv_scale, int T, int H, int E, int C, int K, int R, int tpb, int nseg)
{
    __shared__ PairLds L;
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int H16 = H / 16, NB = H / 128;
    const int ntg = ceil_div(T, tpb);
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb, nt = min(tpb, T - t0);
        __syncthreads();
        stage_pairs(L, idx, slot, rank_slot, nullptr, t0, nt, T, E, C, K, R);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg, seg = item - tl * nseg;
            const int h0 = seg * (16 * kWave) + lane * 16;
            const bool act = h0 < H;
            const bool lead = act && (lane & 7) == 0;
            const int cq = act ? h0 / 16 : 0, cs = act ? h0 / 128 : 0;
            const int npg = MULTI ? ceil_div(K, KG) : 1;
            for (int pg = 0; pg < npg; ++pg) {
                int d[KG];
                u32x4 q[KG];
                float sc[KG];
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const int j = pg * KG + g;
                    const int k = tl * K + (j < K ? j : K - 1);
                    const int sr = wave_uniform(L.src[k]);
                    d[g] = j < K ? wave_uniform(L.dst[k]) : -1;
                    const size_t row = (size_t)(sr >= 0 ? sr : 0);
                    q[g] = stage_q[row * H16 + cq];
                    sc[g] = stage_scale[row * NB + cs];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    if (d[g] < 0) continue;
                    if (act) store16<EP_EXPAND_NT_STORE>(recv_q + (size_t)d[g] * H16 + cq, q[g]);
                    if (lead) recv_scale[(size_t)d[g] * NB + cs] = sc[g];
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// combine, stage 1: per-rank partials
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ void fold_row(float (&acc)[8], float wj, const u32x4 &v)
{
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        acc[2 * k] = __builtin_fmaf(wj, bf16_lo(wd[k]), acc[2 * k]);
        acc[2 * k + 1] = __builtin_fmaf(wj, bf16_hi(wd[k]), acc[2 * k + 1]);
    }
}

__device__ __forceinline__ u32x4 pack_bf16(const float (&acc)[8])
{
    u32x4 o;
    o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    return o;
}

// K <= KG <= 8: every row of the token loaded once, then one fold per rank.
template <int KG, int U>
__device__ __forceinline__ void combine_ranks_item(const PairLds &L, const u32x4 *__restrict__ y,
                                                   u32x4 *__restrict__ part, int tl, int seg,
                                                   int H8, int K)
{
    const int lane = threadIdx.x & (kWave - 1);
    int cidx[U];
    bool cok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (seg * U + u) * kWave + lane;
        cok[u] = c < H8;
        cidx[u] = cok[u] ? c : H8 - 1;
    }
    int rk[KG], pr[KG], yr[KG];
    float wj[KG];
    u32x4 v[KG][U];
#pragma unroll
    for (int g = 0; g < KG; ++g) {
        const int k = tl * K + (g < K ? g : K - 1);
        rk[g] = g < K ? wave_uniform(L.rnk[k]) : -1;
        pr[g] = wave_uniform(L.src[k]);        // the pair's rank row = its partial's row
        yr[g] = g < K ? wave_uniform(L.dst[k]) : -1;
        wj[g] = __int_as_float(wave_uniform(__float_as_int(L.w[k])));
        const u32x4 *src = y + (size_t)(yr[g] >= 0 ? yr[g] : 0) * H8;
#pragma unroll
        for (int u = 0; u < U; ++u) v[g][u] = load16<EP_CR_NT_LOAD>(src + cidx[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < KG; ++g) {
        if (rk[g] < 0) continue;
        bool first = true;
#pragma unroll
        for (int h = 0; h < g; ++h) first = first && rk[h] != rk[g];
        if (!first) continue;                  // this rank's partial was written at its first pair
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[u][c] = 0.0f;
#pragma unroll
        for (int g2 = g; g2 < KG; ++g2) {
            if (rk[g2] != rk[g] || yr[g2] < 0) continue;
#pragma unroll
            for (int u = 0; u < U; ++u) fold_row(acc[u], wj[g2], v[g2][u]);
        }
        u32x4 *dst = part + (size_t)pr[g] * H8;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (cok[u]) store16<EP_CR_NT_STORE>(dst + cidx[u], pack_bf16(acc[u]));
    }
}

// K > 8: pairs in j order; at the first pair of each rank, that rank's pairs are folded one
// row at a time.
__device__ __forceinline__ void combine_ranks_item_seq(const PairLds &L,
                                                       const u32x4 *__restrict__ y,
                                                       u32x4 *__restrict__ part, int tl, int seg,
                                                       int H8, int K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int c = seg * kWave + lane;
    const bool cok = c < H8;
    const int ci = cok ? c : H8 - 1;
    for (int g = 0; g < K; ++g) {
        const int rg = wave_uniform(L.rnk[tl * K + g]);
        if (rg < 0) continue;
        bool first = true;
        for (int h = 0; h < g && first; ++h) first = wave_uniform(L.rnk[tl * K + h]) != rg;
        if (!first) continue;
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int g2 = g; g2 < K; ++g2) {
            const int k = tl * K + g2;
            const int yr = wave_uniform(L.dst[k]);
            if (wave_uniform(L.rnk[k]) != rg || yr < 0) continue;
            const float wj = __int_as_float(wave_uniform(__float_as_int(L.w[k])));
            fold_row(acc, wj, load16<true>(y + (size_t)yr * H8 + ci));
        }
        if (cok) store16<true>(part + (size_t)wave_uniform(L.src[tl * K + g]) * H8 + ci,
                               pack_bf16(acc));
    }
}

template <int KG, int U, bool SEQ>
__global__ __launch_bounds__(kThreads) void combine_ranks_kernel(
    const u32x4 *__restrict__ y, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot, const int32_t *__restrict__ rank_slot,
    const float *__restrict__ w, u32x4 *__restrict__ part, int T, int H8, int E, int C, int K,
    int R, int tpb, int nseg)
{
    __shared__ PairLds L;
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int ntg = ceil_div(T, tpb);
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb, nt = min(tpb, T - t0);
        __syncthreads();
        stage_pairs(L, idx, slot, rank_slot, w, t0, nt, T, E, C, K, R);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg, seg = item - tl * nseg;
            if constexpr (SEQ) combine_ranks_item_seq(L, y, part, tl, seg, H8, K);
            else combine_ranks_item<KG, U>(L, y, part, tl, seg, H8, K);
        }
    }
}

// ------------------------------------------------------------------------------------------
// combine, stage 2: the token's partials summed in ascending rank
// ------------------------------------------------------------------------------------------

// A row of zeros that absent list entries read with weight -0: fmaf(-0, +0, acc) adds an exact
// -0 and leaves every acc as it is, and fmaf(1, v, acc) is exactly acc + v, so the fold needs no
// per-element select. Never written (zero-initialised at load); rows of up to kZeroChunks
// 16-byte chunks use it, longer ones keep the select.
constexpr int kZeroChunks = 4096;
__device__ u32x4 g_zero_row[kZeroChunks];

// NTL: the partial rows are loaded non-temporally (a partial buffer too large to stay in the
// last-level cache between the partial combine and this kernel).
template <int KG, int U, bool MULTI, bool ZROW, bool NTL>
__global__ __launch_bounds__(kThreads) void combine_reduce_kernel(
    const u32x4 *__restrict__ part, const int32_t *__restrict__ rank_slot,
    u32x4 *__restrict__ out, int T, int H8, int R, int Q, int tpb, int nseg)
{
    __shared__ int32_t rs[kStage];
    __shared__ int32_t plist[kStage];     // per token, its partial rows in ascending rank
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int ntg = ceil_div(T, tpb);
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb, nt = min(tpb, T - t0);
        __syncthreads();
        for (int k = threadIdx.x; k < nt * R; k += kThreads) rs[k] = rank_slot[(size_t)t0 * R + k];
        __syncthreads();
        // one wavefront per token: lane r holds rank r's slot (R <= 64); the ranks the token
        // reached take the first entries of its list in ascending rank (ballot position), the
        // rest of its Q entries are -1
        for (int tl = wave; tl < nt; tl += kWaves) {
            const int p = lane < R ? rs[tl * R + lane] : -1;
            const bool ok = lane < R && (unsigned)p < (unsigned)T;
            const uint64_t m = __ballot(ok);
            const int n = count_below(m);
            if (ok && n < Q) plist[tl * Q + n] = lane * T + p;
            if (lane >= (int)__popcll(m) && lane < Q) plist[tl * Q + lane] = -1;
        }
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg, seg = item - tl * nseg;
            int cidx[U];
            bool cok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (seg * U + u) * kWave + lane;
                cok[u] = c < H8;
                cidx[u] = cok[u] ? c : H8 - 1;
            }
            float acc[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[u][c] = 0.0f;
            const int first_row = wave_uniform(plist[tl * Q]);
            const int npg = MULTI ? ceil_div(Q, KG) : 1;
            for (int pg = 0; pg < npg; ++pg) {
                int pr[KG];
                float wg[KG];
                u32x4 v[KG][U];
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const int n = pg * KG + g;
                    pr[g] = n < Q ? wave_uniform(plist[tl * Q + n]) : -1;
                    const u32x4 *src;
                    if constexpr (ZROW) {
                        src = pr[g] >= 0 ? part + (size_t)pr[g] * H8 : g_zero_row;
                        wg[g] = pr[g] >= 0 ? 1.0f : -0.0f;
                    } else {
                        // absent entries reload the first row (a cache hit), or row 0 if none
                        const int rr = pr[g] >= 0 ? pr[g] : (first_row >= 0 ? first_row : 0);
                        src = part + (size_t)rr * H8;
                        wg[g] = 1.0f;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) v[g][u] = load16<NTL>(src + cidx[u]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const bool keep = ZROW || pr[g] >= 0;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t wd[4] = {v[g][u].x, v[g][u].y, v[g][u].z, v[g][u].w};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const float lo = __builtin_fmaf(wg[g], bf16_lo(wd[c]), acc[u][2 * c]);
                            const float hi =
                                __builtin_fmaf(wg[g], bf16_hi(wd[c]), acc[u][2 * c + 1]);
                            acc[u][2 * c] = keep ? lo : acc[u][2 * c];
                            acc[u][2 * c + 1] = keep ? hi : acc[u][2 * c + 1];
                        }
                    }
                }
            }
            u32x4 *dst = out + (size_t)(t0 + tl) * H8;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (cok[u]) store16<true>(dst + cidx[u], pack_bf16(acc[u]));
        }
    }
}

// ------------------------------------------------------------------------------------------
// launch shapes
// ------------------------------------------------------------------------------------------

// Chunks per lane: four on batches of at least ~4096 items, fewer on small ones.
int pick_u(int T, int H8)
{
    if (EP_TWO_STAGE_U) return EP_TWO_STAGE_U;
    for (int u : {4, 2})
        if ((long)T * ceil_div(H8, u * kWave) >= 4096) return u;
    return 1;
}

// Tokens per group: up to 4 at prefill size, with every staged table within kStage entries.
int pick_tpb(int T, int per_token_a, int per_token_b)
{
    int tpb = T >= 2048 ? 4 : 1;
    while (tpb > 1 && (tpb * per_token_a > kStage || tpb * per_token_b > kStage)) --tpb;
    return tpb;
}

// Tokens per group for the staging copy: as the one-stage dispatch, about one item per
// wavefront (two tokens per group at prefill size, four if a row is a single item).
int pick_tpb_copy(int T, int R, int nseg)
{
    int tpb = (T >= 2048 ? 2 : 1) * (nseg == 1 ? 2 : 1);
    while (tpb > 1 && tpb * R > kStage) --tpb;
    return tpb;
}

dim3 grid_for(int T, int tpb) { return dim3(ceil_div(T, tpb)); }

}  // namespace

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------

namespace {

// Counting form of rank_prefix_wave: packed per-lane counts in RQ words of 4 ranks (R <= 4 RQ)
// while they cannot overflow, else ballots.
int pick_rq(int T, int R)
{
    if (T > kPackedRankMaxT) return 0;
    return R <= 4 ? 1 : R <= 16 ? 4 : 0;
}

}  // namespace

hipError_t launch_rank_layout(const ep_shape_t &s, const int32_t *idx, int32_t *rank_slot,
                              int32_t *rank_tokens, hipStream_t stream)
{
    const dim3 grid(s.T > 0 ? ceil_div(s.T, kRankTile) : 1), block(kRankTile);
    const int rq = pick_rq(s.T, s.R);
#define EP_LAUNCH_RL_RQ(KV, RQ)                                                                 \
    return launch(rank_layout_kernel<KV, RQ>, grid, block, 0, stream, idx, s.T, s.K, s.E, s.R,  \
                  rank_slot, rank_tokens)
#define EP_LAUNCH_RL(KV)                                                                        \
    do {                                                                                        \
        if (rq == 1) EP_LAUNCH_RL_RQ(KV, 1);                                                    \
        if (rq == 4) EP_LAUNCH_RL_RQ(KV, 4);                                                    \
        EP_LAUNCH_RL_RQ(KV, 0);                                                                 \
    } while (0)
    if (s.K == 4) EP_LAUNCH_RL(1);
    if (s.K == 8) EP_LAUNCH_RL(2);
    if (s.K == 12) EP_LAUNCH_RL(3);
    if (s.K == 16) EP_LAUNCH_RL(4);
    EP_LAUNCH_RL(0);
#undef EP_LAUNCH_RL
#undef EP_LAUNCH_RL_RQ
}

hipError_t launch_dispatch_ranks_bf16(const ep_shape_t &s, const uint16_t *x,
                                      const int32_t *rank_slot, uint16_t *stage,
                                      hipStream_t stream)
{
    const int H8 = s.H / 8, U = pick_u(s.T, H8), nseg = ceil_div(H8, U * kWave);
    const int tpb = pick_tpb_copy(s.T, s.R, nseg);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *sv = reinterpret_cast<u32x4 *>(stage);
#define EP_LAUNCH_DR(KG, MULTI)                                                                \
    do {                                                                                       \
        if (U >= 4)                                                                            \
            return launch(dispatch_ranks_bf16_kernel<KG, 4, MULTI>, grid, block, 0, stream, xv, \
                          rank_slot, sv, s.T, H8, s.R, tpb, nseg);                             \
        if (U == 2)                                                                            \
            return launch(dispatch_ranks_bf16_kernel<KG, 2, MULTI>, grid, block, 0, stream, xv, \
                          rank_slot, sv, s.T, H8, s.R, tpb, nseg);                             \
        return launch(dispatch_ranks_bf16_kernel<KG, 1, MULTI>, grid, block, 0, stream, xv,     \
                      rank_slot, sv, s.T, H8, s.R, tpb, nseg);                                 \
    } while (0)
    EP_BY_K(s.R, EP_LAUNCH_DR);
#undef EP_LAUNCH_DR
}

namespace {

template <int U>
hipError_t launch_ranks_fp8_u(const ep_shape_t &s, const u32x4 *x, const int32_t *rank_slot,
                              u32x4 *stage_q, float *stage_scale, hipStream_t stream)
{
    const int nseg = ceil_div(s.H, U * 16 * kWave);
    const int tpb = pick_tpb_copy(s.T, s.R, nseg);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
#define EP_LAUNCH_DRQ(KG, MULTI)                                                                \
    return launch(dispatch_ranks_fp8_kernel<KG, U, MULTI>, grid, block, 0, stream, x,          \
                  rank_slot, stage_q, stage_scale, s.T, s.H, s.R, tpb, nseg)
    EP_BY_K(s.R, EP_LAUNCH_DRQ);
#undef EP_LAUNCH_DRQ
}

}  // namespace

hipError_t launch_dispatch_ranks_fp8(const ep_shape_t &s, const uint16_t *x,
                                     const int32_t *rank_slot, uint8_t *stage_q,
                                     float *stage_scale, hipStream_t stream)
{
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *qv = reinterpret_cast<u32x4 *>(stage_q);
    if (pick_u_fp8(s.T, s.H) == 2)
        return launch_ranks_fp8_u<2>(s, xv, rank_slot, qv, stage_scale, stream);
    return launch_ranks_fp8_u<1>(s, xv, rank_slot, qv, stage_scale, stream);
}

namespace {

// Pair groups of the staging copy for R ranks, limited to the ones the rank counters' form RQ
// can meet: pick_rq gives RQ = 1 only for R <= 4 and RQ = 4 only for 4 < R <= 16; RQ = 0 (the
// ballots) means R > 16 or a batch past kPackedRankMaxT, and takes the looping form of groups
// of 8, which serves any R. Other pairings are never built.
#define EP_BY_R(RQ, R, LAUNCH)                                                                  \
    do {                                                                                        \
        if constexpr (RQ == 1) {                                                                \
            if ((R) > 2) LAUNCH(4, false);                                                      \
            if ((R) > 1) LAUNCH(2, false);                                                      \
            LAUNCH(1, false);                                                                   \
        } else if constexpr (RQ == 4) {                                                         \
            if ((R) > 8) LAUNCH(8, true);                                                       \
            LAUNCH(8, false);                                                                   \
        } else {                                                                                \
            LAUNCH(8, true);                                                                    \
        }                                                                                       \
    } while (0)

// Tokens per fused tile: at most one wavefront's worth (one lane per token ranks the tile),
// TT*R <= kRankTile staged rows; on prefill-sized batches 8 for bf16 rows (two workgroups per
// CU, each wavefront copying one half row: 24.8 us at T = 4096 against 25.8 us with 16 tokens
// and whole rows) and 16 for FP8 rows (one workgroup per CU); 4 on small batches. FP8 at
// T = 4096, R = 3: 13.4 us with two 16-channel pieces per lane and 16-token tiles; with one
// piece per lane the kernel fits two workgroups per CU (60 VGPRs, 64 SGPRs), but measured
// 14.1 us at 8-token tiles and 14.2 us at 16; two pieces with 8-token tiles 15.8 us.
int pick_tt_ranks(int T, int R, bool fp8)
{
    int tt = EP_RANKS_FUSED_TT ? EP_RANKS_FUSED_TT : (T >= 2048 ? (fp8 ? 16 : 8) : 4);
    tt = min(tt, kWave);
    while (tt > 1 && tt * R > kRankTile) tt /= 2;
    return tt;
}

template <int KV, int U, int RQ>
hipError_t launch_rank_dispatch_bf16_rq(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                                        int32_t *rank_slot, int32_t *rank_tokens, u32x4 *stage,
                                        hipStream_t stream)
{
    const int H8 = s.H / 8, nseg = ceil_div(H8, U * kWave), TT = pick_tt_ranks(s.T, s.R, false);
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kRankTile);
#define EP_LAUNCH_RLD(KG, MULTI)                                                                \
    return launch(rank_layout_dispatch_bf16_kernel<KV, RQ, KG, U, MULTI>, grid, block, 0,      \
                  stream, x, idx, rank_slot, rank_tokens, stage, s.T, H8, s.K, s.E, s.R, TT,    \
                  nseg)
    EP_BY_R(RQ, s.R, EP_LAUNCH_RLD);
#undef EP_LAUNCH_RLD
}

template <int KV, int U>
hipError_t launch_rank_dispatch_bf16(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                                     int32_t *rank_slot, int32_t *rank_tokens, u32x4 *stage,
                                     hipStream_t stream)
{
    const int rq = pick_rq(s.T, s.R);
    if (rq == 1)
        return launch_rank_dispatch_bf16_rq<KV, U, 1>(s, x, idx, rank_slot, rank_tokens, stage, stream);
    if (rq == 4)
        return launch_rank_dispatch_bf16_rq<KV, U, 4>(s, x, idx, rank_slot, rank_tokens, stage, stream);
    return launch_rank_dispatch_bf16_rq<KV, U, 0>(s, x, idx, rank_slot, rank_tokens, stage, stream);
}

template <int KV, int U, int RQ>
hipError_t launch_rank_dispatch_fp8_rq(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                                       int32_t *rank_slot, int32_t *rank_tokens, u32x4 *stage_q,
                                       float *stage_scale, hipStream_t stream)
{
    const int nseg = ceil_div(s.H, U * 16 * kWave), TT = pick_tt_ranks(s.T, s.R, true);
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kRankTile);
#define EP_LAUNCH_RLQ(KG, MULTI)                                                                \
    return launch(rank_layout_dispatch_fp8_kernel<KV, RQ, KG, U, MULTI>, grid, block, 0,       \
                  stream, x, idx, rank_slot, rank_tokens, stage_q, stage_scale, s.T, s.H, s.K,  \
                  s.E, s.R, TT, nseg)
    EP_BY_R(RQ, s.R, EP_LAUNCH_RLQ);
#undef EP_LAUNCH_RLQ
}

template <int KV, int U>
hipError_t launch_rank_dispatch_fp8(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                                    int32_t *rank_slot, int32_t *rank_tokens, u32x4 *stage_q,
                                    float *stage_scale, hipStream_t stream)
{
    const int rq = pick_rq(s.T, s.R);
    if (rq == 1)
        return launch_rank_dispatch_fp8_rq<KV, U, 1>(s, x, idx, rank_slot, rank_tokens, stage_q,
                                                     stage_scale, stream);
    if (rq == 4)
        return launch_rank_dispatch_fp8_rq<KV, U, 4>(s, x, idx, rank_slot, rank_tokens, stage_q,
                                                     stage_scale, stream);
    return launch_rank_dispatch_fp8_rq<KV, U, 0>(s, x, idx, rank_slot, rank_tokens, stage_q,
                                                 stage_scale, stream);
}

template <int KV>
hipError_t launch_rank_dispatch_bf16_kv(const ep_shape_t &s, const uint16_t *x,
                                        const int32_t *idx, int32_t *rank_slot,
                                        int32_t *rank_tokens, uint16_t *stage, hipStream_t stream)
{
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *sv = reinterpret_cast<u32x4 *>(stage);
    // half rows (two chunks per lane) where the other kernels take whole ones: two 8-token
    // tiles per CU then give every wavefront one item
    const int U = min(pick_u(s.T, s.H / 8), 2);
    if (U == 2) return launch_rank_dispatch_bf16<KV, 2>(s, xv, idx, rank_slot, rank_tokens, sv, stream);
    return launch_rank_dispatch_bf16<KV, 1>(s, xv, idx, rank_slot, rank_tokens, sv, stream);
}

template <int KV>
hipError_t launch_rank_dispatch_fp8_kv(const ep_shape_t &s, const uint16_t *x,
                                       const int32_t *idx, int32_t *rank_slot,
                                       int32_t *rank_tokens, uint8_t *stage_q,
                                       float *stage_scale, hipStream_t stream)
{
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *qv = reinterpret_cast<u32x4 *>(stage_q);
    if ((EP_RANKS_FP8_U ? EP_RANKS_FP8_U : pick_u_fp8(s.T, s.H)) == 2)
        return launch_rank_dispatch_fp8<KV, 2>(s, xv, idx, rank_slot, rank_tokens, qv,
                                               stage_scale, stream);
    return launch_rank_dispatch_fp8<KV, 1>(s, xv, idx, rank_slot, rank_tokens, qv, stage_scale,
                                           stream);
}

}  // namespace

hipError_t launch_rank_layout_dispatch_bf16(const ep_shape_t &s, const uint16_t *x,
                                            const int32_t *idx, int32_t *rank_slot,
                                            int32_t *rank_tokens, uint16_t *stage,
                                            hipStream_t stream)
{
    // no tokens: nothing to copy, and the fused kernel's row loads would have no row to read
    if (s.T == 0) return launch_rank_layout(s, idx, rank_slot, rank_tokens, stream);
    if (s.K == 8)
        return launch_rank_dispatch_bf16_kv<2>(s, x, idx, rank_slot, rank_tokens, stage, stream);
    return launch_rank_dispatch_bf16_kv<0>(s, x, idx, rank_slot, rank_tokens, stage, stream);
}

hipError_t launch_rank_layout_dispatch_fp8(const ep_shape_t &s, const uint16_t *x,
                                           const int32_t *idx, int32_t *rank_slot,
                                           int32_t *rank_tokens, uint8_t *stage_q,
                                           float *stage_scale, hipStream_t stream)
{
    if (s.T == 0) return launch_rank_layout(s, idx, rank_slot, rank_tokens, stream);
    if (s.K == 8)
        return launch_rank_dispatch_fp8_kv<2>(s, x, idx, rank_slot, rank_tokens, stage_q,
                                              stage_scale, stream);
    return launch_rank_dispatch_fp8_kv<0>(s, x, idx, rank_slot, rank_tokens, stage_q,
                                          stage_scale, stream);
}

hipError_t launch_dispatch_expand_bf16(const ep_shape_t &s, const uint16_t *stage,
                                       const int32_t *idx, const int32_t *slot,
                                       const int32_t *rank_slot, uint16_t *recv,
                                       hipStream_t stream)
{
    const int H8 = s.H / 8, U = pick_u(s.T, H8);
    const int nseg = ceil_div(H8, U * kWave);
    const int tpb = pick_tpb(s.T, s.K, s.R);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
    const u32x4 *sv = reinterpret_cast<const u32x4 *>(stage);
    u32x4 *rv = reinterpret_cast<u32x4 *>(recv);
#define EP_LAUNCH_EX(KG, MULTI)                                                                 \
    do {                                                                                        \
        if (U >= 4)                                                                             \
            return launch(expand_bf16_kernel<KG, 4, MULTI>, grid, block, 0, stream, sv, idx,     \
                          slot, rank_slot, rv, s.T, H8, s.E, s.C, s.K, s.R, tpb, nseg);         \
        if (U == 2)                                                                             \
            return launch(expand_bf16_kernel<KG, 2, MULTI>, grid, block, 0, stream, sv, idx,     \
                          slot, rank_slot, rv, s.T, H8, s.E, s.C, s.K, s.R, tpb, nseg);         \
        return launch(expand_bf16_kernel<KG, 1, MULTI>, grid, block, 0, stream, sv, idx, slot,   \
                      rank_slot, rv, s.T, H8, s.E, s.C, s.K, s.R, tpb, nseg);                   \
    } while (0)
    EP_BY_K(s.K, EP_LAUNCH_EX);
#undef EP_LAUNCH_EX
}

hipError_t launch_dispatch_expand_fp8(const ep_shape_t &s, const uint8_t *stage_q,
                                      const float *stage_scale, const int32_t *idx,
                                      const int32_t *slot, const int32_t *rank_slot,
                                      uint8_t *recv_q, float *recv_scale, hipStream_t stream)
{
    const int nseg = ceil_div(s.H, 16 * kWave);
    const int tpb = pick_tpb(s.T, s.K, s.R);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
    const u32x4 *sq = reinterpret_cast<const u32x4 *>(stage_q);
    u32x4 *rq = reinterpret_cast<u32x4 *>(recv_q);
#define EP_LAUNCH_EXQ(KG, MULTI)                                                                 \
    return launch(expand_fp8_kernel<KG, MULTI>, grid, block, 0, stream, sq, stage_scale, idx,    \
                  slot, rank_slot, rq, recv_scale, s.T, s.H, s.E, s.C, s.K, s.R, tpb, nseg)
    EP_BY_K(s.K, EP_LAUNCH_EXQ);
#undef EP_LAUNCH_EXQ
}

hipError_t launch_combine_ranks(const ep_shape_t &s, const uint16_t *y, const int32_t *idx,
                                const int32_t *slot, const int32_t *rank_slot, const float *w,
                                uint16_t *part, hipStream_t stream)
{
    const int H8 = s.H / 8;
    const bool seq = s.K > 8;
    // at most half rows (two chunks per lane, 100 VGPRs, 4 wavefronts per SIMD), with plain
    // partial-row stores: at T = 4096 44.4 against 50.7 us with whole rows and non-temporal
    // stores (bf16, R = 16; pass 136.8-137.4 against 138.8-139.1 us), FP8 (R = 3) 35.2 against
    // 36.0 us; whole rows with plain stores, or one chunk per lane, measured in between. Four
    // tokens per group (pick_tpb) stay: 1, 2 and 8 measured 45.9, 44.9-45.0 and 46.2 us (bf16)
    const int U = seq ? 1 : EP_CR_U ? EP_CR_U : min(pick_u(s.T, H8), 2);
    const int nseg = ceil_div(H8, U * kWave);
    const int tpb = pick_tpb(s.T, s.K, s.R);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
    const u32x4 *yv = reinterpret_cast<const u32x4 *>(y);
    u32x4 *pv = reinterpret_cast<u32x4 *>(part);
    if (seq)
        return launch(combine_ranks_kernel<1, 1, true>, grid, block, 0, stream, yv, idx, slot,
                      rank_slot, w, pv, s.T, H8, s.E, s.C, s.K, s.R, tpb, nseg);
#define EP_LAUNCH_CR(KG)                                                                        \
    do {                                                                                        \
        if constexpr (EP_CR_U >= 4) {                                                           \
            if (U >= 4)                                                                         \
                return launch(combine_ranks_kernel<KG, 4, false>, grid, block, 0, stream, yv,    \
                              idx, slot, rank_slot, w, pv, s.T, H8, s.E, s.C, s.K, s.R, tpb,    \
                              nseg);                                                            \
        }                                                                                       \
        if (U == 2)                                                                             \
            return launch(combine_ranks_kernel<KG, 2, false>, grid, block, 0, stream, yv, idx,   \
                          slot, rank_slot, w, pv, s.T, H8, s.E, s.C, s.K, s.R, tpb, nseg);      \
        return launch(combine_ranks_kernel<KG, 1, false>, grid, block, 0, stream, yv, idx, slot, \
                      rank_slot, w, pv, s.T, H8, s.E, s.C, s.K, s.R, tpb, nseg);                \
    } while (0)
    if (s.K > 4) EP_LAUNCH_CR(8);
    if (s.K > 2) EP_LAUNCH_CR(4);
    if (s.K > 1) EP_LAUNCH_CR(2);
    EP_LAUNCH_CR(1);
#undef EP_LAUNCH_CR
}

hipError_t launch_combine_reduce(const ep_shape_t &s, const uint16_t *part,
                                 const int32_t *rank_slot, uint16_t *out, hipStream_t stream)
{
    const int H8 = s.H / 8, U = pick_u(s.T, H8);
    const int nseg = ceil_div(H8, U * kWave);
    const int Q = s.K < s.R ? s.K : s.R;           // a token reaches at most min(K, R) ranks
    const int tpb = pick_tpb(s.T, s.R, Q);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
    const u32x4 *pv = reinterpret_cast<const u32x4 *>(part);
    u32x4 *ov = reinterpret_cast<u32x4 *>(out);
    // the partial combine's plain stores leave a small partial buffer in the last-level cache:
    // at T = 4096, H = 2048 the FP8 workload's R = 3 (50 MB of rows) reduces in 13.5 against
    // 13.9 us and its pass takes 78.9-79.4 against 81.9-82.3 us read through the caches, while
    // the bf16 workload's R = 16 (268 MB) is faster read non-temporally (22.6 against 23.8 us)
    // rows longer than the zero row (over 64 KiB each) are always read non-temporally
    const bool ntl = H8 > kZeroChunks ||
                     (size_t)s.R * s.T * s.H * sizeof(uint16_t) > (size_t)EP_RED_CACHED_BYTES;
#define EP_LAUNCH_RD_UZN(KG, UU, MULTI, Z, N)                                                   \
    return launch(combine_reduce_kernel<KG, UU, MULTI, Z, N>, grid, block, 0, stream, pv,        \
                  rank_slot, ov, s.T, H8, s.R, Q, tpb, nseg)
#define EP_LAUNCH_RD_ZN(KG, MULTI, Z, N)                                                        \
    do {                                                                                        \
        if (U >= 4) EP_LAUNCH_RD_UZN(KG, 4, MULTI, Z, N);                                       \
        if (U == 2) EP_LAUNCH_RD_UZN(KG, 2, MULTI, Z, N);                                       \
        EP_LAUNCH_RD_UZN(KG, 1, MULTI, Z, N);                                                   \
    } while (0)
#define EP_LAUNCH_RD4_ZN(KG, MULTI, Z, N) EP_LAUNCH_RD_UZN(KG, 4, MULTI, Z, N)
#define EP_LAUNCH_RD12_ZN(KG, MULTI, Z, N)                                                      \
    do {                                                                                        \
        if (U == 2) EP_LAUNCH_RD_UZN(KG, 2, MULTI, Z, N);                                       \
        EP_LAUNCH_RD_UZN(KG, 1, MULTI, Z, N);                                                   \
    } while (0)
// ZN: the launch for one zero-row / load-policy pair (with every chunk count, or some)
#define EP_LAUNCH_RD_SEL(ZN, KG, MULTI)                                                         \
    do {                                                                                        \
        if (H8 <= kZeroChunks) {                                                                \
            if (ntl) ZN(KG, MULTI, true, true);                                                 \
            ZN(KG, MULTI, true, false);                                                         \
        }                                                                                       \
        ZN(KG, MULTI, false, true);                                                             \
    } while (0)
#define EP_LAUNCH_RD(KG, MULTI) EP_LAUNCH_RD_SEL(EP_LAUNCH_RD_ZN, KG, MULTI)
    // lists of 5..8 partials: whole-row items (U = 4) fold them as two groups of four (118
    // VGPRs, 4 wavefronts per SIMD: 22.6 against 23.5 us with one group of eight at T = 4096,
    // R = 16), narrower items as one group of eight
    if (Q > 8) EP_LAUNCH_RD(8, true);
    if (Q > 4) {
        if (U >= 4) EP_LAUNCH_RD_SEL(EP_LAUNCH_RD4_ZN, 4, true);
        EP_LAUNCH_RD_SEL(EP_LAUNCH_RD12_ZN, 8, false);
    }
    if (Q > 2) EP_LAUNCH_RD(4, false);
    if (Q > 1) EP_LAUNCH_RD(2, false);
    EP_LAUNCH_RD(1, false);
#undef EP_LAUNCH_RD
#undef EP_LAUNCH_RD_SEL
#undef EP_LAUNCH_RD12_ZN
#undef EP_LAUNCH_RD4_ZN
#undef EP_LAUNCH_RD_ZN
#undef EP_LAUNCH_RD_UZN
}

}  // namespace ep
