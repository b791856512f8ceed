// Layout and dispatch fused into one kernel on gfx950.
//
// The "normal" EP APIs compute the dispatch layout before dispatch inside one boundary
// (awsome-distributed-ai PR #1238, "What changed"). Here each workgroup of 1024 lanes owns a
// tile of TT tokens (TT*K pairs): it computes the slots of its own pairs exactly as the
// standalone layout does (layout_tile: a histogram of all earlier pairs, then ballot ranks
// inside the tile; no workgroup waits on another), keeps their receive rows in LDS, and
// immediately copies (bf16) or quantises and copies (FP8) its tokens' rows into the receive
// buffer. The workgroup of the last tile also writes counts, offsets, per-rank sums and stats.
// The results are identical to ep_layout followed by ep_dispatch / ep_dispatch_fp8.
//
// Why: the standalone layout is a separate launch (~2.5 µs of launch floor on MI355X) whose
// latency the row copies then wait for. Fused, each tile starts copying as soon as its own
// slots are known, so the layout of later tiles overlaps the copies of earlier ones; and in the
// bf16 kernel each wavefront issues its first row piece's loads together with the layout's own
// loads, since only the stores need the slots.
//
// The packed variants (layout_dispatch_packed_*) write each pair to its row of a packed,
// aligned buffer, offset[e] + slot. Those offsets need every expert's total, so each of their
// tiles counts all pairs, the later ones too (layout_tile<true>), and scans the offsets itself.
// The results are identical to ep_layout_packed followed by ep_dispatch_packed[_fp8].
#include "ep_dispatch_item.h"
#include "ep_internal.h"
#include "ep_layout_tile.h"

#ifndef EP_FUSED_TT
#define EP_FUSED_TT 0        // tokens per tile (0 = choose from the shape)
#endif
#ifndef EP_PACKED_TT
#define EP_PACKED_TT 0       // tokens per tile of the fused packed kernels (0 = as EP_FUSED_TT)
#endif
// Wavefronts per SIMD the FP8 fused kernel is compiled to fit. 8 (two 1024-lane workgroups per
// CU) holds it to 78 scalar registers (22 of them spilled to vector-register lanes) and 63
// VGPRs; unbounded it takes 102 scalar registers and one workgroup per CU.
#ifndef EP_FUSED_FP8_WAVES
#define EP_FUSED_FP8_WAVES 8
#endif

// The expansions (here fused with the expert layout, and expand_*_kernel) store the expert rows
// non-temporally, unlike the one-stage dispatch: in the two-stage pass at T = 4096 the bf16
// layout + expansion takes 46.9 against 48.2-48.4 us and the pass 129.2-129.6 against
// 136.3-136.6 us (the partial combine and the reduce that follow no longer share the caches
// with the expansion's dirty rows); FP8 21.0 against 22.1 us, the pass the same (78.3-78.5 us).
#ifndef EP_EXPAND_NT_STORE
#define EP_EXPAND_NT_STORE 1
#endif
// The layout + expansion kernels load their tile's rank_slot rows with the ids, before the
// layout, and keep them in LDS for the copies (otherwise each pair group reads them from
// global memory, a dependent round trip before its row loads). At T = 4096: bf16 (R = 16)
// 46.6-46.7 against 46.9-47.0 us, FP8 (R = 3) 20.7-20.75 against 20.9-21.1 us.
#ifndef EP_LX_RANK_SLOT_LDS
#define EP_LX_RANK_SLOT_LDS 1
#endif
// Order of the tiles over the XCDs in each fused kernel (xcd_tile, ep_device.h). All keep the
// identity. The bf16 layout + dispatch at T = 4096 ran 25.4-25.6 us with order 1 against
// 26.0-26.3 us in one allocation of the benchmark's buffers, but 27.4 against 25.3 us (step
// 53.1-53.5 against 51.7 us) when the buffers sat elsewhere (the benchmark's other config
// orders): which XCDs write slowly depends on where the written rows lie. The FP8 one: 18.2-18.8
// us with the identity, 18.6-18.8 with order 1, 19.3-19.4 with order 2. The layout + expansion
// kernels: bf16 48.7 us all three ways; FP8 22.0 us with the identity, 22.4 and 23.0 us.
#ifndef EP_FUSED_BF16_XCD_ORDER
#define EP_FUSED_BF16_XCD_ORDER 0
#endif
#ifndef EP_FUSED_FP8_XCD_ORDER
#define EP_FUSED_FP8_XCD_ORDER 0
#endif
#ifndef EP_EXPAND_BF16_XCD_ORDER
#define EP_EXPAND_BF16_XCD_ORDER 0
#endif
#ifndef EP_EXPAND_FP8_XCD_ORDER
#define EP_EXPAND_FP8_XCD_ORDER 0
#endif

namespace ep {

namespace {

// CHUNKED: step 1 of the layout reads the chunk histograms in `hist` (see ep_layout_tile.h).
template <int KG, int U, bool MULTI, bool CHUNKED>
__global__ __launch_bounds__(kTileThreads) void layout_dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx, LayoutOut o,
    u32x4 *__restrict__ recv, int T, int H8, int E, int C, int K, int R, int nbits, int lg_nc,
    int TT, int nseg, const int32_t *__restrict__ hist)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t rows[kTileThreads];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc);
    const int TK = T * K;
    const int tile = xcd_tile<EP_FUSED_BF16_XCD_ORDER>();
    const bool last = tile == (int)gridDim.x - 1;
    const int t0 = tile * TT;
    const int nt = min(TT, T - t0);
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int nitems = nt * nseg;
    // the first item's row loads do not depend on the slots: they are issued before the
    // layout's own loads (which the layout waits for in full), so both round trips overlap.
    // The ids first and the rows after them (which the layout then need not wait for) measured
    // the same at T = 4096 (26.1-26.2 against 26.2-26.4 us) and slower at T = 128 (cold step
    // 12.7 against 12.3-12.5 us).
    RowPiece<U> first;
    if (wave < nitems) first = load_item_bf16<U>(x, t0 + wave / nseg, wave % nseg, H8);
    const TileIds ids = layout_tile_loads<false, CHUNKED>(idx, TK, t0 * K, TT * K);
    layout_tile<false, CHUNKED>(ids, idx, TK, E, C, nbits, t0 * K, TT * K, last, lds, m, o.slot,
                                rows, 1, 0, hist);
    if (wave < nitems)
        store_item_bf16<KG, U, MULTI>(first, recv, rows, wave / nseg, wave % nseg, H8, K);
    for (int item = wave + kTileWaves; item < nitems; item += kTileWaves) {
        const int tl = item / nseg;
        dispatch_item_bf16<KG, U, MULTI>(x, recv, rows, t0 + tl, tl, item - tl * nseg, H8, K);
    }
    if (last) layout_finish<false>(TK, E, C, R, lds, m, o);
}

template <int KG, int U, bool MULTI, bool CHUNKED>
__global__ __launch_bounds__(kTileThreads, EP_FUSED_FP8_WAVES) void layout_dispatch_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx, LayoutOut o,
    u32x4 *__restrict__ recv_q, float *__restrict__ recv_scale, int T, int H, int E, int C,
    int K, int R, int nbits, int lg_nc, int TT, int nseg, const int32_t *__restrict__ hist)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t rows[kTileThreads];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc);
    const int TK = T * K;
    const int tile = xcd_tile<EP_FUSED_FP8_XCD_ORDER>();
    const bool last = tile == (int)gridDim.x - 1;
    const int t0 = tile * TT;
    const int nt = min(TT, T - t0);
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int nitems = nt * nseg;
    // the first item's row loads go out after the layout's id loads, and the cast waits until
    // after the layout: at T = 128 the fused kernel takes 6.3 us against 6.6 us without the
    // early loads (issued before the ids, at T = 4096 they measured 18.6 -> 19.2 us; cast
    // before the layout, 19.0 -> 19.8 us). The row loads sit under a branch (wavefronts with an
    // item), so the layout's waits cover them too; loading them with no branch, which lets the
    // layout wait for the ids alone, measured slower (20.9 against 18.1 us at T = 4096).
    const TileIds ids = layout_tile_loads<false, CHUNKED>(idx, TK, t0 * K, TT * K);
    RawPieceFp8<U> first;
    if (wave < nitems) first = load_item_fp8<U>(x, t0 + wave / nseg, wave % nseg, H);
    layout_tile<false, CHUNKED>(ids, idx, TK, E, C, nbits, t0 * K, TT * K, last, lds, m, o.slot,
                                rows, 1, 0, hist);
    if (wave < nitems)
        store_item_fp8<KG, U, MULTI>(cast_item_fp8<U>(first), recv_q, recv_scale, rows,
                                     wave / nseg, wave % nseg, H, K);
    for (int item = wave + kTileWaves; item < nitems; item += kTileWaves) {
        const int tl = item / nseg;
        dispatch_item_fp8<KG, U, MULTI>(x, recv_q, recv_scale, rows, t0 + tl, tl,
                                        item - tl * nseg, H, K);
    }
    if (last) layout_finish<false>(TK, E, C, R, lds, m, o);
}

// The expert layout fused into the two-stage expansion: layout_tile gives the tile's receive
// rows as in layout_dispatch_bf16_kernel, and each kept pair then copies its rank's staging row
// (row rank_slot[t][r] of rank r = e / (E/R) in the [R][T] staging buffer, e = row / C) instead
// of the token's row of x; a pair whose rank_slot entry is outside [0, T) is not copied. Pairs of one rank
// read the same staging row, so these loads keep the caches (the second read hits).
// A lane takes one 16-byte chunk per pair (U = 1) and the kernel is held to 8 wavefronts per
// SIMD (47 VGPRs, 78 SGPRs: two 1024-lane workgroups per CU). Prefill bf16 (T = 4096, R = 16):
// 48.6 us against 6.7 + 44.8 us for the layout and the expansion apart; half rows per item
// spill under that bound (60.1 us), and without it one workgroup fits per CU (49.6 us).
// The staged row of a pair depends only on its id and rank_slot, so the first item's loads
// could go out before the layout, as the one-stage kernels do with x; measured on MI355X this
// gains under 2% on bf16 (48.5 -> 47.7 us with 4 of 8 pairs early, the 8-pair form spills) and
// costs FP8 6 to 20% (22.1 -> 23.4 / 26.8 us), so the loads stay after the layout.
template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kTileThreads, 8) void layout_expand_bf16_kernel(
    const u32x4 *__restrict__ stage, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ rank_slot, LayoutOut o, u32x4 *__restrict__ recv, int T, int H8,
    int E, int C, int K, int R, int nbits, int lg_nc, int TT, int nseg)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t rows[kTileThreads];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc);
    const int TK = T * K;
    const int tile = xcd_tile<EP_EXPAND_BF16_XCD_ORDER>();
    const bool last = tile == (int)gridDim.x - 1;
    const int t0 = tile * TT;
    const int nt = min(TT, T - t0);
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int nitems = nt * nseg;
    const int EL = E / R;
    const TileIds ids = layout_tile_loads(idx, TK, t0 * K, TT * K);
    // the tile's rank_slot rows (nt * R <= kTileThreads ints), loaded after the ids
    __shared__ int32_t rs_tile[EP_LX_RANK_SLOT_LDS ? kTileThreads : 1];
    const int nrs = nt * R;
    int rs_own = 0;
    if constexpr (EP_LX_RANK_SLOT_LDS) {
        if ((int)threadIdx.x < nrs) rs_own = rank_slot[(size_t)t0 * R + threadIdx.x];
    }
    layout_tile(ids, idx, TK, E, C, nbits, t0 * K, TT * K, last, lds, m, o.slot, rows);
    if constexpr (EP_LX_RANK_SLOT_LDS) {
        if ((int)threadIdx.x < nrs) rs_tile[threadIdx.x] = rs_own;
        __syncthreads();
    }
    // token tl's staging row of rank rk (from LDS, or from global memory)
    auto rank_row = [&](int tl, int rk) -> int {
        if constexpr (EP_LX_RANK_SLOT_LDS) return rs_tile[tl * R + rk];
        else return rank_slot[(size_t)(t0 + tl) * R + rk];
    };
    for (int item = wave; item < nitems; item += kTileWaves) {
        const int tl = item / nseg, seg = item - tl * nseg;
        const int npg = MULTI ? (K + KG - 1) / KG : 1;
        for (int pg = 0; pg < npg; ++pg) {
            int r[KG];
            token_rows<KG>(rows, tl, pg * KG, K, r);
            u32x4 v[KG][U];
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                int sr = -1;
                if (r[g] >= 0) {
                    const int rk = (r[g] / C) / EL;
                    const int p = wave_uniform(rank_row(tl, rk));
                    sr = (unsigned)p < (unsigned)T ? rk * T + p : -1;
                }
                if (sr < 0) r[g] = -1;     // no staged row: the pair is not copied
                const u32x4 *src = stage + (size_t)(sr >= 0 ? sr : 0) * H8;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = (seg * U + u) * kWave + lane;
                    v[g][u] = load16<false>(src + (c < H8 ? c : H8 - 1));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                if (r[g] < 0) continue;
                u32x4 *dst = recv + (size_t)r[g] * H8;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = (seg * U + u) * kWave + lane;
                    if (c < H8) store16<EP_EXPAND_NT_STORE>(dst + c, v[g][u]);
                }
            }
        }
    }
    if (last) layout_finish<false>(TK, E, C, R, lds, m, o);
}

// The same for FP8: a lane copies one 16-byte chunk of codes per pair (a 1024-channel segment
// per wavefront item), and the first lane of each 8-lane group (one 128-channel block) also
// copies the block's scale.
template <int KG, bool MULTI>
__global__ __launch_bounds__(kTileThreads, 8) void layout_expand_fp8_kernel(
    const u32x4 *__restrict__ stage_q, const float *__restrict__ stage_scale,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ rank_slot, LayoutOut o,
    u32x4 *__restrict__ recv_q, float *__restrict__ recv_scale, int T, int H, int E, int C,
    int K, int R, int nbits, int lg_nc, int TT, int nseg)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t rows[kTileThreads];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc);
    const int TK = T * K;
    const int tile = xcd_tile<EP_EXPAND_FP8_XCD_ORDER>();
    const bool last = tile == (int)gridDim.x - 1;
    const int t0 = tile * TT;
    const int nt = min(TT, T - t0);
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int nitems = nt * nseg;
    const int EL = E / R, H16 = H / 16, NB = H / 128;
    const TileIds ids = layout_tile_loads(idx, TK, t0 * K, TT * K);
    // the tile's rank_slot rows (nt * R <= kTileThreads ints), loaded after the ids
    __shared__ int32_t rs_tile[EP_LX_RANK_SLOT_LDS ? kTileThreads : 1];
    const int nrs = nt * R;
    int rs_own = 0;
    if constexpr (EP_LX_RANK_SLOT_LDS) {
        if ((int)threadIdx.x < nrs) rs_own = rank_slot[(size_t)t0 * R + threadIdx.x];
    }
    layout_tile(ids, idx, TK, E, C, nbits, t0 * K, TT * K, last, lds, m, o.slot, rows);
    if constexpr (EP_LX_RANK_SLOT_LDS) {
        if ((int)threadIdx.x < nrs) rs_tile[threadIdx.x] = rs_own;
        __syncthreads();
    }
    // token tl's staging row of rank rk (from LDS, or from global memory)
    auto rank_row = [&](int tl, int rk) -> int {
        if constexpr (EP_LX_RANK_SLOT_LDS) return rs_tile[tl * R + rk];
        else return rank_slot[(size_t)(t0 + tl) * R + rk];
    };
    for (int item = wave; item < nitems; item += kTileWaves) {
        const int tl = item / nseg, seg = item - tl * nseg;
        const int h0 = seg * (16 * kWave) + lane * 16;
        const bool act = h0 < H;
        const bool lead = act && (lane & 7) == 0;
        const int cq = act ? h0 / 16 : 0, cs = act ? h0 / 128 : 0;
        const int npg = MULTI ? (K + KG - 1) / KG : 1;
        for (int pg = 0; pg < npg; ++pg) {
            int r[KG];
            token_rows<KG>(rows, tl, pg * KG, K, r);
            u32x4 q[KG];
            float sc[KG];
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                int sr = -1;
                if (r[g] >= 0) {
                    const int rk = (r[g] / C) / EL;
                    const int p = wave_uniform(rank_row(tl, rk));
                    sr = (unsigned)p < (unsigned)T ? rk * T + p : -1;
                }
                if (sr < 0) r[g] = -1;     // no staged row: the pair is not copied
                const size_t row = (size_t)(sr >= 0 ? sr : 0);
                q[g] = stage_q[row * H16 + cq];
                sc[g] = stage_scale[row * NB + cs];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                if (r[g] < 0) continue;
                if (act) store16<EP_EXPAND_NT_STORE>(recv_q + (size_t)r[g] * H16 + cq, q[g]);
                if (lead) recv_scale[(size_t)r[g] * NB + cs] = sc[g];
            }
        }
    }
    if (last) layout_finish<false>(TK, E, C, R, lds, m, o);
}

// The packed layout and dispatch fused: every tile counts all pairs (ALL in layout_tile), so
// each workgroup knows the packed offsets and copies its tokens to offset[e] + slot at once.
template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kTileThreads) void layout_dispatch_packed_bf16_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx, LayoutOut o,
    u32x4 *__restrict__ recv, int T, int H8, int E, int C, int K, int R, int nbits, int lg_nc,
    int TT, int nseg, int rows_cap)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t rows[kTileThreads];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc, true);
    const int TK = T * K;
    const bool last = blockIdx.x == gridDim.x - 1;
    const int t0 = blockIdx.x * TT;
    const int nt = min(TT, T - t0);
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int nitems = nt * nseg;
    RowPiece<U> first;
    if (wave < nitems) first = load_item_bf16<U>(x, t0 + wave / nseg, wave % nseg, H8);
    const TileIds ids = layout_tile_loads<true>(idx, TK, t0 * K, TT * K);
    layout_tile<true>(ids, idx, TK, E, C, nbits, t0 * K, TT * K, last, lds, m, o.slot, rows,
                      o.align, rows_cap);
    if (wave < nitems)
        store_item_bf16<KG, U, MULTI>(first, recv, rows, wave / nseg, wave % nseg, H8, K);
    for (int item = wave + kTileWaves; item < nitems; item += kTileWaves) {
        const int tl = item / nseg;
        dispatch_item_bf16<KG, U, MULTI>(x, recv, rows, t0 + tl, tl, item - tl * nseg, H8, K);
    }
    if (last) layout_finish<true>(TK, E, C, R, lds, m, o);
}

template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kTileThreads) void layout_dispatch_packed_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx, LayoutOut o,
    u32x4 *__restrict__ recv_q, float *__restrict__ recv_scale, int T, int H, int E, int C,
    int K, int R, int nbits, int lg_nc, int TT, int nseg, int rows_cap)
{
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int32_t rows[kTileThreads];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc, true);
    const int TK = T * K;
    const bool last = blockIdx.x == gridDim.x - 1;
    const int t0 = blockIdx.x * TT;
    const int nt = min(TT, T - t0);
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int nitems = nt * nseg;
    const TileIds ids = layout_tile_loads<true>(idx, TK, t0 * K, TT * K);
    layout_tile<true>(ids, idx, TK, E, C, nbits, t0 * K, TT * K, last, lds, m, o.slot, rows,
                      o.align, rows_cap);
    for (int item = wave; item < nitems; item += kTileWaves) {
        const int tl = item / nseg;
        dispatch_item_fp8<KG, U, MULTI>(x, recv_q, recv_scale, rows, t0 + tl, tl,
                                        item - tl * nseg, H, K);
    }
    if (last) layout_finish<true>(TK, E, C, R, lds, m, o);
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Tokens per tile, with TT*K a multiple of 4 (tile starts stay 16-byte aligned in topk_idx)
// and TT*K <= 1024 pairs. Small batches use small tiles, about 256 of them, so more workgroups
// and CUs share the copies (measured on MI355X at T = 128: one token per tile 12.5 us per
// single-shot bf16 step against 13.3 us with four); on large ones (T = 4096) both dtypes do
// best at 8 tokens per tile, two workgroups per CU (FP8 at T = 4096, E = 96: 18.2 us, against
// 19.3 us with 16-token tiles at one workgroup per CU, 26.2 us with 4-token tiles); at
// T = 2048 bf16 takes 4 (30.5 against 30.9 us per step with 8).
int pick_tt(int T, int K, bool fp8)
{
    int tt = EP_FUSED_TT ? EP_FUSED_TT
                         : fp8 ? (T >= 4096 ? 8 : T >= 2048 ? 16 : T >= 1024 ? 4 : T >= 512 ? 2 : 1)
                               : (T >= 4096 ? 8 : T >= 1024 ? 4 : T >= 512 ? 2 : 1);
    while ((tt * K) % 4 != 0) tt *= 2;
    while (tt > 4 && tt * K > kTileThreads) tt -= 4;
    return tt;
}

// Tiles of the fused packed kernels: every tile counts all pairs, so on prefill-sized batches
// 16 tokens per tile for both dtypes (measured on MI355X at T = 4096: bf16 30.5 us against
// 35.9 us with the plain kernels' 8, and 38.3 us with 32).
int pick_tt_packed(int T, int K, bool fp8)
{
    int tt = EP_PACKED_TT ? EP_PACKED_TT : (T >= 2048 ? 16 : pick_tt(T, K, fp8));
    while ((tt * K) % 4 != 0) tt *= 2;
    while (tt > 4 && tt * K > kTileThreads) tt -= 4;
    return tt;
}

// Chunks per lane so that a tile has about one item per wavefront.
int pick_u(int TT, int H8)
{
    const int nseg_target = TT >= kTileWaves ? 1 : kTileWaves / TT;
    const int u = ceil_div(H8, kWave * nseg_target);
    return u >= 4 ? 4 : (u >= 2 ? 2 : 1);
}

template <int U, bool CHUNKED>
hipError_t launch_bf16_u(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                         const LayoutOut &o, u32x4 *recv, int H8, int TT, int nseg,
                         const int32_t *hist, hipStream_t stream)
{
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kTileThreads);
    const int nbits = expert_bits(s.E), lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc);
#define EP_LAUNCH_FUSED_BF16(KG, MULTI)                                                         \
    return launch(layout_dispatch_bf16_kernel<KG, U, MULTI, CHUNKED>, grid, block, lds, stream, \
                  x, idx, o, recv, s.T, H8, s.E, s.C, s.K, s.R, nbits, lg_nc, TT, nseg, hist)
    EP_BY_K(s.K, EP_LAUNCH_FUSED_BF16);
#undef EP_LAUNCH_FUSED_BF16
}

template <int U, bool CHUNKED>
hipError_t launch_fp8_u(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                        const LayoutOut &o, u32x4 *recv_q, float *recv_scale,
                        const int32_t *hist, hipStream_t stream)
{
    const int TT = pick_tt(s.T, s.K, true);
    const int nseg = ceil_div(s.H, U * 16 * kWave);
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kTileThreads);
    const int nbits = expert_bits(s.E), lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc);
#define EP_LAUNCH_FUSED_FP8(KG, MULTI)                                                          \
    return launch(layout_dispatch_fp8_kernel<KG, U, MULTI, CHUNKED>, grid, block, lds, stream,  \
                  x, idx, o, recv_q, recv_scale, s.T, s.H, s.E, s.C, s.K, s.R, nbits, lg_nc,    \
                  TT, nseg, hist)
    EP_BY_K(s.K, EP_LAUNCH_FUSED_FP8);
#undef EP_LAUNCH_FUSED_FP8
}

template <bool CHUNKED>
hipError_t launch_fused_bf16(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                             const LayoutOut &o, uint16_t *recv, const int32_t *hist,
                             hipStream_t stream)
{
    const int H8 = s.H / 8;
    const int TT = pick_tt(s.T, s.K, false);
    const int U = pick_u(TT, H8);
    const int nseg = ceil_div(H8, U * kWave);
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *rv = reinterpret_cast<u32x4 *>(recv);
    if (U >= 4) return launch_bf16_u<4, CHUNKED>(s, xv, idx, o, rv, H8, TT, nseg, hist, stream);
    if (U == 2) return launch_bf16_u<2, CHUNKED>(s, xv, idx, o, rv, H8, TT, nseg, hist, stream);
    return launch_bf16_u<1, CHUNKED>(s, xv, idx, o, rv, H8, TT, nseg, hist, stream);
}

template <bool CHUNKED>
hipError_t launch_fused_fp8(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                            const LayoutOut &o, uint8_t *recv_q, float *recv_scale,
                            const int32_t *hist, hipStream_t stream)
{
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *qv = reinterpret_cast<u32x4 *>(recv_q);
    if (pick_u_fp8(s.T, s.H) == 2)
        return launch_fp8_u<2, CHUNKED>(s, xv, idx, o, qv, recv_scale, hist, stream);
    return launch_fp8_u<1, CHUNKED>(s, xv, idx, o, qv, recv_scale, hist, stream);
}

}  // namespace

hipError_t launch_layout_dispatch_bf16(const ep_shape_t &s, const uint16_t *x,
                                       const int32_t *idx, const LayoutOut &o, uint16_t *recv,
                                       hipStream_t stream)
{
    return launch_fused_bf16<false>(s, x, idx, o, recv, nullptr, stream);
}

hipError_t launch_layout_dispatch_bf16_chunked(const ep_shape_t &s, const uint16_t *x,
                                               const int32_t *idx, const LayoutOut &o,
                                               uint16_t *recv, int32_t *hist,
                                               hipStream_t stream)
{
    if (hipError_t e = launch_layout_chunk_hist(s, idx, hist, stream)) return e;
    return launch_fused_bf16<true>(s, x, idx, o, recv, hist, stream);
}

hipError_t launch_layout_dispatch_fp8_chunked(const ep_shape_t &s, const uint16_t *x,
                                              const int32_t *idx, const LayoutOut &o,
                                              uint8_t *recv_q, float *recv_scale, int32_t *hist,
                                              hipStream_t stream)
{
    if (hipError_t e = launch_layout_chunk_hist(s, idx, hist, stream)) return e;
    return launch_fused_fp8<true>(s, x, idx, o, recv_q, recv_scale, hist, stream);
}

namespace {

template <int U>
hipError_t launch_expand_u(const ep_shape_t &s, const u32x4 *stage, const int32_t *idx,
                           const int32_t *rank_slot, const LayoutOut &o, u32x4 *recv, int H8,
                           int TT, int nseg, hipStream_t stream)
{
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kTileThreads);
    const int nbits = expert_bits(s.E), lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc);
#define EP_LAUNCH_LX(KG, MULTI)                                                                 \
    return launch(layout_expand_bf16_kernel<KG, U, MULTI>, grid, block, lds, stream, stage, idx, \
                  rank_slot, o, recv, s.T, H8, s.E, s.C, s.K, s.R, nbits, lg_nc, TT, nseg)
    EP_BY_K(s.K, EP_LAUNCH_LX);
#undef EP_LAUNCH_LX
}

}  // namespace

hipError_t launch_layout_expand_bf16(const ep_shape_t &s, const uint16_t *stage,
                                     const int32_t *idx, const int32_t *rank_slot,
                                     const LayoutOut &o, uint16_t *recv, hipStream_t stream)
{
    const int H8 = s.H / 8;
    const int TT = pick_tt(s.T, s.K, false);
    if (TT * s.R > kTileThreads) return hipErrorInvalidConfiguration;   // rank_slot rows in LDS
    const int nseg = ceil_div(H8, kWave);
    return launch_expand_u<1>(s, reinterpret_cast<const u32x4 *>(stage), idx, rank_slot, o,
                              reinterpret_cast<u32x4 *>(recv), H8, TT, nseg, stream);
}

hipError_t launch_layout_expand_fp8(const ep_shape_t &s, const uint8_t *stage_q,
                                    const float *stage_scale, const int32_t *idx,
                                    const int32_t *rank_slot, const LayoutOut &o, uint8_t *recv_q,
                                    float *recv_scale, hipStream_t stream)
{
    const int TT = pick_tt(s.T, s.K, false);
    if (TT * s.R > kTileThreads) return hipErrorInvalidConfiguration;   // rank_slot rows in LDS
    const int nseg = ceil_div(s.H, 16 * kWave);
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kTileThreads);
    const int nbits = expert_bits(s.E), lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc);
    const u32x4 *sq = reinterpret_cast<const u32x4 *>(stage_q);
    u32x4 *rq = reinterpret_cast<u32x4 *>(recv_q);
#define EP_LAUNCH_LXQ(KG, MULTI)                                                                \
    return launch(layout_expand_fp8_kernel<KG, MULTI>, grid, block, lds, stream, sq, stage_scale, \
                  idx, rank_slot, o, rq, recv_scale, s.T, s.H, s.E, s.C, s.K, s.R, nbits, lg_nc,  \
                  TT, nseg)
    EP_BY_K(s.K, EP_LAUNCH_LXQ);
#undef EP_LAUNCH_LXQ
}

hipError_t launch_layout_dispatch_fp8(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                                      const LayoutOut &o, uint8_t *recv_q, float *recv_scale,
                                      hipStream_t stream)
{
    return launch_fused_fp8<false>(s, x, idx, o, recv_q, recv_scale, nullptr, stream);
}

// The fused packed kernels hold a second histogram in LDS; beyond this size (E above ~320)
// the packed layout and the packed dispatch run as two launches, with the same results.
constexpr size_t kPackedFusedLds = 64 << 10;

namespace {

template <int U>
hipError_t launch_packed_bf16_u(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                                const LayoutOut &o, int rows_cap, u32x4 *recv, int H8, int TT,
                                int nseg, int lg_nc, size_t lds, hipStream_t stream)
{
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kTileThreads);
    const int nbits = expert_bits(s.E);
#define EP_LAUNCH_PACKED_BF16(KG, MULTI)                                                        \
    return launch(layout_dispatch_packed_bf16_kernel<KG, U, MULTI>, grid, block, lds, stream,   \
                  x, idx, o, recv, s.T, H8, s.E, s.C, s.K, s.R, nbits, lg_nc, TT, nseg,         \
                  rows_cap)
    EP_BY_K(s.K, EP_LAUNCH_PACKED_BF16);
#undef EP_LAUNCH_PACKED_BF16
}

template <int U>
hipError_t launch_packed_fp8_u(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                               const LayoutOut &o, int rows_cap, u32x4 *recv_q,
                               float *recv_scale, int lg_nc, size_t lds, hipStream_t stream)
{
    const int TT = pick_tt_packed(s.T, s.K, true);
    const int nseg = ceil_div(s.H, U * 16 * kWave);
    const dim3 grid(s.T > 0 ? ceil_div(s.T, TT) : 1), block(kTileThreads);
    const int nbits = expert_bits(s.E);
#define EP_LAUNCH_PACKED_FP8(KG, MULTI)                                                         \
    return launch(layout_dispatch_packed_fp8_kernel<KG, U, MULTI>, grid, block, lds, stream,    \
                  x, idx, o, recv_q, recv_scale, s.T, s.H, s.E, s.C, s.K, s.R, nbits, lg_nc,    \
                  TT, nseg, rows_cap)
    EP_BY_K(s.K, EP_LAUNCH_PACKED_FP8);
#undef EP_LAUNCH_PACKED_FP8
}

}  // namespace

hipError_t launch_layout_dispatch_packed_bf16(const ep_shape_t &s, const uint16_t *x,
                                              const int32_t *idx, const LayoutOut &o,
                                              int rows_cap, uint16_t *recv, hipStream_t stream)
{
    const int lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc, true);
    if (lds > kPackedFusedLds) {
        if (hipError_t e = launch_layout(s, idx, o, stream)) return e;
        return launch_dispatch_bf16(s, x, idx, o.slot, recv, stream, RowMap{o.offset, rows_cap});
    }
    const int H8 = s.H / 8;
    const int TT = pick_tt_packed(s.T, s.K, false);
    const int U = pick_u(TT, H8);
    const int nseg = ceil_div(H8, U * kWave);
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *rv = reinterpret_cast<u32x4 *>(recv);
    if (U >= 4)
        return launch_packed_bf16_u<4>(s, xv, idx, o, rows_cap, rv, H8, TT, nseg, lg_nc, lds, stream);
    if (U == 2)
        return launch_packed_bf16_u<2>(s, xv, idx, o, rows_cap, rv, H8, TT, nseg, lg_nc, lds, stream);
    return launch_packed_bf16_u<1>(s, xv, idx, o, rows_cap, rv, H8, TT, nseg, lg_nc, lds, stream);
}

hipError_t launch_layout_dispatch_packed_fp8(const ep_shape_t &s, const uint16_t *x,
                                             const int32_t *idx, const LayoutOut &o,
                                             int rows_cap, uint8_t *recv_q, float *recv_scale,
                                             hipStream_t stream)
{
    const int lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc, true);
    if (lds > kPackedFusedLds) {
        if (hipError_t e = launch_layout(s, idx, o, stream)) return e;
        return launch_dispatch_fp8(s, x, idx, o.slot, recv_q, recv_scale, stream,
                                   RowMap{o.offset, rows_cap});
    }
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *qv = reinterpret_cast<u32x4 *>(recv_q);
    if (pick_u_fp8(s.T, s.H) == 2)
        return launch_packed_fp8_u<2>(s, xv, idx, o, rows_cap, qv, recv_scale, lg_nc, lds, stream);
    return launch_packed_fp8_u<1>(s, xv, idx, o, rows_cap, qv, recv_scale, lg_nc, lds, stream);
}

}  // namespace ep
