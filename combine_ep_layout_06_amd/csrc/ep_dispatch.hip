// Dispatch on gfx950: scatter each token row to the receive slot of every expert it selected,
// as bf16, or cast once per token to OCP E4M3 with one fp32 scale per 128 channels. The row
// work is dispatch_item_bf16 / dispatch_item_fp8 (ep_dispatch_item.h).
//
// Work split. Tokens are cut into groups of `tpb`; a workgroup of 4 wavefronts takes groups in
// a grid-stride loop. For each group it first stages the receive-row numbers (e*C + slot, or
// offset[e] + slot in a packed buffer, or -1 for a pair that is not kept) of the group's tpb*K
// pairs in LDS with one coalesced pass, so
// no wavefront waits on a dependent global load before its row copy. A wavefront item is one
// token and one segment of its row. HBM traffic: 2*H per token read plus 2*H (bf16) or
// H + 4*H/128 (FP8) per kept pair written.
#include "ep_dispatch_item.h"
#include "ep_internal.h"

#ifndef EP_DISPATCH_U
#define EP_DISPATCH_U 0          // 16-byte chunks per lane per item (0 = choose from the shape)
#endif
#ifndef EP_DISPATCH_TPB
#define EP_DISPATCH_TPB 0        // tokens per group (0 = choose from the shape)
#endif
#ifndef EP_DISPATCH_MAX_BLOCKS
#define EP_DISPATCH_MAX_BLOCKS 0 // grid cap; groups beyond it are taken in a grid-stride loop
#endif

namespace ep {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStage = 256;        // staged pairs per group (tpb * K <= kStage)

// Stage the receive rows of tokens [t0, t0 + nt) into rows[] (one coalesced pass).
__device__ __forceinline__ void stage_rows(int32_t *rows, const int32_t *__restrict__ idx,
                                           const int32_t *__restrict__ slot, int t0, int nt,
                                           int K, int E, int C, const int32_t *poff, int prows)
{
    for (int k = threadIdx.x; k < nt * K; k += kThreads) {
        const size_t i = (size_t)t0 * K + k;
        rows[k] = pair_row(idx[i], slot[i], E, C, poff, prows);
    }
}

template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot, u32x4 *__restrict__ recv, int T, int H8, int E, int C,
    int K, int tpb, int nseg, const int32_t *__restrict__ poff, int prows)
{
    __shared__ int32_t rows[kStage];
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int ntg = (T + tpb - 1) / tpb;
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb;
        const int nt = min(tpb, T - t0);
        __syncthreads();                     // the previous group is done with rows[]
        stage_rows(rows, idx, slot, t0, nt, K, E, C, poff, prows);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg;
            dispatch_item_bf16<KG, U, MULTI>(x, recv, rows, t0 + tl, tl, item - tl * nseg, H8,
                                             K);
        }
    }
}

template <int KG, int U, bool MULTI>
__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot, u32x4 *__restrict__ recv_q,
    float *__restrict__ recv_scale, int T, int H, int E, int C, int K, int tpb, int nseg,
    const int32_t *__restrict__ poff, int prows)
{
    __shared__ int32_t rows[kStage];
    const int wave = wave_uniform(threadIdx.x / kWave);
    const int ntg = (T + tpb - 1) / tpb;
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb;
        const int nt = min(tpb, T - t0);
        __syncthreads();
        stage_rows(rows, idx, slot, t0, nt, K, E, C, poff, prows);
        __syncthreads();
        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg;
            dispatch_item_fp8<KG, U, MULTI>(x, recv_q, recv_scale, rows, t0 + tl, tl,
                                            item - tl * nseg, H, K);
        }
    }
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Chunks per lane: the widest item that still leaves at least 4096 wavefront items (measured
// on MI355X: wide items win on prefill-sized batches, one chunk per lane on small ones).
int pick_u(int T, int H8)
{
    if (EP_DISPATCH_U) return EP_DISPATCH_U;
    for (int u : {4, 2})
        if ((long)T * ceil_div(H8, u * kWave) >= 4096) return u;
    return 1;
}

int pick_tpb(int T, int K, int nseg)
{
    int tpb = EP_DISPATCH_TPB ? EP_DISPATCH_TPB : (T >= 2048 ? 2 : 1) * (nseg == 1 ? 2 : 1);
    while (tpb > 1 && tpb * K > kStage) --tpb;
    return tpb;
}

dim3 grid_for(int T, int tpb)
{
    const int groups = ceil_div(T, tpb);
    return dim3(EP_DISPATCH_MAX_BLOCKS ? min(groups, EP_DISPATCH_MAX_BLOCKS) : groups);
}

template <int U>
hipError_t launch_bf16_u(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                         const int32_t *slot, u32x4 *recv, int H8, int tpb, int nseg,
                         hipStream_t stream, RowMap map)
{
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
#define EP_LAUNCH_BF16(KG, MULTI)                                                            \
    return launch(dispatch_bf16_kernel<KG, U, MULTI>, grid, block, 0, stream, x, idx, slot,  \
                  recv, s.T, H8, s.E, s.C, s.K, tpb, nseg, map.offset, map.rows)
    EP_BY_K(s.K, EP_LAUNCH_BF16);
#undef EP_LAUNCH_BF16
}

template <int U>
hipError_t launch_fp8_u(const ep_shape_t &s, const u32x4 *x, const int32_t *idx,
                        const int32_t *slot, u32x4 *recv_q, float *recv_scale, hipStream_t stream,
                        RowMap map)
{
    const int nseg = ceil_div(s.H, U * 16 * kWave);
    const int tpb = pick_tpb(s.T, s.K, nseg);
    const dim3 grid = grid_for(s.T, tpb), block(kThreads);
#define EP_LAUNCH_FP8(KG, MULTI)                                                              \
    return launch(dispatch_fp8_kernel<KG, U, MULTI>, grid, block, 0, stream, x, idx, slot,    \
                  recv_q, recv_scale, s.T, s.H, s.E, s.C, s.K, tpb, nseg, map.offset, map.rows)
    EP_BY_K(s.K, EP_LAUNCH_FP8);
#undef EP_LAUNCH_FP8
}

}  // namespace

hipError_t launch_dispatch_bf16(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                                const int32_t *slot, uint16_t *recv, hipStream_t stream,
                                RowMap map)
{
    if (s.T == 0) return hipSuccess;
    const int H8 = s.H / 8;
    const int U = pick_u(s.T, H8);
    const int nseg = ceil_div(H8, U * kWave);
    const int tpb = pick_tpb(s.T, s.K, nseg);
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *rv = reinterpret_cast<u32x4 *>(recv);
    if (U >= 4) return launch_bf16_u<4>(s, xv, idx, slot, rv, H8, tpb, nseg, stream, map);
    if (U == 2) return launch_bf16_u<2>(s, xv, idx, slot, rv, H8, tpb, nseg, stream, map);
    return launch_bf16_u<1>(s, xv, idx, slot, rv, H8, tpb, nseg, stream, map);
}

hipError_t launch_dispatch_fp8(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                               const int32_t *slot, uint8_t *recv_q, float *recv_scale,
                               hipStream_t stream, RowMap map)
{
    if (s.T == 0) return hipSuccess;
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *qv = reinterpret_cast<u32x4 *>(recv_q);
    if (pick_u_fp8(s.T, s.H) == 2)
        return launch_fp8_u<2>(s, xv, idx, slot, qv, recv_scale, stream, map);
    return launch_fp8_u<1>(s, xv, idx, slot, qv, recv_scale, stream, map);
}

}  // namespace ep
