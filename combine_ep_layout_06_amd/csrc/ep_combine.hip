// Combine on gfx950: gather each token's kept expert-output rows and form the top-k weighted
// sum in fp32, in ascending j, rounding once to bf16.
//
// Combine reduces the expert outputs with the top-k weights on the token's side (afdEP-comm
// validation record, kernel_timelines: combine_reduce_epilogue), in BF16 whatever the dispatch
// dtype (awsome-distributed-ai PR #1238, review item 1). Traffic: each kept y row is read once
// (2*H), the output row written once (2*H per token).
//
// Work split. Tokens are cut into groups of `tpb`; a workgroup of 4 wavefronts takes groups in
// a grid-stride loop and, for each, stages the receive-row numbers and the weights of the
// group's tpb*K pairs in LDS with one coalesced pass. A wavefront item is one token and one row
// segment; each lane owns U 16-byte chunks (8 bf16 channels each, lane-contiguous, so one load
// instruction covers 1 KiB of a row).
//
// Memory-level parallelism. For a group of KG pairs (KG = K rounded up to a power of two, at
// most 8; whole-row items take groups of 2) the wavefront issues every row load first, as straight-line code (a pair that is not
// kept reads a row of zeros with weight -0, which the fold adds as an exact -0, so no
// per-element select is needed), and only then folds the rows in j order with fmaf. The K row fetches of a token are therefore
// in flight together; a branch around any load would make the compiler wait for earlier
// loads before issuing the next one. Loads of y and stores of out are non-temporal: each byte
// is touched once (non-temporal loads measured ~25% faster here).
//
// Measured on MI355X, this kernel reaches ~95% of a bare probe of the same access pattern
// (eight random 4 KiB rows read per contiguous row written, rows precomputed, the same rows
// re-read after a 2 GiB fill: 22.9 against 24.0 us at T = 4096); a per-wavefront variant that
// prefetched the next token's metadata through scalar loads instead of LDS staging was no
// faster, nor was one wavefront per item with the metadata in lanes and no LDS at all (26.4-
// 26.5 against 26.2-26.6 us in the benchmark, 3.90 against 4.02 us at T = 128), nor a
// wave-uniform branch around each pair's fold in place of the per-element select.
#include "ep_device.h"
#include "ep_internal.h"

#ifndef EP_COMBINE_U
#define EP_COMBINE_U 0          // 16-byte chunks per lane per item (0 = choose from the shape)
#endif
#ifndef EP_COMBINE_TPB
#define EP_COMBINE_TPB 0        // tokens per group (0 = choose from the shape)
#endif
#ifndef EP_COMBINE_MAX_BLOCKS
#define EP_COMBINE_MAX_BLOCKS 0 // grid cap; groups beyond it are taken in a grid-stride loop
#endif
#ifndef EP_COMBINE_NT_LOAD
#define EP_COMBINE_NT_LOAD 1
#endif
#ifndef EP_COMBINE_NT_STORE
#define EP_COMBINE_NT_STORE 1
#endif

namespace ep {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStage = 256;        // staged pairs per group (tpb * K <= kStage)

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A row of zeros that pairs which are not kept read instead of an expert row, with weight -0:
// fmaf(-0, +0, acc) adds an exact -0, which leaves every acc unchanged (+0 and -0 included), so
// the fold needs no per-element select. Never written (zero-initialised at load); rows of up
// to kZeroChunks 16-byte chunks (H <= 32768) use it, longer ones fall back to the select.
constexpr int kZeroChunks = 4096;
__device__ u32x4 g_zero_row[kZeroChunks];

// KG: pairs per group (K <= KG unless MULTI); U: chunks per lane per item; ZROW: H8 <=
// kZeroChunks (pairs that are not kept read the zero row; otherwise a select drops them).
template <int KG, int U, bool MULTI, bool ZROW>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const u32x4 *__restrict__ y, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot, const float *__restrict__ topk_w,
    u32x4 *__restrict__ out, int T, int H8, int E, int C, int K, int tpb, int nseg,
    const int32_t *__restrict__ poff, int prows)
{
    __shared__ int32_t rows[kStage];
    __shared__ float wts[kStage];
    const int wave = uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int ntg = (T + tpb - 1) / tpb;
    for (int tg = blockIdx.x; tg < ntg; tg += gridDim.x) {
        const int t0 = tg * tpb;
        const int nt = min(tpb, T - t0);
        __syncthreads();                     // the previous group is done with rows[] / wts[]
        for (int k = threadIdx.x; k < nt * K; k += kThreads) {
            const size_t i = (size_t)t0 * K + k;
            rows[k] = pair_row(idx[i], slot[i], E, C, poff, prows);
            wts[k] = topk_w[i];
        }
        __syncthreads();

        for (int item = wave; item < nt * nseg; item += kWaves) {
            const int tl = item / nseg;
            const int seg = item - tl * nseg;
            int cidx[U];      // chunk of the row this lane reads (clamped) and whether it is real
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
                for (int k = 0; k < 8; ++k) acc[u][k] = 0.0f;

            const int npg = MULTI ? (K + KG - 1) / KG : 1;
            for (int pg = 0; pg < npg; ++pg) {
                int r[KG];
                float wj[KG];
                u32x4 v[KG][U];
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const int j = pg * KG + g;
                    const int k = tl * K + (j < K ? j : K - 1);
                    const int rr = uniform(rows[k]);
                    r[g] = j < K ? rr : -1;
                    wj[g] = __int_as_float(uniform(__float_as_int(wts[k])));
                    const u32x4 *src;
                    if constexpr (ZROW) {
                        src = r[g] >= 0 ? y + (size_t)r[g] * H8 : g_zero_row;
                        wj[g] = r[g] >= 0 ? wj[g] : -0.0f;
                    } else {
                        src = y + (size_t)(r[g] >= 0 ? r[g] : 0) * H8;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[g][u] = load16<EP_COMBINE_NT_LOAD>(src + cidx[u]);
                }
                // keep the scheduler from pulling any use of a row above the last row load
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const bool keep = ZROW || r[g] >= 0;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t wd[4] = {v[g][u].x, v[g][u].y, v[g][u].z, v[g][u].w};
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float lo = __builtin_fmaf(wj[g], bf16_lo(wd[k]), acc[u][2 * k]);
                            const float hi =
                                __builtin_fmaf(wj[g], bf16_hi(wd[k]), acc[u][2 * k + 1]);
                            acc[u][2 * k] = keep ? lo : acc[u][2 * k];
                            acc[u][2 * k + 1] = keep ? hi : acc[u][2 * k + 1];
                        }
                    }
                }
            }
            u32x4 *dst = out + (size_t)(t0 + tl) * H8;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!cok[u]) continue;
                u32x4 o;
                o.x = bf16_rne(acc[u][0]) | (bf16_rne(acc[u][1]) << 16);
                o.y = bf16_rne(acc[u][2]) | (bf16_rne(acc[u][3]) << 16);
                o.z = bf16_rne(acc[u][4]) | (bf16_rne(acc[u][5]) << 16);
                o.w = bf16_rne(acc[u][6]) | (bf16_rne(acc[u][7]) << 16);
                store16<EP_COMBINE_NT_STORE>(dst + cidx[u], o);
            }
        }
    }
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Chunks per lane and tokens per group, as measured on MI355X: four chunks per lane and four
// tokens per group on prefill-sized batches, one and one on small ones.
int pick_u(int T, int H8)
{
    if (EP_COMBINE_U) return EP_COMBINE_U;
    if ((long)T * ceil_div(H8, 4 * kWave) >= 4096) return 4;
    if ((long)T * ceil_div(H8, 2 * kWave) >= 4096) return 2;
    return 1;
}

int pick_tpb(int T, int K)
{
    int tpb = EP_COMBINE_TPB ? EP_COMBINE_TPB : (T >= 2048 ? 4 : 1);
    while (tpb > 1 && tpb * K > kStage) --tpb;
    return tpb;
}

template <int U>
hipError_t launch_u(const ep_shape_t &s, const u32x4 *y, const int32_t *idx, const int32_t *slot,
                    const float *w, u32x4 *out, int H8, int tpb, int nseg, hipStream_t stream,
                    RowMap map)
{
    const int groups = ceil_div(s.T, tpb);
    const dim3 grid(EP_COMBINE_MAX_BLOCKS ? min(groups, EP_COMBINE_MAX_BLOCKS) : groups);
    const dim3 block(kThreads);
#define EP_COMBINE_LAUNCH(KG, MULTI)                                                            \
    return H8 <= kZeroChunks                                                                    \
               ? launch(combine_kernel<KG, U, MULTI, true>, grid, block, 0, stream, y, idx,     \
                        slot, w, out, s.T, H8, s.E, s.C, s.K, tpb, nseg, map.offset, map.rows) \
               : launch(combine_kernel<KG, U, MULTI, false>, grid, block, 0, stream, y, idx,    \
                        slot, w, out, s.T, H8, s.E, s.C, s.K, tpb, nseg, map.offset, map.rows)
    if (s.K > 8) EP_COMBINE_LAUNCH(8, true);
    if (s.K > 4) {
        // whole-row items (U = 4) fold their rows in groups of two: that build holds 82 VGPRs,
        // so 5 wavefronts per SIMD fit (at T = 4096: 26.5 us, against 26.8 with groups of four
        // at 114 VGPRs, 26.6 with single rows and 27.1 with one group of eight at 162);
        // narrower items keep one group of eight rows in flight, which is faster at decode
        // size (4.0 against 4.4 us at T = 128 with groups of four)
        if constexpr (U >= 4) EP_COMBINE_LAUNCH(2, true);
        else EP_COMBINE_LAUNCH(8, false);
    }
    if (s.K > 2) EP_COMBINE_LAUNCH(4, false);
    if (s.K > 1) EP_COMBINE_LAUNCH(2, false);
    EP_COMBINE_LAUNCH(1, false);
#undef EP_COMBINE_LAUNCH
}

}  // namespace

hipError_t launch_combine(const ep_shape_t &s, const uint16_t *y, const int32_t *idx,
                          const int32_t *slot, const float *w, uint16_t *out, hipStream_t stream,
                          RowMap map)
{
    if (s.T == 0) return hipSuccess;
    const int H8 = s.H / 8;
    const int U = pick_u(s.T, H8);
    const int nseg = ceil_div(H8, U * kWave);
    const int tpb = pick_tpb(s.T, s.K);
    const u32x4 *yv = reinterpret_cast<const u32x4 *>(y);
    u32x4 *ov = reinterpret_cast<u32x4 *>(out);
    if (U >= 4) return launch_u<4>(s, yv, idx, slot, w, ov, H8, tpb, nseg, stream, map);
    if (U == 2) return launch_u<2>(s, yv, idx, slot, w, ov, H8, tpb, nseg, stream, map);
    return launch_u<1>(s, yv, idx, slot, w, ov, H8, tpb, nseg, stream, map);
}

}  // namespace ep
