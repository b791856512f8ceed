// Routing layout on gfx950: per-expert counts, exclusive offsets and stable in-order slots
// under a capacity, with drops. One workgroup of 1024 lanes per tile of 1024 pairs; the
// algorithm is layout_tile / layout_finish (ep_layout_tile.h).
#include "ep_internal.h"
#include "ep_layout_tile.h"

namespace ep {

namespace {

template <bool PACKED>
__global__ __launch_bounds__(kTileThreads) void layout_kernel(const int32_t *__restrict__ idx,
                                                               int TK, int E, int C, int R,
                                                               int nbits, int lg_nc,
                                                               LayoutOut o)
{
    extern __shared__ __align__(16) int32_t lds[];
    const LayoutLdsMap m = layout_lds_map(E, lg_nc);
    const bool last = blockIdx.x == gridDim.x - 1;
    const int tile_begin = blockIdx.x * kTileThreads;
    const TileIds ids = layout_tile_loads(idx, TK, tile_begin, kTileThreads);
    layout_tile(ids, idx, TK, E, C, nbits, tile_begin, kTileThreads, last, lds, m, o.slot,
                nullptr);
    if (last) layout_finish<PACKED>(TK, E, C, R, lds, m, o);
}

// Histogram of each chunk of kLayoutChunk pairs: hist[c][b] = pairs of chunk c in bin b (the
// E experts, then invalid, then unrouted), B = E + 2 words per chunk. One workgroup per chunk,
// one 16-byte vector of ids per lane (the last, partial vector one id at a time).
__global__ __launch_bounds__(kTileThreads) void layout_chunk_hist_kernel(
    const int32_t *__restrict__ idx, int TK, int E, int32_t *__restrict__ hist)
{
    __shared__ int32_t h[EP_MAX_EXPERTS + 2];
    const int tid = threadIdx.x, B = E + 2;
    for (int k = tid; k < B; k += kTileThreads) h[k] = 0;
    const int64_t p = (int64_t)blockIdx.x * kLayoutChunk + 4 * tid;   // kLayoutChunk = 4 * 1024
    int4 v = int4{-1, -1, -1, -1};
    if (p + 3 < TK) {
        v = reinterpret_cast<const int4 *>(idx)[p / 4];
    } else if (p < TK) {
        v.x = idx[p];
        if (p + 1 < TK) v.y = idx[p + 1];
        if (p + 2 < TK) v.z = idx[p + 2];
    }
    __syncthreads();
    const int64_t n = TK - p < 4 ? TK - p : 4;
    const int e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (c < n) atomicAdd(&h[layout_bin(e4[c], E)], 1);
    __syncthreads();
    for (int k = tid; k < B; k += kTileThreads) hist[(size_t)blockIdx.x * B + k] = h[k];
}

}  // namespace

size_t layout_workspace_bytes(const ep_shape_t &s)
{
    const int64_t TK = (int64_t)s.T * s.K;
    return (size_t)layout_chunks((int)TK) * (size_t)(s.E + 2) * sizeof(int32_t);
}

hipError_t launch_layout_chunk_hist(const ep_shape_t &s, const int32_t *idx, int32_t *hist,
                                    hipStream_t stream)
{
    const int TK = s.T * s.K;
    if (TK == 0) return hipSuccess;
    return launch(layout_chunk_hist_kernel, dim3(layout_chunks(TK)), dim3(kTileThreads), 0,
                  stream, idx, TK, s.E, hist);
}

hipError_t launch_layout(const ep_shape_t &s, const int32_t *idx, const LayoutOut &o,
                         hipStream_t stream)
{
    const int TK = s.T * s.K;
    const int tiles = TK > 0 ? (TK + kTileThreads - 1) / kTileThreads : 1;
    const int lg_nc = layout_lg_nc(s.E);
    const size_t lds = layout_lds_bytes(s.E, lg_nc);
    if (o.offset_end)           // packed: counts rounded up to o.align, total rows written
        return launch(layout_kernel<true>, dim3(tiles), dim3(kTileThreads), lds, stream, idx,
                      TK, s.E, s.C, s.R, expert_bits(s.E), lg_nc, o);
    return launch(layout_kernel<false>, dim3(tiles), dim3(kTileThreads), lds, stream, idx, TK,
                  s.E, s.C, s.R, expert_bits(s.E), lg_nc, o);
}

}  // namespace ep
