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

}  // namespace

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
