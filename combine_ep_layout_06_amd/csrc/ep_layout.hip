// Routing layout on gfx950: per-expert counts, exclusive offsets and stable in-order slots
// under a capacity, with drops. One workgroup of 1024 lanes per tile of 1024 pairs; the
// algorithm is layout_tile / layout_finish (ep_layout_tile.h).
#include "ep_internal.h"
#include "ep_layout_tile.h"

namespace ep {

namespace {

__global__ __launch_bounds__(kTileThreads) void layout_kernel(const int32_t *__restrict__ idx,
                                                               int TK, int E, int C, int R,
                                                               int nbits, LayoutOut o)
{
    __shared__ LayoutLds L;
    const bool last = blockIdx.x == gridDim.x - 1;
    layout_tile(idx, TK, E, C, nbits, blockIdx.x * kTileThreads, kTileThreads, last, L, o.slot,
                nullptr);
    if (last) layout_finish(TK, E, C, R, L, o);
}

}  // namespace

hipError_t launch_layout(const ep_shape_t &s, const int32_t *idx, int32_t *slot, int32_t *count,
                         int32_t *offset, int32_t *rank_count, int32_t *rank_offset,
                         int32_t *stats, hipStream_t stream)
{
    const int TK = s.T * s.K;
    const int tiles = TK > 0 ? (TK + kTileThreads - 1) / kTileThreads : 1;
    const LayoutOut o{slot, count, offset, rank_count, rank_offset, stats};
    return launch(layout_kernel, dim3(tiles), dim3(kTileThreads), 0, stream, idx, TK, s.E, s.C,
                  s.R, expert_bits(s.E), o);
}

}  // namespace ep
