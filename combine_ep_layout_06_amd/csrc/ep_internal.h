// Host-side declarations shared by the kernel launchers and the C ABI (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "ep.h"

namespace ep {

// Launch `kernel` with hipLaunchKernel, which returns the launch status itself (so an error
// left behind by an unrelated earlier call is neither reported nor cleared). Arguments are
// converted to the kernel's parameter types first.
template <typename... KArgs, size_t... I>
inline void fill_argv(void **argv, std::tuple<KArgs...> &t, std::index_sequence<I...>)
{
    ((argv[I] = static_cast<void *>(&std::get<I>(t))), ...);
}

// The launches of the calling thread's most recent entry-point call (ep_last_launches): the
// argument checks of each call clear it, and launch() appends to it.
struct LaunchEntry {
    const void *kernel;
    dim3 grid, block;
    size_t shmem;
};
constexpr int kLaunchLogCap = 8;
struct LaunchLog {
    int n = 0;
    LaunchEntry e[kLaunchLogCap];
};
LaunchLog &launch_log();

template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    LaunchLog &log = launch_log();
    if (log.n < kLaunchLogCap)
        log.e[log.n] = LaunchEntry{reinterpret_cast<const void *>(kernel), grid, block, shmem};
    ++log.n;
    std::tuple<KArgs...> typed(static_cast<KArgs>(args)...);
    void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    fill_argv(argv, typed, std::index_sequence_for<KArgs...>{});
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, shmem,
                           stream);
}

// Outputs of the layout (see ep_layout in ep.h); rank_count / rank_offset may be null. A
// non-null offset_end asks for the packed layout: the offsets and rank sums are over the counts
// rounded up to multiples of align (>= 1), and offset_end receives the total number of rows.
struct LayoutOut {
    int32_t *slot, *count, *offset, *rank_count, *rank_offset, *stats;
    int32_t *offset_end = nullptr;
    int align = 1;
};

// Where a kept pair's row is: e*C + slot in the padded [E][C] buffer (offset null), or
// offset[e] + slot in a packed buffer of `rows` rows.
struct RowMap {
    const int32_t *offset = nullptr;
    int rows = 0;
};

hipError_t launch_layout(const ep_shape_t &s, const int32_t *idx, const LayoutOut &o,
                         hipStream_t stream);

hipError_t launch_dispatch_bf16(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                                const int32_t *slot, uint16_t *recv, hipStream_t stream,
                                RowMap map = RowMap());

hipError_t launch_dispatch_fp8(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                               const int32_t *slot, uint8_t *recv_q, float *recv_scale,
                               hipStream_t stream, RowMap map = RowMap());

hipError_t launch_layout_dispatch_bf16(const ep_shape_t &s, const uint16_t *x,
                                       const int32_t *idx, const LayoutOut &o, uint16_t *recv,
                                       hipStream_t stream);

hipError_t launch_layout_expand_bf16(const ep_shape_t &s, const uint16_t *stage,
                                     const int32_t *idx, const int32_t *rank_slot,
                                     const LayoutOut &o, uint16_t *recv, hipStream_t stream);

hipError_t launch_layout_expand_fp8(const ep_shape_t &s, const uint8_t *stage_q,
                                    const float *stage_scale, const int32_t *idx,
                                    const int32_t *rank_slot, const LayoutOut &o, uint8_t *recv_q,
                                    float *recv_scale, hipStream_t stream);

hipError_t launch_layout_dispatch_fp8(const ep_shape_t &s, const uint16_t *x, const int32_t *idx,
                                      const LayoutOut &o, uint8_t *recv_q, float *recv_scale,
                                      hipStream_t stream);

// The chunked form (large batches): chunk histograms into `hist` (layout_workspace_bytes:
// one histogram of E + 2 words per 4096 pairs), then the fused kernel reading them. Same
// outputs as the single launch.
size_t layout_workspace_bytes(const ep_shape_t &s);
hipError_t launch_layout_chunk_hist(const ep_shape_t &s, const int32_t *idx, int32_t *hist,
                                    hipStream_t stream);
hipError_t launch_layout_dispatch_bf16_chunked(const ep_shape_t &s, const uint16_t *x,
                                               const int32_t *idx, const LayoutOut &o,
                                               uint16_t *recv, int32_t *hist,
                                               hipStream_t stream);
hipError_t launch_layout_dispatch_fp8_chunked(const ep_shape_t &s, const uint16_t *x,
                                              const int32_t *idx, const LayoutOut &o,
                                              uint8_t *recv_q, float *recv_scale, int32_t *hist,
                                              hipStream_t stream);

hipError_t launch_combine(const ep_shape_t &s, const uint16_t *y, const int32_t *idx,
                          const int32_t *slot, const float *w, uint16_t *out,
                          hipStream_t stream, RowMap map = RowMap());

// two-stage, rank-deduplicated path
hipError_t launch_rank_layout(const ep_shape_t &s, const int32_t *idx, int32_t *rank_slot,
                              int32_t *rank_tokens, hipStream_t stream);

hipError_t launch_layout_dispatch_packed_bf16(const ep_shape_t &s, const uint16_t *x,
                                              const int32_t *idx, const LayoutOut &o,
                                              int rows_cap, uint16_t *recv, hipStream_t stream);
hipError_t launch_layout_dispatch_packed_fp8(const ep_shape_t &s, const uint16_t *x,
                                             const int32_t *idx, const LayoutOut &o,
                                             int rows_cap, uint8_t *recv_q, float *recv_scale,
                                             hipStream_t stream);
hipError_t launch_rank_layout_dispatch_bf16(const ep_shape_t &s, const uint16_t *x,
                                            const int32_t *idx, int32_t *rank_slot,
                                            int32_t *rank_tokens, uint16_t *stage,
                                            hipStream_t stream);
hipError_t launch_rank_layout_dispatch_fp8(const ep_shape_t &s, const uint16_t *x,
                                           const int32_t *idx, int32_t *rank_slot,
                                           int32_t *rank_tokens, uint8_t *stage_q,
                                           float *stage_scale, hipStream_t stream);
hipError_t launch_dispatch_ranks_bf16(const ep_shape_t &s, const uint16_t *x,
                                      const int32_t *rank_slot, uint16_t *stage,
                                      hipStream_t stream);

hipError_t launch_dispatch_ranks_fp8(const ep_shape_t &s, const uint16_t *x,
                                     const int32_t *rank_slot, uint8_t *stage_q,
                                     float *stage_scale, hipStream_t stream);

hipError_t launch_dispatch_expand_bf16(const ep_shape_t &s, const uint16_t *stage,
                                       const int32_t *idx, const int32_t *slot,
                                       const int32_t *rank_slot, uint16_t *recv,
                                       hipStream_t stream);

hipError_t launch_dispatch_expand_fp8(const ep_shape_t &s, const uint8_t *stage_q,
                                      const float *stage_scale, const int32_t *idx,
                                      const int32_t *slot, const int32_t *rank_slot,
                                      uint8_t *recv_q, float *recv_scale, hipStream_t stream);

hipError_t launch_combine_ranks(const ep_shape_t &s, const uint16_t *y, const int32_t *idx,
                                const int32_t *slot, const int32_t *rank_slot, const float *w,
                                uint16_t *part, hipStream_t stream);

hipError_t launch_combine_reduce(const ep_shape_t &s, const uint16_t *part,
                                 const int32_t *rank_slot, uint16_t *out, hipStream_t stream);

// self-check of the E4M3 encoders
hipError_t launch_check_e4m3(uint32_t first_pattern, uint32_t n, uint32_t *count,
                             uint32_t *first, hipStream_t stream);

}  // namespace ep
