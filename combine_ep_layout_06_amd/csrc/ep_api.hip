// C ABI of libep_mi355x: argument checks on the host, then the gfx950 kernel launches.
// Every entry point is declared and documented in include/ep.h.
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "ep.h"
#include "ep_internal.h"

#ifndef EP_VERSION_STRING
#define EP_VERSION_STRING "0.1.0"
#endif

namespace ep {

LaunchLog &launch_log()
{
    thread_local LaunchLog log;
    return log;
}

}  // namespace ep

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string &what)
{
    g_last_error = what;
    return code;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape rules common to every call. On failure returns a negative code and records why.
// Every entry point that launches kernels starts here, so this also clears the launch log.
int check_shape(const ep_shape_t *s, const char *fn)
{
    ep::launch_log().n = 0;
    std::string f(fn);
    if (!s) return fail(EP_ERR_INVALID, f + ": shape is NULL");
    if (s->T < 0 || s->H < 1 || s->E < 1 || s->K < 1 || s->C < 1 || s->R < 1)
        return fail(EP_ERR_INVALID, f + ": need T >= 0 and H, E, K, C, R >= 1");
    if (s->E % s->R != 0) return fail(EP_ERR_INVALID, f + ": E must be a multiple of R");
    if ((int64_t)s->T * s->K > INT32_MAX) return fail(EP_ERR_INVALID, f + ": T*K exceeds INT32_MAX");
    if ((int64_t)s->E * s->C > INT32_MAX) return fail(EP_ERR_INVALID, f + ": E*C exceeds INT32_MAX");
    return EP_OK;
}

// Limits of the dispatch and combine kernels: 16-byte rows, and the K pairs of a token staged
// in one workgroup's LDS.
int check_rows(const ep_shape_t *s, const char *fn, int h_multiple)
{
    if (s->H % h_multiple != 0)
        return fail(EP_ERR_UNSUPPORTED, std::string(fn) + ": H must be a multiple of " +
                                            std::to_string(h_multiple));
    if (s->K > EP_MAX_TOPK)
        return fail(EP_ERR_UNSUPPORTED, std::string(fn) + ": K exceeds EP_MAX_TOPK");
    return EP_OK;
}

int hip_status(hipError_t e, const char *fn)
{
    if (e == hipSuccess) {
        g_last_error.clear();
        return EP_OK;
    }
    return fail(EP_ERR_HIP, std::string(fn) + ": " + hipGetErrorName(e) + ": " + hipGetErrorString(e));
}

// Checks shared by every call that computes the layout.
int check_layout_args(const ep_shape_t *shape, const int32_t *topk_idx, const int32_t *slot,
                      const int32_t *expert_count, const int32_t *expert_offset,
                      const int32_t *stats, const char *fn)
{
    const std::string f(fn);
    if (int rc = check_shape(shape, fn)) return rc;
    if (shape->E > EP_MAX_EXPERTS) return fail(EP_ERR_UNSUPPORTED, f + ": E exceeds EP_MAX_EXPERTS");
    const bool empty = (int64_t)shape->T * shape->K == 0;
    if ((!empty && (!topk_idx || !slot)) || !expert_count || !expert_offset || !stats)
        return fail(EP_ERR_INVALID, f + ": NULL required pointer");
    if (!aligned(topk_idx, 16))
        return fail(EP_ERR_ALIGN, f + ": topk_idx must be 16-byte aligned");
    return EP_OK;
}

// Limits of the two-stage calls: ranks as 64-bit sets, staging rows r*T + p in int32, expert
// ids below EP_MAX_EXPERTS (the rank of an id is found by a multiply exact up to there).
int check_ranks(const ep_shape_t *s, const char *fn)
{
    if (s->R > EP_MAX_RANKS)
        return fail(EP_ERR_UNSUPPORTED, std::string(fn) + ": R exceeds EP_MAX_RANKS");
    if (s->E > EP_MAX_EXPERTS)
        return fail(EP_ERR_UNSUPPORTED, std::string(fn) + ": E exceeds EP_MAX_EXPERTS");
    if ((int64_t)s->R * s->T > INT32_MAX)
        return fail(EP_ERR_UNSUPPORTED, std::string(fn) + ": R*T exceeds INT32_MAX");
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout(const ep_shape_t *shape, const int32_t *topk_idx, int32_t *slot,
              int32_t *expert_count, int32_t *expert_offset, int32_t *rank_count,
              int32_t *rank_offset, int32_t *stats, hipStream_t stream)
{
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats,
                                   "ep_layout"))
        return rc;
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout(*shape, topk_idx, o, stream), "ep_layout");
}

int ep_layout_dispatch(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                       int32_t *slot, int32_t *expert_count, int32_t *expert_offset,
                       int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                       uint16_t *recv, hipStream_t stream)
{
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats,
                                   "ep_layout_dispatch"))
        return rc;
    if (int rc = check_rows(shape, "ep_layout_dispatch", 8)) return rc;
    if (shape->T > 0 && (!x || !recv))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch: x and recv must be 16-byte aligned");
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout_dispatch_bf16(*shape, x, topk_idx, o, recv, stream),
                      "ep_layout_dispatch");
}

int ep_layout_dispatch_fp8(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                           int32_t *slot, int32_t *expert_count, int32_t *expert_offset,
                           int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                           uint8_t *recv_q, float *recv_scale, hipStream_t stream)
{
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats,
                                   "ep_layout_dispatch_fp8"))
        return rc;
    if (int rc = check_rows(shape, "ep_layout_dispatch_fp8", EP_FP8_BLOCK)) return rc;
    if (shape->T > 0 && (!x || !recv_q || !recv_scale))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_fp8: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv_q, 16) || !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_fp8: x and recv_q must be 16-byte aligned, "
                                  "recv_scale 4-byte aligned");
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout_dispatch_fp8(*shape, x, topk_idx, o, recv_q, recv_scale,
                                                     stream),
                      "ep_layout_dispatch_fp8");
}

namespace {

// The static scratch of ep_layout_dispatch_noalloc: device memory of the library itself, one
// copy per GPU, held until the process ends. In host code `scratch` is only a stand-in for the
// symbol; its device address on the current GPU comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(1) << 20;
__device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

constexpr int kScratchDevices = 64;
void *g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_status[kScratchDevices];
std::once_flag g_scratch_once[kScratchDevices];

// This device's address of `scratch` (looked up on the first call on the device, with the
// device current).
int scratch_on_current_device(void **ptr, const char *fn)
{
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev)) return hip_status(e, fn);
    if (dev < 0 || dev >= kScratchDevices)
        return fail(EP_ERR_UNSUPPORTED, std::string(fn) + ": device ordinal " +
                                            std::to_string(dev) + " beyond the library's " +
                                            std::to_string(kScratchDevices));
    std::call_once(g_scratch_once[dev], [dev] {
        g_scratch_status[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (g_scratch_status[dev] != hipSuccess) return hip_status(g_scratch_status[dev], fn);
    *ptr = g_scratch_ptr[dev];
    return EP_OK;
}

// The workspace of the chunked layout: present, large enough and 16-byte aligned.
int check_workspace(const ep_shape_t *shape, const void *workspace, size_t workspace_bytes,
                    const char *fn)
{
    const size_t need = ep::layout_workspace_bytes(*shape);
    if (need > 0 && !workspace) return fail(EP_ERR_INVALID, std::string(fn) + ": workspace is NULL");
    if (workspace_bytes < need)
        return fail(EP_ERR_INVALID, std::string(fn) + ": workspace_bytes " +
                                        std::to_string(workspace_bytes) + " below the " +
                                        std::to_string(need) + " this shape needs");
    if (!aligned(workspace, 16))
        return fail(EP_ERR_ALIGN, std::string(fn) + ": workspace must be 16-byte aligned");
    return EP_OK;
}

}  // namespace

size_t ep_layout_workspace_bytes(const ep_shape_t *shape)
{
    if (!shape || shape->T < 0 || shape->K < 1 || shape->E < 1 ||
        (int64_t)shape->T * shape->K > INT32_MAX)
        return 0;
    return ep::layout_workspace_bytes(*shape);
}

int ep_layout_dispatch_ws(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                          int32_t *slot, int32_t *expert_count, int32_t *expert_offset,
                          int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                          uint16_t *recv, void *workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_ws";
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats, fn))
        return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (shape->T > 0 && (!x || !recv))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_ws: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_ws: x and recv must be 16-byte aligned");
    if (int rc = check_workspace(shape, workspace, workspace_bytes, fn)) return rc;
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout_dispatch_bf16_chunked(
                          *shape, x, topk_idx, o, recv, static_cast<int32_t *>(workspace), stream),
                      fn);
}

int ep_layout_dispatch_fp8_ws(const ep_shape_t *shape, const uint16_t *x,
                              const int32_t *topk_idx, int32_t *slot, int32_t *expert_count,
                              int32_t *expert_offset, int32_t *rank_count, int32_t *rank_offset,
                              int32_t *stats, uint8_t *recv_q, float *recv_scale,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_fp8_ws";
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats, fn))
        return rc;
    if (int rc = check_rows(shape, fn, EP_FP8_BLOCK)) return rc;
    if (shape->T > 0 && (!x || !recv_q || !recv_scale))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_fp8_ws: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv_q, 16) || !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_fp8_ws: x and recv_q must be 16-byte "
                                  "aligned, recv_scale 4-byte aligned");
    if (int rc = check_workspace(shape, workspace, workspace_bytes, fn)) return rc;
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout_dispatch_fp8_chunked(*shape, x, topk_idx, o, recv_q,
                                                             recv_scale,
                                                             static_cast<int32_t *>(workspace),
                                                             stream),
                      fn);
}

int ep_layout_dispatch_noalloc(const ep_shape_t *shape, const uint16_t *x,
                               const int32_t *topk_idx, int32_t *slot, int32_t *expert_count,
                               int32_t *expert_offset, int32_t *rank_count, int32_t *rank_offset,
                               int32_t *stats, uint16_t *recv, hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_noalloc";
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats, fn))
        return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (shape->T > 0 && (!x || !recv))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_noalloc: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_noalloc: x and recv must be 16-byte aligned");
    const size_t need = ep::layout_workspace_bytes(*shape);
    if (need > kScratchBytes)
        return fail(EP_ERR_UNSUPPORTED, "ep_layout_dispatch_noalloc: this shape needs " +
                                            std::to_string(need) +
                                            " bytes of workspace, more than the library's "
                                            "static scratch of " +
                                            std::to_string(kScratchBytes) +
                                            " (use ep_layout_dispatch_ws)");
    void *ws = nullptr;
    if (int rc = scratch_on_current_device(&ws, fn)) return rc;
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout_dispatch_bf16_chunked(*shape, x, topk_idx, o, recv,
                                                              static_cast<int32_t *>(ws), stream),
                      fn);
}

int ep_dispatch(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                const int32_t *slot, uint16_t *recv, hipStream_t stream)
{
    if (int rc = check_shape(shape, "ep_dispatch")) return rc;
    if (int rc = check_rows(shape, "ep_dispatch", 8)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, "ep_dispatch");
    if (!x || !topk_idx || !slot || !recv)
        return fail(EP_ERR_INVALID, "ep_dispatch: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_dispatch: x and recv must be 16-byte aligned");
    return hip_status(ep::launch_dispatch_bf16(*shape, x, topk_idx, slot, recv, stream),
                      "ep_dispatch");
}

int ep_dispatch_fp8(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                    const int32_t *slot, uint8_t *recv_q, float *recv_scale, hipStream_t stream)
{
    if (int rc = check_shape(shape, "ep_dispatch_fp8")) return rc;
    if (int rc = check_rows(shape, "ep_dispatch_fp8", EP_FP8_BLOCK)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, "ep_dispatch_fp8");
    if (!x || !topk_idx || !slot || !recv_q || !recv_scale)
        return fail(EP_ERR_INVALID, "ep_dispatch_fp8: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv_q, 16) || !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_dispatch_fp8: x and recv_q must be 16-byte aligned, "
                                  "recv_scale 4-byte aligned");
    return hip_status(ep::launch_dispatch_fp8(*shape, x, topk_idx, slot, recv_q, recv_scale,
                                              stream),
                      "ep_dispatch_fp8");
}

int ep_combine(const ep_shape_t *shape, const uint16_t *y, const int32_t *topk_idx,
               const int32_t *slot, const float *topk_w, uint16_t *out, hipStream_t stream)
{
    if (int rc = check_shape(shape, "ep_combine")) return rc;
    if (int rc = check_rows(shape, "ep_combine", 8)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, "ep_combine");
    if (!y || !topk_idx || !slot || !topk_w || !out)
        return fail(EP_ERR_INVALID, "ep_combine: NULL required pointer");
    if (!aligned(y, 16) || !aligned(out, 16))
        return fail(EP_ERR_ALIGN, "ep_combine: y and out must be 16-byte aligned");
    return hip_status(ep::launch_combine(*shape, y, topk_idx, slot, topk_w, out, stream),
                      "ep_combine");
}

int ep_rank_layout(const ep_shape_t *shape, const int32_t *topk_idx, int32_t *rank_slot,
                   int32_t *rank_tokens, hipStream_t stream)
{
    const char *fn = "ep_rank_layout";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if ((shape->T > 0 && (!topk_idx || !rank_slot)) || !rank_tokens)
        return fail(EP_ERR_INVALID, "ep_rank_layout: NULL required pointer");
    if (!aligned(topk_idx, 16) || !aligned(rank_slot, 16))
        return fail(EP_ERR_ALIGN, "ep_rank_layout: topk_idx and rank_slot must be 16-byte aligned");
    return hip_status(ep::launch_rank_layout(*shape, topk_idx, rank_slot, rank_tokens, stream),
                      fn);
}

int ep_dispatch_ranks(const ep_shape_t *shape, const uint16_t *x, const int32_t *rank_slot,
                      uint16_t *stage, hipStream_t stream)
{
    const char *fn = "ep_dispatch_ranks";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!x || !rank_slot || !stage) return fail(EP_ERR_INVALID, "ep_dispatch_ranks: NULL required pointer");
    if (!aligned(x, 16) || !aligned(stage, 16))
        return fail(EP_ERR_ALIGN, "ep_dispatch_ranks: x and stage must be 16-byte aligned");
    return hip_status(ep::launch_dispatch_ranks_bf16(*shape, x, rank_slot, stage, stream), fn);
}

int ep_dispatch_ranks_fp8(const ep_shape_t *shape, const uint16_t *x, const int32_t *rank_slot,
                          uint8_t *stage_q, float *stage_scale, hipStream_t stream)
{
    const char *fn = "ep_dispatch_ranks_fp8";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, EP_FP8_BLOCK)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!x || !rank_slot || !stage_q || !stage_scale)
        return fail(EP_ERR_INVALID, "ep_dispatch_ranks_fp8: NULL required pointer");
    if (!aligned(x, 16) || !aligned(stage_q, 16) || !aligned(stage_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_dispatch_ranks_fp8: x and stage_q must be 16-byte aligned, "
                                  "stage_scale 4-byte aligned");
    return hip_status(ep::launch_dispatch_ranks_fp8(*shape, x, rank_slot, stage_q, stage_scale,
                                                    stream),
                      fn);
}

int ep_rank_layout_dispatch(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                            int32_t *rank_slot, int32_t *rank_tokens, uint16_t *stage,
                            hipStream_t stream)
{
    const char *fn = "ep_rank_layout_dispatch";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if ((shape->T > 0 && (!x || !topk_idx || !rank_slot || !stage)) || !rank_tokens)
        return fail(EP_ERR_INVALID, "ep_rank_layout_dispatch: NULL required pointer");
    if (!aligned(topk_idx, 16) || !aligned(x, 16) || !aligned(stage, 16))
        return fail(EP_ERR_ALIGN, "ep_rank_layout_dispatch: topk_idx, x and stage must be "
                                  "16-byte aligned");
    return hip_status(ep::launch_rank_layout_dispatch_bf16(*shape, x, topk_idx, rank_slot,
                                                           rank_tokens, stage, stream),
                      fn);
}

int ep_rank_layout_dispatch_fp8(const ep_shape_t *shape, const uint16_t *x,
                                const int32_t *topk_idx, int32_t *rank_slot,
                                int32_t *rank_tokens, uint8_t *stage_q, float *stage_scale,
                                hipStream_t stream)
{
    const char *fn = "ep_rank_layout_dispatch_fp8";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, EP_FP8_BLOCK)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if ((shape->T > 0 && (!x || !topk_idx || !rank_slot || !stage_q || !stage_scale)) ||
        !rank_tokens)
        return fail(EP_ERR_INVALID, "ep_rank_layout_dispatch_fp8: NULL required pointer");
    if (!aligned(topk_idx, 16) || !aligned(x, 16) || !aligned(stage_q, 16) ||
        !aligned(stage_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_rank_layout_dispatch_fp8: topk_idx, x and stage_q must be "
                                  "16-byte aligned, stage_scale 4-byte aligned");
    return hip_status(ep::launch_rank_layout_dispatch_fp8(*shape, x, topk_idx, rank_slot,
                                                          rank_tokens, stage_q, stage_scale,
                                                          stream),
                      fn);
}

int ep_dispatch_expand(const ep_shape_t *shape, const uint16_t *stage, const int32_t *topk_idx,
                       const int32_t *slot, const int32_t *rank_slot, uint16_t *recv,
                       hipStream_t stream)
{
    const char *fn = "ep_dispatch_expand";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!stage || !topk_idx || !slot || !rank_slot || !recv)
        return fail(EP_ERR_INVALID, "ep_dispatch_expand: NULL required pointer");
    if (!aligned(stage, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_dispatch_expand: stage and recv must be 16-byte aligned");
    return hip_status(ep::launch_dispatch_expand_bf16(*shape, stage, topk_idx, slot, rank_slot,
                                                      recv, stream),
                      fn);
}

int ep_layout_dispatch_expand(const ep_shape_t *shape, const uint16_t *stage,
                              const int32_t *topk_idx, const int32_t *rank_slot, int32_t *slot,
                              int32_t *expert_count, int32_t *expert_offset, int32_t *rank_count,
                              int32_t *rank_offset, int32_t *stats, uint16_t *recv,
                              hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_expand";
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats, fn))
        return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T > 0 && (!stage || !rank_slot || !recv))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_expand: NULL required pointer");
    if (!aligned(stage, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN,
                    "ep_layout_dispatch_expand: stage and recv must be 16-byte aligned");
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(
        ep::launch_layout_expand_bf16(*shape, stage, topk_idx, rank_slot, o, recv, stream), fn);
}

int ep_layout_dispatch_expand_fp8(const ep_shape_t *shape, const uint8_t *stage_q,
                                  const float *stage_scale, const int32_t *topk_idx,
                                  const int32_t *rank_slot, int32_t *slot, int32_t *expert_count,
                                  int32_t *expert_offset, int32_t *rank_count,
                                  int32_t *rank_offset, int32_t *stats, uint8_t *recv_q,
                                  float *recv_scale, hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_expand_fp8";
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, expert_offset, stats, fn))
        return rc;
    if (int rc = check_rows(shape, fn, EP_FP8_BLOCK)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T > 0 && (!stage_q || !stage_scale || !rank_slot || !recv_q || !recv_scale))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_expand_fp8: NULL required pointer");
    if (!aligned(stage_q, 16) || !aligned(recv_q, 16) || !aligned(stage_scale, 4) ||
        !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_expand_fp8: stage_q and recv_q must be "
                                  "16-byte aligned, the scales 4-byte aligned");
    const ep::LayoutOut o{slot, expert_count, expert_offset, rank_count, rank_offset, stats};
    return hip_status(ep::launch_layout_expand_fp8(*shape, stage_q, stage_scale, topk_idx,
                                                   rank_slot, o, recv_q, recv_scale, stream),
                      fn);
}

int ep_dispatch_expand_fp8(const ep_shape_t *shape, const uint8_t *stage_q,
                           const float *stage_scale, const int32_t *topk_idx,
                           const int32_t *slot, const int32_t *rank_slot, uint8_t *recv_q,
                           float *recv_scale, hipStream_t stream)
{
    const char *fn = "ep_dispatch_expand_fp8";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, EP_FP8_BLOCK)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!stage_q || !stage_scale || !topk_idx || !slot || !rank_slot || !recv_q || !recv_scale)
        return fail(EP_ERR_INVALID, "ep_dispatch_expand_fp8: NULL required pointer");
    if (!aligned(stage_q, 16) || !aligned(recv_q, 16) || !aligned(stage_scale, 4) ||
        !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_dispatch_expand_fp8: stage_q and recv_q must be 16-byte "
                                  "aligned, the scale buffers 4-byte aligned");
    return hip_status(ep::launch_dispatch_expand_fp8(*shape, stage_q, stage_scale, topk_idx, slot,
                                                     rank_slot, recv_q, recv_scale, stream),
                      fn);
}

int ep_combine_ranks(const ep_shape_t *shape, const uint16_t *y, const int32_t *topk_idx,
                     const int32_t *slot, const int32_t *rank_slot, const float *topk_w,
                     uint16_t *part, hipStream_t stream)
{
    const char *fn = "ep_combine_ranks";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!y || !topk_idx || !slot || !rank_slot || !topk_w || !part)
        return fail(EP_ERR_INVALID, "ep_combine_ranks: NULL required pointer");
    if (!aligned(y, 16) || !aligned(part, 16))
        return fail(EP_ERR_ALIGN, "ep_combine_ranks: y and part must be 16-byte aligned");
    return hip_status(ep::launch_combine_ranks(*shape, y, topk_idx, slot, rank_slot, topk_w,
                                               part, stream),
                      fn);
}

int ep_combine_reduce(const ep_shape_t *shape, const uint16_t *part, const int32_t *rank_slot,
                      uint16_t *out, hipStream_t stream)
{
    const char *fn = "ep_combine_reduce";
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, 8)) return rc;
    if (int rc = check_ranks(shape, fn)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!part || !rank_slot || !out)
        return fail(EP_ERR_INVALID, "ep_combine_reduce: NULL required pointer");
    if (!aligned(part, 16) || !aligned(out, 16))
        return fail(EP_ERR_ALIGN, "ep_combine_reduce: part and out must be 16-byte aligned");
    return hip_status(ep::launch_combine_reduce(*shape, part, rank_slot, out, stream), fn);
}

int ep_layout_packed(const ep_shape_t *shape, int32_t alignment, const int32_t *topk_idx,
                     int32_t *slot, int32_t *expert_count, int32_t *packed_offset,
                     int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                     hipStream_t stream)
{
    const char *fn = "ep_layout_packed";
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, packed_offset, stats, fn))
        return rc;
    if (alignment < 1) return fail(EP_ERR_INVALID, "ep_layout_packed: alignment must be >= 1");
    if ((int64_t)shape->E * ((int64_t)shape->C + alignment - 1) > INT32_MAX)
        return fail(EP_ERR_UNSUPPORTED, "ep_layout_packed: E*(C + alignment - 1) exceeds INT32_MAX");
    ep::LayoutOut o{slot, expert_count, packed_offset, rank_count, rank_offset, stats};
    o.offset_end = packed_offset + shape->E;
    o.align = alignment;
    return hip_status(ep::launch_layout(*shape, topk_idx, o, stream), fn);
}

namespace {

int check_packed(const ep_shape_t *shape, int32_t rows, const int32_t *packed_offset,
                 const char *fn, int h_multiple)
{
    if (int rc = check_shape(shape, fn)) return rc;
    if (int rc = check_rows(shape, fn, h_multiple)) return rc;
    if (rows < 0) return fail(EP_ERR_INVALID, std::string(fn) + ": rows must be >= 0");
    if (shape->T > 0 && !packed_offset)
        return fail(EP_ERR_INVALID, std::string(fn) + ": NULL required pointer");
    return EP_OK;
}

}  // namespace

namespace {

// ep_layout_dispatch_packed[_fp8]: the checks of ep_layout_packed and ep_dispatch_packed[_fp8].
int check_layout_dispatch_packed(const ep_shape_t *shape, int32_t alignment, int32_t rows,
                                 const uint16_t *x, const int32_t *topk_idx, const int32_t *slot,
                                 const int32_t *expert_count, const int32_t *packed_offset,
                                 const int32_t *stats, const char *fn, int h_multiple)
{
    const std::string f(fn);
    if (int rc = check_layout_args(shape, topk_idx, slot, expert_count, packed_offset, stats, fn))
        return rc;
    if (int rc = check_rows(shape, fn, h_multiple)) return rc;
    if (alignment < 1) return fail(EP_ERR_INVALID, f + ": alignment must be >= 1");
    if ((int64_t)shape->E * ((int64_t)shape->C + alignment - 1) > INT32_MAX)
        return fail(EP_ERR_UNSUPPORTED, f + ": E*(C + alignment - 1) exceeds INT32_MAX");
    if (rows < 0) return fail(EP_ERR_INVALID, f + ": rows must be >= 0");
    if (shape->T > 0 && !x) return fail(EP_ERR_INVALID, f + ": NULL required pointer");
    if (!aligned(x, 16)) return fail(EP_ERR_ALIGN, f + ": x must be 16-byte aligned");
    return EP_OK;
}

}  // namespace

int ep_layout_dispatch_packed(const ep_shape_t *shape, int32_t alignment, int32_t rows,
                              const uint16_t *x, const int32_t *topk_idx, int32_t *slot,
                              int32_t *expert_count, int32_t *packed_offset, int32_t *rank_count,
                              int32_t *rank_offset, int32_t *stats, uint16_t *recv,
                              hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_packed";
    if (int rc = check_layout_dispatch_packed(shape, alignment, rows, x, topk_idx, slot,
                                              expert_count, packed_offset, stats, fn, 8))
        return rc;
    if (shape->T > 0 && !recv) return fail(EP_ERR_INVALID, "ep_layout_dispatch_packed: NULL required pointer");
    if (!aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_packed: recv must be 16-byte aligned");
    ep::LayoutOut o{slot, expert_count, packed_offset, rank_count, rank_offset, stats};
    o.offset_end = packed_offset + shape->E;
    o.align = alignment;
    return hip_status(ep::launch_layout_dispatch_packed_bf16(*shape, x, topk_idx, o, rows, recv,
                                                             stream),
                      fn);
}

int ep_layout_dispatch_packed_fp8(const ep_shape_t *shape, int32_t alignment, int32_t rows,
                                  const uint16_t *x, const int32_t *topk_idx, int32_t *slot,
                                  int32_t *expert_count, int32_t *packed_offset,
                                  int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                                  uint8_t *recv_q, float *recv_scale, hipStream_t stream)
{
    const char *fn = "ep_layout_dispatch_packed_fp8";
    if (int rc = check_layout_dispatch_packed(shape, alignment, rows, x, topk_idx, slot,
                                              expert_count, packed_offset, stats, fn,
                                              EP_FP8_BLOCK))
        return rc;
    if (shape->T > 0 && (!recv_q || !recv_scale))
        return fail(EP_ERR_INVALID, "ep_layout_dispatch_packed_fp8: NULL required pointer");
    if (!aligned(recv_q, 16) || !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_layout_dispatch_packed_fp8: recv_q must be 16-byte aligned, "
                                  "recv_scale 4-byte aligned");
    ep::LayoutOut o{slot, expert_count, packed_offset, rank_count, rank_offset, stats};
    o.offset_end = packed_offset + shape->E;
    o.align = alignment;
    return hip_status(ep::launch_layout_dispatch_packed_fp8(*shape, x, topk_idx, o, rows, recv_q,
                                                            recv_scale, stream),
                      fn);
}

int ep_dispatch_packed(const ep_shape_t *shape, int32_t rows, const uint16_t *x,
                       const int32_t *topk_idx, const int32_t *slot,
                       const int32_t *packed_offset, uint16_t *recv, hipStream_t stream)
{
    const char *fn = "ep_dispatch_packed";
    if (int rc = check_packed(shape, rows, packed_offset, fn, 8)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!x || !topk_idx || !slot || !recv) return fail(EP_ERR_INVALID, "ep_dispatch_packed: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv, 16))
        return fail(EP_ERR_ALIGN, "ep_dispatch_packed: x and recv must be 16-byte aligned");
    return hip_status(ep::launch_dispatch_bf16(*shape, x, topk_idx, slot, recv, stream,
                                               ep::RowMap{packed_offset, rows}),
                      fn);
}

int ep_dispatch_packed_fp8(const ep_shape_t *shape, int32_t rows, const uint16_t *x,
                           const int32_t *topk_idx, const int32_t *slot,
                           const int32_t *packed_offset, uint8_t *recv_q, float *recv_scale,
                           hipStream_t stream)
{
    const char *fn = "ep_dispatch_packed_fp8";
    if (int rc = check_packed(shape, rows, packed_offset, fn, EP_FP8_BLOCK)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!x || !topk_idx || !slot || !recv_q || !recv_scale)
        return fail(EP_ERR_INVALID, "ep_dispatch_packed_fp8: NULL required pointer");
    if (!aligned(x, 16) || !aligned(recv_q, 16) || !aligned(recv_scale, 4))
        return fail(EP_ERR_ALIGN, "ep_dispatch_packed_fp8: x and recv_q must be 16-byte aligned, "
                                  "recv_scale 4-byte aligned");
    return hip_status(ep::launch_dispatch_fp8(*shape, x, topk_idx, slot, recv_q, recv_scale,
                                              stream, ep::RowMap{packed_offset, rows}),
                      fn);
}

int ep_combine_packed(const ep_shape_t *shape, int32_t rows, const uint16_t *y,
                      const int32_t *topk_idx, const int32_t *slot, const int32_t *packed_offset,
                      const float *topk_w, uint16_t *out, hipStream_t stream)
{
    const char *fn = "ep_combine_packed";
    if (int rc = check_packed(shape, rows, packed_offset, fn, 8)) return rc;
    if (shape->T == 0) return hip_status(hipSuccess, fn);
    if (!y || !topk_idx || !slot || !topk_w || !out)
        return fail(EP_ERR_INVALID, "ep_combine_packed: NULL required pointer");
    if (!aligned(y, 16) || !aligned(out, 16))
        return fail(EP_ERR_ALIGN, "ep_combine_packed: y and out must be 16-byte aligned");
    return hip_status(ep::launch_combine(*shape, y, topk_idx, slot, topk_w, out, stream,
                                         ep::RowMap{packed_offset, rows}),
                      fn);
}

int ep_check_e4m3_conversion(uint32_t first_pattern, uint32_t count, uint32_t *mismatches,
                             uint32_t *first_mismatch, hipStream_t stream)
{
    ep::launch_log().n = 0;
    if (!mismatches || !first_mismatch)
        return fail(EP_ERR_INVALID, "ep_check_e4m3_conversion: NULL required pointer");
    if ((uint64_t)first_pattern + count > (1ull << 32))
        return fail(EP_ERR_INVALID,
                    "ep_check_e4m3_conversion: first_pattern + count exceeds 2^32");
    if (!aligned(mismatches, 4) || !aligned(first_mismatch, 4))
        return fail(EP_ERR_ALIGN, "ep_check_e4m3_conversion: outputs must be 4-byte aligned");
    return hip_status(ep::launch_check_e4m3(first_pattern, count, mismatches, first_mismatch,
                                            stream),
                      "ep_check_e4m3_conversion");
}

int ep_last_launches(ep_launch_record_t *records, int capacity)
{
    const ep::LaunchLog &log = ep::launch_log();
    const int n = log.n < ep::kLaunchLogCap ? log.n : ep::kLaunchLogCap;
    for (int k = 0; records && k < n && k < capacity; ++k) {
        const ep::LaunchEntry &e = log.e[k];
        ep_launch_record_t &r = records[k];
        const char *name = hipKernelNameRefByPtr(e.kernel, nullptr);
        r.kernel = name ? name : "";
        r.grid_x = e.grid.x;
        r.grid_y = e.grid.y;
        r.grid_z = e.grid.z;
        r.block_x = e.block.x;
        r.block_y = e.block.y;
        r.block_z = e.block.z;
        r.dynamic_lds_bytes = (uint32_t)e.shmem;
        hipFuncAttributes a{};
        if (hipFuncGetAttributes(&a, e.kernel) == hipSuccess) {
            r.static_lds_bytes = (uint32_t)a.sharedSizeBytes;
            r.vgprs = a.numRegs;
            r.private_bytes = (uint32_t)a.localSizeBytes;
            r.max_threads_per_block = a.maxThreadsPerBlock;
        } else {
            r.static_lds_bytes = 0;
            r.vgprs = -1;
            r.private_bytes = 0;
            r.max_threads_per_block = -1;
        }
    }
    return log.n;
}

const char *ep_error_string(int code)
{
    switch (code) {
    case EP_OK: return "EP_OK: success";
    case EP_ERR_INVALID: return "EP_ERR_INVALID: invalid shape or NULL pointer";
    case EP_ERR_ALIGN: return "EP_ERR_ALIGN: buffer not aligned";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED: shape not supported by the kernels";
    case EP_ERR_HIP: return "EP_ERR_HIP: HIP runtime error";
    default: return "unknown ep error code";
    }
}

const char *ep_last_error(void) { return g_last_error.c_str(); }

const char *ep_version(void)
{
    static const std::string v = [] {
        char buf[96];
        snprintf(buf, sizeof buf, "libep_mi355x %s (gfx950; HIP %d.%d.%d)", EP_VERSION_STRING,
                 HIP_VERSION_MAJOR, HIP_VERSION_MINOR, HIP_VERSION_PATCH);
        return std::string(buf);
    }();
    return v.c_str();
}

}  // extern "C"
