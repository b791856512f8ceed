// Self-check of the E4M3 encoders the FP8 dispatch uses, on the device it runs on.
//
// The FP8 fast path encodes its quotients with gfx950's packed conversion instruction
// (e4m3_pack4); the plain path and the definition use round-to-nearest-even with saturation
// (e4m3_rne_sat). The fast path is only sound if the two agree on every value it can pass:
// every quotient x / scale is at most 448 (1 + 2^-22) in magnitude. ep_check_e4m3_conversion
// compares the two over any range of fp32 bit patterns, so a test can cover that whole set.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kCheckThreads = 256;

__global__ void e4m3_check_init(uint32_t *count, uint32_t *first)
{
    *count = 0u;
    *first = 0xFFFFFFFFu;
}

// Patterns first_pattern + i for i in [0, n): four per lane per step (one packed conversion),
// the software encoder on each; a lane adds its mismatches once at the end.
__global__ __launch_bounds__(kCheckThreads) void e4m3_check_kernel(uint32_t first_pattern,
                                                                   uint64_t n, uint32_t *count,
                                                                   uint32_t *first)
{
    const uint64_t stride = (uint64_t)gridDim.x * kCheckThreads * 4;
    uint32_t nbad = 0, fbad = 0xFFFFFFFFu;
    for (uint64_t i = ((uint64_t)blockIdx.x * kCheckThreads + threadIdx.x) * 4; i < n;
         i += stride) {
        uint32_t u[4];
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t j = i + k < n ? i + k : n - 1;
            u[k] = first_pattern + (uint32_t)j;
            v[k] = __uint_as_float(u[k]);
        }
        const uint32_t hw = e4m3_pack4(v[0], v[1], v[2], v[3]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (i + k >= n) continue;
            if (((hw >> (8 * k)) & 0xFFu) != e4m3_rne_sat(v[k])) {
                ++nbad;
                fbad = min(fbad, u[k]);
            }
        }
    }
    if (nbad) {
        atomicAdd(count, nbad);
        atomicMin(first, fbad);
    }
}

}  // namespace

hipError_t launch_check_e4m3(uint32_t first_pattern, uint32_t n, uint32_t *count,
                             uint32_t *first, hipStream_t stream)
{
    if (hipError_t e = launch(e4m3_check_init, dim3(1), dim3(1), 0, stream, count, first))
        return e;
    if (n == 0) return hipSuccess;
    const uint64_t per_block = (uint64_t)kCheckThreads * 4 * 64;   // 64 steps per lane
    const uint64_t blocks = ((uint64_t)n + per_block - 1) / per_block;
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536)), block(kCheckThreads);
    return launch(e4m3_check_kernel, grid, block, 0, stream, first_pattern, (uint64_t)n, count,
                  first);
}

}  // namespace ep
