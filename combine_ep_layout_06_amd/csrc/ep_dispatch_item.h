// One dispatch work item: a token row segment copied (bf16) or quantised to FP8 and written to
// the receive rows of the token's kept pairs (internal header).
//
// The receiving side of expert-parallel dispatch expands tokens into the per-expert layout
// (afdEP-comm validation record, kernel_timelines: dispatch_copy_epilogue). Here the tokens are
// local, so a token row is read ONCE and stored to each of its K receive rows.
//
// The caller has the receive-row numbers of its tokens' pairs in LDS: rows[tl*K + j] =
// e*C + slot, or -1 for a pair that is not kept. Each lane moves 16-byte chunks,
// lane-contiguous, so every load and store instruction covers 1 KiB of one row. x loads are
// non-temporal (read once); row stores are plain stores, which measured faster than
// non-temporal ones for this one-row-to-K-rows scatter on MI355X.
//
// FP8: a lane owns 16 consecutive channels (two 16-byte loads, one 16-byte store of codes), so
// a 128-channel block is 8 lanes; the block amax is a DPP max over those 8 lanes. The codes are
// exactly those of the definition, scale = amax / 448 and q = e4m3(x / scale) with IEEE fp32
// divisions (amax = 0: scale 0 and the signed zero of x). The scale is one division; the 16
// quotients of a lane come from one reciprocal and FMA corrections (div_by_rcp, equal to the
// IEEE quotient wherever the code depends on it), and the hardware conversion encodes them. A
// wavefront with a block whose amax is 0, below 2^-60 or not finite takes the plain path: one
// IEEE division per element and the software encoder.
#pragma once

#include "ep_device.h"

#ifndef EP_DISPATCH_NT_LOAD
#define EP_DISPATCH_NT_LOAD 1
#endif
#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 0
#endif

namespace ep {

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Row number of pair (e, s) in the [E][C] receive buffer, or -1 if it is not kept.
__device__ __forceinline__ int recv_row(int e, int s, int E, int C)
{
    return ((unsigned)e < (unsigned)E && (unsigned)s < (unsigned)C) ? e * C + s : -1;
}

// The receive rows of up to KG pairs of local token tl, read from LDS together (uniform).
template <int KG>
__device__ __forceinline__ void token_rows(const int32_t *rows, int tl, int j0, int K,
                                           int (&r)[KG])
{
#pragma unroll
    for (int g = 0; g < KG; ++g) {
        const int j = j0 + g;
        const int v = wave_uniform(rows[tl * K + (j < K ? j : K - 1)]);
        r[g] = j < K ? v : -1;
    }
}

// bf16 item, split in two so a caller can issue the loads before it knows the slots:
// segment `seg` (U chunks per lane) of token t (local index tl).
template <int U>
struct RowPiece {
    u32x4 v[U];
};

template <int U>
__device__ __forceinline__ RowPiece<U> load_item_bf16(const u32x4 *__restrict__ x, int t,
                                                      int seg, int H8)
{
    const int lane = threadIdx.x & (kWave - 1);
    const u32x4 *src = x + (size_t)t * H8;
    RowPiece<U> p;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (seg * U + u) * kWave + lane;
        p.v[u] = load16<EP_DISPATCH_NT_LOAD>(src + (c < H8 ? c : H8 - 1));
    }
    return p;
}

// KG: pairs per group (K <= KG unless MULTI).
template <int KG, int U, bool MULTI>
__device__ __forceinline__ void store_item_bf16(const RowPiece<U> &p, u32x4 *__restrict__ recv,
                                                const int32_t *rows, int tl, int seg, int H8,
                                                int K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int npg = MULTI ? (K + KG - 1) / KG : 1;
    for (int pg = 0; pg < npg; ++pg) {
        int r[KG];
        token_rows<KG>(rows, tl, pg * KG, K, r);
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            if (r[g] < 0) continue;
            u32x4 *dst = recv + (size_t)r[g] * H8;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (seg * U + u) * kWave + lane;
                if (c < H8) store16<EP_DISPATCH_NT_STORE>(dst + c, p.v[u]);
            }
        }
    }
}

template <int KG, int U, bool MULTI>
__device__ __forceinline__ void dispatch_item_bf16(const u32x4 *__restrict__ x,
                                                   u32x4 *__restrict__ recv, const int32_t *rows,
                                                   int t, int tl, int seg, int H8, int K)
{
    store_item_bf16<KG, U, MULTI>(load_item_bf16<U>(x, t, seg, H8), recv, rows, tl, seg, H8, K);
}

// FP8 item, split in three: the row load, the cast (which needs only the row) and the stores
// (which need the slots). Segment `seg` (1024 channels) of token t; H % 128 == 0.
struct RawPieceFp8 {
    u32x4 a, b;       // this lane's 16 channels, zero where it has none
    bool act;         // this lane's channels exist (whole 8-lane groups)
};

struct QuantPiece {
    u32x4 q;          // 16 codes of this lane's channels
    float scale;      // scale of this lane's 128-channel block
    bool act;
};

__device__ __forceinline__ RawPieceFp8 load_item_fp8(const u32x4 *__restrict__ x, int t, int seg,
                                                     int H)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int h0 = seg * (16 * kWave) + lane * 16;   // first channel of this lane
    RawPieceFp8 r;
    r.act = h0 < H;
    r.a = u32x4{0u, 0u, 0u, 0u};
    r.b = r.a;
    if (r.act) {
        const u32x4 *src = x + (size_t)t * (H / 8) + h0 / 8;
        r.a = load16<EP_DISPATCH_NT_LOAD>(src);
        r.b = load16<EP_DISPATCH_NT_LOAD>(src + 1);
    }
    return r;
}

// All 64 lanes take part (the block amax is a DPP max over 8 lanes).
__device__ __forceinline__ QuantPiece cast_item_fp8(const RawPieceFp8 &r)
{
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    float f[16];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        f[2 * k] = bf16_lo(w[k]);
        f[2 * k + 1] = bf16_hi(w[k]);
        m = max(m, (w[k] << 16) & 0x7FFFFFFFu);
        m = max(m, w[k] & 0x7FFF0000u);
    }
    const float amax = group8_max(__uint_as_float(m));   // |x| bits: integer order
    QuantPiece p;
    p.act = r.act;
    p.scale = amax / 448.0f;
    uint32_t q[4] = {0u, 0u, 0u, 0u};
    // 2^-60 <= amax < inf in every lane with channels: |x / scale| <= 448 (1 + 2^-22), inside
    // the range where the hardware conversion is exact, and div_by_rcp's remainders do not
    // underflow (lanes past H hold zeros and store nothing)
    const uint32_t ab = __float_as_uint(amax);
    const bool fast = !r.act || (ab >= 0x21800000u && ab < 0x7F800000u);
    if (__builtin_expect(__ballot(!fast) == 0, 1)) {
        const float y = 1.0f / p.scale;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = e4m3_pack4(div_by_rcp(f[4 * i], p.scale, y),
                              div_by_rcp(f[4 * i + 1], p.scale, y),
                              div_by_rcp(f[4 * i + 2], p.scale, y),
                              div_by_rcp(f[4 * i + 3], p.scale, y));
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t code = (amax == 0.0f) ? ((__float_as_uint(f[k]) >> 24) & 0x80u)
                                                 : e4m3_rne_sat(f[k] / p.scale);
            q[k / 4] |= code << (8 * (k % 4));
        }
    }
    p.q = u32x4{q[0], q[1], q[2], q[3]};
    return p;
}

__device__ __forceinline__ QuantPiece quant_item_fp8(const u32x4 *__restrict__ x, int t, int seg,
                                                     int H)
{
    return cast_item_fp8(load_item_fp8(x, t, seg, H));
}

template <int KG, bool MULTI>
__device__ __forceinline__ void store_item_fp8(const QuantPiece &p, u32x4 *__restrict__ recv_q,
                                               float *__restrict__ recv_scale,
                                               const int32_t *rows, int tl, int seg, int H, int K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int H16 = H / 16, NB = H / 128;
    const int h0 = seg * (16 * kWave) + lane * 16;
    const int npg = MULTI ? (K + KG - 1) / KG : 1;
    for (int pg = 0; pg < npg; ++pg) {
        int r[KG];
        token_rows<KG>(rows, tl, pg * KG, K, r);
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            if (r[g] < 0 || !p.act) continue;
            store16<EP_DISPATCH_NT_STORE>(recv_q + (size_t)r[g] * H16 + h0 / 16, p.q);
            if ((lane & 7) == 0) recv_scale[(size_t)r[g] * NB + h0 / 128] = p.scale;
        }
    }
}

template <int KG, bool MULTI>
__device__ __forceinline__ void dispatch_item_fp8(const u32x4 *__restrict__ x,
                                                  u32x4 *__restrict__ recv_q,
                                                  float *__restrict__ recv_scale,
                                                  const int32_t *rows, int t, int tl, int seg,
                                                  int H, int K)
{
    store_item_fp8<KG, MULTI>(quant_item_fp8(x, t, seg, H), recv_q, recv_scale, rows, tl, seg, H,
                              K);
}

// Instantiate LAUNCH(KG, MULTI) for the pair-group size that fits K.
#define EP_BY_K(K, LAUNCH)                                                                  \
    do {                                                                                    \
        if ((K) > 8) LAUNCH(8, true);                                                       \
        if ((K) > 4) LAUNCH(8, false);                                                      \
        if ((K) > 2) LAUNCH(4, false);                                                      \
        if ((K) > 1) LAUNCH(2, false);                                                      \
        LAUNCH(1, false);                                                                   \
    } while (0)

}  // namespace ep
