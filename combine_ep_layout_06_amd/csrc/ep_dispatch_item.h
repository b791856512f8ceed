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
//
// Non-finite input: a NaN anywhere in a block makes its amax NaN (the integer max of the |x|
// patterns puts every NaN above +inf and every finite value); a NaN amax gives the quiet NaN
// 0x7FC00000 as the scale; every code carries x's own sign bit, so a NaN quotient (x / NaN,
// +-inf / inf) encodes as sign(x) | 0x7F whatever sign the division gave it. An infinite amax
// gives an infinite scale, and the finite elements of that block encode as signed zeros.
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
// (which need the slots). A lane takes U pieces of 16 channels, 1024 channels apart, so every
// load and store instruction covers 1 KiB of one row; segment `seg` is channels
// [seg*U*1024, (seg+1)*U*1024). H % 128 == 0, so a piece's 8-lane groups are whole blocks.
template <int U>
struct RawPieceFp8 {
    u32x4 a[U], b[U];     // each piece's 16 channels, zero where it has none
    bool act[U];          // the piece's channels exist
};

template <int U>
struct QuantPiece {
    u32x4 q[U];           // 16 codes per piece
    float scale[U];       // scale of each piece's 128-channel block
    bool act[U];
};

// First channel of piece u of segment seg for this lane.
__device__ __forceinline__ int fp8_channel(int seg, int u, int U, int lane)
{
    return (seg * U + u) * (16 * kWave) + lane * 16;
}

template <int U>
__device__ __forceinline__ RawPieceFp8<U> load_item_fp8(const u32x4 *__restrict__ x, int t,
                                                        int seg, int H)
{
    const int lane = threadIdx.x & (kWave - 1);
    RawPieceFp8<U> r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int h0 = fp8_channel(seg, u, U, lane);
        r.act[u] = h0 < H;
        r.a[u] = u32x4{0u, 0u, 0u, 0u};
        r.b[u] = r.a[u];
        if (r.act[u]) {
            const u32x4 *src = x + (size_t)t * (H / 8) + h0 / 8;
            r.a[u] = load16<EP_DISPATCH_NT_LOAD>(src);
            r.b[u] = load16<EP_DISPATCH_NT_LOAD>(src + 1);
        }
    }
    return r;
}

// The same loads with no branch: every lane loads (a lane past the row reads the row's first
// chunk), so a caller that issued loads before this one can wait for those alone while these
// are in flight. zero_past_row() must be applied before the cast.
template <int U>
__device__ __forceinline__ RawPieceFp8<U> load_item_fp8_nobranch(const u32x4 *__restrict__ x,
                                                                 int t, int seg, int H)
{
    const int lane = threadIdx.x & (kWave - 1);
    RawPieceFp8<U> r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int h0 = fp8_channel(seg, u, U, lane);
        r.act[u] = h0 < H;
        const u32x4 *src = x + (size_t)t * (H / 8) + (r.act[u] ? h0 / 8 : 0);
        r.a[u] = load16<EP_DISPATCH_NT_LOAD>(src);
        r.b[u] = load16<EP_DISPATCH_NT_LOAD>(src + 1);
    }
    return r;
}

// Zeros in the pieces past the row, as load_item_fp8 leaves them.
template <int U>
__device__ __forceinline__ RawPieceFp8<U> zero_past_row(RawPieceFp8<U> r)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        r.a[u] = r.act[u] ? r.a[u] : z;
        r.b[u] = r.act[u] ? r.b[u] : z;
    }
    return r;
}

// All 64 lanes take part (a block amax is a DPP max over 8 lanes).
template <int U>
__device__ __forceinline__ QuantPiece<U> cast_item_fp8(const RawPieceFp8<U> &r)
{
    QuantPiece<U> p;
    float amax[U];
    bool fast = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t w[8] = {r.a[u].x, r.a[u].y, r.a[u].z, r.a[u].w,
                               r.b[u].x, r.b[u].y, r.b[u].z, r.b[u].w};
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            m = max(m, (w[k] << 16) & 0x7FFFFFFFu);
            m = max(m, w[k] & 0x7FFF0000u);
        }
        amax[u] = group8_max(__uint_as_float(m));   // |x| bits: integer order, NaN on top
        p.act[u] = r.act[u];
        p.scale[u] = __float_as_uint(amax[u]) > 0x7F800000u ? __uint_as_float(0x7FC00000u)
                                                            : amax[u] / 448.0f;
        // 2^-60 <= amax < inf in every piece with channels: |x / scale| <= 448 (1 + 2^-22),
        // inside the range where the hardware conversion is exact, and div_by_rcp's
        // remainders do not underflow (pieces past H hold zeros and store nothing)
        const uint32_t ab = __float_as_uint(amax[u]);
        fast = fast && (!r.act[u] || (ab >= 0x21800000u && ab < 0x7F800000u));
    }
    const bool all_fast = __ballot(!fast) == 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t w[8] = {r.a[u].x, r.a[u].y, r.a[u].z, r.a[u].w,
                               r.b[u].x, r.b[u].y, r.b[u].z, r.b[u].w};
        float f[16];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            f[2 * k] = bf16_lo(w[k]);
            f[2 * k + 1] = bf16_hi(w[k]);
        }
        uint32_t q[4] = {0u, 0u, 0u, 0u};
        if (__builtin_expect(all_fast, 1)) {
            const float y = 1.0f / p.scale[u];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                q[i] = e4m3_pack4(div_by_rcp(f[4 * i], p.scale[u], y),
                                  div_by_rcp(f[4 * i + 1], p.scale[u], y),
                                  div_by_rcp(f[4 * i + 2], p.scale[u], y),
                                  div_by_rcp(f[4 * i + 3], p.scale[u], y));
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t sign = (__float_as_uint(f[k]) >> 24) & 0x80u;
                const uint32_t code =
                    (amax[u] == 0.0f) ? sign
                                      : sign | (e4m3_rne_sat(f[k] / p.scale[u]) & 0x7Fu);
                q[k / 4] |= code << (8 * (k % 4));
            }
        }
        p.q[u] = u32x4{q[0], q[1], q[2], q[3]};
    }
    return p;
}

template <int U>
__device__ __forceinline__ QuantPiece<U> quant_item_fp8(const u32x4 *__restrict__ x, int t,
                                                        int seg, int H)
{
    return cast_item_fp8<U>(load_item_fp8<U>(x, t, seg, H));
}

// Codes: one 16-byte store per piece and row. Scales: the segment's U*8 blocks of a row in one
// store instruction; lane 8i + u (u < U) holds the scale of block i of piece u (every lane of
// that 8-lane group does) and stores it.
template <int KG, int U, bool MULTI>
__device__ __forceinline__ void store_item_fp8(const QuantPiece<U> &p, u32x4 *__restrict__ recv_q,
                                               float *__restrict__ recv_scale,
                                               const int32_t *rows, int tl, int seg, int H, int K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int H16 = H / 16, NB = H / 128;
    const int su = lane & 7;
    const int sblk = (seg * U + su) * 8 + (lane >> 3);
    float sval = p.scale[0];
#pragma unroll
    for (int u = 1; u < U; ++u)
        if (su == u) sval = p.scale[u];
    const bool sact = su < U && sblk < NB;
    const int npg = MULTI ? (K + KG - 1) / KG : 1;
    for (int pg = 0; pg < npg; ++pg) {
        int r[KG];
        token_rows<KG>(rows, tl, pg * KG, K, r);
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            if (r[g] < 0) continue;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (p.act[u])
                    store16<EP_DISPATCH_NT_STORE>(
                        recv_q + (size_t)r[g] * H16 + fp8_channel(seg, u, U, lane) / 16, p.q[u]);
            if (sact) recv_scale[(size_t)r[g] * NB + sblk] = sval;
        }
    }
}

template <int KG, int U, bool MULTI>
__device__ __forceinline__ void dispatch_item_fp8(const u32x4 *__restrict__ x,
                                                  u32x4 *__restrict__ recv_q,
                                                  float *__restrict__ recv_scale,
                                                  const int32_t *rows, int t, int tl, int seg,
                                                  int H, int K)
{
    store_item_fp8<KG, U, MULTI>(quant_item_fp8<U>(x, t, seg, H), recv_q, recv_scale, rows, tl,
                                 seg, H, K);
}

// Pieces per lane for an FP8 dispatch of T tokens of H channels: two when each token still
// fills them and the batch keeps at least 4096 wavefront items, else one (measured on MI355X:
// wide items win on prefill-sized batches, as for bf16 rows).
#ifndef EP_FP8_U
#define EP_FP8_U 0
#endif
inline int pick_u_fp8(int T, int H)
{
    if (EP_FP8_U) return EP_FP8_U;
    const int nseg2 = (H + 2 * 16 * kWave - 1) / (2 * 16 * kWave);
    return (H >= 2 * 16 * kWave && (long)T * nseg2 >= 4096) ? 2 : 1;
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
