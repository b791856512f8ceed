/*
 * A plain C client of libep_mi355x.so: HIP runtime calls and include/ep.h only, no torch and no
 * Python objects. Built by tests/c_abi/build.py into ep_c_client.so; the GPU test calls its one
 * function through ctypes (in-process, so no program is started).
 *
 * It runs layout, the separate bf16 dispatch, the fused layout + dispatch, the FP8 dispatch and
 * combine on a small route with drops, unrouted and invalid ids, and checks each result on the
 * host against what the definitions fix directly:
 *  - slot[i] = number of earlier pairs with the same expert, or -1 past the capacity C or for
 *    an id that is not an expert (brute force over the earlier pairs);
 *  - count = min(demand, C), offset its exclusive scan, per-rank sums, stats;
 *  - every kept pair's receive row is its token's row, every other row keeps a sentinel, and
 *    the fused call writes exactly what the two separate calls write;
 *  - FP8: the scale of each kept row is amax / 448 (the same IEEE division on the host) and
 *    the block's largest |x| encodes to the largest code, 0x7E or 0xFE by sign;
 *  - combine with expert outputs equal to the receive rows and unit weights returns
 *    n_kept(t) * x[t] (small integers, so every sum and the bf16 rounding are exact).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

enum { T = 300, H = 256, E = 32, K = 4, C = 40, R = 4, NB = H / 128 };

static char *g_msg;
static int g_len;

static int fail(const char *what, long at)
{
    snprintf(g_msg, (size_t)g_len, "%s (at %ld)", what, at);
    return 1;
}

#define HIP_OK(call)                                                                      \
    do {                                                                                  \
        if ((call) != hipSuccess) return fail("HIP call failed: " #call, __LINE__);       \
    } while (0)
#define EP_CALL(call)                                                                     \
    do {                                                                                  \
        int rc_ = (call);                                                                 \
        if (rc_ != EP_OK) return fail(ep_last_error(), rc_);                              \
    } while (0)

static uint16_t bf16_of_small_int(int v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);    /* exact: a small integer has no bits below the top 16 */
}

static float float_of_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int run(void)
{
    static int32_t idx[T * K], slot[T * K], slot2[T * K], want_slot[T * K];
    static int32_t cnt[E], off[E], rc[R], ro[R], st[EP_STATS_LEN], cnt2[E], off2[E], rc2[R],
        ro2[R], st2[EP_STATS_LEN];
    static uint16_t x[T * H], recv[E * C * H], recv2[E * C * H], out[T * H];
    static uint8_t q[E * C * H];
    static float scale[E * C * NB], w[T * K];
    const ep_shape_t sh = {T, H, E, K, C, R};

    /* route: K distinct experts per token from a fixed LCG, skewed so some experts overflow C;
     * a few unrouted (-1) and invalid (E, -2) ids */
    uint64_t s = 12345;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < K; ++j) {
            int e, dup;
            do {
                s = s * 6364136223846793005ull + 1442695040888963407ull;
                e = (int)((s >> 33) % (E + 8));
                if (e >= E) e = (e - E) % 4;         /* experts 0..3 take extra load */
                dup = 0;
                for (int j2 = 0; j2 < j; ++j2) dup |= idx[t * K + j2] == e;
            } while (dup);
            idx[t * K + j] = e;
        }
    }
    idx[5 * K + 1] = -1;
    idx[7 * K + 3] = E;
    idx[11 * K + 0] = -2;
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) x[t * H + h] = bf16_of_small_int((t * 7 + h * 3) % 15 - 7);
    for (int i = 0; i < T * K; ++i) w[i] = 1.0f;

    int32_t *d_idx, *d_slot, *d_cnt, *d_off, *d_rc, *d_ro, *d_st;
    uint16_t *d_x, *d_recv, *d_out;
    uint8_t *d_q;
    float *d_scale, *d_w;
    HIP_OK(hipMalloc((void **)&d_idx, sizeof idx));
    HIP_OK(hipMalloc((void **)&d_slot, sizeof slot));
    HIP_OK(hipMalloc((void **)&d_cnt, sizeof cnt));
    HIP_OK(hipMalloc((void **)&d_off, sizeof off));
    HIP_OK(hipMalloc((void **)&d_rc, sizeof rc));
    HIP_OK(hipMalloc((void **)&d_ro, sizeof ro));
    HIP_OK(hipMalloc((void **)&d_st, sizeof st));
    HIP_OK(hipMalloc((void **)&d_x, sizeof x));
    HIP_OK(hipMalloc((void **)&d_recv, sizeof recv));
    HIP_OK(hipMalloc((void **)&d_out, sizeof out));
    HIP_OK(hipMalloc((void **)&d_q, sizeof q));
    HIP_OK(hipMalloc((void **)&d_scale, sizeof scale));
    HIP_OK(hipMalloc((void **)&d_w, sizeof w));
    HIP_OK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));

    /* layout, then the bf16 dispatch into a sentinel-filled buffer */
    EP_CALL(ep_layout(&sh, d_idx, d_slot, d_cnt, d_off, d_rc, d_ro, d_st, 0));
    HIP_OK(hipMemset(d_recv, 0x5A, sizeof recv));
    EP_CALL(ep_dispatch(&sh, d_x, d_idx, d_slot, d_recv, 0));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(slot, d_slot, sizeof slot, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cnt, d_cnt, sizeof cnt, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(off, d_off, sizeof off, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rc, d_rc, sizeof rc, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ro, d_ro, sizeof ro, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(st, d_st, sizeof st, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv, d_recv, sizeof recv, hipMemcpyDeviceToHost));

    /* the layout by brute force */
    int demand[E] = {0}, kept = 0, dropped = 0, unrouted = 0, invalid = 0;
    for (int i = 0; i < T * K; ++i) {
        const int e = idx[i];
        if (e == -1) { want_slot[i] = -1; ++unrouted; continue; }
        if (e < 0 || e >= E) { want_slot[i] = -1; ++invalid; continue; }
        int earlier = 0;
        for (int i2 = 0; i2 < i; ++i2) earlier += idx[i2] == e;
        want_slot[i] = earlier < C ? earlier : -1;
        if (earlier < C) ++kept; else ++dropped;
        ++demand[e];
    }
    if (dropped == 0) return fail("the route was meant to overflow the capacity", 0);
    for (int i = 0; i < T * K; ++i)
        if (slot[i] != want_slot[i]) return fail("slot", i);
    int run_off = 0;
    for (int e = 0; e < E; ++e) {
        const int want = demand[e] < C ? demand[e] : C;
        if (cnt[e] != want) return fail("expert_count", e);
        if (off[e] != run_off) return fail("expert_offset", e);
        run_off += want;
    }
    int run_ro = 0;
    for (int r = 0; r < R; ++r) {
        int sum = 0;
        for (int l = 0; l < E / R; ++l) sum += cnt[r * (E / R) + l];
        if (rc[r] != sum) return fail("rank_count", r);
        if (ro[r] != run_ro) return fail("rank_offset", r);
        run_ro += sum;
    }
    if (st[0] != kept || st[1] != dropped || st[2] != unrouted || st[3] != invalid)
        return fail("stats", st[0]);

    /* the bf16 dispatch: kept rows hold the token's row, all others the sentinel */
    static unsigned char touched[E * C];
    memset(touched, 0, sizeof touched);
    for (int i = 0; i < T * K; ++i) {
        if (want_slot[i] < 0) continue;
        const long row = (long)idx[i] * C + want_slot[i];
        touched[row] = 1;
        if (memcmp(&recv[row * H], &x[(i / K) * H], H * sizeof(uint16_t)) != 0)
            return fail("dispatch row", row);
    }
    for (long row = 0; row < (long)E * C; ++row)
        if (!touched[row])
            for (int h = 0; h < H; ++h)
                if (recv[row * H + h] != 0x5A5A) return fail("row that should be untouched", row);

    /* the fused call writes what the two separate calls wrote */
    HIP_OK(hipMemset(d_recv, 0x5A, sizeof recv));
    EP_CALL(ep_layout_dispatch(&sh, d_x, d_idx, d_slot, d_cnt, d_off, d_rc, d_ro, d_st, d_recv,
                               0));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(slot2, d_slot, sizeof slot2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cnt2, d_cnt, sizeof cnt2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(off2, d_off, sizeof off2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rc2, d_rc, sizeof rc2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ro2, d_ro, sizeof ro2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(st2, d_st, sizeof st2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv2, d_recv, sizeof recv2, hipMemcpyDeviceToHost));
    if (memcmp(slot, slot2, sizeof slot) || memcmp(cnt, cnt2, sizeof cnt) ||
        memcmp(off, off2, sizeof off) || memcmp(rc, rc2, sizeof rc) || memcmp(ro, ro2, sizeof ro) ||
        memcmp(st, st2, sizeof st))
        return fail("fused layout differs from ep_layout", 0);
    if (memcmp(recv, recv2, sizeof recv)) return fail("fused dispatch differs from ep_dispatch", 0);

    /* FP8 dispatch: per-block scales and the code of each block's largest |x| */
    EP_CALL(ep_dispatch_fp8(&sh, d_x, d_idx, d_slot, d_q, d_scale, 0));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(q, d_q, sizeof q, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(scale, d_scale, sizeof scale, hipMemcpyDeviceToHost));
    for (int i = 0; i < T * K; ++i) {
        if (want_slot[i] < 0) continue;
        const long row = (long)idx[i] * C + want_slot[i];
        const int t = i / K;
        for (int b = 0; b < NB; ++b) {
            float amax = 0.0f;
            int at = 0;
            for (int h = 128 * b; h < 128 * (b + 1); ++h) {
                const float a = fabsf(float_of_bf16(x[t * H + h]));
                if (a > amax) { amax = a; at = h; }
            }
            volatile float d = 448.0f;      /* one IEEE fp32 division, as the definition says */
            if (scale[row * NB + b] != amax / d) return fail("fp8 scale", row);
            const uint8_t want = float_of_bf16(x[t * H + at]) < 0 ? 0xFE : 0x7E;
            if (q[row * H + at] != want) return fail("fp8 code of the block amax", row);
        }
    }

    /* combine with y = the receive rows and unit weights: n_kept(t) * x[t] */
    EP_CALL(ep_combine(&sh, d_recv, d_idx, d_slot, d_w, d_out, 0));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    for (int t = 0; t < T; ++t) {
        int n = 0;
        for (int j = 0; j < K; ++j) n += want_slot[t * K + j] >= 0;
        for (int h = 0; h < H; ++h) {
            const float want = (float)n * float_of_bf16(x[t * H + h]);
            const float got = float_of_bf16(out[t * H + h]);
            if (got != want || (want == 0.0f && out[t * H + h] != 0))
                return fail("combine", (long)t * H + h);
        }
    }

    hipFree(d_idx); hipFree(d_slot); hipFree(d_cnt); hipFree(d_off); hipFree(d_rc);
    hipFree(d_ro); hipFree(d_st); hipFree(d_x); hipFree(d_recv); hipFree(d_out); hipFree(d_q);
    hipFree(d_scale); hipFree(d_w);
    snprintf(g_msg, (size_t)g_len, "ok: %d kept, %d dropped, %d unrouted, %d invalid", kept,
             dropped, unrouted, invalid);
    return 0;
}

/* Runs the checks on the current HIP device. Returns 0 if every check passed; msg receives a
 * line that names the first failed check, or a summary. */
int ep_c_client_check(char *msg, int len)
{
    g_msg = msg;
    g_len = len;
    return run();
}
