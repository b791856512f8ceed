/*
 * CPU oracle for one GPU's share of MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * call this code. It is plain, single-threaded C written from the definitions of the
 * operations; it shares no code, header, table or helper with the GPU library, and the GPU
 * library never calls it.
 *
 * Sources of the definitions:
 *  - Dispatch layout (per-expert counts and placement) is the step the "normal" APIs must run
 *    inside the timed boundary: awsome-distributed-ai PR #1238, "What changed" and the
 *    author's reply on what latency means.
 *  - Dispatch expands each token into the expert layout (afdEP-comm validation record,
 *    kernel_timelines: dispatch_copy_epilogue; the use_expanded_layout patch).
 *  - The per-token FP8 cast with one scale per 128 channels: PR #1238 review item 1
 *    (per_token_cast_to_fp8; quantisation inside low_latency_dispatch(use_fp8=True)) and the
 *    logical-payload accounting there (H + 4*H/128 bytes per FP8 row). The e4m3 format is the
 *    OCP 8-bit floating point specification (OFP8) E4M3: bias 7, three mantissa bits, no
 *    infinities, a single NaN code per sign (S.1111.111), largest finite value 448.
 *  - Combine gathers expert outputs back and reduces them with the top-k weights; combine is
 *    BF16 in either dispatch dtype (PR #1238 review item 1; afdEP-comm kernel_timelines:
 *    combine_reduce_epilogue).
 *  - The two-stage path mirrors the pages' kernel chain (afdEP-comm kernel_timelines:
 *    dispatch_impl then dispatch_copy_epilogue; combine_impl then combine_reduce_epilogue):
 *    a token goes to each virtual rank once, the rank expands it into its experts' rows, and
 *    on the way back each rank returns one partial row per token.
 *  - Readings where the pages are silent: pair order i = t*K + j is "token order"; a
 *    capacity-C expert keeps its first C pairs in that order; the receive buffer is
 *    [E][C][H] with expert e = r*(E/R) + l (rank-major); scale = amax / 448 by an IEEE fp32
 *    division and q = e4m3(x / scale) by a second fp32 division; combine accumulates
 *    acc = fmaf(w_j, y_j, acc) in fp32 for j ascending from +0 and rounds once to bf16;
 *    weights of dropped pairs are not renormalised. Two-stage path: a token is sent to rank r
 *    if any of its valid ids is an expert of r (the sender sees only the routing; capacity is
 *    applied to the experts' rows on the receiving side); a rank's tokens keep token order; the
 *    per-rank partial is the same fmaf fold over the token's kept pairs of that rank, rounded
 *    once to bf16 (the combine payload is bf16); the final row is the fp32 sum of the
 *    partials in ascending rank, rounded once to bf16. Packed layout (the expert_alignment
 *    parameter the pages pin to 1 for their runs): each expert's kept count rounded up to a
 *    multiple of the alignment, offsets the exclusive scan of those, pair (t, j) at row
 *    offset[e] + slot of a [rows][H] buffer; padding rows are left as they are.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared (no -ffast-math, no
 * FMA contraction: every fp32 operation below is one IEEE operation).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* Zeroed heap buffer of n elements of sz bytes (at least one); the oracle stops on failure. */
static void *xcalloc(size_t n, size_t sz)
{
    void *p = calloc(n > 0 ? n : 1, sz);
    if (!p) {
        fprintf(stderr, "oracle: out of memory\n");
        abort();
    }
    return p;
}

/* ----------------------------------------------------------------------------------------- */
/* Number formats                                                                             */
/* ----------------------------------------------------------------------------------------- */

float oracle_bf16_to_f32(uint16_t b)
{
    /* bf16 is the upper half of an fp32 pattern: widening is exact. */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * fp32 -> bf16, round to nearest, ties to even, by definition: take the two bf16 values that
 * bracket f (truncation toward zero, and the next one away from zero), compare the distances
 * in double precision (exact for fp32 operands), keep the nearer, on a tie keep the one whose
 * last mantissa bit is 0. Overflow past the largest finite bf16 rounds to infinity as IEEE
 * round-to-nearest does. Every NaN gives the one quiet NaN 0x7FC0: the sign and payload of a
 * NaN that an fp32 sum produces are not fixed by IEEE 754 and differ between processors, so
 * an output that is NaN is written as that single pattern.
 */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u = f32_bits(f);
    if (isnan(f))
        return 0x7FC0u;
    if (isinf(f))
        return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);            /* toward zero */
    if ((u & 0xFFFFu) == 0)
        return lo;                                /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);             /* next magnitude (may be +-inf) */
    double v = fabs((double)f);
    double dlo = v - fabs((double)oracle_bf16_to_f32(lo));
    /* Past the largest finite bf16 the next step is infinity, which IEEE rounding treats as
     * the value 2^128 of an exponent range without bound. */
    double vhi = ((hi & 0x7FFFu) == 0x7F80u) ? ldexp(1.0, 128)
                                             : fabs((double)oracle_bf16_to_f32(hi));
    double dhi = vhi - v;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;
}

/* Value of an OCP E4M3 code's magnitude bits (0x00..0x7E); code 0x7F is NaN. */
double oracle_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0)
        mag = ldexp((double)m, -9);                     /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);     /* normal: (1 + m/8) * 2^(e-7) */
    return (code & 0x80) ? -mag : mag;
}

/*
 * fp32 -> OCP E4M3 with round-to-nearest-even and saturation to +-448 (OFP8 "satfinite"
 * conversion). The magnitude is matched against the 127 finite non-negative codes
 * 0x00..0x7E, which increase with their value: find the largest code whose value is <= |v|,
 * then choose between it and the next code by distance (ties to the code whose last
 * mantissa bit is 0). Magnitudes at or beyond 448 give 448. The sign bit is copied, so
 * -0.0 gives 0x80. NaN input gives the NaN code 0x7F with the sign of v.
 */
uint8_t oracle_e4m3_rne_sat(float v)
{
    uint8_t sign = (f32_bits(v) >> 31) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    /* binary search for the largest code c in [0, 0x7E] with value(c) <= a */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (oracle_e4m3_value((uint8_t)mid) <= a) lo = mid;
        else hi = mid - 1;
    }
    int c = lo;
    double below = oracle_e4m3_value((uint8_t)c);
    if (below == a)
        return (uint8_t)(sign | c);
    double above = oracle_e4m3_value((uint8_t)(c + 1));   /* c < 0x7E since a < 448 */
    double d0 = a - below, d1 = above - a;
    if (d1 < d0 || (d1 == d0 && (c & 1)))
        c = c + 1;
    return (uint8_t)(sign | c);
}

/* ----------------------------------------------------------------------------------------- */
/* Layout                                                                                     */
/* ----------------------------------------------------------------------------------------- */

/*
 * Routing layout for T tokens with K choices each over E experts, capacity C per expert,
 * R virtual ranks of E/R consecutive experts.
 *
 *   Pairs are visited in token order i = t*K + j. id == -1 is unrouted; any other id outside
 *   [0, E) is invalid. Both get slot -1. A routed pair takes the next position of its expert;
 *   positions >= C are dropped (slot -1). So slot[i] = #{i' < i : id[i'] == id[i]} when that
 *   is < C, i.e. stable in-order placement under capacity.
 *
 *   count[e]  = min(raw[e], C)            kept pairs of expert e
 *   offset[e] = sum_{e' < e} count[e']   exclusive scan in expert (= rank-major) order
 *   rank_count[r], rank_offset[r]         the same over the E/R experts of each rank
 *   stats = {kept, dropped, unrouted, invalid}; the four sum to T*K.
 *
 * raw (optional, may be NULL) receives the demand per expert before capacity.
 */
void oracle_layout(int T, int K, int E, int C, int R, const int32_t *topk_idx, int32_t *slot,
                   int32_t *count, int32_t *offset, int32_t *rank_count, int32_t *rank_offset,
                   int32_t *stats, int32_t *raw)
{
    int32_t *demand = xcalloc((size_t)E, sizeof *demand);
    int32_t kept = 0, dropped = 0, unrouted = 0, invalid = 0;
    long n = (long)T * K;
    for (long i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        if (e == -1) { slot[i] = -1; ++unrouted; continue; }
        if (e < 0 || e >= E) { slot[i] = -1; ++invalid; continue; }
        int32_t p = demand[e]++;
        if (p < C) { slot[i] = p; ++kept; }
        else { slot[i] = -1; ++dropped; }
    }
    int32_t run = 0;
    for (int e = 0; e < E; ++e) {
        count[e] = demand[e] < C ? demand[e] : C;
        offset[e] = run;
        run += count[e];
        if (raw) raw[e] = demand[e];
    }
    int EL = E / R;
    run = 0;
    for (int r = 0; r < R; ++r) {
        int32_t s = 0;
        for (int l = 0; l < EL; ++l) s += count[r * EL + l];
        if (rank_count) rank_count[r] = s;
        if (rank_offset) rank_offset[r] = run;
        run += s;
    }
    stats[0] = kept; stats[1] = dropped; stats[2] = unrouted; stats[3] = invalid;
    free(demand);
}

/* A pair takes part in dispatch/combine only if its expert id and slot address a row of the
 * [E][C][H] buffer; anything else is skipped. */
static int pair_kept(int32_t e, int32_t s, int E, int C)
{
    return e >= 0 && e < E && s >= 0 && s < C;
}

/* ----------------------------------------------------------------------------------------- */
/* Dispatch                                                                                   */
/* ----------------------------------------------------------------------------------------- */

/* recv[e][slot[i]][:] = x[i / K][:] for every kept pair i; every other row is left as it is. */
void oracle_dispatch(int T, int H, int E, int K, int C, const uint16_t *x,
                     const int32_t *topk_idx, const int32_t *slot, uint16_t *recv)
{
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j) {
            long i = (long)t * K + j;
            int32_t e = topk_idx[i], s = slot[i];
            if (!pair_kept(e, s, E, C)) continue;
            uint16_t *dst = recv + ((long)e * C + s) * H;
            for (int h = 0; h < H; ++h) dst[h] = x[(long)t * H + h];
        }
}

/*
 * FP8 dispatch. Token t is quantised once, per block b of 128 channels:
 *   amax  = max_h |x[t][h]|                    (exact in fp32)
 *   scale = amax / 448                          (one IEEE fp32 division)
 *   q[h]  = e4m3_rne_sat(x[t][h] / scale)      (one IEEE fp32 division per element)
 * If amax == 0 every x in the block is +-0 and q is that signed zero (scale = 0).
 * Then the q row and the scale row are written to every kept slot of t:
 *   recv_q[e][s][h] = q[h];  recv_scale[e][s][b] = scale_b.
 *
 * Non-finite input (the pages give no rule; this is the library's policy, so that both sides
 * give the same bits):
 *   - a NaN anywhere in the block makes amax NaN (NaN propagates through the max);
 *   - a NaN amax gives the quiet NaN 0x7FC00000 as the scale (not x's payload);
 *   - every code carries x's sign bit: the sign of a quotient is the exclusive-or of the
 *     operands' signs, and the scale is never negative. IEEE 754 fixes that rule for every
 *     result but NaN; it is applied to NaN quotients too, so a NaN quotient (x / NaN, or
 *     +-inf / inf) encodes as sign(x) | 0x7F. An infinite amax gives an infinite scale, so the
 *     finite elements of that block encode as signed zeros.
 */
static void quantise_token(int H, const uint16_t *row, uint8_t *q, float *sc)
{
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int h = 128 * b; h < 128 * b + 128; ++h) {
            float a = fabsf(oracle_bf16_to_f32(row[h]));
            if (isnan(a) || a > amax) amax = a;
            if (isnan(amax)) break;
        }
        float scale = isnan(amax) ? f32_from_bits(0x7FC00000u) : amax / 448.0f;
        sc[b] = scale;
        for (int h = 128 * b; h < 128 * b + 128; ++h) {
            float v = oracle_bf16_to_f32(row[h]);
            uint8_t sign = (row[h] & 0x8000u) ? 0x80 : 0x00;
            q[h] = (amax == 0.0f) ? sign
                                  : (uint8_t)(sign | (oracle_e4m3_rne_sat(v / scale) & 0x7F));
        }
    }
}

void oracle_dispatch_fp8(int T, int H, int E, int K, int C, const uint16_t *x,
                         const int32_t *topk_idx, const int32_t *slot, uint8_t *recv_q,
                         float *recv_scale)
{
    int NB = H / 128;
    uint8_t *q = xcalloc((size_t)H, sizeof *q);
    float *sc = xcalloc((size_t)NB, sizeof *sc);
    for (int t = 0; t < T; ++t) {
        quantise_token(H, x + (long)t * H, q, sc);
        for (int j = 0; j < K; ++j) {
            long i = (long)t * K + j;
            int32_t e = topk_idx[i], s = slot[i];
            if (!pair_kept(e, s, E, C)) continue;
            long r = (long)e * C + s;
            memcpy(recv_q + r * H, q, (size_t)H);
            memcpy(recv_scale + r * NB, sc, (size_t)NB * sizeof(float));
        }
    }
    free(q);
    free(sc);
}

/* ----------------------------------------------------------------------------------------- */
/* Combine                                                                                    */
/* ----------------------------------------------------------------------------------------- */

/*
 * out[t][h] = bf16_rne(acc), acc = +0.0f, then for j = 0 .. K-1 with pair i = t*K + j kept:
 *   acc = fmaf(w[i], float(y[e_i][slot_i][h]), acc)
 * Dropped, unrouted and invalid pairs are skipped; the remaining weights are used as given.
 */
void oracle_combine(int T, int H, int E, int K, int C, const uint16_t *y,
                    const int32_t *topk_idx, const int32_t *slot, const float *topk_w,
                    uint16_t *out)
{
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < K; ++j) {
                long i = (long)t * K + j;
                int32_t e = topk_idx[i], s = slot[i];
                if (!pair_kept(e, s, E, C)) continue;
                float v = oracle_bf16_to_f32(y[((long)e * C + s) * H + h]);
                acc = fmaf(topk_w[i], v, acc);
            }
            out[(long)t * H + h] = oracle_bf16_rne(acc);
        }
}

/* ----------------------------------------------------------------------------------------- */
/* Two-stage path: one copy per (token, virtual rank), then the rank's own expansion           */
/* ----------------------------------------------------------------------------------------- */

/*
 * Rank layout. Expert e belongs to virtual rank e / (E/R). Token t is sent to rank r if any of
 * its pairs holds a valid id (0 <= id < E) of an expert of r, whatever the capacity decides.
 *   rank_slot[t][r] = #{t' < t : t' is sent to r} if t is sent to r, else -1
 *   rank_tokens[r]  = #{t : t is sent to r}
 */
void oracle_rank_layout(int T, int K, int E, int R, const int32_t *topk_idx, int32_t *rank_slot,
                        int32_t *rank_tokens)
{
    int EL = E / R;
    for (int r = 0; r < R; ++r) rank_tokens[r] = 0;
    for (int t = 0; t < T; ++t) {
        int32_t *rs = rank_slot + (long)t * R;
        for (int r = 0; r < R; ++r) rs[r] = -1;
        for (int j = 0; j < K; ++j) {
            int32_t e = topk_idx[(long)t * K + j];
            if (e < 0 || e >= E) continue;
            int r = e / EL;
            if (rs[r] < 0) rs[r] = rank_tokens[r]++;
        }
    }
}

/* Stage 1 of dispatch: stage[r][rank_slot[t][r]][:] = x[t][:] for every rank t is sent to
 * (stage is [R][T][H]); every other row is left as it is. */
void oracle_dispatch_ranks(int T, int H, int R, const uint16_t *x, const int32_t *rank_slot,
                           uint16_t *stage)
{
    for (int t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) {
            int32_t p = rank_slot[(long)t * R + r];
            if (p < 0) continue;
            memcpy(stage + ((long)r * T + p) * H, x + (long)t * H, (size_t)H * sizeof(uint16_t));
        }
}

/* FP8 stage 1: token t quantised once (as in oracle_dispatch_fp8), its codes and scales
 * written to stage_q[r][p] ([R][T][H]) and stage_scale[r][p] ([R][T][H/128]). */
void oracle_dispatch_ranks_fp8(int T, int H, int R, const uint16_t *x, const int32_t *rank_slot,
                               uint8_t *stage_q, float *stage_scale)
{
    int NB = H / 128;
    uint8_t *q = xcalloc((size_t)H, sizeof *q);
    float *sc = xcalloc((size_t)NB, sizeof *sc);
    for (int t = 0; t < T; ++t) {
        quantise_token(H, x + (long)t * H, q, sc);
        for (int r = 0; r < R; ++r) {
            int32_t p = rank_slot[(long)t * R + r];
            if (p < 0) continue;
            memcpy(stage_q + ((long)r * T + p) * H, q, (size_t)H);
            memcpy(stage_scale + ((long)r * T + p) * NB, sc, (size_t)NB * sizeof(float));
        }
    }
    free(q);
    free(sc);
}

/* Stage 2 of dispatch, the rank's own expansion: for every kept pair i = t*K + j of expert e
 * (rank r = e / (E/R)), recv[e][slot[i]][:] = stage[r][rank_slot[t][r]][:]. */
void oracle_dispatch_expand(int T, int H, int E, int K, int C, int R, const uint16_t *stage,
                            const int32_t *topk_idx, const int32_t *slot,
                            const int32_t *rank_slot, uint16_t *recv)
{
    int EL = E / R;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j) {
            long i = (long)t * K + j;
            int32_t e = topk_idx[i], s = slot[i];
            if (!pair_kept(e, s, E, C)) continue;
            int r = e / EL;
            int32_t p = rank_slot[(long)t * R + r];
            if (p < 0) continue;
            memcpy(recv + ((long)e * C + s) * H, stage + ((long)r * T + p) * H,
                   (size_t)H * sizeof(uint16_t));
        }
}

/* FP8 stage 2: codes and scales of the staged row copied to every kept pair's row. */
void oracle_dispatch_expand_fp8(int T, int H, int E, int K, int C, int R, const uint8_t *stage_q,
                                const float *stage_scale, const int32_t *topk_idx,
                                const int32_t *slot, const int32_t *rank_slot, uint8_t *recv_q,
                                float *recv_scale)
{
    int EL = E / R, NB = H / 128;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j) {
            long i = (long)t * K + j;
            int32_t e = topk_idx[i], s = slot[i];
            if (!pair_kept(e, s, E, C)) continue;
            int r = e / EL;
            int32_t p = rank_slot[(long)t * R + r];
            if (p < 0) continue;
            long dst = (long)e * C + s, src = (long)r * T + p;
            memcpy(recv_q + dst * H, stage_q + src * H, (size_t)H);
            memcpy(recv_scale + dst * NB, stage_scale + src * NB, (size_t)NB * sizeof(float));
        }
}

/*
 * Stage 1 of combine, on each rank: one partial row per token sent to the rank,
 *   part[r][rank_slot[t][r]][h] = bf16_rne(acc), acc = +0.0f, then for j = 0 .. K-1 with pair
 *   i = t*K + j kept and its expert in rank r: acc = fmaf(w[i], float(y[e_i][slot_i][h]), acc).
 * A token sent to r whose pairs there were all dropped gets a +0 row.
 */
void oracle_combine_ranks(int T, int H, int E, int K, int C, int R, const uint16_t *y,
                          const int32_t *topk_idx, const int32_t *slot,
                          const int32_t *rank_slot, const float *topk_w, uint16_t *part)
{
    int EL = E / R;
    for (int t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) {
            int32_t p = rank_slot[(long)t * R + r];
            if (p < 0) continue;
            uint16_t *dst = part + ((long)r * T + p) * H;
            for (int h = 0; h < H; ++h) {
                float acc = 0.0f;
                for (int j = 0; j < K; ++j) {
                    long i = (long)t * K + j;
                    int32_t e = topk_idx[i], s = slot[i];
                    if (!pair_kept(e, s, E, C) || e / EL != r) continue;
                    acc = fmaf(topk_w[i], oracle_bf16_to_f32(y[((long)e * C + s) * H + h]), acc);
                }
                dst[h] = oracle_bf16_rne(acc);
            }
        }
}

/* Stage 2 of combine, on the token's side: out[t][h] = bf16_rne(acc), acc = +0.0f, then for
 * r = 0 .. R-1 with t sent to r: acc = acc + float(part[r][rank_slot[t][r]][h]). */
void oracle_combine_reduce(int T, int H, int R, const uint16_t *part, const int32_t *rank_slot,
                           uint16_t *out)
{
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) {
                int32_t p = rank_slot[(long)t * R + r];
                if (p < 0) continue;
                acc = acc + oracle_bf16_to_f32(part[((long)r * T + p) * H + h]);
            }
            out[(long)t * H + h] = oracle_bf16_rne(acc);
        }
}

/* The two-stage combine for a subset of tokens: out row n is token tokens[n]. The token's
 * per-rank partials are formed as in oracle_combine_ranks (rounded to bf16) and summed as in
 * oracle_combine_reduce. */
void oracle_combine_two_stage_tokens(int n_tokens, const int32_t *tokens, int H, int E, int K,
                                     int C, int R, const uint16_t *y, const int32_t *topk_idx,
                                     const int32_t *slot, const int32_t *rank_slot,
                                     const float *topk_w, uint16_t *out)
{
    int EL = E / R;
    for (int n = 0; n < n_tokens; ++n) {
        int t = tokens[n];
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) {
                if (rank_slot[(long)t * R + r] < 0) continue;
                float part = 0.0f;
                for (int j = 0; j < K; ++j) {
                    long i = (long)t * K + j;
                    int32_t e = topk_idx[i], s = slot[i];
                    if (!pair_kept(e, s, E, C) || e / EL != r) continue;
                    part = fmaf(topk_w[i], oracle_bf16_to_f32(y[((long)e * C + s) * H + h]), part);
                }
                acc = acc + oracle_bf16_to_f32(oracle_bf16_rne(part));
            }
            out[(long)n * H + h] = oracle_bf16_rne(acc);
        }
    }
}

/* ----------------------------------------------------------------------------------------- */
/* Packed, aligned receive layout                                                             */
/* ----------------------------------------------------------------------------------------- */

/* offset[0] = 0, offset[e + 1] = offset[e] + (count[e] rounded up to a multiple of align);
 * offset[E] is the number of rows the packed buffer needs. */
void oracle_packed_offsets(int E, int align, const int32_t *count, int32_t *offset)
{
    offset[0] = 0;
    for (int e = 0; e < E; ++e) {
        int32_t padded = (count[e] + align - 1) / align * align;
        offset[e + 1] = offset[e] + padded;
    }
}

/* Row of a kept pair in a packed buffer of `rows` rows, or -1. */
static long packed_row(int32_t e, int32_t s, int E, int C, const int32_t *offset, int rows)
{
    if (!pair_kept(e, s, E, C)) return -1;
    long r = (long)offset[e] + s;
    return (r >= 0 && r < rows) ? r : -1;
}

/* recv[offset[e] + slot[i]][:] = x[i / K][:] for every kept pair i; other rows as they are. */
void oracle_dispatch_packed(int T, int H, int E, int K, int C, int rows, const uint16_t *x,
                            const int32_t *topk_idx, const int32_t *slot, const int32_t *offset,
                            uint16_t *recv)
{
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j) {
            long i = (long)t * K + j;
            long r = packed_row(topk_idx[i], slot[i], E, C, offset, rows);
            if (r < 0) continue;
            memcpy(recv + r * H, x + (long)t * H, (size_t)H * sizeof(uint16_t));
        }
}

/* FP8 into the packed layout: token t quantised once, codes and scales to every kept row. */
void oracle_dispatch_packed_fp8(int T, int H, int E, int K, int C, int rows, const uint16_t *x,
                                const int32_t *topk_idx, const int32_t *slot,
                                const int32_t *offset, uint8_t *recv_q, float *recv_scale)
{
    int NB = H / 128;
    uint8_t *q = xcalloc((size_t)H, sizeof *q);
    float *sc = xcalloc((size_t)NB, sizeof *sc);
    for (int t = 0; t < T; ++t) {
        quantise_token(H, x + (long)t * H, q, sc);
        for (int j = 0; j < K; ++j) {
            long i = (long)t * K + j;
            long r = packed_row(topk_idx[i], slot[i], E, C, offset, rows);
            if (r < 0) continue;
            memcpy(recv_q + r * H, q, (size_t)H);
            memcpy(recv_scale + r * NB, sc, (size_t)NB * sizeof(float));
        }
    }
    free(q);
    free(sc);
}

/* Combine from the packed layout: as oracle_combine with y[e][slot] at row offset[e] + slot. */
void oracle_combine_packed(int T, int H, int E, int K, int C, int rows, const uint16_t *y,
                           const int32_t *topk_idx, const int32_t *slot, const int32_t *offset,
                           const float *topk_w, uint16_t *out)
{
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < K; ++j) {
                long i = (long)t * K + j;
                long r = packed_row(topk_idx[i], slot[i], E, C, offset, rows);
                if (r < 0) continue;
                acc = fmaf(topk_w[i], oracle_bf16_to_f32(y[r * H + h]), acc);
            }
            out[(long)t * H + h] = oracle_bf16_rne(acc);
        }
}

/* Same as oracle_combine for a subset of tokens: out row n is token tokens[n]. */
void oracle_combine_tokens(int n_tokens, const int32_t *tokens, int H, int E, int K, int C,
                           const uint16_t *y, const int32_t *topk_idx, const int32_t *slot,
                           const float *topk_w, uint16_t *out)
{
    for (int n = 0; n < n_tokens; ++n) {
        int t = tokens[n];
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < K; ++j) {
                long i = (long)t * K + j;
                int32_t e = topk_idx[i], s = slot[i];
                if (!pair_kept(e, s, E, C)) continue;
                float v = oracle_bf16_to_f32(y[((long)e * C + s) * H + h]);
                acc = fmaf(topk_w[i], v, acc);
            }
            out[(long)n * H + h] = oracle_bf16_rne(acc);
        }
    }
}

/* Array forms of the two conversions, for the exhaustive format tests. */
void oracle_bf16_rne_array(const float *in, uint16_t *out, long n)
{
    for (long k = 0; k < n; ++k) out[k] = oracle_bf16_rne(in[k]);
}

void oracle_e4m3_rne_sat_array(const float *in, uint8_t *out, long n)
{
    for (long k = 0; k < n; ++k) out[k] = oracle_e4m3_rne_sat(in[k]);
}
