/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel layout / dispatch / combine
 * library (libep_mi355x.so).
 *
 * One GPU's share of expert-parallel dispatch and combine. T tokens, each routed to K experts
 * out of E, are placed into a receive buffer of E experts x C rows (capacity) x H channels.
 * The E experts form R "virtual ranks" of E/R consecutive experts, so the buffer
 * [E][C][H] is rank-major: expert e = r*(E/R) + l. Every operation below is the local part of
 * what the reference pages describe around the inter-GPU transport, which is not part of this
 * library.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller (for example the storage of
 *    torch tensors). The library never allocates, frees or synchronises: each call checks its
 *    arguments on the host, enqueues its kernels on `stream` (0 = the null stream) and returns.
 *    Its only device memory of its own is static, in the loaded code object: two 64 KiB rows of
 *    zeros that combine and the two-stage reduce read, and never write, in place of pairs or
 *    partial rows that are not there.
 *  - bf16 values are passed as their 16-bit patterns (uint16_t); FP8 values as OCP E4M3 codes
 *    (uint8_t, OFP8 specification rev. 1.0: bias 7, 3 mantissa bits, max 448, S.1111.111 NaN).
 *  - Pair index i = t*K + j names choice j of token t ("token order").
 *  - Return value: EP_OK, or a negative EP_ERR_* code. On an argument error nothing is enqueued.
 *    EP_ERR_HIP means a HIP launch failed; ep_last_error() gives the text. Errors inside a
 *    kernel cannot be seen without a synchronisation and are avoided by construction: expert ids
 *    and slots are range-checked on the device, and out-of-range pairs are skipped.
 *  - The library is stateless and reentrant. Calls on one stream execute in order; calls on
 *    different streams that write the same buffers race, as any kernels would.
 */
#ifndef EP_MI355X_EP_H
#define EP_MI355X_EP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem shape. Requirements (else EP_ERR_INVALID): T >= 0, H >= 1, 1 <= K, 1 <= E,
 * 1 <= C, 1 <= R, E % R == 0, T*K <= INT32_MAX, E*C <= INT32_MAX. */
typedef struct ep_shape {
    int32_t T;   /* tokens on this GPU */
    int32_t H;   /* hidden size (channels per row) */
    int32_t E;   /* experts */
    int32_t K;   /* experts chosen per token (top-k) */
    int32_t C;   /* capacity: rows per expert in the receive buffer */
    int32_t R;   /* virtual ranks; each holds E/R consecutive experts */
} ep_shape_t;

enum {
    EP_OK = 0,
    EP_ERR_INVALID = -1,      /* bad shape, NULL required pointer */
    EP_ERR_ALIGN = -2,        /* a row buffer is not 16-byte aligned */
    EP_ERR_UNSUPPORTED = -3,  /* shape outside what the kernels support (see each call) */
    EP_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed */
};

#define EP_STATS_LEN 4         /* stats[] = {kept, dropped, unrouted, invalid} */
#define EP_MAX_EXPERTS 1024    /* largest E the layout kernel supports */
#define EP_MAX_TOPK 256        /* largest K dispatch and combine support */
#define EP_FP8_BLOCK 128       /* channels per FP8 scale */
#define EP_MAX_RANKS 64        /* largest R the two-stage (per-rank) calls support */

/*
 * ep_layout -- routing layout: per-expert counts, exclusive offsets and stable in-order slots
 * under the capacity C, with drops.
 *
 * The "normal" (throughput) EP APIs must compute this before dispatch, inside the timed
 * boundary (awsome-distributed-ai PR #1238, "What changed" and the author's reply on what the
 * latency means); the receive buffers are bounded by a fixed capacity (afdEP-comm validation
 * record, setup: capacity 2048).
 *
 *   topk_idx      [T*K] int32 in   expert of pair i; -1 = unrouted; other ids outside [0, E)
 *                                   are invalid. Both get slot -1 and are counted in stats.
 *                                   16-byte aligned (else EP_ERR_ALIGN).
 *   slot          [T*K] int32 out  #{i' < i : topk_idx[i'] == topk_idx[i]} if that is < C,
 *                                   else -1 (dropped: each expert keeps its first C pairs in
 *                                   token order). This is the handle dispatch and combine use.
 *   expert_count  [E]   int32 out  kept pairs per expert, min(demand, C)
 *   expert_offset [E]   int32 out  exclusive scan of expert_count in expert (rank-major) order
 *   rank_count    [R]   int32 out  kept pairs per virtual rank (may be NULL)
 *   rank_offset   [R]   int32 out  exclusive scan of rank_count (may be NULL)
 *   stats         [EP_STATS_LEN] int32 out  {kept, dropped, unrouted, invalid}; they sum to T*K
 *
 * Requires E <= EP_MAX_EXPERTS (else EP_ERR_UNSUPPORTED). T = 0 is allowed: counts, offsets
 * and stats are written as zeros. All outputs are bit-exact and deterministic.
 */
int ep_layout(const ep_shape_t *shape, const int32_t *topk_idx, int32_t *slot,
              int32_t *expert_count, int32_t *expert_offset, int32_t *rank_count,
              int32_t *rank_offset, int32_t *stats, hipStream_t stream);

/*
 * ep_dispatch -- bf16 scatter of token rows into the rank-major receive buffer.
 *
 * Each token row goes to the receive slot of every expert it selected; the receiving side
 * expands into this per-expert layout (afdEP-comm validation record, kernel_timelines:
 * dispatch_copy_epilogue).
 *
 *   x        [T*H]   uint16 (bf16) in   token rows, 16-byte aligned
 *   topk_idx [T*K]   int32 in, slot [T*K] int32 in (from ep_layout)
 *   recv     [E*C*H] uint16 (bf16) out  recv[e][slot[i]][:] = x[i / K][:] for every pair with
 *                                        0 <= e < E and 0 <= slot[i] < C; other rows untouched
 *
 * Requires H % 8 == 0 (16-byte rows) and K <= EP_MAX_TOPK (else EP_ERR_UNSUPPORTED).
 * Bit-exact copy.
 */
int ep_dispatch(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                const int32_t *slot, uint16_t *recv, hipStream_t stream);

/*
 * ep_dispatch_fp8 -- dispatch with the per-token FP8 cast fused in.
 *
 * Each token is cast once to OCP E4M3 with one fp32 scale per 128 channels, inside the
 * dispatch rather than as a separate pass before it (awsome-distributed-ai PR #1238, review
 * item 1: per_token_cast_to_fp8 outside the kernel versus low_latency_dispatch(use_fp8=True)
 * quantising inside; the logical payload counts H + 4*H/128 bytes per FP8 row). Per token t
 * and block b of channels [128b, 128b+128):
 *     amax  = max |x|;   scale = amax / 448 (IEEE fp32 division, round to nearest even)
 *     q     = e4m3(x / scale)  (IEEE fp32 division, then round to nearest even, saturating
 *             at +-448); if amax == 0 the block is all +-0, scale = 0 and q is that signed zero.
 * Then for every pair with 0 <= e < E and 0 <= slot[i] < C:
 *     recv_q[e][slot[i]][:] = q row,  recv_scale[e][slot[i]][:] = the H/128 scales.
 *
 *   x          [T*H]         uint16 (bf16) in, 16-byte aligned
 *   recv_q     [E*C*H]       uint8 out, 16-byte aligned
 *   recv_scale [E*C*(H/128)] float out, 4-byte aligned
 *
 * Non-finite x (the library's policy; every FP8 path follows it): a NaN in a block makes its
 * amax NaN and its scale the quiet NaN 0x7FC00000; every code carries x's own sign bit, so a
 * quotient that is NaN (x / NaN, +-inf / inf) encodes as sign(x) | 0x7F; an infinite amax gives
 * an infinite scale, and the block's finite values encode as signed zeros.
 *
 * Requires H % 128 == 0 and K <= EP_MAX_TOPK (else EP_ERR_UNSUPPORTED). Bit-exact.
 */
int ep_dispatch_fp8(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                    const int32_t *slot, uint8_t *recv_q, float *recv_scale,
                    hipStream_t stream);

/*
 * ep_layout_dispatch -- ep_layout and ep_dispatch in one launch.
 *
 * The layout is computed inside the same boundary as dispatch, as the "normal" EP APIs require
 * (awsome-distributed-ai PR #1238, "What changed"). Every output (slot, expert_count,
 * expert_offset, rank_count, rank_offset, stats, recv) is bit-identical to calling ep_layout
 * and then ep_dispatch with the same arguments. Each workgroup computes the slots of its own
 * tile of tokens and copies those tokens' rows at once, so there is no second launch and no
 * wait for the whole layout. Arguments, layouts, alignment and limits are the union of the two
 * calls' (E <= EP_MAX_EXPERTS, K <= EP_MAX_TOPK, H % 8 == 0, topk_idx / x / recv 16-byte
 * aligned).
 */
int ep_layout_dispatch(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                       int32_t *slot, int32_t *expert_count, int32_t *expert_offset,
                       int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                       uint16_t *recv, hipStream_t stream);

/*
 * ep_layout_dispatch_fp8 -- ep_layout and ep_dispatch_fp8 in one launch; bit-identical to the
 * two calls in sequence. Requires H % 128 == 0 in addition; recv_scale 4-byte aligned.
 */
int ep_layout_dispatch_fp8(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                           int32_t *slot, int32_t *expert_count, int32_t *expert_offset,
                           int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                           uint8_t *recv_q, float *recv_scale, hipStream_t stream);

/*
 * Large batches: the layout with a workspace.
 *
 * In ep_layout_dispatch every workgroup counts all the pairs before its tile, so the layout's
 * work grows with the square of T*K. The _ws calls split it: a first launch writes the
 * histogram of every chunk of 4096 pairs to a caller-provided workspace, and each tile of the
 * fused layout + dispatch then adds the histograms of the chunks before its own and counts
 * only the earlier pairs of its own chunk. Every output is bit-identical to ep_layout_dispatch
 * (ep_layout_dispatch_fp8); the second launch pays off on large batches (on MI355X from about
 * T*K = 2^16 pairs; below that the single launch is faster).
 *
 * ep_layout_workspace_bytes -- bytes the _ws calls need for this shape:
 *   ceil(T*K / 4096) * (E + 2) * 4 (0 for T*K = 0 or an invalid shape). Host only.
 * ep_layout_dispatch_ws / ep_layout_dispatch_fp8_ws -- the arguments of ep_layout_dispatch
 *   (ep_layout_dispatch_fp8), then:
 *   workspace       device memory owned by the caller, 16-byte aligned (else EP_ERR_ALIGN),
 *                   at least ep_layout_workspace_bytes(shape) bytes (else EP_ERR_INVALID);
 *                   overwritten by the call; nothing needs to be in it beforehand. Two calls
 *                   in flight at once need two workspaces.
 *   workspace_bytes its size.
 */
size_t ep_layout_workspace_bytes(const ep_shape_t *shape);

int ep_layout_dispatch_ws(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                          int32_t *slot, int32_t *expert_count, int32_t *expert_offset,
                          int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                          uint16_t *recv, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

int ep_layout_dispatch_fp8_ws(const ep_shape_t *shape, const uint16_t *x,
                              const int32_t *topk_idx, int32_t *slot, int32_t *expert_count,
                              int32_t *expert_offset, int32_t *rank_count, int32_t *rank_offset,
                              int32_t *stats, uint8_t *recv_q, float *recv_scale,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ep_layout_dispatch_noalloc -- ep_layout_dispatch_ws without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The chunk histograms go to the library's own static
 * scratch: 1 MiB of device memory per GPU, set aside when the library is loaded and held until
 * the process ends; the call itself allocates nothing. A shape whose
 * ep_layout_workspace_bytes exceeds 1 MiB (T*K above 4096 * floor(262144 / (E + 2)) pairs;
 * 8.2 M pairs at E = 128) is rejected with EP_ERR_UNSUPPORTED. Arguments and outputs are those
 * of ep_layout_dispatch, and the outputs are bit-identical to it. Every call on a GPU uses that
 * GPU's one scratch, so two calls that overlap on one GPU (different streams, no ordering)
 * race; calls on one stream are ordered and safe. Nothing in the scratch needs to be zero.
 */
int ep_layout_dispatch_noalloc(const ep_shape_t *shape, const uint16_t *x,
                               const int32_t *topk_idx, int32_t *slot, int32_t *expert_count,
                               int32_t *expert_offset, int32_t *rank_count, int32_t *rank_offset,
                               int32_t *stats, uint16_t *recv, hipStream_t stream);

/*
 * ep_combine -- top-k weighted gather-reduce of expert outputs back onto each token.
 *
 * Combine gathers the expert outputs and reduces them with the top-k weights on the token's
 * side (afdEP-comm validation record, kernel_timelines: combine_reduce_epilogue); it is BF16
 * whatever the dispatch dtype (awsome-distributed-ai PR #1238, review item 1).
 *
 *   y        [E*C*H] uint16 (bf16) in   expert outputs in the receive layout, 16-byte aligned
 *   topk_idx [T*K] int32 in, slot [T*K] int32 in (from ep_layout)
 *   topk_w   [T*K]   float in           top-k weights, used as given (no renormalisation)
 *   out      [T*H]   uint16 (bf16) out  16-byte aligned
 *
 *     out[t][h] = bf16_rne(acc), acc = +0.0f, then for j = 0 .. K-1 ascending, for each pair
 *     with 0 <= e < E and 0 <= slot < C:  acc = fmaf(topk_w[i], y[e][slot][h], acc)
 * Pairs that were dropped, unrouted or invalid contribute nothing; a token with none gives +0.
 * An element whose sum is NaN is written as the quiet NaN 0x7FC0 (whatever the sign and payload
 * of the NaNs that produced it; the same holds for every bf16 result of the library).
 * Requires H % 8 == 0 and K <= EP_MAX_TOPK (else EP_ERR_UNSUPPORTED). Deterministic; every
 * fp32 step is the one written above, so the result is bit-reproducible.
 */
int ep_combine(const ep_shape_t *shape, const uint16_t *y, const int32_t *topk_idx,
               const int32_t *slot, const float *topk_w, uint16_t *out, hipStream_t stream);

/*
 * Packed, aligned receive layout (for grouped-GEMM consumers).
 *
 * The pages run with DeepEP's expert_alignment = 1 (DeepEP-V2 on AWS EFA, the test_ep.py
 * cross-check); alignment A > 1 lets a grouped GEMM take each expert's rows in whole tiles.
 * Here each expert e takes align_up(expert_count[e], A) consecutive rows of a packed buffer
 * [rows][H] starting at packed_offset[e], the exclusive scan of those padded counts
 * (packed_offset[E] = the rows the buffer needs; at most min(T*K, E*C) + E*(A-1)). A kept pair
 * (t, j) of expert e lives in row packed_offset[e] + slot. Padding rows are never written or
 * read. The offsets need every expert's total: ep_layout_packed computes them as a call of its
 * own, and ep_layout_dispatch_packed has every workgroup count all pairs to fuse the two.
 */

/*
 * ep_layout_packed -- ep_layout with the packed offsets.
 *   alignment     >= 1 (1 gives the plain exclusive scan of expert_count)
 *   packed_offset [E+1] int32 out  as above
 *   rank_count / rank_offset (may be NULL): padded rows per rank and their exclusive scan, so a
 *                 rank's experts occupy rows [rank_offset[r], rank_offset[r] + rank_count[r])
 * slot, expert_count and stats are those of ep_layout. Requires E*(C + A - 1) <= INT32_MAX.
 */
int ep_layout_packed(const ep_shape_t *shape, int32_t alignment, const int32_t *topk_idx,
                     int32_t *slot, int32_t *expert_count, int32_t *packed_offset,
                     int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                     hipStream_t stream);

/*
 * ep_dispatch_packed / ep_dispatch_packed_fp8 -- ep_dispatch / ep_dispatch_fp8 into a packed
 * buffer of `rows` rows (recv [rows*H]; recv_q [rows*H], recv_scale [rows*(H/128)]): row
 * packed_offset[e] + slot for every kept pair, skipped if that is not below `rows`. Other rows
 * untouched. The rules of the padded calls apply otherwise.
 */
int ep_dispatch_packed(const ep_shape_t *shape, int32_t rows, const uint16_t *x,
                       const int32_t *topk_idx, const int32_t *slot,
                       const int32_t *packed_offset, uint16_t *recv, hipStream_t stream);

int ep_dispatch_packed_fp8(const ep_shape_t *shape, int32_t rows, const uint16_t *x,
                           const int32_t *topk_idx, const int32_t *slot,
                           const int32_t *packed_offset, uint8_t *recv_q, float *recv_scale,
                           hipStream_t stream);

/*
 * ep_layout_dispatch_packed / ep_layout_dispatch_packed_fp8 -- ep_layout_packed followed by
 * ep_dispatch_packed / ep_dispatch_packed_fp8 into a buffer of `rows` rows, in one launch:
 * every workgroup counts all pairs, so it knows the packed offsets without waiting for the
 * others. Outputs are bit-identical to the two calls and the rules of both apply (alignment
 * >= 1, rows >= 0, topk_idx / x / recv / recv_q 16-byte aligned, recv_scale 4-byte aligned).
 * For large E (the layout's two histograms beyond 64 KB of LDS, E above ~320) the call runs
 * the two steps as two launches.
 */
int ep_layout_dispatch_packed(const ep_shape_t *shape, int32_t alignment, int32_t rows,
                              const uint16_t *x, const int32_t *topk_idx, int32_t *slot,
                              int32_t *expert_count, int32_t *packed_offset, int32_t *rank_count,
                              int32_t *rank_offset, int32_t *stats, uint16_t *recv,
                              hipStream_t stream);

int ep_layout_dispatch_packed_fp8(const ep_shape_t *shape, int32_t alignment, int32_t rows,
                                  const uint16_t *x, const int32_t *topk_idx, int32_t *slot,
                                  int32_t *expert_count, int32_t *packed_offset,
                                  int32_t *rank_count, int32_t *rank_offset, int32_t *stats,
                                  uint8_t *recv_q, float *recv_scale, hipStream_t stream);

/*
 * ep_combine_packed -- ep_combine reading y from a packed buffer of `rows` rows: the expert row
 * of a kept pair is y[packed_offset[e] + slot] (a pair whose row is not below `rows` counts as
 * dropped). Same arithmetic, bit for bit, as ep_combine on the padded buffer.
 */
int ep_combine_packed(const ep_shape_t *shape, int32_t rows, const uint16_t *y,
                      const int32_t *topk_idx, const int32_t *slot, const int32_t *packed_offset,
                      const float *topk_w, uint16_t *out, hipStream_t stream);

/*
 * Two-stage, rank-deduplicated path.
 *
 * The pages' kernel chain moves a token to each virtual rank once (dispatch_impl), and the
 * rank expands it into its experts' rows (dispatch_copy_epilogue); on the way back each rank
 * reduces its experts' outputs per token (combine_impl) before the final top-k reduction on the
 * token's side (combine_reduce_epilogue) (afdEP-comm validation record, kernel_timelines). Here
 * the "transport" is a staging buffer in the same HBM, rank-major: stage[R][T][row], where row
 * p of rank r holds the p-th token (in token order) sent to r. Composed, the calls give the
 * one-stage results: ep_dispatch_ranks + ep_dispatch_expand leave recv exactly as ep_dispatch
 * does (likewise for FP8); ep_combine_ranks + ep_combine_reduce compute the combine with the
 * per-rank partial rounded to bf16 (the precision a rank would send back) and the partials
 * summed in fp32 in ascending rank, which is bit-identical to ep_combine when R = 1.
 *
 * Common requirements (else EP_ERR_UNSUPPORTED): R <= EP_MAX_RANKS, E <= EP_MAX_EXPERTS,
 * R*T <= INT32_MAX; the row-buffer alignment and H rules of the one-stage calls.
 */

/*
 * ep_rank_layout -- which virtual ranks each token goes to, and where.
 *
 * Token t is sent to rank r if any of its ids is a valid expert (0 <= id < E) of rank r,
 * whatever the capacity decides later (the sender sees only the routing).
 *   topk_idx    [T*K] int32 in   16-byte aligned
 *   rank_slot   [T*R] int32 out  #{t' < t : t' sent to r} if t is sent to r, else -1;
 *                                 16-byte aligned
 *   rank_tokens [R]   int32 out  number of tokens sent to each rank
 * T = 0 writes rank_tokens as zeros. Bit-exact and deterministic.
 */
int ep_rank_layout(const ep_shape_t *shape, const int32_t *topk_idx, int32_t *rank_slot,
                   int32_t *rank_tokens, hipStream_t stream);

/*
 * ep_dispatch_ranks -- stage 1 of dispatch: each token row copied once to every rank it is
 * sent to. stage [R*T*H] uint16 (bf16) out, 16-byte aligned: stage[r][rank_slot[t][r]][:] =
 * x[t][:]; rows of tokens a rank does not receive are untouched. H % 8 == 0.
 */
int ep_dispatch_ranks(const ep_shape_t *shape, const uint16_t *x, const int32_t *rank_slot,
                      uint16_t *stage, hipStream_t stream);

/*
 * ep_dispatch_ranks_fp8 -- stage 1 with the FP8 cast: each token quantised once (exactly as in
 * ep_dispatch_fp8) and its codes / scales written to stage_q [R*T*H] uint8 (16-byte aligned)
 * and stage_scale [R*T*(H/128)] float (4-byte aligned) at row rank_slot[t][r] of each rank.
 * H % 128 == 0.
 */
int ep_dispatch_ranks_fp8(const ep_shape_t *shape, const uint16_t *x, const int32_t *rank_slot,
                          uint8_t *stage_q, float *stage_scale, hipStream_t stream);

/*
 * ep_rank_layout_dispatch / ep_rank_layout_dispatch_fp8 -- ep_rank_layout and
 * ep_dispatch_ranks (or ep_dispatch_ranks_fp8) in one launch: each workgroup ranks a tile of
 * tokens against all earlier ones and copies the tile's rows to their staging rows at once, so
 * the layout overlaps the copies. Outputs (rank_slot, rank_tokens, stage / stage_q +
 * stage_scale) are bit-identical to those of the two calls; the argument rules are theirs
 * combined (topk_idx, x, stage / stage_q 16-byte aligned; rank_slot needs no alignment here).
 * T = 0 writes rank_tokens as zeros and nothing else.
 */
int ep_rank_layout_dispatch(const ep_shape_t *shape, const uint16_t *x, const int32_t *topk_idx,
                            int32_t *rank_slot, int32_t *rank_tokens, uint16_t *stage,
                            hipStream_t stream);

int ep_rank_layout_dispatch_fp8(const ep_shape_t *shape, const uint16_t *x,
                                const int32_t *topk_idx, int32_t *rank_slot,
                                int32_t *rank_tokens, uint8_t *stage_q, float *stage_scale,
                                hipStream_t stream);

/*
 * ep_dispatch_expand -- stage 2 of dispatch, each rank's own expansion: for every pair i = t*K
 * + j with 0 <= e < E and 0 <= slot[i] < C, recv[e][slot[i]][:] = stage[e / (E/R)]
 * [rank_slot[t][e / (E/R)]][:]. Other rows of recv are untouched. K <= EP_MAX_TOPK, H % 8 == 0.
 */
int ep_dispatch_expand(const ep_shape_t *shape, const uint16_t *stage, const int32_t *topk_idx,
                       const int32_t *slot, const int32_t *rank_slot, uint16_t *recv,
                       hipStream_t stream);

/*
 * ep_layout_dispatch_expand -- ep_layout and ep_dispatch_expand in one launch: each workgroup
 * lays out a tile of tokens against all earlier ones (as ep_layout_dispatch does) and copies
 * the tile's kept pairs from their ranks' staging rows at once. Outputs (slot, expert_count,
 * expert_offset, rank_count, rank_offset, stats, recv) are bit-identical to those of the two
 * calls, and so are the argument rules (stage and recv 16-byte aligned; rank_count and
 * rank_offset may be NULL). rank_slot is read, not written. bf16 only; H % 8 == 0.
 */
int ep_layout_dispatch_expand(const ep_shape_t *shape, const uint16_t *stage,
                              const int32_t *topk_idx, const int32_t *rank_slot, int32_t *slot,
                              int32_t *expert_count, int32_t *expert_offset, int32_t *rank_count,
                              int32_t *rank_offset, int32_t *stats, uint16_t *recv,
                              hipStream_t stream);

/*
 * ep_layout_dispatch_expand_fp8 -- ep_layout and ep_dispatch_expand_fp8 in one launch, as
 * ep_layout_dispatch_expand: the layout outputs, recv_q and recv_scale are bit-identical to
 * those of the two calls, with their argument rules (stage_q and recv_q 16-byte aligned, the
 * scales 4-byte aligned, H % 128 == 0).
 */
int ep_layout_dispatch_expand_fp8(const ep_shape_t *shape, const uint8_t *stage_q,
                                  const float *stage_scale, const int32_t *topk_idx,
                                  const int32_t *rank_slot, int32_t *slot, int32_t *expert_count,
                                  int32_t *expert_offset, int32_t *rank_count,
                                  int32_t *rank_offset, int32_t *stats, uint8_t *recv_q,
                                  float *recv_scale, hipStream_t stream);

/*
 * ep_dispatch_expand_fp8 -- stage 2 for FP8: codes and scales of the staged row copied to every
 * kept pair's row of recv_q / recv_scale. H % 128 == 0.
 */
int ep_dispatch_expand_fp8(const ep_shape_t *shape, const uint8_t *stage_q,
                           const float *stage_scale, const int32_t *topk_idx,
                           const int32_t *slot, const int32_t *rank_slot, uint8_t *recv_q,
                           float *recv_scale, hipStream_t stream);

/*
 * ep_combine_ranks -- stage 1 of combine, on each rank: one partial row per token the rank
 * received,
 *   part[r][rank_slot[t][r]][h] = bf16_rne(acc), acc = +0.0f, then for j = 0 .. K-1 ascending,
 *   for each kept pair of t whose expert is in rank r: acc = fmaf(topk_w[i], y[e][slot][h], acc)
 * (+0 if all of t's pairs in r were dropped). part [R*T*H] uint16 (bf16), 16-byte aligned; rows
 * of tokens a rank did not receive are untouched. K <= EP_MAX_TOPK, H % 8 == 0.
 */
int ep_combine_ranks(const ep_shape_t *shape, const uint16_t *y, const int32_t *topk_idx,
                     const int32_t *slot, const int32_t *rank_slot, const float *topk_w,
                     uint16_t *part, hipStream_t stream);

/*
 * ep_combine_reduce -- stage 2 of combine, on the token's side:
 *   out[t][h] = bf16_rne(acc), acc = +0.0f, then for r = 0 .. R-1 ascending with t sent to r:
 *   acc = acc + float(part[r][rank_slot[t][r]][h])   (one IEEE fp32 addition each)
 * A token sent nowhere gives +0. out [T*H] uint16 (bf16), 16-byte aligned. H % 8 == 0.
 */
int ep_combine_reduce(const ep_shape_t *shape, const uint16_t *part, const int32_t *rank_slot,
                      uint16_t *out, hipStream_t stream);

/*
 * ep_check_e4m3_conversion -- self-check of the two OCP E4M3 encoders of the FP8 dispatch on
 * the current device.
 *
 * The FP8 cast (ep_dispatch_fp8 and every call that quantises) encodes its quotients x / scale
 * with gfx950's packed fp32 -> E4M3 conversion instruction whenever every block amax of a
 * wavefront's rows is finite and at least 2^-60; then every quotient lies in
 * [-448 (1 + 2^-22), 448 (1 + 2^-22)]. Otherwise it uses a software encoder: round to nearest
 * even, saturating at +-448, NaN -> S.1111.111 (OFP8 specification rev. 1.0, "satfinite"
 * conversion). The fast path is right only where the two agree. This call compares them on
 * every fp32 bit pattern u in [first_pattern, first_pattern + count) (first_pattern + count
 * <= 2^32, else EP_ERR_INVALID):
 *   mismatches     [1] uint32 device out  number of patterns whose two codes differ
 *   first_mismatch [1] uint32 device out  the smallest such pattern (0xFFFFFFFF if none)
 * Both 4-byte aligned (else EP_ERR_ALIGN). Enqueued on `stream` like every other call; the
 * results are there once the stream reaches them.
 */
int ep_check_e4m3_conversion(uint32_t first_pattern, uint32_t count, uint32_t *mismatches,
                             uint32_t *first_mismatch, hipStream_t stream);

/*
 * ep_last_launches -- the kernel launches of the calling thread's most recent call (any entry
 * point above that computes), for recording launch shapes beside measurements (the grid and
 * workgroup sizes a benchmark ran with; awsome-distributed-ai PR #1238, review item 4).
 * Fills up to `capacity` records and returns the number of launches the call made (0 if its
 * arguments were rejected). `kernel` points to the runtime's static copy of the kernel's
 * symbol name (its template arguments give the pair-group size and chunks per lane);
 * vgprs, static_lds_bytes, private_bytes and max_threads_per_block come from
 * hipFuncGetAttributes (-1 if the runtime did not give them). Host memory; no GPU work.
 */
typedef struct ep_launch_record {
    const char *kernel;
    uint32_t grid_x, grid_y, grid_z;        /* workgroups */
    uint32_t block_x, block_y, block_z;     /* lanes per workgroup */
    uint32_t dynamic_lds_bytes;             /* LDS requested at launch */
    uint32_t static_lds_bytes;              /* LDS the kernel declares */
    int32_t vgprs;                          /* vector registers per lane */
    uint32_t private_bytes;                 /* scratch per lane (0: no spills to memory) */
    int32_t max_threads_per_block;
} ep_launch_record_t;

int ep_last_launches(ep_launch_record_t *records, int capacity);

/* Static text for an EP_* code. */
const char *ep_error_string(int code);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *ep_last_error(void);

/* Library version string, including the HIP runtime version it was built against. */
const char *ep_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_EP_H */
