"""Pins for the oracle's two-stage, rank-deduplicated path (CPU only).

The pages' kernel chain sends a token to each virtual rank once (dispatch_impl), expands it
into the rank's expert rows there (dispatch_copy_epilogue), and on the way back reduces per
rank before the final top-k reduction on the token's side (combine_impl, then
combine_reduce_epilogue; afdEP-comm validation record, kernel_timelines). Readings: a token
goes to rank r if any of its valid ids is an expert of r; a rank's tokens keep token order;
the per-rank partial is the ascending-j fmaf fold over the token's kept pairs of that rank,
rounded once to bf16; the final row is the fp32 sum of the partials in ascending rank,
rounded once to bf16.

Pins used here, none of which restates the oracle's loops:
  * rank layout: counting the earlier tokens directly (brute force); a numpy cumulative sum
    over the sent-matrix; with one expert per rank it reduces to the (pinned) expert layout;
  * dispatch: stage 1 then stage 2 is exactly the (pinned) one-stage dispatch, bf16 and FP8;
  * combine: with a single rank it is the (pinned) one-stage combine; two closed forms, the
    identity law (y = recv, unit weights) and one expert per rank, computed with torch's CPU
    bf16 cast and numpy float32 sums in rank order; a rank whose pairs were all dropped
    returns an exact +0 row.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_06_amd import workloads as W

SENT16 = np.uint16(0xBEEF)


def torch_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns by torch's CPU cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def same_up_to_zero_sign(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit-equal, except that +0 and -0 count as equal."""
    a, b = a.astype(np.uint16), b.astype(np.uint16)
    z = lambda v: (v & 0x7FFF) == 0
    return bool(np.all((a == b) | (z(a) & z(b))))


def sent_matrix(idx: np.ndarray, E: int, R: int) -> np.ndarray:
    EL = E // R
    valid = (idx >= 0) & (idx < E)
    rank = np.where(valid, idx // EL, -1)
    return np.stack([(rank == r).any(axis=1) for r in range(R)], axis=1)


def random_case(T, H, E, K, C, R, seed, lo=-2):
    rng = np.random.default_rng(seed)
    idx = rng.integers(lo, E + 1, size=(T, K)).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.random((T, K)).astype(np.float32)
    return idx, x, w


# ------------------------------------------------------------------------------------------
# rank layout
# ------------------------------------------------------------------------------------------

def brute_rank_layout(idx, E, R):
    T, K = idx.shape
    EL = E // R
    sent = [[any(0 <= idx[t, j] < E and idx[t, j] // EL == r for j in range(K))
             for r in range(R)] for t in range(T)]
    rs = np.full((T, R), -1, np.int32)
    for t in range(T):
        for r in range(R):
            if sent[t][r]:
                rs[t, r] = sum(1 for u in range(t) if sent[u][r])
    return rs, np.array([sum(sent[t][r] for t in range(T)) for r in range(R)], np.int32)


@pytest.mark.parametrize("T,K", [(1, 1), (1, 3), (2, 2), (4, 1)])
@pytest.mark.parametrize("R", [1, 2, 4])
def test_rank_layout_exhaustive_tiny(T, K, R):
    E = 4
    ids = [-2, -1, 0, 1, 2, 3, 4]
    for combo in itertools.product(ids, repeat=T * K):
        idx = np.array(combo, np.int32).reshape(T, K)
        got = oracle.rank_layout(idx, E, R)
        rs, rt = brute_rank_layout(idx, E, R)
        assert np.array_equal(got["rank_slot"], rs), combo
        assert np.array_equal(got["rank_tokens"], rt), combo


@pytest.mark.parametrize("seed", range(5))
def test_rank_layout_cumsum_and_invariants(seed):
    idx, _, _ = random_case(300, 8, 24, 6, 10, [1, 2, 3, 6, 24][seed], seed)
    E, R = 24, [1, 2, 3, 6, 24][seed]
    got = oracle.rank_layout(idx, E, R)
    sent = sent_matrix(idx, E, R)
    want = np.where(sent, np.cumsum(sent, axis=0) - 1, -1)
    assert np.array_equal(got["rank_slot"], want)
    assert np.array_equal(got["rank_tokens"], sent.sum(axis=0))
    for r in range(R):
        col = got["rank_slot"][:, r]
        assert np.array_equal(col[col >= 0], np.arange(got["rank_tokens"][r]))


@pytest.mark.parametrize("name", ["decode_bf16", "skew_zipf", "balanced_stride"])
def test_rank_layout_one_expert_per_rank_is_the_expert_layout(name):
    """R = E: rank r is expert r. With distinct experts per token and no drops (C >= T) the
    rank slot of (t, e) is the slot of t's pair with expert e, and rank_tokens is the demand."""
    cfg = W.get_config(name)
    assert cfg.C >= cfg.T
    idx = W.make_inputs(cfg)["topk_idx"]
    got = oracle.rank_layout(idx, cfg.E, cfg.E)
    lay = oracle.layout(idx, cfg.E, cfg.C, cfg.R)
    assert np.array_equal(got["rank_tokens"], lay["raw"])
    t = np.repeat(np.arange(cfg.T), cfg.K)
    assert np.array_equal(got["rank_slot"][t, idx.reshape(-1)], lay["slot"].reshape(-1))
    assert int((got["rank_slot"] >= 0).sum()) == cfg.T * cfg.K


# ------------------------------------------------------------------------------------------
# dispatch: stage 1 + stage 2 = the one-stage dispatch
# ------------------------------------------------------------------------------------------

TWO_STAGE_CASES = [
    # T, H, E, K, C, R, seed  (random ids in [-2, E]: dupes, unrouted, invalid, drops)
    (37, 256, 6, 3, 5, 3, 1),
    (100, 128, 16, 4, 9, 4, 2),
    (64, 128, 8, 8, 40, 8, 3),
    (50, 256, 12, 2, 100, 1, 4),
]


@pytest.mark.parametrize("T,H,E,K,C,R,seed", TWO_STAGE_CASES)
def test_two_stage_dispatch_is_one_stage(T, H, E, K, C, R, seed):
    idx, x, _ = random_case(T, H, E, K, C, R, seed)
    lay = oracle.layout(idx, E, C, R)
    rl = oracle.rank_layout(idx, E, R)
    stage = np.full((R, T, H), SENT16, np.uint16)
    oracle.dispatch_ranks(x, rl["rank_slot"], stage)
    # every sent (t, r) row is x[t]; every other staging row is untouched
    sent = rl["rank_slot"] >= 0
    t_idx, r_idx = np.nonzero(sent)
    assert np.array_equal(stage[r_idx, rl["rank_slot"][t_idx, r_idx]], x[t_idx])
    untouched = np.ones((R, T), bool)
    untouched[r_idx, rl["rank_slot"][t_idx, r_idx]] = False
    assert (stage[untouched] == SENT16).all()
    got = np.full((E, C, H), SENT16, np.uint16)
    oracle.dispatch_expand(stage, idx, lay["slot"], rl["rank_slot"], E, C, got)
    want = np.full((E, C, H), SENT16, np.uint16)
    oracle.dispatch(x, idx, lay["slot"], E, C, want)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("T,H,E,K,C,R,seed", TWO_STAGE_CASES)
def test_two_stage_fp8_dispatch_is_one_stage(T, H, E, K, C, R, seed):
    idx, x, _ = random_case(T, H, E, K, C, R, seed)
    NB = H // 128
    lay = oracle.layout(idx, E, C, R)
    rl = oracle.rank_layout(idx, E, R)
    sq = np.full((R, T, H), 0xA5, np.uint8)
    ss = np.full((R, T, NB), -3.0, np.float32)
    oracle.dispatch_ranks_fp8(x, rl["rank_slot"], sq, ss)
    gq = np.full((E, C, H), 0xA5, np.uint8)
    gs = np.full((E, C, NB), -3.0, np.float32)
    oracle.dispatch_expand_fp8(sq, ss, idx, lay["slot"], rl["rank_slot"], E, C, gq, gs)
    wq = np.full((E, C, H), 0xA5, np.uint8)
    ws = np.full((E, C, NB), -3.0, np.float32)
    oracle.dispatch_fp8(x, idx, lay["slot"], E, C, wq, ws)
    assert np.array_equal(gq, wq)
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))


# ------------------------------------------------------------------------------------------
# combine: per-rank partials, then the reduction in rank order
# ------------------------------------------------------------------------------------------

def two_stage_combine(y, idx, slot, w, E, R):
    rl = oracle.rank_layout(idx, E, R)
    part = oracle.combine_ranks(y, idx, slot, rl["rank_slot"], w)
    return oracle.combine_reduce(part, rl["rank_slot"]), part, rl


def y_for(lay, E, C, H, seed):
    rng = np.random.default_rng(seed + 100)
    return W.f32_to_bf16_bits(rng.standard_normal((E, C, H), dtype=np.float32))


@pytest.mark.parametrize("T,H,E,K,C,R,seed", TWO_STAGE_CASES)
def test_two_stage_combine_single_rank_is_one_stage(T, H, E, K, C, R, seed):
    idx, _, w = random_case(T, H, E, K, C, R, seed)
    lay = oracle.layout(idx, E, C, 1)
    y = y_for(lay, E, C, H, seed)
    got, _, _ = two_stage_combine(y, idx, lay["slot"], w, E, 1)
    assert same_up_to_zero_sign(got, oracle.combine(y, idx, lay["slot"], w))


@pytest.mark.parametrize("T,H,E,K,C,R,seed", TWO_STAGE_CASES)
def test_two_stage_combine_identity_law(T, H, E, K, C, R, seed):
    """y = the dispatch output of x and unit weights: the partial of (t, r) is
    bf16(n_r * x[t]) (n_r = t's kept pairs in r; the fp32 product is exact) and the result is
    bf16 of the fp32 sum of those partials in ascending r."""
    idx, x, _ = random_case(T, H, E, K, C, R, seed)
    lay = oracle.layout(idx, E, C, R)
    y = np.zeros((E, C, H), np.uint16)
    oracle.dispatch(x, idx, lay["slot"], E, C, y)
    w = np.ones((T, K), np.float32)
    got, _, rl = two_stage_combine(y, idx, lay["slot"], w, E, R)
    EL = E // R
    kept = lay["slot"] >= 0
    xf = bf16_to_f32(x)
    acc = np.zeros((T, H), np.float32)
    for r in range(R):
        n_r = (kept & (idx // EL == r)).sum(axis=1).astype(np.float32)
        sent = rl["rank_slot"][:, r] >= 0
        part = bf16_to_f32(torch_bf16(n_r[:, None] * xf))
        acc = np.where(sent[:, None], acc + part, acc).astype(np.float32)
    assert same_up_to_zero_sign(got, torch_bf16(acc))


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_two_stage_combine_one_expert_per_rank(seed):
    """R = E: every partial is one weighted row, bf16(fp32(w * y)), and the result sums them in
    ascending expert order (not in j order) before rounding once."""
    T, H, E, K, C = 80, 64, 8, 5, 100        # C > T: no drops, every pair has its row
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32) * 3
    lay = oracle.layout(idx, E, C, E)
    assert lay["stats"]["dropped"] == 0
    y = y_for(lay, E, C, H, seed)
    got, part, rl = two_stage_combine(y, idx, lay["slot"], w, E, E)
    acc = np.zeros((T, H), np.float32)
    for e in range(E):                      # ascending rank = ascending expert
        t_e, j_e = np.nonzero(idx == e)
        s_e = lay["slot"][t_e, j_e]
        prod = w[t_e, j_e][:, None] * bf16_to_f32(y[e, s_e])     # one fp32 rounding
        p = torch_bf16(prod)
        assert same_up_to_zero_sign(part[e, rl["rank_slot"][t_e, e]], p)
        acc[t_e] = (acc[t_e] + bf16_to_f32(p)).astype(np.float32)
    assert same_up_to_zero_sign(got, torch_bf16(acc))


def test_rank_with_only_dropped_pairs_returns_zero_row():
    """Token 1 goes to rank 0 through expert 0, whose capacity (1) token 0 used up: its
    partial for rank 0 is exactly +0 and the result is its rank-1 pair alone."""
    E, R, C, H = 4, 2, 1, 16
    idx = np.array([[0, 2], [0, 3]], np.int32)
    w = np.array([[0.5, 0.25], [2.0, 0.75]], np.float32)
    lay = oracle.layout(idx, E, C, R)
    assert lay["slot"][1, 0] == -1
    y = y_for(lay, E, C, H, 9)
    got, part, rl = two_stage_combine(y, idx, lay["slot"], w, E, R)
    assert rl["rank_slot"][1, 0] == 1
    assert (part[0, 1] == 0).all()
    one = torch_bf16(np.float32(0.75) * bf16_to_f32(y[3, lay["slot"][1, 1]]))
    assert same_up_to_zero_sign(got[1], one)


def test_final_reduction_is_in_ascending_rank_order():
    """Partials 2^24, 1 and -2^24 on ranks 0, 1, 2: in fp32, (2^24 + 1) rounds back to 2^24, so
    the ascending-rank sum is 0, the descending one 1, and the j-order one (pairs listed as
    ranks 2, 0, 1) also 1. Only the ascending order gives +0."""
    E = R = 3
    C, H = 1, 8
    idx = np.array([[2, 0, 1]], np.int32)
    w = np.ones((1, 3), np.float32)
    y = np.zeros((E, C, H), np.uint16)
    y[0, 0] = 0x4B80          # 2^24
    y[1, 0] = 0x3F80          # 1
    y[2, 0] = 0xCB80          # -2^24
    lay = oracle.layout(idx, E, C, R)
    got, part, _ = two_stage_combine(y, idx, lay["slot"], w, E, R)
    assert (part[:, 0] == y[:, 0]).all()
    assert (got == 0).all()
    assert (oracle.combine(y, idx, lay["slot"], w) == 0x3F80).all()     # j order: 1


@pytest.mark.parametrize("T,H,E,K,C,R,seed", TWO_STAGE_CASES)
def test_two_stage_tokens_subset_matches_full(T, H, E, K, C, R, seed):
    """The token-subset form (used at sizes where the full oracle is slow) gives the full
    result's rows."""
    idx, _, w = random_case(T, H, E, K, C, R, seed)
    lay = oracle.layout(idx, E, C, R)
    y = y_for(lay, E, C, H, seed)
    full, _, rl = two_stage_combine(y, idx, lay["slot"], w, E, R)
    tokens = np.array([T - 1, 0, T // 2, 3, T // 3], np.int32)
    sub = oracle.combine_two_stage_tokens(tokens, y, idx, lay["slot"], rl["rank_slot"], w)
    assert np.array_equal(sub, full[tokens])

