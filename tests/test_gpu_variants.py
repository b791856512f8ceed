"""GPU parity across the kernels' compile-time variants.

From the shape, each entry point chooses how many 16-byte chunks a lane moves per item (U), how
many of a token's pairs (or of its ranks) it copies or folds together (KG, and a looping form
for K > 8), whether a row fits the combine's and the reduce's zero row (H <= 32768), the width
of the rank layout's id loads (K = 4, 8, 12, 16) and of its per-lane rank counters (R <= 4,
R <= 16, else ballots), how many tokens a fused tile takes, and whether the final reduce reads
the partial rows through the caches. The workloads and the other parity tests run only some of
these choices. The (T, H, K, R) below were picked, from those rules, so that every kernel the
library builds runs in at least one case (a kernel trace of `pytest -m gpu` lists none that is
never launched). Every output of every call is compared with the oracle in full: one-stage
dispatch and combine, the layout fused with the dispatch with and without a workspace, the
packed layout, and the two-stage path.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W
import gpu_cases as G
import test_gpu_packed as P
import test_gpu_two_stage as TS

pytestmark = pytest.mark.gpu

# one-stage and packed calls: (T, H, [K, ...]). K = 1, 2, 3, 5, 12 meet the five pair-group forms;
# the shapes give one, two and four chunks per lane to the dispatch, the FP8 dispatch, the
# combine (with and without the zero row) and the fused kernels, whose tiles depend on T and K.
ONE = [
    (1, 128, [1, 2, 3, 5, 12]),
    (1, 4096, [3, 5]),
    (1, 8192, [2]),
    (1, 16384, [12]),
    (1, 32896, [1, 2, 3, 5, 12]),
    (130, 32896, [1, 2, 3, 5, 12]),
    (260, 32896, [1, 2, 3, 5, 12]),
    (2048, 1152, [1, 2, 3, 5, 12]),
    (2048, 4096, [1, 2, 3]),
    (4100, 128, [5, 12]),
]

# two-stage calls: (T, H, [(K, R), ...]). R picks the rank counters (1-4, 5-16, more) and the
# staging copy's groups; K the id loads, the expansion's groups and the partial combine's form
# (K > 8: one row at a time); min(K, R) the reduce's list; R * T * H the reduce's load policy.
TWO = [
    (1, 128, [(1, 1), (4, 2), (4, 17), (5, 5), (8, 2), (8, 9), (8, 17), (12, 3), (16, 1),
              (16, 9)]),
    (1, 32896, [(2, 17), (8, 1), (8, 3), (8, 5), (12, 17)]),
    (130, 4096, [(1, 64), (2, 64), (3, 64), (5, 64), (12, 64)]),
    (130, 32896, [(1, 1), (2, 2), (3, 3), (5, 5), (12, 9)]),
    (260, 32896, [(1, 1), (2, 2), (8, 3), (8, 5), (12, 17)]),
    (2048, 1152, [(1, 1), (1, 16), (2, 2), (2, 16), (3, 3), (3, 16), (5, 16), (8, 5), (12, 9),
                  (12, 16)]),
    (2048, 4096, [(2, 5), (3, 9), (8, 1), (8, 2), (8, 9), (8, 17)]),
    (4100, 128, [(1, 3), (2, 2), (4, 9), (8, 1), (8, 2), (8, 3), (8, 9), (8, 64), (12, 5),
                 (12, 64), (16, 17)]),
    (4100, 2048, [(1, 4)]),
]


def experts(R):
    """E: a multiple of R near 64 (R ranks of E / R experts)."""
    return R * -(-64 // R)


def capacity(T, K, E):
    """ids are drawn from [-2, E]: about T*K/(E + 3) pairs per expert; 85% of that drops the
    last pairs of most experts."""
    return max(1, int(0.85 * T * K / (E + 3)))


ONE_CASES = [pytest.param(T, H, K, id=f"T{T}-H{H}-K{K}") for T, H, ks in ONE for K in ks]
TWO_CASES = [pytest.param(T, H, K, R, id=f"T{T}-H{H}-K{K}-R{R}")
             for T, H, krs in TWO for K, R in krs]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


@pytest.mark.parametrize("T,H,K", ONE_CASES)
def test_one_stage_variants(T, H, K):
    _need_gpu()
    E, R = 64, 4
    C = capacity(T, K, E)
    print(f"[variants] one-stage T={T} H={H} E={E} K={K} C={C} R={R}", flush=True)
    case = G.Case.random(T, H, E, K, C, R, seed=T * 31 + K)
    case.check_dispatch_bf16(full=True)
    case.check_fused(fp8=False, full=True)
    case.check_fused(fp8=False, full=True, ws=True)
    case.check_dispatch_fp8(full=True)
    case.check_fused(fp8=True, full=True)
    case.check_fused(fp8=True, full=True, ws=True)
    got, want = case.check_combine()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("T,H,K", ONE_CASES)
def test_packed_variants(T, H, K):
    _need_gpu()
    E, R = 64, 4
    C = capacity(T, K, E)
    print(f"[variants] packed T={T} H={H} E={E} K={K} C={C} R={R}", flush=True)
    rng = np.random.default_rng(T * 37 + K)
    idx = rng.integers(-2, E + 1, size=(T, K)).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.random((T, K)).astype(np.float32)
    P.run_case(idx, x, w, E, C, R, 16, seed=T + K)


@pytest.mark.parametrize("T,H,K,R", TWO_CASES)
def test_two_stage_variants(T, H, K, R):
    _need_gpu()
    E = experts(R)
    C = capacity(T, K, E)
    print(f"[variants] two-stage T={T} H={H} E={E} K={K} C={C} R={R}", flush=True)
    ts = TS.TwoStage.random(T, H, E, K, C, R, seed=T * 41 + K + R)
    ts.dispatch_bf16_full()
    ts.dispatch_fp8_full()
    ts.combine_full()


# The rank layout counts a lane's earlier tokens per rank in 8-bit fields up to this many
# tokens (at most 252 per lane in a 1024-lane workgroup), and with ballots past it.
PACKED_RANK_MAX_T = 63 * 4 * 1024


@pytest.mark.parametrize("T", [PACKED_RANK_MAX_T, PACKED_RANK_MAX_T + 1])
@pytest.mark.parametrize("K,R", [(8, 3), (6, 4)])
def test_rank_counters_at_their_limit(T, K, R):
    """The largest batch of the packed counters (with K = 8 of 48 experts in 3 ranks ~95% of
    the tokens reach each rank, so a lane's counts come close to the 252 its 8-bit fields
    hold) and the first batch past it: rank layout, and the fused rank layout + staging copy
    (bf16; FP8 too for K = 8), against the oracle in full."""
    _need_gpu()
    H, E = 128, 16 * R
    print(f"[variants] rank counters T={T} H={H} E={E} K={K} R={R}", flush=True)
    rng = np.random.default_rng(T + K)
    idx = rng.integers(-2, E + 1, size=(T, K)).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx_d, x_d = G.to_dev(idx), G.u16_dev(x)
    want = oracle.rank_layout(idx, E, R)
    g = B.ep_rank_layout(idx_d, E, R)
    torch.cuda.synchronize()
    assert np.array_equal(G.to_np(g["rank_slot"]), want["rank_slot"]), "rank_slot"
    assert np.array_equal(G.to_np(g["rank_tokens"]), want["rank_tokens"]), "rank_tokens"
    if K == 8:     # the counters near their limit: most tokens reach every rank
        assert int(want["rank_tokens"].min()) > 0.9 * T
    stage = torch.full((R, T, H), G.SENTINEL16, dtype=torch.int16, device=G.dev())
    f = B.ep_rank_layout_dispatch(x_d, idx_d, E, R, stage=stage)
    torch.cuda.synchronize()
    assert np.array_equal(G.to_np(f["rank_slot"]), want["rank_slot"]), "fused rank_slot"
    assert np.array_equal(G.to_np(f["rank_tokens"]), want["rank_tokens"]), "fused rank_tokens"
    want_stage = np.full((R, T, H), G.SENTINEL16, np.uint16)
    oracle.dispatch_ranks(x, want["rank_slot"], want_stage)
    assert np.array_equal(G.to_np(stage).view(np.uint16), want_stage), "fused stage"
    del stage, want_stage
    if K != 8:
        return
    NB = H // 128
    sq = torch.full((R, T, H), G.SENTINEL8, dtype=torch.uint8, device=G.dev())
    ss = torch.full((R, T, NB), G.SENTINEL_F32, dtype=torch.float32, device=G.dev())
    f = B.ep_rank_layout_dispatch_fp8(x_d, idx_d, E, R, stage_q=sq, stage_scale=ss)
    torch.cuda.synchronize()
    assert np.array_equal(G.to_np(f["rank_slot"]), want["rank_slot"]), "fused FP8 rank_slot"
    wq = np.full((R, T, H), G.SENTINEL8, np.uint8)
    ws = np.full((R, T, NB), G.SENTINEL_F32, np.float32)
    oracle.dispatch_ranks_fp8(x, want["rank_slot"], wq, ws)
    assert np.array_equal(G.to_np(sq), wq), "fused FP8 stage codes"
    assert np.array_equal(G.to_np(ss).view(np.uint32), ws.view(np.uint32)), "fused FP8 scales"
