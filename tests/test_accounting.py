"""Pins for the byte accounting used by the benchmark (CPU only).

The logical-payload definition of awsome-distributed-ai PR #1238 is reproduced from the
values the page prints (tests/golden/logical_payload_pr1238.txt): the per-rank Decode-like
payloads of review item 1 and the whole-job Prefill-like token rates of review item 3.
"""
import os

import pytest

from combine_ep_layout_06_amd import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "logical_payload_pr1238.txt")


def golden_rows():
    with open(GOLDEN) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


@pytest.mark.parametrize("row", golden_rows())
def test_logical_payload_matches_printed_values(row):
    kind, dtype, T, K, H, ranks, gbps, printed, unit = row
    T, K, H, ranks = int(T), int(K), int(H), int(ranks)
    payload = A.logical_payload_bytes(T, K, H, dtype == "fp8")
    if kind == "payload":
        assert round(payload / 1e6, 2) == float(printed)
    else:
        # the same numerator over the same elapsed time gives the page's tokens/s, to the
        # precision of the printed GB/s (two decimals)
        elapsed = payload / (float(gbps) * 1e9)
        assert ranks * T / elapsed == pytest.approx(int(printed), rel=0.005 / float(gbps))


def test_algorithmic_bytes_prefill_bf16():
    # T=4096, H=2048, K=8, no drops: 302.9 MB (reads x once, writes/reads each kept row once)
    T, K, H = 4096, 8, 2048
    b = A.step_bytes(T, K, H, T * K, fp8=False)
    assert b == 8 * T * K + (2 * T * H + 2 * H * T * K + 8 * T * K) + (2 * H * T * K + 12 * T * K + 2 * T * H)
    assert round(b / 1e6, 1) == 302.9
    assert round(A.step_bytes(T, K, H, T * K, fp8=True) / 1e6, 1) == 237.9


def test_two_stage_bytes_reduce_to_one_stage_when_nothing_is_shared():
    """With one expert per rank and distinct experts per token every (token, rank) carries
    exactly one pair (N_tr = N_kept): the expansion and the reduction then only move rows the
    one-stage kernels move directly, so the two stages together cost exactly one extra write and
    read of every row on each side."""
    T, K, H = 4096, 8, 2048
    R = E = 128
    n = T * K
    one_dispatch = A.dispatch_bytes(T, K, H, n, False)
    two_dispatch = (A.dispatch_ranks_bytes(T, R, H, n, False)
                    + A.dispatch_expand_bytes(T, K, R, H, n, n, False))
    assert two_dispatch - one_dispatch == 2 * (2 * H * n) + 2 * 4 * T * R
    one_combine = A.combine_bytes(T, K, H, n)
    two_combine = A.combine_ranks_bytes(T, K, R, H, n, n) + A.combine_reduce_bytes(T, R, H, n)
    assert two_combine - one_combine == 2 * (2 * H * n) + 2 * 4 * T * R

