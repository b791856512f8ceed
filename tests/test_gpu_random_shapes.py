"""GPU parity on seeded random shapes.

Each case draws a shape inside the library's limits (T up to ~5000, H any multiple of 8 or of
128, E up to 1024 split over R ranks from 1 to 64, K from 1 to 20, a capacity between 30% and
130% of the mean demand, a packed alignment of 1, 3, 8, 64 or 100) and random ids in [-2, E]
(duplicates, unrouted and invalid ids), then runs every call family on it and compares every output with the oracle in full: the one-stage
dispatch (bf16 and, where H allows, FP8), the fused layout + dispatch with and without a
workspace, combine, the packed layout at a random alignment, and the two-stage path. The fixed
cases of the other parity tests pick shapes on purpose; these pick the odd ones nobody chose
(K = 7 or 13, H = 2696, 7 ranks of 9 experts, ...).
"""
import numpy as np
import pytest
import torch

from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W
import gpu_cases as G
import test_gpu_packed as P
import test_gpu_two_stage as TS

pytestmark = pytest.mark.gpu

N_CASES = 24
BYTES_MAX = 128 << 20          # bound on each [E][C][H] and [R][T][H] buffer


def draw(i):
    """The i-th shape: (T, H, E, K, C, R, alignment)."""
    rng = np.random.default_rng(20261203 + i)
    T = int([rng.integers(1, 64), rng.integers(64, 1200), rng.integers(1200, 5000)][i % 3])
    H = int(128 * rng.integers(1, 24)) if i % 2 == 0 else int(8 * rng.integers(1, 400))
    R = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32, 48, 64]))
    E = R * int(rng.integers(1, min(64, 1024 // R) + 1))
    K = int(rng.integers(1, 21))
    C = max(1, int(rng.uniform(0.3, 1.3) * T * K / E) + 1)
    while C > 1 and E * C * H * 2 > BYTES_MAX:
        C //= 2
    while T > 1 and (R * T * H * 2 > BYTES_MAX or E * C * H * 2 > BYTES_MAX):
        T //= 2
    # packed alignment, powers of two or not, with its padding rows within the byte bound
    aligns = [a for a in (1, 3, 8, 64, 100) if E * (a - 1) * H * 2 <= BYTES_MAX // 2]
    align = int(rng.choice(aligns))
    return T, H, E, K, C, R, align


CASES = [pytest.param(i, id="case{}-T{}-H{}-E{}-K{}-C{}-R{}-A{}".format(i, *draw(i)))
         for i in range(N_CASES)]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


@pytest.mark.parametrize("i", CASES)
def test_random_shape(i):
    _need_gpu()
    T, H, E, K, C, R, align = draw(i)
    print(f"[random] case {i}: T={T} H={H} E={E} K={K} C={C} R={R} align={align}", flush=True)
    case = G.Case.random(T, H, E, K, C, R, seed=1000 + i)
    case.check_dispatch_bf16(full=True)
    case.check_fused(fp8=False, full=True)
    case.check_fused(fp8=False, full=True, ws=True)
    if H % 128 == 0:
        case.check_dispatch_fp8(full=True)
        case.check_fused(fp8=True, full=True)
        case.check_fused(fp8=True, full=True, ws=True)
    got, want = case.check_combine()
    assert np.array_equal(got, want)
    P.run_case(case.idx, case.x, case.w, E, C, R, align, seed=2000 + i)
    ts = TS.TwoStage(T, H, E, K, C, R, case.idx, case.x, case.w, 3000 + i)
    ts.dispatch_bf16_full()
    if H % 128 == 0:
        ts.dispatch_fp8_full()
    ts.combine_full()


def test_draws_cover_the_odd_cases():
    """The draw covers what the fixed lists do not: K not a power of two, H not a multiple of
    128, ranks and packed alignments that are not powers of two."""
    shapes = [draw(i) for i in range(N_CASES)]
    assert any(K not in (1, 2, 4, 8, 16) for _, _, _, K, _, _, _ in shapes)
    assert any(H % 128 for _, H, _, _, _, _, _ in shapes)
    assert any(R & (R - 1) for _, _, _, _, _, R, _ in shapes)
    assert any(A & (A - 1) for _, _, _, _, _, _, A in shapes)
