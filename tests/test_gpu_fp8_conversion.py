"""The FP8 cast's hardware E4M3 conversion against its software encoder, on the device, over
every fp32 bit pattern (through ep_check_e4m3_conversion).

The fast path of the quantiser encodes quotients x / scale with gfx950's packed conversion
instruction; every such quotient is at most 448 (1 + 2^-22) in magnitude. The path is right
only if the instruction equals round-to-nearest-even with saturation (the OFP8 specification's
satfinite conversion, which the software encoder implements and the oracle pins) on all of
those values. Here the two are compared on all 2^32 patterns: each sign half must agree on
every pattern up to |v| = 464 (the saturation boundary), so the first disagreement of each half
lies above it.
"""
import numpy as np
import pytest
import torch

from combine_ep_layout_06_amd import binding as B

pytestmark = pytest.mark.gpu

F464 = 0x43E80000                          # 464.0
FAST_MAX = np.float32(np.float64(448.0) * (1 + 2.0 ** -22))


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def test_fast_path_range_is_inside_the_checked_range():
    assert FAST_MAX.view(np.uint32) < F464


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_hardware_conversion_equals_software_encoder(sign):
    print(f"[fp8 conversion] sign bit {sign >> 31}: 2^31 patterns", flush=True)
    n, first = B.ep_check_e4m3_conversion(sign, 1 << 31)
    # equal on every pattern with |v| <= 464 (zero, subnormals, normals, the rounding
    # boundary of the largest code), both signs
    assert first is None or (first & 0x7FFFFFFF) > F464, hex(first)
    n_in, _ = B.ep_check_e4m3_conversion(sign, F464 + 1)
    assert n_in == 0
    print(f"[fp8 conversion] sign bit {sign >> 31}: {n} patterns differ, all beyond |v| = 464 "
          f"(first 0x{first:08x})" if first is not None else "none differ", flush=True)


def test_check_reports_a_known_disagreement():
    """The check itself sees a difference where one exists: above 464 the hardware conversion
    gives NaN where the saturating encoder gives 0x7E."""
    n, first = B.ep_check_e4m3_conversion(0x43F00000, 16)       # 480.0 and the next 15
    assert n == 16 and first == 0x43F00000
