"""The C ABI from plain C: tests/c_abi/ep_c_client.c allocates with hipMalloc, calls
ep_layout, ep_dispatch, ep_layout_dispatch, ep_dispatch_fp8 and ep_combine with raw device
pointers, and checks every result on the host against what the definitions fix (brute-force
slots, counts and offsets, row copies and untouched rows, fused = separate, FP8 scales and the
block-amax code, the combine identity law). No torch tensor crosses the boundary; the library
is called in-process through ctypes, so no program is started."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c_abi", "ep_c_client.so")


def test_c_client_checks_pass():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(CLIENT), "build() compiles tests/c_abi/ep_c_client.so"
    print("[c client] T=300 H=256 E=32 K=4 C=40 R=4", flush=True)
    lib = ctypes.CDLL(CLIENT)
    lib.ep_c_client_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    lib.ep_c_client_check.restype = ctypes.c_int
    msg = ctypes.create_string_buffer(256)
    rc = lib.ep_c_client_check(msg, len(msg))
    print(msg.value.decode(), flush=True)
    assert rc == 0, msg.value.decode()
