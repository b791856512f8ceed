"""ep_layout_dispatch_noalloc (the chunked layout + dispatch with the library's static scratch
as its workspace) against ep_layout_dispatch_ws (the same call with a caller workspace), through
the C ABI: every output bit for bit, on two calls in a row, the second with a smaller batch, so
the second call runs over the first call's scratch contents. The layout outputs are also checked
against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W

import gpu_cases as G

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("slot", "expert_count", "expert_offset", "rank_count", "rank_offset", "stats")


def test_noalloc_equals_workspace_form_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()
    E, K, C, R, H = 128, 8, 150, 16, 256           # both batches drop pairs at C = 150
    for T, seed in ((9000, 61), (3001, 62)):          # the second call smaller
        print(f"[no-alloc] T={T} H={H} E={E} K={K} C={C} R={R}", flush=True)
        rng = np.random.default_rng(seed)
        idx = rng.integers(-2, E + 1, size=(T, K)).astype(np.int32)
        x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        x_d, idx_d = G.u16_dev(x), G.to_dev(idx)
        recv_n = torch.full((E, C, H), G.SENTINEL16, dtype=torch.int16, device=G.dev())
        recv_w = torch.full((E, C, H), G.SENTINEL16, dtype=torch.int16, device=G.dev())
        got = B.ep_layout_dispatch_noalloc(x_d, idx_d, recv_n, E, C, R)
        want = B.ep_layout_dispatch_ws(x_d, idx_d, recv_w, E, C, R)
        torch.cuda.synchronize()
        for k in LAYOUT_KEYS:
            assert torch.equal(got[k], want[k]), k
        assert torch.equal(recv_n, recv_w), "recv"
        lay = G.check_layout(idx, E, C, R, got)
        assert lay["stats"]["dropped"] > 0 and lay["stats"]["invalid"] > 0
