"""The decode-size step (fused layout + dispatch, then combine) captured in a HIP graph and
replayed: every replay must leave exactly the outputs of the eager calls.

The library's kernels issue no memset and no allocation, so the captured graph holds only
their launches; the replays are separated by unrelated eager work and synchronisations, and
each replay starts from outputs scribbled over by that eager work.
"""
import numpy as np
import pytest
import torch

from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W
import gpu_cases as G

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _step(cfg, x, idx, w, y, lay, recv, recv_s, out):
    if cfg.fp8:
        B.ep_layout_dispatch_fp8(x, idx, recv, recv_s, cfg.E, cfg.C, cfg.R, **lay)
    else:
        B.ep_layout_dispatch(x, idx, recv, cfg.E, cfg.C, cfg.R, **lay)
    B.ep_combine(y, idx, lay["slot"], w, cfg.C, out=out)


@pytest.mark.parametrize("name", ["decode_bf16", "decode_fp8"])
def test_graph_replay_matches_eager(name):
    _need_gpu()
    cfg = W.get_config(name)
    print(f"[graph] {name}", flush=True)
    inp = W.make_inputs(cfg)
    dev = G.dev()
    x = G.u16_dev(inp["x"])
    idx = G.to_dev(inp["topk_idx"])
    w = G.to_dev(inp["topk_w"])
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    y = torch.randn((cfg.E, cfg.C, cfg.H), generator=gen, device=dev).to(torch.bfloat16)
    y = y.view(torch.int16)
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    lay = dict(slot=mk((cfg.T, cfg.K)), expert_count=mk(cfg.E), expert_offset=mk(cfg.E),
               rank_count=mk(cfg.R), rank_offset=mk(cfg.R), stats=mk(4))
    if cfg.fp8:
        recv = torch.zeros((cfg.E, cfg.C, cfg.H), dtype=torch.uint8, device=dev)
        recv_s = torch.zeros((cfg.E, cfg.C, cfg.H // 128), dtype=torch.float32, device=dev)
    else:
        recv = torch.zeros((cfg.E, cfg.C, cfg.H), dtype=torch.int16, device=dev)
        recv_s = None
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)
    args = (cfg, x, idx, w, y, lay, recv, recv_s, out)

    _step(*args)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in lay.items()}
    want["recv"], want["out"] = recv.clone(), out.clone()
    if recv_s is not None:
        want["recv_s"] = recv_s.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(*args)
    torch.cuda.synchronize()

    for rep in range(4):
        # unrelated eager work between replays, and every output overwritten
        for v in lay.values():
            v.fill_(-5)
        out.fill_(0x1234)
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        g.replay()
        torch.cuda.synchronize()
        for k, v in lay.items():
            assert torch.equal(v, want[k]), f"replay {rep}: {k}"
        assert torch.equal(out, want["out"]), f"replay {rep}: out"
        assert torch.equal(recv, want["recv"]), f"replay {rep}: recv"
        if recv_s is not None:
            assert torch.equal(recv_s, want["recv_s"]), f"replay {rep}: recv_scale"
    # the eager result itself against the oracle's layout
    G.check_layout(inp["topk_idx"], cfg.E, cfg.C, cfg.R, lay)
    del g
