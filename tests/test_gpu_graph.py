"""Passes captured in a HIP graph and replayed: the decode-size step (fused layout + dispatch,
then combine), the two-stage pass and the packed pass. Every replay must leave exactly the
outputs of the eager calls.

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


def _capture_and_replay(step, outputs, partial, tag):
    """Run `step` eagerly, capture it in a graph, then replay it four times, each replay after
    eager work that overwrites every output; each replay must reproduce the eager outputs.

    ``outputs`` are written whole by `step` and get scribbled over before each replay;
    ``partial`` buffers (receive rows of unused slots stay as they were) are zeroed instead, as
    they were before the eager call."""
    step()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in list(outputs.items()) + list(partial.items())}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for v in outputs.values():
            v.view(torch.uint8).fill_(0xA5)
        for v in partial.values():
            v.zero_()
        junk = torch.randn(1 << 20, device=G.dev()).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        g.replay()
        torch.cuda.synchronize()
        for k, v in list(outputs.items()) + list(partial.items()):
            assert torch.equal(v, want[k]), f"{tag} replay {rep}: {k}"
    del g
    return want


def _small_inputs(T=512, H=512, E=64, K=8, C=256, R=8):
    cfg = W.EpConfig("graph_small", T=T, H=H, E=E, K=K, C=C, R=R)
    inp = W.make_inputs(cfg)
    dev = G.dev()
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    return cfg, inp, G.u16_dev(inp["x"]), G.to_dev(inp["topk_idx"]), G.to_dev(inp["topk_w"]), gen


def test_graph_replay_two_stage_pass():
    """The two-stage pass (layout, fused rank layout + staging copy, expansion, partial
    combine, reduce) replayed from a graph, with the FP8 staging copy and expansion too."""
    _need_gpu()
    print("[graph] two-stage pass", flush=True)
    cfg, inp, x, idx, w, gen = _small_inputs()
    dev = G.dev()
    T, H, E, K, C, R = cfg.T, cfg.H, cfg.E, cfg.K, cfg.C, cfg.R
    mk = lambda *n: torch.empty(n, dtype=torch.int32, device=dev)
    lay = dict(slot=mk(T, K), expert_count=mk(E), expert_offset=mk(E), rank_count=mk(R),
               rank_offset=mk(R), stats=mk(4))
    rl = dict(rank_slot=mk(T, R), rank_tokens=mk(R))
    stage = torch.empty((R, T, H), dtype=torch.int16, device=dev)
    recv = torch.zeros((E, C, H), dtype=torch.int16, device=dev)
    y = torch.randn((E, C, H), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    part = torch.empty((R, T, H), dtype=torch.int16, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    stage_q = torch.empty((R, T, H), dtype=torch.uint8, device=dev)
    stage_s = torch.empty((R, T, H // 128), dtype=torch.float32, device=dev)
    recv_q = torch.zeros((E, C, H), dtype=torch.uint8, device=dev)
    recv_s = torch.zeros((E, C, H // 128), dtype=torch.float32, device=dev)

    def step():
        B.ep_layout(idx, E, C, R, **lay)
        B.ep_rank_layout_dispatch(x, idx, E, R, stage=stage, **rl)
        B.ep_dispatch_expand(stage, idx, lay["slot"], rl["rank_slot"], recv, C)
        B.ep_rank_layout_dispatch_fp8(x, idx, E, R, stage_q=stage_q, stage_scale=stage_s, **rl)
        B.ep_dispatch_expand_fp8(stage_q, stage_s, idx, lay["slot"], rl["rank_slot"], recv_q,
                                 recv_s, C)
        B.ep_combine_ranks(y, idx, lay["slot"], rl["rank_slot"], w, C, part=part)
        B.ep_combine_reduce(part, rl["rank_slot"], K, out=out)

    # stage and part are intermediates (rows of unsent (token, rank) pairs are never written);
    # what the pass hands on is compared
    _capture_and_replay(step, dict(lay, **rl, out=out),
                        dict(recv=recv, recv_q=recv_q, recv_s=recv_s), "two-stage")
    G.check_layout(inp["topk_idx"], E, C, R, lay)


def test_graph_replay_packed_pass():
    """The packed pass (fused packed layout + dispatch, then packed combine) replayed from a
    graph, bf16 and FP8."""
    _need_gpu()
    print("[graph] packed pass", flush=True)
    cfg, inp, x, idx, w, gen = _small_inputs()
    dev = G.dev()
    T, H, E, K, C, R = cfg.T, cfg.H, cfg.E, cfg.K, cfg.C, cfg.R
    A = 16
    rows = B.packed_rows_bound(T, K, E, C, A)
    mk = lambda *n: torch.empty(n, dtype=torch.int32, device=dev)
    play = dict(slot=mk(T, K), expert_count=mk(E), packed_offset=mk(E + 1), rank_count=mk(R),
                rank_offset=mk(R), stats=mk(4))
    recv = torch.zeros((rows, H), dtype=torch.int16, device=dev)
    q = torch.zeros((rows, H), dtype=torch.uint8, device=dev)
    sc = torch.zeros((rows, H // 128), dtype=torch.float32, device=dev)
    y = torch.randn((rows, H), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)

    def step():
        B.ep_layout_dispatch_packed(x, idx, recv, E, C, R, A, **play)
        B.ep_layout_dispatch_packed_fp8(x, idx, q, sc, E, C, R, A, **play)
        B.ep_combine_packed(y, idx, play["slot"], play["packed_offset"], w, E, C, out=out)

    _capture_and_replay(step, dict(play, out=out), dict(recv=recv, q=q, sc=sc), "packed")


@pytest.mark.parametrize("name", ["decode_bf16", "decode_fp8"])
def test_recorded_calls_replay_matches_eager(name):
    """binding.record(): the decode step's calls recorded once on batch 0's buffers, then
    replayed after each new batch is copied into those buffers (on the current stream, and on
    a side stream), equal to the checked wrappers on fresh buffers, and the layout to the
    oracle's."""
    _need_gpu()
    cfg = W.get_config(name)
    print(f"[replay] {name}", flush=True)
    dev = G.dev()
    batches = [W.make_inputs(cfg, seed=cfg.seed + k) for k in range(3)]
    x = G.u16_dev(batches[0]["x"])
    idx = G.to_dev(batches[0]["topk_idx"])
    w = G.to_dev(batches[0]["topk_w"])
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    y = torch.randn((cfg.E, cfg.C, cfg.H), generator=gen, device=dev).to(torch.bfloat16)
    y = y.view(torch.int16)

    def recv_bufs():
        if cfg.fp8:
            return (torch.zeros((cfg.E, cfg.C, cfg.H), dtype=torch.uint8, device=dev),
                    torch.zeros((cfg.E, cfg.C, cfg.H // 128), dtype=torch.float32, device=dev))
        return (torch.zeros((cfg.E, cfg.C, cfg.H), dtype=torch.int16, device=dev),)

    def step(recv):
        if cfg.fp8:
            lay = B.ep_layout_dispatch_fp8(x, idx, recv[0], recv[1], cfg.E, cfg.C, cfg.R)
        else:
            lay = B.ep_layout_dispatch(x, idx, recv[0], cfg.E, cfg.C, cfg.R)
        return lay, B.ep_combine(y, idx, lay["slot"], w, cfg.C)

    recv = recv_bufs()
    with B.record() as cl:
        lay, out = step(recv)
    assert [c[1] for c in cl.calls] == [
        "ep_layout_dispatch_fp8" if cfg.fp8 else "ep_layout_dispatch", "ep_combine"]
    side = torch.cuda.Stream()
    for k, b in enumerate(batches + batches[:1]):
        x.copy_(G.u16_dev(b["x"]))
        idx.copy_(G.to_dev(b["topk_idx"]))
        w.copy_(G.to_dev(b["topk_w"]))
        for t in recv:
            t.zero_()
        out.fill_(0x1234)
        if k % 2:
            side.wait_stream(torch.cuda.current_stream())
            cl.replay(stream=side)
            torch.cuda.current_stream().wait_stream(side)
        else:
            cl.replay()
        torch.cuda.synchronize()
        fresh = recv_bufs()
        lay2, out2 = step(fresh)
        torch.cuda.synchronize()
        for key in lay:
            assert torch.equal(lay[key], lay2[key]), f"batch {k}: {key}"
        assert torch.equal(out, out2), f"batch {k}: out"
        for a, b2 in zip(recv, fresh):
            assert torch.equal(a, b2), f"batch {k}: recv"
        G.check_layout(b["topk_idx"], cfg.E, cfg.C, cfg.R, lay)
