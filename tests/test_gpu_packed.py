"""GPU parity of the packed, aligned receive layout (ep_layout_packed, ep_dispatch_packed[_fp8],
ep_combine_packed) against the oracle, bit for bit.

Every case compares whole packed buffers (the full workloads too), with a sentinel in every row
nobody may write and NaN in every packed y row nobody may read, and every output element.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W
import gpu_cases as G

pytestmark = pytest.mark.gpu

S16, S8, SF = G.SENTINEL16, G.SENTINEL8, G.SENTINEL_F32


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def run_case(idx, x, w, E, C, R, align, rows=None, fp8=True, seed=0):
    """Every output of the packed layout, dispatch (bf16 and FP8, separate and fused) and
    combine against the oracle, whole buffers: the rows past the buffer a call is given keep
    their sentinel, and every y row that no kept pair addresses is NaN."""
    T, K = idx.shape
    H = x.shape[1]
    idx_d, x_d, w_d = G.to_dev(idx.astype(np.int32)), G.u16_dev(x), G.to_dev(w.astype(np.float32))
    g = B.ep_layout_packed(idx_d, E, C, R, align)
    torch.cuda.synchronize()
    lay = oracle.layout(idx, E, C, R)
    off = oracle.packed_offsets(lay["count"], align)
    assert np.array_equal(G.to_np(g["slot"]), lay["slot"]), "slot"
    assert np.array_equal(G.to_np(g["expert_count"]), lay["count"]), "count"
    assert np.array_equal(G.to_np(g["stats"]), lay["stats_array"]), "stats"
    assert np.array_equal(G.to_np(g["packed_offset"]), off), "packed_offset"
    EL = E // R
    assert np.array_equal(G.to_np(g["rank_offset"]), off[:-1:EL][:R]), "rank_offset"
    assert np.array_equal(G.to_np(g["rank_count"]), off[EL::EL] - off[:-1:EL][:R]), "rank_count"
    rows = int(off[-1]) if rows is None else rows
    slot = lay["slot"]
    NB = H // 128

    # bf16 dispatch
    recv = torch.full((rows + 4, H), S16, dtype=torch.int16, device=G.dev())
    B.ep_dispatch_packed(x_d, idx_d, g["slot"], g["packed_offset"], recv[:rows], E, C)
    torch.cuda.synchronize()
    want = np.full((rows + 4, H), S16, np.uint16)
    oracle.dispatch_packed(x, idx, slot, off, E, C, want[:rows])
    assert np.array_equal(G.to_np(recv).view(np.uint16), want), "packed recv"
    del recv
    # FP8 dispatch
    if fp8 and H % 128 == 0:
        q = torch.full((rows, H), S8, dtype=torch.uint8, device=G.dev())
        sc = torch.full((rows, NB), SF, dtype=torch.float32, device=G.dev())
        B.ep_dispatch_packed_fp8(x_d, idx_d, g["slot"], g["packed_offset"], q, sc, E, C)
        torch.cuda.synchronize()
        wq = np.full((rows, H), S8, np.uint8)
        ws = np.full((rows, NB), SF, np.float32)
        oracle.dispatch_packed_fp8(x, idx, slot, off, E, C, wq, ws)
        assert np.array_equal(G.to_np(q), wq), "packed codes"
        assert np.array_equal(G.to_np(sc).view(np.uint32), ws.view(np.uint32)), "packed scales"
        del q, sc
    # the packed layout and dispatch in one launch: the same outputs
    lay_want = dict(slot=lay["slot"], expert_count=lay["count"], stats=lay["stats_array"],
                    packed_offset=off, rank_offset=off[:-1:EL][:R],
                    rank_count=off[EL::EL] - off[:-1:EL][:R])
    recv = torch.full((rows + 4, H), S16, dtype=torch.int16, device=G.dev())
    f = B.ep_layout_dispatch_packed(x_d, idx_d, recv[:rows], E, C, R, align)
    torch.cuda.synchronize()
    for k, v in lay_want.items():
        assert np.array_equal(G.to_np(f[k]), v), f"fused {k}"
    assert np.array_equal(G.to_np(recv).view(np.uint16), want), "fused packed recv"
    del recv, want
    if fp8 and H % 128 == 0:
        q = torch.full((rows, H), S8, dtype=torch.uint8, device=G.dev())
        sc = torch.full((rows, NB), SF, dtype=torch.float32, device=G.dev())
        f = B.ep_layout_dispatch_packed_fp8(x_d, idx_d, q, sc, E, C, R, align)
        torch.cuda.synchronize()
        for k, v in lay_want.items():
            assert np.array_equal(G.to_np(f[k]), v), f"fused fp8 {k}"
        assert np.array_equal(G.to_np(q), wq), "fused packed codes"
        assert np.array_equal(G.to_np(sc).view(np.uint32), ws.view(np.uint32)), "fused scales"
        del q, sc, wq, ws
    # combine from a packed y: kept rows from the expert-output stream, every other row NaN
    e_f, s_f = idx.reshape(-1), slot.reshape(-1)
    keep = (e_f >= 0) & (e_f < E) & (s_f >= 0) & (s_f < C)
    r_f = np.where(keep, off[np.clip(e_f, 0, E - 1)] + s_f, -1)
    live = keep & (r_f < rows)
    y_host = np.full((rows, H), W.BF16_NAN, np.uint16)
    y_host[r_f[live]] = W.y_rows(int(live.sum()), H, seed)
    y = G.u16_dev(y_host)
    out = B.ep_combine_packed(y, idx_d, g["slot"], g["packed_offset"], w_d, E, C)
    torch.cuda.synchronize()
    got = G.to_np(out).view(np.uint16)
    want_out = oracle.combine_packed(y_host, idx, slot, off, w, E, C)
    assert np.array_equal(got, want_out), "packed combine"
    assert not np.isnan(W.bf16_bits_to_f32(got)).any(), "a padding or NaN row of y was read"


SMALL = [
    # T, H, E, K, C, R
    (37, 256, 6, 3, 5, 3),
    (100, 520, 16, 4, 9, 4),
    (257, 1024, 32, 8, 40, 8),
    (300, 384, 128, 16, 24, 16),
    (2051, 256, 256, 8, 80, 8),       # prefill-sized tiles, E = 256: the fused layout+dispatch
    (700, 128, 512, 4, 9, 4),         # E = 512: its histograms exceed the fused kernel's LDS,
                                      # the call runs as two launches
    (40, 256, 300, 256, 20, 3),       # K = EP_MAX_TOPK
    (600, 256, 32, 6, 40, 4),         # 512 <= T < 1024: fused tiles of two tokens
    (40, 32896, 6, 3, 12, 3),         # rows longer than the combine's zero row
]


@pytest.mark.parametrize("align", [1, 16, 128])
@pytest.mark.parametrize("T,H,E,K,C,R", SMALL)
def test_packed_small(T, H, E, K, C, R, align):
    _need_gpu()
    print(f"[packed] small T={T} H={H} E={E} K={K} C={C} R={R} align={align}", flush=True)
    rng = np.random.default_rng(T + H + align)
    idx = rng.integers(-2, E + 1, size=(T, K)).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.random((T, K)).astype(np.float32)
    run_case(idx, x, w, E, C, R, align, seed=T)


def test_packed_truncated_buffer():
    """A buffer shorter than the offsets need: pairs past its end are not written and count as
    dropped in combine, exactly as the oracle says."""
    _need_gpu()
    rng = np.random.default_rng(5)
    T, H, E, K, C, R = 200, 256, 16, 4, 60, 4
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.random((T, K)).astype(np.float32)
    off = oracle.packed_offsets(oracle.layout(idx, E, C, R)["count"], 8)
    run_case(idx, x, w, E, C, R, 8, rows=int(off[-1]) - 37)


@pytest.mark.parametrize("name,align", [("unbalanced_r4", 128), ("unbalanced_r4_c512", 64),
                                        ("decode_bf16", 16), ("prefill_bf16", 128)])
def test_packed_workloads(name, align):
    _need_gpu()
    cfg = W.get_config(name)
    print(f"[packed] {name} align={align}", flush=True)
    inp = W.make_inputs(cfg)
    run_case(inp["topk_idx"], inp["x"], inp["topk_w"], cfg.E, cfg.C, cfg.R, align,
             seed=cfg.seed)


def test_packed_empty_tokens():
    """T = 0: zero offsets (the packed buffer needs no rows), zero counts and stats, nothing
    written."""
    _need_gpu()
    E, C, R, H = 16, 4, 4, 256
    idx = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    x = torch.zeros((0, H), dtype=torch.int16, device="cuda")
    i32 = lambda n, v: torch.full((n,), v, dtype=torch.int32, device="cuda")
    g = B.ep_layout_packed(idx, E, C, R, 16, packed_offset=i32(E + 1, 7))
    torch.cuda.synchronize()
    assert G.to_np(g["packed_offset"]).tolist() == [0] * (E + 1)
    assert G.to_np(g["expert_count"]).tolist() == [0] * E
    assert G.to_np(g["stats"]).tolist() == [0, 0, 0, 0]
    recv = torch.full((8, H), S16, dtype=torch.int16, device="cuda")
    f = B.ep_layout_dispatch_packed(x, idx, recv, E, C, R, 16, packed_offset=i32(E + 1, 7),
                                    stats=i32(4, 7))
    q = torch.full((8, H), S8, dtype=torch.uint8, device="cuda")
    sc = torch.full((8, H // 128), SF, dtype=torch.float32, device="cuda")
    f8 = B.ep_layout_dispatch_packed_fp8(x, idx, q, sc, E, C, R, 16, stats=i32(4, 7))
    out = B.ep_combine_packed(recv, idx, g["slot"], g["packed_offset"],
                              torch.zeros((0, 8), device="cuda"), E, C)
    torch.cuda.synchronize()
    assert G.to_np(f["packed_offset"]).tolist() == [0] * (E + 1)
    assert G.to_np(f["stats"]).tolist() == [0, 0, 0, 0] == G.to_np(f8["stats"]).tolist()
    assert int((recv != S16).sum()) == 0 and int((q != S8).sum()) == 0
    assert out.shape == (0, H)
