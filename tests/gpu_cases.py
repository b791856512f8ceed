"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the oracle on the
same seeded inputs, and compare.

Nothing here computes an expected value itself: expected values come from ``oracle`` only.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W

SENTINEL16 = 0x5A5A        # bf16 pattern left in receive rows nobody may touch
SENTINEL8 = 0xA5
SENTINEL_F32 = -7.25
BF16_NAN = 0x7FC0          # unreferenced y rows hold NaN: a stray combine read shows up


def dev():
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def u16_dev(a: np.ndarray) -> torch.Tensor:
    return to_dev(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def kept_pairs(lay):
    """(pair index, token, expert, slot) of every kept pair, from the oracle's layout."""
    slot = lay["slot"].reshape(-1)
    i = np.nonzero(slot >= 0)[0]
    return i, slot[i]


def check_layout(idx: np.ndarray, E: int, C: int, R: int, g: dict) -> dict:
    """Run ep_layout's outputs against the oracle, bit for bit. Returns the oracle result."""
    want = oracle.layout(idx, E, C, R)
    assert np.array_equal(to_np(g["slot"]).reshape(idx.shape), want["slot"]), "slot"
    assert np.array_equal(to_np(g["expert_count"]), want["count"]), "expert_count"
    assert np.array_equal(to_np(g["expert_offset"]), want["offset"]), "expert_offset"
    assert np.array_equal(to_np(g["rank_count"]), want["rank_count"]), "rank_count"
    assert np.array_equal(to_np(g["rank_offset"]), want["rank_offset"]), "rank_offset"
    assert np.array_equal(to_np(g["stats"]), want["stats_array"]), "stats"
    return want


def ulp_distance_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 ulps on the monotonic integer line (+0 and -0 coincide)."""
    def mono(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(mono(a) - mono(b))


class Case:
    """One parity case: inputs on host and device, the oracle layout, and the GPU layout."""

    def __init__(self, T, H, E, K, C, R, x, idx, w, seed=0):
        self.T, self.H, self.E, self.K, self.C, self.R = T, H, E, K, C, R
        self.x, self.idx, self.w, self.seed = x, idx, w, seed
        self.x_d = u16_dev(x)
        self.idx_d = to_dev(idx.astype(np.int32))
        self.w_d = to_dev(w.astype(np.float32))
        torch.cuda.synchronize()
        self.g = B.ep_layout(self.idx_d, E, C, R)
        torch.cuda.synchronize()
        self.lay = check_layout(idx, E, C, R, self.g)

    @classmethod
    def from_config(cls, cfg: W.EpConfig):
        inp = W.make_inputs(cfg)
        return cls(cfg.T, cfg.H, cfg.E, cfg.K, cfg.C, cfg.R, inp["x"], inp["topk_idx"],
                   inp["topk_w"], cfg.seed)

    @classmethod
    def random(cls, T, H, E, K, C, R, seed=0, lo=-2, hi=None):
        rng = np.random.default_rng(seed)
        hi = E + 1 if hi is None else hi
        idx = rng.integers(lo, hi, size=(T, K)).astype(np.int32)
        x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        w = rng.random((T, K)).astype(np.float32)
        return cls(T, H, E, K, C, R, x, idx, w, seed)

    # -------------------------------------------------------------------------------------
    def check_dispatch_bf16(self, full: bool):
        E, C, H = self.E, self.C, self.H
        recv = torch.full((E, C, H), SENTINEL16, dtype=torch.int16, device=dev())
        B.ep_dispatch(self.x_d, self.idx_d, self.g["slot"], recv, C)
        torch.cuda.synchronize()
        i, s = kept_pairs(self.lay)
        e = self.idx.reshape(-1)[i]
        t = i // self.K
        if full:
            want = np.full((E, C, H), SENTINEL16, dtype=np.uint16)
            oracle.dispatch(self.x, self.idx, self.lay["slot"], E, C, want)
            assert np.array_equal(to_np(recv).view(np.uint16), want)
            return
        # large buffers: the kept rows one by one against the oracle's rows, then every other
        # row must still hold the sentinel
        want = np.empty((E, C, H), dtype=np.uint16)          # only kept rows get written
        oracle.dispatch(self.x, self.idx, self.lay["slot"], E, C, want)
        rows = torch.from_numpy((e.astype(np.int64) * C + s)).to(dev())
        got = recv.view(E * C, H).index_select(0, rows)
        assert np.array_equal(to_np(got).view(np.uint16), want[e, s]), "kept rows"
        assert np.array_equal(want[e, s], self.x[t]), "oracle round trip"
        recv.view(E * C, H).index_fill_(0, rows, SENTINEL16)
        assert int((recv != SENTINEL16).sum()) == 0, "rows outside the kept set were written"

    def check_dispatch_fp8(self, full: bool):
        E, C, H = self.E, self.C, self.H
        NB = H // 128
        q = torch.full((E, C, H), SENTINEL8, dtype=torch.uint8, device=dev())
        sc = torch.full((E, C, NB), SENTINEL_F32, dtype=torch.float32, device=dev())
        B.ep_dispatch_fp8(self.x_d, self.idx_d, self.g["slot"], q, sc, C)
        torch.cuda.synchronize()
        i, s = kept_pairs(self.lay)
        e = self.idx.reshape(-1)[i]
        if full:
            wq = np.full((E, C, H), SENTINEL8, dtype=np.uint8)
            ws = np.full((E, C, NB), SENTINEL_F32, dtype=np.float32)
            oracle.dispatch_fp8(self.x, self.idx, self.lay["slot"], E, C, wq, ws)
            assert np.array_equal(to_np(q), wq), "codes"
            assert np.array_equal(to_np(sc).view(np.uint32), ws.view(np.uint32)), "scales"
            return
        wq = np.empty((E, C, H), dtype=np.uint8)
        ws = np.empty((E, C, NB), dtype=np.float32)
        oracle.dispatch_fp8(self.x, self.idx, self.lay["slot"], E, C, wq, ws)
        rows = torch.from_numpy((e.astype(np.int64) * C + s)).to(dev())
        gq = to_np(q.view(E * C, H).index_select(0, rows))
        gs = to_np(sc.view(E * C, NB).index_select(0, rows))
        assert np.array_equal(gq, wq[e, s]), "codes"
        assert np.array_equal(gs.view(np.uint32), ws[e, s].view(np.uint32)), "scales"
        q.view(E * C, H).index_fill_(0, rows, SENTINEL8)
        sc.view(E * C, NB).index_fill_(0, rows, SENTINEL_F32)
        assert int((q != SENTINEL8).sum()) == 0 and int((sc != SENTINEL_F32).sum()) == 0

    def check_fused(self, fp8: bool, full: bool, ws: bool = False, workspace=None):
        """ep_layout_dispatch[_fp8] (ws: the two-launch form with a workspace,
        ep_layout_dispatch[_fp8]_ws): every layout output bit-equal to the oracle's, and the
        receive buffers exactly as the separate dispatch must leave them. ``workspace`` (ws
        only): a device tensor to use, e.g. one holding stale data from another call."""
        E, C, H, R = self.E, self.C, self.H, self.R
        i, s = kept_pairs(self.lay)
        e = self.idx.reshape(-1)[i]
        rows = torch.from_numpy((e.astype(np.int64) * C + s)).to(dev())
        if fp8:
            NB = H // 128
            q = torch.full((E, C, H), SENTINEL8, dtype=torch.uint8, device=dev())
            sc = torch.full((E, C, NB), SENTINEL_F32, dtype=torch.float32, device=dev())
            if ws:
                g = B.ep_layout_dispatch_fp8_ws(self.x_d, self.idx_d, q, sc, E, C, R,
                                                workspace=workspace)
            else:
                g = B.ep_layout_dispatch_fp8(self.x_d, self.idx_d, q, sc, E, C, R)
        else:
            recv = torch.full((E, C, H), SENTINEL16, dtype=torch.int16, device=dev())
            if ws:
                g = B.ep_layout_dispatch_ws(self.x_d, self.idx_d, recv, E, C, R,
                                            workspace=workspace)
            else:
                g = B.ep_layout_dispatch(self.x_d, self.idx_d, recv, E, C, R)
        torch.cuda.synchronize()
        check_layout(self.idx, E, C, R, g)
        if fp8:
            wq = np.full((E, C, H), SENTINEL8, dtype=np.uint8) if full else np.empty((E, C, H), np.uint8)
            ws = (np.full((E, C, NB), SENTINEL_F32, dtype=np.float32) if full
                  else np.empty((E, C, NB), np.float32))
            oracle.dispatch_fp8(self.x, self.idx, self.lay["slot"], E, C, wq, ws)
            if full:
                assert np.array_equal(to_np(q), wq) and np.array_equal(to_np(sc).view(np.uint32), ws.view(np.uint32))
                return
            assert np.array_equal(to_np(q.view(E * C, H).index_select(0, rows)), wq[e, s])
            assert np.array_equal(to_np(sc.view(E * C, NB).index_select(0, rows)).view(np.uint32),
                                  ws[e, s].view(np.uint32))
            q.view(E * C, H).index_fill_(0, rows, SENTINEL8)
            sc.view(E * C, NB).index_fill_(0, rows, SENTINEL_F32)
            assert int((q != SENTINEL8).sum()) == 0 and int((sc != SENTINEL_F32).sum()) == 0
        else:
            want = np.full((E, C, H), SENTINEL16, dtype=np.uint16) if full else np.empty((E, C, H), np.uint16)
            oracle.dispatch(self.x, self.idx, self.lay["slot"], E, C, want)
            if full:
                assert np.array_equal(to_np(recv).view(np.uint16), want)
                return
            got = to_np(recv.view(E * C, H).index_select(0, rows)).view(np.uint16)
            assert np.array_equal(got, want[e, s])
            recv.view(E * C, H).index_fill_(0, rows, SENTINEL16)
            assert int((recv != SENTINEL16).sum()) == 0

    def make_y(self):
        """y on host and device: kept rows from the seeded expert-output stream, in pair
        order; every other row NaN on the device (and never read by the oracle)."""
        E, C, H = self.E, self.C, self.H
        i, s = kept_pairs(self.lay)
        e = self.idx.reshape(-1)[i]
        rows_np = W.y_rows(len(i), H, self.seed)
        y_host = np.empty((E, C, H), dtype=np.uint16)
        y_host[e, s] = rows_np
        y = torch.full((E, C, H), BF16_NAN, dtype=torch.int16, device=dev())
        if len(i):
            rows = torch.from_numpy((e.astype(np.int64) * C + s)).to(dev())
            y.view(E * C, H).index_copy_(0, rows, u16_dev(rows_np))
        return y_host, y

    def check_combine(self, y_host=None, y=None, w=None):
        if y is None:
            y_host, y = self.make_y()
        w = self.w if w is None else w
        w_d = self.w_d if w is self.w else to_dev(w.astype(np.float32))
        out = B.ep_combine(y, self.idx_d, self.g["slot"], w_d, self.C)
        torch.cuda.synchronize()
        got = to_np(out).view(np.uint16)
        want = oracle.combine(y_host, self.idx, self.lay["slot"], w)
        assert not np.isnan(W.bf16_bits_to_f32(got)).any(), "a NaN row of y was read"
        ulp = ulp_distance_bf16(got, want)
        assert ulp.max(initial=0) <= 1, f"max ulp {ulp.max()}"
        return got, want
