"""GPU parity of the two-stage, rank-deduplicated path (ep_rank_layout, ep_dispatch_ranks[_fp8],
ep_dispatch_expand[_fp8], ep_layout_dispatch_expand[_fp8], ep_combine_ranks, ep_combine_reduce) against
the oracle.

Small shapes compare whole buffers bit for bit, with sentinels in every row a call must not
touch. The full workloads compare the rank layout in full, every staged row (bf16 and FP8) with
the oracle's staging copy, the composed dispatch with the one-stage dispatch (itself checked
against the oracle), and every partial row and every output element of the two-stage combine
with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W
import gpu_cases as G

pytestmark = pytest.mark.gpu

S16 = G.SENTINEL16
S8 = G.SENTINEL8
SF = G.SENTINEL_F32


LAYOUT_KEYS = ("slot", "expert_count", "expert_offset", "rank_count", "rank_offset", "stats")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


class TwoStage:
    """Inputs on host and device, the expert layout (GPU, checked against the oracle) and the
    rank layout (GPU, checked against the oracle)."""

    def __init__(self, T, H, E, K, C, R, idx, x, w, seed):
        self.T, self.H, self.E, self.K, self.C, self.R = T, H, E, K, C, R
        self.idx, self.x, self.w, self.seed = idx, x, w, seed
        self.case = G.Case(T, H, E, K, C, R, x, idx, w, seed)     # checks the expert layout
        self.slot = self.case.lay["slot"]
        self.rl = oracle.rank_layout(idx, E, R)
        self.g = B.ep_rank_layout(self.case.idx_d, E, R)
        torch.cuda.synchronize()
        assert np.array_equal(G.to_np(self.g["rank_slot"]), self.rl["rank_slot"]), "rank_slot"
        assert np.array_equal(G.to_np(self.g["rank_tokens"]), self.rl["rank_tokens"]), "rank_tokens"

    @classmethod
    def random(cls, T, H, E, K, C, R, seed, lo=-2):
        rng = np.random.default_rng(seed)
        idx = rng.integers(lo, E + 1, size=(T, K)).astype(np.int32)
        x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        w = rng.random((T, K)).astype(np.float32)
        return cls(T, H, E, K, C, R, idx, x, w, seed)

    @classmethod
    def from_config(cls, cfg):
        inp = W.make_inputs(cfg)
        return cls(cfg.T, cfg.H, cfg.E, cfg.K, cfg.C, cfg.R, inp["topk_idx"], inp["x"],
                   inp["topk_w"], cfg.seed)

    # ------------------------------------------------------------------------------------
    def dispatch_bf16_full(self):
        T, H, E, C, R = self.T, self.H, self.E, self.C, self.R
        stage = torch.full((R, T, H), S16, dtype=torch.int16, device=G.dev())
        B.ep_dispatch_ranks(self.case.x_d, self.g["rank_slot"], stage)
        torch.cuda.synchronize()
        want_stage = np.full((R, T, H), S16, np.uint16)
        oracle.dispatch_ranks(self.x, self.rl["rank_slot"], want_stage)
        assert np.array_equal(G.to_np(stage).view(np.uint16), want_stage), "stage"
        recv = torch.full((E, C, H), S16, dtype=torch.int16, device=G.dev())
        B.ep_dispatch_expand(stage, self.case.idx_d, self.case.g["slot"], self.g["rank_slot"],
                             recv, C)
        torch.cuda.synchronize()
        want = np.full((E, C, H), S16, np.uint16)
        oracle.dispatch_expand(want_stage, self.idx, self.slot, self.rl["rank_slot"], E, C, want)
        assert np.array_equal(G.to_np(recv).view(np.uint16), want), "recv"
        one = np.full((E, C, H), S16, np.uint16)
        oracle.dispatch(self.x, self.idx, self.slot, E, C, one)
        assert np.array_equal(want, one), "two-stage oracle differs from one-stage"
        # the expert layout fused with the expansion: the layout's outputs and the same recv
        lx_recv = torch.full((E, C, H), S16, dtype=torch.int16, device=G.dev())
        lx = B.ep_layout_dispatch_expand(stage, self.case.idx_d, self.g["rank_slot"], lx_recv,
                                         E, C)
        torch.cuda.synchronize()
        for k in LAYOUT_KEYS:
            assert torch.equal(lx[k], self.case.g[k]), f"fused layout+expand {k}"
        assert np.array_equal(G.to_np(lx_recv).view(np.uint16), want), "fused layout+expand recv"
        # the fused rank layout + stage 1: the same three outputs
        fused = torch.full((R, T, H), S16, dtype=torch.int16, device=G.dev())
        f = B.ep_rank_layout_dispatch(self.case.x_d, self.case.idx_d, E, R, stage=fused)
        torch.cuda.synchronize()
        assert np.array_equal(G.to_np(f["rank_slot"]), self.rl["rank_slot"]), "fused rank_slot"
        assert np.array_equal(G.to_np(f["rank_tokens"]), self.rl["rank_tokens"]), "fused rank_tokens"
        assert np.array_equal(G.to_np(fused).view(np.uint16), want_stage), "fused stage"

    def dispatch_fp8_full(self):
        T, H, E, C, R = self.T, self.H, self.E, self.C, self.R
        NB = H // 128
        sq = torch.full((R, T, H), S8, dtype=torch.uint8, device=G.dev())
        ss = torch.full((R, T, NB), SF, dtype=torch.float32, device=G.dev())
        B.ep_dispatch_ranks_fp8(self.case.x_d, self.g["rank_slot"], sq, ss)
        torch.cuda.synchronize()
        wq = np.full((R, T, H), S8, np.uint8)
        ws = np.full((R, T, NB), SF, np.float32)
        oracle.dispatch_ranks_fp8(self.x, self.rl["rank_slot"], wq, ws)
        assert np.array_equal(G.to_np(sq), wq), "stage codes"
        assert np.array_equal(G.to_np(ss).view(np.uint32), ws.view(np.uint32)), "stage scales"
        fq = torch.full((R, T, H), S8, dtype=torch.uint8, device=G.dev())
        fs = torch.full((R, T, NB), SF, dtype=torch.float32, device=G.dev())
        f = B.ep_rank_layout_dispatch_fp8(self.case.x_d, self.case.idx_d, self.E, R, stage_q=fq,
                                          stage_scale=fs)
        torch.cuda.synchronize()
        assert np.array_equal(G.to_np(f["rank_slot"]), self.rl["rank_slot"]), "fused rank_slot"
        assert np.array_equal(G.to_np(f["rank_tokens"]), self.rl["rank_tokens"]), "fused rank_tokens"
        assert np.array_equal(G.to_np(fq), wq), "fused stage codes"
        assert np.array_equal(G.to_np(fs).view(np.uint32), ws.view(np.uint32)), "fused stage scales"
        del fq, fs
        rq = torch.full((E, C, H), S8, dtype=torch.uint8, device=G.dev())
        rs = torch.full((E, C, NB), SF, dtype=torch.float32, device=G.dev())
        B.ep_dispatch_expand_fp8(sq, ss, self.case.idx_d, self.case.g["slot"],
                                 self.g["rank_slot"], rq, rs, C)
        torch.cuda.synchronize()
        oq = np.full((E, C, H), S8, np.uint8)
        os_ = np.full((E, C, NB), SF, np.float32)
        oracle.dispatch_fp8(self.x, self.idx, self.slot, E, C, oq, os_)
        assert np.array_equal(G.to_np(rq), oq), "recv codes"
        assert np.array_equal(G.to_np(rs).view(np.uint32), os_.view(np.uint32)), "recv scales"
        # the expert layout fused with the FP8 expansion
        lq = torch.full((E, C, H), S8, dtype=torch.uint8, device=G.dev())
        ls = torch.full((E, C, NB), SF, dtype=torch.float32, device=G.dev())
        lx = B.ep_layout_dispatch_expand_fp8(sq, ss, self.case.idx_d, self.g["rank_slot"], lq, ls,
                                             E, C)
        torch.cuda.synchronize()
        for k in LAYOUT_KEYS:
            assert torch.equal(lx[k], self.case.g[k]), f"fused FP8 layout+expand {k}"
        assert np.array_equal(G.to_np(lq), oq), "fused FP8 layout+expand codes"
        assert np.array_equal(G.to_np(ls).view(np.uint32), os_.view(np.uint32)), "fused scales"

    def combine_full(self):
        T, H, R = self.T, self.H, self.R
        y_host, y = self.case.make_y()
        part = torch.full((R, T, H), S16, dtype=torch.int16, device=G.dev())
        B.ep_combine_ranks(y, self.case.idx_d, self.case.g["slot"], self.g["rank_slot"],
                           self.case.w_d, self.C, part=part)
        torch.cuda.synchronize()
        want_part = oracle.combine_ranks(y_host, self.idx, self.slot, self.rl["rank_slot"], self.w)
        got_part = G.to_np(part).view(np.uint16)
        sent = self.rl["rank_slot"] >= 0
        t_i, r_i = np.nonzero(sent)
        p_i = self.rl["rank_slot"][t_i, r_i]
        assert np.array_equal(got_part[r_i, p_i], want_part[r_i, p_i]), "partial rows"
        mask = np.ones((R, T), bool)
        mask[r_i, p_i] = False
        assert (got_part[mask] == np.uint16(S16)).all(), "rows outside the sent set were written"
        out = B.ep_combine_reduce(part, self.g["rank_slot"], self.K)
        torch.cuda.synchronize()
        want = oracle.combine_reduce(want_part, self.rl["rank_slot"])
        got = G.to_np(out).view(np.uint16)
        assert np.array_equal(got, want), "combine_reduce"
        return got, y


SMALL = [
    # T, H, E, K, C, R
    (1, 8, 1, 1, 1, 1),
    (3, 24, 4, 2, 2, 2),
    (37, 256, 6, 3, 5, 3),
    (100, 520, 16, 4, 9, 4),          # H/8 = 65: one chunk past a full wavefront
    (257, 1024, 32, 8, 40, 8),
    (300, 384, 128, 16, 24, 16),      # K = 16: the sequential partial-combine path
    (2049, 256, 8, 1, 300, 2),        # K = 1
    (400, 128, 64, 8, 60, 64),        # one expert per rank, R at its maximum
    (150, 1152, 12, 5, 80, 1),        # a single rank; FP8 segment 2 is partial
    (9000, 64, 32, 8, 4000, 8),       # rank layout past five tiles: the batched prefix loop
    (6000, 64, 24, 6, 3000, 6),       # the same with K = 6 (ids one at a time)
    (40, 256, 300, 256, 20, 3),       # K = EP_MAX_TOPK
    (40, 32896, 6, 3, 12, 3),         # rows longer than the zero row: the reduce's select
]


@pytest.mark.parametrize("T,H,E,K,C,R", SMALL)
def test_two_stage_small(T, H, E, K, C, R):
    _need_gpu()
    print(f"[two-stage] small T={T} H={H} E={E} K={K} C={C} R={R}", flush=True)
    ts = TwoStage.random(T, H, E, K, C, R, seed=T + H + R)
    ts.dispatch_bf16_full()
    if H % 128 == 0:
        ts.dispatch_fp8_full()
    got, y = ts.combine_full()
    if R == 1:    # a single rank: the one-stage combine, bit for bit (up to the sign of zero)
        one = G.to_np(B.ep_combine(y, ts.case.idx_d, ts.case.g["slot"], ts.case.w_d, C))
        torch.cuda.synchronize()
        assert G.ulp_distance_bf16(got, one.view(np.uint16)).max(initial=0) == 0


@pytest.mark.parametrize("name", ["decode_bf16", "decode_fp8", "skew_zipf_c256",
                                  "prefill_bf16", "prefill_fp8"])
def test_two_stage_workloads(name):
    """Full workloads: rank layout in full; the composed dispatch equals the one-stage GPU
    dispatch; sampled output rows against the oracle's two-stage combine."""
    _need_gpu()
    cfg = W.get_config(name)
    print(f"[two-stage] {name}", flush=True)
    ts = TwoStage.from_config(cfg)
    T, H, E, C, R, K = cfg.T, cfg.H, cfg.E, cfg.C, cfg.R, cfg.K
    c = ts.case
    if cfg.fp8:
        NB = H // 128
        sq = torch.empty((R, T, H), dtype=torch.uint8, device=G.dev())
        ss = torch.empty((R, T, NB), dtype=torch.float32, device=G.dev())
        B.ep_dispatch_ranks_fp8(c.x_d, ts.g["rank_slot"], sq, ss)
        f = B.ep_rank_layout_dispatch_fp8(c.x_d, c.idx_d, E, R)
        torch.cuda.synchronize()
        assert torch.equal(f["rank_slot"], ts.g["rank_slot"])
        assert torch.equal(f["rank_tokens"], ts.g["rank_tokens"])
        sent = torch.from_numpy(ts.rl["rank_slot"] >= 0).to(G.dev())
        tt, rr = torch.nonzero(sent, as_tuple=True)
        rows = rr * T + ts.g["rank_slot"][tt, rr].long()
        assert torch.equal(f["stage_q"].view(R * T, H)[rows], sq.view(R * T, H)[rows])
        assert torch.equal(f["stage_scale"].view(R * T, -1)[rows].view(torch.int32),
                           ss.view(R * T, -1)[rows].view(torch.int32))
        del f
        # every staged row against the oracle's staging copy
        wq = np.empty((R, T, H), np.uint8)
        ws = np.empty((R, T, NB), np.float32)
        oracle.dispatch_ranks_fp8(ts.x, ts.rl["rank_slot"], wq, ws)
        t_i, r_i = np.nonzero(ts.rl["rank_slot"] >= 0)
        p_i = ts.rl["rank_slot"][t_i, r_i]
        assert np.array_equal(G.to_np(sq)[r_i, p_i], wq[r_i, p_i]), "staged codes"
        assert np.array_equal(G.to_np(ss)[r_i, p_i].view(np.uint32),
                              ws[r_i, p_i].view(np.uint32)), "staged scales"
        del wq, ws
        q2 = torch.full((E, C, H), S8, dtype=torch.uint8, device=G.dev())
        s2 = torch.full((E, C, NB), SF, dtype=torch.float32, device=G.dev())
        B.ep_dispatch_expand_fp8(sq, ss, c.idx_d, c.g["slot"], ts.g["rank_slot"], q2, s2, C)
        q1 = torch.full((E, C, H), S8, dtype=torch.uint8, device=G.dev())
        s1 = torch.full((E, C, NB), SF, dtype=torch.float32, device=G.dev())
        B.ep_dispatch_fp8(c.x_d, c.idx_d, c.g["slot"], q1, s1, C)
        torch.cuda.synchronize()
        assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
        del q2, s2
        q3 = torch.full((E, C, H), S8, dtype=torch.uint8, device=G.dev())
        s3 = torch.full((E, C, NB), SF, dtype=torch.float32, device=G.dev())
        lx = B.ep_layout_dispatch_expand_fp8(sq, ss, c.idx_d, ts.g["rank_slot"], q3, s3, E, C)
        torch.cuda.synchronize()
        assert torch.equal(q1, q3) and torch.equal(s1.view(torch.int32), s3.view(torch.int32))
        for k in LAYOUT_KEYS:
            assert torch.equal(lx[k], c.g[k]), f"fused FP8 layout+expand {k}"
        del sq, ss, q1, q3, s1, s3
    else:
        stage = torch.empty((R, T, H), dtype=torch.int16, device=G.dev())
        B.ep_dispatch_ranks(c.x_d, ts.g["rank_slot"], stage)
        f = B.ep_rank_layout_dispatch(c.x_d, c.idx_d, E, R)
        torch.cuda.synchronize()
        assert torch.equal(f["rank_slot"], ts.g["rank_slot"])
        assert torch.equal(f["rank_tokens"], ts.g["rank_tokens"])
        sent = torch.from_numpy(ts.rl["rank_slot"] >= 0).to(G.dev())
        tt, rr = torch.nonzero(sent, as_tuple=True)
        rows = rr * T + ts.g["rank_slot"][tt, rr].long()
        assert torch.equal(f["stage"].view(R * T, H)[rows], stage.view(R * T, H)[rows])
        del f
        r2 = torch.full((E, C, H), S16, dtype=torch.int16, device=G.dev())
        B.ep_dispatch_expand(stage, c.idx_d, c.g["slot"], ts.g["rank_slot"], r2, C)
        r1 = torch.full((E, C, H), S16, dtype=torch.int16, device=G.dev())
        B.ep_dispatch(c.x_d, c.idx_d, c.g["slot"], r1, C)
        torch.cuda.synchronize()
        assert torch.equal(r1, r2)
        del r2
        r3 = torch.full((E, C, H), S16, dtype=torch.int16, device=G.dev())
        lx = B.ep_layout_dispatch_expand(stage, c.idx_d, ts.g["rank_slot"], r3, E, C)
        torch.cuda.synchronize()
        assert torch.equal(r1, r3), "fused layout+expand recv"
        for k in LAYOUT_KEYS:
            assert torch.equal(lx[k], c.g[k]), f"fused layout+expand {k}"
        del r3
        # every staged row against the oracle's staging copy (and it is the token's row)
        want_stage = np.empty((R, T, H), np.uint16)
        oracle.dispatch_ranks(ts.x, ts.rl["rank_slot"], want_stage)
        t_i, r_i = np.nonzero(ts.rl["rank_slot"] >= 0)
        p_i = ts.rl["rank_slot"][t_i, r_i]
        got = G.to_np(stage).view(np.uint16)[r_i, p_i]
        assert np.array_equal(got, want_stage[r_i, p_i]), "staged rows"
        assert np.array_equal(want_stage[r_i, p_i], ts.x[t_i]), "oracle staging round trip"
        del stage, r1, want_stage, got
    torch.cuda.empty_cache()
    y_host, y = c.make_y()
    part = B.ep_combine_ranks(y, c.idx_d, c.g["slot"], ts.g["rank_slot"], c.w_d, C)
    out = B.ep_combine_reduce(part, ts.g["rank_slot"], K)
    torch.cuda.synchronize()
    # every partial row and every output element against the oracle
    want_part = oracle.combine_ranks(y_host, ts.idx, ts.slot, ts.rl["rank_slot"], ts.w)
    t_i, r_i = np.nonzero(ts.rl["rank_slot"] >= 0)
    p_i = ts.rl["rank_slot"][t_i, r_i]
    assert np.array_equal(G.to_np(part).view(np.uint16)[r_i, p_i], want_part[r_i, p_i]), \
        "partial rows"
    want = oracle.combine_reduce(want_part, ts.rl["rank_slot"])
    del want_part
    got = G.to_np(out).view(np.uint16)
    assert np.array_equal(got, want), "combine_reduce"
    # against the one-stage combine at every element: the two results differ by the rounding
    # of each partial to bf16 plus the two final roundings, so
    #   |out2 - out1| <= 2^-8 * (sum_r |partial_r| + |out1| + |out2|) + 2^-20 * sum_r |partial_r|
    # (bf16 keeps 8 significant bits: rounding moves a value by at most 2^-8 of it; the last
    # term covers the fp32 sums)
    one = B.ep_combine(y, c.idx_d, c.g["slot"], c.w_d, C)
    torch.cuda.synchronize()
    f64 = lambda a: W.bf16_bits_to_f32(np.ascontiguousarray(a).view(np.uint16)).astype(np.float64)
    out2, out1 = f64(G.to_np(out)), f64(G.to_np(one))
    part_np = G.to_np(part).view(np.uint16)
    mag = np.zeros((T, H), np.float64)
    for r in range(R):
        sent = ts.rl["rank_slot"][:, r] >= 0
        rows = ts.rl["rank_slot"][sent, r]
        mag[sent] += np.abs(f64(part_np[r, rows]))
    bound = 2.0 ** -8 * (mag + np.abs(out1) + np.abs(out2)) + 2.0 ** -20 * mag
    excess = np.abs(out2 - out1) - bound
    assert excess.max() <= 0, f"two-stage vs one-stage beyond the rounding bound: {excess.max()}"
    d = G.ulp_distance_bf16(G.to_np(out).view(np.uint16), G.to_np(one).view(np.uint16))
    print(f"[two-stage] {name}: equal to one-stage in {np.mean(d == 0):.3f} of elements, "
          f"all within the rounding bound", flush=True)


def test_two_stage_empty_and_unrouted():
    _need_gpu()
    idx = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    g = B.ep_rank_layout(idx, 8, 4)
    torch.cuda.synchronize()
    assert G.to_np(g["rank_tokens"]).tolist() == [0, 0, 0, 0]
    x0 = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    for fn in (B.ep_rank_layout_dispatch, B.ep_rank_layout_dispatch_fp8):
        rt = torch.full((4,), 7, dtype=torch.int32, device="cuda")
        fn(x0, idx, 8, 4, rank_tokens=rt)
        torch.cuda.synchronize()
        assert G.to_np(rt).tolist() == [0, 0, 0, 0]
    # T = 0 through the fused layout + expansion: zero counts, nothing copied
    recv = torch.full((8, 2, 256), S16, dtype=torch.int16, device="cuda")
    lx = B.ep_layout_dispatch_expand(torch.zeros((4, 0, 256), dtype=torch.int16, device="cuda"),
                                     idx, torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                                     recv, 8, 2)
    torch.cuda.synchronize()
    assert G.to_np(lx["expert_count"]).tolist() == [0] * 8
    assert (G.to_np(recv).view(np.uint16) == np.uint16(S16)).all()
    # the same for FP8: zero counts and stats, nothing copied
    rq = torch.full((8, 2, 256), S8, dtype=torch.uint8, device="cuda")
    rs = torch.full((8, 2, 2), SF, dtype=torch.float32, device="cuda")
    lq = B.ep_layout_dispatch_expand_fp8(torch.zeros((4, 0, 256), dtype=torch.uint8, device="cuda"),
                                         torch.zeros((4, 0, 2), dtype=torch.float32, device="cuda"),
                                         idx, torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                                         rq, rs, 8, 2,
                                         stats=torch.full((4,), 7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert G.to_np(lq["expert_count"]).tolist() == [0] * 8
    assert G.to_np(lq["stats"]).tolist() == [0, 0, 0, 0]
    assert int((rq != S8).sum()) == 0 and int((rs != SF).sum()) == 0
    # every id unrouted or invalid: nothing is sent anywhere, the output is +0
    ts = TwoStage(16, 64, 8, 4, 4, 4, np.where(np.arange(64).reshape(16, 4) % 2, -1, 9)
                  .astype(np.int32), W.f32_to_bf16_bits(np.ones((16, 64), np.float32)),
                  np.ones((16, 4), np.float32), 0)
    assert (ts.rl["rank_slot"] == -1).all()
    got, _ = ts.combine_full()
    assert (got == 0).all()


def test_two_stage_pass_with_layout_on_a_second_stream():
    """The expert layout on a second stream, beside the fused rank layout + staging copy on the
    first (both read only the batch), the expansion and the combines after the first waits for
    the second: the same outputs as the five launches in one stream, and the oracle's layouts."""
    _need_gpu()
    print("[two-stage] layout on a second stream", flush=True)
    T, H, E, K, C, R = 700, 512, 64, 8, 80, 16
    case = G.Case.random(T, H, E, K, C, R, seed=31, lo=0, hi=E)
    y_host, y = case.make_y()
    dev = G.dev()

    def run(overlap):
        mk = lambda *n: torch.empty(n, dtype=torch.int32, device=dev)
        lay = dict(slot=mk(T, K), expert_count=mk(E), expert_offset=mk(E), rank_count=mk(R),
                   rank_offset=mk(R), stats=mk(4))
        stage = torch.empty((R, T, H), dtype=torch.int16, device=dev)
        recv = torch.full((E, C, H), S16, dtype=torch.int16, device=dev)
        part = torch.empty((R, T, H), dtype=torch.int16, device=dev)
        torch.cuda.synchronize()
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        if overlap:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                B.ep_layout(case.idx_d, E, C, R, **lay)
        else:
            B.ep_layout(case.idx_d, E, C, R, **lay)
        rl = B.ep_rank_layout_dispatch(case.x_d, case.idx_d, E, R, stage=stage)
        if overlap:
            main.wait_stream(side)
        B.ep_dispatch_expand(stage, case.idx_d, lay["slot"], rl["rank_slot"], recv, C)
        B.ep_combine_ranks(y, case.idx_d, lay["slot"], rl["rank_slot"], case.w_d, C, part=part)
        out = B.ep_combine_reduce(part, rl["rank_slot"], K)
        torch.cuda.synchronize()
        return lay, rl, recv, out

    lay0, rl0, recv0, out0 = run(False)
    for rep in range(3):
        lay1, rl1, recv1, out1 = run(True)
        for k in lay0:
            assert torch.equal(lay0[k], lay1[k]), f"rep {rep}: {k}"
        assert torch.equal(rl0["rank_slot"], rl1["rank_slot"]), f"rep {rep}: rank_slot"
        assert torch.equal(recv0, recv1), f"rep {rep}: recv"
        assert torch.equal(out0, out1), f"rep {rep}: out"
    G.check_layout(case.idx, E, C, R, lay1)
    want = oracle.rank_layout(case.idx, E, R)
    assert np.array_equal(G.to_np(rl1["rank_slot"]), want["rank_slot"])
