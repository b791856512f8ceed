"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on the same
seeded inputs.

Bars: layout, dispatch and the FP8 cast bit-exact; combine within 1 bf16 ulp per element (and,
by construction, expected bit-exact: both sides fold fmaf in ascending j from +0).

Full-size workloads run in the launch configuration the benchmark uses (the library picks it
from the shape). Their receive buffers are 1-2 GiB, so dispatch is checked row by row on every
kept pair plus a sentinel check of all other rows; combine is compared on every output element.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_06_amd import binding as B
from combine_ep_layout_06_amd import workloads as W

pytestmark = pytest.mark.gpu

import gpu_cases as G  # noqa: E402  (tests/ is on sys.path under pytest)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


FULL_CONFIGS = ["decode_bf16", "decode_fp8", "skew_zipf", "skew_zipf_c1024", "skew_zipf_c256",
                "prefill_bf16", "prefill_fp8", "balanced_stride"]


@pytest.mark.parametrize("name", FULL_CONFIGS)
def test_config_full_path(name):
    cfg = W.get_config(name)
    print(f"[parity] {name} T={cfg.T} H={cfg.H} E={cfg.E} K={cfg.K} C={cfg.C} R={cfg.R}",
          flush=True)
    case = G.Case.from_config(cfg)
    if cfg.fp8:
        case.check_dispatch_fp8(full=False)
    else:
        case.check_dispatch_bf16(full=False)
    got, want = case.check_combine()
    assert np.array_equal(got, want), "combine not bit-exact"
    if name.startswith("skew_zipf_c"):
        assert case.lay["stats"]["dropped"] > 0


@pytest.mark.parametrize("name", FULL_CONFIGS)
def test_config_fused_layout_dispatch(name):
    """ep_layout_dispatch[_fp8] on the full workloads, in both dispatch dtypes."""
    cfg = W.get_config(name)
    print(f"[parity] fused {name}", flush=True)
    case = G.Case.from_config(cfg)
    case.check_fused(fp8=False, full=False)
    case.check_fused(fp8=True, full=False)


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_fp8"])
def test_config_other_dispatch_dtype(name):
    """The dispatch dtype a workload does not use in the benchmark, for coverage."""
    cfg = W.get_config(name)
    case = G.Case.from_config(cfg)
    if cfg.fp8:
        case.check_dispatch_bf16(full=False)
    else:
        case.check_dispatch_fp8(full=False)


# small shapes that span several tiles and ragged tails, compared on whole buffers
SMALL = [
    # T, H, E, K, C, R
    (1, 8, 1, 1, 1, 1),
    (3, 24, 4, 2, 2, 2),
    (37, 256, 6, 3, 5, 3),
    (100, 520, 16, 4, 9, 4),          # H/8 = 65 chunks: one lane past a full wavefront
    (257, 1024, 32, 8, 40, 8),
    (1500, 128, 64, 6, 100, 4),       # T*K = 9000: nine layout tiles, a ragged last tile
    (300, 384, 128, 16, 24, 16),      # K = 16: two groups of 8 pairs
    (2049, 256, 8, 1, 300, 2),        # K = 1
    (2048, 3072, 16, 4, 600, 4),      # FP8 with two 1024-channel pieces per lane: 2 segments,
                                      # the second one's upper piece past H
    (2051, 256, 16, 4, 700, 4),       # fused tiles of 4 tokens (bf16) and 16 (FP8) with a
                                      # 3-token last tile
    (4099, 256, 16, 4, 1100, 4),      # bf16 fused tiles of 8 tokens, a 3-token last tile
    (40, 32896, 6, 3, 12, 3),         # H/8 = 4112 chunks, longer than the combine's zero row:
                                      # dropped pairs take the per-pair select
    (4100, 512, 64, 8, 200, 8),       # whole-row combine items folding rows in groups of two
                                      # with drops, unrouted and invalid ids
    (40, 256, 300, 256, 20, 3),       # K = EP_MAX_TOPK: 32 pair groups per token, full tiles
    (700, 256, 64, 6, 60, 8),         # 512 <= T < 1024: fused tiles of two tokens
    (600, 256, 32, 5, 90, 4),         # two tokens would make 10 pairs: tiles of four tokens
]


@pytest.mark.parametrize("T,H,E,K,C,R", SMALL)
def test_small_random_routes(T, H, E, K, C, R):
    """Random ids in [-2, E]: duplicates, unrouted (-1), invalid (-2 and E), and drops."""
    print(f"[parity] small T={T} H={H} E={E} K={K} C={C} R={R}", flush=True)
    case = G.Case.random(T, H, E, K, C, R, seed=T + H)
    case.check_dispatch_bf16(full=True)
    case.check_fused(fp8=False, full=True)
    if H % 128 == 0:
        case.check_dispatch_fp8(full=True)
        case.check_fused(fp8=True, full=True)
    got, want = case.check_combine()
    assert np.array_equal(got, want)


def test_empty_tokens():
    idx = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    g = B.ep_layout(idx, 16, 4, 4)
    torch.cuda.synchronize()
    assert G.to_np(g["expert_count"]).tolist() == [0] * 16
    assert G.to_np(g["expert_offset"]).tolist() == [0] * 16
    assert G.to_np(g["stats"]).tolist() == [0, 0, 0, 0]
    x = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    recv = torch.full((16, 4, 256), G.SENTINEL16, dtype=torch.int16, device="cuda")
    gf = B.ep_layout_dispatch(x, idx, recv, 16, 4, 4,
                              expert_count=torch.full((16,), 7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert G.to_np(gf["expert_count"]).tolist() == [0] * 16
    assert G.to_np(gf["stats"]).tolist() == [0, 0, 0, 0]
    B.ep_dispatch(x, idx, g["slot"], recv, 4)
    out = B.ep_combine(recv, idx, g["slot"], torch.zeros((0, 8), device="cuda"), 4)
    torch.cuda.synchronize()
    assert out.shape == (0, 256) and int((recv != G.SENTINEL16).sum()) == 0


def test_all_unrouted_and_all_to_one_expert():
    T, H, E, K, C, R = 64, 128, 8, 4, 3, 2
    rng = np.random.default_rng(1)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.random((T, K)).astype(np.float32)
    case = G.Case(T, H, E, K, C, R, x, np.full((T, K), -1, np.int32), w)
    assert case.lay["stats"]["unrouted"] == T * K
    case.check_dispatch_bf16(full=True)
    got, _ = case.check_combine()
    assert (got == 0).all()
    case = G.Case(T, H, E, K, C, R, x, np.full((T, K), 5, np.int32), w)
    assert case.lay["stats"]["dropped"] == T * K - C
    case.check_dispatch_bf16(full=True)
    case.check_dispatch_fp8(full=True)
    case.check_fused(fp8=False, full=True)
    case.check_fused(fp8=True, full=True)
    case.check_combine()


def test_max_experts_and_many_pairs():
    """E at its maximum (EP_MAX_EXPERTS) and 2^17 pairs (128 layout tiles), with drops."""
    cfg = W.EpConfig("max_e", T=16384, H=128, E=B.EP_MAX_EXPERTS, K=8, C=100, R=8)
    inp = W.make_inputs(cfg)
    case = G.Case(cfg.T, cfg.H, cfg.E, cfg.K, cfg.C, cfg.R, inp["x"], inp["topk_idx"],
                  inp["topk_w"])
    assert case.lay["stats"]["dropped"] > 0
    case.check_dispatch_bf16(full=False)
    case.check_fused(fp8=False, full=False)     # tiles past 32768 earlier ids: batched prefix
    case.check_fused(fp8=True, full=False)
    case.check_combine()


def test_balanced_route_counts_closed_form():
    cfg = W.get_config("balanced_stride")
    case = G.Case.from_config(cfg)
    per = cfg.T * cfg.K // cfg.E
    assert G.to_np(case.g["expert_count"]).tolist() == [per] * cfg.E


def test_fp8_every_bf16_value_through_the_quantiser():
    """Blocks whose amax is 448 have scale exactly 1, so the kernel's codes are e4m3(x) for
    every finite bf16 x with |x| <= 448 (both signs); a second pass with amax 3 exercises the
    division on the same values scaled into range."""
    vals = np.arange(0, 0x43E1, dtype=np.uint32)                     # +0 .. 448 as bf16 bits
    vals = np.concatenate([vals, vals | 0x8000]).astype(np.uint16)
    for amax_bits in (0x43E0, 0x4040):                                # 448.0, 3.0
        amax = W.bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0]
        keep = W.bf16_bits_to_f32(vals)
        v = vals[np.abs(keep) <= amax]
        per_block = 127
        nblk = -(-v.size // per_block)
        blocks = np.zeros((nblk, 128), dtype=np.uint16)
        flat = np.zeros(nblk * per_block, dtype=np.uint16)
        flat[:v.size] = v
        blocks[:, 1:] = flat.reshape(nblk, per_block)
        blocks[:, 0] = amax_bits
        H = 2048
        T = -(-nblk // (H // 128))
        x = np.zeros((T * (H // 128), 128), dtype=np.uint16)
        x[:nblk] = blocks
        x[nblk:, 0] = amax_bits
        x = x.reshape(T, H)
        idx = (np.arange(T, dtype=np.int32) % 4)[:, None]
        case = G.Case(T, H, 4, 1, T, 1, x, idx, np.ones((T, 1), np.float32))
        case.check_dispatch_fp8(full=True)
        case.check_fused(fp8=True, full=True)


def _fp8_blocks_case(blocks, H=2048):
    """Run [n][128] bf16 blocks (each block's amax in its own channels) through both FP8
    dispatch paths, against the oracle, one token row per H // 128 blocks."""
    nb = H // 128
    T = -(-blocks.shape[0] // nb)
    x = np.zeros((T * nb, 128), dtype=np.uint16)
    x[:blocks.shape[0]] = blocks
    x[blocks.shape[0]:, 0] = blocks[0, 0]                # no all-zero padding blocks
    x = x.reshape(T, H)
    idx = (np.arange(T, dtype=np.int32) % 4)[:, None]
    case = G.Case(T, H, 4, 1, T, 1, x, idx, np.ones((T, 1), np.float32))
    case.check_dispatch_fp8(full=True)
    case.check_fused(fp8=True, full=True)


def test_fp8_quotients_where_a_reciprocal_product_rounds_differently():
    """Inputs where RN(x * RN(1/scale)) and the IEEE quotient RN(x / scale) give different e4m3
    codes (found here by search on the CPU): the kernel must produce the codes of the IEEE
    quotient, as the definition and the oracle do."""
    rng = np.random.default_rng(7)
    pos = np.arange(1, 0x7F80, dtype=np.uint32)
    xf = (pos << 16).view(np.float32)
    blocks = []
    for ab in rng.integers(0x2180, 0x7F00, size=1500):
        amax = (np.uint32(ab) << 16).view(np.float32)
        s = np.float32(amax / np.float32(448.0))
        y = np.float32(np.float32(1.0) / s)
        xs = xf[xf <= amax]
        exact = torch.from_numpy((xs / s).astype(np.float32)).to(torch.float8_e4m3fn)
        recip = torch.from_numpy((xs * y).astype(np.float32)).to(torch.float8_e4m3fn)
        diff = np.nonzero((exact.view(torch.uint8) != recip.view(torch.uint8)).numpy())[0]
        if diff.size:
            v = (xs[diff].view(np.uint32) >> 16).astype(np.uint16)[:63]
            b = np.zeros(128, np.uint16)
            b[0] = ab
            b[1:1 + v.size] = v
            b[64:64 + v.size] = v | 0x8000
            blocks.append(b)
    assert len(blocks) > 100, len(blocks)
    _fp8_blocks_case(np.stack(blocks))


def test_fp8_small_amax_every_smaller_value():
    """Blocks whose amax is just above 2^-60 (the smallest amax of the reciprocal path) or a
    little larger, holding every bf16 value below it of both signs, subnormals included: the
    FMA remainders come closest to underflow here."""
    for ab in (0x2180, 0x21C1, 0x2300, 0x2F7F):
        amax = (np.uint32(ab) << 16).view(np.float32)
        vals = np.arange(0, 0x7F80, dtype=np.uint32)
        vals = vals[(vals << 16).view(np.float32) <= amax].astype(np.uint16)
        vals = np.concatenate([vals, vals | 0x8000])
        per = 127
        n = -(-vals.size // per)
        flat = np.zeros(n * per, np.uint16)
        flat[:vals.size] = vals
        blocks = np.zeros((n, 128), np.uint16)
        blocks[:, 0] = ab
        blocks[:, 1:] = flat.reshape(n, per)
        _fp8_blocks_case(blocks)


def test_fp8_degenerate_blocks():
    """All-zero blocks (scale 0, signed-zero codes), bf16 subnormals, a tiny amax."""
    H = 512
    x = np.zeros((3, H), dtype=np.uint16)
    x[0, :128] = 0x8000                                   # -0 block
    x[0, 128:256] = 0x0001                                # smallest bf16 subnormal
    x[0, 256] = 0x0080                                    # smallest bf16 normal, rest zero
    x[0, 257] = 0x8001
    x[1] = W.f32_to_bf16_bits(np.linspace(-1e-38, 1e-38, H).astype(np.float32))
    x[2] = W.f32_to_bf16_bits(np.linspace(-3e4, 3e4, H).astype(np.float32))
    idx = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    case = G.Case(3, H, 2, 2, 4, 1, x, idx, np.ones((3, 2), np.float32))
    case.check_dispatch_fp8(full=True)
    case.check_fused(fp8=True, full=True)


def test_combine_identity_law_on_gpu():
    """y := the GPU's own bf16 dispatch output, unit weights: out = bf16(n_kept * x), checked
    against the oracle (bit-exact) and, for tokens with all K pairs kept, against 8x."""
    cfg = W.get_config("decode_bf16")
    case = G.Case.from_config(cfg)
    recv = torch.full((cfg.E, cfg.C, cfg.H), G.BF16_NAN, dtype=torch.int16, device="cuda")
    B.ep_dispatch(case.x_d, case.idx_d, case.g["slot"], recv, cfg.C)
    ones = torch.ones((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    out = B.ep_combine(recv, case.idx_d, case.g["slot"], ones, cfg.C)
    torch.cuda.synchronize()
    want = W.f32_to_bf16_bits(8.0 * W.bf16_bits_to_f32(case.x))
    assert np.array_equal(G.to_np(out).view(np.uint16), want)


def test_combine_dropped_pairs_leave_signed_zero_and_inf():
    """A pair that is not kept must leave the running sum exactly as it is, -0 and +-Inf
    included (the oracle skips it). Token 1's only kept product underflows to -0 and a dropped
    pair follows; token 0 sums +Inf and a finite row, then a dropped pair; token 2 has an
    invalid and an unrouted id around a kept pair that gives -0 again; token 3 has nothing
    kept (+0). Every output row is compared bit for bit with the oracle."""
    print("[parity] combine: dropped pairs after -0 and Inf sums", flush=True)
    T, H, E, K, C = 4, 256, 4, 3, 1
    idx = np.array([[0, 1, 1], [2, 1, 0], [-1, 3, 7], [1, 2, 0]], dtype=np.int32)
    lay = oracle.layout(idx, E, C, 1)
    slot = lay["slot"]
    # kept: (0,0) e0 s0, (0,1) e1 s0, (1,0) e2 s0, (2,1) e3 s0; every other pair dropped or
    # not routed
    assert [tuple(p) for p in np.argwhere(slot >= 0)] == [(0, 0), (0, 1), (1, 0), (2, 1)]
    f = np.zeros((E, C, H), dtype=np.float32)
    f[0, 0] = np.inf
    f[1, 0] = 1.0
    f[2, 0] = -1.0e-20
    f[3, 0] = 2.0e-20
    y = W.f32_to_bf16_bits(f)
    w = np.full((T, K), 1.0, dtype=np.float32)
    w[1, 0] = 1.0e-30          # -1e-50 underflows: fmaf gives -0
    w[2, 1] = -1.0e-30         # -2e-50: -0 again
    want = oracle.combine(y, idx, slot, w)
    assert (want[1] == 0x8000).all() and (want[2] == 0x8000).all()
    assert (want[0] == 0x7F80).all() and (want[3] == 0x0000).all()
    y_d = torch.from_numpy(y.view(np.int16)).to(G.dev())
    out = B.ep_combine(y_d, G.to_dev(idx), G.to_dev(slot), G.to_dev(w), C)
    torch.cuda.synchronize()
    assert np.array_equal(G.to_np(out).view(np.uint16), want)


def test_deterministic_repeat():
    cfg = W.get_config("skew_zipf_c256")
    case = G.Case.from_config(cfg)
    y_host, y = case.make_y()
    outs = []
    for _ in range(3):
        g = B.ep_layout(case.idx_d, cfg.E, cfg.C, cfg.R)
        outs.append(G.to_np(B.ep_combine(y, case.idx_d, g["slot"], case.w_d, cfg.C)).copy())
        assert np.array_equal(G.to_np(g["slot"]), case.lay["slot"])
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_concurrent_streams_on_separate_buffers():
    """The library is stateless: two streams, each running fused layout + dispatch and combine
    on its own batch and buffers with no synchronisation between them, give each batch's
    oracle result."""
    print("[parity] two concurrent streams", flush=True)
    cases = [G.Case.random(700, 512, 32, 4, 60, 4, seed=s) for s in (21, 22)]
    work = []
    for c in cases:
        y_host, y = c.make_y()
        recv = torch.full((c.E, c.C, c.H), G.SENTINEL16, dtype=torch.int16, device=G.dev())
        work.append((c, y_host, y, recv, torch.cuda.Stream()))
    torch.cuda.synchronize()
    results = []
    for rep in range(3):
        outs = []
        for c, y_host, y, recv, st in work:
            with torch.cuda.stream(st):
                lay = B.ep_layout_dispatch(c.x_d, c.idx_d, recv, c.E, c.C, c.R)
                outs.append((lay, B.ep_combine(y, c.idx_d, lay["slot"], c.w_d, c.C)))
        torch.cuda.synchronize()
        results.append(outs)
    for outs in results:
        for (c, y_host, y, recv, st), (lay, out) in zip(work, outs):
            assert np.array_equal(G.to_np(lay["slot"]), c.lay["slot"])
            want = oracle.combine(y_host, c.idx, c.lay["slot"], c.w)
            assert np.array_equal(G.to_np(out).view(np.uint16), want)
            d = np.full((c.E, c.C, c.H), G.SENTINEL16, dtype=np.uint16)
            oracle.dispatch(c.x, c.idx, c.lay["slot"], c.E, c.C, d)
            assert np.array_equal(G.to_np(recv).view(np.uint16), d)


def test_non_default_stream():
    cfg = W.get_config("decode_bf16")
    case = G.Case.from_config(cfg)
    y_host, y = case.make_y()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = B.ep_layout(case.idx_d, cfg.E, cfg.C, cfg.R)
        out = B.ep_combine(y, case.idx_d, g["slot"], case.w_d, cfg.C)
    s.synchronize()
    want = oracle.combine(y_host, case.idx, case.lay["slot"], case.w)
    assert np.array_equal(G.to_np(out).view(np.uint16), want)


def _non_finite_x(T, H, seed):
    """Token rows with NaN (both signs, with payloads) and +-inf planted in some 128-channel
    blocks: blocks with a NaN, blocks with infinities only, blocks with both, and clean blocks
    around them."""
    rng = np.random.default_rng(seed)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    nb = H // 128
    for t in range(0, T, 3):
        b = int(rng.integers(0, nb))
        kind = t % 4
        h = 128 * b + rng.integers(0, 128, size=3)
        if kind == 0:
            x[t, h[0]] = 0xFFC5                      # -NaN with a payload
        elif kind == 1:
            x[t, h[0]] = 0x7F80
            x[t, h[1]] = 0xFF80                      # +inf and -inf, no NaN
        elif kind == 2:
            x[t, h[0]] = 0x7F80
            x[t, h[1]] = 0x7FC1                      # inf and NaN together: the NaN rule
        else:
            x[t, 128 * b:128 * b + 128] = 0x7FC0     # a whole block of NaN
    return x


def test_fp8_non_finite_blocks():
    """The NaN/inf policy (NaN propagates into the block's amax, a NaN amax gives the quiet NaN
    scale, every code keeps x's sign, a NaN quotient encodes as sign | 0x7F) on every FP8
    path: the one-stage dispatch, the fused layout + dispatch, the two-stage staging copy (and
    its fused form) with the expansion, and the packed dispatch, against the oracle."""
    print("[parity] FP8 non-finite blocks", flush=True)
    T, H, E, K, C, R = 97, 1024, 12, 4, 40, 3
    x = _non_finite_x(T, H, seed=41)
    rng = np.random.default_rng(42)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    case = G.Case(T, H, E, K, C, R, x, idx, w)
    case.check_dispatch_fp8(full=True)
    case.check_fused(fp8=True, full=True)
    import test_gpu_two_stage as TS
    ts = TS.TwoStage(T, H, E, K, C, R, idx, x, w, 0)
    ts.dispatch_fp8_full()
    import test_gpu_packed as PK
    PK.run_case(idx, x, w, E, C, R, 16, fp8=True, seed=3)
    # the policy really is exercised: NaN scales and NaN codes of both signs were produced
    q = np.zeros((E, C, H), np.uint8)
    sc = np.zeros((E, C, H // 128), np.float32)
    oracle.dispatch_fp8(x, idx, case.lay["slot"], E, C, q, sc)
    assert (sc.view(np.uint32) == 0x7FC00000).any() and (sc == np.inf).any()
    assert (q == 0x7F).any() and (q == 0xFF).any()


def test_combine_nan_and_inf_rows():
    """Kept expert rows holding NaN (both signs, payloads) and +-inf: every output element
    whose fp32 sum is NaN is the quiet NaN 0x7FC0, the rest as the oracle computes them, bit
    for bit; also through the two-stage partial combine and reduce."""
    print("[parity] combine with NaN/inf rows", flush=True)
    T, H, E, K, C, R = 200, 512, 16, 4, 60, 4
    case = G.Case.random(T, H, E, K, C, R, seed=43, lo=0, hi=E)
    y_host, _ = case.make_y()
    rng = np.random.default_rng(44)
    i, s = G.kept_pairs(case.lay)
    e = case.idx.reshape(-1)[i]
    for k in rng.choice(len(i), size=60, replace=False):
        h = rng.integers(0, H, size=2)
        y_host[e[k], s[k], h[0]] = rng.choice([0x7FC0, 0xFFC0, 0x7FA3, 0x7F80, 0xFF80])
        y_host[e[k], s[k], h[1]] = rng.choice([0x7F80, 0xFF80])
    y = G.u16_dev(y_host)
    out = B.ep_combine(y, case.idx_d, case.g["slot"], case.w_d, C)
    torch.cuda.synchronize()
    want = oracle.combine(y_host, case.idx, case.lay["slot"], case.w)
    got = G.to_np(out).view(np.uint16)
    assert (want == 0x7FC0).sum() > 20 and ((want & 0x7FFF) == 0x7F80).any()
    assert np.array_equal(got, want)
    rl = B.ep_rank_layout(case.idx_d, E, R)
    part = B.ep_combine_ranks(y, case.idx_d, case.g["slot"], rl["rank_slot"], case.w_d, C)
    out2 = B.ep_combine_reduce(part, rl["rank_slot"], K)
    torch.cuda.synchronize()
    orl = oracle.rank_layout(case.idx, E, R)
    wp = oracle.combine_ranks(y_host, case.idx, case.lay["slot"], orl["rank_slot"], case.w)
    sent = orl["rank_slot"] >= 0
    t_i, r_i = np.nonzero(sent)
    p_i = orl["rank_slot"][t_i, r_i]
    assert np.array_equal(G.to_np(part).view(np.uint16)[r_i, p_i], wp[r_i, p_i])
    assert np.array_equal(G.to_np(out2).view(np.uint16),
                          oracle.combine_reduce(wp, orl["rank_slot"]))


# the layout with a workspace (chunk histograms of 4096 pairs): shapes whose tiles start in
# every position of a chunk, tiles that straddle chunk boundaries (K = 6, 5), a batch that is
# one chunk exactly or one pair more, a ragged last vector (T*K % 4 != 0), E at its maximum
# (E + 2 = 1026 bins: more bins than lanes), drops, unrouted and invalid ids
WS_SMALL = [
    # T, H, E, K, C, R
    (512, 128, 16, 8, 300, 4),        # T*K = 4096: one chunk
    (513, 128, 16, 8, 300, 4),        # 4104: a second chunk of 8 pairs
    (1367, 256, 64, 6, 90, 8),        # 8202: K = 6, tiles of 8 tokens cross chunk boundaries
    (2459, 128, 32, 5, 500, 4),       # 12295: K = 5, T*K % 4 = 3
    (3000, 256, 1024, 8, 40, 8),      # E = 1024: 1026 bins
    (4099, 256, 16, 4, 1100, 4),      # ragged last tile
    (9000, 128, 128, 8, 700, 16),     # 72000 pairs, 18 chunks, drops
]


@pytest.mark.parametrize("T,H,E,K,C,R", WS_SMALL)
def test_layout_dispatch_with_workspace(T, H, E, K, C, R):
    print(f"[parity] layout+dispatch with workspace T={T} H={H} E={E} K={K} C={C} R={R}",
          flush=True)
    case = G.Case.random(T, H, E, K, C, R, seed=T + K)
    case.check_fused(fp8=False, full=True, ws=True)
    if H % 128 == 0:
        case.check_fused(fp8=True, full=True, ws=True)


@pytest.mark.parametrize("name", ["decode_fp8", "skew_zipf_c256", "prefill_bf16", "prefill_fp8"])
def test_config_layout_dispatch_with_workspace(name):
    """The workspace form on the full workloads, both dispatch dtypes, with a workspace that
    holds stale data (the call must not depend on its contents)."""
    cfg = W.get_config(name)
    print(f"[parity] workspace form {name}", flush=True)
    case = G.Case.from_config(cfg)
    n = B.layout_workspace_bytes(cfg.T, cfg.K, cfg.E)
    stale = torch.full((n,), 0x5A, dtype=torch.uint8, device=G.dev())
    case.check_fused(fp8=False, full=False, ws=True, workspace=stale)
    stale.fill_(0xC3)
    case.check_fused(fp8=True, full=False, ws=True, workspace=stale)


def test_layout_dispatch_with_workspace_many_pairs():
    """2^17 pairs (32 chunks), E at its maximum, drops: the chunk sums over many chunks."""
    cfg = W.EpConfig("max_e_ws", T=16384, H=128, E=B.EP_MAX_EXPERTS, K=8, C=100, R=8)
    inp = W.make_inputs(cfg)
    case = G.Case(cfg.T, cfg.H, cfg.E, cfg.K, cfg.C, cfg.R, inp["x"], inp["topk_idx"],
                  inp["topk_w"])
    assert case.lay["stats"]["dropped"] > 0
    case.check_fused(fp8=False, full=False, ws=True)
    case.check_fused(fp8=True, full=False, ws=True)


def test_layout_dispatch_with_workspace_empty():
    E, C, R, H = 16, 4, 4, 256
    idx = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    x = torch.zeros((0, H), dtype=torch.int16, device="cuda")
    recv = torch.full((E, C, H), G.SENTINEL16, dtype=torch.int16, device="cuda")
    g = B.ep_layout_dispatch_ws(x, idx, recv, E, C, R, workspace=torch.empty(0, dtype=torch.uint8,
                                                                              device="cuda"),
                                expert_count=torch.full((E,), 7, dtype=torch.int32, device="cuda"))
    q = torch.full((E, C, H), G.SENTINEL8, dtype=torch.uint8, device="cuda")
    sc = torch.full((E, C, H // 128), G.SENTINEL_F32, dtype=torch.float32, device="cuda")
    g8 = B.ep_layout_dispatch_fp8_ws(x, idx, q, sc, E, C, R)
    torch.cuda.synchronize()
    assert G.to_np(g["expert_count"]).tolist() == [0] * E
    assert G.to_np(g["stats"]).tolist() == [0, 0, 0, 0] == G.to_np(g8["stats"]).tolist()
    assert int((recv != G.SENTINEL16).sum()) == 0 and int((q != G.SENTINEL8).sum()) == 0
