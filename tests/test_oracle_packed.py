"""Pins for the oracle's packed, aligned receive layout and for the unbalanced route (CPU only).

The pages pin the expert alignment to 1 in their runs (DeepEP-V2 on AWS EFA, the
test_ep.py cross-check: expert_alignment=1) and note that the route generator is perfectly
balanced while the benchmark also has an --unbalanced-ratio axis they did not run. Readings:
with alignment A each expert's kept count is rounded up to a multiple of A, offsets are the
exclusive scan of those, pair (t, j) lands at row offset[e] + slot of a packed [rows][H] buffer,
and padding rows are left untouched; an unbalanced ratio rho makes a seeded eighth of the
experts rho times as likely as the others.

Pins: the offsets' defining property (each padded count is the one multiple of A in
[count, count + A)) and their equality with the pinned layout offsets at A = 1; the packed
dispatch equal to a gather of the pinned one-stage dispatch (bf16 and FP8) with padding rows
untouched; the packed combine over gathered expert outputs equal to the pinned one-stage
combine; truncated buffers drop exactly the pairs past their end.
"""
import numpy as np
import pytest

import oracle
from combine_ep_layout_06_amd import workloads as W

SENT16 = np.uint16(0xBEEF)


def small(T, H, E, K, C, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-2, E + 1, size=(T, K)).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.random((T, K)).astype(np.float32)
    return idx, x, w


@pytest.mark.parametrize("align", [1, 2, 7, 16, 128])
def test_packed_offsets_definition(align):
    rng = np.random.default_rng(align)
    count = rng.integers(0, 300, size=97).astype(np.int32)
    count[::11] = 0
    off = oracle.packed_offsets(count, align)
    d = np.diff(off)
    assert off[0] == 0 and (d >= 0).all()
    assert (d % align == 0).all() and (d >= count).all() and (d < count + align).all()
    assert off[-1] == d.sum()


@pytest.mark.parametrize("name", ["decode_bf16", "skew_zipf_c256", "unbalanced_r4_c512"])
def test_packed_offsets_at_alignment_one_are_the_layout_offsets(name):
    cfg = W.get_config(name)
    lay = oracle.layout(W.make_inputs(cfg)["topk_idx"], cfg.E, cfg.C, cfg.R)
    off = oracle.packed_offsets(lay["count"], 1)
    assert np.array_equal(off[:-1], lay["offset"]) and off[-1] == lay["stats"]["kept"]


CASES = [(37, 64, 6, 3, 5, 1), (100, 128, 16, 4, 9, 2), (64, 256, 8, 8, 40, 3)]


def gathered_rows(idx, slot, off, E, C):
    """(e, s, packed row) of every kept pair."""
    e = idx.reshape(-1)
    s = slot.reshape(-1)
    keep = (e >= 0) & (e < E) & (s >= 0) & (s < C)
    return e[keep], s[keep], off[e[keep]] + s[keep]


@pytest.mark.parametrize("T,H,E,K,C,seed", CASES)
@pytest.mark.parametrize("align", [1, 16])
def test_packed_dispatch_is_a_gather_of_the_padded_one(T, H, E, K, C, seed, align):
    idx, x, _ = small(T, H, E, K, C, seed)
    lay = oracle.layout(idx, E, C, 1)
    off = oracle.packed_offsets(lay["count"], align)
    padded = np.full((E, C, H), SENT16, np.uint16)
    oracle.dispatch(x, idx, lay["slot"], E, C, padded)
    packed = np.full((off[-1] + 3, H), SENT16, np.uint16)
    oracle.dispatch_packed(x, idx, lay["slot"], off, E, C, packed)
    e, s, r = gathered_rows(idx, lay["slot"], off, E, C)
    assert np.array_equal(packed[r], padded[e, s])
    other = np.ones(packed.shape[0], bool)
    other[r] = False
    assert (packed[other] == SENT16).all()


@pytest.mark.parametrize("T,H,E,K,C,seed", [(37, 128, 6, 3, 5, 1), (64, 256, 8, 8, 40, 3)])
def test_packed_fp8_dispatch_is_a_gather_of_the_padded_one(T, H, E, K, C, seed):
    idx, x, _ = small(T, H, E, K, C, seed)
    NB = H // 128
    lay = oracle.layout(idx, E, C, 1)
    off = oracle.packed_offsets(lay["count"], 8)
    pq = np.full((E, C, H), 0xA5, np.uint8)
    ps = np.full((E, C, NB), -3.0, np.float32)
    oracle.dispatch_fp8(x, idx, lay["slot"], E, C, pq, ps)
    q = np.full((off[-1], H), 0xA5, np.uint8)
    sc = np.full((off[-1], NB), -3.0, np.float32)
    oracle.dispatch_packed_fp8(x, idx, lay["slot"], off, E, C, q, sc)
    e, s, r = gathered_rows(idx, lay["slot"], off, E, C)
    assert np.array_equal(q[r], pq[e, s])
    assert np.array_equal(sc[r].view(np.uint32), ps[e, s].view(np.uint32))


@pytest.mark.parametrize("T,H,E,K,C,seed", CASES)
@pytest.mark.parametrize("align", [1, 128])
def test_packed_combine_is_the_padded_combine(T, H, E, K, C, seed, align):
    idx, _, w = small(T, H, E, K, C, seed)
    lay = oracle.layout(idx, E, C, 1)
    off = oracle.packed_offsets(lay["count"], align)
    rng = np.random.default_rng(seed + 7)
    y = W.f32_to_bf16_bits(rng.standard_normal((E, C, H), dtype=np.float32))
    yp = np.full((off[-1], H), W.BF16_NAN, np.uint16)        # padding rows: NaN, never read
    e, s, r = gathered_rows(idx, lay["slot"], off, E, C)
    yp[r] = y[e, s]
    got = oracle.combine_packed(yp, idx, lay["slot"], off, w, E, C)
    assert np.array_equal(got, oracle.combine(y, idx, lay["slot"], w))


def test_truncated_packed_buffer_drops_the_pairs_past_its_end():
    T, H, E, K, C = 50, 32, 4, 3, 40
    idx, x, w = small(T, H, E, K, C, 11)
    lay = oracle.layout(idx, E, C, 1)
    off = oracle.packed_offsets(lay["count"], 4)
    rows = int(off[-1]) - 9
    packed = np.full((rows, H), SENT16, np.uint16)
    oracle.dispatch_packed(x, idx, lay["slot"], off, E, C, packed)
    full = np.full((off[-1], H), SENT16, np.uint16)
    oracle.dispatch_packed(x, idx, lay["slot"], off, E, C, full)
    assert np.array_equal(packed, full[:rows])
    # combine: a pair past the end counts as dropped
    slot = lay["slot"].copy()
    past = (idx >= 0) & (idx < E) & (slot >= 0) & (off[np.clip(idx, 0, E - 1)] + slot >= rows)
    assert past.any()
    slot[past] = -1
    yp = W.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((off[-1], H), dtype=np.float32))
    got = oracle.combine_packed(yp[:rows].copy(), idx, lay["slot"], off, w, E, C)
    assert np.array_equal(got, oracle.combine_packed(yp, idx, slot, off, w, E, C))


@pytest.mark.parametrize("name", ["unbalanced_r4", "unbalanced_r4_c512"])
def test_unbalanced_route(name):
    """K distinct valid experts per token; the seeded hot eighth carries about rho times the
    load of the rest (sampling without replacement compresses it a little: ~3.8 for rho = 4,
    K = 8 of 128)."""
    cfg = W.get_config(name)
    idx = W.make_inputs(cfg)["topk_idx"]
    assert idx.min() >= 0 and idx.max() < cfg.E
    srt = np.sort(idx, axis=1)
    assert not (srt[:, 1:] == srt[:, :-1]).any()
    load = np.bincount(idx.ravel(), minlength=cfg.E)
    hot = np.argsort(-load)[:cfg.E // 8]
    cold = np.setdiff1d(np.arange(cfg.E), hot)
    ratio = load[hot].mean() / load[cold].mean()
    assert 3.0 < ratio < 4.5, ratio
    lay = oracle.layout(idx, cfg.E, cfg.C, cfg.R)
    assert (lay["stats"]["dropped"] > 0) == (cfg.C < load.max())
