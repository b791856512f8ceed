"""Seeded synthetic workloads for one GPU's share of MoE expert-parallel dispatch/combine.

This module only draws inputs. It holds none of the method's arithmetic: no histogram, no
slot assignment, no quantiser, no reduction. The tests, the benchmark and the oracle all take
their inputs from here, so that every side sees the same bytes.

Shapes follow the afdEP-comm validation record (its ``setup`` key: hidden 2048, top-k 8 of 128
experts, 96 experts for the 1A:3F split, capacity 2048) and the Decode-like (128 tokens per rank)
and Prefill-like (4,096 tokens per rank) profiles of awsome-distributed-ai PR #1238 ("What
changed"). The pages use synthetic routes themselves (a deterministic route; ``--routing
random``), so nothing public is being stood in for.

Draw order for one config and seed, from ``numpy.random.default_rng(seed)``:

1. ``x``: fp32 N(0, 1), shape [T, H]. With ``outliers`` set, a Bernoulli(0.01) mask is drawn
   next and the masked elements are multiplied by 50. Then rounded to bf16 (RNE).
2. The route ``topk_idx`` [T, K] (int32), by the config's routing rule.
3. Logits N(0, 1) [T, K]; weights = softmax over the K selected logits, computed in fp64,
   stored as fp32.

Expert outputs ``y`` come from a second generator, ``default_rng([seed, 1])``, as a stream of
bf16 rows (``y_rows``); the caller decides where in ``[E][C][H]`` each row goes.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

__all__ = ["EpConfig", "CONFIGS", "get_config", "make_inputs", "y_rows", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "BF16_NAN", "fingerprint", "balanced_route"]

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class EpConfig:
    """One workload: T tokens of hidden size H routed top-K over E experts with capacity C.

    The E experts are laid out as R virtual ranks of E/R experts each (rank-major).
    ``route`` is one of ``uniform`` (K distinct experts per token, uniformly at random),
    ``zipf`` (K distinct experts sampled without replacement from a Zipf(s) law over a seeded
    expert permutation), ``balanced`` (the closed-form stride route; see ``balanced_route``) or
    ``unbalanced`` (K distinct experts without replacement, where a seeded eighth of the experts
    is ``unbalanced_ratio`` times as likely as the others).
    ``fp8`` selects the FP8 dispatch for the benchmark step; combine is bf16 in every config.
    """
    name: str
    T: int
    H: int
    E: int
    K: int
    C: int
    R: int
    route: str = "uniform"
    fp8: bool = False
    outliers: bool = False
    zipf_s: float = 1.2
    unbalanced_ratio: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def EL(self) -> int:
        return self.E // self.R

    def shape(self) -> dict:
        return dict(T=self.T, H=self.H, E=self.E, K=self.K, C=self.C, R=self.R)


# The five workloads. Decode-like: 128 tokens; Prefill-like: 4,096 tokens (PR #1238, "What
# changed"). Hidden 2048, top-8 of 128 experts, 96 experts for the 1A:3F split (afdEP-comm
# validation record, ``setup``).
CONFIGS: dict[str, EpConfig] = {c.name: c for c in [
    EpConfig("decode_bf16", T=128, H=2048, E=128, K=8, C=2048, R=16,
             note="Decode-like, bf16 dispatch + combine"),
    EpConfig("decode_fp8", T=128, H=2048, E=128, K=8, C=2048, R=16, fp8=True, outliers=True,
             note="Decode-like, FP8 e4m3 dispatch with per-128-channel scales, 1% x50 outliers"),
    EpConfig("skew_zipf", T=2048, H=2048, E=128, K=8, C=2048, R=16, route="zipf",
             note="Zipf(1.2) routing; with K distinct experts per token no expert can exceed T=C"),
    EpConfig("skew_zipf_c1024", T=2048, H=2048, E=128, K=8, C=1024, R=16, route="zipf",
             note="Zipf(1.2) routing with capacity 1024: hot experts drop in token order"),
    EpConfig("skew_zipf_c256", T=2048, H=2048, E=128, K=8, C=256, R=16, route="zipf",
             note="Zipf(1.2) routing with capacity 256: many experts drop in token order"),
    EpConfig("prefill_bf16", T=4096, H=2048, E=128, K=8, C=4096, R=16,
             note="Prefill-like, bf16 dispatch + combine, 16 virtual ranks x 8 experts"),
    EpConfig("prefill_fp8", T=4096, H=2048, E=96, K=8, C=4096, R=3, fp8=True,
             note="Prefill-like FP8 dispatch on 96 experts, 3 virtual ranks x 32 experts"),
    EpConfig("balanced_stride", T=1024, H=2048, E=128, K=8, C=4096, R=16, route="balanced",
             note="Closed-form stride route: every expert receives exactly T*K/E pairs"),
    # The second family: the pages' balanced stride route above and a skew with a named
    # unbalanced ratio (the benchmark's --unbalanced-ratio axis, which the pages name but did not
    # run). A seeded 16 of the 128 experts are 4 times as likely as the rest.
    EpConfig("unbalanced_r4", T=4096, H=2048, E=128, K=8, C=4096, R=16, route="unbalanced",
             unbalanced_ratio=4.0,
             note="Prefill-like, hot eighth of the experts 4x as likely; no drops (C = T)"),
    EpConfig("unbalanced_r4_c512", T=4096, H=2048, E=128, K=8, C=512, R=16,
             route="unbalanced", unbalanced_ratio=4.0,
             note="The same with capacity 512: the hot experts drop in token order"),
]}


def get_config(name: str) -> EpConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def balanced_route(T: int, K: int, E: int, seed: int = 0) -> np.ndarray:
    """The stride route of PR #1238's review (item 9): expert = (17 t + 31 j + seed) mod E.

    31 is odd, so for E a power of two the K experts of one token are distinct whenever K <= E;
    17 is odd too, so over any E consecutive tokens each expert is hit once per j. With T a
    multiple of E every expert therefore receives exactly T*K/E pairs.
    """
    t = np.arange(T, dtype=np.int64)[:, None]
    j = np.arange(K, dtype=np.int64)[None, :]
    return ((t * 17 + j * 31 + seed) % E).astype(np.int32)


def _route(cfg: EpConfig, rng: np.random.Generator) -> np.ndarray:
    T, E, K = cfg.T, cfg.E, cfg.K
    if cfg.route == "uniform":
        # K distinct experts per token, uniformly: the first K of a random permutation
        # (argsort of iid uniform keys), drawn independently per token.
        keys = rng.random((T, E))
        return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    if cfg.route == "zipf":
        # p[perm[r]] proportional to (r + 1)^-s over a seeded expert permutation; K distinct
        # experts per token by successive sampling without replacement, drawn with the
        # Gumbel-top-K construction (equal in distribution to sequential draws).
        perm = rng.permutation(E)
        p = np.empty(E, dtype=np.float64)
        p[perm] = (np.arange(E, dtype=np.float64) + 1.0) ** (-cfg.zipf_s)
        p /= p.sum()
        g = rng.gumbel(size=(T, E))
        keys = np.log(p)[None, :] + g
        return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    if cfg.route == "balanced":
        return balanced_route(T, K, E, cfg.seed)
    if cfg.route == "unbalanced":
        # a seeded eighth of the experts (at least one) has weight `unbalanced_ratio`, the
        # rest weight 1; K distinct experts per token by the Gumbel-top-K construction
        perm = rng.permutation(E)
        p = np.ones(E, dtype=np.float64)
        p[perm[:max(1, E // 8)]] = cfg.unbalanced_ratio
        p /= p.sum()
        g = rng.gumbel(size=(T, E))
        keys = np.log(p)[None, :] + g
        return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    raise ValueError(f"unknown route {cfg.route!r}")


def make_inputs(cfg: EpConfig, seed: int | None = None) -> dict:
    """Draw (x, topk_idx, topk_w) for one workload. Returns numpy arrays:

    ``x`` uint16 [T, H] (bf16 bits), ``topk_idx`` int32 [T, K], ``topk_w`` float32 [T, K].
    """
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    T, H, K = cfg.T, cfg.H, cfg.K
    x = rng.standard_normal((T, H), dtype=np.float32)
    if cfg.outliers:
        mask = rng.random((T, H)) < 0.01
        x[mask] *= np.float32(50.0)
    x_bits = f32_to_bf16_bits(x)
    idx = _route(cfg, rng)
    logits = rng.standard_normal((T, K)).astype(np.float64)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return {"x": x_bits, "topk_idx": np.ascontiguousarray(idx, dtype=np.int32),
            "topk_w": np.ascontiguousarray(w, dtype=np.float32)}


def y_rows(n: int, H: int, seed: int = 0, *, start: int = 0) -> np.ndarray:
    """Rows ``start .. start+n-1`` of the expert-output stream: bf16 bits [n, H], N(0, 1).

    The stream is drawn from ``default_rng([seed, 1])`` in row order; asking for a later
    window draws (and discards) the rows before it so a window never depends on how the
    stream was split.
    """
    rng = np.random.default_rng([seed, 1])
    if start:
        rng.standard_normal((start, H), dtype=np.float32)
    return f32_to_bf16_bits(rng.standard_normal((n, H), dtype=np.float32))


def fingerprint(*arrays: np.ndarray, cfg: EpConfig | None = None) -> str:
    """SHA-256 over the config and the raw bytes of the given arrays (provenance record)."""
    h = hashlib.sha256()
    if cfg is not None:
        h.update(repr(dataclasses.astuple(cfg)).encode())
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()
