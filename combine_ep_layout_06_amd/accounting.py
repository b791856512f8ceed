"""Byte accounting for one dispatch + combine.

Two numerators are used:

* **Logical payload** (awsome-distributed-ai PR #1238, "What changed": one useful-payload
  definition for every backend; review item 1 prints its values). Every selected
  (token, expert) assignment moves one dispatch row and one combine row. A bf16 dispatch row
  is 2*H bytes; an FP8 dispatch row is H bytes of e4m3 plus one fp32 scale per 128 channels;
  the combine row is bf16 (2*H) in either case. Throughput = payload / elapsed.

* **Algorithmic HBM bytes**: what the kernels must read and write at minimum with no padding
  and no re-reads: the route and slots, each token row read once, each kept row written once
  by dispatch and read once by combine, each output row written once. This is the numerator of
  the roofline fraction against the HBM peak.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12   # MI355X HBM3E, published peak


def logical_payload_bytes(T: int, K: int, H: int, fp8: bool) -> int:
    """Useful payload per rank for one dispatch + combine of T tokens with top-K routing."""
    if fp8:
        return T * K * (H + 4 * (H // 128)) + 2 * T * K * H
    return 4 * T * K * H


def layout_bytes(T: int, K: int) -> int:
    """Layout: read topk_idx, write slot (int32 each). Counts and offsets are O(E)."""
    return 8 * T * K


def dispatch_bytes(T: int, K: int, H: int, n_kept: int, fp8: bool) -> int:
    """Dispatch: read x once, read idx and slot, write one row (and a scale row) per kept pair."""
    route = 8 * T * K
    if fp8:
        return 2 * T * H + H * n_kept + 4 * (H // 128) * n_kept + route
    return 2 * T * H + 2 * H * n_kept + route


def combine_bytes(T: int, K: int, H: int, n_kept: int) -> int:
    """Combine: read each kept y row once, read idx, slot and weights, write out once."""
    return 2 * H * n_kept + 12 * T * K + 2 * T * H


def step_bytes(T: int, K: int, H: int, n_kept: int, fp8: bool) -> int:
    """Algorithmic HBM bytes of layout + dispatch + combine."""
    return (layout_bytes(T, K) + dispatch_bytes(T, K, H, n_kept, fp8)
            + combine_bytes(T, K, H, n_kept))


# ------------------------------------------------------------------------------------------
# two-stage, rank-deduplicated path: N_tr = sum over ranks of the tokens sent there (one staging
# row and one partial row each), N_kept = kept pairs
# ------------------------------------------------------------------------------------------

def rank_layout_bytes(T: int, K: int, R: int) -> int:
    """Rank layout: read topk_idx, write rank_slot [T, R]."""
    return 4 * T * K + 4 * T * R


def dispatch_ranks_bytes(T: int, R: int, H: int, n_tr: int, fp8: bool) -> int:
    """Stage 1: read x once and rank_slot, write one staging row (and scale row) per (token,
    rank)."""
    row = H + 4 * (H // 128) if fp8 else 2 * H
    return 2 * T * H + row * n_tr + 4 * T * R


def dispatch_expand_bytes(T: int, K: int, R: int, H: int, n_tr: int, n_kept: int,
                          fp8: bool) -> int:
    """Stage 2: read each staging row once, write one row per kept pair; idx, slot, rank_slot."""
    row = H + 4 * (H // 128) if fp8 else 2 * H
    return row * (n_tr + n_kept) + 8 * T * K + 4 * T * R


def combine_ranks_bytes(T: int, K: int, R: int, H: int, n_tr: int, n_kept: int) -> int:
    """Stage 1 of combine: read each kept y row, write one partial row per (token, rank)."""
    return 2 * H * (n_kept + n_tr) + 12 * T * K + 4 * T * R


def combine_reduce_bytes(T: int, R: int, H: int, n_tr: int) -> int:
    """Stage 2 of combine: read each partial row once, write out once."""
    return 2 * H * n_tr + 2 * T * H + 4 * T * R

