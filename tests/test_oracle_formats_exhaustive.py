"""The oracle's two number formats over every one of the 2^32 fp32 bit patterns (CPU only).

oracle_bf16_rne against torch's float32 -> bfloat16 cast (NaN: the quiet NaN 0x7FC0), and
oracle_e4m3_rne_sat against torch's float32 -> float8_e4m3fn cast below 464 with the closed
forms of saturation and NaN above it (the OCP 8-bit floating point specification, E4M3 with
saturating conversion). The sweep runs in a pool of worker processes, about a minute on eight
cores; the workers are in tests/exhaustive_formats.py.
"""
import multiprocessing as mp
import os

import pytest

CHUNK = 1 << 24
STARTS = range(0, 1 << 32, CHUNK)


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _sweep(fn_name):
    import exhaustive_formats as X
    fn = getattr(X, fn_name)
    ctx = mp.get_context("spawn")
    with ctx.Pool(_workers()) as pool:
        res = pool.starmap(fn, [(s, CHUNK) for s in STARTS])
    nbad = sum(r[0] for r in res)
    first = next((r[1] for r in res if r[1] is not None), None)
    return nbad, first


def test_bf16_rne_every_fp32_pattern():
    nbad, first = _sweep("check_bf16_chunk")
    assert nbad == 0, f"{nbad} patterns differ, first 0x{first:08x}"


def test_e4m3_rne_sat_every_fp32_pattern():
    nbad, first = _sweep("check_e4m3_chunk")
    assert nbad == 0, f"{nbad} patterns differ, first 0x{first:08x}"
