"""Workers of the exhaustive number-format sweeps (tests/test_oracle_formats_exhaustive.py).

Each call checks one chunk of the 2^32 fp32 bit patterns and returns the number of patterns
where the oracle's encoder disagrees with its reference, plus the first such pattern. The
references are library routines and closed forms, never the oracle:

* bf16: torch's CPU float32 -> bfloat16 cast (round to nearest even) for every non-NaN
  pattern; every NaN must give the quiet NaN 0x7FC0 (the oracle's NaN rule; torch writes its
  own NaN pattern).
* OCP E4M3: torch's CPU float32 -> float8_e4m3fn cast (round to nearest even) for every
  |v| < 464, the range where its overflow handling plays no part; |v| >= 464 (infinities
  included) saturates to sign | 0x7E; NaN gives sign | 0x7F.
"""
from __future__ import annotations

import numpy as np


def _patterns(start: int, n: int) -> np.ndarray:
    return np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)


def check_bf16_chunk(start: int, n: int):
    import torch
    import oracle
    torch.set_num_threads(1)
    bits = _patterns(start, n)
    v = bits.view(np.float32)
    got = oracle.bf16_rne(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    want = np.where(nan, np.uint16(0x7FC0), want)
    bad = np.nonzero(got != want)[0]
    return int(bad.size), (int(bits[bad[0]]) if bad.size else None)


def check_e4m3_chunk(start: int, n: int):
    import torch
    import oracle
    torch.set_num_threads(1)
    bits = _patterns(start, n)
    v = bits.view(np.float32)
    got = oracle.e4m3_rne_sat(v)
    sign = ((bits >> 24) & 0x80).astype(np.uint8)
    nan = np.isnan(v)
    a = np.abs(v)
    small = ~nan & (a < 464.0)
    safe = np.where(small, v, np.float32(0))
    want = torch.from_numpy(safe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    want = np.where(small, want, np.where(nan, sign | 0x7F, sign | 0x7E)).astype(np.uint8)
    bad = np.nonzero(got != want)[0]
    return int(bad.size), (int(bits[bad[0]]) if bad.size else None)
