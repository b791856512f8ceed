"""CPU oracle for MoE expert-parallel layout, dispatch (bf16 and FP8 e4m3) and combine.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``ep_oracle.c`` (plain single-threaded C, built
with gcc by ``oracle/build.py``) with numpy arrays. It shares nothing with the GPU library.

Every function here is pinned by the ``-m "not gpu"`` tests against something other than
itself: brute-force enumeration and a stable sort for the layout, a numpy scatter for the
dispatch, torch's CPU casts and an exhaustive table search for the number formats, the
identity/one-hot laws and an fp64 bound for combine. The two-stage path is pinned by its
reductions to the pinned one-stage functions (one expert per rank, a single rank), by the
composed dispatch being the one-stage dispatch, and by closed forms (identity law, one expert
per rank).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# EP_ORACLE_LIB selects another build of ep_oracle.c (the sanitizer build of the tests)
_LIB_PATH = os.environ.get("EP_ORACLE_LIB") or os.path.join(_HERE, "liboracle_ep.so")
_lib = None

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_c_int, _c_long = ctypes.c_int, ctypes.c_long


def lib():
    """Load the oracle library, building it with gcc if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_rne_sat.argtypes = [ctypes.c_float]
        L.oracle_e4m3_rne_sat.restype = ctypes.c_uint8
        opt_i32p = ctypes.c_void_p
        L.oracle_layout.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, _i32p, _i32p,
                                    _i32p, _i32p, opt_i32p, opt_i32p, _i32p, opt_i32p]
        L.oracle_layout.restype = None
        L.oracle_dispatch.argtypes = [_c_int] * 5 + [_u16p, _i32p, _i32p, _u16p]
        L.oracle_dispatch.restype = None
        L.oracle_dispatch_fp8.argtypes = [_c_int] * 5 + [_u16p, _i32p, _i32p, _u8p, _f32p]
        L.oracle_dispatch_fp8.restype = None
        L.oracle_combine.argtypes = [_c_int] * 5 + [_u16p, _i32p, _i32p, _f32p, _u16p]
        L.oracle_combine.restype = None
        L.oracle_combine_tokens.argtypes = ([_c_int, _i32p] + [_c_int] * 4
                                            + [_u16p, _i32p, _i32p, _f32p, _u16p])
        L.oracle_combine_tokens.restype = None
        L.oracle_rank_layout.argtypes = [_c_int] * 4 + [_i32p, _i32p, _i32p]
        L.oracle_rank_layout.restype = None
        L.oracle_dispatch_ranks.argtypes = [_c_int] * 3 + [_u16p, _i32p, _u16p]
        L.oracle_dispatch_ranks.restype = None
        L.oracle_dispatch_ranks_fp8.argtypes = [_c_int] * 3 + [_u16p, _i32p, _u8p, _f32p]
        L.oracle_dispatch_ranks_fp8.restype = None
        L.oracle_dispatch_expand.argtypes = [_c_int] * 6 + [_u16p, _i32p, _i32p, _i32p, _u16p]
        L.oracle_dispatch_expand.restype = None
        L.oracle_dispatch_expand_fp8.argtypes = ([_c_int] * 6
                                                 + [_u8p, _f32p, _i32p, _i32p, _i32p, _u8p, _f32p])
        L.oracle_dispatch_expand_fp8.restype = None
        L.oracle_combine_ranks.argtypes = [_c_int] * 6 + [_u16p, _i32p, _i32p, _i32p, _f32p, _u16p]
        L.oracle_combine_ranks.restype = None
        L.oracle_combine_reduce.argtypes = [_c_int] * 3 + [_u16p, _i32p, _u16p]
        L.oracle_combine_reduce.restype = None
        L.oracle_combine_two_stage_tokens.argtypes = ([_c_int, _i32p] + [_c_int] * 5
                                                      + [_u16p, _i32p, _i32p, _i32p, _f32p, _u16p])
        L.oracle_combine_two_stage_tokens.restype = None
        L.oracle_packed_offsets.argtypes = [_c_int, _c_int, _i32p, _i32p]
        L.oracle_packed_offsets.restype = None
        L.oracle_dispatch_packed.argtypes = [_c_int] * 6 + [_u16p, _i32p, _i32p, _i32p, _u16p]
        L.oracle_dispatch_packed.restype = None
        L.oracle_dispatch_packed_fp8.argtypes = ([_c_int] * 6
                                                 + [_u16p, _i32p, _i32p, _i32p, _u8p, _f32p])
        L.oracle_dispatch_packed_fp8.restype = None
        L.oracle_combine_packed.argtypes = [_c_int] * 6 + [_u16p, _i32p, _i32p, _i32p, _f32p, _u16p]
        L.oracle_combine_packed.restype = None
        L.oracle_bf16_rne_array.argtypes = [_f32p, _u16p, _c_long]
        L.oracle_bf16_rne_array.restype = None
        L.oracle_e4m3_rne_sat_array.argtypes = [_f32p, _u8p, _c_long]
        L.oracle_e4m3_rne_sat_array.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------------------------------
# number formats
# ------------------------------------------------------------------------------------------

def bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(a.reshape(-1), out.reshape(-1), a.size)
    return out


def e4m3_rne_sat(a: np.ndarray) -> np.ndarray:
    """fp32 array -> OCP E4M3 codes, round to nearest even, saturating at +-448."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().oracle_e4m3_rne_sat_array(a.reshape(-1), out.reshape(-1), a.size)
    return out


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


# ------------------------------------------------------------------------------------------
# the hot path, step by step
# ------------------------------------------------------------------------------------------

def layout(topk_idx: np.ndarray, E: int, C: int, R: int) -> dict:
    """Routing layout. ``topk_idx`` int32 [T, K]. Returns slot [T, K], count [E], offset [E],
    rank_count [R], rank_offset [R], raw [E] and stats {kept, dropped, unrouted, invalid}."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    slot = np.empty((T, K), dtype=np.int32)
    count = np.empty(E, dtype=np.int32)
    offset = np.empty(E, dtype=np.int32)
    rank_count = np.empty(R, dtype=np.int32)
    rank_offset = np.empty(R, dtype=np.int32)
    raw = np.empty(E, dtype=np.int32)
    stats = np.empty(4, dtype=np.int32)
    lib().oracle_layout(T, K, E, C, R, idx, slot, count, offset, _ptr(rank_count),
                        _ptr(rank_offset), stats, _ptr(raw))
    return dict(slot=slot, count=count, offset=offset, rank_count=rank_count,
                rank_offset=rank_offset, raw=raw,
                stats=dict(kept=int(stats[0]), dropped=int(stats[1]),
                           unrouted=int(stats[2]), invalid=int(stats[3])),
                stats_array=stats)


def dispatch(x: np.ndarray, topk_idx: np.ndarray, slot: np.ndarray, E: int, C: int,
             recv: np.ndarray) -> np.ndarray:
    """bf16 dispatch into ``recv`` (uint16 [E, C, H]), in place; returns ``recv``."""
    T, H = x.shape
    K = topk_idx.shape[1]
    assert recv.shape == (E, C, H) and recv.dtype == np.uint16 and recv.flags.c_contiguous
    lib().oracle_dispatch(T, H, E, K, C, np.ascontiguousarray(x), np.ascontiguousarray(topk_idx),
                          np.ascontiguousarray(slot), recv)
    return recv


def dispatch_fp8(x: np.ndarray, topk_idx: np.ndarray, slot: np.ndarray, E: int, C: int,
                 recv_q: np.ndarray, recv_scale: np.ndarray):
    """FP8 dispatch into ``recv_q`` (uint8 [E, C, H]) and ``recv_scale`` (float32 [E, C, H/128])."""
    T, H = x.shape
    K = topk_idx.shape[1]
    assert H % 128 == 0
    assert recv_q.shape == (E, C, H) and recv_q.dtype == np.uint8
    assert recv_scale.shape == (E, C, H // 128) and recv_scale.dtype == np.float32
    lib().oracle_dispatch_fp8(T, H, E, K, C, np.ascontiguousarray(x),
                              np.ascontiguousarray(topk_idx), np.ascontiguousarray(slot),
                              recv_q, recv_scale)
    return recv_q, recv_scale


def combine(y: np.ndarray, topk_idx: np.ndarray, slot: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """Combine from ``y`` (uint16 [E, C, H]) -> out (uint16 [T, H])."""
    E, C, H = y.shape
    T, K = topk_idx.shape
    out = np.empty((T, H), dtype=np.uint16)
    lib().oracle_combine(T, H, E, K, C, np.ascontiguousarray(y), np.ascontiguousarray(topk_idx),
                         np.ascontiguousarray(slot), np.ascontiguousarray(topk_w, dtype=np.float32),
                         out)
    return out


def combine_tokens(tokens: np.ndarray, y: np.ndarray, topk_idx: np.ndarray, slot: np.ndarray,
                   topk_w: np.ndarray) -> np.ndarray:
    """Combine for a subset of tokens; row n of the result is token ``tokens[n]``."""
    E, C, H = y.shape
    T, K = topk_idx.shape
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    assert tok.size == 0 or (tok.min() >= 0 and tok.max() < T)
    out = np.empty((tok.size, H), dtype=np.uint16)
    lib().oracle_combine_tokens(tok.size, tok, H, E, K, C, np.ascontiguousarray(y),
                                np.ascontiguousarray(topk_idx), np.ascontiguousarray(slot),
                                np.ascontiguousarray(topk_w, dtype=np.float32), out)
    return out


# ------------------------------------------------------------------------------------------
# the two-stage path: one copy per (token, virtual rank), then the rank's own expansion
# ------------------------------------------------------------------------------------------

def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype)


def rank_layout(topk_idx: np.ndarray, E: int, R: int) -> dict:
    """Which virtual ranks each token goes to. Returns ``rank_slot`` int32 [T, R] (the token's
    position among the rank's tokens, -1 if not sent) and ``rank_tokens`` int32 [R]."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    rank_slot = np.empty((T, R), dtype=np.int32)
    rank_tokens = np.empty(R, dtype=np.int32)
    lib().oracle_rank_layout(T, K, E, R, idx, rank_slot, rank_tokens)
    return dict(rank_slot=rank_slot, rank_tokens=rank_tokens)


def dispatch_ranks(x: np.ndarray, rank_slot: np.ndarray, stage: np.ndarray) -> np.ndarray:
    """Stage 1 of dispatch into ``stage`` (uint16 [R, T, H]), in place."""
    T, H = x.shape
    R = rank_slot.shape[1]
    assert stage.shape == (R, T, H) and stage.dtype == np.uint16 and stage.flags.c_contiguous
    lib().oracle_dispatch_ranks(T, H, R, _c(x), _c(rank_slot), stage)
    return stage


def dispatch_ranks_fp8(x: np.ndarray, rank_slot: np.ndarray, stage_q: np.ndarray,
                       stage_scale: np.ndarray):
    """FP8 stage 1 into ``stage_q`` (uint8 [R, T, H]) and ``stage_scale`` (float32 [R, T, H/128])."""
    T, H = x.shape
    R = rank_slot.shape[1]
    assert H % 128 == 0
    assert stage_q.shape == (R, T, H) and stage_q.dtype == np.uint8
    assert stage_scale.shape == (R, T, H // 128) and stage_scale.dtype == np.float32
    lib().oracle_dispatch_ranks_fp8(T, H, R, _c(x), _c(rank_slot), stage_q, stage_scale)
    return stage_q, stage_scale


def dispatch_expand(stage: np.ndarray, topk_idx: np.ndarray, slot: np.ndarray,
                    rank_slot: np.ndarray, E: int, C: int, recv: np.ndarray) -> np.ndarray:
    """Stage 2 of dispatch from ``stage`` [R, T, H] into ``recv`` (uint16 [E, C, H]), in place."""
    R, T, H = stage.shape
    K = topk_idx.shape[1]
    assert recv.shape == (E, C, H) and recv.dtype == np.uint16 and recv.flags.c_contiguous
    lib().oracle_dispatch_expand(T, H, E, K, C, R, _c(stage), _c(topk_idx), _c(slot),
                                 _c(rank_slot), recv)
    return recv


def dispatch_expand_fp8(stage_q, stage_scale, topk_idx, slot, rank_slot, E, C, recv_q,
                        recv_scale):
    """FP8 stage 2 into ``recv_q`` [E, C, H] and ``recv_scale`` [E, C, H/128], in place."""
    R, T, H = stage_q.shape
    K = topk_idx.shape[1]
    assert recv_q.shape == (E, C, H) and recv_scale.shape == (E, C, H // 128)
    lib().oracle_dispatch_expand_fp8(T, H, E, K, C, R, _c(stage_q), _c(stage_scale),
                                     _c(topk_idx), _c(slot), _c(rank_slot), recv_q, recv_scale)
    return recv_q, recv_scale


def combine_ranks(y: np.ndarray, topk_idx: np.ndarray, slot: np.ndarray, rank_slot: np.ndarray,
                  topk_w: np.ndarray) -> np.ndarray:
    """Stage 1 of combine: per-rank partial rows, uint16 [R, T, H]; rows of tokens a rank did
    not receive are left as zero here (the kernels leave them untouched)."""
    E, C, H = y.shape
    T, K = topk_idx.shape
    R = rank_slot.shape[1]
    part = np.zeros((R, T, H), dtype=np.uint16)
    lib().oracle_combine_ranks(T, H, E, K, C, R, _c(y), _c(topk_idx), _c(slot), _c(rank_slot),
                               _c(topk_w, np.float32), part)
    return part


def combine_reduce(part: np.ndarray, rank_slot: np.ndarray) -> np.ndarray:
    """Stage 2 of combine: out uint16 [T, H] from the partial rows ``part`` [R, T, H]."""
    R, T, H = part.shape
    out = np.empty((T, H), dtype=np.uint16)
    lib().oracle_combine_reduce(T, H, R, _c(part), _c(rank_slot), out)
    return out


def combine_two_stage_tokens(tokens: np.ndarray, y: np.ndarray, topk_idx: np.ndarray,
                             slot: np.ndarray, rank_slot: np.ndarray,
                             topk_w: np.ndarray) -> np.ndarray:
    """The two-stage combine for a subset of tokens; row n of the result is token tokens[n]."""
    E, C, H = y.shape
    T, K = topk_idx.shape
    R = rank_slot.shape[1]
    tok = _c(tokens, np.int32)
    assert tok.size == 0 or (tok.min() >= 0 and tok.max() < T)
    out = np.empty((tok.size, H), dtype=np.uint16)
    lib().oracle_combine_two_stage_tokens(tok.size, tok, H, E, K, C, R, _c(y), _c(topk_idx),
                                          _c(slot), _c(rank_slot), _c(topk_w, np.float32), out)
    return out


# ------------------------------------------------------------------------------------------
# packed, aligned receive layout
# ------------------------------------------------------------------------------------------

def packed_offsets(count: np.ndarray, align: int) -> np.ndarray:
    """offset [E+1]: exclusive scan of the kept counts rounded up to multiples of ``align``;
    offset[E] is the number of rows of the packed buffer."""
    cnt = _c(count, np.int32)
    off = np.empty(cnt.size + 1, dtype=np.int32)
    lib().oracle_packed_offsets(cnt.size, int(align), cnt, off)
    return off


def dispatch_packed(x, topk_idx, slot, offset, E, C, recv):
    """bf16 dispatch into the packed ``recv`` (uint16 [rows, H]), in place."""
    T, H = x.shape
    K = topk_idx.shape[1]
    rows = recv.shape[0]
    assert recv.shape == (rows, H) and recv.dtype == np.uint16 and recv.flags.c_contiguous
    lib().oracle_dispatch_packed(T, H, E, K, C, rows, _c(x), _c(topk_idx), _c(slot), _c(offset),
                                 recv)
    return recv


def dispatch_packed_fp8(x, topk_idx, slot, offset, E, C, recv_q, recv_scale):
    """FP8 dispatch into the packed ``recv_q`` [rows, H] and ``recv_scale`` [rows, H/128]."""
    T, H = x.shape
    K = topk_idx.shape[1]
    rows = recv_q.shape[0]
    assert recv_q.shape == (rows, H) and recv_scale.shape == (rows, H // 128)
    lib().oracle_dispatch_packed_fp8(T, H, E, K, C, rows, _c(x), _c(topk_idx), _c(slot),
                                     _c(offset), recv_q, recv_scale)
    return recv_q, recv_scale


def combine_packed(y, topk_idx, slot, offset, topk_w, E, C):
    """Combine from the packed ``y`` (uint16 [rows, H]) -> out (uint16 [T, H])."""
    rows, H = y.shape
    T, K = topk_idx.shape
    out = np.empty((T, H), dtype=np.uint16)
    lib().oracle_combine_packed(T, H, E, K, C, rows, _c(y), _c(topk_idx), _c(slot), _c(offset),
                                _c(topk_w, np.float32), out)
    return out

