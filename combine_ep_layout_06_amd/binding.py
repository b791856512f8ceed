"""ctypes binding of libep_mi355x.so (include/ep.h) for torch tensors.

Argument marshalling only: each function checks dtypes, devices, sizes and contiguity, then
passes ``data_ptr()`` values and torch's current HIP stream to the C entry point of the same
name. Under ``record()`` the C calls are captured into a CallList instead, whose ``replay()``
re-issues them without the Python-side checks (for loops that refill the same buffers). Every
step of the computation runs in the library's gfx950 kernels; there is no other code path. If
the library is missing the functions raise instead of computing anything.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

from .build import LIB

EP_OK, EP_ERR_INVALID, EP_ERR_ALIGN, EP_ERR_UNSUPPORTED, EP_ERR_HIP = 0, -1, -2, -3, -4
EP_STATS_LEN = 4
EP_MAX_EXPERTS = 1024
EP_MAX_TOPK = 256
EP_FP8_BLOCK = 128
EP_MAX_RANKS = 64

#: every entry point the header declares
EXPORTED = ("ep_layout", "ep_dispatch", "ep_dispatch_fp8", "ep_layout_dispatch",
            "ep_layout_dispatch_fp8", "ep_combine", "ep_rank_layout", "ep_dispatch_ranks",
            "ep_dispatch_ranks_fp8", "ep_rank_layout_dispatch", "ep_rank_layout_dispatch_fp8",
            "ep_dispatch_expand", "ep_dispatch_expand_fp8", "ep_layout_dispatch_expand",
            "ep_layout_dispatch_expand_fp8",
            "ep_combine_ranks", "ep_combine_reduce", "ep_layout_packed", "ep_dispatch_packed",
            "ep_dispatch_packed_fp8", "ep_layout_dispatch_packed", "ep_layout_dispatch_packed_fp8",
            "ep_combine_packed", "ep_check_e4m3_conversion", "ep_last_launches",
            "ep_layout_workspace_bytes", "ep_layout_dispatch_ws", "ep_layout_dispatch_fp8_ws",
            "ep_layout_dispatch_noalloc", "ep_error_string", "ep_last_error", "ep_version")


class EpShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("C", ctypes.c_int32), ("R", ctypes.c_int32)]


class EpLaunchRecord(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p),
                ("grid_x", ctypes.c_uint32), ("grid_y", ctypes.c_uint32),
                ("grid_z", ctypes.c_uint32), ("block_x", ctypes.c_uint32),
                ("block_y", ctypes.c_uint32), ("block_z", ctypes.c_uint32),
                ("dynamic_lds_bytes", ctypes.c_uint32), ("static_lds_bytes", ctypes.c_uint32),
                ("vgprs", ctypes.c_int32), ("private_bytes", ctypes.c_uint32),
                ("max_threads_per_block", ctypes.c_int32)]


class EpError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        super().__init__(f"{fn} failed with {code}: {detail}")
        self.code = code


_lib = None


def library_path() -> str:
    return os.environ.get("EP_MI355X_LIB", LIB)


def load_library():
    """Load the HIP library once. Raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m combine_ep_layout_06_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(path)
        vp, sp = ctypes.c_void_p, ctypes.POINTER(EpShape)
        L.ep_layout.argtypes = [sp] + [vp] * 7 + [vp]
        L.ep_dispatch.argtypes = [sp, vp, vp, vp, vp, vp]
        L.ep_dispatch_fp8.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.ep_combine.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.ep_layout_dispatch.argtypes = [sp] + [vp] * 10
        L.ep_layout_dispatch_fp8.argtypes = [sp] + [vp] * 11
        L.ep_rank_layout.argtypes = [sp, vp, vp, vp, vp]
        L.ep_dispatch_ranks.argtypes = [sp, vp, vp, vp, vp]
        L.ep_dispatch_ranks_fp8.argtypes = [sp, vp, vp, vp, vp, vp]
        L.ep_rank_layout_dispatch.argtypes = [sp] + [vp] * 6
        L.ep_rank_layout_dispatch_fp8.argtypes = [sp] + [vp] * 7
        L.ep_dispatch_expand.argtypes = [sp] + [vp] * 6
        L.ep_dispatch_expand_fp8.argtypes = [sp] + [vp] * 8
        L.ep_layout_dispatch_expand.argtypes = [sp] + [vp] * 11
        L.ep_layout_dispatch_expand_fp8.argtypes = [sp] + [vp] * 13
        L.ep_combine_ranks.argtypes = [sp] + [vp] * 7
        L.ep_combine_reduce.argtypes = [sp] + [vp] * 4
        i32 = ctypes.c_int32
        L.ep_layout_packed.argtypes = [sp, i32] + [vp] * 8
        L.ep_dispatch_packed.argtypes = [sp, i32] + [vp] * 6
        L.ep_dispatch_packed_fp8.argtypes = [sp, i32] + [vp] * 7
        L.ep_combine_packed.argtypes = [sp, i32] + [vp] * 7
        L.ep_layout_dispatch_packed.argtypes = [sp, i32, i32] + [vp] * 10
        L.ep_layout_dispatch_packed_fp8.argtypes = [sp, i32, i32] + [vp] * 11
        L.ep_check_e4m3_conversion.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp, vp, vp]
        L.ep_last_launches.argtypes = [ctypes.POINTER(EpLaunchRecord), ctypes.c_int]
        L.ep_layout_dispatch_ws.argtypes = [sp] + [vp] * 10 + [ctypes.c_size_t, vp]
        L.ep_layout_dispatch_fp8_ws.argtypes = [sp] + [vp] * 11 + [ctypes.c_size_t, vp]
        L.ep_layout_dispatch_noalloc.argtypes = [sp] + [vp] * 10
        for fn in EXPORTED:
            if fn.startswith("ep_") and fn not in ("ep_error_string", "ep_last_error",
                                                   "ep_version", "ep_layout_workspace_bytes"):
                getattr(L, fn).restype = ctypes.c_int
        L.ep_layout_workspace_bytes.argtypes = [sp]
        L.ep_layout_workspace_bytes.restype = ctypes.c_size_t
        L.ep_error_string.argtypes = [ctypes.c_int]
        L.ep_error_string.restype = ctypes.c_char_p
        L.ep_last_error.argtypes = []
        L.ep_last_error.restype = ctypes.c_char_p
        L.ep_version.argtypes = []
        L.ep_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def ep_version() -> str:
    return load_library().ep_version().decode()


def ep_error_string(code: int) -> str:
    return load_library().ep_error_string(code).decode()


def _check(fn: str, rc: int):
    if rc != EP_OK:
        raise EpError(fn, rc, load_library().ep_last_error().decode())


_shapes: dict = {}


def _shape(T, H, E, K, C, R) -> EpShape:
    # one EpShape per distinct shape (the C calls only read it)
    key = (T, H, E, K, C, R)
    sh = _shapes.get(key)
    if sh is None:
        if len(_shapes) >= 4096:
            _shapes.clear()
        sh = _shapes[key] = EpShape(*(int(v) for v in key))
    return sh


# torch's current HIP stream of the current device as a raw handle, without building a Stream
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


class CallList:
    """Entry-point calls captured by `record`: the same C calls with the same device pointers,
    re-issued by `replay` with none of the wrappers' checks or allocations. It holds references
    to every tensor the calls use, so the buffers live as long as the list."""

    def __init__(self):
        self.calls = []      # (C function, name, shape, pointer and int arguments, stream)
        self._tensors = []
        self.device = None   # the device of the recorded tensors

    def __len__(self):
        return len(self.calls)

    def replay(self, stream=None):
        """Issue the recorded calls in order, each on the stream it was recorded with if one was
        given then, else on ``stream`` (default: torch's current stream)."""
        if not self.calls:
            return
        _require_current("replay", self.device)
        s = _stream(stream)
        for fn, name, sh, args, st in self.calls:
            rc = fn(ctypes.byref(sh), *args, s if st is None else st)
            if rc != EP_OK:
                _check(name, rc)


_recording = threading.local()


@contextlib.contextmanager
def record():
    """Inside the block, the entry-point functions validate their arguments and allocate any
    missing outputs as usual, but the C calls are captured instead of issued. Yields the
    CallList; its ``replay()`` then launches the same kernels on the same buffers, which is
    all a serving loop needs when each step refills the same input tensors."""
    prev = getattr(_recording, "calls", None)
    cl = CallList()
    _recording.calls = cl
    try:
        yield cl
    finally:
        _recording.calls = prev


def _require_current(name: str, dev):
    """The library launches on the current HIP device, so the tensors must live there (device
    pointers of another GPU, or host pointers, would be read by the kernels)."""
    if dev is not None and dev.type == "cuda" and dev.index == torch.cuda.current_device():
        return
    try:
        cur = f"cuda:{torch.cuda.current_device()}"
    except RuntimeError:
        cur = "none (no GPU)"
    raise ValueError(f"{name}: the tensors are on {dev}, but the library launches on the current "
                     f"HIP device ({cur}); move them there or call under torch.cuda.device()")


def _call(name: str, sh: EpShape, *args, stream=None):
    """Issue (or record) one C call; tensor arguments are passed as their data pointers."""
    fn = getattr(load_library(), name)
    cargs = [a.data_ptr() if isinstance(a, torch.Tensor) else a for a in args]
    dev = next((a.device for a in args if isinstance(a, torch.Tensor)), None)
    cl = getattr(_recording, "calls", None)
    if cl is not None:
        if cl.calls and dev != cl.device:
            raise ValueError(f"{name}: a recorded list holds calls on one device only "
                             f"({cl.device}, not {dev})")
        cl.device = dev
        cl._tensors.extend([a for a in args if isinstance(a, torch.Tensor)])
        cl.calls.append((fn, name, sh, tuple(cargs),
                         None if stream is None else stream.cuda_stream))
        return
    _require_current(name, dev)
    rc = fn(ctypes.byref(sh), *cargs, _stream(stream))
    if rc != EP_OK:
        _check(name, rc)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, numel: int, device):
    if t.dtype != dtype or t.device != device or not t.is_contiguous() or t.numel() != numel:
        _reject(t, name, dtype, numel, device)


def _reject(t: torch.Tensor, name: str, dtype: torch.dtype, numel: int, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")


def _bf16(t: torch.Tensor) -> torch.dtype:
    # bf16 rows may be passed as torch.bfloat16 or as their int16/uint16 bit patterns
    return t.dtype if t.dtype in (torch.bfloat16, torch.int16, torch.uint16) else torch.bfloat16


def ep_layout(topk_idx: torch.Tensor, E: int, C: int, R: int, *, slot=None, expert_count=None,
              expert_offset=None, rank_count=None, rank_offset=None, stats=None, stream=None):
    """Routing layout. ``topk_idx`` int32 [T, K] on the GPU. Returns a dict of the outputs
    (``slot`` [T, K], ``expert_count`` [E], ``expert_offset`` [E], ``rank_count`` [R],
    ``rank_offset`` [R], ``stats`` [4] = kept, dropped, unrouted, invalid); any of them may be
    passed in preallocated."""
    dev = topk_idx.device
    T, K = topk_idx.shape
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    slot = mk((T, K)) if slot is None else slot
    expert_count = mk(E) if expert_count is None else expert_count
    expert_offset = mk(E) if expert_offset is None else expert_offset
    rank_count = mk(R) if rank_count is None else rank_count
    rank_offset = mk(R) if rank_offset is None else rank_offset
    stats = mk(EP_STATS_LEN) if stats is None else stats
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    for name, t, n in (("expert_count", expert_count, E), ("expert_offset", expert_offset, E),
                       ("rank_count", rank_count, R), ("rank_offset", rank_offset, R),
                       ("stats", stats, EP_STATS_LEN)):
        _need(t, name, torch.int32, n, dev)
    sh = _shape(T, 1, E, K, C, R)
    _call("ep_layout", sh, topk_idx, slot, expert_count, expert_offset, rank_count, rank_offset,
          stats, stream=stream)
    return dict(slot=slot, expert_count=expert_count, expert_offset=expert_offset,
                rank_count=rank_count, rank_offset=rank_offset, stats=stats)


def _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                    rank_offset, stats):
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    out = dict(slot=mk((T, K)) if slot is None else slot,
               expert_count=mk(E) if expert_count is None else expert_count,
               expert_offset=mk(E) if expert_offset is None else expert_offset,
               rank_count=mk(R) if rank_count is None else rank_count,
               rank_offset=mk(R) if rank_offset is None else rank_offset,
               stats=mk(EP_STATS_LEN) if stats is None else stats)
    _need(out["slot"], "slot", torch.int32, T * K, dev)
    for name, n in (("expert_count", E), ("expert_offset", E), ("rank_count", R),
                    ("rank_offset", R), ("stats", EP_STATS_LEN)):
        _need(out[name], name, torch.int32, n, dev)
    return out


def _layout_ts(lay):
    return [lay[k] for k in ("slot", "expert_count", "expert_offset", "rank_count",
                             "rank_offset", "stats")]


def ep_layout_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, recv: torch.Tensor, E: int,
                       C: int, R: int, *, slot=None, expert_count=None, expert_offset=None,
                       rank_count=None, rank_offset=None, stats=None, stream=None):
    """ep_layout + bf16 dispatch in one launch. Returns the layout dict (as ep_layout);
    ``recv`` [E, C, H] is written in place."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv, "recv", _bf16(recv), E * C * H, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch", sh, x, topk_idx, *_layout_ts(lay), recv, stream=stream)
    return lay


def layout_workspace_bytes(T: int, K: int, E: int) -> int:
    """Bytes of workspace the _ws calls need for T tokens, top-K, E experts."""
    return int(load_library().ep_layout_workspace_bytes(ctypes.byref(_shape(T, 1, E, K, 1, 1))))


def _workspace(workspace, T, K, E, dev):
    need = layout_workspace_bytes(T, K, E)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the batch's device")
    return workspace, workspace.numel() * workspace.element_size()


def ep_layout_dispatch_ws(x: torch.Tensor, topk_idx: torch.Tensor, recv: torch.Tensor, E: int,
                          C: int, R: int, *, workspace=None, slot=None, expert_count=None,
                          expert_offset=None, rank_count=None, rank_offset=None, stats=None,
                          stream=None):
    """ep_layout_dispatch in two launches through a workspace (chunk histograms): the same
    outputs, faster on large batches. ``workspace``: a device tensor of at least
    layout_workspace_bytes(T, K, E) bytes (allocated here if not given)."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv, "recv", _bf16(recv), E * C * H, dev)
    ws, nbytes = _workspace(workspace, T, K, E, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_ws", sh, x, topk_idx, *_layout_ts(lay), recv, ws, nbytes,
          stream=stream)
    return lay


def ep_layout_dispatch_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, recv: torch.Tensor,
                               E: int, C: int, R: int, *, slot=None, expert_count=None,
                               expert_offset=None, rank_count=None, rank_offset=None, stats=None,
                               stream=None):
    """ep_layout_dispatch_ws with the library's static scratch as the workspace (no workspace
    argument; the C call allocates nothing). Pass every output to allocate nothing here
    either."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv, "recv", _bf16(recv), E * C * H, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_noalloc", sh, x, topk_idx, *_layout_ts(lay), recv, stream=stream)
    return lay


def ep_layout_dispatch_fp8_ws(x: torch.Tensor, topk_idx: torch.Tensor, recv_q: torch.Tensor,
                              recv_scale: torch.Tensor, E: int, C: int, R: int, *,
                              workspace=None, slot=None, expert_count=None, expert_offset=None,
                              rank_count=None, rank_offset=None, stats=None, stream=None):
    """ep_layout_dispatch_fp8 in two launches through a workspace (see ep_layout_dispatch_ws)."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv_q, "recv_q", recv_q.dtype if recv_q.dtype in (torch.uint8, torch.float8_e4m3fn)
          else torch.uint8, E * C * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, E * C * (H // EP_FP8_BLOCK), dev)
    ws, nbytes = _workspace(workspace, T, K, E, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_fp8_ws", sh, x, topk_idx, *_layout_ts(lay), recv_q, recv_scale,
          ws, nbytes, stream=stream)
    return lay


def ep_layout_dispatch_fp8(x: torch.Tensor, topk_idx: torch.Tensor, recv_q: torch.Tensor,
                           recv_scale: torch.Tensor, E: int, C: int, R: int, *, slot=None,
                           expert_count=None, expert_offset=None, rank_count=None,
                           rank_offset=None, stats=None, stream=None):
    """ep_layout + FP8 dispatch in one launch. Returns the layout dict; ``recv_q`` and
    ``recv_scale`` are written in place."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv_q, "recv_q", recv_q.dtype if recv_q.dtype in (torch.uint8, torch.float8_e4m3fn)
          else torch.uint8, E * C * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, E * C * (H // EP_FP8_BLOCK), dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_fp8", sh, x, topk_idx, *_layout_ts(lay), recv_q, recv_scale,
          stream=stream)
    return lay


def ep_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor, recv: torch.Tensor,
                C: int, *, stream=None):
    """bf16 dispatch: ``x`` [T, H] bf16 -> ``recv`` [E, C, H] bf16 (written in place)."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    E = recv.numel() // (C * H)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(recv, "recv", _bf16(recv), E * C * H, dev)
    sh = _shape(T, H, E, K, C, 1)
    _call("ep_dispatch", sh, x, topk_idx, slot, recv, stream=stream)
    return recv


def ep_dispatch_fp8(x: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                    recv_q: torch.Tensor, recv_scale: torch.Tensor, C: int, *, stream=None):
    """FP8 dispatch: ``x`` [T, H] bf16 -> ``recv_q`` [E, C, H] uint8 (OCP E4M3 codes) and
    ``recv_scale`` [E, C, H/128] float32 (written in place)."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    E = recv_q.numel() // (C * H)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(recv_q, "recv_q", recv_q.dtype if recv_q.dtype in (torch.uint8, torch.float8_e4m3fn)
          else torch.uint8, E * C * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, E * C * (H // EP_FP8_BLOCK), dev)
    sh = _shape(T, H, E, K, C, 1)
    _call("ep_dispatch_fp8", sh, x, topk_idx, slot, recv_q, recv_scale, stream=stream)
    return recv_q, recv_scale


def ep_combine(y: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
               topk_w: torch.Tensor, C: int, *, out=None, stream=None):
    """Combine: ``y`` [E, C, H] bf16 -> ``out`` [T, H] bf16."""
    dev = y.device
    T, K = topk_idx.shape
    H = y.shape[-1]
    E = y.numel() // (C * H)
    out = torch.empty((T, H), dtype=_bf16(y), device=dev) if out is None else out
    _need(y, "y", _bf16(y), E * C * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(topk_w, "topk_w", torch.float32, T * K, dev)
    _need(out, "out", _bf16(out), T * H, dev)
    sh = _shape(T, H, E, K, C, 1)
    _call("ep_combine", sh, y, topk_idx, slot, topk_w, out, stream=stream)
    return out


# ------------------------------------------------------------------------------------------
# two-stage, rank-deduplicated path (stage buffers are [R, T, ...])
# ------------------------------------------------------------------------------------------

def ep_rank_layout(topk_idx: torch.Tensor, E: int, R: int, *, rank_slot=None, rank_tokens=None,
                   stream=None):
    """Which virtual ranks each token goes to: ``rank_slot`` int32 [T, R] (position among the
    rank's tokens, -1 if not sent) and ``rank_tokens`` int32 [R]."""
    dev = topk_idx.device
    T, K = topk_idx.shape
    rank_slot = torch.empty((T, R), dtype=torch.int32, device=dev) if rank_slot is None else rank_slot
    rank_tokens = (torch.empty(R, dtype=torch.int32, device=dev) if rank_tokens is None
                   else rank_tokens)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(rank_tokens, "rank_tokens", torch.int32, R, dev)
    sh = _shape(T, 1, E, K, 1, R)
    _call("ep_rank_layout", sh, topk_idx, rank_slot, rank_tokens, stream=stream)
    return dict(rank_slot=rank_slot, rank_tokens=rank_tokens)


def ep_dispatch_ranks(x: torch.Tensor, rank_slot: torch.Tensor, stage: torch.Tensor, *,
                      stream=None):
    """Stage 1 of dispatch: ``x`` [T, H] bf16 -> ``stage`` [R, T, H] bf16 (in place)."""
    dev = x.device
    T, H = x.shape
    R = rank_slot.shape[1]
    _need(x, "x", _bf16(x), T * H, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(stage, "stage", _bf16(stage), R * T * H, dev)
    sh = _shape(T, H, R, 1, 1, R)
    _call("ep_dispatch_ranks", sh, x, rank_slot, stage, stream=stream)
    return stage


def ep_dispatch_ranks_fp8(x: torch.Tensor, rank_slot: torch.Tensor, stage_q: torch.Tensor,
                          stage_scale: torch.Tensor, *, stream=None):
    """FP8 stage 1: ``stage_q`` [R, T, H] uint8 and ``stage_scale`` [R, T, H/128] float32."""
    dev = x.device
    T, H = x.shape
    R = rank_slot.shape[1]
    _need(x, "x", _bf16(x), T * H, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(stage_q, "stage_q", torch.uint8, R * T * H, dev)
    _need(stage_scale, "stage_scale", torch.float32, R * T * (H // EP_FP8_BLOCK), dev)
    sh = _shape(T, H, R, 1, 1, R)
    _call("ep_dispatch_ranks_fp8", sh, x, rank_slot, stage_q, stage_scale, stream=stream)
    return stage_q, stage_scale


def ep_rank_layout_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, R: int, *,
                            stage=None, rank_slot=None, rank_tokens=None, stream=None):
    """ep_rank_layout and ep_dispatch_ranks in one launch: ``x`` [T, H] bf16 -> ``stage``
    [R, T, H] bf16 (rows of tokens a rank does not receive untouched), ``rank_slot`` [T, R],
    ``rank_tokens`` [R]."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    stage = torch.empty((R, T, H), dtype=_bf16(x), device=dev) if stage is None else stage
    rank_slot = torch.empty((T, R), dtype=torch.int32, device=dev) if rank_slot is None else rank_slot
    rank_tokens = (torch.empty(R, dtype=torch.int32, device=dev) if rank_tokens is None
                   else rank_tokens)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(rank_tokens, "rank_tokens", torch.int32, R, dev)
    _need(stage, "stage", _bf16(stage), R * T * H, dev)
    sh = _shape(T, H, E, K, 1, R)
    _call("ep_rank_layout_dispatch", sh, x, topk_idx, rank_slot, rank_tokens, stage, stream=stream)
    return dict(stage=stage, rank_slot=rank_slot, rank_tokens=rank_tokens)


def ep_rank_layout_dispatch_fp8(x: torch.Tensor, topk_idx: torch.Tensor, E: int, R: int, *,
                                stage_q=None, stage_scale=None, rank_slot=None,
                                rank_tokens=None, stream=None):
    """ep_rank_layout and ep_dispatch_ranks_fp8 in one launch: ``stage_q`` [R, T, H] uint8,
    ``stage_scale`` [R, T, H/128] float32, ``rank_slot`` [T, R], ``rank_tokens`` [R]."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    NB = H // EP_FP8_BLOCK
    stage_q = torch.empty((R, T, H), dtype=torch.uint8, device=dev) if stage_q is None else stage_q
    stage_scale = (torch.empty((R, T, NB), dtype=torch.float32, device=dev)
                   if stage_scale is None else stage_scale)
    rank_slot = torch.empty((T, R), dtype=torch.int32, device=dev) if rank_slot is None else rank_slot
    rank_tokens = (torch.empty(R, dtype=torch.int32, device=dev) if rank_tokens is None
                   else rank_tokens)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(rank_tokens, "rank_tokens", torch.int32, R, dev)
    _need(stage_q, "stage_q", torch.uint8, R * T * H, dev)
    _need(stage_scale, "stage_scale", torch.float32, R * T * NB, dev)
    sh = _shape(T, H, E, K, 1, R)
    _call("ep_rank_layout_dispatch_fp8", sh, x, topk_idx, rank_slot, rank_tokens, stage_q,
          stage_scale, stream=stream)
    return dict(stage_q=stage_q, stage_scale=stage_scale, rank_slot=rank_slot,
                rank_tokens=rank_tokens)


def ep_dispatch_expand(stage: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                       rank_slot: torch.Tensor, recv: torch.Tensor, C: int, *, stream=None):
    """Stage 2 of dispatch: ``stage`` [R, T, H] -> ``recv`` [E, C, H] bf16 (in place)."""
    dev = stage.device
    R, T, H = stage.shape
    K = topk_idx.shape[1]
    E = recv.numel() // (C * H)
    _need(stage, "stage", _bf16(stage), R * T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(recv, "recv", _bf16(recv), E * C * H, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_dispatch_expand", sh, stage, topk_idx, slot, rank_slot, recv, stream=stream)
    return recv


def ep_layout_dispatch_expand(stage: torch.Tensor, topk_idx: torch.Tensor,
                              rank_slot: torch.Tensor, recv: torch.Tensor, E: int, C: int, *,
                              slot=None, expert_count=None, expert_offset=None, rank_count=None,
                              rank_offset=None, stats=None, stream=None):
    """ep_layout + stage 2 of dispatch in one launch: ``stage`` [R, T, H] -> ``recv`` [E, C, H]
    bf16 (in place). Returns the layout dict (as ep_layout)."""
    dev = stage.device
    R, T, H = stage.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(stage, "stage", _bf16(stage), R * T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(recv, "recv", _bf16(recv), E * C * H, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_expand", sh, stage, topk_idx, rank_slot, *_layout_ts(lay), recv,
          stream=stream)
    return lay


def ep_layout_dispatch_expand_fp8(stage_q: torch.Tensor, stage_scale: torch.Tensor,
                                  topk_idx: torch.Tensor, rank_slot: torch.Tensor,
                                  recv_q: torch.Tensor, recv_scale: torch.Tensor, E: int, C: int,
                                  *, slot=None, expert_count=None, expert_offset=None,
                                  rank_count=None, rank_offset=None, stats=None, stream=None):
    """ep_layout + FP8 stage 2 in one launch: codes and scales of the staged rows -> ``recv_q``
    [E, C, H] and ``recv_scale`` [E, C, H/128] (in place). Returns the layout dict."""
    dev = stage_q.device
    R, T, H = stage_q.shape
    K = topk_idx.shape[1]
    lay = _layout_outputs(dev, T, K, E, R, slot, expert_count, expert_offset, rank_count,
                          rank_offset, stats)
    _need(stage_q, "stage_q", stage_q.dtype if stage_q.dtype in (torch.uint8, torch.float8_e4m3fn)
          else torch.uint8, R * T * H, dev)
    _need(stage_scale, "stage_scale", torch.float32, R * T * (H // EP_FP8_BLOCK), dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(recv_q, "recv_q", recv_q.dtype if recv_q.dtype in (torch.uint8, torch.float8_e4m3fn)
          else torch.uint8, E * C * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, E * C * (H // EP_FP8_BLOCK), dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_expand_fp8", sh, stage_q, stage_scale, topk_idx, rank_slot,
          *_layout_ts(lay), recv_q, recv_scale, stream=stream)
    return lay


def ep_dispatch_expand_fp8(stage_q: torch.Tensor, stage_scale: torch.Tensor,
                           topk_idx: torch.Tensor, slot: torch.Tensor, rank_slot: torch.Tensor,
                           recv_q: torch.Tensor, recv_scale: torch.Tensor, C: int, *,
                           stream=None):
    """FP8 stage 2: codes and scales of the staged rows -> ``recv_q`` [E, C, H] and
    ``recv_scale`` [E, C, H/128] (in place)."""
    dev = stage_q.device
    R, T, H = stage_q.shape
    K = topk_idx.shape[1]
    E = recv_q.numel() // (C * H)
    NB = H // EP_FP8_BLOCK
    _need(stage_q, "stage_q", torch.uint8, R * T * H, dev)
    _need(stage_scale, "stage_scale", torch.float32, R * T * NB, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(recv_q, "recv_q", torch.uint8, E * C * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, E * C * NB, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_dispatch_expand_fp8", sh, stage_q, stage_scale, topk_idx, slot, rank_slot, recv_q,
          recv_scale, stream=stream)
    return recv_q, recv_scale


def ep_combine_ranks(y: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                     rank_slot: torch.Tensor, topk_w: torch.Tensor, C: int, *, part=None,
                     stream=None):
    """Stage 1 of combine: ``y`` [E, C, H] bf16 -> per-rank partial rows ``part`` [R, T, H]."""
    dev = y.device
    T, K = topk_idx.shape
    R = rank_slot.shape[1]
    H = y.shape[-1]
    E = y.numel() // (C * H)
    part = torch.empty((R, T, H), dtype=_bf16(y), device=dev) if part is None else part
    _need(y, "y", _bf16(y), E * C * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(topk_w, "topk_w", torch.float32, T * K, dev)
    _need(part, "part", _bf16(part), R * T * H, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_combine_ranks", sh, y, topk_idx, slot, rank_slot, topk_w, part, stream=stream)
    return part


def ep_combine_reduce(part: torch.Tensor, rank_slot: torch.Tensor, K: int, *, out=None,
                      stream=None):
    """Stage 2 of combine: ``part`` [R, T, H] -> ``out`` [T, H] bf16. K (the top-k of the
    routing) bounds the ranks a token reaches."""
    dev = part.device
    R, T, H = part.shape
    out = torch.empty((T, H), dtype=_bf16(part), device=dev) if out is None else out
    _need(part, "part", _bf16(part), R * T * H, dev)
    _need(rank_slot, "rank_slot", torch.int32, T * R, dev)
    _need(out, "out", _bf16(out), T * H, dev)
    sh = _shape(T, H, R, K, 1, R)
    _call("ep_combine_reduce", sh, part, rank_slot, out, stream=stream)
    return out


# ------------------------------------------------------------------------------------------
# packed, aligned receive layout (buffers are [rows, ...])
# ------------------------------------------------------------------------------------------

def packed_rows_bound(T: int, K: int, E: int, C: int, alignment: int) -> int:
    """Rows that always suffice for a packed buffer: every kept pair plus each expert's padding."""
    return min(T * K, E * C) + E * (alignment - 1)


def ep_layout_packed(topk_idx: torch.Tensor, E: int, C: int, R: int, alignment: int, *,
                     slot=None, expert_count=None, packed_offset=None, rank_count=None,
                     rank_offset=None, stats=None, stream=None):
    """Layout with packed offsets: returns ``slot``, ``expert_count``, ``packed_offset``
    [E + 1] (offset of each expert's rows, then the rows needed), ``rank_count``,
    ``rank_offset`` (padded rows per rank) and ``stats``."""
    dev = topk_idx.device
    T, K = topk_idx.shape
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    slot = mk((T, K)) if slot is None else slot
    expert_count = mk(E) if expert_count is None else expert_count
    packed_offset = mk(E + 1) if packed_offset is None else packed_offset
    rank_count = mk(R) if rank_count is None else rank_count
    rank_offset = mk(R) if rank_offset is None else rank_offset
    stats = mk(EP_STATS_LEN) if stats is None else stats
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    for name, t, n in (("expert_count", expert_count, E), ("packed_offset", packed_offset, E + 1),
                       ("rank_count", rank_count, R), ("rank_offset", rank_offset, R),
                       ("stats", stats, EP_STATS_LEN)):
        _need(t, name, torch.int32, n, dev)
    sh = _shape(T, 1, E, K, C, R)
    _call("ep_layout_packed", sh, int(alignment), topk_idx, slot, expert_count, packed_offset,
          rank_count, rank_offset, stats, stream=stream)
    return dict(slot=slot, expert_count=expert_count, packed_offset=packed_offset,
                rank_count=rank_count, rank_offset=rank_offset, stats=stats)


def ep_dispatch_packed(x: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                       packed_offset: torch.Tensor, recv: torch.Tensor, E: int, C: int, *,
                       stream=None):
    """bf16 dispatch into the packed ``recv`` [rows, H] (in place)."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    rows = recv.shape[0]
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(packed_offset, "packed_offset", torch.int32, E + 1, dev)
    _need(recv, "recv", _bf16(recv), rows * H, dev)
    sh = _shape(T, H, E, K, C, 1)
    _call("ep_dispatch_packed", sh, int(rows), x, topk_idx, slot, packed_offset, recv,
          stream=stream)
    return recv


def ep_dispatch_packed_fp8(x: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                           packed_offset: torch.Tensor, recv_q: torch.Tensor,
                           recv_scale: torch.Tensor, E: int, C: int, *, stream=None):
    """FP8 dispatch into the packed ``recv_q`` [rows, H] and ``recv_scale`` [rows, H/128]."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    rows = recv_q.shape[0]
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(packed_offset, "packed_offset", torch.int32, E + 1, dev)
    _need(recv_q, "recv_q", torch.uint8, rows * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, rows * (H // EP_FP8_BLOCK), dev)
    sh = _shape(T, H, E, K, C, 1)
    _call("ep_dispatch_packed_fp8", sh, int(rows), x, topk_idx, slot, packed_offset, recv_q,
          recv_scale, stream=stream)
    return recv_q, recv_scale


def _packed_layout_outputs(dev, T, K, E, R, slot, expert_count, packed_offset, rank_count,
                           rank_offset, stats):
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    out = dict(slot=mk((T, K)) if slot is None else slot,
               expert_count=mk(E) if expert_count is None else expert_count,
               packed_offset=mk(E + 1) if packed_offset is None else packed_offset,
               rank_count=mk(R) if rank_count is None else rank_count,
               rank_offset=mk(R) if rank_offset is None else rank_offset,
               stats=mk(EP_STATS_LEN) if stats is None else stats)
    _need(out["slot"], "slot", torch.int32, T * K, dev)
    for name, n in (("expert_count", E), ("packed_offset", E + 1), ("rank_count", R),
                    ("rank_offset", R), ("stats", EP_STATS_LEN)):
        _need(out[name], name, torch.int32, n, dev)
    return out


def ep_layout_dispatch_packed(x: torch.Tensor, topk_idx: torch.Tensor, recv: torch.Tensor, E: int,
                              C: int, R: int, alignment: int, *, slot=None, expert_count=None,
                              packed_offset=None, rank_count=None, rank_offset=None, stats=None,
                              stream=None):
    """ep_layout_packed and ep_dispatch_packed in one launch: the packed layout's outputs (a
    dict as ep_layout_packed returns) and ``recv`` [rows, H] bf16 filled in place."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    rows = recv.shape[0]
    o = _packed_layout_outputs(dev, T, K, E, R, slot, expert_count, packed_offset, rank_count,
                               rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv, "recv", _bf16(recv), rows * H, dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_packed", sh, int(alignment), int(rows), x, topk_idx, o["slot"],
          o["expert_count"], o["packed_offset"], o["rank_count"], o["rank_offset"], o["stats"],
          recv, stream=stream)
    return o


def ep_layout_dispatch_packed_fp8(x: torch.Tensor, topk_idx: torch.Tensor, recv_q: torch.Tensor,
                                  recv_scale: torch.Tensor, E: int, C: int, R: int,
                                  alignment: int, *, slot=None, expert_count=None,
                                  packed_offset=None, rank_count=None, rank_offset=None,
                                  stats=None, stream=None):
    """ep_layout_packed and ep_dispatch_packed_fp8 in one launch: the packed layout's outputs,
    ``recv_q`` [rows, H] and ``recv_scale`` [rows, H/128] filled in place."""
    dev = x.device
    T, H = x.shape
    K = topk_idx.shape[1]
    rows = recv_q.shape[0]
    o = _packed_layout_outputs(dev, T, K, E, R, slot, expert_count, packed_offset, rank_count,
                               rank_offset, stats)
    _need(x, "x", _bf16(x), T * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(recv_q, "recv_q", torch.uint8, rows * H, dev)
    _need(recv_scale, "recv_scale", torch.float32, rows * (H // EP_FP8_BLOCK), dev)
    sh = _shape(T, H, E, K, C, R)
    _call("ep_layout_dispatch_packed_fp8", sh, int(alignment), int(rows), x, topk_idx, o["slot"],
          o["expert_count"], o["packed_offset"], o["rank_count"], o["rank_offset"], o["stats"],
          recv_q, recv_scale, stream=stream)
    return o


def ep_combine_packed(y: torch.Tensor, topk_idx: torch.Tensor, slot: torch.Tensor,
                      packed_offset: torch.Tensor, topk_w: torch.Tensor, E: int, C: int, *,
                      out=None, stream=None):
    """Combine from the packed ``y`` [rows, H] -> ``out`` [T, H] bf16."""
    dev = y.device
    T, K = topk_idx.shape
    rows, H = y.shape
    out = torch.empty((T, H), dtype=_bf16(y), device=dev) if out is None else out
    _need(y, "y", _bf16(y), rows * H, dev)
    _need(topk_idx, "topk_idx", torch.int32, T * K, dev)
    _need(slot, "slot", torch.int32, T * K, dev)
    _need(packed_offset, "packed_offset", torch.int32, E + 1, dev)
    _need(topk_w, "topk_w", torch.float32, T * K, dev)
    _need(out, "out", _bf16(out), T * H, dev)
    sh = _shape(T, H, E, K, C, 1)
    _call("ep_combine_packed", sh, int(rows), y, topk_idx, slot, packed_offset, topk_w, out,
          stream=stream)
    return out



def ep_check_e4m3_conversion(first_pattern: int, count: int, *, device=None, stream=None):
    """Compare the FP8 cast's two E4M3 encoders (the hardware conversion and the software
    one) on the fp32 bit patterns [first_pattern, first_pattern + count) on the current
    device. Returns (mismatches, smallest mismatching pattern or None) after synchronising."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    res = torch.empty(2, dtype=torch.int32, device=dev)
    _require_current("ep_check_e4m3_conversion", dev)
    L = load_library()
    rc = L.ep_check_e4m3_conversion(first_pattern, count, res.data_ptr(), res.data_ptr() + 4,
                                    _stream(stream))
    _check("ep_check_e4m3_conversion", rc)
    torch.cuda.synchronize(dev)
    n, first = (int(v) & 0xFFFFFFFF for v in res.cpu().tolist())
    return n, (None if n == 0 else first)


_resources = None


def kernel_resources() -> dict:
    """The compiler's resource figures per kernel symbol, written by the build beside the
    library (empty if that file is missing)."""
    global _resources
    if _resources is None:
        import json
        path = os.path.join(os.path.dirname(library_path()), "kernel_resources.json")
        try:
            with open(path) as f:
                _resources = json.load(f).get("kernels", {})
        except (OSError, ValueError):
            _resources = {}
    return _resources


def last_launches() -> list:
    """The kernel launches of this thread's most recent library call: per launch the kernel
    symbol, grid and workgroup sizes, LDS, and the register figures of the runtime and of the
    compiler's report."""
    L = load_library()
    recs = (EpLaunchRecord * 8)()
    n = L.ep_last_launches(recs, 8)
    res = kernel_resources()
    out = []
    for r in recs[:min(n, 8)]:
        name = (r.kernel or b"").decode()
        d = {"kernel": name, "grid": [r.grid_x, r.grid_y, r.grid_z],
             "block": [r.block_x, r.block_y, r.block_z],
             "dynamic_lds_bytes": r.dynamic_lds_bytes, "static_lds_bytes": r.static_lds_bytes,
             "vgprs": r.vgprs, "private_bytes": r.private_bytes}
        if name in res:
            d["compiler"] = res[name]
        out.append(d)
    return out
