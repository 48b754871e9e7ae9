"""ctypes binding of libvamla.so (C ABI in include/vamla.h).

Argument marshalling only: tensors are passed as device pointers together with
the current HIP stream of torch; every step of the verify path runs in the HIP
kernels behind the ABI.  Importing this module does not load the library; the
first call does, and raises if libvamla.so has not been built.  There is no
CPU fallback.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libvamla.so")

D_QK = 576
D_V = 512
MAX_TREE = 65
MAX_HEADS = 128
KEY_TILE = 32
ROW_TILE = 64
FLAG_DEVICE_LENGTHS = 1
FLAG_DEBUG_VALIDATE = 2

STATUS = {
    0: "VAMLA_OK", -1: "VAMLA_ERR_INVALID_ARG", -2: "VAMLA_ERR_UNSUPPORTED", -3: "VAMLA_ERR_WORKSPACE",
    -4: "VAMLA_ERR_ARCH", -5: "VAMLA_ERR_LAUNCH", -6: "VAMLA_ERR_INVALID_TREE", -7: "VAMLA_ERR_INVALID_SLOT",
    -8: "VAMLA_ERR_INVALID_LENGTHS", -9: "VAMLA_ERR_STATIC_LIMIT",
}
STATIC_WORKSPACE_BYTES = 64 << 20
READ_ROWS_SINK_WORDS = 4608                # include/vamla.h VAMLA_READ_ROWS_SINK_WORDS

EXPORTS = ("vamla_status_string", "vamla_plan", "vamla_workspace_size", "vamla_validate", "verify_attn_mla",
           "vamla_split_partials", "vamla_lse_merge", "vamla_slot_gather", "verify_attn_mla_static",
           "vamla_read_rows")


class VamlaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("pool_slots", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("max_tree", ctypes.c_int32),
        ("total_tree", ctypes.c_int32),
        ("max_prefix", ctypes.c_int64),
        ("total_prefix", ctypes.c_int64),
        ("chunk", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("cu_prefix", ctypes.c_void_p),
        ("cu_tree", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class VamlaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int32),
        ("row_tiles", ctypes.c_int32),
        ("max_chunks", ctypes.c_int32),
        ("grid_items", ctypes.c_int32),
        ("off_part_o", ctypes.c_size_t),
        ("off_part_lse", ctypes.c_size_t),
        ("off_debug_record", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class VamlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_msg(status)})")


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libvamla.so once; raise if it is missing (no fallback path)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speculative_decoding_tree_verify_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER
    L.vamla_status_string.restype = ctypes.c_char_p
    L.vamla_status_string.argtypes = [ctypes.c_int]
    L.vamla_plan.argtypes = [P(VamlaParams), P(VamlaPlanInfo)]
    L.vamla_workspace_size.argtypes = [P(VamlaParams), P(ctypes.c_size_t)]
    L.vamla_validate.argtypes = [P(VamlaParams), vp, vp, vp, vp, vp]
    L.verify_attn_mla.argtypes = [P(VamlaParams), vp, vp, vp, vp, vp, vp, vp, vp]
    L.vamla_split_partials.argtypes = [P(VamlaParams), vp, vp, vp, vp, vp, vp]
    L.vamla_lse_merge.argtypes = [P(VamlaParams), vp, vp, vp]
    L.vamla_slot_gather.argtypes = [vp, vp, i64, vp, vp]
    L.verify_attn_mla_static.argtypes = [P(VamlaParams), vp, vp, vp, vp, vp, vp, vp, vp]
    L.vamla_read_rows.argtypes = [vp, vp, i64, vp, vp]
    for name in EXPORTS:
        if name != "vamla_status_string":
            getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def _msg(status: int) -> str:
    try:
        return lib().vamla_status_string(status).decode()
    except Exception:  # library not loadable: plain code only
        return str(status)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise VamlaError(status, where)


# --------------------------------------------------------------------------
# parameters
# --------------------------------------------------------------------------

@dataclass
class Problem:
    """Host-known scalars of one verify call (no device reads needed)."""
    batch: int
    num_heads: int
    pool_slots: int
    softmax_scale: float
    max_tree: int
    total_tree: int
    max_prefix: int
    total_prefix: int
    chunk: int = 0
    flags: int = 0

    def params(self, cu_prefix_ptr: int = 0, cu_tree_ptr: int = 0, workspace_ptr: int = 0,
               workspace_bytes: int = 0) -> VamlaParams:
        return VamlaParams(self.batch, self.num_heads, D_QK, D_V, self.pool_slots, self.softmax_scale,
                           self.max_tree, self.total_tree, self.max_prefix, self.total_prefix, self.chunk, self.flags,
                           cu_prefix_ptr, cu_tree_ptr, workspace_ptr, workspace_bytes)

    @staticmethod
    def from_host(cu_prefix, cu_tree, num_heads: int, pool_slots: int, softmax_scale: float,
                  chunk: int = 0) -> "Problem":
        """Derive the scalars from host copies of the cumulative length arrays."""
        cp = [int(x) for x in cu_prefix]
        ct = [int(x) for x in cu_tree]
        B = len(cp) - 1
        return Problem(batch=B, num_heads=num_heads, pool_slots=pool_slots, softmax_scale=float(softmax_scale),
                       max_tree=max(ct[b + 1] - ct[b] for b in range(B)), total_tree=ct[-1],
                       max_prefix=max(cp[b + 1] - cp[b] for b in range(B)), total_prefix=cp[-1], chunk=chunk)


def plan(prob: Problem) -> VamlaPlanInfo:
    info = VamlaPlanInfo()
    p = prob.params()
    _check(lib().vamla_plan(ctypes.byref(p), ctypes.byref(info)), "vamla_plan")
    return info


def workspace_size(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    p = prob.params()
    _check(lib().vamla_workspace_size(ctypes.byref(p), ctypes.byref(n)), "vamla_workspace_size")
    return int(n.value)


def validate(prob: Problem, parent, cu_tree, cu_prefix, prefix_slot_idx=None, tree_slot_idx=None) -> int:
    """Host-side validation of index arrays (numpy int32, contiguous).  Returns the status."""
    import numpy as np

    def ptr(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=np.int32)
        keep.append(a)
        return a.ctypes.data
    keep = []
    p = prob.params()
    return int(lib().vamla_validate(ctypes.byref(p), ptr(parent), ptr(cu_tree), ptr(cu_prefix),
                                    ptr(prefix_slot_idx), ptr(tree_slot_idx)))


# --------------------------------------------------------------------------
# device calls (torch tensors on the current HIP device)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _device(*tensors):
    """The one GPU that every given tensor (None entries skipped) is on: the
    call runs with it as the current device, on its stream."""
    devs = {t.device for t in tensors if t is not None}
    if any(d.type != "cuda" for d in devs):
        raise ValueError("tensor must be on the GPU")
    if len(devs) != 1:
        raise ValueError(f"tensors must all be on one GPU, got {sorted(str(d) for d in devs)}")
    return next(iter(devs))


def _stream(stream=None, device=None) -> int:
    """The HIP stream to enqueue on: the given one (which must belong to
    device), else the device's current stream (read as its raw handle when
    torch offers that, which costs a tenth of building a Stream object)."""
    torch = _torch()
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None and device is not None:
            return raw(device.index)
        stream = torch.cuda.current_stream(device)
    if device is not None and stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    return stream.cuda_stream


def _on(device):
    """Context that makes device current for the call (the library's arch
    check and static workspace are per device); nothing to do when it is
    current already."""
    torch = _torch()
    if torch.cuda.current_device() == device.index:
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _bits(t, what: str):
    """bf16 tensors are passed as their 16-bit patterns."""
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"{what} must be bfloat16 (or its 16-bit pattern), got {t.dtype}")


class Workspace:
    """Caller-owned scratch sized by vamla_workspace_size (allocated by torch)."""

    def __init__(self, prob: Problem, device=None):
        torch = _torch()
        if device is not None and torch.device(device).type != "cuda":
            raise ValueError("the workspace must be on the GPU")
        self.nbytes = workspace_size(prob)
        # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device or "cuda")
        assert self.buf.data_ptr() % 256 == 0

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()


def _params(prob: Problem, cu_prefix, cu_tree, ws: Workspace) -> VamlaParams:
    _index(cu_prefix, prob.batch + 1, "cu_prefix")
    _index(cu_tree, prob.batch + 1, "cu_tree")
    return prob.params(_ptr(cu_prefix), _ptr(cu_tree), ws.ptr, ws.nbytes)


# Shape and dtype checks: the kernels trust every size they are given, so a
# wrong dtype (an int64 index tensor read as int32 pairs) or a short output
# buffer would be read or written past its end.  These run before any launch.

def _index(t, min_numel: int, what: str) -> None:
    torch = _torch()
    if t is None:
        raise ValueError(f"{what} is required")
    if t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32, got {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{what} has {t.numel()} elements, needs at least {min_numel}")


def _shaped(t, shape, dtypes, what: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _bf16_like():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _check_pool(kv_pool, pool_slots: int) -> None:
    if kv_pool.dim() != 2 or kv_pool.shape[1] != D_QK:
        raise ValueError(f"kv_pool must have shape [P, {D_QK}], got {tuple(kv_pool.shape)}")
    if kv_pool.dtype not in _bf16_like():
        raise TypeError(f"kv_pool must be bfloat16, got {kv_pool.dtype}")
    if kv_pool.shape[0] < pool_slots:
        raise ValueError(f"kv_pool has {kv_pool.shape[0]} rows, pool_slots says {pool_slots}")


def _check_inputs(prob: Problem, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree) -> None:
    T, H = prob.total_tree, prob.num_heads
    _index(cu_prefix, prob.batch + 1, "cu_prefix")
    _index(cu_tree, prob.batch + 1, "cu_tree")
    _shaped(q, (T, H, D_QK), _bf16_like(), "q")
    _check_pool(kv_pool, prob.pool_slots)
    if prob.total_prefix:
        _index(prefix_slot_idx, prob.total_prefix, "prefix_slot_idx")
    _index(tree_slot_idx, T, "tree_slot_idx")
    _index(parent, T, "parent")


def _check_outputs(prob: Problem, out, lse) -> None:
    torch = _torch()
    T, H = prob.total_tree, prob.num_heads
    _shaped(out, (T, H, D_V), (torch.bfloat16,), "out")
    _shaped(lse, (T, H), (torch.float32,), "lse")


def verify_attn_mla(prob: Problem, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree,
                    ws: Optional[Workspace] = None, out=None, lse=None, stream=None) -> Tuple[object, object]:
    """out [T, H, 512] bf16, lse [T, H] fp32 for every tree node and head."""
    torch = _torch()
    _check_inputs(prob, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree)
    T, H = prob.total_tree, prob.num_heads
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _check_outputs(prob, out, lse)
    ws = ws or Workspace(prob, q.device)
    dev = _device(q, kv_pool, prefix_slot_idx if prob.total_prefix else None, tree_slot_idx, parent, cu_prefix,
                  cu_tree, out, lse, ws.buf)
    p = _params(prob, cu_prefix, cu_tree, ws)
    with _on(dev):
        st = lib().verify_attn_mla(ctypes.byref(p), _ptr(_bits(q, "q")), _ptr(_bits(kv_pool, "kv_pool")),
                                   _ptr(prefix_slot_idx) if prob.total_prefix else None, _ptr(tree_slot_idx),
                                   _ptr(parent), _ptr(out), _ptr(lse), _stream(stream, dev))
    _check(st, "verify_attn_mla")
    return out, lse


def verify_attn_mla_static(prob: Problem, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree,
                           out=None, lse=None, stream=None) -> Tuple[object, object]:
    """verify_attn_mla with the library's static device workspace (the C
    entry point allocates nothing; out / lse are allocated here only when
    not given)."""
    torch = _torch()
    _check_inputs(prob, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree)
    T, H = prob.total_tree, prob.num_heads
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _check_outputs(prob, out, lse)
    dev = _device(q, kv_pool, prefix_slot_idx if prob.total_prefix else None, tree_slot_idx, parent, cu_prefix,
                  cu_tree, out, lse)
    p = prob.params(_ptr(cu_prefix), _ptr(cu_tree))
    # the static workspace is per device: the call runs with dev current
    with _on(dev):
        st = lib().verify_attn_mla_static(ctypes.byref(p), _ptr(_bits(q, "q")), _ptr(_bits(kv_pool, "kv_pool")),
                                          _ptr(prefix_slot_idx) if prob.total_prefix else None,
                                          _ptr(tree_slot_idx), _ptr(parent), _ptr(out), _ptr(lse),
                                          _stream(stream, dev))
    _check(st, "verify_attn_mla_static")
    return out, lse


def split_partials(prob: Problem, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree,
                   ws: Workspace, stream=None):
    """Stage 1: chunk partials into the workspace (the last chunk of each
    request also covers its tree keys)."""
    _check_inputs(prob, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree)
    dev = _device(q, kv_pool, prefix_slot_idx if prob.total_prefix else None, tree_slot_idx, parent, cu_prefix,
                  cu_tree, ws.buf)
    p = _params(prob, cu_prefix, cu_tree, ws)
    with _on(dev):
        _check(lib().vamla_split_partials(ctypes.byref(p), _ptr(_bits(q, "q")), _ptr(_bits(kv_pool, "kv_pool")),
                                          _ptr(prefix_slot_idx) if prob.total_prefix else None,
                                          _ptr(tree_slot_idx), _ptr(parent), _stream(stream, dev)),
               "vamla_split_partials")


def lse_merge(prob: Problem, cu_prefix, cu_tree, ws: Workspace, out, lse, stream=None):
    _check_outputs(prob, out, lse)
    dev = _device(cu_prefix, cu_tree, ws.buf, out, lse)
    p = _params(prob, cu_prefix, cu_tree, ws)
    with _on(dev):
        _check(lib().vamla_lse_merge(ctypes.byref(p), _ptr(out), _ptr(lse), _stream(stream, dev)),
               "vamla_lse_merge")


def slot_gather(kv_pool, idx, dst=None, stream=None):
    """dst[l] = kv_pool[idx[l]] (bit-exact)."""
    torch = _torch()
    _index(idx, 0, "idx")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != D_QK or kv_pool.dtype not in _bf16_like():
        raise ValueError(f"kv_pool must be bfloat16 [P, {D_QK}], got {kv_pool.dtype} {tuple(kv_pool.shape)}")
    n = idx.numel()
    if dst is None:
        dst = torch.empty((n, D_QK), dtype=kv_pool.dtype, device=kv_pool.device)
    _shaped(dst, (n, D_QK), _bf16_like(), "dst")
    dev = _device(kv_pool, idx, dst)
    with _on(dev):
        _check(lib().vamla_slot_gather(_ptr(_bits(kv_pool, "kv_pool")), _ptr(idx) if n else None, n,
                                       _ptr(dst) if n else None, _stream(stream, dev)), "vamla_slot_gather")
    return dst


def read_rows(kv_pool, idx, sink=None, stream=None):
    """Reads the rows kv_pool[idx] and folds them into sink (uint32
    [READ_ROWS_SINK_WORDS], as int32): the XOR of its words is the XOR of every
    32-bit word of those rows.  A read-rate calibration, no compute."""
    torch = _torch()
    _index(idx, 0, "idx")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != D_QK or kv_pool.dtype not in _bf16_like():
        raise ValueError(f"kv_pool must be bfloat16 [P, {D_QK}], got {kv_pool.dtype} {tuple(kv_pool.shape)}")
    if sink is None:
        sink = torch.empty(READ_ROWS_SINK_WORDS, dtype=torch.int32, device=kv_pool.device)
    _shaped(sink, (READ_ROWS_SINK_WORDS,), (torch.int32,), "sink")
    n = idx.numel()
    dev = _device(kv_pool, idx, sink)
    with _on(dev):
        _check(lib().vamla_read_rows(_ptr(_bits(kv_pool, "kv_pool")), _ptr(idx) if n else None, n, _ptr(sink),
                                     _stream(stream, dev)), "vamla_read_rows")
    return sink


def workspace_views(prob: Problem, ws: Workspace):
    """Typed views of the workspace regions (for stage-level checks):
    part_o [B, tiles, chunks, 128, 64, 4], part_lse [B, tiles, chunks, 64]
    (float32)."""
    torch = _torch()
    info = plan(prob)
    B, R, C = prob.batch, info.row_tiles, info.max_chunks
    f = ws.buf.view(torch.float32) if ws.buf.numel() % 4 == 0 else ws.buf[: ws.buf.numel() // 4 * 4].view(torch.float32)

    def region(off, shape):
        n = 1
        for s in shape:
            n *= s
        return f[off // 4: off // 4 + n].view(*shape)
    return dict(plan=info,
                part_o=region(info.off_part_o, (B, R, C, D_V // 4, ROW_TILE, 4)),
                part_lse=region(info.off_part_lse, (B, R, C, ROW_TILE)))


def debug_record(prob: Problem, ws: Workspace, with_restarts: bool = False):
    """The device-side check's record (VAMLA_FLAG_DEBUG_VALIDATE) as a host
    tuple (status, array, index); (0, 0, 0) when the index data was valid.
    with_restarts appends the split pass's restart count.  Reads the
    workspace after the caller's stream has finished the call."""
    torch = _torch()
    info = plan(prob)
    off = info.off_debug_record
    rec = ws.buf[off:off + 16].view(torch.int32).cpu().tolist()
    return (rec[0], rec[1], rec[2], rec[3]) if with_restarts else (rec[0], rec[1], rec[2])
