"""Python binding of libkvsel (ctypes): argument marshalling only.

Every function here mirrors one entry point of include/kvsel.h and passes
device pointers (torch tensors' data_ptr()) and the current HIP stream; all of
the computation happens in the HIP kernels behind the C ABI.  A missing or
unloadable library raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvsel.so")

KVSEL_OK, KVSEL_ERR_INVALID_ARG, KVSEL_ERR_UNSUPPORTED, KVSEL_ERR_WORKSPACE, KVSEL_ERR_HIP = range(5)
KVSEL_F32, KVSEL_BF16 = 0, 1
KVSEL_POOL_HEAD, KVSEL_POOL_GROUP = 0, 1
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}

# the exported symbols of include/kvsel.h
EXPORTS = ("kvsel_workspace_size", "kvsel_sparse_attn_workspace_size", "kvsel_select", "kvsel_sparse_attn",
           "kvsel_prefill_chunk", "kvsel_prefill_chunk_noalloc", "kvsel_decode_reuse", "kvsel_compacted_view",
           "kvsel_last_error",
           "kvsel_version", "kvsel_trace_start", "kvsel_trace_stop", "kvsel_trace_read", "kvsel_kernel_name")
KERNELS = ("qstats", "qtopk", "qpack", "scan", "topb", "gather", "pack", "attn", "append", "qpool", "reuse")


class Heads(ctypes.Structure):
    _fields_ = [("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class Params(ctypes.Structure):
    """n_q, budget and the pooling order (KVSEL_POOL_HEAD by default)."""
    _fields_ = [("n_q", ctypes.c_int32), ("budget", ctypes.c_int32), ("pooling", ctypes.c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("block_table", ctypes.c_void_p)]


class SelCache(ctypes.Structure):
    """The selected-entry cache of kvsel_decode_reuse (device pointers)."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("counts", ctypes.c_void_p)]


class Batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("prior_len_host", ctypes.POINTER(ctypes.c_int64)), ("prior_len_dev", ctypes.c_void_p)]


class KvselError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvsel {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvsel.so (built by chunked_prefill_kv_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it first (python -m chunked_prefill_kv_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kvsel_workspace_size.argtypes = [P(Heads), P(Batch), P(Params), P(sz)]
    lib.kvsel_sparse_attn_workspace_size.argtypes = [P(Heads), P(Batch), i32, P(sz)]
    lib.kvsel_select.argtypes = [P(Heads), P(Batch), P(Params), vp, P(Cache), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kvsel_sparse_attn.argtypes = [P(Heads), P(Batch), vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.kvsel_prefill_chunk.argtypes = [P(Heads), P(Batch), P(Params), vp, vp, vp, P(Cache), vp, i32, vp, vp, sz, vp]
    lib.kvsel_decode_reuse.argtypes = [P(Heads), P(Batch), P(Params), vp, vp, vp, P(Cache), P(SelCache), vp, i32, vp, vp,
                                       sz, vp]
    lib.kvsel_prefill_chunk_noalloc.argtypes = [P(Heads), P(Batch), P(Params), vp, vp, vp, P(Cache), vp, i32, vp, vp]
    lib.kvsel_compacted_view.argtypes = [P(Heads), P(Batch), P(Params), P(Cache), P(i32), P(sz), P(sz), P(i32), P(i32)]
    for name in ("kvsel_workspace_size", "kvsel_sparse_attn_workspace_size", "kvsel_select", "kvsel_sparse_attn",
                 "kvsel_prefill_chunk", "kvsel_prefill_chunk_noalloc", "kvsel_decode_reuse", "kvsel_compacted_view"):
        getattr(lib, name).restype = ctypes.c_int
    lib.kvsel_last_error.argtypes = []
    lib.kvsel_last_error.restype = ctypes.c_char_p
    lib.kvsel_version.argtypes = []
    lib.kvsel_version.restype = ctypes.c_int32
    lib.kvsel_trace_start.argtypes = [ctypes.c_uint32]
    lib.kvsel_trace_stop.argtypes = []
    lib.kvsel_trace_read.argtypes = [P(ctypes.c_int32), P(ctypes.c_float), i32]
    for name in ("kvsel_trace_start", "kvsel_trace_stop", "kvsel_trace_read"):
        getattr(lib, name).restype = ctypes.c_int
    lib.kvsel_kernel_name.argtypes = [i32]
    lib.kvsel_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != KVSEL_OK:
        raise KvselError(status, _lib.kvsel_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVSEL_BF16
    if t.dtype == torch.float32:
        return KVSEL_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def heads(h_q: int, h_kv: int, d: int, dtype: int, scale: float = 0.0) -> Heads:
    return Heads(h_q, h_kv, d, dtype, scale)


def batch(prior_len_host: Sequence[int], chunk_len: int, prior_len_dev: Optional[torch.Tensor]) -> Batch:
    n = len(prior_len_host)
    arr = (ctypes.c_int64 * n)(*[int(x) for x in prior_len_host])
    b = Batch(n, chunk_len, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), _ptr(prior_len_dev))
    b._keep = (arr, prior_len_dev)   # the struct holds raw pointers: keep both arrays alive with it
    return b


def cache(k: torch.Tensor, v: torch.Tensor, capacity: int, block_size: int = 0,
          block_table: Optional[torch.Tensor] = None) -> Cache:
    mb = 0 if block_table is None else block_table.shape[1]
    c = Cache(k.data_ptr(), v.data_ptr(), capacity, block_size, mb, _ptr(block_table))
    c._keep = (k, v, block_table)    # raw pointers in the struct: keep the tensors alive with it
    return c


def workspace_size(h: Heads, b: Batch, p: Params) -> int:
    n = ctypes.c_size_t(0)
    _check(load().kvsel_workspace_size(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), ctypes.byref(n)))
    return n.value


def sparse_attn_workspace_size(h: Heads, b: Batch, n_sel_max: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().kvsel_sparse_attn_workspace_size(ctypes.byref(h), ctypes.byref(b), n_sel_max, ctypes.byref(n)))
    return n.value


def kvsel_select(h: Heads, b: Batch, p: Params, q: torch.Tensor, c: Cache, idx: torch.Tensor,
                 k_sel: Optional[torch.Tensor], v_sel: Optional[torch.Tensor], q_keep: Optional[torch.Tensor],
                 scores: Optional[torch.Tensor], ws: torch.Tensor) -> None:
    _check(load().kvsel_select(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), q.data_ptr(), ctypes.byref(c),
                               idx.data_ptr(), _ptr(k_sel), _ptr(v_sel), _ptr(q_keep), _ptr(scores),
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream()))


def kvsel_sparse_attn(h: Heads, b: Batch, q: torch.Tensor, k_sel: Optional[torch.Tensor],
                      v_sel: Optional[torch.Tensor], n_sel: torch.Tensor, n_sel_max: int, k_chunk: torch.Tensor,
                      v_chunk: torch.Tensor, out: torch.Tensor, ws: torch.Tensor) -> None:
    _check(load().kvsel_sparse_attn(ctypes.byref(h), ctypes.byref(b), q.data_ptr(), _ptr(k_sel), _ptr(v_sel),
                                    n_sel.data_ptr(), n_sel_max, k_chunk.data_ptr(), v_chunk.data_ptr(),
                                    out.data_ptr(), dtype_code(out), ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream()))


def kvsel_prefill_chunk(h: Heads, b: Batch, p: Params, q: torch.Tensor, k_chunk: torch.Tensor,
                        v_chunk: torch.Tensor, c: Cache, out: torch.Tensor, idx: Optional[torch.Tensor],
                        ws: torch.Tensor) -> None:
    _check(load().kvsel_prefill_chunk(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), q.data_ptr(),
                                      k_chunk.data_ptr(), v_chunk.data_ptr(), ctypes.byref(c), out.data_ptr(),
                                      dtype_code(out), _ptr(idx), ws.data_ptr(), ws.numel() * ws.element_size(),
                                      _stream()))


def sel_cache(k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, counts: Optional[torch.Tensor] = None) -> SelCache:
    c = SelCache(k.data_ptr(), v.data_ptr(), pos.data_ptr(), _ptr(counts))
    c._keep = (k, v, pos, counts)    # raw pointers in the struct: keep the tensors alive with it
    return c


def kvsel_decode_reuse(h: Heads, b: Batch, p: Params, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       c: Cache, sel: SelCache, out: torch.Tensor, idx: Optional[torch.Tensor], ws: torch.Tensor) -> None:
    _check(load().kvsel_decode_reuse(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), q.data_ptr(), k_new.data_ptr(),
                                     v_new.data_ptr(), ctypes.byref(c), ctypes.byref(sel), out.data_ptr(),
                                     dtype_code(out), _ptr(idx), ws.data_ptr(), ws.numel() * ws.element_size(),
                                     _stream()))


def kvsel_prefill_chunk_noalloc(h: Heads, b: Batch, p: Params, q: torch.Tensor, k_chunk: torch.Tensor,
                                v_chunk: torch.Tensor, c: Cache, out: torch.Tensor,
                                idx: Optional[torch.Tensor]) -> None:
    _check(load().kvsel_prefill_chunk_noalloc(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), q.data_ptr(),
                                              k_chunk.data_ptr(), v_chunk.data_ptr(), ctypes.byref(c),
                                              out.data_ptr(), dtype_code(out), _ptr(idx), _stream()))


def compacted_view(h: Heads, b: Batch, p: Params, c: Cache) -> Optional[dict]:
    """Where kvsel_prefill_chunk leaves the compacted key/value lists in its workspace
    (None when the call reads the kept rows in place): byte offsets, slots per
    (sequence, KV head) and whether the values are stored transposed."""
    packed, slots, vt = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    ko, vo = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().kvsel_compacted_view(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), ctypes.byref(c),
                                       ctypes.byref(packed), ctypes.byref(ko), ctypes.byref(vo), ctypes.byref(slots),
                                       ctypes.byref(vt)))
    if not packed.value:
        return None
    return {"k_offset": ko.value, "v_offset": vo.value, "slots": slots.value, "v_transposed": bool(vt.value)}


def trace_start(kernels=KERNELS) -> None:
    """Bracket every later launch of the named kernels with HIP events on its stream."""
    mask = 0
    for k in kernels:
        mask |= 1 << KERNELS.index(k)
    _check(load().kvsel_trace_start(mask))


def trace_stop() -> None:
    _check(load().kvsel_trace_stop())


def trace_read() -> dict:
    """{kernel: (launches, total_ms)} for the traced launches since the last read."""
    n = len(KERNELS)
    launches = (ctypes.c_int32 * n)()
    ms = (ctypes.c_float * n)()
    _check(load().kvsel_trace_read(launches, ms, n))
    return {KERNELS[i]: (launches[i], ms[i]) for i in range(n) if launches[i]}


def last_error() -> str:
    return load().kvsel_last_error().decode()


def version() -> int:
    return load().kvsel_version()
