"""ctypes binding of libhpcattn (include/hpcattn.h), with the same names.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libhpcattn.so.  Tensors are passed by ``data_ptr()`` and the
stream is torch's current HIP stream unless one is given.  Importing this
module loads the library and raises ImportError if it has not been built
(``python -m load_balanced_split_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhpcattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libhpcattn.so is not built; run `python -m load_balanced_split_amd.build` "
        "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)

PAGE_SIZE = 64
MAX_BATCH = 8192
MAX_GROUP = 16
MAX_ROWS = 64
KV_BF16 = 0
KV_FP8_E4M3 = 1

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_LAUNCH, ERR_ARG = 0, -1, -2, -3, -4, -5, -6
MAPERR_NEG_LEN, MAPERR_OVERFLOW = 1, 2
NOALLOC_SCRATCH_BYTES = 32 << 20
NOALLOC_MAX_SEGMENTS = 65536


class hpcattn_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("q_rows", ctypes.c_int32),
    ]


PROLOGUE_ROPE, PROLOGUE_HADAMARD = 1, 2
PROLOGUE_MAX_HEADS = 65536


class hpcattn_prologue_dims(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("rope_base", ctypes.c_float),
    ]


class hpcattn_task_map(ctypes.Structure):
    _fields_ = [
        ("words", ctypes.c_void_p),
        ("bytes", ctypes.c_size_t),
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_bins", ctypes.c_int32),
        ("min_tiles", ctypes.c_int32),
    ]


_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_fp = ctypes.POINTER(ctypes.c_float)
_sig = {
    "hpcattn_task_map_bytes": (ctypes.c_size_t, [_i32, _i32, _i32]),
    "hpcattn_max_partials": (_i64, [_i32, _i32, _i32]),
    "hpcattn_static_max_partials": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "hpcattn_suggest_num_bins": (_i32, [_i32, _i32, _i32]),
    "hpcattn_plan": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32,
                                    ctypes.POINTER(hpcattn_task_map), _vp]),
    "hpcattn_decode": (ctypes.c_int, [ctypes.POINTER(hpcattn_dims), _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, ctypes.POINTER(hpcattn_task_map), _vp, _vp,
                                      _i64, _vp]),
    "hpcattn_decode_combine": (ctypes.c_int, [ctypes.POINTER(hpcattn_dims), _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp, ctypes.POINTER(hpcattn_task_map),
                                              _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp]),
    "hpcattn_decode_combine_noalloc": (ctypes.c_int, [ctypes.POINTER(hpcattn_dims), _vp, _vp,
                                                      _vp, _vp, _vp, _vp, _vp,
                                                      ctypes.POINTER(hpcattn_task_map), _vp,
                                                      _vp, _vp]),
    "hpcattn_combine": (ctypes.c_int, [ctypes.POINTER(hpcattn_dims),
                                       ctypes.POINTER(hpcattn_task_map), _vp, _vp, _vp, _vp,
                                       _vp]),
    "hpcattn_static_decode": (ctypes.c_int, [ctypes.POINTER(hpcattn_dims), _i32, _i32, _i32,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _i64, _vp, _vp, _vp]),
    "hpcattn_probe_stream_read": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _i32, _vp, _vp]),
    "hpcattn_prologue": (ctypes.c_int, [ctypes.POINTER(hpcattn_prologue_dims), _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hpcattn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "hpcattn_version": (ctypes.c_int, []),
}
EXPORTS = tuple(_sig)
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class HpcattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, hpcattn_strerror(status), status))


def _check(status: int, where: str) -> None:
    if status != OK:
        raise HpcattnError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhpcattn must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_req, num_pages,
              kv_dtype=KV_BF16, sm_scale=None, q_rows=1) -> hpcattn_dims:
    """q_rows: query rows per request (1 for decode, 1 + drafts to verify)."""
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    return hpcattn_dims(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_req,
                        num_pages, kv_dtype, sm_scale, q_rows)


class TaskMap:
    """A device task-map buffer (int32 tensor) with its ABI handle."""

    def __init__(self, words, batch: int, num_kv_heads: int, num_bins: int):
        self.words = words
        self.handle = hpcattn_task_map(_ptr(words), words.numel() * 4, batch, num_kv_heads,
                                       num_bins, 0)

    @property
    def num_bins(self) -> int:
        return self.handle.num_bins


def hpcattn_task_map_bytes(batch: int, num_kv_heads: int, num_bins: int) -> int:
    return int(_lib.hpcattn_task_map_bytes(batch, num_kv_heads, num_bins))


def hpcattn_max_partials(batch: int, num_kv_heads: int, num_bins: int) -> int:
    return int(_lib.hpcattn_max_partials(batch, num_kv_heads, num_bins))


def hpcattn_static_max_partials(batch, num_kv_heads, policy, param, max_seq_len) -> int:
    return int(_lib.hpcattn_static_max_partials(batch, num_kv_heads, policy, param, max_seq_len))


def hpcattn_suggest_num_bins(head_dim: int, kv_dtype: int, rows: int) -> int:
    """Co-resident decode workgroups on the current device for rows = q_rows * G
    query rows per KV head (needs a GPU)."""
    n = int(_lib.hpcattn_suggest_num_bins(head_dim, kv_dtype, rows))
    _check(min(n, 0), "hpcattn_suggest_num_bins")
    return n


def hpcattn_strerror(status: int) -> str:
    return _lib.hpcattn_strerror(status).decode()


def hpcattn_version() -> int:
    return int(_lib.hpcattn_version())


def alloc_task_map(batch: int, num_kv_heads: int, num_bins: int, device) -> TaskMap:
    """A zeroed task-map buffer: until hpcattn_plan writes it, every bin is
    empty, so a decode on it does no work (and reads no descriptor)."""
    import torch
    n = hpcattn_task_map_bytes(batch, num_kv_heads, num_bins) // 4
    return TaskMap(torch.zeros(n, dtype=torch.int32, device=device), batch, num_kv_heads,
                   num_bins)


def hpcattn_plan(seq_lens, num_kv_heads: int, num_bins: int, min_tiles: int,
                 task_map: TaskMap, stream=None) -> TaskMap:
    """Build the task map for this decode step (seq_lens: device int32 [B])."""
    _check(_lib.hpcattn_plan(_ptr(seq_lens), int(seq_lens.numel()), num_kv_heads, num_bins,
                             min_tiles, ctypes.byref(task_map.handle), _stream(stream)),
           "hpcattn_plan")
    return task_map


def hpcattn_decode(dims: hpcattn_dims, q, k_pages, v_pages, page_table, task_map: TaskMap,
                   part_o, part_lse, q_scale=None, k_scale=None, v_scale=None,
                   stream=None) -> None:
    rows = part_o.shape[0] if hasattr(part_o, "shape") else 0
    _check(_lib.hpcattn_decode(ctypes.byref(dims), _ptr(q), _ptr(q_scale), _ptr(k_pages),
                               _ptr(v_pages), _ptr(k_scale), _ptr(v_scale), _ptr(page_table),
                               ctypes.byref(task_map.handle), _ptr(part_o), _ptr(part_lse),
                               rows, _stream(stream)),
           "hpcattn_decode")


def hpcattn_decode_combine(dims: hpcattn_dims, q, k_pages, v_pages, page_table,
                           task_map: TaskMap, part_o, part_lse, tickets, out, out_lse=None,
                           q_scale=None, k_scale=None, v_scale=None, stream=None) -> None:
    """Decode + combine in one launch; tickets: int32 [>= B * H_kv], zero."""
    rows = part_o.shape[0] if hasattr(part_o, "shape") else 0
    nt = tickets.numel() if hasattr(tickets, "numel") else 0
    _check(_lib.hpcattn_decode_combine(ctypes.byref(dims), _ptr(q), _ptr(q_scale),
                                       _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(page_table),
                                       ctypes.byref(task_map.handle), _ptr(part_o),
                                       _ptr(part_lse), rows, _ptr(tickets), nt, _ptr(out),
                                       _ptr(out_lse), _stream(stream)),
           "hpcattn_decode_combine")


def hpcattn_decode_combine_noalloc(dims: hpcattn_dims, q, k_pages, v_pages, page_table,
                                   task_map: TaskMap, out, out_lse=None, q_scale=None,
                                   k_scale=None, v_scale=None, stream=None) -> None:
    """Decode + combine with the partials and tickets in the library's fixed
    per-device scratch: the caller passes no workspace."""
    _check(_lib.hpcattn_decode_combine_noalloc(ctypes.byref(dims), _ptr(q), _ptr(q_scale),
                                               _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                               _ptr(v_scale), _ptr(page_table),
                                               ctypes.byref(task_map.handle), _ptr(out),
                                               _ptr(out_lse), _stream(stream)),
           "hpcattn_decode_combine_noalloc")


def hpcattn_combine(dims: hpcattn_dims, task_map: TaskMap, part_o, part_lse, out,
                    out_lse=None, stream=None) -> None:
    _check(_lib.hpcattn_combine(ctypes.byref(dims), ctypes.byref(task_map.handle),
                                _ptr(part_o), _ptr(part_lse), _ptr(out), _ptr(out_lse),
                                _stream(stream)),
           "hpcattn_combine")


def hpcattn_static_decode(dims: hpcattn_dims, policy: int, param: int, max_seq_len: int,
                          seq_lens, q, k_pages, v_pages, page_table, part_o, part_lse, out,
                          out_lse=None, q_scale=None, k_scale=None, v_scale=None,
                          stream=None) -> None:
    rows = part_o.shape[0] if hasattr(part_o, "shape") else 0
    _check(_lib.hpcattn_static_decode(ctypes.byref(dims), policy, param, max_seq_len,
                                      _ptr(seq_lens), _ptr(q), _ptr(q_scale), _ptr(k_pages),
                                      _ptr(v_pages), _ptr(k_scale), _ptr(v_scale),
                                      _ptr(page_table), _ptr(part_o), _ptr(part_lse), rows,
                                      _ptr(out), _ptr(out_lse), _stream(stream)),
           "hpcattn_static_decode")


def hpcattn_probe_stream_read(buf, workgroups: int, sink, nontemporal: bool = False,
                              chunked: bool = False, stream=None) -> None:
    """Streaming read of a whole contiguous device tensor (measurement only);
    `chunked` reads it as scattered 16 KB chunks."""
    flags = (1 if nontemporal else 0) | (2 if chunked else 0)
    _check(_lib.hpcattn_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(),
                                          workgroups, flags, _ptr(sink), _stream(stream)),
           "hpcattn_probe_stream_read")


def hpcattn_prologue(dims: hpcattn_prologue_dims, qkv, positions, cache_slots, q_out,
                     k_pages, v_pages, q_norm_w=None, k_norm_w=None, q_scale=None,
                     k_scale=None, v_scale=None, stream=None) -> None:
    """QK-Norm -> RoPE -> [Hadamard] -> quantise Q and store K/V in the cache."""
    _check(_lib.hpcattn_prologue(ctypes.byref(dims), _ptr(qkv), _ptr(positions),
                                 _ptr(cache_slots), _ptr(q_norm_w), _ptr(k_norm_w),
                                 _ptr(q_out), _ptr(q_scale), _ptr(k_pages), _ptr(v_pages),
                                 _ptr(k_scale), _ptr(v_scale), _stream(stream)),
           "hpcattn_prologue")
