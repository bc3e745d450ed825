"""Oracle: a plain fp64 CPU reference for load-balanced split-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and never imports it; inputs come from numpy arrays that the
caller made with the seeded workload generator.

What it computes is written in ``oracle.c`` next to this file, each function
citing the passage of the pages it follows ("HPC-Ops x SGLang", sections
"Attention: load balancing for variable-length decode" and "Scheduling around
live KV work"; "Hy3 preview full-stack inference optimization", section 2.1.1).

Arrays:
  q          [B, H_q, D]              uint16 (bf16 bits) or uint8 (e4m3 bytes),
             or [B, R, H_q, D] for R query rows per request (the confirmed
             token and R - 1 drafts: row r sits at position L_b - R + r and
             sees tokens [0, L_b - R + r]); outputs then carry the R axis too
  k_pages    [num_pages, H_kv, 64, D] same element type as q
  v_pages    [num_pages, H_kv, 64, D]
  q_scale    [B, H_q] (or [B, R, H_q]) float32, fp8 only
  k_scale    [num_pages, H_kv, 64] float32, v_scale likewise (fp8 only)
  page_table [B, max_pages] int32
  seq_lens   [B] int32
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

TILE = 64


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-shared", "-fPIC",
             _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_fp8", ctypes.c_int32),
        ("q_rows", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # ORACLE_LIB names another build of oracle.c (the sanitizer run of
            # the test suite builds one with -fsanitize=address,undefined).
            path = os.environ.get("ORACLE_LIB") or build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
            dp = ctypes.POINTER(_Dims)
            lib.orc_bf16_value.argtypes = [i32]
            lib.orc_bf16_value.restype = f64
            lib.orc_e4m3_value.argtypes = [i32]
            lib.orc_e4m3_value.restype = f64
            lib.orc_attend_range.argtypes = [dp, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                             P, P]
            lib.orc_attend_range.restype = ctypes.c_int
            lib.orc_attention.argtypes = [dp, P, P, P, P, P, P, P, P, P, i32, P, P]
            lib.orc_attention.restype = ctypes.c_int
            lib.orc_lse_merge.argtypes = [i32, i32, P, P, P, P]
            lib.orc_lse_merge.restype = None
            lib.orc_plan_words.argtypes = [i32, i32, i32]
            lib.orc_plan_words.restype = i64
            lib.orc_plan.argtypes = [P, i32, i32, i32, i32, P, i64]
            lib.orc_plan.restype = i64
            lib.orc_partials.argtypes = [dp, P, P, P, P, P, P, P, P, i32, P, P]
            lib.orc_partials.restype = ctypes.c_int
            lib.orc_combine.argtypes = [dp, P, i32, P, P, P, P]
            lib.orc_combine.restype = ctypes.c_int
            lib.orc_max_threads.argtypes = []
            lib.orc_max_threads.restype = i32
            lib.orc_set_threads.argtypes = [i32]
            lib.orc_set_threads.restype = None
            lib.orc_e4m3_encode.argtypes = [f64]
            lib.orc_e4m3_encode.restype = i32
            lib.orc_prologue.argtypes = [i32, i32, i32, i32, P, P, P, P, f64, i32, f64, i32,
                                         P, P, P, P, P, P, P, P, P]
            lib.orc_prologue.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Inputs:
    """Validated, contiguous views of one attention problem."""

    def __init__(self, q, k_pages, v_pages, page_table, num_kv_heads, sm_scale,
                 q_scale=None, k_scale=None, v_scale=None):
        fp8 = q.dtype == np.uint8
        et = np.uint8 if fp8 else np.uint16
        if q.dtype not in (np.uint8, np.uint16):
            raise TypeError("q must hold bf16 bits (uint16) or e4m3 bytes (uint8)")
        self.q = _c(q, et)
        self.k = _c(k_pages, et)
        self.v = _c(v_pages, et)
        self.pt = _c(page_table, np.int32)
        if self.q.ndim == 3:
            B, Hq, D = self.q.shape
            self.R = 1
        elif self.q.ndim == 4:
            B, self.R, Hq, D = self.q.shape
        else:
            raise ValueError("q must be [B, H_q, D] or [B, R, H_q, D]")
        if self.R < 1:
            raise ValueError("at least one query row per request")
        if self.k.shape[1:] != (num_kv_heads, TILE, D) or self.v.shape != self.k.shape:
            raise ValueError("k/v pools must be [num_pages, H_kv, 64, D]")
        if Hq % num_kv_heads:
            raise ValueError("H_q must be a multiple of H_kv")
        if fp8:
            if q_scale is None or k_scale is None or v_scale is None:
                raise ValueError("fp8 inputs need q_scale, k_scale and v_scale")
            self.qs = _c(q_scale, np.float32)
            self.ks = _c(k_scale, np.float32)
            self.vs = _c(v_scale, np.float32)
        else:
            self.qs = self.ks = self.vs = None
        self.dims = _Dims(B, Hq, num_kv_heads, D, self.pt.shape[1], self.k.shape[0],
                          1 if fp8 else 0, self.R, float(sm_scale))
        self.B, self.Hq, self.D = B, Hq, D
        self.G = Hq // num_kv_heads

    def args(self):
        return (ctypes.byref(self.dims), _ptr(self.q), _ptr(self.qs), _ptr(self.k),
                _ptr(self.v), _ptr(self.ks), _ptr(self.vs), _ptr(self.pt))


def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(int(bits))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e4m3_table() -> np.ndarray:
    """fp64 value of each of the 256 OCP E4M3FN codes."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def attend_range(q, k_pages, v_pages, page_table, b, h, tok0, tok1, *, num_kv_heads,
                 sm_scale, q_scale=None, k_scale=None, v_scale=None, seq_len=None):
    """Attention of the query rows of (request b, KV head h) over tokens
    [tok0, tok1), row r within its visible length seq_len - (R - 1 - r)
    (seq_len defaults to tok1).  Returns (o [R G, D], lse [R G]) in fp64,
    row r G + g for query head h G + g."""
    x = _Inputs(q, k_pages, v_pages, page_table, num_kv_heads, sm_scale,
                q_scale, k_scale, v_scale)
    n = x.R * x.G
    o = np.zeros((n, x.D), np.float64)
    lse = np.zeros((n,), np.float64)
    ln = tok1 if seq_len is None else seq_len
    rc = _load().orc_attend_range(*x.args(), int(b), int(h), int(tok0), int(tok1), int(ln),
                                  _ptr(o), _ptr(lse))
    if rc:
        raise RuntimeError("orc_attend_range failed")
    return o, lse


def attention(q, k_pages, v_pages, page_table, seq_lens, *, num_kv_heads, sm_scale,
              q_scale=None, k_scale=None, v_scale=None, pairs=None):
    """Decode attention of every request over its whole live KV.

    pairs: optional iterable of (b, h) to compute; other rows stay NaN.
    Returns (out, lse) in fp64, shaped like q without D: [B, H_q, D] and
    [B, H_q], or [B, R, H_q, D] and [B, R, H_q]."""
    x = _Inputs(q, k_pages, v_pages, page_table, num_kv_heads, sm_scale,
                q_scale, k_scale, v_scale)
    lens = _c(seq_lens, np.int32)
    lead = x.q.shape[:-1]
    out = np.full(lead + (x.D,), np.nan, np.float64)
    lse = np.full(lead, np.nan, np.float64)
    pr = None if pairs is None else np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
    n = 0 if pr is None else pr.shape[0]
    rc = _load().orc_attention(*x.args(), _ptr(lens), _ptr(pr), n, _ptr(out), _ptr(lse))
    if rc:
        raise RuntimeError("orc_attention failed")
    return out, lse


def lse_merge(lse, o):
    """Merge n partials (lse [n], o [n, W]) under the global softmax."""
    lse = _c(lse, np.float64)
    o = _c(o, np.float64).reshape(lse.shape[0], -1)
    out = np.zeros((o.shape[1],), np.float64)
    out_lse = np.zeros((1,), np.float64)
    _load().orc_lse_merge(lse.shape[0], o.shape[1], _ptr(lse), _ptr(o), _ptr(out), _ptr(out_lse))
    return out, float(out_lse[0])


def plan_words(batch: int, num_kv_heads: int, num_bins: int) -> int:
    return int(_load().orc_plan_words(batch, num_kv_heads, num_bins))


def plan(seq_lens, num_kv_heads: int, num_bins: int, min_tiles: int) -> np.ndarray:
    """The task map as int32 words (layout in oracle.c)."""
    lens = _c(seq_lens, np.int32)
    n = plan_words(lens.shape[0], num_kv_heads, num_bins)
    m = np.zeros((n,), np.int32)
    rc = _load().orc_plan(_ptr(lens), lens.shape[0], num_kv_heads, num_bins, min_tiles,
                          _ptr(m), n)
    if rc < 0:
        raise ValueError("orc_plan rejected its input (code %d)" % rc)
    return m


def parse_map(words, num_bins: int) -> dict:
    """Split task-map words into named arrays (the oracle's own reading)."""
    w = np.asarray(words, np.int32)
    B, Hkv = int(w[5]), int(w[6])
    S = B * Hkv
    o = 8
    d = {"T": int(w[0]), "P_eff": int(w[1]), "q": int(w[2]), "r": int(w[3]),
         "num_desc": int(w[4]), "B": B, "H_kv": Hkv, "err": int(w[7])}
    d["seq_lens"] = w[o:o + B]; o += B
    d["bin_desc_off"] = w[o:o + num_bins + 1]; o += num_bins + 1
    d["seg_desc_off"] = w[o:o + S + 1]; o += S + 1
    d["desc"] = w[o:o + 4 * (S + num_bins - 1)].reshape(-1, 4)[: d["num_desc"]]
    return d


def partials(q, k_pages, v_pages, page_table, task_map, num_bins, *, num_kv_heads,
             sm_scale, q_scale=None, k_scale=None, v_scale=None):
    """Per-descriptor partial (o [num_desc, R G, D], lse [num_desc, R G])
    following a task map."""
    x = _Inputs(q, k_pages, v_pages, page_table, num_kv_heads, sm_scale,
                q_scale, k_scale, v_scale)
    m = _c(task_map, np.int32)
    nd = int(m[4])
    po = np.zeros((max(nd, 1), x.R * x.G, x.D), np.float64)
    pl = np.zeros((max(nd, 1), x.R * x.G), np.float64)
    rc = _load().orc_partials(*x.args(), _ptr(m), int(num_bins), _ptr(po), _ptr(pl))
    if rc:
        raise RuntimeError("orc_partials failed")
    return po[:nd], pl[:nd]


def combine(task_map, num_bins, part_o, part_lse, *, num_q_heads, head_dim, q_rows=1):
    """Merge per-descriptor partials into (out [B, H_q, D], lse [B, H_q]),
    or [B, R, H_q, D] and [B, R, H_q] for q_rows = R > 1."""
    m = _c(task_map, np.int32)
    B, Hkv = int(m[5]), int(m[6])
    dims = _Dims(B, num_q_heads, Hkv, head_dim, 0, 0, 0, int(q_rows), 0.0)
    po = _c(part_o, np.float64)
    pl = _c(part_lse, np.float64)
    if po.size == 0:
        po = np.zeros((1,), np.float64)
        pl = np.zeros((1,), np.float64)
    lead = (B, num_q_heads) if q_rows == 1 else (B, int(q_rows), num_q_heads)
    out = np.zeros(lead + (head_dim,), np.float64)
    lse = np.zeros(lead, np.float64)
    rc = _load().orc_combine(ctypes.byref(dims), _ptr(m), int(num_bins), _ptr(po), _ptr(pl),
                             _ptr(out), _ptr(lse))
    if rc:
        raise RuntimeError("orc_combine failed")
    return out, lse


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def e4m3_encode(v: float) -> int:
    """Nearest OCP E4M3FN code (ties to even, saturating at +-448)."""
    return int(_load().orc_e4m3_encode(float(v)))


def prologue(qkv, positions, *, num_q_heads, num_kv_heads, head_dim, q_norm_w=None,
             k_norm_w=None, eps=1e-6, rope=True, rope_base=10000.0, hadamard=False):
    """The attention prologue for T tokens (qkv: uint16 bf16 bits
    [T, (H_q + 2 H_kv) * D]).  Returns a dict of fp64 values before rounding
    (q_val [T,H_q,D], k_val, v_val [T,H_kv,D]), fp8 scales (q_scale [T,H_q],
    k_scale, v_scale [T,H_kv]) and codes (q_code, k_code, v_code, uint8)."""
    qkv = _c(qkv, np.uint16)
    T = qkv.shape[0]
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    if qkv.size != T * (Hq + 2 * Hkv) * D:
        raise ValueError("qkv must be [T, (H_q + 2 H_kv) * D]")
    pos = _c(positions, np.int32)
    qw = _c(q_norm_w, np.float32)
    kw = _c(k_norm_w, np.float32)
    out = {
        "q_val": np.zeros((T, Hq, D)), "k_val": np.zeros((T, Hkv, D)),
        "v_val": np.zeros((T, Hkv, D)), "q_scale": np.zeros((T, Hq)),
        "k_scale": np.zeros((T, Hkv)), "v_scale": np.zeros((T, Hkv)),
        "q_code": np.zeros((T, Hq, D), np.uint8), "k_code": np.zeros((T, Hkv, D), np.uint8),
        "v_code": np.zeros((T, Hkv, D), np.uint8)}
    rc = _load().orc_prologue(T, Hq, Hkv, D, _ptr(qkv), _ptr(pos), _ptr(qw), _ptr(kw),
                              float(eps), 1 if rope else 0, float(rope_base),
                              1 if hadamard else 0,
                              *[_ptr(out[k]) for k in ("q_val", "k_val", "v_val", "q_scale",
                                                        "k_scale", "v_scale", "q_code",
                                                        "k_code", "v_code")])
    if rc:
        raise RuntimeError("orc_prologue failed")
    return out
