"""Host-side checks of the C ABI: no GPU needed, no kernel is launched.

Every call below fails validation on the host before anything is enqueued,
so fake (non-NULL) device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hpcattn.h")
LIB = os.path.join(ROOT, "load_balanced_split_amd", "libhpcattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhpcattn.so not built")


@pytest.fixture(scope="module")
def H():
    from load_balanced_split_amd import hpcattn
    return hpcattn


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hpcattn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(H):
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(H.EXPORTS)
    assert H.hpcattn_version() == 200


def test_size_queries_match_layout(H):
    for B, Hkv, P in [(1, 1, 1), (4, 1, 8), (64, 8, 512), (128, 8, 1024), (3, 2, 7)]:
        assert H.hpcattn_task_map_bytes(B, Hkv, P) == 4 * oracle.plan_words(B, Hkv, P)
        assert H.hpcattn_max_partials(B, Hkv, P) == B * Hkv + P - 1
    assert H.hpcattn_task_map_bytes(0, 1, 1) == 0
    assert H.hpcattn_max_partials(1, 0, 1) == 0
    assert H.hpcattn_static_max_partials(4, 2, 0, 8, 1000) == 64
    assert H.hpcattn_static_max_partials(4, 2, 1, 256, 1000) == 4 * 2 * 4
    assert H.hpcattn_static_max_partials(4, 2, 1, 100, 1000) == 0     # not a multiple of 64
    assert H.hpcattn_static_max_partials(4, 2, 2, 8, 1000) == 0       # unknown policy


FAKE = 0x10000   # never dereferenced: each call below is rejected first


def _map(H, B=4, Hkv=1, P=8, nbytes=None):
    if nbytes is None:
        nbytes = H.hpcattn_task_map_bytes(B, Hkv, P)
    return H.hpcattn_task_map(FAKE, nbytes, B, Hkv, P, 2)


def test_plan_rejects_bad_arguments(H):
    lib = H._lib
    m = _map(H)
    assert lib.hpcattn_plan(None, 4, 1, 8, 2, ctypes.byref(m), None) == H.ERR_NULL
    assert lib.hpcattn_plan(FAKE, 4, 1, 8, 2, None, None) == H.ERR_NULL
    assert lib.hpcattn_plan(FAKE, 0, 1, 8, 2, ctypes.byref(m), None) == H.ERR_SHAPE
    assert lib.hpcattn_plan(FAKE, H.MAX_BATCH + 1, 1, 8, 2, ctypes.byref(m), None) == H.ERR_SHAPE
    assert lib.hpcattn_plan(FAKE, 4, 0, 8, 2, ctypes.byref(m), None) == H.ERR_SHAPE
    assert lib.hpcattn_plan(FAKE, 4, 1, 0, 2, ctypes.byref(m), None) == H.ERR_SHAPE
    assert lib.hpcattn_plan(FAKE, 4, 1, 8, 0, ctypes.byref(m), None) == H.ERR_ARG
    small = _map(H, nbytes=H.hpcattn_task_map_bytes(4, 1, 8) - 4)
    assert lib.hpcattn_plan(FAKE, 4, 1, 8, 2, ctypes.byref(small), None) == H.ERR_WORKSPACE
    nowords = H.hpcattn_task_map(None, 1 << 20, 4, 1, 8, 2)
    assert lib.hpcattn_plan(FAKE, 4, 1, 8, 2, ctypes.byref(nowords), None) == H.ERR_NULL


def _dims(H, **kw):
    d = dict(batch=4, num_q_heads=4, num_kv_heads=1, head_dim=64, max_pages_per_req=16,
             num_pages=22, kv_dtype=H.KV_BF16, sm_scale=0.125, q_rows=1)
    d.update(kw)
    return H.hpcattn_dims(**d)


def _decode(H, dims, m, q_scale=None, k_scale=None, v_scale=None, rows=1 << 20, part=FAKE,
            ptrs=FAKE):
    return H._lib.hpcattn_decode(ctypes.byref(dims) if dims is not None else None, ptrs,
                                 q_scale, ptrs, ptrs, k_scale, v_scale, ptrs,
                                 ctypes.byref(m) if m is not None else None, part, part, rows,
                                 None)


def test_decode_rejects_bad_arguments(H):
    m = _map(H)
    assert _decode(H, None, m) == H.ERR_NULL
    assert _decode(H, _dims(H), None) == H.ERR_NULL
    assert _decode(H, _dims(H), m, ptrs=None) == H.ERR_NULL
    assert _decode(H, _dims(H), m, part=None) == H.ERR_NULL
    assert _decode(H, _dims(H, num_q_heads=6, num_kv_heads=4), m) == H.ERR_SHAPE   # H_q % H_kv
    assert _decode(H, _dims(H, num_q_heads=34, num_kv_heads=2), m) == H.ERR_SHAPE  # G > 16
    assert _decode(H, _dims(H, head_dim=96), m) == H.ERR_SHAPE
    assert _decode(H, _dims(H, num_pages=0), m) == H.ERR_SHAPE
    assert _decode(H, _dims(H, batch=5), m) == H.ERR_SHAPE        # map planned for B = 4
    assert _decode(H, _dims(H, kv_dtype=7), m) == H.ERR_DTYPE
    assert _decode(H, _dims(H), m, q_scale=FAKE) == H.ERR_DTYPE   # bf16 with scales
    assert _decode(H, _dims(H, kv_dtype=H.KV_FP8_E4M3), m, q_scale=FAKE,
                   k_scale=FAKE) == H.ERR_DTYPE                    # fp8 missing v_scale
    assert _decode(H, _dims(H, sm_scale=float("nan")), m) == H.ERR_ARG
    assert _decode(H, _dims(H, q_rows=0), m) == H.ERR_SHAPE       # at least one row
    assert _decode(H, _dims(H, q_rows=17), m) == H.ERR_SHAPE      # R G = 68 > 64 rows
    assert _decode(H, _dims(H, num_q_heads=16, q_rows=5), m) == H.ERR_SHAPE   # 80 rows
    # q_rows * G taken in int32 would wrap to 16 rows and pass: rejected, no launch
    assert _decode(H, _dims(H, num_q_heads=16, q_rows=2 ** 28 + 1), m) == H.ERR_SHAPE
    assert _decode(H, _dims(H, num_q_heads=16, q_rows=2 ** 31 - 1), m) == H.ERR_SHAPE
    assert _decode(H, _dims(H), m, rows=4 * 1 + 8 - 2) == H.ERR_WORKSPACE
    small = _map(H, nbytes=16)
    assert _decode(H, _dims(H), small) == H.ERR_WORKSPACE


def test_decode_combine_rejects_bad_arguments(H):
    lib = H._lib
    m = _map(H)   # B = 4, H_kv = 1, P = 8

    def dc(dims, tickets=FAKE, nt=4, out=FAKE, rows=1 << 20, mp=m):
        return lib.hpcattn_decode_combine(ctypes.byref(dims), FAKE, None, FAKE, FAKE, None, None,
                                          FAKE, ctypes.byref(mp), FAKE, FAKE, rows, tickets, nt,
                                          out, None, None)

    assert dc(_dims(H), tickets=None) == H.ERR_NULL
    assert dc(_dims(H), out=None) == H.ERR_NULL
    assert dc(_dims(H), nt=3) == H.ERR_WORKSPACE          # fewer tickets than B * H_kv
    assert dc(_dims(H), rows=4 + 8 - 2) == H.ERR_WORKSPACE
    assert dc(_dims(H, batch=5)) == H.ERR_SHAPE
    assert dc(_dims(H, q_rows=0)) == H.ERR_SHAPE
    assert dc(_dims(H, kv_dtype=H.KV_FP8_E4M3)) == H.ERR_DTYPE


def test_noalloc_rejects_bad_arguments_and_oversized_problems(H):
    lib = H._lib

    def na(dims, mp, out=FAKE, ptrs=FAKE):
        return lib.hpcattn_decode_combine_noalloc(ctypes.byref(dims), ptrs, None, ptrs, ptrs,
                                                  None, None, ptrs, ctypes.byref(mp), out, None,
                                                  None)

    m = _map(H)
    assert na(_dims(H), m, out=None) == H.ERR_NULL
    assert na(_dims(H), m, ptrs=None) == H.ERR_NULL
    assert na(_dims(H, batch=5), m) == H.ERR_SHAPE
    assert na(_dims(H, kv_dtype=H.KV_FP8_E4M3), m) == H.ERR_DTYPE
    assert na(_dims(H), _map(H, nbytes=16)) == H.ERR_WORKSPACE
    # partials of 8192 x 2 segments + 511 bins, 8 rows of D = 128: 67 MB > 32 MiB
    big = H.hpcattn_task_map(FAKE, H.hpcattn_task_map_bytes(8192, 2, 512), 8192, 2, 512, 1)
    assert na(_dims(H, batch=8192, num_q_heads=16, num_kv_heads=2, head_dim=128), big) == \
        H.ERR_WORKSPACE
    # more segments than tickets
    many = H.hpcattn_task_map(FAKE, H.hpcattn_task_map_bytes(8192, 9, 1), 8192, 9, 1, 1)
    assert na(_dims(H, batch=8192, num_q_heads=9, num_kv_heads=9, head_dim=64), many) == \
        H.ERR_WORKSPACE


def test_combine_and_static_reject_bad_arguments(H):
    lib = H._lib
    m = _map(H)
    d = _dims(H)
    assert lib.hpcattn_combine(ctypes.byref(d), ctypes.byref(m), FAKE, FAKE, None, None,
                               None) == H.ERR_NULL
    assert lib.hpcattn_combine(ctypes.byref(_dims(H, batch=3)), ctypes.byref(m), FAKE, FAKE,
                               FAKE, None, None) == H.ERR_SHAPE

    def st(dims, policy, param, max_len=1000, rows=1 << 20, seq=FAKE):
        return lib.hpcattn_static_decode(ctypes.byref(dims), policy, param, max_len, seq, FAKE,
                                         None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, rows,
                                         FAKE, None, None)

    assert st(d, 2, 8) == H.ERR_ARG
    assert st(d, 0, 0) == H.ERR_ARG
    assert st(d, 1, 100) == H.ERR_ARG
    assert st(d, 1, 256, max_len=-1) == H.ERR_ARG
    assert st(d, 0, 8, rows=4 * 8 - 1) == H.ERR_WORKSPACE
    assert st(d, 0, 8, seq=None) == H.ERR_NULL
    assert st(_dims(H, head_dim=32), 0, 8) == H.ERR_SHAPE


def test_suggest_and_probe_reject_bad_arguments(H):
    lib = H._lib
    assert lib.hpcattn_suggest_num_bins(96, H.KV_BF16, 8) == H.ERR_ARG
    assert lib.hpcattn_suggest_num_bins(128, 5, 8) == H.ERR_ARG
    assert lib.hpcattn_suggest_num_bins(128, H.KV_BF16, 65) == H.ERR_ARG
    assert lib.hpcattn_probe_stream_read(None, 1024, 8, 0, FAKE, None) == H.ERR_NULL
    assert lib.hpcattn_probe_stream_read(FAKE, 1000, 8, 0, FAKE, None) == H.ERR_ARG
    assert lib.hpcattn_probe_stream_read(FAKE, 1024, 0, 0, FAKE, None) == H.ERR_ARG
    assert lib.hpcattn_probe_stream_read(FAKE, 1024, 8, 4, FAKE, None) == H.ERR_ARG
    assert lib.hpcattn_probe_stream_read(FAKE, 3 * 16384, 8, 2, FAKE, None) == H.ERR_ARG


def test_prologue_rejects_bad_arguments(H):
    lib = H._lib

    def pro(fp8=False, scales=False, flags=1, eps=1e-6, base=10000.0, D=128, T=4, nulls=()):
        d = H.hpcattn_prologue_dims(T, 8, 2, D, 4, H.KV_FP8_E4M3 if fp8 else H.KV_BF16, flags,
                                    eps, base)
        ptr = {k: (None if k in nulls else FAKE) for k in
               ("qkv", "pos", "slots", "q", "k", "v")}
        sc = FAKE if scales else None
        return lib.hpcattn_prologue(ctypes.byref(d), ptr["qkv"], ptr["pos"], ptr["slots"],
                                    None, None, ptr["q"], sc, ptr["k"], ptr["v"], sc, sc, None)

    assert lib.hpcattn_prologue(None, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, FAKE,
                                None, None, None) == H.ERR_NULL
    assert pro(D=96) == H.ERR_SHAPE
    assert pro(T=-1) == H.ERR_SHAPE
    # no tokens: a no-op (no launch), NULL buffers accepted
    assert pro(T=0, nulls=("qkv", "pos", "slots", "q", "k", "v")) == H.OK
    assert pro(T=0, D=96) == H.ERR_SHAPE
    assert pro(flags=4) == H.ERR_ARG
    assert pro(eps=-1.0) == H.ERR_ARG
    assert pro(base=0.0) == H.ERR_ARG
    assert pro(nulls=("qkv",)) == H.ERR_NULL
    assert pro(nulls=("slots",)) == H.ERR_NULL
    assert pro(nulls=("pos",)) == H.ERR_NULL             # RoPE needs positions
    assert pro(fp8=True, scales=False) == H.ERR_DTYPE     # fp8 needs scales
    assert pro(fp8=False, scales=True) == H.ERR_DTYPE     # bf16 takes none
    # H_q + 2 H_kv taken in int32 would wrap negative and pass the row bound
    big = H.hpcattn_prologue_dims(4, 2 ** 31 - 1, 2 ** 30, 128, 4, H.KV_BF16, 1, 1e-6, 1e4)
    assert lib.hpcattn_prologue(ctypes.byref(big), FAKE, FAKE, FAKE, None, None, FAKE, None,
                                FAKE, FAKE, None, None, None) == H.ERR_SHAPE

    def shape(T, Hq, Hkv):
        d = H.hpcattn_prologue_dims(T, Hq, Hkv, 128, 4, H.KV_BF16, 1, 1e-6, 1e4)
        return lib.hpcattn_prologue(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, None,
                                    FAKE, FAKE, None, None, None)
    # one token with more heads than the kernel indexes in int32
    assert shape(1, 2 ** 31 - 1, 1) == H.ERR_SHAPE
    assert shape(1, H.PROLOGUE_MAX_HEADS - 1, 1) == H.ERR_SHAPE
    # the grid's extent: T * 64 * min(ceil(heads / 16), 16) work-items below 2^32
    assert shape(2 ** 22, 240, 8) == H.ERR_SHAPE         # 256 heads: 16 waves per token
    assert shape(13421773, 64, 8) == H.ERR_SHAPE         # 80 heads: 5 waves per token


def test_strerror_covers_every_status(H):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert H.hpcattn_strerror(code) != "unknown status"
    assert H.hpcattn_strerror(-99) == "unknown status"



def test_binding_constants_match_the_header(H):
    """Every integer #define of include/hpcattn.h (HPCATTN_X) that the Python
    binding mirrors as X has the same value there."""
    text = open(os.path.join(ROOT, "include", "hpcattn.h")).read()
    seen = 0
    for m in re.finditer(r"^#define HPCATTN_(\w+) +([^/\n]+?)\s*(?:/\*.*)?$", text, re.M):
        name, expr = m.group(1), re.sub(r"(\d+)u\b", r"\1", m.group(2))
        if re.fullmatch(r"[\d()< ]+", expr) and hasattr(H, name):
            assert getattr(H, name) == eval(expr), name
            seen += 1
    assert seen >= 8, seen
