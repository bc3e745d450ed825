"""Pins for the oracle's attention prologue (QK-Norm -> RoPE -> Hadamard ->
fp8 quantisation) against things other than itself:

- the E4M3FN encoder: every finite code round-trips, midpoints go to the
  even code, out-of-range values saturate, and it agrees with torch's
  float8_e4m3fn cast (a library routine) on random in-range values;
- RoPE: the same rotation written as complex multiplication
  z_i * exp(i pos theta_i) with numpy complex arithmetic; position 0 is the
  identity; rotations compose (a then b = a + b); q.k depends only on the
  position difference;
- Hadamard: scipy.linalg.hadamard (a library routine), and it is orthogonal;
- RMSNorm: with eps = 0 the output has unit RMS and is invariant to scaling
  the input; the weight multiplies element-wise;
- the quantised rows: the largest |value| maps to code +-448, every code is
  within half an E4M3 step of value / scale.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

TABLE = None


def table():
    global TABLE
    if TABLE is None:
        TABLE = oracle.e4m3_table()
    return TABLE


def bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bits_f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- encoder

def test_e4m3_encode_round_trips_every_finite_code():
    t = table()
    for c in range(256):
        if np.isnan(t[c]):
            continue
        got = oracle.e4m3_encode(t[c])
        assert t[got] == t[c], c          # +0/-0 may swap sign codes only as values


def test_e4m3_encode_ties_to_even_and_saturates():
    t = table()
    pos = [c for c in range(0x7F)]
    for c in pos[:-1]:
        mid = (t[c] + t[c + 1]) / 2
        got = oracle.e4m3_encode(mid)
        assert got in (c, c + 1) and got % 2 == 0, (c, mid, got)
        assert oracle.e4m3_encode(-mid) == got | 0x80
    assert oracle.e4m3_encode(448.0) == 0x7E and oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(-1e9) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00 and oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(2.0 ** -10) in (0x00, 0x01)   # half the smallest subnormal


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (0.01, 1.0, 30.0, 200.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], np.uint8)
    t = table()
    assert (t[got] == t[ref]).all()


# ---------------------------------------------------------------- prologue

def run(x, pos, Hq=2, Hkv=1, D=16, **kw):
    """x: float [T, Hq + 2 Hkv, D] -> oracle prologue on its bf16 rounding."""
    T = x.shape[0]
    bits = bf16_bits(x.reshape(T, -1))
    out = oracle.prologue(bits, np.asarray(pos, np.int32), num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=D, **kw)
    return bits_f64(bits).reshape(T, Hq + 2 * Hkv, D), out


def rope_complex(v, pos, base):
    """RoPE as complex multiplication of the pairs (i, i + D/2)."""
    D = v.shape[-1]
    half = D // 2
    theta = base ** (-2.0 * np.arange(half) / D)
    z = v[..., :half] + 1j * v[..., half:]
    z = z * np.exp(1j * pos * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("D", [16, 64, 128])
def test_rope_is_complex_rotation(D):
    rng = np.random.default_rng(D)
    x = rng.standard_normal((5, 4, D))
    pos = [0, 1, 17, 4095, 131071]
    xin, out = run(x, pos, Hq=2, Hkv=1, D=D, rope=True, rope_base=10000.0)
    for t, p in enumerate(pos):
        np.testing.assert_allclose(out["q_val"][t], rope_complex(xin[t, :2], p, 10000.0),
                                   rtol=0, atol=1e-9)
        np.testing.assert_allclose(out["k_val"][t, 0], rope_complex(xin[t, 2], p, 10000.0),
                                   rtol=0, atol=1e-9)
        np.testing.assert_array_equal(out["v_val"][t, 0], xin[t, 3])   # V untouched
    np.testing.assert_allclose(out["q_val"][0], xin[0, :2], atol=0)    # position 0


def test_rope_composes_and_is_relative():
    rng = np.random.default_rng(3)
    D = 32
    x = rng.standard_normal((1, 4, D))
    base = 500000.0
    _, a = run(x, [5], D=D, rope_base=base)
    # Composition: rotating the position-5 output by 7 more equals position 12.
    xb = bits_f64(bf16_bits(x)).reshape(1, 4, D)
    np.testing.assert_allclose(rope_complex(a["q_val"][0], 7, base),
                               rope_complex(xb[0, :2], 12, base), atol=1e-9)
    # q.k at positions (m, n) depends only on m - n.
    xx = np.repeat(x, 3, axis=0)
    _, b = run(xx, [10, 300, 9000], D=D, rope_base=base)
    _, c = run(xx, [0, 290, 8990], D=D, rope_base=base)
    # the same pair shifted: q at 10 with k at 300 vs q at 0 with k at 290
    d1 = b["q_val"][0, 0] @ b["k_val"][1, 0]
    d2 = c["q_val"][0, 0] @ c["k_val"][1, 0]
    assert abs(d1 - d2) < 1e-9


def test_hadamard_matches_scipy_and_is_orthogonal():
    rng = np.random.default_rng(4)
    for D in (16, 64, 128):
        x = rng.standard_normal((3, 4, D))
        xin, out = run(x, [0, 1, 2], D=D, rope=False, hadamard=True)
        H = scipy.linalg.hadamard(D) / math.sqrt(D)
        for t in range(3):
            np.testing.assert_allclose(out["q_val"][t], xin[t, :2] @ H.T, atol=1e-12)
            np.testing.assert_allclose(out["k_val"][t, 0], H @ xin[t, 2], atol=1e-12)
            np.testing.assert_allclose(np.linalg.norm(out["k_val"][t, 0]),
                                       np.linalg.norm(xin[t, 2]), rtol=1e-12)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(5)
    D = 64
    x = rng.standard_normal((2, 4, D))
    ones = np.ones(D, np.float32)
    _, a = run(x, [0, 0], D=D, rope=False, q_norm_w=ones, k_norm_w=ones, eps=0.0)
    rms = np.sqrt((a["q_val"] ** 2).mean(-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-12)
    _, b = run(x * 4.0, [0, 0], D=D, rope=False, q_norm_w=ones, k_norm_w=ones, eps=0.0)
    np.testing.assert_allclose(b["k_val"], a["k_val"], rtol=1e-12)   # scale invariance
    w = rng.uniform(0.5, 2.0, D).astype(np.float32)
    _, c = run(x, [0, 0], D=D, rope=False, q_norm_w=w, k_norm_w=ones, eps=0.0)
    np.testing.assert_allclose(c["q_val"], a["q_val"] * w.astype(np.float64), rtol=1e-12)
    np.testing.assert_allclose(c["k_val"], a["k_val"], rtol=0)          # K keeps its weight
    # eps keeps an all-zero row finite
    _, z = run(np.zeros((1, 4, D)), [3], D=D, q_norm_w=ones, k_norm_w=ones, eps=1e-6)
    assert (z["q_val"] == 0).all() and (z["q_scale"] == 1.0).all()
    assert (table()[z["q_code"]] == 0).all()    # +0 or -0 codes


def test_quantised_rows():
    rng = np.random.default_rng(6)
    D = 128
    x = rng.standard_normal((4, 4, D)) * rng.uniform(0.01, 50, (4, 4, 1))
    ones = np.ones(D, np.float32)
    _, o = run(x, [1, 2, 3, 4], D=D, q_norm_w=ones, k_norm_w=ones, hadamard=True)
    t = table()
    for name in ("q", "k", "v"):
        val, scale, code = o[name + "_val"], o[name + "_scale"], o[name + "_code"]
        amax = np.abs(val).max(-1)
        np.testing.assert_allclose(scale, amax / 448.0, rtol=1e-15)
        deq = t[code]
        assert np.isfinite(deq).all()
        assert (np.abs(deq).max(-1) == 448.0).all()
        # half of the local E4M3 step: 2^(e - 3) / 2 for |x| in [2^e, 2^(e+1)), min 2^-10
        y = val / scale[..., None]
        e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
        half_step = 2.0 ** (e - 4)
        assert (np.abs(deq - y) <= half_step * (1 + 1e-12)).all()
