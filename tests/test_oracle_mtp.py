"""Pins for the oracle's multi-row decode (R query rows per request: the
confirmed token and R - 1 drafts verified in one forward; row r sits at
position L - R + r and sees tokens [0, L - R + r]) against things other than
itself:

- numpy brute force: the [R, L] score matrix of each head with the causal
  mask built by np.triu, softmax by direct exp / sum;
- torch float64 scaled_dot_product_attention (a library routine) with the
  bottom-right causal mask from torch.tril;
- row r equals plain single-row decode over the first L - (R - 1 - r) tokens
  (catches a mask offset that is reversed or off by one);
- partials over any task map, merged by the combine, equal the single pass
  (including partials whose rows see no token, lse = -inf);
- closed forms for requests shorter than R: rows that see nothing give
  o = 0, lse = -inf; a row that sees one token gives that token's V;
- R = 1 given as a 4-D q equals the 3-D layout.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle import TILE, _bf16_bits, _bits_to_f64, _e4m3_to_f64
from load_balanced_split_amd import workloads as wl


def _problem(rng, lens, Hkv, G, D, R, fp8=False):
    lens = np.asarray(lens, np.int32)
    pt, num_pages = wl.page_table(lens, seed=int(rng.integers(1 << 30)), spare_pages=2)
    B, Hq = lens.shape[0], Hkv * G
    qf = rng.standard_normal((B, R, Hq, D)) * 2.0
    kf = rng.standard_normal((num_pages, Hkv, TILE, D))
    vf = rng.standard_normal((num_pages, Hkv, TILE, D))
    if not fp8:
        return dict(q=_bf16_bits(qf), k_pages=_bf16_bits(kf), v_pages=_bf16_bits(vf),
                    page_table=pt, seq_lens=lens, num_kv_heads=Hkv, sm_scale=1 / math.sqrt(D))
    q, qs = wl.quantize_e4m3(torch.from_numpy(qf).float())
    k, ks = wl.quantize_e4m3(torch.from_numpy(kf).float())
    v, vs = wl.quantize_e4m3(torch.from_numpy(vf).float())
    return dict(q=q.numpy(), k_pages=k.numpy(), v_pages=v.numpy(), q_scale=qs.numpy(),
                k_scale=ks.numpy(), v_scale=vs.numpy(), page_table=pt, seq_lens=lens,
                num_kv_heads=Hkv, sm_scale=1 / math.sqrt(D))


def _values(p):
    """fp64 q [B, R, Hq, D], K, V [num_pages, Hkv, 64, D]."""
    fp8 = p["q"].dtype == np.uint8
    dec = _e4m3_to_f64 if fp8 else _bits_to_f64
    q, K, V = dec(p["q"]), dec(p["k_pages"]), dec(p["v_pages"])
    if fp8:
        q = q * p["q_scale"][..., None]
        K = K * p["k_scale"][..., None]
        V = V * p["v_scale"][..., None]
    return q, K, V


def _gather(p, K, V, b, h):
    L = int(p["seq_lens"][b])
    t = np.arange(L)
    pages = p["page_table"][b][t // TILE]
    return K[pages, h, t % TILE, :], V[pages, h, t % TILE, :]


def _brute(p):
    """Masked-matrix attention in numpy: S = q K^T, mask = triu above the
    diagonal shifted by L - R, softmax by exp / sum."""
    q, K, V = _values(p)
    B, R, Hq, D = q.shape
    G = Hq // p["num_kv_heads"]
    out = np.zeros((B, R, Hq, D))
    lse = np.full((B, R, Hq), -np.inf)
    for b in range(B):
        L = int(p["seq_lens"][b])
        masked = np.triu(np.ones((R, L), bool), k=L - R + 1)   # t > L - R + r
        for j in range(Hq):
            Kb, Vb = _gather(p, K, V, b, j // G)
            S = p["sm_scale"] * (q[b, :, j, :] @ Kb.T)        # [R, L]
            E = np.where(masked, 0.0, np.exp(S))
            for r in range(R):
                z = E[r].sum()
                if z > 0:
                    out[b, r, j] = E[r] @ Vb / z
                    lse[b, r, j] = math.log(z)
    return out, lse


def _oracle(p, **kw):
    return oracle.attention(p["q"], p["k_pages"], p["v_pages"], p["page_table"], p["seq_lens"],
                            num_kv_heads=p["num_kv_heads"], sm_scale=p["sm_scale"],
                            q_scale=p.get("q_scale"), k_scale=p.get("k_scale"),
                            v_scale=p.get("v_scale"), **kw)


@pytest.mark.parametrize("R,G,fp8", [(2, 4, False), (3, 1, False), (6, 8, False),
                                     (4, 2, True), (6, 4, True)])
def test_multi_row_matches_brute_force(R, G, fp8):
    rng = np.random.default_rng(100 * R + G)
    lens = [R, 1, 0, 64, 65, 130, 64 + R - 1, 300]
    p = _problem(rng, lens, 2, G, 64, R, fp8)
    o, l = _oracle(p)
    bo, bl = _brute(p)
    assert o.shape == bo.shape and l.shape == bl.shape
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-11)
    fin = np.isfinite(bl)
    assert (np.isfinite(l) == fin).all()
    np.testing.assert_allclose(l[fin], bl[fin], rtol=0, atol=1e-11)


def test_multi_row_matches_torch_sdpa_with_causal_mask():
    rng = np.random.default_rng(7)
    R, G, Hkv, D = 5, 4, 2, 64
    lens = [5, 77, 200, 1000]
    p = _problem(rng, lens, Hkv, G, D, R)
    o, l = _oracle(p)
    q, K, V = _values(p)
    for b, L in enumerate(lens):
        mask = torch.ones(R, L, dtype=torch.bool).tril(diagonal=L - R)   # bottom-right causal
        for j in range(Hkv * G):
            Kb, Vb = _gather(p, K, V, b, j // G)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, :, j, :])[None], torch.from_numpy(Kb)[None],
                torch.from_numpy(Vb)[None], attn_mask=mask[None], scale=p["sm_scale"])[0]
            np.testing.assert_allclose(o[b, :, j], ref.numpy(), rtol=0, atol=1e-12)


def test_row_r_is_single_row_decode_over_its_prefix():
    rng = np.random.default_rng(8)
    R, G, Hkv, D = 4, 2, 2, 64
    lens = np.array([3, 64, 67, 129, 500], np.int32)
    p = _problem(rng, lens, Hkv, G, D, R)
    o, l = _oracle(p)
    for r in range(R):
        single = dict(p, q=np.ascontiguousarray(p["q"][:, r]),
                      seq_lens=np.maximum(lens - (R - 1 - r), 0).astype(np.int32))
        so, sl = _oracle(single)
        np.testing.assert_array_equal(o[:, r], so)
        np.testing.assert_array_equal(l[:, r], sl)
    # and the mask direction: the last row sees the whole request, the first
    # does not see the drafts after it
    full = dict(p, q=np.ascontiguousarray(p["q"][:, R - 1]))
    fo, _ = _oracle(full)
    np.testing.assert_array_equal(o[:, R - 1], fo)
    assert not np.allclose(o[1:, 0], fo[1:])


@pytest.mark.parametrize("P,m", [(1, 1), (3, 1), (8, 2), (40, 1), (16, 64)])
def test_multi_row_partials_combine_equal_single_pass(P, m):
    rng = np.random.default_rng(P * 7 + m)
    R, G, Hkv, D = 6, 2, 2, 64
    # tails of 1..R - 1 tokens put fully masked rows into one-tile partials
    lens = [64 * 3 + 2, 64 + 5, 0, 1, 64 * 7, 64 * 2 + 1, 6]
    p = _problem(rng, lens, Hkv, G, D, R)
    o, l = _oracle(p)
    tm = oracle.plan(p["seq_lens"], Hkv, P, m)
    po, pl = oracle.partials(p["q"], p["k_pages"], p["v_pages"], p["page_table"], tm, P,
                             num_kv_heads=Hkv, sm_scale=p["sm_scale"])
    assert po.shape[1:] == (R * G, D)
    if P >= 8:
        assert np.isneginf(pl).any()      # some partial rows see no token
    co, cl = oracle.combine(tm, P, po, pl, num_q_heads=Hkv * G, head_dim=D, q_rows=R)
    np.testing.assert_allclose(co, o, rtol=0, atol=1e-12)
    fin = np.isfinite(l)
    assert (np.isfinite(cl) == fin).all()
    np.testing.assert_allclose(cl[fin], l[fin], rtol=0, atol=1e-12)


def test_requests_shorter_than_rows_closed_form():
    rng = np.random.default_rng(9)
    R, G, Hkv, D = 4, 2, 1, 64
    p = _problem(rng, [0, 2], Hkv, G, D, R)
    o, l = _oracle(p)
    assert (o[0] == 0).all() and np.isneginf(l[0]).all()      # L = 0: nothing visible
    assert (o[1, :2] == 0).all() and np.isneginf(l[1, :2]).all()   # rows 0, 1 see nothing
    q, K, V = _values(p)
    Kb, Vb = _gather(p, K, V, 1, 0)
    for g in range(G):                                          # row 2 sees token 0 only
        np.testing.assert_array_equal(o[1, 2, g], Vb[0])
        assert l[1, 2, g] == pytest.approx(p["sm_scale"] * (q[1, 2, g] @ Kb[0]), abs=1e-12)


def test_one_row_in_4d_layout_equals_3d():
    rng = np.random.default_rng(10)
    p = _problem(rng, [17, 64, 200], 2, 4, 64, 1)
    o4, l4 = _oracle(p)
    p3 = dict(p, q=np.ascontiguousarray(p["q"][:, 0]))
    o3, l3 = _oracle(p3)
    np.testing.assert_array_equal(o4[:, 0], o3)
    np.testing.assert_array_equal(l4[:, 0], l3)
