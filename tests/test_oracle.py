"""Pins for the fp64 attention oracle against things other than itself.

- numpy brute force: direct exp(s) / sum exp(s) over K/V gathered with numpy
  fancy indexing (no max subtraction, no page arithmetic shared with the oracle);
- torch float64 scaled_dot_product_attention (a library routine) on the Tiny
  workload;
- closed forms (q = 0, equal keys, constant V, one token, one dominant key);
- the split/merge identity of the log-sum-exp combine;
- the OCP E4M3FN code table via torch.float8_e4m3fn and the format's anchors.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from load_balanced_split_amd import workloads as wl

TILE = 64


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _random_problem(rng, lens, Hkv, G, D, fp8=False, scale=1.0):
    lens = np.asarray(lens, np.int32)
    pt, num_pages = wl.page_table(lens, seed=int(rng.integers(1 << 30)), spare_pages=3)
    B, Hq = lens.shape[0], Hkv * G
    qf = rng.standard_normal((B, Hq, D)) * scale
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


def _brute(p):
    """Decode attention by the textbook formula, in numpy fp64."""
    fp8 = p["q"].dtype == np.uint8
    dec = _e4m3_to_f64 if fp8 else _bits_to_f64
    q = dec(p["q"])
    K = dec(p["k_pages"])
    V = dec(p["v_pages"])
    if fp8:
        q = q * p["q_scale"][..., None]
        K = K * p["k_scale"][..., None]
        V = V * p["v_scale"][..., None]
    B, Hq, D = q.shape
    Hkv = p["num_kv_heads"]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(p["seq_lens"][b])
        t = np.arange(L)
        pages = p["page_table"][b][t // TILE]
        slots = t % TILE
        for j in range(Hq):
            h = j // G
            Kb = K[pages, h, slots, :]          # [L, D]
            Vb = V[pages, h, slots, :]
            s = p["sm_scale"] * (Kb @ q[b, j])
            e = np.exp(s)
            out[b, j] = (e[:, None] * Vb).sum(0) / e.sum()
            lse[b, j] = math.log(e.sum())
    return out, lse


def _oracle(p, **kw):
    return oracle.attention(p["q"], p["k_pages"], p["v_pages"], p["page_table"], p["seq_lens"],
                            num_kv_heads=p["num_kv_heads"], sm_scale=p["sm_scale"],
                            q_scale=p.get("q_scale"), k_scale=p.get("k_scale"),
                            v_scale=p.get("v_scale"), **kw)


# ---------------------------------------------------------------- decoders

def test_bf16_decoder_all_codes():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_decoder_matches_torch_and_format_anchors():
    table = oracle.e4m3_table()
    ref = _e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    ok = np.isnan(ref) == np.isnan(table)
    assert ok.all()
    fin = ~np.isnan(ref)
    assert (table[fin] == ref[fin]).all()
    # Anchors from the OCP 8-bit floating point definition of E4M3FN.
    assert table[0x7E] == 448.0 and table[0xFE] == -448.0
    assert table[0x38] == 1.0 and table[0xB8] == -1.0
    assert table[0x08] == 2.0 ** -6          # smallest normal
    assert table[0x01] == 2.0 ** -9          # smallest subnormal
    assert table[0x00] == 0.0 and math.copysign(1, table[0x80]) == -1
    assert np.isfinite(table[fin]).all() and np.nanmax(np.abs(table)) == 448.0


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_matches_numpy_brute_force(fp8, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 200, size=3)
    lens[0] = 1
    p = _random_problem(rng, lens, Hkv=2, G=3, D=16, fp8=fp8)
    out, lse = _oracle(p)
    ref_o, ref_l = _brute(p)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def test_attention_matches_torch_sdpa_on_tiny():
    prob = wl.make_problem("tiny", seed=0)
    p = dict(q=wl.as_numpy(prob.q), k_pages=wl.as_numpy(prob.k_pages[0]),
             v_pages=wl.as_numpy(prob.v_pages[0]), page_table=prob.page_table,
             seq_lens=prob.seq_lens, num_kv_heads=1, sm_scale=prob.sm_scale)
    out, lse = _oracle(p)
    q = prob.q.double()
    K = prob.k_pages[0].double()
    V = prob.v_pages[0].double()
    for b, L in enumerate(prob.seq_lens):
        t = torch.arange(int(L))
        pages = torch.from_numpy(prob.page_table[b]).long()[t // TILE]
        Kb = K[pages, 0, t % TILE].unsqueeze(0).expand(4, -1, -1)   # [H_q, L, D]
        Vb = V[pages, 0, t % TILE].unsqueeze(0).expand(4, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b].unsqueeze(1), Kb, Vb, scale=prob.sm_scale).squeeze(1)
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)
        s = prob.sm_scale * torch.einsum("hd,hld->hl", q[b], Kb)
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(7)
    D, Hkv, G = 32, 2, 2
    p = _random_problem(rng, [130, 1, 64], Hkv, G, D)
    # q = 0: uniform weights -> mean of V; lse = ln L.
    p0 = dict(p, q=np.zeros_like(p["q"]))
    out, lse = _oracle(p0)
    V = _bits_to_f64(p["v_pages"])
    for b, L in enumerate(p["seq_lens"]):
        t = np.arange(L)
        pages = p["page_table"][b][t // TILE]
        for j in range(Hkv * G):
            vb = V[pages, j // G, t % TILE]
            np.testing.assert_allclose(out[b, j], vb.mean(0), atol=1e-13)
            assert abs(lse[b, j] - math.log(L)) < 1e-13
    # Constant V rows -> output is that constant, whatever the weights.
    pc = dict(p, v_pages=np.full_like(p["v_pages"], _bf16_bits(np.array([0.375]))[0]))
    out, _ = _oracle(pc)
    np.testing.assert_allclose(out, 0.375, atol=1e-14)
    # One token (request 1): output is v_0 and lse is s_0.
    out, lse = _oracle(p)
    q = _bits_to_f64(p["q"])
    K = _bits_to_f64(p["k_pages"])
    pg = p["page_table"][1][0]
    for j in range(Hkv * G):
        np.testing.assert_allclose(out[1, j], V[pg, j // G, 0], atol=0)
        s0 = p["sm_scale"] * float(K[pg, j // G, 0] @ q[1, j])
        assert abs(lse[1, j] - s0) < 1e-12
    # All keys equal: uniform weights again, lse = s + ln L.
    kk = np.empty_like(p["k_pages"])
    kk[...] = p["k_pages"][0, 0, 0]
    pk = dict(p, k_pages=kk)
    out, lse = _oracle(pk)
    k0 = _bits_to_f64(p["k_pages"][0, 0, 0])
    for b, L in enumerate(p["seq_lens"]):
        t = np.arange(L)
        pages = p["page_table"][b][t // TILE]
        for j in range(Hkv * G):
            vb = V[pages, j // G, t % TILE]
            np.testing.assert_allclose(out[b, j], vb.mean(0), atol=1e-13)
            s = p["sm_scale"] * float(k0 @ q[b, j])
            assert abs(lse[b, j] - (s + math.log(L))) < 1e-12


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    D = 16
    p = _random_problem(rng, [100], 1, 1, D)
    q = _bits_to_f64(p["q"])[0, 0]
    t_star = 77
    pg = p["page_table"][0][t_star // TILE]
    kk = p["k_pages"].copy()
    kk[pg, 0, t_star % TILE] = _bf16_bits(q * 64.0)   # score ~ 64 |q|^2 / 4, far above the rest
    out, _ = _oracle(dict(p, k_pages=kk))
    V = _bits_to_f64(p["v_pages"])
    np.testing.assert_allclose(out[0, 0], V[pg, 0, t_star % TILE], atol=1e-9)


def test_empty_request_gives_zero_and_minus_inf():
    rng = np.random.default_rng(4)
    p = _random_problem(rng, [0, 5], 1, 2, 16)
    out, lse = _oracle(p)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    ref_o, _ = _brute(dict(p, seq_lens=np.array([5], np.int32), q=p["q"][1:],
                           page_table=p["page_table"][1:]))
    np.testing.assert_allclose(out[1], ref_o[0], atol=1e-12)


def test_pairs_subset_matches_full():
    rng = np.random.default_rng(5)
    p = _random_problem(rng, [70, 200, 3], 2, 2, 16)
    full, full_l = _oracle(p)
    part, part_l = _oracle(p, pairs=[(1, 1), (2, 0)])
    np.testing.assert_array_equal(part[1, 2:4], full[1, 2:4])
    np.testing.assert_array_equal(part[2, 0:2], full[2, 0:2])
    assert np.isnan(part[0]).all()


# ---------------------------------------------------------------- split identity

@pytest.mark.parametrize("fp8", [False, True])
def test_split_then_merge_equals_single_pass(fp8):
    rng = np.random.default_rng(11)
    p = _random_problem(rng, [777], 2, 4, 32, fp8=fp8)
    kw = dict(num_kv_heads=2, sm_scale=p["sm_scale"], q_scale=p.get("q_scale"),
              k_scale=p.get("k_scale"), v_scale=p.get("v_scale"))
    args = (p["q"], p["k_pages"], p["v_pages"], p["page_table"])
    for trial in range(20):
        h = int(rng.integers(2))
        cuts = np.sort(rng.integers(0, 778, size=int(rng.integers(0, 12))))
        edges = np.concatenate([[0], cuts, [777]])     # may hold empty ranges
        whole_o, whole_l = oracle.attend_range(*args, 0, h, 0, 777, **kw)
        parts = [oracle.attend_range(*args, 0, h, int(a), int(z), **kw)
                 for a, z in zip(edges[:-1], edges[1:])]
        for g in range(4):
            lse = np.array([pl[g] for _, pl in parts])
            o = np.stack([po[g] for po, _ in parts])
            m_o, m_l = oracle.lse_merge(lse, o)
            np.testing.assert_allclose(m_o, whole_o[g], rtol=0, atol=1e-12)
            assert abs(m_l - whole_l[g]) < 1e-12


def test_lse_merge_degenerate_cases():
    o, l = oracle.lse_merge(np.array([-np.inf, -np.inf]), np.ones((2, 3)))
    assert (o == 0).all() and l == -np.inf
    o, l = oracle.lse_merge(np.array([0.25]), np.array([[1.0, -2.0]]))
    assert (o == [1.0, -2.0]).all() and l == 0.25
    # Two equal-weight partials average; the lse adds ln 2.
    o, l = oracle.lse_merge(np.array([1.5, 1.5]), np.array([[1.0], [3.0]]))
    assert o[0] == 2.0 and abs(l - (1.5 + math.log(2))) < 1e-15


# ---------------------------------------------------------------- partitioned path

@pytest.mark.parametrize("P,m", [(1, 1), (3, 1), (8, 2), (16, 2), (64, 1), (7, 5)])
def test_plan_partials_combine_equals_single_pass(P, m):
    rng = np.random.default_rng(100 + P)
    p = _random_problem(rng, [17, 64, 200, 1000, 0, 65], 2, 2, 16)
    out, lse = _oracle(p)
    tm = oracle.plan(p["seq_lens"], 2, P, m)
    po, pl = oracle.partials(p["q"], p["k_pages"], p["v_pages"], p["page_table"], tm, P,
                             num_kv_heads=2, sm_scale=p["sm_scale"])
    c_o, c_l = oracle.combine(tm, P, po, pl, num_q_heads=4, head_dim=16)
    np.testing.assert_allclose(c_o, out, rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(c_l[fin], lse[fin], rtol=0, atol=1e-12)
    assert (np.isneginf(c_l) == ~fin).all()


def test_uniform_batch_invariant_to_bin_count():
    rng = np.random.default_rng(9)
    p = _random_problem(rng, [300] * 5, 2, 2, 16)
    ref = None
    for P in (1, 2, 5, 8, 13, 64):
        tm = oracle.plan(p["seq_lens"], 2, P, 1)
        po, pl = oracle.partials(p["q"], p["k_pages"], p["v_pages"], p["page_table"], tm, P,
                                 num_kv_heads=2, sm_scale=p["sm_scale"])
        o, _ = oracle.combine(tm, P, po, pl, num_q_heads=4, head_dim=16)
        if ref is None:
            ref = o
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
