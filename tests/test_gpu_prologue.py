"""Parity of the fused attention prologue (QK-Norm -> RoPE -> [Hadamard] ->
bf16 or fp8 with per-row scales, K/V stored into the paged cache) with the
fp64 oracle prologue on the same bf16 inputs.

bf16 outputs: within one bf16 rounding plus fp32 arithmetic error of the
oracle (|d| <= 2^-8 |x| + 1e-5).  fp8: scales within 1e-5 relative; each
code equals the oracle's nearest-even code, except where the oracle's
value / scale lies within fp32 error of the midpoint between two codes, where
either neighbour is accepted (the two sides compute value / scale in fp32 and
fp64 and may round a near-tie differently).  Cache slots that are not
written keep their bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import compare, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu

TABLE = None


def table():
    global TABLE
    if TABLE is None:
        TABLE = oracle.e4m3_table()
    return TABLE


@pytest.fixture(scope="module")
def H():
    from load_balanced_split_amd import hpcattn
    return hpcattn


def make_inputs(T, Hq, Hkv, D, num_pages, seed, scale=3.0):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rng = np.random.default_rng(seed)
    qkv = (torch.randn((T, (Hq + 2 * Hkv) * D), generator=gen, device="cuda") * scale) \
        .to(torch.bfloat16)
    pos = torch.from_numpy(rng.integers(0, 131072, size=T).astype(np.int32)).cuda()
    slots = rng.choice(num_pages * 64, size=T, replace=False).astype(np.int32)
    slots[1::7] = -1                                 # some tokens are not stored
    qw = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).cuda()
    kw = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).cuda()
    return qkv, pos, torch.from_numpy(slots).cuda(), qw, kw


def run_gpu(H, qkv, pos, slots, qw, kw, Hq, Hkv, D, num_pages, fp8, flags):
    T = qkv.shape[0]
    dims = H.hpcattn_prologue_dims(T, Hq, Hkv, D, num_pages,
                                   H.KV_FP8_E4M3 if fp8 else H.KV_BF16, flags, 1e-6, 10000.0)
    dt = torch.uint8 if fp8 else torch.bfloat16
    sentinel = 0x5A if fp8 else 0.3125
    q_out = torch.zeros((T, Hq, D), dtype=dt, device="cuda")
    kp = torch.full((num_pages, Hkv, 64, D), sentinel, dtype=dt, device="cuda")
    vp = torch.full((num_pages, Hkv, 64, D), sentinel, dtype=dt, device="cuda")
    sc = {}
    if fp8:
        sc = dict(q_scale=torch.zeros((T, Hq), device="cuda"),
                  k_scale=torch.full((num_pages, Hkv, 64), -1.0, device="cuda"),
                  v_scale=torch.full((num_pages, Hkv, 64), -1.0, device="cuda"))
    H.hpcattn_prologue(dims, qkv, pos, slots, q_out, kp, vp, q_norm_w=qw, k_norm_w=kw, **sc)
    sync()
    return q_out, kp, vp, sc


def check_codes(got, ref, val, scale, what):
    """got: GPU codes; ref: the oracle's codes; val, scale: the oracle's values."""
    t = table()
    y = val / scale[..., None]
    deq = t[got.astype(np.int64)]
    assert np.isfinite(deq).all(), what
    err_gpu = np.abs(deq - y)
    err_ref = np.abs(t[ref.astype(np.int64)] - y)     # the nearest code's error
    # fp32 error of a value scales with its row (|y| <= 448), not with y
    slack = 1e-5 * np.abs(y) + 2e-6 * 448.0
    ok = (got == ref) | (err_gpu <= err_ref + slack)
    if got.size == 0:
        return
    mism = float((got != ref).mean())
    say("%s: %d codes, %.4f%% differ from the oracle (all at near-ties)" % (what, got.size,
                                                                             100 * mism))
    assert ok.all(), what
    assert mism < 5e-3, what


CASES = [  # (T, Hq, Hkv, D, flags)
    (64, 8, 1, 128, 1), (64, 64, 8, 128, 1), (37, 4, 2, 64, 1), (50, 8, 2, 128, 3),
    (16, 4, 4, 64, 3), (33, 16, 2, 128, 0), (1, 2, 1, 64, 2),
    (1100, 16, 2, 128, 3), (1030, 8, 8, 64, 1),
    # large calls: thousands of workgroups, every flag path at D = 128 and 64
    (4099, 64, 8, 128, 3), (9001, 32, 8, 64, 1),
    # more than 256 heads: a token takes several workgroups of 16 waves
    (5, 256, 8, 128, 3), (3, 300, 2, 64, 1),
]


@pytest.mark.parametrize("T,Hq,Hkv,D,flags", CASES)
@pytest.mark.parametrize("fp8", [False, True])
def test_prologue_matches_oracle(H, T, Hq, Hkv, D, flags, fp8):
    check_against_oracle(H, T, Hq, Hkv, D, flags, fp8)


@pytest.mark.parametrize("T,Hq,Hkv,D,flags,norm", [
    (37, 8, 2, 128, 3, "none"), (20, 4, 4, 64, 1, "none"),
    (37, 8, 2, 128, 3, "q only"), (29, 16, 2, 64, 2, "k only")])
@pytest.mark.parametrize("fp8", [False, True])
def test_prologue_without_norm_weights(H, T, Hq, Hkv, D, flags, norm, fp8):
    """QK-Norm is skipped for a kind whose weights are NULL (no RMS factor)."""
    check_against_oracle(H, T, Hq, Hkv, D, flags, fp8, use_qw=norm == "q only",
                         use_kw=norm == "k only")


def check_against_oracle(H, T, Hq, Hkv, D, flags, fp8, use_qw=True, use_kw=True):
    num_pages = max(2, (T + 63) // 64 + 3)
    qkv, pos, slots, qw, kw = make_inputs(T, Hq, Hkv, D, num_pages, seed=T * 31 + D + flags)
    qw = qw if use_qw else None
    kw = kw if use_kw else None
    q_out, kp, vp, sc = run_gpu(H, qkv, pos, slots, qw, kw, Hq, Hkv, D, num_pages, fp8, flags)
    ref = oracle.prologue(wl.as_numpy(qkv), pos.cpu().numpy(), num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D,
                          q_norm_w=None if qw is None else qw.cpu().numpy(),
                          k_norm_w=None if kw is None else kw.cpu().numpy(), eps=1e-6,
                          rope=bool(flags & H.PROLOGUE_ROPE), rope_base=10000.0,
                          hadamard=bool(flags & H.PROLOGUE_HADAMARD))
    sl = slots.cpu().numpy()
    stored = np.nonzero(sl >= 0)[0]
    page, slot = sl[stored] // 64, sl[stored] % 64
    what = "T=%d Hq=%d Hkv=%d D=%d flags=%d %s" % (T, Hq, Hkv, D, flags, "fp8" if fp8 else "bf16")
    if not fp8:
        qg = q_out.float().cpu().numpy()
        assert (np.abs(qg - ref["q_val"]) <= 2.0 ** -8 * np.abs(ref["q_val"]) + 1e-5).all(), what
        kg = kp.float().cpu().numpy()[page, :, slot]
        vg = vp.float().cpu().numpy()[page, :, slot]
        kr, vr = ref["k_val"][stored], ref["v_val"][stored]
        assert (np.abs(kg - kr) <= 2.0 ** -8 * np.abs(kr) + 1e-5).all(), what
        np.testing.assert_array_equal(vg, vr)          # V passes through unchanged
        untouched = np.ones((num_pages, 64), bool)
        untouched[page, slot] = False
        assert (kp.float().cpu().numpy()[untouched[:, None, :].repeat(Hkv, 1)] == 0.3125).all()
        say(what, "bf16 ok")
        return
    qs = sc["q_scale"].cpu().numpy()
    np.testing.assert_allclose(qs, ref["q_scale"], rtol=1e-5)
    check_codes(q_out.cpu().numpy(), ref["q_code"], ref["q_val"], ref["q_scale"], what + " q")
    ks = sc["k_scale"].cpu().numpy()[page, :, slot]
    vs = sc["v_scale"].cpu().numpy()[page, :, slot]
    np.testing.assert_allclose(ks, ref["k_scale"][stored], rtol=1e-5)
    np.testing.assert_allclose(vs, ref["v_scale"][stored], rtol=1e-5)
    check_codes(kp.cpu().numpy()[page, :, slot], ref["k_code"][stored], ref["k_val"][stored],
                ref["k_scale"][stored], what + " k")
    check_codes(vp.cpu().numpy()[page, :, slot], ref["v_code"][stored], ref["v_val"][stored],
                ref["v_scale"][stored], what + " v")
    untouched = np.ones((num_pages, 64), bool)
    untouched[page, slot] = False
    assert (sc["k_scale"].cpu().numpy().transpose(0, 2, 1)[untouched] == -1.0).all()
    assert (kp.cpu().numpy().transpose(0, 2, 1, 3)[untouched] == 0x5A).all()


def test_prologue_then_decode_end_to_end(H):
    """A decode step: the prologue writes each request's new token (at
    position L_b - 1) into the fp8 cache and emits fp8 Q; then plan, decode
    and combine.  The oracle runs its own prologue on the same inputs, puts
    its own codes into a copy of the same starting cache, and computes the
    attention; the outputs agree within the fp8 tolerance."""
    from load_balanced_split_amd import runner
    lens = np.array([1, 65, 700, 3000, 64, 130], np.int32)
    w = wl.Workload("custom", None, 2, 16, 128, "fp8")
    prob = wl.make_problem("fp8", seed=12, device="cuda", lens=lens, workload=w)
    B, Hq, Hkv, D = len(lens), 16, 2, 128
    start_k = wl.as_numpy(prob.k_pages[0]).copy()
    start_v = wl.as_numpy(prob.v_pages[0]).copy()
    start_ks = wl.as_numpy(prob.k_scale[0]).copy()
    start_vs = wl.as_numpy(prob.v_scale[0]).copy()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    qkv = torch.randn((B, (Hq + 2 * Hkv) * D), generator=gen, device="cuda").to(torch.bfloat16)
    pos = torch.from_numpy(lens - 1).cuda()
    slot = np.array([prob.page_table[b, (L - 1) // 64] * 64 + (L - 1) % 64
                     for b, L in enumerate(lens)], np.int32)
    slots = torch.from_numpy(slot).cuda()
    qw = torch.ones(D, device="cuda")
    kw = torch.ones(D, device="cuda")
    dims = H.hpcattn_prologue_dims(B, Hq, Hkv, D, prob.num_pages, H.KV_FP8_E4M3,
                                   H.PROLOGUE_ROPE | H.PROLOGUE_HADAMARD, 1e-6, 10000.0)
    H.hpcattn_prologue(dims, qkv, pos, slots, prob.q, prob.k_pages[0], prob.v_pages[0],
                       q_norm_w=qw, k_norm_w=kw, q_scale=prob.q_scale, k_scale=prob.k_scale[0],
                       v_scale=prob.v_scale[0])
    run = runner.DecodeRunner(prob)
    out, lse = run.run()
    sync()
    # Oracle side, from the same starting cache and inputs only.
    ref = oracle.prologue(wl.as_numpy(qkv), lens - 1, num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=D, q_norm_w=np.ones(D, np.float32),
                          k_norm_w=np.ones(D, np.float32), eps=1e-6, rope=True,
                          rope_base=10000.0, hadamard=True)
    k, v, ks, vs = start_k, start_v, start_ks, start_vs
    for b in range(B):
        pg, sl = slot[b] // 64, slot[b] % 64
        k[pg, :, sl] = ref["k_code"][b]
        v[pg, :, sl] = ref["v_code"][b]
        ks[pg, :, sl] = ref["k_scale"][b]
        vs[pg, :, sl] = ref["v_scale"][b]
    ref_o, ref_l = oracle.attention(ref["q_code"], k, v, prob.page_table, lens,
                                    num_kv_heads=Hkv, sm_scale=prob.sm_scale,
                                    q_scale=ref["q_scale"].astype(np.float32), k_scale=ks,
                                    v_scale=vs)
    rows = [(b, j) for b in range(B) for j in range(Hq)]
    compare(out, lse, ref_o, ref_l, rows, True, "prologue + decode (fp8)")


@pytest.mark.parametrize("fp8", [False, True])
def test_prologue_with_no_tokens_writes_nothing(H, fp8):
    """T = 0 is a valid call that launches nothing: the cache keeps its bytes."""
    Hq, Hkv, D, num_pages = 8, 2, 128, 2
    qkv = torch.zeros((0, (Hq + 2 * Hkv) * D), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros((0,), dtype=torch.int32, device="cuda")
    slots = torch.zeros((0,), dtype=torch.int32, device="cuda")
    q_out, kp, vp, sc = run_gpu(H, qkv, pos, slots, None, None, Hq, Hkv, D, num_pages, fp8, 3)
    assert q_out.numel() == 0
    if fp8:
        assert (kp == 0x5A).all() and (vp == 0x5A).all()
        assert (sc["k_scale"] == -1.0).all() and (sc["v_scale"] == -1.0).all()
    else:
        assert (kp.float() == 0.3125).all() and (vp.float() == 0.3125).all()


@pytest.mark.parametrize("fp8", [False, True])
def test_prologue_into_pools_beyond_2gib(H, fp8):
    """KV stored into a pool of 2.6 GB (bf16, 20000 pages; fp8, 40000): the
    tokens' cache slots lie in the pool's upper half, so the byte offsets of
    the stores pass 2^31.  The stored K/V (values, or codes
    and scales) match the oracle, and every page no token was sent to keeps
    its sentinel."""
    T, Hq, Hkv, D = 512, 64, 8, 128
    flags = H.PROLOGUE_ROPE | H.PROLOGUE_HADAMARD
    num_pages = 40000 if fp8 else 20000
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    rng = np.random.default_rng(77)
    qkv = (torch.randn((T, (Hq + 2 * Hkv) * D), generator=gen, device="cuda") * 3.0) \
        .to(torch.bfloat16)
    pos = torch.from_numpy(rng.integers(0, 131072, size=T).astype(np.int32)).cuda()
    sl = rng.choice(np.arange(num_pages // 2 * 64, num_pages * 64), size=T,
                    replace=False).astype(np.int32)
    sl[1::7] = -1
    slots = torch.from_numpy(sl).cuda()
    qw = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).cuda()
    kw = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).cuda()
    q_out, kp, vp, sc = run_gpu(H, qkv, pos, slots, qw, kw, Hq, Hkv, D, num_pages, fp8, flags)
    pool_bytes = kp.numel() * kp.element_size()
    assert pool_bytes > (1 << 31), pool_bytes
    ref = oracle.prologue(wl.as_numpy(qkv), pos.cpu().numpy(), num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, q_norm_w=qw.cpu().numpy(),
                          k_norm_w=kw.cpu().numpy(), eps=1e-6, rope=True, rope_base=10000.0,
                          hadamard=True)
    stored = np.nonzero(sl >= 0)[0]
    page = torch.from_numpy((sl[stored] // 64).astype(np.int64)).cuda()
    slot = torch.from_numpy((sl[stored] % 64).astype(np.int64)).cuda()
    what = "pool of %.2f GB, %s" % (pool_bytes / 1e9, "fp8" if fp8 else "bf16")
    touched = torch.zeros(num_pages, dtype=torch.bool, device="cuda")
    touched[page] = True
    sentinel = 0x5A if fp8 else 0.3125
    assert bool((kp[~touched] == sentinel).all()) and bool((vp[~touched] == sentinel).all()), what
    if not fp8:
        kg = kp[page, :, slot].float().cpu().numpy()
        vg = vp[page, :, slot].float().cpu().numpy()
        kr, vr = ref["k_val"][stored], ref["v_val"][stored]
        assert (np.abs(kg - kr) <= 2.0 ** -8 * np.abs(kr) + 1e-5).all(), what
        np.testing.assert_array_equal(vg, vr)
    else:
        ks = sc["k_scale"][page, :, slot].cpu().numpy()
        vs = sc["v_scale"][page, :, slot].cpu().numpy()
        np.testing.assert_allclose(ks, ref["k_scale"][stored], rtol=1e-5)
        np.testing.assert_allclose(vs, ref["v_scale"][stored], rtol=1e-5)
        check_codes(kp[page, :, slot].cpu().numpy(), ref["k_code"][stored],
                    ref["k_val"][stored], ref["k_scale"][stored], what + " k")
        check_codes(vp[page, :, slot].cpu().numpy(), ref["v_code"][stored],
                    ref["v_val"][stored], ref["v_scale"][stored], what + " v")
    say(what, "ok")



@pytest.mark.parametrize("fp8", [False, True])
def test_prologue_graph_replays(H, fp8):
    """The prologue captured in a HIP graph: from the same starting buffers,
    every replay writes exactly what the eager call wrote (Q out, the cache
    pages, fp8 scales), with eager calls on the same buffers between
    replays."""
    T, Hq, Hkv, D = 300, 64, 8, 128
    flags = H.PROLOGUE_ROPE | H.PROLOGUE_HADAMARD
    num_pages = (T + 63) // 64 + 3
    qkv, pos, slots, qw, kw = make_inputs(T, Hq, Hkv, D, num_pages, seed=5)
    q0, k0, v0, s0 = run_gpu(H, qkv, pos, slots, qw, kw, Hq, Hkv, D, num_pages, fp8, flags)
    dims = H.hpcattn_prologue_dims(T, Hq, Hkv, D, num_pages,
                                   H.KV_FP8_E4M3 if fp8 else H.KV_BF16, flags, 1e-6, 10000.0)
    sentinel = 0x5A if fp8 else 0.3125
    q_out, kp, vp = torch.empty_like(q0), torch.empty_like(k0), torch.empty_like(v0)
    sc = {n: torch.empty_like(t) for n, t in s0.items()}

    def reset():   # the starting contents run_gpu gave the eager call
        q_out.zero_()
        kp.fill_(sentinel)
        vp.fill_(sentinel)
        for n, t in sc.items():
            t.fill_(0.0 if n == "q_scale" else -1.0)

    def call():
        H.hpcattn_prologue(dims, qkv, pos, slots, q_out, kp, vp, q_norm_w=qw, k_norm_w=kw, **sc)

    reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        reset()
        g.replay()
        sync()
        assert torch.equal(q_out, q0) and torch.equal(kp, k0) and torch.equal(vp, v0), i
        for n, t in sc.items():
            assert torch.equal(t, s0[n]), (n, i)
        reset()
        call()   # eager work on the same buffers between replays
        sync()
