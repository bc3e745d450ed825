"""Parity of multi-row decode (R query rows per request: the confirmed token
and R - 1 drafts, causal among themselves) with the fp64 oracle, through the
C ABI: plan -> decode -> combine, and the static split path.

The plan and task map are those of plain decode (the tile count comes from
L_b); one K/V tile serves all R G rows of its KV head.  Tolerances as for
plain decode: bf16 max-abs <= 2e-2, mean-abs <= 2e-3; fp8 max-abs <= 6e-2;
LSE <= 2e-2.  Rows that see no token (requests shorter than R) must give
exactly out = 0 and lse = -inf.  Dead KV slots hold NaN.
"""
import numpy as np
import pytest

from helpers import compare, host_inputs, oracle_attention, sample_pairs, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


def workload(Hkv, G, D, rows, kv="bf16", P=8, m=1):
    return wl.Workload("custom", None, Hkv, Hkv * G, D, kv, num_bins=P, min_tiles=m,
                       q_rows=rows)


def flat_rows(pairs, rows, G):
    """(b R + r, h G + g) rows of the [B R, H_q, D] view for (b, h) pairs."""
    return [(b * rows + r, h * G + g) for b, h in pairs for r in range(rows) for g in range(G)]


def check(out, lse, ref_o, ref_l, pairs, w, what):
    B, Rr = ref_o.shape[0], w.q_rows
    o = out.view(B * Rr, w.num_q_heads, w.head_dim)
    l = lse.view(B * Rr, w.num_q_heads)
    ro = ref_o.reshape(B * Rr, w.num_q_heads, w.head_dim)
    rl = ref_l.reshape(B * Rr, w.num_q_heads)
    rows = flat_rows(pairs, Rr, w.group)
    stats = compare(o, l, ro, rl, rows, w.kv_dtype == "fp8", what)
    # rows with no visible token: exactly zero output
    dead = [(i, j) for i, j in rows if np.isneginf(rl[i, j])]
    if dead:
        og = o.float().cpu().numpy()
        assert all((og[i, j] == 0).all() for i, j in dead), what
    return stats


def run_case(R, prob, what, P=None, m=None, pairs=None):
    w = prob.workload
    say("case:", what, "lens", prob.seq_lens[:10].tolist(), "B", len(prob.seq_lens),
        "rows", w.q_rows)
    run = R.DecodeRunner(prob, num_bins=P, min_tiles=m)
    run.run()
    sync()
    assert tuple(run.out.shape) == w.q_shape(len(prob.seq_lens))
    h = host_inputs(prob)
    ref_o, ref_l = oracle_attention(h, pairs)
    if pairs is None:
        pairs = [(b, hh) for b in range(len(prob.seq_lens)) for hh in range(w.num_kv_heads)]
    return check(run.out, run.out_lse, ref_o, ref_l, pairs, w, what), run


CASES = [  # (H_kv, G, D, R): R G = 6, 8, 16, 24, 48, 64 (1 to 4 column blocks)
    (2, 1, 64, 6), (2, 4, 64, 2), (2, 8, 128, 2), (2, 8, 128, 3), (2, 8, 128, 6),
    (1, 16, 128, 4), (2, 4, 64, 16), (3, 2, 128, 5),
]


@pytest.mark.parametrize("Hkv,G,D,rows", CASES)
def test_multi_row_ragged(R, Hkv, G, D, rows):
    # lengths below, at and just above R, ragged tails that end inside the
    # last R tokens, and whole pages
    lens = np.array([0, 1, rows - 1, rows, 64, 64 + rows - 2, 130, 1000, 2049], np.int32)
    lens = np.maximum(lens, 0)
    for P, m in ((1, 1), (7, 2), (64, 1)):
        prob = wl.make_problem("tiny", seed=P + rows, device="cuda", lens=lens, poison=True,
                               workload=workload(Hkv, G, D, rows))
        run_case(R, prob, "rows=%d Hkv=%d G=%d D=%d P=%d m=%d" % (rows, Hkv, G, D, P, m),
                 P=P, m=m)


@pytest.mark.parametrize("D,rows", [(64, 6), (128, 6), (128, 2)])
def test_multi_row_fp8(R, D, rows):
    lens = np.array([1, 64, 65, 500, 3000, 0, 129, rows], np.int32)
    for P in (1, 9, 64):
        prob = wl.make_problem("fp8", seed=P, device="cuda", lens=lens, poison=True,
                               workload=workload(2, 8, D, rows, "fp8"))
        run_case(R, prob, "fp8 rows=%d D=%d P=%d" % (rows, D, P), P=P, m=1)


def test_multi_row_sharp_softmax(R):
    lens = np.array([300, 4096, 17, 20000], np.int32)
    w = workload(8, 8, 128, 6)
    prob = wl.make_problem("mixed", seed=9, device="cuda", lens=lens, layers=1, q_mult=8.0,
                           poison=True, workload=w)
    stats, _ = run_case(R, prob, "rows=6 sharp softmax (Q x 8)", P=64, m=1)
    assert stats["rel_l2"] <= 2e-2


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("policy,param", [(0, 1), (0, 5), (1, 256), (1, 4096)])
def test_multi_row_static(R, policy, param, kv):
    lens = np.array([0, 3, 64, 70, 1000, 5000], np.int32)
    w = workload(2, 8, 128, 6, kv)
    prob = wl.make_problem("tiny", seed=param, device="cuda", lens=lens, poison=True,
                           workload=w)
    run = R.DecodeRunner(prob)
    run.static(policy, param)
    sync()
    ref_o, ref_l = oracle_attention(host_inputs(prob))
    pairs = [(b, h) for b in range(len(lens)) for h in range(2)]
    check(run.out, run.out_lse, ref_o, ref_l, pairs, w,
          "static %s rows=6 policy=%d param=%d" % (kv, policy, param))


@pytest.mark.parametrize("name,npairs", [("mtp", 8), ("mtp_fp8", 5)])
def test_full_size_multi_row_sampled(R, name, npairs):
    """The draft-verify workloads at full size in the benchmark's launch
    configuration; the oracle checks a seeded sample of (request, KV head)
    pairs including the longest request."""
    prob = wl.make_problem(name, seed=0, device="cuda", layers=1)
    pairs = sample_pairs(prob, npairs, seed=2)
    run = R.DecodeRunner(prob)
    run.run()
    sync()
    h = host_inputs(prob)
    ref_o, ref_l = oracle_attention(h, pairs)
    check(run.out, run.out_lse, ref_o, ref_l, pairs, prob.workload, name)
