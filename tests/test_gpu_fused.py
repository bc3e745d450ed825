"""Parity of hpcattn_decode_combine (decode and combine in one launch) with
the fp64 oracle, through the C ABI.

The fused call writes a one-chunk segment's output directly and has the last
workgroup of a multi-chunk segment merge its partials (a per-segment ticket),
in the one-row kernel and in the shared-tile multi-row kernels (with and
without a staging wave).  Where fusing does not pay (a mean of 8 or more
chunks per segment) the call runs decode and combine as two launches; the
cases below cover both (small P relative to the segments fuse, large P does
not).
Checked here: the oracle tolerances of plain decode (bf16 max-abs <= 2e-2,
mean-abs <= 2e-3; fp8 max-abs <= 6e-2; LSE <= 2e-2) on ragged and empty
requests, one and many chunks per segment, several bins counts, multi-row
steps and fp8; agreement with the two-launch path; the tickets back at zero
after every call, over many layers and graph replays; and workspace errors.
"""
import numpy as np
import pytest
import torch

from helpers import compare, host_inputs, oracle_attention, rows_of, sample_pairs, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


def workload(Hkv, G, D, kv="bf16", P=8, m=1, rows=1):
    return wl.Workload("custom", None, Hkv, Hkv * G, D, kv, num_bins=P, min_tiles=m,
                       q_rows=rows)


def check(out, lse, ref_o, ref_l, pairs, w, what):
    """Compare over (b, h) pairs, flattening the R axis of multi-row steps."""
    B, Rr = ref_o.shape[0], w.q_rows
    if Rr == 1:
        return compare(out, lse, ref_o, ref_l, rows_of(pairs, w.group), w.kv_dtype == "fp8", what)
    o = out.view(B * Rr, w.num_q_heads, w.head_dim)
    l = lse.view(B * Rr, w.num_q_heads)
    ro = ref_o.reshape(B * Rr, w.num_q_heads, w.head_dim)
    rl = ref_l.reshape(B * Rr, w.num_q_heads)
    rows = [(b * Rr + r, h * w.group + g) for b, h in pairs for r in range(Rr)
            for g in range(w.group)]
    return compare(o, l, ro, rl, rows, w.kv_dtype == "fp8", what)


def run_fused(R, prob, what, P=None, m=None):
    w = prob.workload
    say("case:", what, "lens", prob.seq_lens[:10].tolist(), "B", len(prob.seq_lens))
    run = R.DecodeRunner(prob, num_bins=P, min_tiles=m)
    run.out.fill_(float("nan"))          # every row must be written
    run.out_lse.fill_(float("nan"))
    run.plan()
    run.decode_combine()
    sync()
    assert int(run.tickets.abs().sum().item()) == 0, what + ": tickets not reset"
    h = host_inputs(prob)
    ref_o, ref_l = oracle_attention(h)
    pairs = [(b, hh) for b in range(len(prob.seq_lens)) for hh in range(w.num_kv_heads)]
    return check(run.out, run.out_lse, ref_o, ref_l, pairs, w, what), run


SHAPES = [(1, 4, 64), (2, 8, 128), (1, 16, 128), (3, 3, 128)]


@pytest.mark.parametrize("Hkv,G,D", SHAPES)
def test_fused_ragged_lengths(R, Hkv, G, D):
    # empty, one-token, whole-page and long requests; P from one bin (every
    # segment one chunk) to many (long segments in many chunks)
    lens = np.array([0, 1, 63, 64, 65, 127, 1000, 2049, 7, 0], np.int32)
    for P, m in ((1, 1), (7, 3), (64, 1), (300, 1)):
        prob = wl.make_problem("tiny", seed=P, device="cuda", lens=lens, poison=True,
                               workload=workload(Hkv, G, D, P=P, m=m))
        run_fused(R, prob, "fused Hkv=%d G=%d D=%d P=%d m=%d" % (Hkv, G, D, P, m), P=P, m=m)


@pytest.mark.parametrize("D", [64, 128])
def test_fused_fp8(R, D):
    lens = np.array([1, 64, 65, 500, 3000, 0, 129], np.int32)
    for P in (1, 5, 64):
        prob = wl.make_problem("fp8", seed=P, device="cuda", lens=lens, poison=True,
                               workload=workload(2, 8, D, "fp8", P=P))
        run_fused(R, prob, "fused fp8 D=%d P=%d" % (D, P), P=P, m=1)


@pytest.mark.parametrize("G,rows,kv", [(8, 2, "bf16"), (8, 6, "bf16"), (16, 4, "bf16"),
                                       (8, 3, "fp8"), (8, 6, "fp8")])
def test_fused_multi_row(R, G, rows, kv):
    lens = np.array([0, 1, rows, 64, 64 + rows - 2, 130, 1000, 2049], np.int32)
    for P in (1, 9, 64):
        prob = wl.make_problem("tiny", seed=P + rows, device="cuda", lens=lens, poison=True,
                               workload=workload(2, G, 128, kv, P=P, rows=rows))
        run_fused(R, prob, "fused rows=%d G=%d %s P=%d" % (rows, G, kv, P), P=P, m=1)


def test_fused_matches_two_launches_over_layers(R):
    """Mixed lengths, the default bins and floor, several layers with one
    plan: the fused call agrees with decode + combine (the merge order
    differs, so within a few bf16 ulps), and its tickets stay at zero."""
    prob = wl.make_problem("mixed", seed=3, device="cuda", layers=3,
                           lens=wl.seq_lens("mixed", 3)[:24])
    run = R.DecodeRunner(prob)
    run.plan()
    for layer in range(3):
        run.decode(layer)
        run.combine()
        ref_o, ref_l = run.out.clone(), run.out_lse.clone()
        run.decode_combine(layer)
        sync()
        assert int(run.tickets.abs().sum().item()) == 0
        d = (run.out.float() - ref_o.float()).abs().max().item()
        dl = (run.out_lse - ref_l).abs().max().item()
        say("layer %d: fused vs two launches max |out| diff %.3g, |lse| diff %.3g" % (layer, d, dl))
        assert d <= 2e-2 and dl <= 1e-4


@pytest.mark.parametrize("G,rows,kv", [(8, 6, "bf16"), (8, 6, "fp8"), (16, 4, "bf16"),
                                       (8, 3, "bf16")])
def test_fused_multi_row_matches_two_launches(R, G, rows, kv):
    """Multi-row steps on the shared-tile kernels (2 to 4 column blocks, the
    staging-wave instance at 6 rows of 8 heads): the fused call agrees with
    decode + combine over two layers on one plan, one- and many-chunk
    segments alike, and leaves its tickets at zero."""
    lens = wl.seq_lens("mixed", 5)[:12]
    prob = wl.make_problem("mixed", seed=5, device="cuda", layers=2, lens=lens, poison=True,
                           workload=workload(2, G, 128, kv, P=40, m=1, rows=rows))
    run = R.DecodeRunner(prob, num_bins=40, min_tiles=1)
    run.plan()
    for layer in range(2):
        run.decode(layer)
        run.combine()
        ref_o, ref_l = run.out.clone(), run.out_lse.clone()
        run.out.fill_(float("nan"))
        run.decode_combine(layer)
        sync()
        assert int(run.tickets.abs().sum().item()) == 0
        d = (run.out.float() - ref_o.float()).abs().max().item()
        dl = (run.out_lse - ref_l).abs().max().item()
        say("rows=%d G=%d %s layer %d: fused vs two launches |out| %.3g |lse| %.3g"
            % (rows, G, kv, layer, d, dl))
        assert d <= 2e-2 and dl <= 1e-4


def test_fused_multi_row_graph_replays(R):
    """The fused draft-verify step (6 rows of 8 heads, staging-wave kernel)
    captured in a HIP graph: every replay equals eager, with eager work
    between replays, and the tickets stay at zero."""
    lens = wl.seq_lens("mixed", 7)[:10]
    prob = wl.make_problem("mixed", seed=7, device="cuda", layers=2, lens=lens,
                           workload=workload(8, 8, 128, P=64, m=1, rows=6))
    run = R.DecodeRunner(prob, num_bins=64, min_tiles=1)
    run.plan()
    run.decode_combine(1)
    sync()
    eager = run.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.plan()
        run.decode_combine(0)
        run.decode_combine(1)
    for i in range(4):
        run.out.zero_()
        g.replay()
        sync()
        assert torch.equal(run.out, eager), "replay %d" % i
        assert int(run.tickets.abs().sum().item()) == 0
        run.decode_combine(0)
        sync()


def test_fused_graph_replays(R):
    """The fused step captured in a HIP graph: every replay equals eager."""
    lens = wl.seq_lens("mixed", 4)[:16]
    prob = wl.make_problem("mixed", seed=4, device="cuda", layers=2, lens=lens)
    run = R.DecodeRunner(prob)
    run.plan()
    run.decode_combine(1)
    sync()
    eager = run.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.plan()
        run.decode_combine(0)
        run.decode_combine(1)
    for i in range(4):
        run.out.zero_()
        g.replay()
        sync()
        assert torch.equal(run.out, eager), "replay %d" % i
        assert int(run.tickets.abs().sum().item()) == 0


@pytest.mark.parametrize("name,npairs", [("mixed", 8), ("single_long", 8), ("heavy_tail", 8),
                                         ("mtp", 6)])
def test_fused_full_size_sampled(R, name, npairs):
    """Full-size workloads in the benchmark's launch configuration, sampled
    against the oracle."""
    prob = wl.make_problem(name, seed=0, device="cuda", layers=1)
    pairs = sample_pairs(prob, npairs, seed=3)
    run = R.DecodeRunner(prob)
    run.plan()
    run.decode_combine()
    sync()
    assert int(run.tickets.abs().sum().item()) == 0
    ref_o, ref_l = oracle_attention(host_inputs(prob), pairs)
    check(run.out, run.out_lse, ref_o, ref_l, pairs, prob.workload, "fused " + name)


def test_fused_rejects_small_ticket_buffer(R):
    from load_balanced_split_amd import hpcattn as H
    prob = wl.make_problem("tiny", seed=0, device="cuda")
    run = R.DecodeRunner(prob)
    run.plan()
    small = torch.zeros(len(prob.seq_lens) * prob.workload.num_kv_heads - 1, dtype=torch.int32,
                        device="cuda")
    with pytest.raises(H.HpcattnError) as e:
        H.hpcattn_decode_combine(run.dims, prob.q, prob.k_pages[0], prob.v_pages[0],
                                 run.page_table, run.task_map, run.part_o, run.part_lse, small,
                                 run.out, run.out_lse)
    assert e.value.status == H.ERR_WORKSPACE
