"""hpcattn_decode_combine_noalloc through the C ABI: the allocation-free
decode + combine, whose partials and tickets live in the library's fixed
per-device scratch array, against hpcattn_decode_combine (the caller brings
those buffers) and against the fp64 oracle.

Calls follow each other on one device and share the array, so the cases run
in a row: a larger batch, then a smaller one (the second call must not see
the first call's partials as tickets), the larger one again (the tickets
were left at zero), the path that does not fuse (many chunks per segment),
a multi-row step on the staging-wave kernel, fp8, and replays of a captured
graph.  The fused
kernels and the merge order are the same in both calls, so the outputs are
compared for equality, and with the oracle at the parity tolerances (bf16
max-abs <= 2e-2, mean-abs <= 2e-3; fp8 max-abs <= 6e-2; LSE <= 2e-2).
"""
import numpy as np
import pytest
import torch

from helpers import compare, host_inputs, oracle_attention, rows_of, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from load_balanced_split_amd import hpcattn as H
    from load_balanced_split_amd import runner
    return H, runner


def workload(Hkv, G, D, kv="bf16", P=None, m=32, rows=1):
    return wl.Workload("custom", None, Hkv, Hkv * G, D, kv, num_bins=P, min_tiles=m,
                       q_rows=rows)


def noalloc(H, run, layer=0):
    """The allocation-free call into fresh NaN-filled outputs."""
    kv = run._kv(layer)
    out = torch.full_like(run.out, float("nan"))
    lse = torch.full_like(run.out_lse, float("nan"))
    H.hpcattn_decode_combine_noalloc(run.dims, run.prob.q, kv["k_pages"], kv["v_pages"],
                                     run.page_table, run.task_map, out, lse, kv.get("q_scale"),
                                     kv.get("k_scale"), kv.get("v_scale"))
    return out, lse


def check_case(M, prob, what, P=None, m=None):
    """Plan, then the caller-buffer call and the allocation-free call; equal
    outputs, both within the oracle's tolerance on every row."""
    H, R = M
    w = prob.workload
    say("case:", what, "B", len(prob.seq_lens), "lens", prob.seq_lens[:6].tolist())
    run = R.DecodeRunner(prob, num_bins=P, min_tiles=m)
    run.plan()
    ref_o, ref_l = [t.clone() for t in run.decode_combine(0)]
    out, lse = noalloc(H, run)
    sync()
    assert int(run.tickets.abs().sum().item()) == 0
    assert torch.equal(out, ref_o), what + ": out differs from hpcattn_decode_combine"
    assert torch.equal(torch.isnan(lse), torch.isnan(ref_l))
    fin = torch.isfinite(ref_l)
    assert torch.equal(lse[fin], ref_l[fin]), what + ": out_lse differs"
    o_ref, l_ref = oracle_attention(host_inputs(prob))
    B, Rr = len(prob.seq_lens), w.q_rows
    pairs = [(b, hh) for b in range(B) for hh in range(w.num_kv_heads)]
    if Rr == 1:
        compare(out, lse, o_ref, l_ref, rows_of(pairs, w.group), w.kv_dtype == "fp8", what)
    else:
        rows = [(b * Rr + r, hh * w.group + g) for b, hh in pairs for r in range(Rr)
                for g in range(w.group)]
        compare(out.view(B * Rr, w.num_q_heads, w.head_dim), lse.view(B * Rr, w.num_q_heads),
                o_ref.reshape(B * Rr, w.num_q_heads, w.head_dim),
                l_ref.reshape(B * Rr, w.num_q_heads), rows, w.kv_dtype == "fp8", what)
    return out, lse


def test_noalloc_matches_caller_buffers_in_a_row(M):
    lens_big = wl.seq_lens("mixed", 3)[:24]
    big = wl.make_problem("mixed", seed=3, device="cuda", layers=1, lens=lens_big, poison=True)
    o1, l1 = check_case(M, big, "larger batch (24 requests, 8 KV heads, fused)")
    small = wl.make_problem("tiny", seed=0, device="cuda", poison=True)
    check_case(M, small, "smaller batch (tiny, 4 requests, 1 KV head)", P=8, m=2)
    ragged = wl.make_problem("tiny", seed=5, device="cuda", poison=True,
                             lens=np.array([0, 1, 63, 64, 65, 1000, 0, 7], np.int32),
                             workload=workload(2, 8, 128, P=7, m=1))
    check_case(M, ragged, "ragged and empty requests, P = 7", P=7, m=1)
    o3, l3 = check_case(M, big, "larger batch again")
    assert torch.equal(o1, o3) and torch.equal(torch.isnan(l1), torch.isnan(l3))


def test_noalloc_unfused_paths_and_fp8(M):
    # one long request over 8 heads: 64 chunks per segment, decode then combine
    long_ = wl.make_problem("tiny", seed=1, device="cuda", poison=True,
                            lens=np.array([20000], np.int32), workload=workload(8, 8, 128))
    check_case(M, long_, "many chunks per segment (two launches)")
    mtp = wl.make_problem("tiny", seed=2, device="cuda", poison=True,
                          lens=np.array([6, 64, 70, 1000, 3000], np.int32),
                          workload=workload(2, 8, 128, rows=6, P=16, m=1))
    check_case(M, mtp, "6 rows of 8 heads (shared-tile kernel with a staging wave, fused)", P=16,
               m=1)
    fp8 = wl.make_problem("fp8", seed=4, device="cuda", poison=True,
                          lens=np.array([1, 64, 65, 500, 3000, 0, 129], np.int32),
                          workload=workload(2, 8, 128, "fp8", P=5, m=1))
    check_case(M, fp8, "fp8, P = 5", P=5, m=1)


def test_noalloc_graph_replays(M):
    H, R = M
    prob = wl.make_problem("mixed", seed=6, device="cuda", layers=1,
                           lens=wl.seq_lens("mixed", 6)[:16])
    run = R.DecodeRunner(prob)
    run.plan()
    eager_o, eager_l = noalloc(H, run)
    sync()
    out = torch.empty_like(eager_o)
    lse = torch.empty_like(eager_l)
    kv = run._kv(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        H.hpcattn_decode_combine_noalloc(run.dims, prob.q, kv["k_pages"], kv["v_pages"],
                                         run.page_table, run.task_map, out, lse)
    for i in range(4):
        out.zero_()
        g.replay()
        sync()
        assert torch.equal(out, eager_o), "replay %d" % i
        # eager work on the same array between replays
        noalloc(H, run)
        sync()
