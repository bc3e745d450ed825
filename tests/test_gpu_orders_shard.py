"""Parity of the heavy-tail batch in its two order checks and of one GPU's
head shard of the mixed batch, against the fp64 oracle, through the C ABI.

* Heavy-tail (120 requests of 1024 +- 10% and 8 of 65536 tokens) with the
  8 long requests first and last in the batch: plan -> decode -> combine and
  the fused decode + combine, in the benchmark's launch configuration
  (default bins and floor), and the static split-KV baseline at one point.
  The sample always holds the first and the last long request.
* The head shard of the mixed batch under tensor parallelism 8 ("HPC-Ops x
  SGLang", serving with 8-way tensor parallelism; each GPU holds 1 KV head
  and its 8 query heads): 64 mixed-length requests, one plan reused by two
  layers, both paths.  At 64 segments over the default bins every segment is
  cut into about 9 chunks, so the combine merges many partials.
Tolerances as everywhere: bf16 max-abs <= 2e-2, mean-abs <= 2e-3, LSE <= 2e-2.
"""
import numpy as np
import pytest

from helpers import compare, host_inputs, oracle_attention, rows_of, sample_pairs, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


def pairs_with_long(prob, n, seed):
    """n sampled (b, h) pairs plus the first and the last long request."""
    longs = np.flatnonzero(prob.seq_lens == prob.seq_lens.max())
    pairs = set(sample_pairs(prob, n, seed=seed))
    pairs.update({(int(longs[0]), 0), (int(longs[-1]), prob.workload.num_kv_heads - 1)})
    return sorted(pairs)


@pytest.mark.parametrize("name", ["heavy_tail_long_first", "heavy_tail_long_last"])
def test_heavy_tail_orders(R, name):
    prob = wl.make_problem(name, seed=0, device="cuda", layers=1)
    pairs = pairs_with_long(prob, 8, seed=4)
    say("case:", name, "long at", np.flatnonzero(prob.seq_lens == 65536).tolist(),
        "pairs", pairs)
    run = R.DecodeRunner(prob)
    ref_o, ref_l = oracle_attention(host_inputs(prob), pairs)
    rows = rows_of(pairs, prob.workload.group)
    run.plan()
    run.decode()
    run.combine()
    sync()
    compare(run.out, run.out_lse, ref_o, ref_l, rows, False, name + " two launches")
    run.out.fill_(float("nan"))
    run.decode_combine()
    sync()
    assert int(run.tickets.abs().sum().item()) == 0
    compare(run.out, run.out_lse, ref_o, ref_l, rows, False, name + " fused")
    run.static(0, 8)
    sync()
    compare(run.out, run.out_lse, ref_o, ref_l, rows, False, name + " static splits=8")


def test_heavy_tail_orders_share_one_balance(R):
    """The bins do not depend on where the long requests sit: every order has
    the same total, the same bin sizes and at most B H_kv + P - 1 chunks."""
    heads = []
    for name in ("heavy_tail", "heavy_tail_long_first", "heavy_tail_long_last"):
        prob = wl.make_problem(name, seed=0, device="cuda", layers=1)
        run = R.DecodeRunner(prob)
        run.plan()
        sync()
        words = run.task_map.words.cpu().numpy()
        say(name, "header", words[:8].tolist())
        heads.append(tuple(words[:4].tolist()))
        assert words[4] <= len(prob.seq_lens) * 8 + run.num_bins - 1
        del run, prob
    assert heads[0] == heads[1] == heads[2]


def test_mixed_head_shard(R):
    prob = wl.make_problem("mixed_shard", seed=0, device="cuda", layers=2)
    w = prob.workload
    assert (w.num_kv_heads, w.group, w.head_dim) == (1, 8, 128)
    pairs = sample_pairs(prob, 12, seed=5)
    run = R.DecodeRunner(prob)
    run.plan()
    sync()
    nd = run.num_desc()
    say("mixed shard: bins", run.num_bins, "chunks", nd, "per segment", nd / 64)
    rows = rows_of(pairs, w.group)
    for layer in range(2):   # one plan, two layers
        ref_o, ref_l = oracle_attention(host_inputs(prob, layer), pairs)
        run.decode(layer)
        run.combine()
        sync()
        compare(run.out, run.out_lse, ref_o, ref_l, rows, False, "shard layer %d" % layer)
        run.out.fill_(float("nan"))
        run.decode_combine(layer)
        sync()
        assert int(run.tickets.abs().sum().item()) == 0
        compare(run.out, run.out_lse, ref_o, ref_l, rows, False, "shard fused layer %d" % layer)
