"""Parity of the static split-KV ablation (both policies) with the oracle."""
import numpy as np
import pytest

from helpers import compare, host_inputs, oracle_attention, rows_of, sample_pairs, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


def all_pairs(prob):
    return [(b, h) for b in range(len(prob.seq_lens)) for h in range(prob.workload.num_kv_heads)]


@pytest.mark.parametrize("policy,param", [(0, 1), (0, 3), (0, 8), (0, 64), (1, 64), (1, 256),
                                          (1, 1024)])
def test_static_small(R, policy, param):
    lens = np.array([0, 1, 63, 64, 65, 1000, 2049, 300], np.int32)
    w = wl.Workload("custom", None, 2, 16, 128, "bf16")
    prob = wl.make_problem("tiny", seed=4, device="cuda", lens=lens, poison=True, workload=w)
    run = R.DecodeRunner(prob)
    # Empty splits write lse = -inf and no O row: NaN left in those rows must
    # not reach the output.
    run.static_buffers(policy, param)[0].fill_(float("nan"))
    run.static(policy, param)
    sync()
    h = host_inputs(prob)
    ref_o, ref_l = oracle_attention(h)
    compare(run.out, run.out_lse, ref_o, ref_l, rows_of(all_pairs(prob), 8), False,
            "static policy=%d param=%d" % (policy, param))


def test_static_fp8(R):
    lens = np.array([5, 640, 3001], np.int32)
    w = wl.Workload("custom", None, 2, 16, 128, "fp8")
    prob = wl.make_problem("fp8", seed=6, device="cuda", lens=lens, poison=True, workload=w)
    run = R.DecodeRunner(prob)
    for policy, param in ((0, 4), (1, 512)):
        run.static(policy, param)
        sync()
        h = host_inputs(prob)
        ref_o, ref_l = oracle_attention(h)
        compare(run.out, run.out_lse, ref_o, ref_l, rows_of(all_pairs(prob), 8), True,
                "static fp8 policy=%d" % policy)


def test_static_heavy_tail_full_size(R):
    prob = wl.make_problem("heavy_tail", seed=0, device="cuda")
    pairs = sample_pairs(prob, 8, seed=2)
    run = R.DecodeRunner(prob)
    h = host_inputs(prob)
    ref_o, ref_l = oracle_attention(h, pairs)
    for policy, param in ((0, 16), (1, 2048)):
        run.static(policy, param)
        sync()
        compare(run.out, run.out_lse, ref_o, ref_l, rows_of(pairs, 8), False,
                "heavy_tail static policy=%d param=%d" % (policy, param))
