"""A decode step captured in a HIP graph replays exactly like the eager calls.

The library enqueues kernels only (no memset, no copy, no sync), so a
captured plan -> decode -> combine must reproduce the eager result bit for
bit on every replay, with eager work on other inputs in between.
"""
import numpy as np
import pytest
import torch

from helpers import say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


@pytest.mark.parametrize("name,lens", [("tiny", None), ("mixed", [300, 4096, 17, 20000, 65]),
                                       ("fp8", [1000, 70, 5000]),
                                       ("mtp", [300, 4096, 17, 2000, 65]),
                                       ("mtp_fp8", [1000, 70, 5000])])
def test_graph_replay_matches_eager(R, name, lens):
    # mtp / mtp_fp8: 6 query rows of 8 heads, the shared-tile kernel with its
    # staging wave
    prob = wl.make_problem(name, seed=11, device="cuda", layers=2,
                           lens=None if lens is None else np.array(lens, np.int32))
    run = R.DecodeRunner(prob)
    # Eager reference for both layers.
    ref = []
    for layer in range(2):
        out, lse = run.run(layer)
        sync()
        ref.append((out.clone(), lse.clone()))
    other = R.DecodeRunner(wl.make_problem("tiny", seed=5, device="cuda"))

    g = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.graph(g):
        run.plan()
        for layer in range(2):
            run.decode(layer)
            run.combine()
            outs.append((run.out, run.out_lse))   # layer 1 overwrites; keep the last
    sync()
    for rep in range(4):
        run.out.zero_()
        run.out_lse.zero_()
        g.replay()
        sync()
        assert torch.equal(run.out, ref[1][0]), rep
        assert torch.equal(run.out_lse, ref[1][1]), rep
        other.run()            # eager work between replays
        sync()
    say(name, "graph replays match eager bit for bit")


def test_two_streams_at_once_match_one_after_the_other(R):
    """Two independent decode steps enqueued on two streams, their kernels
    free to overlap (bf16 one-row, and the fp8 fused call on the staging-wave
    kernel): each result equals the same step run alone.  The library keeps
    no state between calls that the two could share."""
    a = R.DecodeRunner(wl.make_problem("mixed", seed=21, device="cuda", layers=1,
                                       lens=wl.seq_lens("mixed", 21)[:24]))
    # 8 requests of 6 rows over 64 bins: a mean of 2 chunks per segment, so
    # the call fuses
    b = R.DecodeRunner(wl.make_problem("mtp_fp8", seed=22, device="cuda", layers=1,
                                       lens=wl.seq_lens("mtp_fp8", 22)[:8]), num_bins=64)
    a.run(0)
    b.plan()
    b.decode_combine(0)
    sync()
    ref_a, ref_b = a.out.clone(), b.out.clone()
    a.out.zero_()
    b.out.zero_()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    sync()
    for rep in range(3):
        a.plan(sa)
        b.plan(sb)
        a.decode(0, sa)
        b.decode_combine(0, sb)
        a.combine(sa)
        sync()
        assert torch.equal(a.out, ref_a) and torch.equal(b.out, ref_b), rep
        assert int(b.tickets.abs().sum().item()) == 0
        a.out.zero_()
        b.out.zero_()
        sync()
