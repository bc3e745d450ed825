"""Data errors never fault (include/hpcattn.h, conventions): a page id outside
[0, num_pages) or a tile past max_pages_per_req is skipped, and its tokens
contribute nothing.

The expected output is the oracle's attention over the same KV bytes with
those tiles taken out of the page table (and the lengths shortened by their
tokens).  Attention over a set of tokens does not depend on their order, so
removing a tile is the same as skipping it.  With several query rows per
request the causal mask is anchored at the end of the request, so there
only tiles before the last one are made invalid.
"""
import numpy as np
import pytest
import torch

from helpers import compare, host_inputs, oracle_attention, rows_of, say, sync
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


def clean_table(pt, lens, num_pages):
    """The page table and lengths without the tiles the kernels skip: tiles
    whose page id is outside [0, num_pages) and tiles past the table."""
    out = np.full_like(pt, -1)
    new_lens = lens.copy()
    for b in range(pt.shape[0]):
        L = int(lens[b])
        n = min((L + 63) // 64, pt.shape[1])
        valid = [t for t in range(n) if 0 <= pt[b, t] < num_pages]
        out[b, :len(valid)] = pt[b, valid]
        new_lens[b] = sum(min(64, L - 64 * t) for t in valid)
    return out, new_lens


def run_case(R, kv, rows, table_lens, bad_ids, beyond, what):
    """table_lens: lengths the page table is built for; bad_ids: {(b, tile):
    page id}; beyond: {b: extra tokens past the table}."""
    w = wl.Workload("custom", None, 2, 16, 128, kv, num_bins=16, min_tiles=1, q_rows=rows)
    prob = wl.make_problem("tiny", seed=5, device="cuda", lens=np.array(table_lens, np.int32),
                           workload=w)
    run = R.DecodeRunner(prob, num_bins=16, min_tiles=1)
    pt = prob.page_table.copy()
    lens = prob.seq_lens.copy()
    for (b, t), page in bad_ids.items():
        pt[b, t] = page
    for b, extra in beyond.items():
        lens[b] += extra
    run.page_table.copy_(torch.from_numpy(pt))
    run.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    say("case:", what, "lens", lens.tolist(), "bad", bad_ids, "beyond", beyond)
    run.run()
    sync()
    h = host_inputs(prob)
    h["page_table"], h["seq_lens"] = clean_table(pt, lens, prob.num_pages)
    assert (h["seq_lens"] < lens).any()   # some tokens really are skipped
    ref_o, ref_l = oracle_attention(h)
    if rows > 1:   # [B, R, H_q, ...] -> rows of [B R, H_q, ...]
        B = len(lens)
        out = run.out.view(B * rows, w.num_q_heads, w.head_dim)
        lse = run.out_lse.view(B * rows, w.num_q_heads)
        ref_o = ref_o.reshape(B * rows, w.num_q_heads, w.head_dim)
        ref_l = ref_l.reshape(B * rows, w.num_q_heads)
        pairs = [(b * rows + r, hh) for b in range(B) for r in range(rows) for hh in range(2)]
    else:
        out, lse = run.out, run.out_lse
        pairs = [(b, hh) for b in range(len(lens)) for hh in range(2)]
    compare(out, lse, ref_o, ref_l, rows_of(pairs, 8), kv == "fp8", what)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_bad_page_ids_and_lengths_past_the_table(R, kv):
    table = [1000, 200, 640, 256, 70]
    num_pages_hint = 10 ** 6   # any id at or past the pool size
    bad = {(0, 3): -5, (1, 0): num_pages_hint, (2, 9): num_pages_hint + 3}
    # request 0 runs 200 tokens past max_pages_per_req (16 pages), request 3
    # 100 tokens past its pages (into the table's -1 padding)
    run_case(R, kv, 1, table, bad, {0: 200, 3: 100}, "one row %s" % kv)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_bad_page_ids_multi_row(R, kv):
    # 6 rows of 8 heads: the shared-tile kernel with its staging wave
    table = [1000, 300, 640]
    bad = {(0, 3): -1, (0, 7): 1 << 30, (1, 1): -7, (2, 0): 1 << 29}
    run_case(R, kv, 6, table, bad, {}, "six rows %s" % kv)
