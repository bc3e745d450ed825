"""Parity of the dynamic decode path (plan -> decode -> combine, through the C
ABI) with the fp64 oracle, on the same bytes.

Tolerances: bf16 KV max-abs <= 2e-2 and mean-abs <= 2e-3; fp8 KV max-abs
<= 6e-2 (the oracle decodes the same e4m3 bytes and scales); LSE <= 2e-2.
Dead KV slots past each length hold NaN, so any read of them fails a test.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import (compare, host_inputs, oracle_attention, rows_of, sample_pairs, say,
                     sync)
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from load_balanced_split_amd import runner
    return runner


def custom_workload(Hkv, G, D, kv="bf16", P=8, m=1):
    return wl.Workload("custom", None, Hkv, Hkv * G, D, kv, num_bins=P, min_tiles=m)


def run_and_compare(R, prob, what, P=None, m=None, pairs=None, layer=0):
    say("case:", what, "lens", prob.seq_lens[:8].tolist(), "B", len(prob.seq_lens))
    run = R.DecodeRunner(prob, num_bins=P, min_tiles=m)
    run.plan()
    run.decode(layer)
    run.combine()
    sync()
    h = host_inputs(prob, layer)
    ref_o, ref_l = oracle_attention(h, pairs)
    G = prob.workload.group
    if pairs is None:
        pairs = [(b, hh) for b in range(len(prob.seq_lens)) for hh in range(prob.workload.num_kv_heads)]
    return compare(run.out, run.out_lse, ref_o, ref_l, rows_of(pairs, G),
                   prob.workload.kv_dtype == "fp8", what), run


def test_tiny_end_to_end(R):
    for P, m in ((8, 2), (16, 2), (1, 1), (64, 1)):
        prob = wl.make_problem("tiny", seed=0, device="cuda", poison=True)
        run_and_compare(R, prob, "tiny P=%d m=%d" % (P, m), P=P, m=m)


def test_tiny_partials_match_oracle_partials(R):
    prob = wl.make_problem("tiny", seed=1, device="cuda", poison=True)
    run = R.DecodeRunner(prob)
    run.plan()
    run.decode()
    sync()
    words = run.task_map.words.cpu().numpy()
    P = run.num_bins
    assert words.tolist() == oracle.plan(prob.seq_lens, 1, P, run.min_tiles).tolist()
    h = host_inputs(prob)
    po, pl = oracle.partials(h["q"], h["k_pages"], h["v_pages"], h["page_table"], words, P,
                             num_kv_heads=1, sm_scale=prob.sm_scale)
    nd = int(words[4])
    go = run.part_o[:nd].cpu().numpy().astype(np.float64)
    gl = run.part_lse[:nd].cpu().numpy().astype(np.float64)
    err_o = np.abs(go - po).max(axis=(1, 2))
    err_l = np.abs(gl - pl).max(axis=1)
    say("per-descriptor max |o| err", np.round(err_o, 5).tolist())
    say("per-descriptor max |lse| err", np.round(err_l, 5).tolist())
    assert err_o.max() <= 1e-2 and err_l.max() <= 1e-2


SHAPES = [  # (H_kv, G, D)
    (1, 1, 64), (2, 4, 64), (2, 8, 128), (1, 16, 128), (2, 16, 64), (3, 3, 128), (8, 8, 128),
]


@pytest.mark.parametrize("Hkv,G,D", SHAPES)
def test_random_shapes_and_ragged_lengths(R, Hkv, G, D):
    lens = np.array([0, 1, 63, 64, 65, 127, 1000, 2049, 7], np.int32)
    for P, m in ((1, 1), (7, 3), (64, 1), (300, 2)):
        prob = wl.make_problem("tiny", seed=P, device="cuda", lens=lens, poison=True,
                               workload=custom_workload(Hkv, G, D))
        run_and_compare(R, prob, "shape Hkv=%d G=%d D=%d P=%d m=%d" % (Hkv, G, D, P, m),
                        P=P, m=m)


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_small_parity(R, D):
    lens = np.array([1, 64, 65, 500, 3000, 0, 129], np.int32)
    for P in (1, 5, 64):
        prob = wl.make_problem("fp8", seed=P, device="cuda", lens=lens, poison=True,
                               workload=custom_workload(2, 8, D, "fp8"))
        run_and_compare(R, prob, "fp8 D=%d P=%d" % (D, P), P=P, m=1)


FP8_SHAPES = [  # (H_kv, G, D): one and two 8-row halves, odd groups, both head dims
    (1, 1, 64), (1, 16, 128), (3, 3, 128), (2, 16, 64),
]


@pytest.mark.parametrize("Hkv,G,D", FP8_SHAPES)
def test_fp8_shapes_and_ragged_lengths(R, Hkv, G, D):
    """fp8 K goes through per-wave LDS rows (whole-row loads); these shapes
    cover both row widths (64 and 128 bytes) and both merge widths."""
    lens = np.array([0, 1, 63, 64, 65, 127, 1000, 2049, 7], np.int32)
    for P, m in ((1, 1), (7, 3), (300, 2)):
        prob = wl.make_problem("fp8", seed=P + D, device="cuda", lens=lens, poison=True,
                               workload=custom_workload(Hkv, G, D, "fp8"))
        run_and_compare(R, prob, "fp8 shape Hkv=%d G=%d D=%d P=%d m=%d" % (Hkv, G, D, P, m),
                        P=P, m=m)


def test_fp8_decodes_every_code_exactly(R):
    """One token per request, V = every finite e4m3 code, v_scale = 1: the
    output is that token's V, exactly representable in bf16."""
    from load_balanced_split_amd import hpcattn as H
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0           # the two NaN codes
    lens = np.array([1, 1], np.int32)
    prob = wl.make_problem("fp8", seed=3, device="cuda", lens=lens, poison=True,
                           workload=custom_workload(1, 2, 128, "fp8"))
    pt = prob.page_table
    for b in range(2):
        prob.v_pages[0][int(pt[b, 0]), 0, 0, :] = torch.from_numpy(codes[128 * b:128 * b + 128]).cuda()
        prob.v_scale[0][int(pt[b, 0]), 0, 0] = 1.0
    run = R.DecodeRunner(prob)
    out, _ = run.run()
    sync()
    table = oracle.e4m3_table()
    got = out.float().cpu().numpy()
    for b in range(2):
        want = table[codes[128 * b:128 * b + 128]]
        for j in range(2):
            assert (got[b, j] == want).all(), (b, j)


def test_bin_count_invariance_on_uniform_batch(R):
    lens = np.full(16, 1000, np.int32)
    outs = []
    for P in (8, 64, 256, 1024):
        prob = wl.make_problem("mixed", seed=5, device="cuda", lens=lens, layers=1, poison=True)
        stats, run = run_and_compare(R, prob, "uniform P=%d" % P, P=P, m=1)
        outs.append(run.out.float().cpu().numpy())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


def test_sharp_softmax(R):
    lens = np.array([300, 4096, 17, 20000], np.int32)
    prob = wl.make_problem("mixed", seed=9, device="cuda", lens=lens, layers=1, q_mult=8.0,
                           poison=True)
    stats, _ = run_and_compare(R, prob, "sharp softmax (Q x 8)", P=64, m=1)
    assert stats["rel_l2"] <= 2e-2


def test_out_lse_optional(R):
    from load_balanced_split_amd import hpcattn as H
    prob = wl.make_problem("tiny", seed=2, device="cuda")
    run = R.DecodeRunner(prob)
    out, lse = run.run()
    ref = out.clone()
    H.hpcattn_combine(run.dims, run.task_map, run.part_o, run.part_lse, run.out, None)
    sync()
    assert torch.equal(ref, run.out)


@pytest.mark.parametrize("name,npairs", [("single_long", 8), ("mixed", 10),
                                         ("heavy_tail", 10), ("fp8", 6)])
def test_full_size_configs_sampled(R, name, npairs):
    """Each config at its full size, in the launch configuration the benchmark
    times (default bins and floor); the oracle checks a seeded sample of
    (request, KV head) pairs, always including the longest request."""
    layers = 2 if name == "mixed" else 1
    prob = wl.make_problem(name, seed=0, device="cuda", layers=layers)
    pairs = sample_pairs(prob, npairs, seed=1)
    run = R.DecodeRunner(prob)
    run.plan()
    for layer in range(layers):   # one plan, reused by every layer
        run.decode(layer)
        run.combine()
        sync()
        h = host_inputs(prob, layer)
        ref_o, ref_l = oracle_attention(h, pairs)
        compare(run.out, run.out_lse, ref_o, ref_l, rows_of(pairs, prob.workload.group),
                prob.workload.kv_dtype == "fp8", "%s layer %d" % (name, layer))
        del h, ref_o, ref_l


@pytest.mark.parametrize("kv,rows,long_len", [("bf16", 1, (1 << 20) - 37),
                                               ("fp8", 1, (1 << 21) - 37),
                                               ("bf16", 6, (1 << 20) - 37)])
def test_kv_pools_beyond_2gib(R, kv, rows, long_len):
    """A request of one or two million tokens among shorter ones, 8 KV heads:
    each KV pool holds more than 2^31 bytes, so tile addresses pass 2^31
    (the page ids are shuffled over the whole pool).  One-row bf16 and fp8,
    and the draft-verify staging-wave kernel.  Default bins and floor; the
    oracle checks the long request's last KV head and a short request (and
    the long one's first head for one row), with dead slots poisoned."""
    lens = np.array([long_len, 5000, 0, 130001], np.int32)
    w = wl.Workload("custom", None, 8, 64, 128, kv, min_tiles=32, q_rows=rows)
    prob = wl.make_problem("tiny", seed=21, device="cuda", lens=lens, poison=True, workload=w)
    pool_bytes = prob.k_pages[0].numel() * prob.k_pages[0].element_size()
    assert pool_bytes > (1 << 31), pool_bytes
    run = R.DecodeRunner(prob)
    run.plan()
    run.decode()
    run.combine()
    sync()
    pairs = [(0, 7), (3, 5)] + ([(0, 0)] if rows == 1 else [])
    ref_o, ref_l = oracle_attention(host_inputs(prob), pairs)
    what = "%s, %d row(s), pools of %.2f GB" % (kv, rows, pool_bytes / 1e9)
    if rows == 1:
        compare(run.out, run.out_lse, ref_o, ref_l, rows_of(pairs, 8), kv == "fp8", what)
    else:
        B = len(lens)
        o = run.out.view(B * rows, 64, 128)
        l = run.out_lse.view(B * rows, 64)
        cmp_rows = [(b * rows + r, h * 8 + g) for b, h in pairs for r in range(rows)
                    for g in range(8)]
        compare(o, l, ref_o.reshape(B * rows, 64, 128), ref_l.reshape(B * rows, 64), cmp_rows,
                False, what)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_maximum_batch(R, kv):
    """The largest batch the library takes (8192 requests), ragged lengths
    from 0 to 300 tokens, through plan -> decode -> combine and through the
    fused call, against the oracle on every request."""
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 301, size=8192).astype(np.int32)
    lens[::97] = 0                      # empty requests among them
    w = custom_workload(1, 4, 64, kv, P=1024, m=1)
    prob = wl.make_problem("tiny", seed=3, device="cuda", lens=lens, poison=True, workload=w)
    assert len(prob.seq_lens) == 8192
    _, run = run_and_compare(R, prob, "max batch %s, two launches" % kv, P=1024, m=1)
    out2, lse2 = run.out.clone(), run.out_lse.clone()
    run.decode_combine(0)
    sync()
    # the fused call agrees with decode + combine (up to the merge order)
    assert torch.allclose(run.out.float(), out2.float(), atol=2e-2, rtol=0)
    fin = torch.isfinite(lse2)
    assert torch.equal(torch.isfinite(run.out_lse), fin)
    assert torch.allclose(run.out_lse[fin], lse2[fin], atol=1e-4, rtol=0)
    assert int(run.tickets.abs().sum()) == 0


@pytest.mark.parametrize("kv,rows,per_cu", [("bf16", 8, 2), ("fp8", 8, 3),
                                            ("bf16", 48, 2), ("fp8", 48, 4)])
def test_suggested_bins_are_the_measured_residency(kv, rows, per_cu):
    """The default bin count is CUs x the workgroups each CU holds: two for
    the one-row bf16 kernel (LDS padding holds it there; its registers would
    admit three), three for one-row fp8, and for 6 rows of 8 heads (the
    shared-tile kernel with its staging wave) two for bf16 and four for fp8.
    A change to a kernel's registers or LDS that moves these fails here."""
    from load_balanced_split_amd import hpcattn as H
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    code = H.KV_BF16 if kv == "bf16" else H.KV_FP8_E4M3
    n = H.hpcattn_suggest_num_bins(128, code, rows)
    say("suggested bins", kv, "rows", rows, "->", n, "on", cus, "CUs")
    assert n == cus * per_cu
