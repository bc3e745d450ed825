"""Pins for the oracle's task map (the assign step) on the CPU.

- the hand-worked Tiny example (tests/golden/plan_tiny.json);
- a literal per-tile greedy fill, written independently here: walk the
  global tiles in (request, KV head, tile) order, put each into the current
  bin until that bin holds its budget, then spill into the next bin; compared
  word for word with the oracle over every small case;
- invariants that hold whatever the formula: each tile covered exactly once,
  sorted descriptors that never cross a segment, bin sizes within one tile,
  the minimum-work floor, the descriptor bound.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

TILE = 64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_tiny.json")


def greedy_fill(lens, Hkv, P, m):
    """Per-tile greedy bin fill ("fill each bin to its budget, then spill").

    Budget: T tiles over P_eff bins, the first T mod P_eff bins one tile more;
    the floor keeps at least m tiles of work per used bin."""
    n = [(L + TILE - 1) // TILE for L in lens]
    tiles = [(b, h, t) for b in range(len(lens)) for h in range(Hkv) for t in range(n[b])]
    T = len(tiles)
    P_eff = min(P, max(1, T // m))
    budgets = [T // P_eff + (1 if i < T % P_eff else 0) for i in range(P_eff)] + [0] * (P - P_eff)
    owner = []
    i, fill = 0, 0
    for _ in tiles:
        while i < P and fill == budgets[i]:
            i, fill = i + 1, 0
        owner.append(i)
        fill += 1
    # Runs of consecutive tiles with the same (bin, request, head) are descriptors.
    desc, desc_bin = [], []
    for k, (b, h, t) in enumerate(tiles):
        if desc and desc_bin[-1] == owner[k] and desc[-1][0] == b and desc[-1][1] == h \
                and desc[-1][3] == t:
            desc[-1][3] = t + 1
        else:
            desc.append([b, h, t, t + 1])
            desc_bin.append(owner[k])
    S = len(lens) * Hkv
    bin_off = [sum(1 for x in desc_bin if x < i) for i in range(P + 1)]
    seg_off = [sum(1 for d in desc if d[0] * Hkv + d[1] < s) for s in range(S + 1)]
    words = [T, P_eff, T // P_eff, T % P_eff, len(desc), len(lens), Hkv, 0]
    words += list(lens) + bin_off + seg_off
    flat = [x for d in desc for x in d]
    words += flat + [0] * (4 * (S + P - 1) - len(flat))
    return np.array(words, np.int32)


def check_invariants(lens, Hkv, P, m, words):
    d = oracle.parse_map(words, P)
    n = [(L + TILE - 1) // TILE for L in lens]
    T = Hkv * sum(n)
    S = len(lens) * Hkv
    assert d["T"] == T and d["err"] == 0
    assert list(d["seq_lens"]) == list(lens)
    P_eff = d["P_eff"]
    desc = d["desc"]
    # Every (b, h, tile) covered exactly once.
    cover = {}
    for b, h, t0, t1 in desc:
        assert 0 <= t0 < t1 <= n[b]
        for t in range(t0, t1):
            cover[(b, h, t)] = cover.get((b, h, t), 0) + 1
    assert len(cover) == T and set(cover.values()) <= {1}
    # Sorted in global tile order.
    keys = [(b * Hkv + h, t0) for b, h, t0, _ in desc]
    assert keys == sorted(keys)
    # CSR offsets agree with the descriptor list.
    bo, so = d["bin_desc_off"], d["seg_desc_off"]
    assert bo[0] == 0 and bo[-1] == len(desc) and (np.diff(bo) >= 0).all()
    assert so[0] == 0 and so[-1] == len(desc) and (np.diff(so) >= 0).all()
    for s in range(S):
        for k in range(so[s], so[s + 1]):
            assert desc[k][0] * Hkv + desc[k][1] == s
    sizes = np.array([sum(desc[k][3] - desc[k][2] for k in range(bo[i], bo[i + 1]))
                      for i in range(P)])
    assert sizes.sum() == T
    used = sizes[:P_eff]
    assert (sizes[P_eff:] == 0).all()
    assert used.max() - used.min() <= 1
    assert len(desc) <= max(0, S + P_eff - 1) or T == 0
    if T // m >= P:                     # floor inactive: all P bins within a tile of T / P
        assert P_eff == P
        assert (np.abs(sizes - T / P) < 1).all()
    elif T >= m:                        # floor active: every used bin has >= m tiles
        assert (used >= m).all()
    else:                               # too little work for two bins: one bin holds all
        assert P_eff == 1 and sizes[0] == T
    # One descriptor per (bin, segment) intersection: none is split needlessly.
    for i in range(P):
        segs = [desc[k][0] * Hkv + desc[k][1] for k in range(bo[i], bo[i + 1])]
        assert len(segs) == len(set(segs))


def test_worked_examples():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        P = c["num_bins"]
        w = oracle.plan(c["seq_lens"], c["num_kv_heads"], P, c["min_tiles"])
        d = oracle.parse_map(w, P)
        for key in ("T", "P_eff", "q", "r", "num_desc"):
            assert d[key] == c[key], key
        assert d["desc"].tolist() == c["desc"]
        assert d["bin_desc_off"].tolist() == c["bin_desc_off"]
        assert d["seg_desc_off"].tolist() == c["seg_desc_off"]
        check_invariants(c["seq_lens"], c["num_kv_heads"], P, c["min_tiles"], w)


def test_matches_per_tile_greedy_fill_exhaustively():
    lens_pool = [0, 1, 63, 64, 65, 128, 200, 300]
    count = 0
    for B in (1, 2, 3):
        for lens in itertools.product(lens_pool, repeat=B):
            if B == 3 and len(set(lens)) < 2:
                continue
            for Hkv in (1, 2):
                for P in range(1, 7):
                    for m in range(1, 5):
                        w = oracle.plan(list(lens), Hkv, P, m)
                        ref = greedy_fill(list(lens), Hkv, P, m)
                        assert w.tolist() == ref.tolist(), (lens, Hkv, P, m)
                        count += 1
    assert count > 10000


@pytest.mark.parametrize("seed", range(6))
def test_invariants_on_random_batches(seed):
    rng = np.random.default_rng(seed)
    for _ in range(25):
        B = int(rng.integers(1, 130))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        lens = np.floor(np.exp(rng.uniform(0, np.log(70000), size=B))).astype(int)
        lens[rng.random(B) < 0.05] = 0
        P = int(rng.choice([1, 8, 64, 256, 512, 1024, 777]))
        m = int(rng.choice([1, 2, 4, 16]))
        w = oracle.plan(lens.tolist(), Hkv, P, m)
        check_invariants(lens.tolist(), Hkv, P, m, w)


def test_edge_cases():
    # No live KV at all: one (empty) bin, no descriptors, all offsets zero.
    w = oracle.plan([0, 0, 0], 2, 8, 2)
    d = oracle.parse_map(w, 8)
    assert (d["T"], d["P_eff"], d["q"], d["r"], d["num_desc"]) == (0, 1, 0, 0, 0)
    assert (d["bin_desc_off"] == 0).all() and (d["seg_desc_off"] == 0).all()
    # One token.
    d = oracle.parse_map(oracle.plan([1], 1, 4, 1), 4)
    assert d["desc"].tolist() == [[0, 0, 0, 1]] and d["P_eff"] == 1
    # Exactly 65536 tokens = 1024 full tiles over 8 heads and 512 bins.
    w = oracle.plan([65536], 8, 512, 4)
    d = oracle.parse_map(w, 512)
    assert d["T"] == 8192 and d["q"] == 16 and d["r"] == 0 and d["num_desc"] == 512
    check_invariants([65536], 8, 512, 4, w)
    # Fewer tiles than bins, and fewer than the floor.
    for lens, P, m in (([100, 5], 16, 1), ([100, 5], 16, 8), ([3000], 1, 1), ([64] * 7, 3, 100)):
        check_invariants(lens, 1, P, m, oracle.plan(lens, 1, P, m))
    # Bad arguments are rejected.
    for args in (([5], 1, 0, 1), ([5], 1, 4, 0), ([5], 0, 4, 1), ([-1], 1, 4, 1)):
        with pytest.raises(ValueError):
            oracle.plan(*args)


def test_descriptor_bound_is_tight():
    # Two segments of 5 tiles over bins of 3,3,2,2 tiles: no bin boundary
    # (3, 6, 8) meets the segment boundary (5), so each one splits a segment
    # and the count reaches S + P_eff - 1.
    w = oracle.plan([5 * TILE, 5 * TILE], 1, 4, 1)
    d = oracle.parse_map(w, 4)
    assert d["P_eff"] == 4 and d["num_desc"] == 2 + 4 - 1
