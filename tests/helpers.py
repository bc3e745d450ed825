"""Shared helpers of the GPU tests: run the HIP path and the oracle on the same
bytes and compare.  The oracle always reads the bytes copied back from the
device, never anything the HIP path computed."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from load_balanced_split_amd import workloads as wl

# Tolerances of the method's outputs against the fp64 oracle.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
FP8_MAX_ABS = 6e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_inputs(prob: wl.Problem, layer: int = 0) -> dict:
    """The problem's device tensors as host arrays, in the oracle's terms."""
    d = dict(q=wl.as_numpy(prob.q), k_pages=wl.as_numpy(prob.k_pages[layer]),
             v_pages=wl.as_numpy(prob.v_pages[layer]), page_table=prob.page_table,
             seq_lens=prob.seq_lens, num_kv_heads=prob.workload.num_kv_heads,
             sm_scale=prob.sm_scale)
    if prob.workload.kv_dtype == "fp8":
        d.update(q_scale=wl.as_numpy(prob.q_scale), k_scale=wl.as_numpy(prob.k_scale[layer]),
                 v_scale=wl.as_numpy(prob.v_scale[layer]))
    return d


def oracle_attention(h: dict, pairs=None):
    return oracle.attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["seq_lens"],
                            num_kv_heads=h["num_kv_heads"], sm_scale=h["sm_scale"],
                            q_scale=h.get("q_scale"), k_scale=h.get("k_scale"),
                            v_scale=h.get("v_scale"), pairs=pairs)


def rows_of(pairs, G):
    """(b, j) query rows covered by (b, h) pairs."""
    return [(b, h * G + g) for b, h in pairs for g in range(G)]


def compare(out_dev, lse_dev, ref_o, ref_l, rows, fp8: bool, what: str):
    """Element-wise comparison of the selected rows; returns error stats."""
    o = out_dev.float().cpu().numpy().astype(np.float64)
    l = lse_dev.cpu().numpy().astype(np.float64)
    bi = np.array([r[0] for r in rows])
    ji = np.array([r[1] for r in rows])
    err = np.abs(o[bi, ji] - ref_o[bi, ji])
    ref = ref_o[bi, ji]
    rel_l2 = float(np.linalg.norm(o[bi, ji] - ref) / max(np.linalg.norm(ref), 1e-30))
    fin = np.isfinite(ref_l[bi, ji])
    lerr = np.abs(l[bi, ji][fin] - ref_l[bi, ji][fin])
    assert (np.isneginf(l[bi, ji]) == ~fin).all(), what + ": lse -inf pattern differs"
    stats = dict(max_abs=float(err.max()) if err.size else 0.0,
                 mean_abs=float(err.mean()) if err.size else 0.0,
                 rel_l2=rel_l2, lse_max_abs=float(lerr.max()) if lerr.size else 0.0)
    say("%s: %s" % (what, stats))
    assert np.isfinite(o[bi, ji]).all(), what + ": non-finite output"
    if fp8:
        assert stats["max_abs"] <= FP8_MAX_ABS, (what, stats)
    else:
        assert stats["max_abs"] <= BF16_MAX_ABS, (what, stats)
        assert stats["mean_abs"] <= BF16_MEAN_ABS, (what, stats)
    assert stats["lse_max_abs"] <= 2e-2, (what, stats)
    return stats


def sample_pairs(prob: wl.Problem, n: int, seed: int = 0):
    """n (b, h) pairs, always including the longest request."""
    rng = np.random.default_rng(seed)
    B, Hkv = prob.seq_lens.shape[0], prob.workload.num_kv_heads
    longest = int(np.argmax(prob.seq_lens))
    pairs = {(longest, int(rng.integers(Hkv)))}
    while len(pairs) < min(n, B * Hkv):
        pairs.add((int(rng.integers(B)), int(rng.integers(Hkv))))
    return sorted(pairs)


def sync():
    torch.cuda.synchronize()
