"""The device assign kernel matches the oracle's task map word for word."""
import numpy as np
import pytest
import torch

import oracle
from helpers import say
from load_balanced_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    from load_balanced_split_amd import hpcattn
    return hpcattn


def device_plan(H, lens, Hkv, P, m):
    lens_t = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    tm = H.alloc_task_map(len(lens), Hkv, P, "cuda")
    tm.words.fill_(-7)   # every word must be written
    H.hpcattn_plan(lens_t, Hkv, P, m, tm)
    torch.cuda.synchronize()
    return tm.words.cpu().numpy()


def test_plan_tiny_worked_examples(H):
    for P in (8, 16):
        got = device_plan(H, [17, 64, 200, 1000], 1, P, 2)
        ref = oracle.plan([17, 64, 200, 1000], 1, P, 2)
        assert got.tolist() == ref.tolist(), P


@pytest.mark.parametrize("name", ["single_long", "mixed", "heavy_tail", "fp8"])
def test_plan_configs(H, name):
    w = wl.WORKLOADS[name]
    lens = wl.seq_lens(name, 0)
    for P in (256, 512, 768, 1024):
        for m in (1, 4, 16):
            got = device_plan(H, lens, w.num_kv_heads, P, m)
            ref = oracle.plan(lens, w.num_kv_heads, P, m)
            assert got.tolist() == ref.tolist(), (name, P, m)
    say(name, "T =", int(oracle.plan(lens, 8, 512, 4)[0]))


def test_plan_random_trials(H):
    rng = np.random.default_rng(1234)
    for trial in range(300):
        B = int(rng.integers(1, 300))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        kind = trial % 3
        if kind == 0:
            lens = rng.integers(0, 5000, size=B)
        elif kind == 1:
            lens = np.floor(np.exp(rng.uniform(0, np.log(200000), size=B)))
        else:
            lens = np.full(B, int(rng.integers(0, 3000)))
        lens = lens.astype(np.int32)
        P = int(rng.choice([1, 3, 8, 64, 256, 512, 1000, 1024, 2048]))
        m = int(rng.choice([1, 2, 4, 16]))
        got = device_plan(H, lens, Hkv, P, m)
        ref = oracle.plan(lens, Hkv, P, m)
        assert got.tolist() == ref.tolist(), (trial, B, Hkv, P, m)


def test_plan_edge_cases(H):
    cases = [([0], 1, 1, 1), ([0, 0, 0], 2, 8, 2), ([1], 1, 4, 1), ([65536], 8, 512, 4),
             ([100, 5], 1, 16, 8), ([64] * 7, 1, 3, 100), ([131072], 8, 4096, 1),
             (list(range(1, 2049)), 1, 64, 1), ([5] * H.MAX_BATCH, 1, 1024, 1)]
    for lens, Hkv, P, m in cases:
        got = device_plan(H, lens, Hkv, P, m)
        ref = oracle.plan(lens, Hkv, P, m)
        assert got.tolist() == ref.tolist(), (len(lens), Hkv, P, m)


def test_plan_negative_length_sets_error_word(H):
    got = device_plan(H, [100, -5, 64], 1, 4, 1)
    assert got[7] == H.MAPERR_NEG_LEN
    ref = oracle.plan([100, 0, 64], 1, 4, 1)
    got[7] = 0
    assert got.tolist() == ref.tolist()
