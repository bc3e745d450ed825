"""Seeded synthetic decode-attention workloads.

This module only draws inputs: sequence lengths, a shuffled page table, and
N(0,1) Q/K/V (bf16, or e4m3 bytes with per-token per-head fp32 scales).  It
holds none of the attention arithmetic and imports neither the HIP library
nor the oracle, so both can be fed from it.

Workloads follow the length mixes the pages benchmark ("HPC-Ops x SGLang",
"Performance evaluation / H20 operator benchmarks / Attention": A requests of
KV length B, from uniform to heavily skewed batches, fp8 KV cache, page size
64 in the serving setup).  The pages measure on synthetic length mixes, not on
a public dataset.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, Optional

import numpy as np
import torch

PAGE = 64          # tokens per KV page (= tokens per tile)
E4M3_MAX = 448.0   # largest finite OCP E4M3FN value


def _log_uniform(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """floor(exp(U[ln lo, ln hi))) clamped to [lo, hi]."""
    x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(x, lo, hi).astype(np.int32)


def _tiny(rng):
    return np.array([17, 64, 200, 1000], np.int32)


def _single_long(rng):
    return np.array([131072], np.int32)


def _mixed(rng):
    return _log_uniform(rng, 64, 256, 32768)


def _heavy_tail(rng, order: str = "random"):
    short = rng.integers(922, 1126, size=120, endpoint=True).astype(np.int32)
    long_ = np.full(8, 65536, np.int32)
    if order == "long_first":
        return np.concatenate([long_, short])
    if order == "long_last":
        return np.concatenate([short, long_])
    lens = np.concatenate([short, long_])
    return lens[rng.permutation(lens.shape[0])].astype(np.int32)


def _heavy_tail_long_first(rng):
    return _heavy_tail(rng, "long_first")


def _heavy_tail_long_last(rng):
    return _heavy_tail(rng, "long_last")


def _fp8(rng):
    return _log_uniform(rng, 32, 1024, 131072)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    lens: Callable[[np.random.Generator], np.ndarray]
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    kv_dtype: str            # "bf16" or "fp8"
    layers: int = 1          # distinct KV pools per step
    num_bins: Optional[int] = None  # persistent workgroups (one bin each); None: as many
                                    # as the device holds at once
    min_tiles: int = 32      # minimum-work floor, tiles per bin
    q_rows: int = 1          # query rows per request: 1 + draft tokens to verify

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def q_shape(self, batch: int):
        """[B, H_q, D], or [B, R, H_q, D] with R = q_rows > 1."""
        if self.q_rows == 1:
            return (batch, self.num_q_heads, self.head_dim)
        return (batch, self.q_rows, self.num_q_heads, self.head_dim)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", _tiny, 1, 4, 64, "bf16", num_bins=8, min_tiles=2),
    "single_long": Workload("single_long", _single_long, 8, 64, 128, "bf16"),
    "mixed": Workload("mixed", _mixed, 8, 64, 128, "bf16", layers=32),
    "heavy_tail": Workload("heavy_tail", _heavy_tail, 8, 64, 128, "bf16"),
    # The same lengths with the 8 long requests first, or last, in the batch
    # (order checks: a static grid dispatches its long workgroups first or
    # last; the dynamic bins do not depend on the order).
    "heavy_tail_long_first": Workload("heavy_tail_long_first", _heavy_tail_long_first, 8, 64,
                                      128, "bf16"),
    "heavy_tail_long_last": Workload("heavy_tail_long_last", _heavy_tail_long_last, 8, 64, 128,
                                     "bf16"),
    "fp8": Workload("fp8", _fp8, 8, 64, 128, "fp8"),
    # A draft-verify step ("SGLang Low-Latency Mode", section 1: the confirmed
    # token and five drafts per request, six rows) over the mixed length mix.
    "mtp": Workload("mtp", _mixed, 8, 64, 128, "bf16", layers=32, q_rows=6),
    "mtp_fp8": Workload("mtp_fp8", _fp8, 8, 64, 128, "fp8", q_rows=6),
    # One GPU's share of the mixed batch when the heads are split over 8 GPUs
    # ("HPC-Ops x SGLang", SGLang serving with tensor parallelism 8): 1 KV
    # head and its 8 query heads per GPU, the same lengths, 32 layers.  Its
    # ~6.6K tiles would make only ~206 bins of the 32-tile floor, fewer than
    # the CUs; a floor of 8 tiles gives the 512 bins of the full batch.
    "mixed_shard": Workload("mixed_shard", _mixed, 1, 8, 128, "bf16", layers=32, min_tiles=8),
}


def seq_lens(name: str, seed: int = 0, **kw) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return WORKLOADS[name].lens(rng, **kw) if kw else WORKLOADS[name].lens(rng)


def page_table(lens: np.ndarray, seed: int = 0, spare_pages: int = 0):
    """Each request's pages are taken in order from one pool, then the whole
    pool is permuted with a seeded permutation.  Rows are padded with -1.
    Returns (page_table int32 [B, max_pages], num_pages)."""
    lens = np.asarray(lens, np.int64)
    n = (lens + PAGE - 1) // PAGE
    total = int(n.sum()) + spare_pages
    max_pages = max(1, int(n.max()) if n.size else 1)
    rng = np.random.default_rng(seed + 0x5EED)
    perm = rng.permutation(max(total, 1)).astype(np.int32)
    pt = np.full((lens.shape[0], max_pages), -1, np.int32)
    off = 0
    for b, nb in enumerate(n):
        pt[b, :nb] = perm[off:off + nb]
        off += int(nb)
    return pt, max(total, 1)


def randn_bf16(shape, gen: torch.Generator, device) -> torch.Tensor:
    """N(0,1) float32 draws rounded to nearest-even bf16."""
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def quantize_e4m3(x: torch.Tensor):
    """Per-row (last dim) e4m3 quantisation of float data: scale = amax / 448,
    bytes = RNE(x / scale) in OCP E4M3FN.  Returns (uint8 bytes, fp32 scale)."""
    amax = x.abs().amax(dim=-1).to(torch.float32)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def poison_dead_slots(pool: torch.Tensor, lens: np.ndarray, pt: np.ndarray, value) -> None:
    """Fill the slots past each request's length in its last page with a NaN
    pattern, so that any read of dead KV shows up in the output.  `pool` is a
    KV pool [num_pages, Hkv, 64, D] or a scale pool [num_pages, Hkv, 64]."""
    for b, L in enumerate(np.asarray(lens)):
        L = int(L)
        if L % PAGE:
            pool[int(pt[b, L // PAGE]), :, L % PAGE:] = value


@dataclasses.dataclass
class Problem:
    """One layer's inputs (or several layers' KV pools) on one device."""
    workload: Workload
    seq_lens: np.ndarray
    page_table: np.ndarray
    num_pages: int
    q: torch.Tensor                          # bf16 [B,Hq,D] ([B,R,Hq,D]) or uint8
    k_pages: list                            # per layer [num_pages,Hkv,64,D]
    v_pages: list
    q_scale: Optional[torch.Tensor] = None   # fp32 [B,Hq] ([B,R,Hq])
    k_scale: Optional[list] = None           # per layer fp32 [num_pages,Hkv,64]
    v_scale: Optional[list] = None
    sm_scale: float = 1.0


def make_problem(name: str, seed: int = 0, device="cpu", layers: Optional[int] = None,
                 lens: Optional[np.ndarray] = None, poison: bool = False,
                 q_mult: float = 1.0, workload: Optional[Workload] = None) -> Problem:
    """Draw a workload's inputs.  `lens` overrides the drawn lengths; `layers`
    overrides the number of distinct KV pools; `poison` fills dead slots with
    NaN; `q_mult` scales Q before rounding (a sharper softmax)."""
    w = workload or WORKLOADS[name]
    L = seq_lens(name, seed) if lens is None else np.asarray(lens, np.int32)
    pt, num_pages = page_table(L, seed)
    nl = w.layers if layers is None else layers
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 17)
    B, Hq, Hkv, D = L.shape[0], w.num_q_heads, w.num_kv_heads, w.head_dim
    pool_shape = (num_pages, Hkv, PAGE, D)
    sm_scale = 1.0 / math.sqrt(D)
    qshape = w.q_shape(B)
    if w.kv_dtype == "bf16":
        q = (torch.randn(qshape, generator=gen, device=device) * q_mult).to(torch.bfloat16)
        ks, vs = [], []
        for _ in range(nl):
            k = randn_bf16(pool_shape, gen, device)
            v = randn_bf16(pool_shape, gen, device)
            if poison:
                nan = float("nan")
                poison_dead_slots(k, L, pt, nan)
                poison_dead_slots(v, L, pt, nan)
            ks.append(k)
            vs.append(v)
        return Problem(w, L, pt, num_pages, q.contiguous(), ks, vs, sm_scale=sm_scale)
    if w.kv_dtype == "fp8":
        qf = torch.randn(qshape, generator=gen, device=device) * q_mult
        q, q_scale = quantize_e4m3(qf)
        ks, vs, kss, vss = [], [], [], []
        for _ in range(nl):
            k, kscale = quantize_e4m3(torch.randn(pool_shape, generator=gen, device=device))
            v, vscale = quantize_e4m3(torch.randn(pool_shape, generator=gen, device=device))
            if poison:
                poison_dead_slots(k, L, pt, 0x7F)
                poison_dead_slots(v, L, pt, 0x7F)
                poison_dead_slots(kscale, L, pt, float("nan"))
                poison_dead_slots(vscale, L, pt, float("nan"))
            ks.append(k)
            vs.append(v)
            kss.append(kscale)
            vss.append(vscale)
        return Problem(w, L, pt, num_pages, q, ks, vs, q_scale, kss, vss, sm_scale)
    raise ValueError("unknown kv dtype %r" % w.kv_dtype)


def as_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's raw elements: bf16 as uint16 bits, uint8 as-is,
    float32 / int32 unchanged."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def kv_bytes_per_token(w: Workload) -> int:
    """Algorithmic KV bytes read per live token per layer: K and V for every
    KV head, plus the two fp32 scales per head in the fp8 layout."""
    if w.kv_dtype == "bf16":
        return 2 * w.num_kv_heads * w.head_dim * 2
    return 2 * w.num_kv_heads * (w.head_dim + 4)
