"""Device buffers for one decode-attention problem, driven through the C ABI.

Plumbing only: it allocates torch tensors for the task map, partials and
outputs, and calls hpcattn_plan / hpcattn_decode / hpcattn_combine /
hpcattn_static_decode.  All arithmetic happens in libhpcattn's kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import hpcattn as H
from .workloads import Problem


class DecodeRunner:
    def __init__(self, prob: Problem, num_bins: Optional[int] = None,
                 min_tiles: Optional[int] = None, device="cuda"):
        w = prob.workload
        self.prob = prob
        self.device = device
        B = prob.seq_lens.shape[0]
        self.B, self.Hq, self.Hkv, self.D = B, w.num_q_heads, w.num_kv_heads, w.head_dim
        self.G = self.Hq // self.Hkv
        self.R = w.q_rows
        self.rows = self.R * self.G          # query rows per KV head
        self.fp8 = w.kv_dtype == "fp8"
        if num_bins is None:
            num_bins = w.num_bins
        if num_bins is None:
            num_bins = H.hpcattn_suggest_num_bins(self.D, H.KV_FP8_E4M3 if self.fp8 else H.KV_BF16,
                                                  self.rows)
        self.num_bins = num_bins
        self.min_tiles = w.min_tiles if min_tiles is None else min_tiles
        self.dims = H.make_dims(B, self.Hq, self.Hkv, self.D, prob.page_table.shape[1],
                                prob.num_pages, H.KV_FP8_E4M3 if self.fp8 else H.KV_BF16,
                                prob.sm_scale, self.R)
        self.seq_lens = torch.from_numpy(prob.seq_lens.astype(np.int32)).to(device)
        self.page_table = torch.from_numpy(prob.page_table).to(device)
        self.task_map = H.alloc_task_map(B, self.Hkv, self.num_bins, device)
        rows = H.hpcattn_max_partials(B, self.Hkv, self.num_bins)
        self.part_o = torch.empty((rows, self.rows, self.D), dtype=torch.float32, device=device)
        self.part_lse = torch.empty((rows, self.rows), dtype=torch.float32, device=device)
        lead = w.q_shape(B)[:-1]
        self.out = torch.empty(lead + (self.D,), dtype=torch.bfloat16, device=device)
        self.out_lse = torch.empty(lead, dtype=torch.float32, device=device)
        # tickets of the fused decode + combine: zero once, kept zero by it
        self.tickets = torch.zeros(B * self.Hkv, dtype=torch.int32, device=device)
        self._static = {}

    def _kv(self, layer: int):
        p = self.prob
        if self.fp8:
            return dict(k_pages=p.k_pages[layer], v_pages=p.v_pages[layer], q_scale=p.q_scale,
                        k_scale=p.k_scale[layer], v_scale=p.v_scale[layer])
        return dict(k_pages=p.k_pages[layer], v_pages=p.v_pages[layer])

    def plan(self, stream=None):
        H.hpcattn_plan(self.seq_lens, self.Hkv, self.num_bins, self.min_tiles, self.task_map,
                       stream)

    def decode(self, layer: int = 0, stream=None):
        kv = self._kv(layer)
        H.hpcattn_decode(self.dims, self.prob.q, kv["k_pages"], kv["v_pages"], self.page_table,
                         self.task_map, self.part_o, self.part_lse, kv.get("q_scale"),
                         kv.get("k_scale"), kv.get("v_scale"), stream)

    def decode_combine(self, layer: int = 0, stream=None):
        """Decode + combine of one layer in one launch; returns (out, out_lse)."""
        kv = self._kv(layer)
        H.hpcattn_decode_combine(self.dims, self.prob.q, kv["k_pages"], kv["v_pages"],
                                 self.page_table, self.task_map, self.part_o, self.part_lse,
                                 self.tickets, self.out, self.out_lse, kv.get("q_scale"),
                                 kv.get("k_scale"), kv.get("v_scale"), stream)
        return self.out, self.out_lse

    def combine(self, stream=None):
        H.hpcattn_combine(self.dims, self.task_map, self.part_o, self.part_lse, self.out,
                          self.out_lse, stream)

    def run(self, layer: int = 0, stream=None):
        """plan + decode + combine for one layer; returns (out, out_lse)."""
        self.plan(stream)
        self.decode(layer, stream)
        self.combine(stream)
        return self.out, self.out_lse

    def static_buffers(self, policy: int, param: int):
        key = (policy, param)
        if key not in self._static:
            max_len = int(self.prob.seq_lens.max()) if self.B else 0
            rows = H.hpcattn_static_max_partials(self.B, self.Hkv, policy, param, max_len)
            if rows <= 0:
                raise ValueError("bad static policy %r" % (key,))
            self._static[key] = (
                torch.empty((rows, self.rows, self.D), dtype=torch.float32, device=self.device),
                torch.empty((rows, self.rows), dtype=torch.float32, device=self.device),
                max_len)
        return self._static[key]

    def release_static(self):
        """Drop the static sweep's partial buffers."""
        self._static.clear()

    def static(self, policy: int, param: int, layer: int = 0, stream=None):
        """Static split-KV decode + combine; returns (out, out_lse)."""
        po, pl, max_len = self.static_buffers(policy, param)
        kv = self._kv(layer)
        H.hpcattn_static_decode(self.dims, policy, param, max_len, self.seq_lens, self.prob.q,
                                kv["k_pages"], kv["v_pages"], self.page_table, po, pl,
                                self.out, self.out_lse, kv.get("q_scale"), kv.get("k_scale"),
                                kv.get("v_scale"), stream)
        return self.out, self.out_lse

    def num_desc(self) -> int:
        return int(self.task_map.words[4].item())
