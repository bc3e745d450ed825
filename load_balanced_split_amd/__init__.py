"""Load-balanced split-KV decode attention over a paged GQA KV cache, for
MI355X (gfx950).

The compute path is the C-ABI library ``libhpcattn.so`` built from
``csrc/`` (hand-written HIP kernels); ``hpcattn`` is its thin ctypes binding
and ``workloads`` draws seeded synthetic inputs.  Importing this package loads
nothing; ``from load_balanced_split_amd import hpcattn`` loads the library and
raises if it has not been built.
"""
__all__ = ["hpcattn", "workloads"]
