"""Decode steps replayed from HIP graphs, one per batch-size bucket.

Capturing a step (the append of the new tokens plus the decode) into a graph
and replaying it removes the per-call launch work from the host; a graph has
fixed shapes, so graphs are recorded for a few batch sizes ("buckets") and a
batch runs on the smallest bucket that holds it, its inputs padded (the
bucketed graphs of "CUDA Graph" / "Implémentation avec seau de taille de lot"
in the nano-vLLM article).  Padding rows append nothing (slot -1) and decode
an empty context (length 0, output 0).

Both library calls only enqueue kernels on the current stream (no host
synchronisation, allocation or memset), which is what makes them capturable.
"""
from __future__ import annotations

from typing import Sequence

import torch

from . import cache_append, decode, decode_workspace_size


class DecodeGraphs:
    """Graphs of ``cache_append + decode`` over one layer's bf16/fp32 caches
    [num_blocks, block_size, Hkv, d] for each batch size in ``buckets``.

    run() copies a batch into the static inputs of the smallest bucket that
    holds it, replays that graph and returns a view of the outputs.
    """

    def __init__(self, k_cache, v_cache, num_q_heads: int, max_blocks_per_seq: int, scale: float,
                 buckets: Sequence[int] = (1, 4, 16, 64, 128), warmup: int = 2):
        self.k_cache, self.v_cache = k_cache, v_cache
        self.buckets = sorted(int(b) for b in buckets)
        nb, bs, hkv, d = k_cache.shape
        self.scale = float(scale)
        dev, dt = k_cache.device, k_cache.dtype
        B = self.buckets[-1]
        self.q = torch.zeros((B, num_q_heads, d), dtype=dt, device=dev)
        self.out = torch.zeros((B, num_q_heads, d), dtype=dt, device=dev)
        self.k_new = torch.zeros((B, hkv, d), dtype=dt, device=dev)
        self.v_new = torch.zeros((B, hkv, d), dtype=dt, device=dev)
        self.slots = torch.full((B,), -1, dtype=torch.int32, device=dev)
        self.block_tables = torch.full((B, max_blocks_per_seq), -1, dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros((B,), dtype=torch.int32, device=dev)
        n = decode_workspace_size(B, num_q_heads, hkv, d, d, bs, max_blocks_per_seq)
        self.workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.graphs = {}
        pool = None
        for b in reversed(self.buckets):
            for _ in range(warmup):  # first calls cache device properties outside capture
                self._step(b)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, pool=pool):
                self._step(b)
            if pool is None:
                pool = g.pool()
            self.graphs[b] = g
        torch.cuda.synchronize()

    def _step(self, b: int) -> None:
        cache_append(self.k_cache, self.v_cache, self.k_new[:b], self.v_new[:b], self.slots[:b])
        decode(self.out[:b], self.q[:b], self.k_cache, self.v_cache, self.block_tables[:b],
               self.context_lens[:b], self.scale, self.workspace)

    def bucket_for(self, batch: int) -> int:
        for b in self.buckets:
            if batch <= b:
                return b
        raise ValueError(f"batch {batch} exceeds the largest bucket {self.buckets[-1]}")

    def run(self, q, k_new, v_new, slot_mapping, block_tables, context_lens):
        """Append the batch's new tokens and decode it; returns out[:batch]."""
        n = q.shape[0]
        b = self.bucket_for(n)
        self.q[:n].copy_(q)
        self.k_new[:n].copy_(k_new)
        self.v_new[:n].copy_(v_new)
        self.slots[:n].copy_(slot_mapping)
        self.slots[n:b].fill_(-1)
        w = block_tables.shape[1]
        self.block_tables[:n, :w].copy_(block_tables)
        self.block_tables[:n, w:].fill_(-1)
        self.context_lens[:n].copy_(context_lens)
        self.context_lens[n:b].fill_(0)
        self.graphs[b].replay()
        return self.out[:n]
