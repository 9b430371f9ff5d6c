"""A continuous-batching decode loop over one layer's paged KV cache.

The caller side of the hot path: it turns token ids into block tables and
slot mappings with the host block manager (prefix sharing by chained block
hashes, reference counts, copy-on-write; "Implémentation du cache" in the
nano-vLLM article, PagedAttention's sharing in the CS336 lecture 10 notes),
and runs each decode step as the pages order it: the new tokens' K/V are
written into their slots first, then attention reads every cached token
including them ("Traitement par lots continu" and "Écriture dans le cache"
in the nano-vLLM article; step 1 before step 2 in "Optimisation de
l'inférence").  Sequences join and leave between steps (continuous
batching); a step decodes whichever sequences it is given.

Every step of the computation runs in libpa's kernels; this module only
keeps the bookkeeping and moves arrays.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import (BlockManager, cache_append, copy_blocks, decode,
               decode_workspace_size)


class DecodeLoop:
    """K/V pools of ``num_blocks`` blocks of ``block_size`` tokens, the block
    manager that hands them out, and the per-step work of a decode batch.

    dtype is torch.bfloat16 or torch.float32 (q, K/V rows and outputs share
    it).  With ``graph_buckets`` the append + decode of a step are replayed
    from HIP graphs recorded for those batch sizes (the batch is padded to
    the smallest bucket that holds it); the copy-on-write copies stay eager.
    """

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, num_q_heads: int,
                 head_dim: int, max_blocks_per_seq: int, scale: float, dtype, device="cuda",
                 graph_buckets: Optional[Sequence[int]] = None):
        import torch

        if num_q_heads % num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        self.block_size, self.max_blocks = block_size, max_blocks_per_seq
        self.num_kv_heads, self.num_q_heads, self.head_dim = num_kv_heads, num_q_heads, head_dim
        self.scale, self.dtype, self.device = float(scale), dtype, torch.device(device)
        shape = (num_blocks, block_size, num_kv_heads, head_dim)
        self.k_cache = torch.zeros(shape, dtype=dtype, device=self.device)
        self.v_cache = torch.zeros(shape, dtype=dtype, device=self.device)
        self.manager = BlockManager(num_blocks, block_size)
        self._num_tokens: Dict[int, int] = {}
        self._workspace = None
        self._ws_batch = 0
        self.graphs = None
        if graph_buckets:
            from .graphs import DecodeGraphs

            self.graphs = DecodeGraphs(self.k_cache, self.v_cache, num_q_heads, max_blocks_per_seq,
                                       scale, buckets=graph_buckets)
        self.copied_blocks = 0  # copy-on-write blocks copied so far

    # ---- sequences ------------------------------------------------------------
    def add(self, seq_id: int, tokens, k_rows, v_rows) -> int:
        """Admit a sequence with its prompt.  k_rows, v_rows: [len(tokens),
        Hkv, d] device tensors, the prompt's K/V.  Leading blocks whose tokens
        a live sequence already holds are shared, and their K/V are not
        written again; returns how many prompt tokens were found cached."""
        import torch

        n = len(tokens)
        cached = self.manager.add_sequence(seq_id, tokens)
        self._num_tokens[seq_id] = n
        if cached < n:
            bt = self.manager.block_table(seq_id, self.max_blocks)
            pos = np.arange(cached, n)
            slots = (bt[pos // self.block_size] * self.block_size + pos % self.block_size)
            cache_append(self.k_cache, self.v_cache, k_rows[cached:].contiguous(),
                         v_rows[cached:].contiguous(),
                         torch.from_numpy(slots.astype(np.int32)).to(self.device))
        return cached

    def fork(self, parent: int, child: int) -> None:
        """child starts as a copy of parent, sharing its blocks (a parallel
        sample of the same prompt); the first write into a shared partial
        block copies it."""
        self.manager.fork(parent, child)
        self._num_tokens[child] = self._num_tokens[parent]

    def free(self, seq_id: int) -> None:
        """Retire a sequence; its blocks return to the pool when no other
        sequence holds them."""
        self.manager.free(seq_id)
        del self._num_tokens[seq_id]

    def num_tokens(self, seq_id: int) -> int:
        return self._num_tokens[seq_id]

    def block_table(self, seq_id: int):
        return self.manager.block_table(seq_id, self.max_blocks)

    @property
    def live(self):
        return sorted(self._num_tokens)

    # ---- one decode step --------------------------------------------------------
    def step(self, seq_ids: Sequence[int], new_tokens: Sequence[int], q, k_new, v_new):
        """One decode step for the listed sequences: each gets one more token
        (new_tokens[i], whose K/V rows are k_new[i], v_new[i], [Hkv, d]) and
        its query q[i] ([Hq, d]) attends to all of its cached tokens, the new
        one included.  Returns out [len(seq_ids), Hq, d]."""
        import torch

        b = len(seq_ids)
        if b == 0:  # nothing to decode this step
            return torch.empty((0, self.num_q_heads, self.head_dim), dtype=self.dtype,
                               device=self.device)
        slots = np.empty(b, np.int32)
        for i, (sid, tok) in enumerate(zip(seq_ids, new_tokens)):
            slots[i] = self.manager.append_token(sid, int(tok))
            self._num_tokens[sid] += 1
        src, dst = self.manager.take_copies()
        if len(src):  # copy-on-write: a shared partial block is copied before the write
            s_d = torch.from_numpy(src).to(self.device)
            d_d = torch.from_numpy(dst).to(self.device)
            copy_blocks(self.k_cache, s_d, d_d)
            copy_blocks(self.v_cache, s_d, d_d)
            self.copied_blocks += len(src)
        tables = np.stack([self.manager.block_table(s, self.max_blocks) for s in seq_ids])
        lens = np.array([self._num_tokens[s] for s in seq_ids], np.int32)
        slots_d = torch.from_numpy(slots).to(self.device)
        tables_d = torch.from_numpy(tables).to(self.device)
        lens_d = torch.from_numpy(lens).to(self.device)
        if self.graphs is not None:
            return self.graphs.run(q, k_new, v_new, slots_d, tables_d, lens_d)
        cache_append(self.k_cache, self.v_cache, k_new, v_new, slots_d)
        if self._workspace is None or b > self._ws_batch:
            n = decode_workspace_size(b, self.num_q_heads, self.num_kv_heads, self.head_dim,
                                      self.head_dim, self.block_size, self.max_blocks)
            self._workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
            self._ws_batch = b
        out = torch.empty((b, self.num_q_heads, self.head_dim), dtype=self.dtype,
                          device=self.device)
        decode(out, q, self.k_cache, self.v_cache, tables_d, lens_d, self.scale, self._workspace)
        return out
