"""Seeded synthetic inputs for paged decode attention, plus byte/flop accounting.

This module builds inputs only. It holds none of the attention arithmetic: the
CPU oracle (``oracle/``) and the HIP library (``paged_kv_cache_58_amd``) both
consume what it produces, and neither is imported here.

Shapes follow the workloads the pages describe:

* "Optimisation de l'inférence" (aiengineeringfromscratch, phase 10 lesson 12),
  section "PagedAttention": fixed pages of 16 tokens placed anywhere in a pool,
  reached through a per-request page list; exercise 3 there gives the GQA shape
  of 64 query heads over 8 KV heads, and the "MODEL_CONFIGS" table of step 6
  gives Llama-3-70B as 80 layers, 8 KV heads, head_dim 128.
* "Cache KV, attention et optimisation de l'inference" (phase 07 lesson 12),
  "Mathématiques de cache KV": the 7B MHA shape (32 heads, d_head 128) and the
  per-token byte counts that pin the accounting below.
* CS336 lecture 10 notes ("第 10 讲：推理"), "核心概念与定义", MLA bullet: a
  cached latent of 512 + 64 RoPE dims = 576 per token.
* nano-vLLM article ("Maîtriser les mécanismes clés de l'inférence ... nano-vLLM"),
  section "Cache KV / Implémentation du cache": one pool tensor of
  [num_blocks, block_size, kv_heads, head_dim] per layer for K and for V, and
  the cache-write kernel addressed through a slot mapping with -1 meaning skip.

Random draws. Every array comes from its own child of
``numpy.random.SeedSequence(seed)`` (children in the fixed order context_lens,
block permutation, q, K pool, V pool, new-token k/v). Large arrays are filled in
chunks of ``CHUNK`` values, chunk i from grandchild i, so the result does not
depend on how many threads fill them. Values are standard normal float32; bf16
inputs are the round-to-nearest-even bf16 of those float32 draws, stored as
uint16 bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

CHUNK = 1 << 22  # values per independently seeded chunk
BASE_SEED = 58000
BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)


@dataclass(frozen=True)
class Spec:
    """A decode workload: sizes plus how context lengths are drawn."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    block_size: int
    dtype: str  # "f32" or "bf16"
    ctx_fixed: Optional[tuple] = None  # explicit context lengths, or
    ctx_range: Optional[tuple] = None  # (lo, hi) inclusive uniform integers
    mla: bool = False  # one latent cache; V = first head_dim_v dims of each K row
    pool_blocks: Optional[int] = None  # pool size; default = blocks the sequences need
    scale: Optional[float] = None  # softmax scale; default 1/sqrt(head_dim_k)
    index: int = 0  # position in the named list (seed offset)

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def softmax_scale(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim_k)
        return float(np.float32(s))

    @property
    def max_ctx(self) -> int:
        if self.ctx_fixed is not None:
            return max(self.ctx_fixed) if len(self.ctx_fixed) else 0
        return int(self.ctx_range[1])

    @property
    def max_blocks_per_seq(self) -> int:
        # room for every sequence's longest context plus one appended token
        return -(-(self.max_ctx + 1) // self.block_size)


# The five configurations the build is measured on (sizes from the pages; see
# the module docstring).  c1 is small enough for the oracle to finish instantly.
CONFIGS = {
    "c1": Spec("tiny_paged_fp32", 4, 4, 2, 64, 64, 16, "f32",
               ctx_fixed=(17, 64, 100, 255), pool_blocks=40, index=1),
    "c2": Spec("mha7b_bf16", 32, 32, 32, 128, 128, 16, "bf16",
               ctx_range=(512, 4096), index=2),
    "c3": Spec("gqa70b_bf16", 100, 64, 8, 128, 128, 16, "bf16",
               ctx_range=(1024, 8192), index=3),
    "c4": Spec("longctx_gqa_bf16", 4, 64, 8, 128, 128, 16, "bf16",
               ctx_fixed=(131072,) * 4, index=4),
    "c5": Spec("mla_latent_bf16", 64, 128, 1, 576, 512, 64, "bf16",
               ctx_range=(2048, 8192), mla=True, scale=1.0 / math.sqrt(576), index=5),
}


@dataclass
class Workload:
    spec: Spec
    seed: int
    q: np.ndarray  # [B, Hq, dk] float32 or uint16 (bf16 bits)
    k_cache: np.ndarray  # [N, bs, Hkv, dk]
    v_cache: Optional[np.ndarray]  # [N, bs, Hkv, dv] or None for the latent cache
    block_tables: np.ndarray  # [B, max_blocks] int32, -1 padded
    context_lens: np.ndarray  # [B] int32
    k_new: np.ndarray  # [B, Hkv, dk]
    v_new: Optional[np.ndarray]  # [B, Hkv, dv] or None
    slot_mapping: np.ndarray  # [B] int32: slot of position context_lens[b]
    blocks_used: np.ndarray = field(default=None)  # [B] blocks each sequence owns

    @property
    def scale(self) -> float:
        return self.spec.softmax_scale

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_f32(ss: np.random.SeedSequence, n: int) -> np.ndarray:
    """n standard-normal float32 values, chunk i drawn from ss.spawn()[i]."""
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // CHUNK))
    kids = ss.spawn(nchunks)

    def fill(i: int) -> None:
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        if hi > lo:
            g = np.random.Generator(np.random.PCG64(kids[i]))
            g.standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 bit patterns."""
    import torch  # plumbing only: a fast multi-threaded RNE cast

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _values(ss: np.random.SeedSequence, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    f = _normal_f32(ss, n)
    if dtype == "f32":
        return f.reshape(shape)
    return f32_to_bf16_bits(f).reshape(shape)


def _nan_value(dtype: str):
    return F32_NAN_BITS.view(np.float32) if dtype == "f32" else BF16_NAN


def make_workload(spec, seed: Optional[int] = None, poison: bool = True,
                  context_lens: Optional[Sequence[int]] = None) -> Workload:
    """Build a seeded workload for ``spec`` (a Spec or a name in CONFIGS).

    ``context_lens`` overrides the drawn lengths (the draw still happens so the
    other arrays stay the same for a given seed).  With ``poison`` every pool
    slot no sequence attends to (the tail of each sequence's last blocks and
    every unused block) holds NaN, so a kernel that reads past a context shows.
    """
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if seed is None:
        seed = BASE_SEED + spec.index
    root = np.random.SeedSequence(seed)
    ss_ctx, ss_perm, ss_q, ss_k, ss_v, ss_new = root.spawn(6)
    B, bs = spec.num_seqs, spec.block_size

    # 1. context lengths
    if spec.ctx_fixed is not None:
        ctx = np.array(spec.ctx_fixed, dtype=np.int64)
    else:
        lo, hi = spec.ctx_range
        ctx = np.random.Generator(np.random.PCG64(ss_ctx)).integers(
            lo, hi, size=B, endpoint=True)
    if context_lens is not None:
        ctx = np.asarray(context_lens, dtype=np.int64)
        assert ctx.shape == (B,)
    max_blocks = max(spec.max_blocks_per_seq, int(-(-(ctx.max(initial=0) + 1) // bs)))

    # 2. pool and block tables: each sequence owns ceil((ctx+1)/bs) blocks (room
    # for one appended token), taken as consecutive slices of a random
    # permutation of the pool.
    used = -(-(ctx + 1) // bs)
    total = int(used.sum())
    N = spec.pool_blocks if spec.pool_blocks is not None else total
    N = max(N, total)
    perm = np.random.Generator(np.random.PCG64(ss_perm)).permutation(N).astype(np.int32)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, : used[b]] = perm[off: off + used[b]]
        off += used[b]

    Hq, Hkv, dk, dv = spec.num_q_heads, spec.num_kv_heads, spec.head_dim_k, spec.head_dim_v
    # 3.-5. q, K pool, V pool
    q = _values(ss_q, (B, Hq, dk), spec.dtype)
    k_cache = _values(ss_k, (N, bs, Hkv, dk), spec.dtype)
    v_cache = None if spec.mla else _values(ss_v, (N, bs, Hkv, dv), spec.dtype)
    # 6. the new token's k and v for the append step
    kv_new = _values(ss_new, (B, Hkv, dk + (0 if spec.mla else dv)), spec.dtype)
    k_new = np.ascontiguousarray(kv_new[:, :, :dk])
    v_new = None if spec.mla else np.ascontiguousarray(kv_new[:, :, dk:])

    # slot of logical position ctx_b: physical block * bs + offset in block
    slot = np.empty(B, dtype=np.int32)
    for b in range(B):
        slot[b] = bt[b, ctx[b] // bs] * bs + ctx[b] % bs

    if poison:
        nan = _nan_value(spec.dtype)
        owned = np.zeros(N, dtype=bool)
        for b in range(B):
            owned[bt[b, : used[b]]] = True
            for t in range(int(ctx[b]), int(used[b]) * bs):
                p, r = bt[b, t // bs], t % bs
                k_cache[p, r] = nan
                if v_cache is not None:
                    v_cache[p, r] = nan
        k_cache[~owned] = nan
        if v_cache is not None:
            v_cache[~owned] = nan

    return Workload(spec=spec, seed=seed, q=q, k_cache=k_cache, v_cache=v_cache,
                    block_tables=bt, context_lens=ctx.astype(np.int32), k_new=k_new,
                    v_new=v_new, slot_mapping=slot, blocks_used=used.astype(np.int32))


def custom_spec(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
                ctx, head_dim_v=None, mla=False, pool_blocks=None, scale=None,
                name="custom") -> Spec:
    return Spec(name, num_seqs, num_q_heads, num_kv_heads, head_dim,
                head_dim if head_dim_v is None else head_dim_v, block_size, dtype,
                ctx_fixed=tuple(int(c) for c in ctx), mla=mla,
                pool_blocks=pool_blocks, scale=scale)


# ---------------------------------------------------------------------------
# Accounting (measurement, not method arithmetic).
# ---------------------------------------------------------------------------

def kv_bytes_per_token_layer(num_kv_heads, head_dim_k, head_dim_v, elt, mla=False) -> int:
    """Bytes of cached K and V one token holds in one layer.

    Matches the pages' count 2 * kv_heads * head_dim * bytes ("Mathématiques de
    cache KV"); a latent cache stores its row once because V is a view of it.
    """
    if mla:
        return num_kv_heads * head_dim_k * elt
    return num_kv_heads * (head_dim_k + head_dim_v) * elt


def algorithmic_bytes(w: Workload) -> int:
    """HBM bytes one decode call must move: every attended K/V row once, q, O,
    the block ids it dereferences, and the context lengths."""
    s = w.spec
    ctx = w.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * kv_bytes_per_token_layer(s.num_kv_heads, s.head_dim_k,
                                                     s.head_dim_v, s.elt, s.mla)
    q = s.num_seqs * s.num_q_heads * s.head_dim_k * s.elt
    o = s.num_seqs * s.num_q_heads * s.head_dim_v * s.elt
    ids = 4 * int((-(-ctx // s.block_size)).sum())
    return kv + q + o + ids + 4 * s.num_seqs


def kv_read_bytes(w: Workload) -> int:
    s = w.spec
    return int(w.context_lens.astype(np.int64).sum()) * kv_bytes_per_token_layer(
        s.num_kv_heads, s.head_dim_k, s.head_dim_v, s.elt, s.mla)


def algorithmic_flops(w: Workload) -> int:
    """2 flops per multiply-add of q.k and p.v over every attended token."""
    s = w.spec
    return 2 * s.num_q_heads * (s.head_dim_k + s.head_dim_v) * int(
        w.context_lens.astype(np.int64).sum())


def append_bytes(w: Workload) -> int:
    s = w.spec
    row = s.num_kv_heads * (s.head_dim_k + (0 if s.mla else s.head_dim_v)) * s.elt
    return 2 * row * int((w.slot_mapping >= 0).sum()) + 4 * s.num_seqs


# MXFP8 caches: one E4M3 byte per value plus one E8M0 byte per 32 values.
MX_BLOCK = 32


def mxfp8_kv_bytes_per_token_layer(num_kv_heads, head_dim) -> int:
    return 2 * num_kv_heads * (head_dim + head_dim // MX_BLOCK)


def algorithmic_bytes_mxfp8(w: Workload) -> int:
    """algorithmic_bytes() with the K/V rows stored as MXFP8 (q and O stay in
    the workload's dtype)."""
    s = w.spec
    ctx = w.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * mxfp8_kv_bytes_per_token_layer(s.num_kv_heads, s.head_dim_k)
    q = s.num_seqs * s.num_q_heads * s.head_dim_k * s.elt
    o = s.num_seqs * s.num_q_heads * s.head_dim_v * s.elt
    ids = 4 * int((-(-ctx // s.block_size)).sum())
    return kv + q + o + ids + 4 * s.num_seqs


def append_bytes_mxfp8(w: Workload) -> int:
    """Bytes one quantizing append moves: the source rows read, codes and
    scales written, and the slot ids."""
    s = w.spec
    n = int((w.slot_mapping >= 0).sum())
    src = 2 * s.num_kv_heads * s.head_dim_k * s.elt
    return n * (src + mxfp8_kv_bytes_per_token_layer(s.num_kv_heads, s.head_dim_k)) + 4 * s.num_seqs


def multi_query(w: Workload, q_len: int) -> np.ndarray:
    """Seeded queries for q_len new tokens per sequence, [B, q_len, Hq, d_k] in
    the workload's dtype, drawn from their own branch of the workload's seed
    (independent of every other array)."""
    s = w.spec
    ss = np.random.SeedSequence([w.seed, 1000 + q_len])
    return _values(ss, (s.num_seqs, q_len, s.num_q_heads, s.head_dim_k), s.dtype)
