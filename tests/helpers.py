"""Independent test helpers: contiguous-layout references and a paged packer.

Nothing here is shared with the oracle or the HIP library.  The packer places
contiguous per-sequence K/V into a block pool by whole blocks (reshape and
fancy indexing), so it does not repeat the per-token index arithmetic that the
oracle uses to read the pool back.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import bf16_bits_to_f32


def pack_paged(seqs, bs, pool_blocks=None, rng=None, fill=0.0, dtype=np.float32):
    """seqs: list of arrays [L_b, Hkv, d].  Returns (pool [N, bs, Hkv, d],
    block_tables [B, max_blocks] int32 padded with -1)."""
    rng = np.random.default_rng(0) if rng is None else rng
    Hkv, d = seqs[0].shape[1], seqs[0].shape[2]
    nblk = [max(1, -(-s.shape[0] // bs)) for s in seqs]
    total = sum(nblk)
    N = total if pool_blocks is None else max(pool_blocks, total)
    perm = rng.permutation(N)
    pool = np.full((N, bs, Hkv, d), fill, dtype=dtype)
    maxb = max(nblk)
    bt = np.full((len(seqs), maxb), -1, dtype=np.int32)
    off = 0
    for b, s in enumerate(seqs):
        n = nblk[b]
        padded = np.full((n * bs, Hkv, d), fill, dtype=dtype)
        padded[: s.shape[0]] = s
        ids = perm[off: off + n]
        pool[ids] = padded.reshape(n, bs, Hkv, d)
        bt[b, :n] = ids
        off += n
    return pool, bt


def sdpa_reference(q, K, V, scale):
    """torch scaled_dot_product_attention in float64 on the CPU.

    q [Hq, dk], K [L, Hkv, dk], V [L, Hkv, dv]; KV heads are repeated so that
    query head h reads KV head h // (Hq / Hkv)."""
    q = torch.as_tensor(np.asarray(q, dtype=np.float64))
    K = torch.as_tensor(np.asarray(K, dtype=np.float64))
    V = torch.as_tensor(np.asarray(V, dtype=np.float64))
    Hq, Hkv = q.shape[0], K.shape[1]
    G = Hq // Hkv
    Kh = K.permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, dk]
    Vh = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], Kh, Vh, scale=float(scale))
    return out[:, 0, :].numpy()


def numpy_textbook(q, K, V, scale):
    """Max-subtracted softmax attention for one query per head, numpy float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    G = q.shape[0] // K.shape[1]
    Kh = np.repeat(K.transpose(1, 0, 2), G, axis=0)
    Vh = np.repeat(V.transpose(1, 0, 2), G, axis=0)
    s = np.einsum("hd,hld->hl", q, Kh) * scale
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return np.einsum("hl,hld->hd", w, Vh)


def as_f64(x):
    """Widen float32 or bf16 bit patterns to float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def gather_sequence(pool, block_tables, b, L):
    """Contiguous [L, Hkv, d] view of sequence b, gathered by whole blocks."""
    bs = pool.shape[1]
    n = -(-L // bs)
    ids = block_tables[b, :n]
    return pool[ids].reshape(n * bs, *pool.shape[2:])[:L]
