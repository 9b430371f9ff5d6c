"""Pins of the oracle's multi-query decode (several new tokens per sequence,
causal among themselves).

The oracle composes the pinned single-query decode over each query's visible
prefix.  These checks come from elsewhere: torch's scaled_dot_product_attention
with a boolean mask built from the pages' upper-triangular rule (query i of
the last sq sees keys j <= i + sk - sq, "Étape 2: Attention avec KV Cache"),
the pages' own additive -1e9 form in numpy, and closed-form cases.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import pack_paged


def causal_sdpa(q, K, V, scale):
    """q [Q, Hq, d], K/V [L, Hkv, d] contiguous; the last Q keys are the queries'."""
    Q, Hq, _ = q.shape
    L, Hkv = K.shape[0], K.shape[1]
    G = Hq // Hkv
    mask = ~np.triu(np.ones((Q, L), dtype=bool), k=L - Q + 1)  # True = attend
    qt = torch.as_tensor(q, dtype=torch.float64).permute(1, 0, 2)  # [Hq, Q, d]
    Kt = torch.as_tensor(K, dtype=torch.float64).permute(1, 0, 2).repeat_interleave(G, 0)
    Vt = torch.as_tensor(V, dtype=torch.float64).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=torch.as_tensor(mask),
                                                         scale=float(scale))
    return o.permute(1, 0, 2).numpy()


def pages_formula(q, K, V, scale):
    """The pages' masked softmax in float64: scores + triu mask * (-1e9)."""
    Q, Hq, _ = q.shape
    L, Hkv = K.shape[0], K.shape[1]
    G = Hq // Hkv
    out = np.empty(q.shape[:2] + (V.shape[2],))
    mask = np.triu(np.ones((Q, L)), k=L - Q + 1)
    for h in range(Hq):
        s = q[:, h].astype(np.float64) @ K[:, h // G].astype(np.float64).T * scale + mask * -1e9
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = (w / w.sum(axis=1, keepdims=True)) @ V[:, h // G].astype(np.float64)
    return out


def test_visible_lengths():
    v = oracle.visible_lengths(np.array([5, 2, 0, 8, 3]), 3)
    assert v.tolist() == [[3, 4, 5], [0, 1, 2], [0, 0, 0], [6, 7, 8], [1, 2, 3]]


@pytest.mark.parametrize("Q", [1, 3, 8])
def test_multi_matches_masked_sdpa_and_pages_formula(Q):
    rng = np.random.default_rng(40 + Q)
    lens = [Q, Q + 5, 40, 77]
    hkv, G, d, bs = 2, 4, 16, 8
    ks = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vs = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    kp, bt = pack_paged(ks, bs, pool_blocks=30, rng=np.random.default_rng(5))
    vp, _ = pack_paged(vs, bs, pool_blocks=30, rng=np.random.default_rng(5))
    q = rng.standard_normal((len(lens), Q, hkv * G, d)).astype(np.float32)
    got = oracle.decode_multi(q, kp, vp, bt, np.array(lens, np.int32), 0.3)
    for b in range(len(lens)):
        assert np.allclose(got[b], causal_sdpa(q[b], ks[b], vs[b], 0.3), rtol=1e-12, atol=1e-13)
        assert np.allclose(got[b], pages_formula(q[b], ks[b], vs[b], 0.3), rtol=1e-12, atol=1e-13)


def test_multi_with_one_query_is_the_single_query_decode():
    rng = np.random.default_rng(50)
    lens = [3, 30, 64]
    ks = [rng.standard_normal((L, 1, 8)).astype(np.float32) for L in lens]
    kp, bt = pack_paged(ks, 4, rng=np.random.default_rng(1))
    vp, _ = pack_paged([k * 2 for k in ks], 4, rng=np.random.default_rng(1))
    q = rng.standard_normal((3, 1, 2, 8)).astype(np.float32)
    cl = np.array(lens, np.int32)
    a = oracle.decode_multi(q, kp, vp, bt, cl, 0.5)[:, 0]
    b = oracle.decode(np.ascontiguousarray(q[:, 0]), kp, vp, bt, cl, 0.5)
    assert np.array_equal(a, b)


def test_fresh_chunk_first_query_sees_only_the_first_token():
    """L == q_len (a chunk that starts the sequence): query 0 attends to
    token 0 alone, so its output is exactly v_0; the last query sees all."""
    rng = np.random.default_rng(51)
    L = Q = 6
    K = rng.standard_normal((L, 1, 8)).astype(np.float32)
    V = rng.standard_normal((L, 1, 8)).astype(np.float32)
    kp, bt = pack_paged([K], 4)
    vp, _ = pack_paged([V], 4)
    q = rng.standard_normal((1, Q, 1, 8)).astype(np.float32)
    got = oracle.decode_multi(q, kp, vp, bt, np.array([L], np.int32), 0.7)
    assert np.array_equal(got[0, 0, 0], V[0, 0].astype(np.float64))
    full = oracle.decode(np.ascontiguousarray(q[:, -1]), kp, vp, bt, np.array([L], np.int32), 0.7)
    assert np.array_equal(got[0, -1], full[0])
