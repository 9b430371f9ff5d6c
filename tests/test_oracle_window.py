"""Pins of the oracle's sliding-window decode, log-sum-exp and per-token
attention mass: the pinned C decode (no window), torch SDPA and
torch.logsumexp / softmax on contiguous windows, and closed forms."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import pack_paged, sdpa_reference


def _case(seed, lens, hkv=2, G=4, d=16, bs=8):
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vs = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    kp, bt = pack_paged(ks, bs, pool_blocks=sum(-(-L // bs) for L in lens) + 2, rng=np.random.default_rng(seed))
    vp, _ = pack_paged(vs, bs, pool_blocks=sum(-(-L // bs) for L in lens) + 2, rng=np.random.default_rng(seed))
    q = rng.standard_normal((len(lens), hkv * G, d)).astype(np.float32)
    return q, ks, vs, kp, vp, bt, np.array(lens, np.int32)


def test_no_window_equals_the_c_oracle():
    q, ks, vs, kp, vp, bt, cl = _case(1, [1, 9, 40, 77])
    o, lse = oracle.decode_window(q, kp, vp, bt, cl, 0.3, window=0)
    assert np.allclose(o, oracle.decode(q, kp, vp, bt, cl, 0.3), rtol=1e-12, atol=1e-14)
    o2, lse2 = oracle.decode_window(q, kp, vp, bt, cl, 0.3, window=1000)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("window", [1, 5, 16, 33])
def test_window_matches_sdpa_on_the_contiguous_window(window):
    q, ks, vs, kp, vp, bt, cl = _case(2, [3, 20, 64, 90])
    o, lse = oracle.decode_window(q, kp, vp, bt, cl, 0.25, window=window)
    for b, L in enumerate(cl):
        st = max(0, L - window)
        K, V = ks[b][st:], vs[b][st:]
        assert np.allclose(o[b], sdpa_reference(q[b], K, V, 0.25), rtol=1e-12, atol=1e-13)
        G = q.shape[1] // K.shape[1]
        s = torch.einsum("hd,thd->ht", torch.as_tensor(q[b], dtype=torch.float64),
                         torch.as_tensor(K, dtype=torch.float64).repeat_interleave(G, 1)) * 0.25
        assert np.allclose(lse[b], torch.logsumexp(s, dim=1).numpy(), rtol=1e-13, atol=1e-13)


def test_window_one_returns_the_last_value():
    q, ks, vs, kp, vp, bt, cl = _case(3, [7, 30])
    o, lse = oracle.decode_window(q, kp, vp, bt, cl, 0.5, window=1)
    for b, L in enumerate(cl):
        G = q.shape[1] // ks[b].shape[1]
        for h in range(q.shape[1]):
            assert np.array_equal(o[b, h], vs[b][L - 1, h // G].astype(np.float64))
            assert lse[b, h] == 0.5 * float(np.dot(q[b, h].astype(np.float64),
                                                   ks[b][L - 1, h // G].astype(np.float64)))


def test_empty_context():
    q, ks, vs, kp, vp, bt, cl = _case(4, [5, 9])
    o, lse = oracle.decode_window(q, kp, vp, bt, np.array([0, 9], np.int32), 0.5)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("window", [0, 12])
def test_scores_are_the_groups_softmax_mass(window):
    q, ks, vs, kp, vp, bt, cl = _case(5, [4, 25, 60])
    _, lse = oracle.decode_window(q, kp, vp, bt, cl, 0.4, window=window)
    sc = oracle.attention_scores(q, kp, bt, cl, lse, 0.4, window=window, max_context=64)
    G = q.shape[1] // ks[0].shape[1]
    for b, L in enumerate(cl):
        st = max(0, L - window) if window else 0
        assert np.all(sc[b, :, :st] == 0) and np.all(sc[b, :, L:] == 0)
        assert np.allclose(sc[b].sum(axis=1), G, rtol=1e-12)   # each head's weights sum to 1
        K = torch.as_tensor(ks[b][st:L], dtype=torch.float64)
        for g in range(K.shape[1]):
            qg = torch.as_tensor(q[b, g * G:(g + 1) * G], dtype=torch.float64)
            p = torch.softmax(0.4 * qg @ K[:, g].T, dim=1).sum(0).numpy()
            assert np.allclose(sc[b, g, st:L], p, rtol=1e-12, atol=1e-15)
