"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: a library routine on a
contiguous layout, a closed form, an invariant the pages state, or numbers the
pages print.  A planted-mistake test (test_oracle_mutants.py) checks that these
pins catch plausible slips in the oracle's code.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from tests.helpers import (as_f64, gather_sequence, numpy_textbook, pack_paged,
                           sdpa_reference)
from workloads import CONFIGS, custom_spec, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_seqs(rng, lens, Hkv, d):
    return [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]


# --- P-1: paged oracle == library attention on the contiguous layout ----------

@pytest.mark.parametrize("lens,Hq,Hkv,d,bs", [
    ([1, 5, 16, 17], 4, 2, 64, 16),
    ([300, 33, 2], 8, 8, 32, 16),
    ([100, 250], 8, 1, 64, 16),
    ([64, 65, 7], 6, 3, 16, 8),
    ([129], 2, 2, 48, 64),
])
def test_p1_paged_matches_contiguous_sdpa(lens, Hq, Hkv, d, bs):
    rng = np.random.default_rng(1234 + sum(lens))
    ks = _rand_seqs(rng, lens, Hkv, d)
    vs = _rand_seqs(rng, lens, Hkv, d)
    q = rng.standard_normal((len(lens), Hq, d)).astype(np.float32)
    prng = np.random.default_rng(99)
    kpool, bt = pack_paged(ks, bs, pool_blocks=sum(-(-L // bs) for L in lens) + 3,
                           rng=np.random.default_rng(5))
    vpool, bt2 = pack_paged(vs, bs, pool_blocks=kpool.shape[0], rng=np.random.default_rng(5))
    assert np.array_equal(bt, bt2)
    scale = 1.0 / math.sqrt(d)
    got = oracle.decode(q, kpool, vpool, bt, np.array(lens, np.int32), scale)
    for b, L in enumerate(lens):
        ref = sdpa_reference(q[b], ks[b], vs[b], scale)
        ref2 = numpy_textbook(q[b], ks[b], vs[b], scale)
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got[b], ref2, rtol=1e-12, atol=1e-13)
    del prng


def test_p1_config1_matches_sdpa_on_gathered_blocks():
    """c1 exactly: oracle vs library attention on sequences gathered by blocks."""
    w = make_workload("c1")
    got = oracle.decode_workload(w)
    for b in range(w.spec.num_seqs):
        L = int(w.context_lens[b])
        K = gather_sequence(w.k_cache, w.block_tables, b, L)
        V = gather_sequence(w.v_cache, w.block_tables, b, L)
        assert np.isfinite(K).all() and np.isfinite(V).all()
        ref = sdpa_reference(w.q[b], K, V, w.scale)
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-13)


def test_p1_bf16_widening_matches_numpy():
    """bf16 inputs: the oracle equals itself run on numpy-widened float32 copies."""
    w = make_workload(custom_spec(3, 4, 2, 64, 16, "bf16", ctx=[40, 1, 77]))
    got = oracle.decode_workload(w)
    f = oracle.decode(workloads.bf16_bits_to_f32(w.q), workloads.bf16_bits_to_f32(w.k_cache),
                      workloads.bf16_bits_to_f32(w.v_cache), w.block_tables, w.context_lens,
                      w.scale)
    assert np.array_equal(got, f)
    for b in range(3):
        L = int(w.context_lens[b])
        K = as_f64(gather_sequence(w.k_cache, w.block_tables, b, L))
        V = as_f64(gather_sequence(w.v_cache, w.block_tables, b, L))
        np.testing.assert_allclose(got[b], sdpa_reference(as_f64(w.q[b]), K, V, w.scale),
                                   rtol=1e-12, atol=1e-13)


def test_p1_latent_mode_matches_sdpa():
    """Latent cache: V is the leading dv values of each 576-wide K row."""
    spec = custom_spec(2, 8, 1, 576, 64, "bf16", ctx=[70, 130], head_dim_v=512, mla=True,
                       scale=1.0 / math.sqrt(576))
    w = make_workload(spec)
    assert w.v_cache is None
    got = oracle.decode_workload(w)
    assert got.shape == (2, 8, 512)
    for b in range(2):
        L = int(w.context_lens[b])
        K = as_f64(gather_sequence(w.k_cache, w.block_tables, b, L))
        ref = sdpa_reference(as_f64(w.q[b]), K, K[:, :, :512], w.scale)
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-13)


# --- closed forms ---------------------------------------------------------------

def test_closed_form_two_tokens():
    """q = a e0, k0 = e0, k1 = 0: O = (e^{a s} v0 + v1) / (e^{a s} + 1)."""
    d, a, scale = 8, 3.0, 0.5
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = a
    K = np.zeros((2, 1, d), np.float32)
    K[0, 0, 0] = 1.0
    V = np.arange(2 * d, dtype=np.float32).reshape(2, 1, d) / 7.0
    pool_k, bt = pack_paged([K], 4)
    pool_v, _ = pack_paged([V], 4)
    got = oracle.decode(q, pool_k, pool_v, bt, np.array([2], np.int32), scale)[0, 0]
    e = math.exp(a * scale)
    want = (e * V[0, 0].astype(np.float64) + V[1, 0]) / (e + 1.0)
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=1e-15)


# --- P-2 .. P-9: invariants ---------------------------------------------------

def test_p2_block_permutation_is_bitwise_invariant():
    w = make_workload("c1")
    base = oracle.decode_workload(w)
    rng = np.random.default_rng(7)
    pi = rng.permutation(w.num_blocks).astype(np.int32)
    kp = np.empty_like(w.k_cache)
    vp = np.empty_like(w.v_cache)
    kp[pi] = w.k_cache
    vp[pi] = w.v_cache
    bt = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    got = oracle.decode(w.q, kp, vp, bt, w.context_lens, w.scale)
    assert np.array_equal(got, base)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p3_context_one_returns_v_exactly(dtype):
    w = make_workload(custom_spec(3, 4, 2, 64, 16, dtype, ctx=[1, 1, 1]))
    got = oracle.decode_workload(w)
    for b in range(3):
        blk = w.block_tables[b, 0]
        v0 = as_f64(w.v_cache[blk, 0])  # [Hkv, d]
        want = np.repeat(v0, 2, axis=0)
        assert np.array_equal(got[b], want)


def test_p4_identical_keys_and_zero_scale_give_mean_of_v():
    rng = np.random.default_rng(3)
    L, Hkv, d = 37, 2, 16
    krow = rng.standard_normal((1, Hkv, d)).astype(np.float32)
    K = np.repeat(krow, L, axis=0)
    V = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    kp, bt = pack_paged([K], 16, rng=np.random.default_rng(1))
    vp, _ = pack_paged([V], 16, rng=np.random.default_rng(1))
    mean = np.repeat(V.astype(np.float64).mean(axis=0), 2, axis=0)
    got = oracle.decode(q, kp, vp, bt, np.array([L], np.int32), 0.25)[0]
    np.testing.assert_allclose(got, mean, rtol=0, atol=1e-13)
    # scale = 0 makes every score equal for arbitrary keys
    K2 = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    kp2, _ = pack_paged([K2], 16, rng=np.random.default_rng(1))
    got2 = oracle.decode(q, kp2, vp, bt, np.array([L], np.int32), 0.0)[0]
    np.testing.assert_allclose(got2, mean, rtol=0, atol=1e-13)


def test_p5_gqa_equals_mha_with_repeated_kv_heads():
    w = make_workload(custom_spec(2, 8, 2, 32, 16, "f32", ctx=[45, 90]))
    got = oracle.decode_workload(w)
    G = 4
    k_rep = np.ascontiguousarray(np.repeat(w.k_cache, G, axis=2))
    v_rep = np.ascontiguousarray(np.repeat(w.v_cache, G, axis=2))
    mha = oracle.decode(w.q, k_rep, v_rep, w.block_tables, w.context_lens, w.scale)
    assert np.array_equal(got, mha)


def test_p6_one_dominant_key_selects_its_value():
    rng = np.random.default_rng(11)
    L, d, star = 50, 32, 23
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    K = rng.standard_normal((L, 1, d)).astype(np.float32)
    K[star, 0] = (50.0 * q[0, 0] / np.linalg.norm(q[0, 0])).astype(np.float32)
    V = rng.standard_normal((L, 1, d)).astype(np.float32)
    kp, bt = pack_paged([K], 16)
    vp, _ = pack_paged([V], 16)
    scale = 1.0
    got = oracle.decode(q, kp, vp, bt, np.array([L], np.int32), scale)[0, 0]
    s = (K[:, 0].astype(np.float64) @ q[0, 0].astype(np.float64)) * scale
    gap = s[star] - np.delete(s, star).max()
    assert gap > 30
    bound = (L - 1) * math.exp(-gap) * 2 * np.abs(V).max()
    assert np.abs(got - V[star, 0]).max() <= bound + 1e-15


def test_p6_scores_beyond_exp_range_stay_finite():
    """Max subtraction (step 2 of the first page's attention): scores of ~1000
    give the top key's value, not inf/NaN."""
    q = np.zeros((1, 1, 4), np.float32)
    q[0, 0, 0] = 1.0
    K = np.zeros((3, 1, 4), np.float32)
    K[:, 0, 0] = [10.0, 1.0, 0.0]
    V = np.arange(12, dtype=np.float32).reshape(3, 1, 4)
    kp, bt = pack_paged([K], 2)
    vp, _ = pack_paged([V], 2)
    got = oracle.decode(q, kp, vp, bt, np.array([3], np.int32), 100.0)[0, 0]
    # the runner-up weight is exp(-100) relative: far below double rounding of V
    assert np.array_equal(got, V[0, 0].astype(np.float64))


def _tile_stats(q, K, V, scale):
    """One tile on its own: its largest score m, l = sum of exp(s - m) over
    the tile, and the tile's own normalised output."""
    sc = (K @ q) * scale
    m = float(sc.max())
    e = np.exp(sc - m)
    l = float(e.sum())
    return (e @ V) / l, m, l


def _fold(a, b):
    """Combine two (normalised output, max, sum) triples over disjoint token
    sets into the triple of their union: the running max is the larger max,
    each side's sum is re-referenced to it, and the outputs mix in proportion
    to the re-referenced sums ('Étape 2: softmax en carreaux' keeps exactly
    this pair of running statistics while it walks the tiles)."""
    (oa, ma, la), (ob, mb, lb) = a, b
    m = max(ma, mb)
    wa, wb = la * math.exp(ma - m), lb * math.exp(mb - m)
    return (wa * oa + wb * ob) / (wa + wb), m, wa + wb


def _tiled_attention(q, K, V, scale, tile):
    """One query vector over K, V cut into tiles of `tile` tokens: every
    tile's statistics formed alone, then folded left to right, float64."""
    acc = None
    for start in range(0, K.shape[0], tile):
        t = _tile_stats(q, K[start:start + tile], V[start:start + tile], scale)
        acc = t if acc is None else _fold(acc, t)
    return acc


def _merge_partitions(parts):
    """Combine (acc, m, l) partials into one output by log-sum-exp weights."""
    M = max(p[1] for p in parts)
    num = sum(math.exp(p[1] - M) * p[0] * p[2] for p in parts)
    den = sum(math.exp(p[1] - M) * p[2] for p in parts)
    return num / den


@pytest.mark.parametrize("tile", [1, 3, 16, 512])
def test_p7_tiled_and_partitioned_equal_one_shot(tile):
    w = make_workload(custom_spec(2, 4, 2, 64, 16, "f32", ctx=[700, 130]))
    got = oracle.decode_workload(w)
    for b in range(2):
        L = int(w.context_lens[b])
        K = gather_sequence(w.k_cache, w.block_tables, b, L).astype(np.float64)
        V = gather_sequence(w.v_cache, w.block_tables, b, L).astype(np.float64)
        for h in range(4):
            g = h // 2
            qv = w.q[b, h].astype(np.float64)
            o, _, _ = _tiled_attention(qv, K[:, g], V[:, g], w.scale, tile)
            np.testing.assert_allclose(o, got[b, h], rtol=1e-12, atol=1e-13)
            # split into partitions of `part` tokens, each tiled, then merged
            part = max(tile, 64)
            parts = [_tiled_attention(qv, K[s:s + part, g], V[s:s + part, g], w.scale, tile)
                     for s in range(0, L, part)]
            np.testing.assert_allclose(_merge_partitions(parts), got[b, h], rtol=1e-12,
                                       atol=1e-13)


def test_p8_block_size_invariance():
    rng = np.random.default_rng(21)
    lens = [200, 64, 5]
    ks = _rand_seqs(rng, lens, 2, 32)
    vs = _rand_seqs(rng, lens, 2, 32)
    q = rng.standard_normal((3, 4, 32)).astype(np.float32)
    outs = []
    for bs in (16, 64):
        kp, bt = pack_paged(ks, bs, rng=np.random.default_rng(bs))
        vp, _ = pack_paged(vs, bs, rng=np.random.default_rng(bs))
        outs.append(oracle.decode(q, kp, vp, bt, np.array(lens, np.int32), 0.2))
    assert np.array_equal(outs[0], outs[1])


def test_p9_poison_outside_context_is_never_read():
    w = make_workload("c1", poison=True)
    clean = make_workload("c1", poison=False)
    a = oracle.decode_workload(w)
    k = np.where(np.isnan(w.k_cache), np.float32(0), w.k_cache)
    v = np.where(np.isnan(w.v_cache), np.float32(0), w.v_cache)
    b = oracle.decode(w.q, k, v, w.block_tables, w.context_lens, w.scale)
    assert np.isfinite(a).all()
    assert np.array_equal(a, b)
    assert np.array_equal(a, oracle.decode_workload(clean))


def test_context_zero_gives_zero():
    w = make_workload(custom_spec(2, 2, 1, 16, 16, "f32", ctx=[0, 3]))
    got = oracle.decode_workload(w)
    assert np.array_equal(got[0], np.zeros((2, 16)))
    assert np.isfinite(got[1]).all()


# --- P-10: append ---------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c5"])
def test_p10_append_bitwise_and_skip(name):
    if name == "c5":
        spec = custom_spec(3, 8, 1, 576, 64, "bf16", ctx=[63, 64, 200], head_dim_v=512,
                           mla=True)
        w = make_workload(spec)
    else:
        w = make_workload(name)
    k0 = w.k_cache.copy()
    v0 = None if w.v_cache is None else w.v_cache.copy()
    slots = w.slot_mapping.copy()
    slots[1] = -1
    oracle.append(w.k_cache, w.v_cache, w.k_new, w.v_new, slots)
    # independent expectation: scatter rows into a flat [slots, row] view
    ek = k0.reshape(-1, k0.shape[2] * k0.shape[3]).copy()
    for i, s in enumerate(slots):
        if s >= 0:
            ek[s] = w.k_new[i].reshape(-1)
    assert np.array_equal(w.k_cache.reshape(ek.shape).view(np.uint8), ek.view(np.uint8))
    if v0 is not None:
        ev = v0.reshape(-1, v0.shape[2] * v0.shape[3]).copy()
        for i, s in enumerate(slots):
            if s >= 0:
                ev[s] = w.v_new[i].reshape(-1)
        assert np.array_equal(w.v_cache.reshape(ev.shape).view(np.uint8), ev.view(np.uint8))
    # all -1: nothing changes
    k1 = w.k_cache.copy()
    oracle.append(w.k_cache, w.v_cache, w.k_new, w.v_new, np.full_like(slots, -1))
    assert np.array_equal(k1.view(np.uint8), w.k_cache.view(np.uint8))


def test_p10_append_then_decode_equals_contiguous():
    """Cached decode after appending the new token == attention over [K; k_new]."""
    w = make_workload("c1")
    oracle.append(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping)
    L1 = w.context_lens + 1
    got = oracle.decode_workload(w, context_lens=L1)
    for b in range(w.spec.num_seqs):
        L = int(w.context_lens[b])
        K = gather_sequence(w.k_cache, w.block_tables, b, L)
        V = gather_sequence(w.v_cache, w.block_tables, b, L)
        K1 = np.concatenate([K, w.k_new[b][None]], axis=0)
        V1 = np.concatenate([V, w.v_new[b][None]], axis=0)
        np.testing.assert_allclose(got[b], sdpa_reference(w.q[b], K1, V1, w.scale),
                                   rtol=1e-12, atol=1e-13)


def test_append_rejects_out_of_range_slot():
    w = make_workload("c1")
    bad = w.slot_mapping.copy()
    bad[0] = w.num_blocks * w.spec.block_size
    with pytest.raises(RuntimeError):
        oracle.append(w.k_cache, w.v_cache, w.k_new, w.v_new, bad)


# --- P-11: byte accounting against the pages' printed numbers -------------------

def test_p11_bytes_match_pages():
    with open(os.path.join(GOLDEN, "kv_bytes_pages.json")) as f:
        entries = json.load(f)["entries"]
    for e in entries:
        per = workloads.kv_bytes_per_token_layer(e["kv_heads"], e["head_dim"], e["head_dim"],
                                                 e["elt_bytes"])
        total = per * e["layers"] * e.get("tokens", 1)
        assert total == e["bytes"], e["what"]


def test_p11_config_bytes():
    s3, s4 = CONFIGS["c3"], CONFIGS["c4"]
    assert workloads.kv_bytes_per_token_layer(s3.num_kv_heads, 128, 128, 2) == 4096
    # c4: 4 sequences x 131072 tokens x 4 KB = 2 GiB of K/V for one layer
    assert 4 * 131072 * 4096 == 2 ** 31
    s2 = CONFIGS["c2"]
    assert workloads.kv_bytes_per_token_layer(s2.num_kv_heads, 128, 128, 2) == 16384
    s5 = CONFIGS["c5"]
    assert workloads.kv_bytes_per_token_layer(1, 576, 512, 2, mla=True) == 1152
    assert s4.max_blocks_per_seq == 8193 and s5.max_blocks_per_seq == 129


def test_sampled_rows_with_duplicates_match_full_decode():
    """Row sampling (used at full sizes) equals the full decode, duplicates included."""
    w = make_workload(custom_spec(3, 8, 2, 32, 16, "f32", ctx=[50, 400, 7]))
    full = oracle.decode_workload(w)
    pairs = [(1, 3), (1, 3), (0, 0), (2, 7), (1, 3), (0, 0)]
    part = oracle.decode_workload(w, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(part[b, h], full[b, h])
    assert np.isnan(part[2, 0]).all()
