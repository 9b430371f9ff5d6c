"""GPU parity of pa_cache_append and the grouped-query pa_decode path against
the CPU oracle (runs on an MI355X through the C ABI)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import compare, host_array, say, to_device, widen
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(autouse=True, params=["valu", "mfma"])
def grouped_path(request, monkeypatch):
    """Every test runs on both grouped kernels: VALU dot products, and the
    matrix-core kernel (taken for bf16 with head dim 128; other shapes stay
    on the VALU kernel either way)."""
    monkeypatch.setenv("PA_GQA_MFMA", "1" if request.param == "mfma" else "0")
    return request.param


def _append_bitwise(d, slots=None):
    w = d.w
    sm = w.slot_mapping if slots is None else slots
    hk = w.k_cache.copy()
    hv = None if w.v_cache is None else w.v_cache.copy()
    oracle.append(hk, hv, w.k_new, w.v_new, sm)
    d.append(None if slots is None else torch.from_numpy(sm).to(d.q.device))
    torch.cuda.synchronize()
    gk = host_array(d.k_cache)
    assert np.array_equal(gk.view(np.uint8), hk.view(np.uint8)), "K pool differs after append"
    if hv is not None:
        gv = host_array(d.v_cache)
        assert np.array_equal(gv.view(np.uint8), hv.view(np.uint8)), "V pool differs after append"
    return hk, hv


def test_config1_append_and_decode(dev):
    say("case: c1 tiny fp32, decode(ctx), append, decode(ctx+1)")
    w = make_workload("c1")
    d = to_device(w, dev)
    stats = compare(d.decode(), oracle.decode_workload(w), "f32")
    say(f"  decode(ctx): {stats}")
    hk, hv = _append_bitwise(d)
    L1 = w.context_lens + 1
    out = d.decode(context_lens=torch.from_numpy(L1).to(dev))
    ref = oracle.decode(w.q, hk, hv, w.block_tables, L1, w.scale)
    say(f"  decode(ctx+1): {compare(out, ref, 'f32')}")


CASES = [
    # dtype, head_dim, q heads, kv heads, context lengths
    ("f32", 64, 4, 2, [17, 64, 100, 255]),
    ("f32", 64, 8, 1, [1, 16, 513, 1029]),
    ("f32", 128, 4, 4, [0, 33, 700]),
    ("bf16", 128, 16, 2, [1, 15, 16, 17, 511, 512, 513, 1300]),
    ("bf16", 128, 4, 4, [2, 31, 1025, 2049]),
    ("bf16", 128, 8, 4, [0, 100, 600]),
    ("bf16", 64, 16, 4, [3, 17, 520, 1100]),
    ("bf16", 64, 2, 2, [1, 48, 1500]),
]


@pytest.mark.parametrize("dtype,D,hq,hkv,ctx", CASES)
def test_decode_parity_small(dev, dtype, D, hq, hkv, ctx):
    say(f"case: {dtype} D={D} Hq={hq} Hkv={hkv} ctx={ctx}")
    w = make_workload(custom_spec(len(ctx), hq, hkv, D, 16, dtype, ctx=ctx), seed=7 + D + hq)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), dtype)}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_score_range_exercises_rescale(dev, dtype):
    """scale = 1 on unit-variance data: scores spread over tens of units, so the
    running max is raised many times inside a partition."""
    say(f"case: rescale-heavy {dtype}")
    spec = custom_spec(3, 16, 2, 128, 16, dtype, ctx=[700, 2000, 64], scale=1.0)
    w = make_workload(spec, seed=3)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), dtype)}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_context_one_returns_v_bitwise(dev, dtype):
    say(f"case: ctx=1 {dtype}")
    w = make_workload(custom_spec(4, 16, 2, 128, 16, dtype, ctx=[1, 1, 1, 1]), seed=5)
    d = to_device(w, dev)
    got = host_array(d.decode())
    for b in range(4):
        v0 = w.v_cache[w.block_tables[b, 0], 0]  # [Hkv, D]
        want = np.repeat(v0, 8, axis=0)
        assert np.array_equal(got[b].view(np.uint8), want.view(np.uint8))


def test_deterministic_and_permutation_invariant(dev):
    say("case: determinism + block permutation")
    w = make_workload(custom_spec(3, 64, 8, 128, 16, "bf16", ctx=[900, 3000, 17]), seed=11)
    d = to_device(w, dev)
    a = host_array(d.decode())
    b = host_array(d.decode())
    assert np.array_equal(a, b)
    rng = np.random.default_rng(1)
    pi = rng.permutation(w.num_blocks).astype(np.int32)
    kp = np.empty_like(w.k_cache)
    vp = np.empty_like(w.v_cache)
    kp[pi] = w.k_cache
    vp[pi] = w.v_cache
    bt = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = make_workload(custom_spec(3, 64, 8, 128, 16, "bf16", ctx=[900, 3000, 17]), seed=11)
    w2.k_cache, w2.v_cache, w2.block_tables = kp, vp, bt
    c = host_array(to_device(w2, dev).decode())
    assert np.array_equal(a, c)


def test_nan_poison_equals_zero_fill(dev):
    say("case: NaN poison vs zero fill")
    w = make_workload(custom_spec(3, 16, 2, 128, 16, "bf16", ctx=[5, 250, 1000]), seed=2)
    a = host_array(to_device(w, dev).decode())
    z = np.where(np.isnan(widen(w.k_cache)), 0, 1).astype(bool)
    w.k_cache = np.where(z, w.k_cache, np.uint16(0))
    w.v_cache = np.where(np.isnan(widen(w.v_cache)), np.uint16(0), w.v_cache)
    assert not np.isnan(widen(w.k_cache)).any()
    b = host_array(to_device(w, dev).decode())
    assert np.array_equal(a, b)
    assert np.isfinite(widen(a)).all()


def test_gqa_equals_mha_on_expanded_cache(dev):
    say("case: GQA vs MHA with repeated KV heads")
    w = make_workload(custom_spec(2, 16, 2, 128, 16, "bf16", ctx=[400, 1500]), seed=9)
    ref = oracle.decode_workload(w)
    gqa_t = to_device(w, dev).decode()
    compare(gqa_t, ref, "bf16")
    gqa = widen(host_array(gqa_t))
    w.k_cache = np.ascontiguousarray(np.repeat(w.k_cache, 8, axis=2))
    w.v_cache = np.ascontiguousarray(np.repeat(w.v_cache, 8, axis=2))
    mha = widen(host_array(to_device(w, dev).decode()))
    diff = float(np.abs(gqa - mha).max())
    say(f"  max |gqa - mha| {diff:.2e}")
    assert diff <= 1.5e-2


@pytest.mark.parametrize("waves", ["1", "7", "300", "4096"])
@pytest.mark.parametrize("ring", ["2", "4"])
def test_stream_split_does_not_change_result(dev, waves, ring, monkeypatch):
    """The stream-K split (work-groups sharing the block order) and the LDS
    ring depth change only rounding: 1 work-group walks every segment, 7 and
    300 cut segments at uneven places, 4096 leaves most work-groups idle."""
    say(f"case: {waves} stream work-groups, ring {ring}")
    monkeypatch.setenv("PA_STREAM_WAVES", waves)
    monkeypatch.setenv("PA_RING_DEPTH", ring)
    w = make_workload(custom_spec(5, 16, 2, 128, 16, "bf16", ctx=[1, 333, 0, 4148, 70]), seed=4)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


@pytest.mark.parametrize("team", ["1", "2", "4"])
@pytest.mark.parametrize("waves", ["3", "5", "300"])
def test_head_teams_do_not_change_result(dev, team, waves, monkeypatch):
    """Teams of 1, 2 or 4 waves (one KV head each) sharing a stream share, with
    share counts that are not multiples of a team (3 and 5 waves leave one
    team), over empty, one-token, block-edge and long contexts."""
    say(f"case: teams of {team}, {waves} stream waves")
    monkeypatch.setenv("PA_TEAM_HEADS", team)
    monkeypatch.setenv("PA_STREAM_WAVES", waves)
    w = make_workload(custom_spec(6, 64, 8, 128, 16, "bf16", ctx=[1, 700, 0, 2049, 16, 95]),
                      seed=21)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


@pytest.mark.parametrize("ctx0", [2048, 2304, 4000])
def test_reduce_one_wave_rows_many_slots(dev, ctx0, monkeypatch):
    """2048 (sequence, query head) rows, so that the reduce runs one wave per
    row, and a first context whose segment the 16-block minimum shares cut
    into 8, 9 or 16 partial slots (the reduce loads a wave's slots eight at a
    time: one full batch, one slot more, two batches); the other contexts are
    short, ragged and partly empty."""
    say(f"case: one-wave reduce rows, first context {ctx0}")
    monkeypatch.setenv("PA_STREAM_WAVES", "600")
    ctx = [ctx0] + [(7 * i) % 40 for i in range(63)]
    w = make_workload(custom_spec(64, 32, 4, 128, 16, "bf16", ctx=ctx), seed=23)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


def test_many_sequences(dev, grouped_path):
    """300 short ragged sequences, some empty: more than the 256 whose block
    counts the stream shares keep in registers."""
    say(f"case: 300 sequences, {grouped_path} kernel")
    ctx = [(53 * i) % 311 for i in range(300)]
    w = make_workload(custom_spec(300, 64, 8, 128, 16, "bf16", ctx=ctx), seed=41)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


@pytest.mark.parametrize("dtype,D,hq,hkv", [("bf16", 128, 64, 8), ("f32", 64, 4, 2),
                                            ("bf16", 64, 16, 4)])
def test_long_segments_refill_block_ids(dev, dtype, D, hq, hkv, monkeypatch):
    """Few work-groups over long contexts: each walks hundreds of blocks of one
    segment, so the block-id buffers refill many times (64 ids per chunk)."""
    say(f"case: long segments {dtype} D={D}")
    monkeypatch.setenv("PA_STREAM_WAVES", "3")
    w = make_workload(custom_spec(2, hq, hkv, D, 16, dtype, ctx=[6000, 3001]), seed=12)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), dtype)}")


def test_append_skip_and_latent(dev):
    say("case: append with -1 slots; latent-mode append")
    w = make_workload(custom_spec(4, 8, 2, 64, 16, "bf16", ctx=[3, 16, 40, 0]), seed=6)
    d = to_device(w, dev)
    sm = w.slot_mapping.copy()
    sm[1] = -1
    _append_bitwise(d, sm)
    spec = custom_spec(3, 16, 1, 576, 64, "bf16", ctx=[63, 64, 300], head_dim_v=512, mla=True)
    wl = make_workload(spec, seed=8)
    _append_bitwise(to_device(wl, dev))


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_full_config_parity(dev, name):
    say(f"case: full config {name}: generate")
    w = make_workload(name)
    d = to_device(w, dev)
    say(f"  {name}: decode(ctx) vs oracle on every row")
    stats = compare(d.decode(), oracle.decode_workload(w), "bf16")
    say(f"  {name}: {stats}")
    hk, hv = _append_bitwise(d)
    say(f"  {name}: append bit-exact; decode(ctx+1) vs oracle on every row")
    L1 = w.context_lens + 1
    out = d.decode(context_lens=torch.from_numpy(L1).to(dev))
    ref = oracle.decode(w.q, hk, hv, w.block_tables, L1, w.scale)
    say(f"  {name}: {compare(out, ref, 'bf16')}")
    del d
    torch.cuda.empty_cache()
