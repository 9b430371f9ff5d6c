"""GPU parity of the latent (MLA-style) pa_decode path against the CPU oracle:
one 576-wide cached latent per token is the key and its first 512 values the
value, shared by every query head."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import compare, host_array, say, to_device, widen
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(576)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _spec(hq, ctx, scale=SCALE):
    return custom_spec(len(ctx), hq, 1, 576, 64, "bf16", ctx=ctx, head_dim_v=512, mla=True,
                       scale=scale)


@pytest.mark.parametrize("hq,ctx", [
    (128, [1, 63, 64, 65, 700]),
    (16, [0, 130, 1000]),
    (32, [200, 5]),
    (48, [64, 129, 300]),
    (80, [1, 500]),
])
def test_latent_parity_small(dev, hq, ctx):
    say(f"case: latent Hq={hq} ctx={ctx}")
    w = make_workload(_spec(hq, ctx), seed=20 + hq)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


def test_latent_rescale_heavy(dev):
    """Scale 0.5 on 576 unit-variance dims: scores spread over tens of units,
    a few tokens carry each head, and |O| reaches the size of single V
    values.  There the bf16 output's own rounding is the largest error: the
    exact result rounded to bf16 is already that far from it (the floor
    printed), and the GPU must stay within 2e-3 of that floor."""
    say("case: latent, scale 0.5 (wide score range)")
    w = make_workload(_spec(64, [900, 333], scale=0.5), seed=3)
    d = to_device(w, dev)
    ref = oracle.decode_workload(w)
    got = d.decode()
    stats = compare(got, ref, 'bf16')
    exact_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    floor = float(np.abs(exact_bf16 - ref).max())
    say(f"  {stats}; bf16 rounding of the exact output alone: {floor:.4f}")
    assert stats["max_abs"] <= floor + 2e-3


@pytest.mark.parametrize("scale", [0.0, -SCALE])
def test_latent_zero_and_negative_scale(dev, scale):
    """The scale is applied inside the exponentials with the max taken over
    the raw scores: a negative scale negates q instead (here the mirror of
    the usual 1/sqrt(576)), and zero gives the plain mean of the values
    (uniform weights)."""
    say(f"case: latent, scale {scale}")
    w = make_workload(_spec(128, [1, 100, 333, 64], scale=scale), seed=13)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


def test_latent_context_one_is_v_bitwise(dev):
    say("case: latent ctx=1")
    w = make_workload(_spec(128, [1, 1, 1]), seed=4)
    got = host_array(to_device(w, dev).decode())
    for b in range(3):
        row = w.k_cache[w.block_tables[b, 0], 0, 0, :512]
        want = np.broadcast_to(row, (128, 512))
        assert np.array_equal(got[b].view(np.uint16), want)


def test_latent_poison_and_determinism(dev):
    say("case: latent NaN poison vs zero fill, two runs")
    w = make_workload(_spec(32, [70, 1, 190]), seed=5)
    d = to_device(w, dev)
    a = host_array(d.decode())
    assert np.array_equal(a, host_array(d.decode()))
    w.k_cache = np.where(np.isnan(widen(w.k_cache)), np.uint16(0), w.k_cache)
    b = host_array(to_device(w, dev).decode())
    assert np.array_equal(a, b)


@pytest.mark.parametrize("waves", ["1", "3", "7", "24", "64", "512"])
def test_latent_stream_split(dev, waves, monkeypatch):
    """Grids of 1, 3 and 7 work-groups give each sequence one or two parts;
    24, 64 and 512 (multiples of 8) place a sequence's parts on one XCD
    (part j is work-group 8 (j mod grid/8) + j / (grid/8))."""
    say(f"case: latent, {waves} stream work-groups")
    monkeypatch.setenv("PA_STREAM_WAVES", waves)
    w = make_workload(_spec(128, [1, 1300, 0, 4100, 64]), seed=6)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


@pytest.mark.parametrize("waves", ["0", "512"])
def test_latent_many_sequences(dev, waves, monkeypatch):
    """300 short ragged sequences, some empty: more than the 256 whose unit
    counts the part search keeps in registers, and more than one work-group
    per CU.  With the default width the grid is one work-group per sequence
    (every sequence one part, written by the partition itself); with 512
    work-groups the longer sequences get two parts and their parts share an
    XCD."""
    say(f"case: latent, 300 sequences, PA_STREAM_WAVES={waves}")
    if waves != "0":
        monkeypatch.setenv("PA_STREAM_WAVES", waves)
    ctx = [(37 * i) % 229 for i in range(300)]
    w = make_workload(_spec(16, ctx), seed=31)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


@pytest.mark.parametrize("grid", ["8", "9", "17"])
def test_latent_reduce_part_batches(dev, grid, monkeypatch):
    """One sequence of 72 units cut into 8, 9 or 15 parts by 8, 9 or 17
    work-groups (the reduce loads a sequence's parts eight at a time: one
    full batch, one part more, two batches)."""
    say(f"case: latent, 72 units over {grid} work-groups")
    monkeypatch.setenv("PA_STREAM_WAVES", grid)
    w = make_workload(_spec(128, [2304]), seed=24)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")


def test_latent_append_then_decode(dev):
    say("case: latent append + decode(ctx + 1)")
    w = make_workload(_spec(128, [63, 64, 500]), seed=7)
    d = to_device(w, dev)
    hk = w.k_cache.copy()
    oracle.append(hk, None, w.k_new, None, w.slot_mapping)
    d.append()
    L1 = w.context_lens + 1
    out = d.decode(context_lens=torch.from_numpy(L1).to(dev))
    ref = oracle.decode(w.q, hk, None, w.block_tables, L1, w.scale, head_dim_v=512)
    say(f"  {compare(out, ref, 'bf16')}")


def test_config5_full(dev):
    """The latent workload at full size: decode(ctx) on every (sequence, head)
    row, the append of each sequence's new latent row bit-exact over the
    whole pool, then decode(ctx + 1) on every row."""
    say("case: full config c5 (MLA latent decode): decode(ctx) vs oracle on every row")
    w = make_workload("c5")
    d = to_device(w, dev)
    say(f"  c5: {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")
    hk = w.k_cache.copy()
    oracle.append(hk, None, w.k_new, None, w.slot_mapping)
    d.append()
    torch.cuda.synchronize()
    assert np.array_equal(host_array(d.k_cache).view(np.uint8), hk.view(np.uint8)), \
        "latent pool differs after append"
    say("  c5: append bit-exact; decode(ctx+1) vs oracle on every row")
    L1 = w.context_lens + 1
    out = d.decode(context_lens=torch.from_numpy(L1).to(dev))
    ref = oracle.decode(w.q, hk, None, w.block_tables, L1, w.scale, head_dim_v=512)
    say(f"  c5: {compare(out, ref, 'bf16')}")
    del d
    torch.cuda.empty_cache()
