"""Seeded random shapes within what the library runs, on the GPU against the
fp64 oracle: the grouped path on both kernels, with and without a sliding
window, and the latent path, over random batch sizes, head layouts, ragged
contexts (empty, one-token and one-block ones among them) and split widths.
Every case prints its shape before it runs."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_58_amd as pa
from tests.gpu_util import compare, say, to_device
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _contexts(rng, n: int, hi: int) -> list[int]:
    ctx = rng.integers(0, hi + 1, size=n)
    for p, v in zip(rng.choice(n, size=min(n, 3), replace=False), (0, 1, 16)):
        ctx[p] = v
    return [int(c) for c in ctx]


@pytest.mark.parametrize("case", range(12))
def test_grouped_random(dev, case, monkeypatch):
    rng = np.random.default_rng(1000 + case)
    dtype = ("bf16", "f32")[case % 2]
    D = (64, 128)[(case // 2) % 2]
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 41))
    ctx = _contexts(rng, B, 2500)
    window = int(rng.choice([0, 0, 1, 100, 700]))
    mfma = "1" if case % 3 == 0 else "0"
    waves = str(rng.choice(["", "7", "64", "300"]))
    say(f"case {case}: grouped {dtype} d={D} G={G} hkv={hkv} B={B} window={window} "
        f"PA_GQA_MFMA={mfma} PA_STREAM_WAVES={waves or 'default'} ctx[:6]={ctx[:6]}")
    monkeypatch.setenv("PA_GQA_MFMA", mfma)
    if waves:
        monkeypatch.setenv("PA_STREAM_WAVES", waves)
    w = make_workload(custom_spec(B, G * hkv, hkv, D, 16, dtype, ctx=ctx), seed=50 + case)
    d = to_device(w, dev)
    out = torch.empty_like(d.q)
    pa.decode_ex(out, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale,
                 d.workspace, window=window)
    ref, _ = oracle.decode_window(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, window=window)
    say(f"  {compare(out, ref, dtype)}")


@pytest.mark.parametrize("case", range(6))
def test_latent_random(dev, case, monkeypatch):
    rng = np.random.default_rng(2000 + case)
    hq = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    B = int(rng.integers(1, 17))
    ctx = _contexts(rng, B, 3000)
    waves = str(rng.choice(["", "5", "24", "200"]))
    say(f"case {case}: latent Hq={hq} B={B} PA_STREAM_WAVES={waves or 'default'} ctx[:6]={ctx[:6]}")
    if waves:
        monkeypatch.setenv("PA_STREAM_WAVES", waves)
    spec = custom_spec(B, hq, 1, 576, 64, "bf16", ctx=ctx, head_dim_v=512, mla=True,
                       scale=1.0 / math.sqrt(576))
    w = make_workload(spec, seed=70 + case)
    d = to_device(w, dev)
    say(f"  {compare(d.decode(), oracle.decode_workload(w), 'bf16')}")
