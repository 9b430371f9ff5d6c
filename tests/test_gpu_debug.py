"""The PA_DEBUG build on the GPU, on valid inputs only: every call's device
pass finds no violation (a violation would raise PA_ERR_INDEX) and every
output is bitwise that of the release build.  Out-of-range ids are tested
on the CPU only (tests/test_debug_checks.py)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_58_amd as pa
from tests.gpu_util import device_tensor, host_array, say, to_device
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _both(monkeypatch, fn):
    """fn() under the release build, then under the debug build."""
    monkeypatch.setenv("PA_DEBUG", "0")
    assert not pa.is_debug_build()
    a = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv("PA_DEBUG", "1")
    assert pa.is_debug_build()
    b = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv("PA_DEBUG", "0")
    return a, b


def _same(a, b):
    assert np.array_equal(host_array(a).view(np.uint8), host_array(b).view(np.uint8))


@pytest.mark.parametrize("dtype,D,hq,hkv,ctx", [
    ("bf16", 128, 64, 8, [1, 17, 300, 1025, 0]),
    ("f32", 64, 4, 2, [17, 64, 100, 255]),
    ("bf16", 128, 32, 32, [700, 5]),
])
def test_debug_append_and_decode_match_release(dev, monkeypatch, dtype, D, hq, hkv, ctx):
    say(f"case: debug build, {dtype} D={D} hq={hq} hkv={hkv} ctx={ctx}")
    w = make_workload(custom_spec(len(ctx), hq, hkv, D, 16, dtype, ctx=ctx), seed=31)
    L1 = torch.from_numpy(w.context_lens + 1).to(dev)

    def run():
        d = to_device(w, dev)
        d.append()
        return d.decode(context_lens=L1), d.k_cache, d.v_cache

    (o1, k1, v1), (o2, k2, v2) = _both(monkeypatch, run)
    _same(o1, o2)
    _same(k1, k2)
    _same(v1, v2)


def test_debug_latent_matches_release(dev, monkeypatch):
    say("case: debug build, latent")
    w = make_workload(custom_spec(3, 128, 1, 576, 64, "bf16", ctx=[1, 700, 65], head_dim_v=512,
                                  mla=True, scale=1 / 24), seed=32)

    def run():
        d = to_device(w, dev)
        d.append()
        return d.decode(context_lens=torch.from_numpy(w.context_lens + 1).to(dev)), d.k_cache

    (o1, k1), (o2, k2) = _both(monkeypatch, run)
    _same(o1, o2)
    _same(k1, k2)


def test_debug_window_multi_mxfp8_scores_copy(dev, monkeypatch):
    say("case: debug build, window + lse, scores, several queries, MXFP8, block copy")
    ctx = [33, 400, 1500]
    w = make_workload(custom_spec(3, 16, 2, 128, 16, "bf16", ctx=ctx), seed=33)
    B, hq, hkv = 3, 16, 2

    def run():
        d = to_device(w, dev)
        out = torch.empty_like(d.q)
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
        pa.decode_ex(out, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale,
                     d.workspace, window=100, lse=lse)
        maxc = int(w.block_tables.shape[1] * 16)
        scores = torch.zeros((B, hkv, maxc), dtype=torch.float32, device=dev)
        pa.attention_scores(scores, d.q, d.k_cache, d.block_tables, d.context_lens, lse,
                            w.scale, window=100)
        q4 = d.q.reshape(B, 1, hq, 128).repeat(1, 4, 1, 1).contiguous()
        out4 = torch.empty_like(q4)
        ws4 = pa.alloc_multi_workspace(q4, hkv, 16, d.block_tables)
        pa.decode_multi(out4, q4, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                        w.scale, ws4)
        pools = pa.alloc_mxfp8_cache(w.num_blocks, 16, hkv, 128, dev, fill=0)
        sl = torch.arange(0, 64, dtype=torch.int32, device=dev)
        g = torch.Generator().manual_seed(5)
        rows = torch.randn((64, hkv, 128), generator=g).to(torch.bfloat16).to(dev)
        pa.cache_append_mxfp8(*pools, rows, rows, sl)
        ctx_mx = torch.tensor([64, 5, 0], dtype=torch.int32, device=dev)
        bt_mx = torch.zeros_like(d.block_tables)
        bt_mx[0, :4] = torch.arange(4, dtype=torch.int32)
        out_mx = torch.empty_like(d.q)
        pa.decode_mxfp8(out_mx, d.q, *pools, bt_mx, ctx_mx, w.scale,
                        pa.alloc_mxfp8_workspace(d.q, pools[0], bt_mx))
        src = torch.tensor([0, 1], dtype=torch.int32, device=dev)
        dst = torch.tensor([w.num_blocks - 1, w.num_blocks - 2], dtype=torch.int32, device=dev)
        pa.copy_blocks(d.k_cache, src, dst)
        return out, lse, scores, out4, pools[0], pools[2], out_mx, d.k_cache

    a, b = _both(monkeypatch, run)
    for x, y in zip(a, b):
        _same(x, y)
