"""pa_decode_noalloc (the decode whose partials live in the library's per-GPU
scratch array instead of a caller's workspace) against pa_decode through the
C ABI: bitwise equal outputs on two calls in a row, the second with a
smaller input, on both grouped kernels; an oversized request is refused on
the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_58_amd as pa
from tests.gpu_util import compare, host_array, say, to_device
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _pair(w, dev):
    d = to_device(w, dev)
    ref = d.decode()
    got = torch.full_like(ref, float("nan"))
    pa.decode_noalloc(got, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_noalloc_equals_decode_twice(dev, monkeypatch, kernel):
    monkeypatch.setenv("PA_GQA_MFMA", "1" if kernel == "mfma" else "0")
    cases = [("c3", None), ("small", [1, 700, 0, 33])]
    for name, ctx in cases:
        say(f"case: decode_noalloc {kernel} {name}")
        w = make_workload(name) if ctx is None else make_workload(
            custom_spec(len(ctx), 16, 2, 128, 16, "bf16", ctx=ctx), seed=61)
        ref, got = _pair(w, dev)
        assert np.array_equal(host_array(ref).view(np.uint16), host_array(got).view(np.uint16))
        if ctx is not None:
            say(f"  {compare(got, oracle.decode_workload(w), 'bf16')}")


def test_noalloc_fp32_and_mha(dev):
    for spec, seed in ((custom_spec(3, 8, 2, 64, 16, "f32", ctx=[17, 300, 5]), 62),
                       (custom_spec(2, 8, 8, 128, 16, "bf16", ctx=[900, 1]), 63)):
        say(f"case: decode_noalloc {spec.dtype} hq={spec.num_q_heads} hkv={spec.num_kv_heads}")
        w = make_workload(spec, seed=seed)
        ref, got = _pair(w, dev)
        assert np.array_equal(host_array(ref).view(np.uint8), host_array(got).view(np.uint8))


def test_noalloc_refuses_oversized(dev):
    say("case: decode_noalloc beyond its scratch")
    w = make_workload(custom_spec(1, 128, 1, 576, 64, "bf16", ctx=[100], head_dim_v=512,
                                  mla=True, scale=1 / 24), seed=64)
    d = to_device(w, dev)
    out = torch.empty((1, 128, 512), dtype=torch.bfloat16, device=dev)
    with pytest.raises(pa.PAError) as e:
        pa.decode_noalloc(out, d.q, d.k_cache, None, d.block_tables, d.context_lens, w.scale)
    assert e.value.status == 5 and "scratch" in e.value.detail
