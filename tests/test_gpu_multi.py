"""GPU parity of pa_decode_multi (several new query tokens per sequence,
causal among themselves) against the oracle, over bf16 and MXFP8 caches
(runs on an MI355X through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_58_amd as pa
from tests.gpu_util import compare, device_tensor, host_array, say, to_device
from tests.test_gpu_mxfp8 import MxCase
from workloads import custom_spec, f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def multi_q(spec, Q, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((spec.num_seqs, Q, spec.num_q_heads, spec.head_dim_k)).astype(np.float32)
    return f32_to_bf16_bits(q)


def run_multi(dev, d, qh, k_scale=None, v_scale=None, kc=None, vc=None):
    q = device_tensor(qh, dev)
    B, Q, hq, D = q.shape
    kc = d.k_cache if kc is None else kc
    vc = d.v_cache if vc is None else vc
    hkv = kc.shape[2] if k_scale is None else kc.shape[1]
    ws = pa.alloc_multi_workspace(q, hkv, 16, d.block_tables if hasattr(d, "block_tables") else d.bt)
    out = torch.empty_like(q)
    bt = d.block_tables if hasattr(d, "block_tables") else d.bt
    cl = d.context_lens if hasattr(d, "context_lens") else d.cl
    pa.decode_multi(out, q, kc, vc, bt, cl, d.w.scale, ws, k_scale=k_scale, v_scale=v_scale)
    return out


CASES = [
    # q heads, kv heads, q_len, contexts (L counts the q_len new tokens)
    (64, 8, 2, [2, 17, 300, 1025]),
    (64, 8, 4, [4, 5, 16, 33, 700]),
    (64, 8, 8, [8, 40, 129, 2000]),
    (16, 2, 3, [1, 3, 50, 515]),           # 24 columns: a ragged second tile; L < q_len
    (32, 32, 5, [0, 5, 6, 100, 1300]),     # MHA, empty context
    (8, 8, 16, [16, 31, 500]),             # 16 queries of one head per column tile
]


@pytest.mark.parametrize("hq,hkv,Q,ctx", CASES)
def test_decode_multi_bf16_parity(dev, hq, hkv, Q, ctx):
    say(f"case: decode_multi bf16 hq={hq} hkv={hkv} q_len={Q} ctx={ctx}")
    w = make_workload(custom_spec(len(ctx), hq, hkv, 128, 16, "bf16", ctx=ctx))
    d = to_device(w, dev)
    qh = multi_q(w.spec, Q, 70 + Q)
    got = run_multi(dev, d, qh)
    ref = oracle.decode_multi(qh, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale)
    stats = compare(got.reshape(len(ctx), Q * hq, 128), ref.reshape(len(ctx), Q * hq, 128), "bf16")
    say(f"  {stats}")


@pytest.mark.parametrize("hq,hkv,Q,ctx", [(64, 8, 4, [4, 9, 300, 1500]), (16, 2, 3, [1, 3, 77]),
                                          (32, 32, 2, [2, 1000])])
def test_decode_multi_mxfp8_parity(dev, hq, hkv, Q, ctx):
    say(f"case: decode_multi mxfp8 hq={hq} hkv={hkv} q_len={Q} ctx={ctx}")
    c = MxCase(custom_spec(len(ctx), hq, hkv, 128, 16, "bf16", ctx=ctx), dev)
    qh = multi_q(c.w.spec, Q, 90 + Q)
    got = run_multi(dev, c, qh, k_scale=c.gpu[2], v_scale=c.gpu[3], kc=c.gpu[0], vc=c.gpu[1])
    ref = oracle.decode_multi(qh, c.host[0], c.host[1], c.w.block_tables, c.w.context_lens,
                              c.w.scale, mxfp8=(c.host[2], c.host[3]))
    stats = compare(got.reshape(len(ctx), Q * hq, 128), ref.reshape(len(ctx), Q * hq, 128), "bf16")
    say(f"  {stats}")


def test_decode_multi_one_query_equals_decode(dev, monkeypatch):
    """q_len = 1 through pa_decode_multi is the matrix-core single-query
    decode, bit for bit."""
    say("case: decode_multi with q_len 1 vs pa_decode on the matrix-core kernel")
    monkeypatch.setenv("PA_GQA_MFMA", "1")
    w = make_workload(custom_spec(5, 64, 8, 128, 16, "bf16", ctx=[1, 16, 17, 400, 3000]))
    d = to_device(w, dev)
    a = host_array(d.decode())
    qh = w.q[:, None]  # [B, 1, Hq, d]
    b = host_array(run_multi(dev, d, np.ascontiguousarray(qh)))
    assert np.array_equal(a, b[:, 0])


@pytest.mark.parametrize("waves", ["1", "13", "500"])
def test_decode_multi_stream_split(dev, waves, monkeypatch):
    say(f"case: decode_multi q_len 4 with PA_STREAM_WAVES={waves}")
    monkeypatch.setenv("PA_STREAM_WAVES", waves)
    w = make_workload(custom_spec(3, 64, 8, 128, 16, "bf16", ctx=[4, 700, 2500]))
    d = to_device(w, dev)
    qh = multi_q(w.spec, 4, 99)
    got = run_multi(dev, d, qh)
    ref = oracle.decode_multi(qh, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale)
    compare(got.reshape(3, 4 * 64, 128), ref.reshape(3, 4 * 64, 128), "bf16")


def test_decode_multi_fresh_chunk_first_query_is_v0(dev):
    """A sequence whose whole context is the chunk (L = q_len): query 0 sees
    token 0 alone, so its output is v_0 rounded to bf16 (exact weights 1)."""
    say("case: decode_multi fresh chunk, query 0 returns v0")
    Q = 6
    w = make_workload(custom_spec(2, 16, 2, 128, 16, "bf16", ctx=[Q, Q]))
    d = to_device(w, dev)
    qh = multi_q(w.spec, Q, 7)
    got = host_array(run_multi(dev, d, qh))
    bs = 16
    for b in range(2):
        p = w.block_tables[b, 0]
        v0 = w.v_cache[p, 0]  # [Hkv, d] bf16 bits
        for h in range(16):
            assert np.array_equal(got[b, 0, h], v0[h // 8])
