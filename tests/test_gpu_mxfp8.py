"""GPU parity of the MXFP8 KV cache: pa_cache_append_mxfp8 against the oracle's
quantizing append (bit for bit), and pa_decode_mxfp8 against the oracle's
decode over its own MXFP8 caches (runs on an MI355X through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_58_amd as pa
from tests.gpu_util import compare, device_tensor, host_array, say
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu

POISON_CODE, POISON_SCALE = 0x7F, 0xFF  # E4M3 NaN, E8M0 NaN


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def host_pools(nb, bs, hkv, d=128, code=POISON_CODE, scale=POISON_SCALE):
    return (np.full((nb, hkv, bs, d), code, np.uint8), np.full((nb, hkv, d, bs), code, np.uint8),
            np.full((nb, hkv, bs, d // 32), scale, np.uint8),
            np.full((nb, hkv, bs, d // 32), scale, np.uint8))


def device_pools(host, dev):
    return tuple(torch.from_numpy(a.copy()).to(dev) for a in host)


def valid_slots(w, seqs=None):
    """Slots of every cached token t < L_b of the listed sequences."""
    bs = w.spec.block_size
    seqs = range(w.spec.num_seqs) if seqs is None else seqs
    parts = []
    for b in seqs:
        t = np.arange(int(w.context_lens[b]))
        parts.append(w.block_tables[b, t // bs] * bs + t % bs)
    return np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)


def pool_rows(pool, slots, bs):
    return np.ascontiguousarray(pool[slots // bs, slots % bs])


class MxCase:
    """A seeded bf16 workload whose cached rows are appended into MXFP8 pools,
    on the GPU through the library and on the host through the oracle."""

    def __init__(self, spec, dev, seqs_for_oracle=None, fill=(POISON_CODE, POISON_SCALE)):
        w = make_workload(spec)
        self.w = w
        s = w.spec
        bs, hkv = s.block_size, s.num_kv_heads
        nb = w.k_cache.shape[0]
        slots = valid_slots(w)
        self.gpu = device_pools(host_pools(nb, bs, hkv, code=fill[0], scale=fill[1]), dev)
        if slots.size:
            pa.cache_append_mxfp8(*self.gpu, device_tensor(pool_rows(w.k_cache, slots, bs), dev),
                                  device_tensor(pool_rows(w.v_cache, slots, bs), dev),
                                  torch.from_numpy(slots).to(dev))
        self.host = host_pools(nb, bs, hkv, code=fill[0], scale=fill[1])
        oslots = slots if seqs_for_oracle is None else valid_slots(w, seqs_for_oracle)
        if oslots.size:
            oracle.append_mxfp8(*self.host, pool_rows(w.k_cache, oslots, bs),
                                pool_rows(w.v_cache, oslots, bs), oslots)
        self.q = device_tensor(w.q, dev)
        self.bt = torch.from_numpy(w.block_tables).to(dev)
        self.cl = torch.from_numpy(w.context_lens).to(dev)
        self.ws = pa.alloc_mxfp8_workspace(self.q, self.gpu[0], self.bt)

    def decode(self):
        s = self.w.spec
        out = torch.empty((s.num_seqs, s.num_q_heads, 128), dtype=torch.bfloat16,
                          device=self.q.device)
        pa.decode_mxfp8(out, self.q, *self.gpu, self.bt, self.cl, self.w.scale, self.ws)
        return out

    def oracle_decode(self, pairs=None):
        return oracle.decode_mxfp8(self.w.q, *self.host, self.w.block_tables, self.w.context_lens,
                                   self.w.scale, pairs=pairs)


def _special_rows(rng, n, hkv, d):
    x = rng.standard_normal((n, hkv, d)).astype(np.float32)
    x[0] = 0.0                                   # all-zero blocks: scale byte 0
    x[1, :, 5] *= 300.0                          # outlier channel
    x[2] *= 1e-30                                # tiny magnitudes
    x[3, :, :32] = 448.0 * 2.0 ** -3             # block max exactly at the top code
    x[3, :, 1] = (416.0 + 448.0) / 2 * 2.0 ** -3  # a tie between two codes
    x[4, :, 64:96] *= 1e4
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_mxfp8_bitexact(dev, dtype):
    say(f"case: mxfp8 append {dtype}, 300 tokens, 4 KV heads, 40 blocks of 16")
    rng = np.random.default_rng(31)
    n, hkv, nb, bs = 300, 4, 40, 16
    k = _special_rows(rng, n, hkv, 128)
    v = _special_rows(rng, n, hkv, 128)[::-1].copy()
    if dtype == "bf16":
        tk = torch.from_numpy(k).to(torch.bfloat16)
        tv = torch.from_numpy(v).to(torch.bfloat16)
        hk = tk.view(torch.int16).numpy().view(np.uint16)
        hv = tv.view(torch.int16).numpy().view(np.uint16)
    else:
        tk, tv, hk, hv = torch.from_numpy(k), torch.from_numpy(v), k, v
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[[7, 100, 299]] = -1
    host = host_pools(nb, bs, hkv)
    gpu = device_pools(host, dev)
    pa.cache_append_mxfp8(*gpu, tk.to(dev), tv.to(dev), torch.from_numpy(slots).to(dev))
    oracle.append_mxfp8(*host, hk, hv, slots)
    torch.cuda.synchronize()
    for name, g, h in zip(("k codes", "v codes", "k scales", "v scales"), gpu, host):
        got = g.cpu().numpy()
        assert np.array_equal(got, h), f"{name}: {np.count_nonzero(got != h)} bytes differ"


CASES = [
    # q heads, kv heads, context lengths
    (8, 8, [1, 15, 16, 17, 300]),
    (16, 8, [0, 33, 700]),
    (32, 8, [2, 31, 1025, 2049]),
    (64, 8, [1, 16, 513, 1300]),
    (4, 2, [40, 2000]),
]


@pytest.mark.parametrize("hq,hkv,ctx", CASES)
def test_decode_mxfp8_parity(dev, hq, hkv, ctx):
    say(f"case: mxfp8 decode hq={hq} hkv={hkv} ctx={ctx}")
    spec = custom_spec(len(ctx), hq, hkv, 128, 16, "bf16", ctx=ctx)
    c = MxCase(spec, dev)
    for g, h in zip(c.gpu, c.host):
        assert np.array_equal(g.cpu().numpy(), h), "GPU and oracle MXFP8 pools differ"
    stats = compare(c.decode(), c.oracle_decode(), "bf16")
    say(f"  {stats}")


def test_decode_mxfp8_context_one_returns_dequantized_v(dev):
    say("case: mxfp8 decode with one cached token per sequence")
    spec = custom_spec(6, 16, 2, 128, 16, "bf16", ctx=[1] * 6)
    c = MxCase(spec, dev)
    got = host_array(c.decode())
    ref = c.oracle_decode()  # exactly the dequantized first V row (one weight of 1)
    ref_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(got, ref_bf16.view(torch.int16).numpy().view(np.uint16))


def test_decode_mxfp8_poison_equals_zero_fill(dev):
    say("case: mxfp8 decode, NaN-poisoned vs zero-filled unused slots")
    spec = custom_spec(5, 16, 2, 128, 16, "bf16", ctx=[3, 17, 40, 100, 250])
    a = MxCase(spec, dev)
    b = MxCase(spec, dev, fill=(0, 0))
    ga, gb = host_array(a.decode()), host_array(b.decode())
    assert np.isfinite(ga.view(np.uint16).astype(np.float32)).all()
    assert np.array_equal(ga, gb)


@pytest.mark.parametrize("waves", ["1", "7", "300"])
@pytest.mark.parametrize("ring", ["2", "4"])
def test_decode_mxfp8_stream_split(dev, waves, ring, monkeypatch):
    say(f"case: mxfp8 decode with PA_STREAM_WAVES={waves} PA_RING_DEPTH={ring}")
    monkeypatch.setenv("PA_STREAM_WAVES", waves)
    monkeypatch.setenv("PA_RING_DEPTH", ring)
    spec = custom_spec(4, 64, 8, 128, 16, "bf16", ctx=[1, 200, 1500, 4100])
    c = MxCase(spec, dev)
    compare(c.decode(), c.oracle_decode(), "bf16")


def test_decode_mxfp8_llama70b_shape(dev):
    """The 70B-style GQA decode layer (100 sequences, 64 q / 8 KV heads, ctx
    U[1024, 8192]) in MXFP8; the oracle covers 6 of the sequences."""
    say("case: mxfp8 decode at the c3 shape (sampled sequences vs oracle)")
    w0 = make_workload("c3")
    seqs = [0, 17, 42, 63, 88, 99]
    c = MxCase(w0.spec, dev, seqs_for_oracle=seqs)
    bs, hkv = c.w.spec.block_size, c.w.spec.num_kv_heads
    got_pools = [g.cpu().numpy() for g in c.gpu]
    for b in seqs:  # the GPU append of these sequences' tiles matches the oracle's
        ids = c.w.block_tables[b, : -(-int(c.w.context_lens[b]) // bs)]
        for g, h in zip(got_pools, c.host):
            assert np.array_equal(g[ids], h[ids])
    pairs = [(b, h) for b in seqs for h in range(c.w.spec.num_q_heads)]
    ref = c.oracle_decode(pairs=pairs)
    stats = compare(c.decode(), ref, "bf16", rows=pairs)
    say(f"  {stats}")
