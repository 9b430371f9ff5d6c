"""P-7 on the GPU: the split-context partials the partition kernels leave in
the workspace, one (acc, m, l) per (partition, query head), against fp64
values computed here from the gathered K/V of exactly that partition's
tokens.

The pages' tiled softmax ("Étape 2: softmax en carreaux", "Cache KV,
attention et optimisation de l'inference") carries a running max m and a
running sum l of exp(s - m), with the output accumulated against the same m.
A partition's (acc, l) are therefore defined up to the reference m the
kernel chose (it raises m lazily, only when a score passes it by more than
2^8 in weight), so what is compared is what m does not change:
  * acc / l, the partition's own softmax output, against the fp64 one;
  * m + log2 l, the partition's log-sum-exp (base 2, scores in log2 units),
    against log2 sum_t 2^(x_t), within a bound derived from the arithmetic;
  * and m itself lies within [max_t x_t - 8, max_t x_t].
The shares (which tokens each partial covers) are recomputed from the
stream-K rule: the (sequence, head chunk, block) order cut into equal
shares of at least 16 blocks, one per team of waves.  PA_STREAM_WAVES fixes
the wave count so that partitions fall at uneven places.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from tests.gpu_util import host_array, say, to_device, widen
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
U32, U16 = 2.0 ** -24, 2.0 ** -8
STREAM_WAVES_MAX = 4096  # partial slots the workspace holds beyond one per (sequence, KV head)
WAVES_PER_GROUP = 4      # waves of a partition work-group (both grouped kernels, these shapes)
MIN_SHARE = 16


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def team_heads(hkv, group):
    cap = WAVES_PER_GROUP if group > 1 else 1
    t = 1
    while 2 * t <= cap and WAVES_PER_GROUP % (2 * t) == 0 and hkv % (2 * t) == 0:
        t *= 2
    return t


def partitions(ctx, hkv, group, waves, bs=16):
    """(b, g, first block, end block, partial row of query head 0 of g) of
    every partial the stream-K schedule writes."""
    th = team_heads(hkv, group)
    nc = hkv // th
    nshares = max(waves // th, 1)
    nb = [(c + bs - 1) // bs for c in ctx]
    pre = np.concatenate([[0], np.cumsum(nb)])
    total = nc * int(pre[-1])
    share = max((total + nshares - 1) // nshares, MIN_SHARE)
    out = []
    for b in range(len(ctx)):
        for ch in range(nc):
            lo = nc * int(pre[b]) + ch * nb[b]
            hi = lo + nb[b]
            for sid in range(lo // share, (hi - 1) // share + 1) if hi > lo else []:
                x0, x1 = max(lo, sid * share), min(hi, (sid + 1) * share)
                for hw in range(th):
                    row = ((sid + b * nc + ch) * th + hw) * group
                    out.append((b, ch * th + hw, x0 - lo, x1 - lo, row))
    return out


def read_partials(ws: np.ndarray, B, hkv, group, D):
    rows = (STREAM_WAVES_MAX + B * hkv) * group
    acc = ws[: rows * D * 4].view(np.float32).reshape(rows, D)
    ml_off = (rows * D * 4 + 255) // 256 * 256
    ml = ws[ml_off: ml_off + rows * 8].view(np.float32).reshape(rows, 2)
    return acc.astype(np.float64), ml.astype(np.float64)


CASES = [
    # dtype, head dim, q heads, kv heads, contexts, stream waves
    ("bf16", 128, 16, 2, [1, 333, 0, 4148, 70], 1),
    ("bf16", 128, 16, 2, [1, 333, 0, 4148, 70], 7),
    ("bf16", 128, 64, 8, [700, 2049, 16, 95], 13),
    ("bf16", 128, 64, 8, [700, 2049, 16, 95], 300),
    ("bf16", 128, 8, 8, [513, 40, 1200], 5),
    ("f32", 64, 8, 2, [1029, 17, 250], 6),
]


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("dtype,D,hq,hkv,ctx,waves", CASES)
def test_partition_partials_match_fp64(dev, monkeypatch, kernel, dtype, D, hq, hkv, ctx, waves):
    if kernel == "mfma" and (dtype != "bf16" or D != 128):
        pytest.skip("the matrix-core kernel runs bf16 with head dim 128")
    say(f"case: partials {kernel} {dtype} D={D} hq={hq} hkv={hkv} ctx={ctx} waves={waves}")
    monkeypatch.setenv("PA_GQA_MFMA", "1" if kernel == "mfma" else "0")
    monkeypatch.setenv("PA_STREAM_WAVES", str(waves))
    w = make_workload(custom_spec(len(ctx), hq, hkv, D, 16, dtype, ctx=ctx), seed=41 + hq)
    d = to_device(w, dev)
    d.workspace.fill_(0xFF)  # rows a kernel writes are then told apart from stale ones
    d.decode()
    torch.cuda.synchronize()
    G = hq // hkv
    acc, ml = read_partials(host_array(d.workspace), len(ctx), hkv, G, D)
    q = widen(w.q)
    kc, vc = widen(w.k_cache), widen(w.v_cache)
    parts = partitions(ctx, hkv, G, waves)
    assert parts, "no partials"
    gmax = gl2 = 0.0
    num = den = 0.0
    for b, g, blk0, blk1, row0 in parts:
        t = np.arange(blk0 * 16, min(blk1 * 16, ctx[b]))
        pb = w.block_tables[b, t // 16]
        k, v = kc[pb, t % 16, g], vc[pb, t % 16, g]
        for h in range(G):
            qh = q[b, g * G + h]
            x = (k @ qh) * w.scale * LOG2E
            xm = x.max()
            wt = np.exp2(x - xm)
            o_ref = (wt @ v) / wt.sum()
            lse2_ref = xm + math.log2(wt.sum())
            m, l = ml[row0 + h]
            assert np.isfinite(m) and l > 0, (b, g, h, m, l)
            assert xm - 8 - 1e-3 <= m <= xm + 1e-3, (b, g, h, m, xm)
            mag = (np.abs(k) @ np.abs(qh)).max()
            bound = ((D + 1) * U32 * abs(w.scale) * mag * LOG2E +
                     ((t.size + 2) * U32 + (U16 if dtype == "bf16" else 0.0)) / math.log(2) * 1.01)
            e2 = abs(m + math.log2(l) - lse2_ref)
            assert e2 <= bound, (b, g, h, e2, bound)
            gl2 = max(gl2, e2)
            o = acc[row0 + h] / l
            gmax = max(gmax, float(np.abs(o - o_ref).max()))
            num += float(((o - o_ref) ** 2).sum())
            den += float((o_ref ** 2).sum())
    rel = math.sqrt(num / den)
    say(f"  {len(parts)} partials: max |O_p - ref| {gmax:.2e}, rel-L2 {rel:.2e}, "
        f"max |lse2_p - ref| {gl2:.2e}")
    tol = {"f32": (2e-3, 1e-5), "bf16": (1.5e-2, 1e-2)}[dtype]
    assert gmax <= tol[0] and rel <= tol[1]
