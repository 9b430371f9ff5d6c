"""GPU parity of pa_decode_ex (sliding window, exported log-sum-exp) and
pa_attention_scores against the oracle (runs on an MI355X through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_58_amd as pa
from tests.gpu_util import compare, say, to_device
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24  # fp32 unit roundoff
U16 = 2.0 ** -8   # bf16 unit roundoff (8 significant bits)


def lse_bound(w, window):
    """Per-row a-priori bound on |lse_gpu - lse| from the kernels' arithmetic:
    each score is an fp32 sum of d products (bf16 x bf16 products are exact
    in fp32; fp32 products add one rounding), so |ds| <= (d + 1) u32 scale
    max_t sum_i |q_i k_ti|, which moves lse by at most as much; the weights
    summed into l are exp2 values rounded once to fp32 (and, on bf16 inputs,
    once more to bf16, relative error <= u16) and added in fp32 over the n
    attended tokens, so l is off by a factor within (1 +- (n + 2) u32
    [+ u16]), log of which bounds the rest; plus the final rounding of lse."""
    import numpy as np
    from tests.gpu_util import widen

    s = w.spec
    q, kc = widen(w.q), widen(w.k_cache)
    G = s.num_q_heads // s.num_kv_heads
    out = np.zeros((s.num_seqs, s.num_q_heads))
    for b in range(s.num_seqs):
        L = int(w.context_lens[b])
        t0 = max(0, L - window) if window else 0
        t = np.arange(t0, L)
        if t.size == 0:
            continue
        k = kc[w.block_tables[b, t // 16], t % 16]  # [n, Hkv, d]
        for h in range(s.num_q_heads):
            mag = np.abs(k[:, h // G, :]) @ np.abs(q[b, h])
            ds = (s.head_dim_k + 1) * U32 * abs(w.scale) * mag.max()
            rel = (t.size + 2) * U32 + (U16 if s.dtype == "bf16" else 0.0)
            out[b, h] = ds + rel * 1.01 + 4 * U32 * (1.0 + abs(w.scale) * mag.max())
    return out


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(autouse=True, params=["valu", "mfma"])
def grouped_path(request, monkeypatch):
    monkeypatch.setenv("PA_GQA_MFMA", "1" if request.param == "mfma" else "0")
    return request.param


CASES = [
    # dtype, head dim, q heads, kv heads, window, contexts
    ("bf16", 128, 64, 8, 0, [1, 17, 300, 1025]),
    ("bf16", 128, 64, 8, 256, [1, 17, 300, 1025, 4000]),
    ("bf16", 128, 32, 32, 33, [5, 33, 34, 700]),
    ("bf16", 128, 16, 2, 1, [1, 2, 100]),
    ("f32", 64, 8, 2, 100, [50, 101, 513]),
    ("bf16", 128, 8, 4, 4096, [0, 10, 5000]),
]


@pytest.mark.parametrize("dtype,D,hq,hkv,window,ctx", CASES)
def test_decode_ex_window_and_lse(dev, dtype, D, hq, hkv, window, ctx):
    say(f"case: decode_ex {dtype} d={D} hq={hq} hkv={hkv} window={window} ctx={ctx}")
    w = make_workload(custom_spec(len(ctx), hq, hkv, D, 16, dtype, ctx=ctx))
    d = to_device(w, dev)
    out = torch.empty_like(d.q)
    lse = torch.empty((len(ctx), hq), dtype=torch.float32, device=dev)
    pa.decode_ex(out, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale,
                 d.workspace, window=window, lse=lse)
    ref_o, ref_lse = oracle.decode_window(w.q, w.k_cache, w.v_cache, w.block_tables,
                                          w.context_lens, w.scale, window=window)
    compare(out, ref_o, dtype)
    got = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got), fin)
    bound = lse_bound(w, window)
    err = np.abs(got[fin] - ref_lse[fin]).max() if fin.any() else 0.0
    say(f"  lse max |delta| {err:.2e} (bound {bound[fin].max() if fin.any() else 0:.2e})")
    assert np.all(np.abs(got[fin] - ref_lse[fin]) <= bound[fin])


# Scores: every group size of the streaming kernel (1, 2, 4, 8, 16; runs of
# 16 blocks, so contexts past 256 tokens span several waves), fp32 rows of
# 128 (two blocks in flight), and the per-block kernel for 16 fp32 heads of
# 128 and for a group of 3; "tight" sizes the scores row to the longest
# context + 5 tokens instead of the table's capacity.
SCORE_CASES = [
    # dtype, head dim, q heads, kv heads, window, contexts, width
    CASES[1] + ("table",),
    CASES[3] + ("table",),
    CASES[4] + ("table",),
    ("bf16", 128, 32, 32, 0, [5, 33, 700, 2100], "tight"),
    ("bf16", 128, 8, 4, 4096, [0, 10, 5000], "table"),
    ("bf16", 128, 32, 2, 0, [1, 16, 17, 1100], "tight"),
    ("bf16", 64, 64, 4, 300, [7, 299, 301, 1500], "table"),
    ("f32", 128, 16, 2, 0, [3, 600, 1030], "tight"),
    ("f32", 128, 16, 1, 50, [40, 500], "table"),
    ("bf16", 128, 6, 2, 0, [9, 400, 777], "tight"),
]


@pytest.mark.parametrize("dtype,D,hq,hkv,window,ctx,width", SCORE_CASES)
def test_attention_scores(dev, dtype, D, hq, hkv, window, ctx, width):
    say(f"case: attention scores {dtype} d={D} hq={hq} hkv={hkv} window={window} ctx={ctx} {width}")
    w = make_workload(custom_spec(len(ctx), hq, hkv, D, 16, dtype, ctx=ctx))
    d = to_device(w, dev)
    _, ref_lse = oracle.decode_window(w.q, w.k_cache, w.v_cache, w.block_tables,
                                      w.context_lens, w.scale, window=window)
    maxc = int(w.block_tables.shape[1] * 16)
    if width == "tight":
        maxc = min(maxc, int(max(ctx)) + 5)
    scores = torch.full((len(ctx), hkv, maxc), 7.0, dtype=torch.float32, device=dev)
    lse_d = torch.from_numpy(ref_lse.astype(np.float32)).to(dev)
    pa.attention_scores(scores, d.q, d.k_cache, d.block_tables, d.context_lens, lse_d, w.scale,
                        window=window)
    ref = oracle.attention_scores(w.q, w.k_cache, w.block_tables, w.context_lens,
                                  ref_lse.astype(np.float32).astype(np.float64), w.scale,
                                  window=window, max_context=maxc)
    got = scores.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    say(f"  scores max |delta| {err:.2e}")
    assert np.allclose(got, ref, rtol=1e-4, atol=1e-5)
    # end to end: the GPU's own lse, each KV head's scores sum to G (the
    # decode runs groups of 1, 2, 4 and 8)
    if hq // hkv not in (1, 2, 4, 8):
        return
    lse = torch.empty((len(ctx), hq), dtype=torch.float32, device=dev)
    out = torch.empty_like(d.q)
    pa.decode_ex(out, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale,
                 d.workspace, window=window, lse=lse)
    pa.attention_scores(scores, d.q, d.k_cache, d.block_tables, d.context_lens, lse, w.scale,
                        window=window)
    sums = scores.sum(dim=2).cpu().numpy()
    G = hq // hkv
    live = np.asarray(ctx) > 0  # an empty context scores nothing
    assert np.allclose(sums[live], G, rtol=2e-2)
    assert np.all(sums[~live] == 0)
