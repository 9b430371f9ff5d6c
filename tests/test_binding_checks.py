"""The Python binding rejects mismatched tensors before any pointer reaches
the library: dtypes, shapes and devices are checked on the host (CPU
tensors here, so a call that got past the checks would fail on the device
test; none of these reach the C ABI)."""
from __future__ import annotations

import pytest
import torch

import paged_kv_cache_58_amd as pa

B, HQ, HKV, D, NB, BS, MB = 3, 8, 2, 128, 12, 16, 4


def _decode_args(**over):
    a = dict(out=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
             q=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
             k_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.bfloat16),
             v_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.bfloat16),
             block_tables=torch.zeros(B, MB, dtype=torch.int32),
             context_lens=torch.zeros(B, dtype=torch.int32),
             scale=0.1, workspace=torch.zeros(256, dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(k_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.float32)), "dtype"),
    (dict(v_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.float32)), "dtype"),
    (dict(out=torch.zeros(B, HQ, D, dtype=torch.float32)), "dtype"),
    (dict(k_cache=torch.zeros(NB, BS, HKV, 64, dtype=torch.bfloat16)), "head dim"),
    (dict(v_cache=torch.zeros(NB, 8, HKV, D, dtype=torch.bfloat16)), "does not match"),
    (dict(out=torch.zeros(B, HQ, 64, dtype=torch.bfloat16)), "head dim"),
    (dict(out=torch.zeros(B + 1, HQ, D, dtype=torch.bfloat16)), "does not match"),
    (dict(block_tables=torch.zeros(B, MB, dtype=torch.int64)), "int32"),
    (dict(context_lens=torch.zeros(B, dtype=torch.int64)), "int32"),
    (dict(block_tables=torch.zeros(B + 1, MB, dtype=torch.int32)), "rows"),
    (dict(context_lens=torch.zeros(B - 1, dtype=torch.int32)), "rows"),
    (dict(q=torch.zeros(B, HQ, D, 1, dtype=torch.bfloat16)), "dims"),
    ({}, "GPU tensor"),
])
def test_decode_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        pa.decode(**_decode_args(**over))


def test_decode_ex_and_multi_reject():
    a = _decode_args()
    with pytest.raises(ValueError, match="lse"):
        pa.decode_ex(**a, lse=torch.zeros(B, HQ, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="v_cache is required"):
        pa.decode_ex(**{**a, "v_cache": None})
    q4 = torch.zeros(B, 2, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="int32"):
        pa.decode_multi(**{**a, "q": q4, "out": q4.clone(),
                           "context_lens": torch.zeros(B, dtype=torch.int64)})
    with pytest.raises(ValueError, match="both"):
        pa.decode_multi(**{**a, "q": q4, "out": q4.clone()},
                        k_scale=torch.zeros(1, dtype=torch.uint8))


def _append_args(**over):
    n = 5
    a = dict(k_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.bfloat16),
             v_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.bfloat16),
             k=torch.zeros(n, HKV, D, dtype=torch.bfloat16),
             v=torch.zeros(n, HKV, D, dtype=torch.bfloat16),
             slot_mapping=torch.zeros(n, dtype=torch.int32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(slot_mapping=torch.zeros(5, dtype=torch.int64)), "int32"),
    (dict(k=torch.zeros(5, HKV, D, dtype=torch.float32)), "dtype"),
    (dict(v_cache=torch.zeros(NB, BS, HKV, D, dtype=torch.float32)), "dtype"),
    (dict(k=torch.zeros(4, HKV, D, dtype=torch.bfloat16)), "is not"),
    (dict(v=torch.zeros(5, HKV, 64, dtype=torch.bfloat16)), "is not"),
    (dict(v=None), "both"),
    (dict(v_cache=torch.zeros(NB, BS, 1, D, dtype=torch.bfloat16)), "does not match"),
    ({}, "GPU tensor"),
])
def test_append_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        pa.cache_append(**_append_args(**over))


def test_mxfp8_rejects():
    pools = [torch.zeros(NB, HKV, BS, D, dtype=torch.uint8),
             torch.zeros(NB, HKV, D, BS, dtype=torch.uint8),
             torch.zeros(NB, HKV, BS, D // 32, dtype=torch.uint8),
             torch.zeros(NB, HKV, BS, D // 32, dtype=torch.uint8)]
    k = torch.zeros(5, HKV, D, dtype=torch.bfloat16)
    sm = torch.zeros(5, dtype=torch.int32)
    bad = list(pools)
    bad[1] = torch.zeros(NB, HKV, BS, D, dtype=torch.uint8)  # V not transposed
    with pytest.raises(ValueError, match="v_cache"):
        pa.cache_append_mxfp8(*bad, k, k, sm)
    with pytest.raises(ValueError, match="dtype"):
        pa.cache_append_mxfp8(*pools, k, k.float(), sm)
    with pytest.raises(ValueError, match="int32"):
        pa.cache_append_mxfp8(*pools, k, k, sm.long())
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    bt, cl = torch.zeros(B, MB, dtype=torch.int32), torch.zeros(B, dtype=torch.int32)
    ws = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="bf16"):
        pa.decode_mxfp8(q.float(), q.float(), *pools, bt, cl, 0.1, ws)
    with pytest.raises(ValueError, match="rows"):
        pa.decode_mxfp8(q.clone(), q, *pools, bt[:1], cl, 0.1, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.decode_mxfp8(q.clone(), q, *pools, bt, cl, 0.1, ws)


def test_scores_and_copy_reject():
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    kc = torch.zeros(NB, BS, HKV, D, dtype=torch.bfloat16)
    bt, cl = torch.zeros(B, MB, dtype=torch.int32), torch.zeros(B, dtype=torch.int32)
    lse = torch.zeros(B, HQ)
    with pytest.raises(ValueError, match="scores"):
        pa.attention_scores(torch.zeros(B, HKV + 1, 64), q, kc, bt, cl, lse, 0.1)
    with pytest.raises(ValueError, match="lse"):
        pa.attention_scores(torch.zeros(B, HKV, 64), q, kc, bt, cl, lse[:, :2], 0.1)
    with pytest.raises(ValueError, match="int32"):
        pa.copy_blocks(kc, torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="rows"):
        pa.copy_blocks(kc, torch.zeros(2, dtype=torch.int32), torch.zeros(3, dtype=torch.int32))
