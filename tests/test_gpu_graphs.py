"""Decode steps replayed from HIP graphs (paged_kv_cache_58_amd.graphs): each
replay, with the program's own eager work and synchronisations between
replays, equals the eager append + decode of the same batch bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_58_amd as pa
from paged_kv_cache_58_amd.graphs import DecodeGraphs
from tests.gpu_util import device_tensor, say
from workloads import custom_spec, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_bucketed_graph_replays_equal_eager(dev, path, monkeypatch):
    monkeypatch.setenv("PA_GQA_MFMA", "1" if path == "mfma" else "0")
    say(f"case: decode graphs, buckets (1, 4, 8), {path} kernel")
    ctx = [5, 40, 300, 17, 1000, 64, 3, 700]
    w = make_workload(custom_spec(8, 16, 2, 128, 16, "bf16", ctx=ctx))
    kc, vc = device_tensor(w.k_cache, dev), device_tensor(w.v_cache, dev)
    q_all, kn, vn = device_tensor(w.q, dev), device_tensor(w.k_new, dev), device_tensor(w.v_new, dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    L1 = torch.from_numpy(w.context_lens + 1).to(dev)
    graphs = DecodeGraphs(kc, vc, 16, w.block_tables.shape[1], w.scale, buckets=(1, 4, 8))
    for rep in range(3):
        for idx in ([0, 1, 2], list(range(8)), [5], [7, 3, 4, 6]):
            sel = torch.tensor(idx, device=dev)
            ws = pa.alloc_workspace(q_all[sel], kc, bt[sel])
            eager = torch.empty((len(idx), 16, 128), dtype=torch.bfloat16, device=dev)
            pa.cache_append(kc, vc, kn[sel], vn[sel], sm[sel])
            pa.decode(eager, q_all[sel].contiguous(), kc, vc, bt[sel].contiguous(),
                      L1[sel].contiguous(), w.scale, ws)
            torch.cuda.synchronize()
            got = graphs.run(q_all[sel], kn[sel], vn[sel], sm[sel], bt[sel], L1[sel]).clone()
            torch.cuda.synchronize()
            # eager work of the program between replays
            _ = (torch.randn(1 << 16, device=dev) * 2).sum().item()
            assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), (rep, idx)
    assert graphs.bucket_for(3) == 4 and graphs.bucket_for(8) == 8
    with pytest.raises(ValueError):
        graphs.bucket_for(9)
