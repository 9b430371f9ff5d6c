"""The continuous-batching decode loop (paged_kv_cache_58_amd.engine.DecodeLoop)
on the GPU: sequences are admitted with prompts that share system-prompt
blocks, decoded step by step (pa_bm_append_token -> pa_copy_blocks for
copy-on-write -> pa_cache_append -> pa_decode), forked (parallel samples of one
prompt) and retired, while new ones reuse the cached prefixes of live ones.

The K/V of a token is a fixed function of (token id, position), so a shared
prefix has the same K/V in every sequence, as a model's would.  Every step
checks (1) the cache bit for bit: each live sequence's slots hold exactly its
tokens' K/V, and (2) the decode against the oracle on a freshly packed pool of
the same sequences (its own block placement).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_58_amd as pa
from tests.gpu_util import compare, device_tensor, host_array, say
from tests.helpers import pack_paged
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

HKV, G, D, BS = 2, 4, 128, 16
HQ = HKV * G
VOCAB, MAXPOS = 64, 512


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


class TokenKV:
    """K/V rows of a token at a position: seeded tables, bf16."""

    def __init__(self, seed=321):
        rng = np.random.default_rng(seed)
        self.kt = rng.standard_normal((VOCAB, HKV, D)).astype(np.float32)
        self.vt = rng.standard_normal((VOCAB, HKV, D)).astype(np.float32)
        self.kp = (0.5 * rng.standard_normal((MAXPOS, HKV, D))).astype(np.float32)
        self.vp = (0.5 * rng.standard_normal((MAXPOS, HKV, D))).astype(np.float32)

    def rows(self, tokens, positions):
        t, p = np.asarray(tokens), np.asarray(positions)
        return (f32_to_bf16_bits(self.kt[t] + self.kp[p]), f32_to_bf16_bits(self.vt[t] + self.vp[p]))


def _run_loop(dev, graph_buckets=None, steps=12):
    """Drive paged_kv_cache_58_amd.engine.DecodeLoop for `steps` steps with
    admissions (prompts sharing system-prompt blocks), forks and retirements;
    check the cache and the decode at every step.  Returns the outputs."""
    from paged_kv_cache_58_amd.engine import DecodeLoop

    rng = np.random.default_rng(9)
    tkv = TokenKV()
    nb, max_blocks = 160, MAXPOS // BS
    loop = DecodeLoop(nb, BS, HKV, HQ, D, max_blocks, D ** -0.5, torch.bfloat16, dev,
                      graph_buckets=graph_buckets)
    sys_prompts = [list(rng.integers(0, VOCAB, 32)), list(rng.integers(0, VOCAB, 40))]
    tokens = {}  # seq id -> token list (the ground truth of what is cached)
    next_id = 0
    shared_hits = 0
    outs = []

    def admit():
        nonlocal next_id, shared_hits
        prompt = sys_prompts[rng.integers(0, 2)] + list(rng.integers(0, VOCAB, rng.integers(1, 40)))
        k, v = tkv.rows(prompt, np.arange(len(prompt)))
        shared_hits += loop.add(next_id, prompt, device_tensor(k, dev), device_tensor(v, dev))
        tokens[next_id] = list(prompt)
        next_id += 1

    for _ in range(5):
        admit()
    for step in range(steps):
        live = sorted(tokens)
        if step % 4 == 1:  # parallel sample: fork a sequence
            p = live[rng.integers(0, len(live))]
            loop.fork(p, next_id)
            tokens[next_id] = list(tokens[p])
            next_id += 1
        if step % 5 == 3:  # retire one, admit one
            sid = live[rng.integers(0, len(live))]
            loop.free(sid)
            del tokens[sid]
            admit()
        live = sorted(tokens)
        assert live == loop.live
        toks = [int(rng.integers(0, VOCAB)) for _ in live]
        poss = [len(tokens[sid]) for sid in live]
        k, v = tkv.rows(toks, poss)
        q = f32_to_bf16_bits(rng.standard_normal((len(live), HQ, D)).astype(np.float32))
        out = loop.step(live, toks, device_tensor(q, dev), device_tensor(k, dev),
                        device_tensor(v, dev))
        for sid, t in zip(live, toks):
            tokens[sid].append(t)
        torch.cuda.synchronize()
        outs.append(host_array(out).copy())

        # (1) the cache holds exactly each live sequence's K/V
        bts = np.stack([loop.block_table(sid) for sid in live])
        lens = np.array([len(tokens[sid]) for sid in live], np.int32)
        assert [loop.num_tokens(s) for s in live] == lens.tolist()
        hk, hv = host_array(loop.k_cache), host_array(loop.v_cache)
        for i, sid in enumerate(live):
            pos = np.arange(lens[i])
            ek, ev = tkv.rows(tokens[sid], pos)
            blk, row = bts[i, pos // BS], pos % BS
            assert np.array_equal(hk[blk, row], ek) and np.array_equal(hv[blk, row], ev), \
                f"step {step}: cache of sequence {sid} differs"

        # (2) the decode against the oracle on a pool packed independently
        seqs_k, seqs_v = zip(*[tkv.rows(tokens[sid], np.arange(len(tokens[sid]))) for sid in live])
        pk, pbt = pack_paged(list(seqs_k), BS, rng=np.random.default_rng(step), dtype=np.uint16)
        pv, _ = pack_paged(list(seqs_v), BS, rng=np.random.default_rng(step), dtype=np.uint16)
        ref = oracle.decode(q, pk, pv, pbt, lens, D ** -0.5)
        compare(out, ref, "bf16")
    say(f"  {next_id} sequences, {shared_hits} prompt tokens found cached, "
        f"{loop.copied_blocks} copy-on-write blocks")
    assert shared_hits > 0 and loop.copied_blocks > 0
    return outs


def test_continuous_batching_with_prefix_sharing_and_copy_on_write(dev):
    say("case: DecodeLoop (block manager, copy-on-write, append, decode), 12 steps")
    _run_loop(dev)


def test_continuous_batching_from_graph_buckets(dev):
    """The same loop with each step's append + decode replayed from graph
    buckets: identical to the eager loop bit for bit."""
    say("case: DecodeLoop on graph buckets (4, 8) vs eager")
    eager = _run_loop(dev)
    graphed = _run_loop(dev, graph_buckets=(4, 8))
    for a, b in zip(eager, graphed):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_copy_blocks_mxfp8_pools(dev):
    """pa_copy_blocks on the four arrays of an MXFP8 cache (different block sizes)."""
    say("case: copy_blocks on MXFP8 pool arrays")
    pools = pa.alloc_mxfp8_cache(12, 16, 2, 128, dev)
    for t in pools:
        t.copy_(torch.randint(0, 256, t.shape, dtype=torch.uint8, device=dev))
    before = [t.cpu().numpy().copy() for t in pools]
    src = torch.tensor([3, 7, 0], dtype=torch.int32, device=dev)
    dst = torch.tensor([5, 1, 11], dtype=torch.int32, device=dev)
    for t in pools:
        pa.copy_blocks(t, src, dst)
    for t, b in zip(pools, before):
        exp = b.copy()
        exp[[5, 1, 11]] = b[[3, 7, 0]]
        assert np.array_equal(t.cpu().numpy(), exp)
