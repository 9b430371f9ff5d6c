#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

A step is one pass of the whole hot path over one batch: pa_cache_append of
each sequence's new token through the slot mapping, then pa_decode of every
sequence over its context including that token.  Inputs are seeded synthetic
data of the named workload, resident in HBM before timing starts.  With
--kv-format mxfp8 the caches hold the workload's K/V rows quantized to MXFP8
(quantized by the library before timing) and the step is
pa_cache_append_mxfp8 + pa_decode_mxfp8.  With --q-len K > 1 the decode is
pa_decode_multi: the last K cached tokens of every sequence (the appended one
among them) are its queries, causal among themselves, the shape of verifying
K - 1 drafted tokens plus the new one in one pass.  --q-heads H runs the
latent workload with H query heads (its share of a 128-head model split over
GPUs by heads); the context lengths stay those of the workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix peak
METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + decode tokens/s"
WORKLOAD_TEXT = {
    "c1": "tiny paged decode fp32: 4 seqs ctx {17,64,100,255}, 4 q / 2 kv heads, d 64, block 16",
    "c2": "7B-style MHA decode layer bf16: batch 32, 32 q = 32 kv heads, d 128, block 16, "
          "ctx U[512,4096]",
    "c3": "Llama-3-70B-style GQA decode layer bf16: batch 100, 64 q / 8 kv heads, d 128, "
          "block 16, ctx U[1024,8192], shuffled blocks",
    "c4": "long-context GQA decode bf16: batch 4 x ctx 131072, 64 q / 8 kv heads, d 128, block 16",
    "c5": "MLA-style latent decode bf16: batch 64, 128 heads over one 576-dim latent "
          "(V = first 512), block 64, ctx U[2048,8192]",
}
# The sources each decode path is built from (its kernels, the append before
# it, the shared device code and the host planning that sets its launch): a
# measurement of one path stays valid while these hash the same.
_SHARED_SOURCES = ["device_common.h", "plan.cpp", "plan.h"]
KERNEL_SOURCES = {
    "grouped": ["grouped_decode.hip", "append.hip"] + _SHARED_SOURCES,
    "mfma": ["gqa_mfma_decode.hip", "append.hip"] + _SHARED_SOURCES,
    "mxfp8": ["gqa_mfma_decode.hip", "mxfp8_append.hip"] + _SHARED_SOURCES,
    "latent": ["latent_decode.hip", "append.hip"] + _SHARED_SOURCES,
}


FLUSH_BYTES = 512 << 20
GROUPED = "grouped_partition_kernel + stream_reduce_kernel"
GROUPED_MFMA = "gqa_mfma_partition_kernel + stream_reduce_kernel"


def kernel_name(spec, mx: bool, q_len: int, window: int) -> str:
    """The kernels one decode call of this run launches (the partition kernel
    dominates; the reduce is 2-10% of the time)."""
    if spec.mla:
        return "latent_partition_kernel + latent_reduce_kernel"
    if mx:
        return "gqa_mfma_partition_kernel (MXFP8 operands) + stream_reduce_kernel"
    if q_len > 1:
        return GROUPED_MFMA
    if spec.dtype == "bf16" and spec.head_dim_k == 128 and os.environ.get("PA_GQA_MFMA", "0") not in ("", "0"):
        return GROUPED_MFMA
    return GROUPED


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def code_tokens(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: what
    the compiler sees, so that a comment edit keeps a measurement valid.
    (String literals in these sources hold no comment markers.)"""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def traffic_family(key: str) -> str:
    """The decode path a traffic_<key>.json describes: <config>, <config>_mfma
    (the matrix-core variant of a native bf16 config) or <config>_mxfp8."""
    if key.endswith("_mxfp8"):
        return "mxfp8"
    if key.endswith("_mfma"):
        return "mfma"
    import workloads

    return "latent" if workloads.CONFIGS[key].mla else "grouped"


def kernel_source_hash(family: str) -> str:
    """Hash of the code (comments and layout excluded) of one path's sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "paged_kv_cache_58_amd", "csrc", name), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(key: str, decode_bytes: int):
    """HBM traffic per decode from committed rocprofv3 --pmc summaries, or None
    when they are missing or were taken on different sources of that path."""
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(traffic_family(key)):
        return None
    return t.get("hbm_bytes_per_decode")


def valid_slots(w, seqs=None):
    """Slots of every cached token t < ctx_b of the listed sequences."""
    import numpy as np

    bs = w.spec.block_size
    seqs = range(w.spec.num_seqs) if seqs is None else seqs
    parts = []
    for b in seqs:
        t = np.arange(int(w.context_lens[b]))
        parts.append(w.block_tables[b, t // bs] * bs + t % bs)
    return np.concatenate(parts).astype(np.int32)


def sample_seqs(spec):
    import numpy as np

    return sorted(set(np.linspace(0, spec.num_seqs - 1, min(6, spec.num_seqs)).astype(int).tolist()))


def oracle_mx_pools(w, seqs, oracle):
    """The oracle's own MXFP8 pools holding the listed sequences' cached rows
    and their appended token."""
    import numpy as np

    spec = w.spec
    bs = spec.block_size
    nb = w.num_blocks
    pools = (np.full((nb, spec.num_kv_heads, bs, 128), 0x7F, np.uint8),
             np.full((nb, spec.num_kv_heads, 128, bs), 0x7F, np.uint8),
             np.full((nb, spec.num_kv_heads, bs, 4), 0x7F, np.uint8),
             np.full((nb, spec.num_kv_heads, bs, 4), 0x7F, np.uint8))
    sl = valid_slots(w, seqs)
    oracle.append_mxfp8(*pools, np.ascontiguousarray(w.k_cache[sl // bs, sl % bs]),
                        np.ascontiguousarray(w.v_cache[sl // bs, sl % bs]), sl)
    new = np.full(spec.num_seqs, -1, np.int32)
    new[seqs] = w.slot_mapping[seqs]
    oracle.append_mxfp8(*pools, w.k_new, w.v_new, new)
    return pools


def multi_oracle_check(w, L1, got, q_host, decode_bytes, args, oracle, mx):
    """Oracle check of a several-queries run on a sample of sequences (all
    queries and heads), also timed as the CPU leg."""
    import numpy as np

    spec = w.spec
    seqs = sample_seqs(spec)
    Q = q_host.shape[1]
    if mx:
        pools = oracle_mx_pools(w, seqs, oracle)
        caches, mxs = (pools[0], pools[1]), (pools[2], pools[3])
    else:
        hk, hv = w.k_cache.copy(), w.v_cache.copy()
        oracle.append(hk, hv, w.k_new, w.v_new, w.slot_mapping)
        caches, mxs = (hk, hv), None
    pairs = [(b, i) for b in seqs for i in range(Q)]
    t_c = time.perf_counter()
    ref = oracle.decode_multi(q_host, caches[0], caches[1], w.block_tables, L1, w.scale,
                              mxfp8=mxs, pairs=pairs)
    cpu_s = time.perf_counter() - t_c
    sel = np.array(pairs)
    d = np.abs(got[sel[:, 0], sel[:, 1]] - ref[sel[:, 0], sel[:, 1]])
    frac = float(L1[seqs].sum()) / float(L1.sum())
    cpu = None
    if not args.no_cpu_baseline:
        cpu = {"value": round(decode_bytes * frac / cpu_s / 1e9, 3), "unit": "GB/s",
               "cores": oracle.default_threads(), "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"oracle decode of {len(seqs)} of the {spec.num_seqs} sequences x {Q} "
                         f"queries x all heads ({frac:.1%} of the attended tokens), fp64, "
                         f"{cpu_s:.2f} s wall; GB/s over that sample's share of the bytes",
               "tokens_per_s": round(len(seqs) * Q / cpu_s, 3)}
        log(f"[bench] oracle (sample, q_len {Q}): {cpu_s:.2f}s")
    return d, cpu


def window_oracle_check(w, L1, got, window, decode_bytes, args, oracle):
    """Oracle check of a sliding-window run on a sample of sequences (all
    heads), also timed as the CPU leg."""
    import numpy as np

    spec = w.spec
    seqs = sample_seqs(spec)
    hk, hv = w.k_cache.copy(), w.v_cache.copy()
    oracle.append(hk, hv, w.k_new, w.v_new, w.slot_mapping)
    t_c = time.perf_counter()
    ref, _ = oracle.decode_window(w.q[seqs], hk, hv, w.block_tables[seqs], L1[seqs], w.scale,
                                  window=window)
    cpu_s = time.perf_counter() - t_c
    d = np.abs(got[seqs] - ref)
    att = np.minimum(L1, window)
    frac = float(att[seqs].sum()) / float(att.sum())
    cpu = None
    if not args.no_cpu_baseline:
        cpu = {"value": round(decode_bytes * frac / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1,
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"numpy oracle windowed decode of {len(seqs)} of the {spec.num_seqs} "
                         f"sequences ({frac:.1%} of the attended tokens), fp64, {cpu_s:.2f} s "
                         f"wall; GB/s over that sample's share of the bytes",
               "tokens_per_s": round(len(seqs) / cpu_s, 3)}
        log(f"[bench] oracle (window sample): {cpu_s:.2f}s")
    return d, cpu


def mx_oracle_check(w, L1, got, decode_bytes, args, oracle):
    """Oracle check of an MXFP8 run on a sample of sequences: the oracle
    quantizes those sequences' rows (and the appended token) into its own
    pools and decodes them; that decode is also the timed CPU leg."""
    import numpy as np

    spec = w.spec
    seqs = sample_seqs(spec)
    pools = oracle_mx_pools(w, seqs, oracle)
    pairs = [(b, h) for b in seqs for h in range(spec.num_q_heads)]
    threads = oracle.default_threads()
    t_c = time.perf_counter()
    ref = oracle.decode_mxfp8(w.q, *pools, w.block_tables, L1, w.scale, pairs=pairs,
                              threads=threads)
    cpu_s = time.perf_counter() - t_c
    sel = np.array(pairs)
    d = np.abs(got[sel[:, 0], sel[:, 1]] - ref[sel[:, 0], sel[:, 1]])
    frac = float(L1[seqs].sum()) / float(L1.sum())
    cpu = None
    if not args.no_cpu_baseline:
        cpu = {"value": round(decode_bytes * frac / cpu_s / 1e9, 3), "unit": "GB/s",
               "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"oracle MXFP8 decode of {len(seqs)} of the {spec.num_seqs} sequences "
                         f"({frac:.1%} of the attended tokens, all {spec.num_q_heads} heads), "
                         f"fp64, {cpu_s:.2f} s wall; GB/s over that sample's share of the bytes",
               "tokens_per_s": round(len(seqs) / cpu_s, 3)}
        log(f"[bench] oracle (mxfp8 sample): {cpu_s:.2f}s on {threads} threads")
    return d, cpu


def native_oracle_check(w, L1, got, decode_bytes, args, oracle):
    """Oracle check of a run on the workload's own caches: 128 sampled rows
    with --no-cpu-baseline, else the full decode, timed (median of 3) as the
    CPU leg."""
    import numpy as np

    spec = w.spec
    hk = w.k_cache.copy()
    hv = None if w.v_cache is None else w.v_cache.copy()
    oracle.append(hk, hv, w.k_new, w.v_new, w.slot_mapping)
    if args.no_cpu_baseline:
        rng = np.random.default_rng(0)
        rows = [(int(b), int(h)) for b, h in zip(rng.integers(0, spec.num_seqs, 128),
                                                 rng.integers(0, spec.num_q_heads, 128))]
        ref = oracle.decode(w.q, hk, hv, w.block_tables, L1, w.scale, pairs=rows,
                            head_dim_v=spec.head_dim_v)
        sel = np.array(rows)
        return np.abs(got[sel[:, 0], sel[:, 1]] - ref[sel[:, 0], sel[:, 1]]), None
    threads = oracle.default_threads()
    times = []
    for _ in range(3):  # median of three full decodes
        t_c = time.perf_counter()
        ref = oracle.decode(w.q, hk, hv, w.block_tables, L1, w.scale, threads=threads,
                            head_dim_v=spec.head_dim_v)
        times.append(time.perf_counter() - t_c)
    cpu_s = float(np.median(times))
    cpu = {"value": round(decode_bytes / cpu_s / 1e9, 3), "unit": "GB/s",
           "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
           "sample": f"the full decode of the {args.config} batch "
                     f"({spec.num_seqs} seqs x {spec.num_q_heads} heads), fp64, "
                     f"median of 3 runs, {cpu_s:.2f} s wall each",
           "tokens_per_s": round(spec.num_seqs / cpu_s, 3)}
    log(f"[bench] oracle: {cpu_s:.2f}s per decode on {threads} threads")
    return np.abs(got - ref), cpu


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--kv-format", default="native", choices=["native", "mxfp8"],
                    help="cache format: the workload's dtype, or MXFP8 (bf16 d=128 shapes)")
    ap.add_argument("--q-heads", type=int, default=0,
                    help="latent workload only: its query heads (16..128, a multiple of 16, as "
                         "a 128-head model split over GPUs by heads); 0 keeps the workload's")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (pa_decode_multi when > 1)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens (pa_decode_ex; 0 = the whole context)")
    ap.add_argument("--scores", action="store_true",
                    help="also time pa_attention_scores (per-token attention mass over the "
                         "window, from pa_decode_ex's log-sum-exp) on the same workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by KV head or sequence with no exchange; see DESIGN.md)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_58_amd as pa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    spec = workloads.CONFIGS[args.config]
    H = args.q_heads
    if H:
        if not spec.mla or H % 16 or not 16 <= H <= 128:
            log(f"--q-heads takes 16..128 (a multiple of 16) on the latent workload, not {args.config}")
            return 2
        # same seed (the spec's index), so the same context lengths and latent
        spec = dataclasses.replace(spec, num_q_heads=H)

    t0 = time.time()
    w = workloads.make_workload(spec)
    log(f"[bench] generated {args.config} in {time.time() - t0:.1f}s: "
        f"{w.num_blocks} blocks, sum ctx {int(w.context_lens.sum())}")

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    mx = args.kv_format == "mxfp8"
    if mx and (spec.dtype != "bf16" or spec.mla or spec.head_dim_k != 128):
        log(f"--kv-format mxfp8 runs the bf16 head-dim-128 workloads, not {args.config}")
        return 2
    Q = args.q_len
    if Q > 1 and (spec.dtype != "bf16" or spec.mla or spec.head_dim_k != 128):
        log(f"--q-len > 1 runs the bf16 head-dim-128 workloads, not {args.config}")
        return 2
    W = args.window
    if W and (mx or Q > 1 or spec.mla):
        log("--window runs the single-query grouped workloads on their own caches")
        return 2
    q_host = w.q if Q == 1 else workloads.multi_query(w, Q)
    q = to_dev(q_host)
    k_new, v_new = to_dev(w.k_new), to_dev(w.v_new)
    bt = torch.from_numpy(w.block_tables).to(dev)
    L1 = (w.context_lens + 1).astype(np.int32)  # context after the append
    cl = torch.from_numpy(L1).to(dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    out = torch.empty(q.shape[:-1] + (spec.head_dim_v,), dtype=q.dtype, device=dev)
    if not mx:
        kc, vc = to_dev(w.k_cache), to_dev(w.v_cache)

        def append():
            pa.cache_append(kc, vc, k_new, v_new, sm)

        if Q == 1 and W:
            ws = pa.alloc_workspace(q, kc, bt, head_dim_v=spec.head_dim_v)

            def decode():
                pa.decode_ex(out, q, kc, vc, bt, cl, w.scale, ws, window=W)
        elif Q == 1:
            ws = pa.alloc_workspace(q, kc, bt, head_dim_v=spec.head_dim_v)

            def decode():
                pa.decode(out, q, kc, vc, bt, cl, w.scale, ws)
        else:
            ws = pa.alloc_multi_workspace(q, spec.num_kv_heads, spec.block_size, bt)

            def decode():
                pa.decode_multi(out, q, kc, vc, bt, cl, w.scale, ws)
    else:
        # MXFP8 pools (unused slots hold the E4M3 NaN code), filled with every
        # cached row of the workload by the library's quantizing append
        bs = spec.block_size
        pools = pa.alloc_mxfp8_cache(w.num_blocks, bs, spec.num_kv_heads, 128, dev, fill=0x7F)
        slots = valid_slots(w)
        for lo in range(0, slots.size, 1 << 16):
            sl = slots[lo: lo + (1 << 16)]
            pa.cache_append_mxfp8(*pools, to_dev(np.ascontiguousarray(w.k_cache[sl // bs, sl % bs])),
                                  to_dev(np.ascontiguousarray(w.v_cache[sl // bs, sl % bs])),
                                  torch.from_numpy(sl).to(dev))
        def append():
            pa.cache_append_mxfp8(*pools, k_new, v_new, sm)

        if Q == 1:
            ws = pa.alloc_mxfp8_workspace(q, pools[0], bt)

            def decode():
                pa.decode_mxfp8(out, q, *pools, bt, cl, w.scale, ws)
        else:
            ws = pa.alloc_multi_workspace(q, spec.num_kv_heads, spec.block_size, bt)

            def decode():
                pa.decode_multi(out, q, pools[0], pools[1], bt, cl, w.scale, ws,
                                k_scale=pools[2], v_scale=pools[3])
    torch.cuda.synchronize()

    def step():
        append()
        decode()

    # L2 (4 MB per XCD) and MALL (256 MB) flush between the cold repetitions
    # below, outside their event pairs: a kernel that reads 512 MiB (twice the
    # MALL).  A write flush would leave up to 256 MB of dirty MALL lines whose
    # write-back lands inside the next timed call.
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    flush_sink = torch.empty((), dtype=torch.int64, device=dev)

    def flush():
        torch.sum(flush_buf, 0, dtype=torch.int64, out=flush_sink)

    # Clock ramp: the GPU runs its first few hundred ms of work at lower
    # clocks, so flush reads (not steps of the hot path) run for ~0.5 s first.
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < 0.5:
        for _ in range(20):
            flush()
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps back to back between two events on torch's
    # current stream (the stream the binding hands to the library), nothing
    # else in between: events between the calls would add their own gaps.
    K = args.steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(K):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)

    # The same steps with an event around each call (the per-call warm times;
    # the events cost a few us per step, so this loop is not the timed one).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        append()
        ev[i][1].record()
        decode()
        ev[i][2].record()
    torch.cuda.synchronize()
    t_append_warm = np.array([e[0].elapsed_time(e[1]) for e in ev])
    t_decode_warm = np.array([e[1].elapsed_time(e[2]) for e in ev])
    ms_per_step = total_ms / K

    def cold_times(fn_append, fn_decode, reps):
        """Per-call event times with L2 and MALL flushed before every call."""
        ta, td = [], []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            flush()
            e[0].record()
            fn_append()
            e[1].record()
            flush()
            e[2].record()
            fn_decode()
            e[3].record()
            torch.cuda.synchronize()
            ta.append(e[0].elapsed_time(e[1]))
            td.append(e[2].elapsed_time(e[3]))
        return np.array(ta), np.array(td)

    # The same K steps again, each call on cold caches: the per-kernel times
    # the roofline is quoted on.
    t_append, t_decode = cold_times(append, decode, K)

    # The other grouped kernel on the same inputs, for comparison (the
    # matrix-core variant of the single-query GQA decode).
    alt = None
    if kernel_name(spec, mx, Q, W) == GROUPED:
        os.environ["PA_GQA_MFMA"] = "1"
        try:
            for _ in range(max(args.warmup, 3)):
                decode()
            _, t_alt = cold_times(lambda: None, decode, K)
        finally:
            del os.environ["PA_GQA_MFMA"]
        alt = {"kernel": GROUPED_MFMA, "us_decode": round(float(np.mean(t_alt)) * 1e3, 2)}
        decode()  # the default kernel's output for the oracle check below
        torch.cuda.synchronize()
    scores_leg = None
    if args.scores:
        if mx or Q > 1 or spec.mla:
            log("--scores runs on the single-query grouped workloads' own caches")
            return 2
        # lse from the windowed decode, then the scores pass alone, cold
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        ws_s = pa.alloc_workspace(q, kc, bt)
        pa.decode_ex(out, q, kc, vc, bt, cl, w.scale, ws_s, window=W, lse=lse)
        max_ctx = int(bt.shape[1]) * spec.block_size
        scores_t = torch.empty((spec.num_seqs, spec.num_kv_heads, max_ctx), dtype=torch.float32,
                               device=dev)

        def scores_call():
            pa.attention_scores(scores_t, q, kc, bt, cl, lse, w.scale, window=W)

        for _ in range(max(args.warmup, 3)):
            scores_call()
        _, t_sc = cold_times(lambda: None, scores_call, K)
        att = np.minimum(L1, W) if W else L1
        sc_bytes = (int(att.sum()) * spec.num_kv_heads * spec.head_dim_k * spec.elt +  # K rows once
                    spec.num_seqs * spec.num_q_heads * (spec.head_dim_k * spec.elt + 4) +  # q, lse
                    spec.num_seqs * spec.num_kv_heads * max_ctx * 4 +  # scores written
                    4 * int(((L1 + spec.block_size - 1) // spec.block_size).sum()))  # block ids
        us_sc = float(np.mean(t_sc)) * 1e3
        scores_leg = {"kernel": "attention_scores_kernel", "us": round(us_sc, 2),
                      "algorithmic_bytes": sc_bytes,
                      "roofline": {"bound": "hbm", "achieved": round(sc_bytes / (us_sc * 1e-6) / 1e9, 2),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(sc_bytes / (us_sc * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
        log(f"[bench] attention scores: {us_sc:.1f} us = {scores_leg['roofline']['frac']:.1%} of HBM")
        decode()  # the timed step's output for the oracle check below
        torch.cuda.synchronize()
    del flush_buf

    # accounting over the context actually attended (ctx + 1)
    # accounting over the tokens attended (the window's, with --window)
    L_att = np.minimum(L1, W) if W else L1
    w_after = workloads.Workload(**{**w.__dict__, "context_lens": L_att.astype(np.int32)})
    decode_bytes = (workloads.algorithmic_bytes_mxfp8 if mx else workloads.algorithmic_bytes)(w_after)
    # q and O scale with the queries per sequence; the cache is read once
    qo_bytes = spec.num_seqs * spec.num_q_heads * (spec.head_dim_k + spec.head_dim_v) * spec.elt
    decode_bytes += (Q - 1) * qo_bytes
    append_bytes = (workloads.append_bytes_mxfp8 if mx else workloads.append_bytes)(w)
    if Q == 1:
        flops = workloads.algorithmic_flops(w_after)
    else:  # each query over the tokens it sees
        seen = int(np.clip(L1[:, None] - Q + 1 + np.arange(Q)[None, :], 0, None).sum())
        flops = 2 * spec.num_q_heads * (spec.head_dim_k + spec.head_dim_v) * seen
    step_bytes = decode_bytes + append_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_ms = float(np.mean(t_decode))
    achieved = decode_bytes / (dec_ms * 1e-3) / 1e9
    log(f"[bench] {K} steps: {ms_per_step * 1e3:.1f} us/step back to back (decode "
        f"{np.mean(t_decode_warm) * 1e3:.1f} us); cold caches: append "
        f"{np.mean(t_append) * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us = {achieved:.0f} GB/s = "
        f"{achieved / HBM_PEAK_GBS:.1%} of HBM peak")
    if alt is not None:
        alt["frac"] = round(decode_bytes / (alt["us_decode"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        log(f"[bench] {alt['kernel']}: decode {alt['us_decode']:.1f} us = {alt['frac']:.1%}")

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + written once")
        del src, dst

    # correctness of the timed output against the oracle (also the CPU leg)
    import oracle

    got = out.float().cpu().numpy().astype(np.float64)
    if W:
        d, cpu = window_oracle_check(w, L1, got, W, decode_bytes, args, oracle)
    elif Q > 1:
        d, cpu = multi_oracle_check(w, L1, got, q_host, decode_bytes, args, oracle, mx)
    elif mx:
        d, cpu = mx_oracle_check(w, L1, got, decode_bytes, args, oracle)
    else:
        d, cpu = native_oracle_check(w, L1, got, decode_bytes, args, oracle)
    max_err = float(d.max())

    key = args.config + ("_mxfp8" if mx else "_mfma" if kernel_name(spec, mx, Q, W) == GROUPED_MFMA else "")
    traffic = load_traffic(key, decode_bytes) if Q == 1 and not W and not H else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config] + (
                       ", KV cache in MXFP8 (E4M3 + E8M0 per 32 values)" if mx else "") + (
                       f", {Q} causal query tokens per sequence" if Q > 1 else "") + (
                       f", sliding window of {W} tokens" if W else "") + (
                       f", {H} query heads instead of {workloads.CONFIGS[args.config].num_q_heads}"
                       if H else ""),
                   "name": spec.name + ("-mxfp8" if mx else "") + (f"-q{Q}" if Q > 1 else "") +
                           (f"-h{H}" if H else "") +
                           (f"-w{W}" if W else ""),
                   "kv_format": args.kv_format,
                   "global_batch": spec.num_seqs, "seq_len": int(L1.max()),
                   "mean_context": float(L1.mean()), "parallelism": "single GPU"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(spec.num_seqs * Q / (ms_per_step * 1e-3), 1),
        "q_len": Q,
        "us_append": round(float(np.mean(t_append)) * 1e3, 2),
        "us_decode": round(dec_ms * 1e3, 2),
        "us_decode_median": round(float(np.median(t_decode)) * 1e3, 2),
        "us_decode_p10_p90": [round(float(np.percentile(t_decode, 10)) * 1e3, 2),
                              round(float(np.percentile(t_decode, 90)) * 1e3, 2)],
        "us_decode_warm": round(float(np.mean(t_decode_warm)) * 1e3, 2),
        "timing": "us_append / us_decode: per-call HIP events with L2 and MALL flushed "
                  "(512 MiB read) before every call; ms_per_step: the K steps back to back "
                  "between two events; us_decode_warm: a second back-to-back pass with an "
                  "event around each call",
        "decode_tflops": round(flops / (dec_ms * 1e-3) / 1e12, 3),
        "roofline": {"bound": "hbm", "kernel": kernel_name(spec, mx, Q, W),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": decode_bytes},
        "other_kernel": alt,
        "attention_scores": scores_leg,
        "cpu_baseline": cpu,
        "max_abs_err_vs_oracle": max_err,
        "wall_s_timed": round(wall, 4),
    }
    if mx:
        result["dtype"] = "fp8-e4m3 (MXFP8 cache), bf16 q/out, fp32 accumulate"
    if spec.mla:
        # the latent contraction sits near the ridge: its matrix-core roofline too
        tflops = flops / (dec_ms * 1e-3) / 1e12
        result["roofline_mfma"] = {"bound": "mfma", "achieved": round(tflops, 2),
                                   "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "algorithmic_flops": flops}
    print(json.dumps(result), flush=True)
    tol = 2e-3 if spec.dtype == "f32" else 1.5e-2
    if not max_err <= tol:
        log(f"[bench] PARITY FAILURE: max |delta| {max_err} > {tol}")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
