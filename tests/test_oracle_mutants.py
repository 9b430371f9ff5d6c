"""Planted mistakes: a copy of the oracle with one plausible slip must fail a pin.

Each mutant is built from the oracle source with one textual change, compiled
into a temporary directory with gcc, and run through the same independent
checks the pins use (library attention on a contiguous layout, numpy widening,
exact append).  Only CPU code is involved, and every mutation keeps its memory
accesses inside the arrays it is given.
"""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.helpers import as_f64, gather_sequence, pack_paged, sdpa_reference
from workloads import custom_spec, make_workload

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

MUTANTS = {
    "gqa_head_modulo": ("const int g = h / G;", "const int g = h % Hkv;"),
    "row_from_block_index": ("const int r = t % bs;\n        const int64_t k_off",
                             "const int r = (t / bs) % bs;\n        const int64_t k_off"),
    "dropped_scale": ("s[t] = scale * dot;", "s[t] = dot;"),
    "wrong_exp_sign": ("const double w = exp(s[t] - m);", "const double w = exp(m - s[t]);"),
    "no_normalisation": ("out_row[j] = o[j] / denom;", "out_row[j] = o[j];"),
    "dropped_kv_head": ("const int64_t k_off = ((p * bs + r) * Hkv + g) * (int64_t)dk;",
                        "const int64_t k_off = ((p * bs + r) * Hkv) * (int64_t)dk;"),
    "latent_row_stride": ("v_off = ((p * bs + r) * Hkv + g) * (int64_t)dk;",
                          "v_off = ((p * bs + r) * Hkv + g) * (int64_t)dv;"),
    "bf16_shift": ("[idx] << 16;", "[idx] << 15;"),
    "max_skips_first": ("double m = s[0];", "double m = 0.0;\n    (void)0;"),
    "block_table_row": ("t / bs];\n        const int r = t % bs;\n        const int64_t k_off",
                        "(t / bs) / 2];\n        const int r = t % bs;\n        const int64_t k_off"),
    "v_block_table_row": ("t / bs];\n        const int r = t % bs;\n        int64_t v_off",
                          "(t / bs) / 2];\n        const int r = t % bs;\n        int64_t v_off"),
    "append_next_row": ("memcpy((char *)k_cache + s * k_row,",
                        "memcpy((char *)k_cache + (s / 2) * k_row,"),
    "append_v_stride": ("(const char *)v + (int64_t)i * v_token_stride * elt_bytes",
                        "(const char *)v + (int64_t)i * k_token_stride * elt_bytes"),
}


def _checks_pass(lib) -> bool:
    """True when every independent check passes for this library."""
    # GQA paged vs contiguous library attention (f32, several lengths)
    rng = np.random.default_rng(4)
    lens = [1, 17, 40]
    ks = [rng.standard_normal((L, 2, 16)).astype(np.float32) for L in lens]
    vs = [rng.standard_normal((L, 2, 16)).astype(np.float32) for L in lens]
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    kp, bt = pack_paged(ks, 8, pool_blocks=12, rng=np.random.default_rng(2))
    vp, _ = pack_paged(vs, 8, pool_blocks=12, rng=np.random.default_rng(2))
    got = oracle.decode(q, kp, vp, bt, np.array(lens, np.int32), 0.3, lib=lib)
    for b in range(3):
        if not np.allclose(got[b], sdpa_reference(q[b], ks[b], vs[b], 0.3), rtol=1e-12,
                           atol=1e-13):
            return False
    # scores far beyond exp's range: only a max-subtracted softmax stays finite
    q1 = np.zeros((1, 1, 4), np.float32)
    q1[0, 0, 0] = 1.0
    K1 = np.zeros((3, 1, 4), np.float32)
    K1[:, 0, 0] = [10.0, 1.0, 0.0]
    V1 = np.arange(12, dtype=np.float32).reshape(3, 1, 4)
    kp1, bt1 = pack_paged([K1], 2)
    vp1, _ = pack_paged([V1], 2)
    o1 = oracle.decode(q1, kp1, vp1, bt1, np.array([3], np.int32), 100.0, lib=lib)[0, 0]
    if not np.allclose(o1, V1[0, 0], rtol=0, atol=1e-40):
        return False
    # bf16 widening and latent mode against numpy widening + library attention
    spec = custom_spec(2, 4, 1, 24, 8, "bf16", ctx=[9, 20], head_dim_v=16, mla=True,
                       scale=1.0 / math.sqrt(24))
    w = make_workload(spec)
    got = oracle.decode_workload(w, lib=lib)
    for b in range(2):
        L = int(w.context_lens[b])
        K = as_f64(gather_sequence(w.k_cache, w.block_tables, b, L))
        ref = sdpa_reference(as_f64(w.q[b]), K, K[:, :, :16], w.scale)
        if not np.allclose(got[b], ref, rtol=1e-12, atol=1e-13):
            return False
    # append: exact scatter, with a -1 and a v stride different from k's
    w = make_workload(custom_spec(3, 2, 1, 8, 4, "f32", ctx=[3, 5, 0], head_dim_v=4))
    k0, v0 = w.k_cache.copy(), w.v_cache.copy()
    slots = w.slot_mapping.copy()
    slots[2] = -1
    oracle.append(w.k_cache, w.v_cache, w.k_new, w.v_new, slots, lib=lib)
    ek, ev = k0.reshape(-1, 8).copy(), v0.reshape(-1, 4).copy()
    for i, s in enumerate(slots):
        if s >= 0:
            ek[s] = w.k_new[i].reshape(-1)
            ev[s] = w.v_new[i].reshape(-1)
    same = lambda a, b: np.array_equal(a.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8))
    return same(w.k_cache, ek) and same(w.v_cache, ev)


def _build(tmp_path, text, tag):
    src = tmp_path / f"{tag}.c"
    so = tmp_path / f"lib{tag}.so"
    src.write_text(text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", "-o",
                    str(so), str(src), "-lm"], check=True)
    return oracle.load_library(str(so))


def test_unmutated_copy_passes(tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert _checks_pass(_build(tmp_path, text, "orig"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not found once"
    lib = _build(tmp_path, text.replace(old, new), name)
    assert not _checks_pass(lib), f"planted mistake {name} was not caught"
