"""Pins of the oracle's MXFP8 part (E4M3 values with E8M0 block scales).

Each check comes from outside the oracle: torch's float8_e4m3fn conversions
(an independent implementation of the same OCP format), closed-form values of
the format, brute force over all 256 codes, the error bound of rounding to
nearest, and the oracle's already pinned float decode applied to caches that
the test dequantizes itself with torch.  A last group plants slips in a copy
of the oracle source and checks that these pins catch them.
"""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import pack_paged

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")
ALL = np.arange(256, dtype=np.uint8)


def torch_e4m3_values(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn conversion, as bytes (inputs within +-448)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Test-side dequantization with torch: code value * 2^(e - 127), blocks of 32."""
    vals = torch_e4m3_values(codes)
    exps = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1)
    return np.ldexp(vals, exps)


# ---- the E4M3 element format ------------------------------------------------

def test_e4m3_values_match_torch_for_every_code():
    got = oracle.e4m3_values(ALL)
    ref = torch_e4m3_values(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_forms():
    v = oracle.e4m3_values(ALL)
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0        # 1.75 * 2^8, the largest
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])   # the only NaNs
    assert np.isnan(v).sum() == 2
    assert v[0x78] == 256.0 and v[0x38] == 1.0 and v[0x30] == 0.5
    assert v[0x08] == 2.0 ** -6                          # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9  # subnormals m * 2^-9
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..0x7E ascend
    assert np.array_equal(v[0x80:0xFF], -pos)            # sign bit mirrors


def test_e4m3_encode_round_trips_every_finite_code():
    finite = ALL[~np.isnan(oracle.e4m3_values(ALL))]
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_values(finite)), finite)


def test_e4m3_encode_matches_torch_including_ties():
    rng = np.random.default_rng(5)
    mags = np.exp2(rng.uniform(-14, math.log2(447.9), 20000))
    x = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    # exact midpoints between neighbouring codes: round half to even decides them
    pos = oracle.e4m3_values(ALL[:0x7F])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 2.0 ** -10, 447.99])])
    got = oracle.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, torch_e4m3_encode(x))


def test_e4m3_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(300) * 10, rng.uniform(-448, 448, 300),
                        rng.standard_normal(100) * 0.01])
    vals = oracle.e4m3_values(ALL)
    finite = ~np.isnan(vals)
    got = oracle.e4m3_values(oracle.e4m3_encode(x))
    for xi, gi in zip(x, got):
        best = np.min(np.abs(vals[finite] - xi))
        assert abs(gi - xi) == best


def test_e4m3_encode_saturates():
    big = np.array([448.0, 448.5, 463.9, 464.0, 480.0, 1e6, 1e300])
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)


# ---- E8M0 block scales ---------------------------------------------------------

def test_e8m0_values():
    v = oracle.e8m0_values(ALL)
    assert math.isnan(v[255])
    assert np.array_equal(v[:255], np.ldexp(1.0, np.arange(255) - 127))


@pytest.mark.parametrize("k", [-100, -20, -8, 0, 5, 100])
def test_mx_scale_puts_block_max_at_top_code(k):
    """A block whose largest magnitude is 448 * 2^k gets X = k (floor(log2 448)
    = 8), and that element becomes the largest code exactly."""
    rng = np.random.default_rng(7)
    x = rng.uniform(-1, 1, 32) * 447 * 2.0 ** k
    x[11] = -448 * 2.0 ** k
    codes, scales = oracle.mx_quantize(x.astype(np.float32)[None, :])
    assert scales[0, 0] == 127 + k
    assert codes[0, 11] == 0xFE


def test_mx_scale_special_blocks():
    z = np.zeros((1, 64), np.float32)
    z[0, 40] = 1.0  # second block: amax 1 -> X = -8, 1 * 2^8 = 256 = code 0x78
    codes, scales = oracle.mx_quantize(z)
    assert list(scales[0]) == [0, 119]          # all-zero block -> X = -127 (byte 0)
    assert np.all(codes[0, :32] == 0) and codes[0, 40] == 0x78
    tiny = np.full((1, 32), np.float32(2.0 ** -149))  # float32's smallest subnormal
    assert oracle.mx_quantize(tiny)[1][0, 0] == 0    # floor(log2) - 8 clamps to -127
    huge = np.full((1, 32), np.float32(3e38))        # floor(log2 3e38) = 127 -> X = 119
    c, s = oracle.mx_quantize(huge)
    assert s[0, 0] == 127 + 119 and np.all(c == 0x7E)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_mx_quantize_error_bound(kind):
    """Every element is within half a quantum of its dequantized value, the
    quantum being that of E4M3 at the scaled magnitude (the block max never
    saturates by more than the top binade's spacing)."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[::7, 5] *= 300.0  # outlier channels
    if kind == "bf16":
        xb = torch.from_numpy(x).to(torch.bfloat16)
        src = xb.view(torch.int16).numpy().view(np.uint16)
        x = xb.to(torch.float32).numpy()
    else:
        src = x
    codes, scales = oracle.mx_quantize(src)
    deq = dequant(codes, scales)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1)
    y = np.abs(np.ldexp(x.astype(np.float64), -X))
    e = np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -30))), -6)
    half_q = np.ldexp(0.5, (e - 3 + X).astype(np.int64))
    err = np.abs(deq - x)
    sat = y > 448
    assert np.all(err[~sat] <= half_q[~sat])
    assert np.all(err[sat] <= np.ldexp(64.0, X[sat]))
    # The scale rule puts the block max in [256, 512) after scaling; past 448
    # it saturates, so the block max loses at most 1 - 448/512 = 1/8, and
    # some block here does hit that regime.
    amax = np.abs(x).reshape(64, 4, 32).max(-1)
    d_amax = np.abs(deq).reshape(64, 4, 32).max(-1)
    assert np.all(np.abs(d_amax - amax) <= amax * 2.0 ** -3)
    assert np.any(np.abs(d_amax - amax) > amax * 2.0 ** -4)


# ---- cache layout and decode -----------------------------------------------------

def _mx_pool(rng, nb, bs, hkv, d, poison=0x7F):
    k8 = np.full((nb, hkv, bs, d), poison, np.uint8)
    v8 = np.full((nb, hkv, d, bs), poison, np.uint8)
    ks = np.full((nb, hkv, bs, d // 32), 200, np.uint8)
    vs = np.full((nb, hkv, bs, d // 32), 200, np.uint8)
    return k8, v8, ks, vs


def test_append_mxfp8_places_rows_and_columns():
    rng = np.random.default_rng(9)
    nb, bs, hkv, d = 5, 4, 2, 64
    k8, v8, ks, vs = _mx_pool(rng, nb, bs, hkv, d)
    n = 6
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32) * 3
    slots = np.array([7, -1, 0, 19, 12, 5], np.int32)
    before = [a.copy() for a in (k8, v8, ks, vs)]
    oracle.append_mxfp8(k8, v8, ks, vs, k, v, slots)
    kc, kscale = oracle.mx_quantize(k)
    vc, vscale = oracle.mx_quantize(v)
    ek, ev, eks, evs = [a.copy() for a in before]
    for i, s in enumerate(slots):
        if s < 0:
            continue
        p, r = divmod(int(s), bs)
        ek[p, :, r, :] = kc[i]
        ev[p, :, :, r] = vc[i]
        eks[p, :, r, :] = kscale[i]
        evs[p, :, r, :] = vscale[i]
    for got, exp in zip((k8, v8, ks, vs), (ek, ev, eks, evs)):
        assert np.array_equal(got, exp)


def _fill_mx_sequences(rng, lens, hkv, d, bs, dtype="bf16", q_heads=None):
    """Random K/V per sequence, packed paged (block ids permuted), quantized
    into MXFP8 caches by the oracle's append; returns everything plus the
    test's own float32 dequantized pools in the standard layout."""
    ks_seq = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vs_seq = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    _, bt = pack_paged(ks_seq, bs, pool_blocks=sum(-(-L // bs) for L in lens) + 3,
                       rng=np.random.default_rng(3))
    nb = int(bt.max()) + 4
    k8, v8, kscale, vscale = _mx_pool(rng, nb, bs, hkv, d)
    for b, L in enumerate(lens):
        slots = np.array([bt[b, t // bs] * bs + t % bs for t in range(L)], np.int32)
        oracle.append_mxfp8(k8, v8, kscale, vscale, ks_seq[b], vs_seq[b], slots)
    kf = dequant(k8, kscale).transpose(0, 2, 1, 3).astype(np.float32)          # [nb, bs, hkv, d]
    vf = dequant(v8.transpose(0, 1, 3, 2), vscale).transpose(0, 2, 1, 3).astype(np.float32)
    return k8, v8, kscale, vscale, kf, vf, bt


def test_decode_mxfp8_equals_float_decode_of_dequantized_pool():
    rng = np.random.default_rng(10)
    lens = [1, 7, 33, 70]
    hkv, d, bs, hq = 2, 64, 8, 8
    k8, v8, kscale, vscale, kf, vf, bt = _fill_mx_sequences(rng, lens, hkv, d, bs)
    assert np.all(np.isfinite(kf[~np.isnan(kf)]))
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    cl = np.array(lens, np.int32)
    got = oracle.decode_mxfp8(q, k8, v8, kscale, vscale, bt, cl, 0.2)
    ref = oracle.decode(q, np.nan_to_num(kf), np.nan_to_num(vf), bt, cl, 0.2)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_decode_mxfp8_block_permutation_invariant():
    rng = np.random.default_rng(11)
    lens = [20, 45]
    hkv, d, bs, hq = 1, 32, 4, 2
    k8, v8, kscale, vscale, _, _, bt = _fill_mx_sequences(rng, lens, hkv, d, bs)
    q = rng.standard_normal((2, hq, d)).astype(np.float32)
    cl = np.array(lens, np.int32)
    a = oracle.decode_mxfp8(q, k8, v8, kscale, vscale, bt, cl, 0.3)
    perm = rng.permutation(k8.shape[0])
    inv = np.argsort(perm)
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    b = oracle.decode_mxfp8(q, k8[perm], v8[perm], kscale[perm], vscale[perm], bt2, cl, 0.3)
    assert np.array_equal(a, b)


# ---- planted slips ---------------------------------------------------------------

MX_MUTANTS = {
    "ties_away": ("nearbyint(a / quantum)", "round(a / quantum)"),
    "scale_offset_7": ("int x = (e2 - 1) - 8;", "int x = (e2 - 1) - 7;"),
    "no_saturation": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 480.0) return sign | 0x7F;"),
    "subnormal_quantum": ("if (a == 0.0 || ex < -6) ex = -6;", "if (a == 0.0 || ex < -7) ex = -7;"),
    "e4m3_bias_8": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "v_not_transposed": ("v8[(tile * d + e) * bs + r] = row[e];", "v8[(tile * bs + r) * d + e] = row[e];"),
    "decode_v_scale_of_k": ("oracle_e8m0_value(vs[(tile * bs + r) * nsc + j / 32]);",
                            "oracle_e8m0_value(ks[(tile * bs + r) * nsc + j / 32]);"),
    "decode_k_scale_block": ("ks[(tile * bs + r) * nsc + i / 32]", "ks[(tile * bs + r) * nsc + i / 64]"),
    "append_head_ignored": ("const int64_t tile = p * Hkv + h;", "const int64_t tile = p * Hkv;"),
}


def _mx_checks_pass(lib) -> bool:
    vals = np.array([lib.oracle_e4m3_value(int(c)) for c in ALL])
    ref = torch_e4m3_values(ALL)
    if not (np.array_equal(np.isnan(vals), np.isnan(ref))
            and np.array_equal(vals[~np.isnan(ref)], ref[~np.isnan(ref)])):
        return False
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(4000) * rng.choice([1e-3, 1, 100], 4000)).astype(np.float32)
    pos = ref[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([np.clip(x, -447, 447), mids, np.float32([500.0, -1e9])])
    got = oracle.e4m3_encode(x.astype(np.float64), lib=lib)
    exp = torch_e4m3_encode(np.clip(x, -448, 448))
    if not np.array_equal(got, exp):
        return False
    blk = rng.uniform(-1, 1, (1, 32)).astype(np.float32)
    blk[0, 3] = 448 * 2.0 ** -5
    c, s = oracle.mx_quantize(blk, lib=lib)
    if s[0, 0] != 127 - 5 or c[0, 3] != 0x7E:
        return False
    # layout and decode against the test's own dequantization and the float oracle
    lens = [5, 30]
    hkv, d, bs, hq = 2, 64, 8, 4
    ks_seq = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vs_seq = [(rng.standard_normal((L, hkv, d)) * 8).astype(np.float32) for L in lens]
    _, bt = pack_paged(ks_seq, bs, rng=np.random.default_rng(1))
    nb = int(bt.max()) + 1
    k8, v8, kscale, vscale = _mx_pool(rng, nb, bs, hkv, d, poison=0)
    for b, L in enumerate(lens):
        slots = np.array([bt[b, t // bs] * bs + t % bs for t in range(L)], np.int32)
        oracle.append_mxfp8(k8, v8, kscale, vscale, ks_seq[b], vs_seq[b], slots, lib=lib)
    kf = dequant(k8, kscale).transpose(0, 2, 1, 3).astype(np.float32)
    vf = dequant(v8.transpose(0, 1, 3, 2), vscale).transpose(0, 2, 1, 3).astype(np.float32)
    for b, L in enumerate(lens):  # the pools hold the sequences' rows to within the bound
        for t in range(L):        # (1/8 relative at worst, where a block max saturates)
            p, r = bt[b, t // bs], t % bs
            if not np.allclose(kf[p, r], ks_seq[b][t], rtol=2.0 ** -3, atol=2.0 ** -6):
                return False
            if not np.allclose(vf[p, r], vs_seq[b][t], rtol=2.0 ** -3, atol=2.0 ** -3):
                return False
    q = rng.standard_normal((2, hq, d)).astype(np.float32)
    cl = np.array(lens, np.int32)
    got = oracle.decode_mxfp8(q, k8, v8, kscale, vscale, bt, cl, 0.25, lib=lib)
    ref = oracle.decode(q, kf, vf, bt, cl, 0.25)
    return bool(np.allclose(got, ref, rtol=1e-12, atol=1e-14))


def _build(tmp_path, text, tag):
    src = tmp_path / f"{tag}.c"
    so = tmp_path / f"lib{tag}.so"
    src.write_text(text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", "-o",
                    str(so), str(src), "-lm"], check=True)
    return oracle.load_library(str(so))


def test_mx_unmutated_copy_passes(tmp_path):
    with open(SRC) as f:
        assert _mx_checks_pass(_build(tmp_path, f.read(), "orig"))


@pytest.mark.parametrize("name", sorted(MX_MUTANTS))
def test_mx_mutant_is_caught(tmp_path, name):
    old, new = MX_MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not found once"
    assert not _mx_checks_pass(_build(tmp_path, text.replace(old, new), name)), \
        f"planted mistake {name} was not caught"
