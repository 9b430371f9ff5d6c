"""CPU oracle for paged decode attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (``paged_kv_cache_58_amd``)
never does, and this package imports nothing from the product.

The arithmetic lives in ``pa_oracle.c`` (plain C, double precision, OpenMP over
(sequence, head)); this file only builds and calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """ctypes handle with argument types set, for liboracle.so or a rebuilt copy."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_decode.restype = I
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, ctypes.c_double, I, I, I, I, I,
                                  I, I, I, P, I, I]
    lib.oracle_append.restype = I
    lib.oracle_append.argtypes = [P, P, P, ctypes.c_int64, P, ctypes.c_int64, P, I, I,
                                  I, I, I, I, I]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_array.argtypes = [P, ctypes.c_int64, P]
    lib.oracle_mx_quantize.restype = I
    lib.oracle_mx_quantize.argtypes = [P, I, ctypes.c_int64, I, P, P]
    lib.oracle_append_mxfp8.restype = I
    lib.oracle_append_mxfp8.argtypes = [P, P, P, P, P, ctypes.c_int64, P, ctypes.c_int64, P,
                                        I, I, I, I, I, I]
    lib.oracle_decode_mxfp8.restype = I
    lib.oracle_decode_mxfp8.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_double, I, I, I, I,
                                        I, I, I, P, I, I]
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        override = os.environ.get("ORACLE_LIB")  # a rebuilt copy (sanitizer runs)
        if override:
            _lib = load_library(override)
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        _lib = load_library(_LIB_PATH)
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: Optional[np.ndarray],
           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
           head_dim_v: Optional[int] = None, pairs: Optional[Sequence] = None,
           threads: Optional[int] = None, lib=None) -> np.ndarray:
    """Attention output in float64, shape [num_seqs, Hq, dv].

    q [B, Hq, dk]; caches [num_blocks, bs, Hkv, d]; v_cache None = latent mode,
    where V is the first ``head_dim_v`` values of each K row.  With ``pairs``
    (an iterable of (b, h)) only those rows are computed; the rest stay NaN.
    """
    lib = _load(lib)
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    dtype = _dtype_code(q)
    assert _dtype_code(k_cache) == dtype
    if v_cache is not None:
        v_cache = np.ascontiguousarray(v_cache)
        assert _dtype_code(v_cache) == dtype
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, dk = q.shape
    nb, bs, Hkv, dk2 = k_cache.shape
    assert dk2 == dk
    if v_cache is not None:
        dv = v_cache.shape[3]
    else:
        dv = dk if head_dim_v is None else int(head_dim_v)
    out = np.full((B, Hq, dv), np.nan, dtype=np.float64)
    if pairs is not None:
        # each (b, h) once: rows are independent, duplicates would only repeat work
        pr = np.ascontiguousarray(
            np.unique(np.asarray(list(pairs), dtype=np.int32).reshape(-1, 2), axis=0))
        n_pairs = pr.shape[0]
    else:
        pr, n_pairs = None, 0
    n_threads = default_threads() if threads is None else int(threads)
    rc = lib.oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                           _ptr(cl), float(scale), B, Hq, Hkv, dk, dv, bs, bt.shape[1],
                           dtype, _ptr(pr), n_pairs, n_threads)
    if rc != 0:
        raise RuntimeError(f"oracle_decode failed with code {rc}")
    return out


def decode_workload(w, pairs=None, threads=None, context_lens=None, lib=None) -> np.ndarray:
    """Oracle decode over a ``workloads.Workload`` (optionally other lengths)."""
    cl = w.context_lens if context_lens is None else context_lens
    return decode(w.q, w.k_cache, w.v_cache, w.block_tables, cl, w.scale,
                  head_dim_v=w.spec.head_dim_v, pairs=pairs, threads=threads, lib=lib)


def append(k_cache: np.ndarray, v_cache: Optional[np.ndarray], k: np.ndarray,
           v: Optional[np.ndarray], slot_mapping: np.ndarray, lib=None) -> None:
    """In-place byte copy of each token's k (and v) row into its slot."""
    lib = _load(lib)
    assert k_cache.flags.c_contiguous and (v_cache is None or v_cache.flags.c_contiguous)
    nb, bs, Hkv, dk = k_cache.shape
    dv = 0 if v_cache is None else v_cache.shape[3]
    elt = k_cache.dtype.itemsize
    k2 = np.ascontiguousarray(k).reshape(k.shape[0], -1)
    v2 = None if v is None else np.ascontiguousarray(v).reshape(v.shape[0], -1)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    rc = lib.oracle_append(_ptr(k_cache), _ptr(v_cache), _ptr(k2), k2.shape[1], _ptr(v2),
                           0 if v2 is None else v2.shape[1], _ptr(sm), sm.shape[0], nb, bs,
                           Hkv, dk, dv, elt)
    if rc != 0:
        raise RuntimeError(f"oracle_append failed with code {rc}")


# ---------------------------------------------------------------------------
# MXFP8 KV cache (OCP Microscaling: E4M3 values, one E8M0 scale per 32).  The
# arithmetic is in pa_oracle.c; layouts there: K codes [nb, Hkv, bs, d], V
# codes [nb, Hkv, d, bs], scales [nb, Hkv, bs, d / 32].
# ---------------------------------------------------------------------------

def e4m3_values(codes: np.ndarray, lib=None) -> np.ndarray:
    """float64 value of every E4M3 byte in ``codes`` (NaN for S.1111.111)."""
    lib = _load(lib)
    lut = np.array([lib.oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)
    return lut[np.asarray(codes, dtype=np.uint8)]


def e8m0_values(scales: np.ndarray, lib=None) -> np.ndarray:
    """float64 value 2^(e - 127) of every E8M0 byte (NaN for 0xFF)."""
    lib = _load(lib)
    lut = np.array([lib.oracle_e8m0_value(c) for c in range(256)], dtype=np.float64)
    return lut[np.asarray(scales, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray, lib=None) -> np.ndarray:
    """Nearest E4M3 byte of each finite float64, ties to even, saturating at +-448."""
    lib = _load(lib)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def mx_quantize(x: np.ndarray, lib=None):
    """Rows of the last axis (length a multiple of 32) -> (E4M3 codes, E8M0 scales)."""
    lib = _load(lib)
    x = np.ascontiguousarray(x)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (d // 32,), dtype=np.uint8)
    rc = lib.oracle_mx_quantize(_ptr(x), _dtype_code(x), rows, d, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise RuntimeError(f"oracle_mx_quantize failed with code {rc}")
    return codes, scales


def append_mxfp8(k8: np.ndarray, v8: np.ndarray, ks: np.ndarray, vs: np.ndarray,
                 k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, lib=None) -> None:
    """In-place quantizing append of each token's k and v rows into its slot."""
    lib = _load(lib)
    for a in (k8, v8, ks, vs):
        assert a.flags.c_contiguous and a.dtype == np.uint8
    nb, Hkv, bs, d = k8.shape
    assert v8.shape == (nb, Hkv, d, bs) and ks.shape == vs.shape == (nb, Hkv, bs, d // 32)
    k2 = np.ascontiguousarray(k).reshape(k.shape[0], -1)
    v2 = np.ascontiguousarray(v).reshape(v.shape[0], -1)
    assert _dtype_code(k2) == _dtype_code(v2)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    rc = lib.oracle_append_mxfp8(_ptr(k8), _ptr(v8), _ptr(ks), _ptr(vs), _ptr(k2), k2.shape[1],
                                 _ptr(v2), v2.shape[1], _ptr(sm), sm.shape[0], nb, bs, Hkv, d,
                                 _dtype_code(k2))
    if rc != 0:
        raise RuntimeError(f"oracle_append_mxfp8 failed with code {rc}")


def decode_mxfp8(q: np.ndarray, k8: np.ndarray, v8: np.ndarray, ks: np.ndarray, vs: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 pairs: Optional[Sequence] = None, threads: Optional[int] = None,
                 lib=None) -> np.ndarray:
    """float64 attention output [B, Hq, d] over MXFP8 caches (values dequantized)."""
    lib = _load(lib)
    q = np.ascontiguousarray(q)
    B, Hq, d = q.shape
    nb, Hkv, bs, d2 = k8.shape
    assert d2 == d and v8.shape == (nb, Hkv, d, bs) and ks.shape == vs.shape == (nb, Hkv, bs, d // 32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    if pairs is not None:
        pr = np.ascontiguousarray(
            np.unique(np.asarray(list(pairs), dtype=np.int32).reshape(-1, 2), axis=0))
        n_pairs = pr.shape[0]
    else:
        pr, n_pairs = None, 0
    n_threads = default_threads() if threads is None else int(threads)
    rc = lib.oracle_decode_mxfp8(_ptr(out), _ptr(q), _ptr(np.ascontiguousarray(k8)),
                                 _ptr(np.ascontiguousarray(v8)), _ptr(np.ascontiguousarray(ks)),
                                 _ptr(np.ascontiguousarray(vs)), _ptr(bt), _ptr(cl), float(scale),
                                 B, Hq, Hkv, d, bs, bt.shape[1], _dtype_code(q), _ptr(pr),
                                 n_pairs, n_threads)
    if rc != 0:
        raise RuntimeError(f"oracle_decode_mxfp8 failed with code {rc}")
    return out


# ---------------------------------------------------------------------------
# Several new query tokens per sequence, causal among themselves
# ---------------------------------------------------------------------------

def visible_lengths(context_lens: np.ndarray, q_len: int) -> np.ndarray:
    """[B, q_len] number of cached tokens query i of sequence b may attend:
    the last q_len of the L_b cached tokens are the queries themselves, and
    query i sits at position L_b - q_len + i, seeing tokens 0 .. that
    position (the causal mask of "Étape 2: Attention avec KV Cache").  A
    query whose position would be negative sees nothing."""
    L = np.asarray(context_lens, dtype=np.int64)[:, None]
    return np.clip(L - q_len + 1 + np.arange(q_len)[None, :], 0, None).astype(np.int32)


def decode_multi(q: np.ndarray, k_cache, v_cache, block_tables, context_lens, scale,
                 mxfp8: Optional[tuple] = None, pairs: Optional[Sequence] = None,
                 threads: Optional[int] = None) -> np.ndarray:
    """float64 [B, q_len, Hq, d]: each query row through the single-query
    oracle over its visible prefix.  q [B, q_len, Hq, d].  With ``mxfp8`` =
    (k_scale, v_scale) the caches are MXFP8 codes (decode_mxfp8's layouts).
    ``pairs`` optionally lists (b, i) query rows to compute (others NaN)."""
    B, Q = q.shape[0], q.shape[1]
    vis = visible_lengths(context_lens, Q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    todo = [(b, i) for b in range(B) for i in range(Q)] if pairs is None else list(pairs)
    out = np.full(q.shape[:3] + ((v_cache.shape[2] if mxfp8 else v_cache.shape[3]),),
                  np.nan, dtype=np.float64)
    for b, i in todo:
        q1 = np.ascontiguousarray(q[b, i][None])
        cl = vis[b, i:i + 1]
        if mxfp8 is None:
            out[b, i] = decode(q1, k_cache, v_cache, bt[b:b + 1], cl, scale, threads=threads)[0]
        else:
            out[b, i] = decode_mxfp8(q1, k_cache, v_cache, mxfp8[0], mxfp8[1], bt[b:b + 1], cl,
                                     scale, threads=threads)[0]
    return out


# ---------------------------------------------------------------------------
# Sliding window, log-sum-exp, per-token attention mass (numpy, float64)
# ---------------------------------------------------------------------------

def _widen64(a: np.ndarray) -> np.ndarray:
    """float32 or bf16 bit patterns (uint16) widened exactly to float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def window_start(L: int, window: int) -> int:
    """First token a query of a length-L sequence attends with a sliding
    window of ``window`` tokens (0: no window)."""
    return L - window if (window > 0 and L > window) else 0


def _gather(pool, bt_row, start, L, bs):
    t = np.arange(start, L)
    return _widen64(pool[bt_row[t // bs], t % bs])  # [n, Hkv, d]


def decode_window(q, k_cache, v_cache, block_tables, context_lens, scale, window=0):
    """Plain softmax attention of each query over its sequence's tokens
    [max(0, L - window), L) in float64.  Returns (O [B, Hq, dv], lse [B, Hq])
    with lse = log(sum_t exp(s_t)), s_t = scale * q . k_t; a sequence with
    no token gives O = 0 and lse = -inf."""
    B, Hq, _ = q.shape
    bs, Hkv = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    dv = v_cache.shape[3]
    O = np.zeros((B, Hq, dv))
    lse = np.full((B, Hq), -np.inf)
    qq = _widen64(q)
    for b in range(B):
        L = int(context_lens[b])
        st = window_start(L, window)
        if L <= st:
            continue
        K = _gather(k_cache, block_tables[b], st, L, bs)
        V = _gather(v_cache, block_tables[b], st, L, bs)
        for h in range(Hq):
            g = h // G
            s = scale * (K[:, g] @ qq[b, h])
            m = s.max()
            w = np.exp(s - m)
            O[b, h] = (w @ V[:, g]) / w.sum()
            lse[b, h] = m + np.log(w.sum())
    return O, lse


def attention_scores(q, k_cache, block_tables, context_lens, lse, scale, window=0,
                     max_context=None):
    """[B, Hkv, max_context] float64: for each token t of the window, the sum
    over the query heads h of KV head g of exp(scale q_h . k_t - lse[b, h]);
    0 elsewhere."""
    B, Hq, _ = q.shape
    bs, Hkv = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    if max_context is None:
        max_context = int(np.max(context_lens)) if B else 0
    out = np.zeros((B, Hkv, max_context))
    qq = _widen64(q)
    for b in range(B):
        L = int(context_lens[b])
        st = window_start(L, window)
        if L <= st:
            continue
        K = _gather(k_cache, block_tables[b], st, L, bs)
        for g in range(Hkv):
            for h in range(g * G, (g + 1) * G):
                out[b, g, st:L] += np.exp(scale * (K[:, g] @ qq[b, h]) - lse[b, h])
    return out
