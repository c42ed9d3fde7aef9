"""CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU
baseline leg use this package; the GPU library never imports or links it, and
the two share no code. ``oracle.c`` holds the arithmetic (fp64 scoring and
the pinned selection steps); this module only builds it and marshals numpy
arrays.

Sources (cited by page title and section): "Speculative Prefill: Turbocharging
TTFT with Lightweight and Training-Free Token Importance Estimation" (paper
review page: Core algorithm, Core formulas) and "SpecPrefill - Implementation
Guide" (How It Works, v3 Improvements, v3.1 Optimizations, Configuration
Reference).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
TOPK, MASS = 0, 1
NORMS = {"minmax": 0, "percentile": 1, "zscore": 2}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, strict IEEE: no FMA
    contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i32, dbl, vp, lng, flt = (ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_long,
                                  ctypes.c_float)
        lib.oracle_softmax_row.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl, i32,
                                           i32, i32, vp]
        lib.oracle_score.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl, i32, vp]
        lib.oracle_score_lastrow.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl,
                                             i32, vp]
        lib.oracle_select.argtypes = [vp, i32, i32, i32, i32, flt, flt, i32, flt, i32, flt, i32,
                                      flt, flt, lng, lng, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_select_threshold.argtypes = [vp, i32, i32, flt, i32, i32, lng, lng, vp, vp, vp]
        for f in (lib.oracle_softmax_row, lib.oracle_score, lib.oracle_score_lastrow,
                  lib.oracle_select, lib.oracle_select_threshold):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("Q/K must be float32 or bf16 bit patterns (uint16)")


def _dims(Q: np.ndarray, K: np.ndarray):
    L, H, N, d = Q.shape
    L2, Hkv, MN, d2 = K.shape
    if L2 != L or d2 != d or MN <= N:
        raise ValueError("shape mismatch: Q [L,H,N,d], K [L,Hkv,M+N,d]")
    return L, H, Hkv, d, N, MN - N


def softmax_row(Q, K, l, h, j, scale=0.0) -> np.ndarray:
    """Probabilities of look-ahead row (l, h, j) over its M+j+1 visible keys."""
    Q = np.ascontiguousarray(Q)
    K = np.ascontiguousarray(K)
    dt = _dtype_of(Q)
    L, H, Hkv, d, N, M = _dims(Q, K)
    p = np.empty(M + j + 1, np.float64)
    rc = _load().oracle_softmax_row(Q.ctypes.data, K.ctypes.data, dt, L, H, Hkv, d, N, M,
                                    float(scale), l, h, j, p.ctypes.data)
    if rc:
        raise ValueError(f"oracle_softmax_row failed ({rc})")
    return p


def score(Q, K, scale=0.0, nthreads=0) -> np.ndarray:
    """importance[M] (float64) of one request: Q [L,H,N,d], K [L,Hkv,M+N,d]."""
    Q = np.ascontiguousarray(Q)
    K = np.ascontiguousarray(K)
    if _dtype_of(Q) != _dtype_of(K):
        raise TypeError("Q and K dtypes differ")
    L, H, Hkv, d, N, M = _dims(Q, K)
    out = np.empty(M, np.float64)
    rc = _load().oracle_score(Q.ctypes.data, K.ctypes.data, _dtype_of(Q), L, H, Hkv, d, N, M,
                              float(scale), int(nthreads), out.ctypes.data)
    if rc:
        raise ValueError(f"oracle_score failed ({rc})")
    return out


def score_lastrow(Q, Q_last, K, scale=0.0, nthreads=0) -> np.ndarray:
    """importance[M] (float64) with the last prompt token's query row Q_last
    [L,H,d] as one more step (see oracle_score_lastrow)."""
    Q = np.ascontiguousarray(Q)
    Q_last = np.ascontiguousarray(Q_last)
    K = np.ascontiguousarray(K)
    if not (_dtype_of(Q) == _dtype_of(K) == _dtype_of(Q_last)):
        raise TypeError("Q, Q_last and K dtypes differ")
    L, H, Hkv, d, N, M = _dims(Q, K)
    if Q_last.shape != (L, H, d):
        raise ValueError("Q_last must be [L, H, d]")
    out = np.empty(M, np.float64)
    rc = _load().oracle_score_lastrow(Q.ctypes.data, Q_last.ctypes.data, K.ctypes.data,
                                      _dtype_of(Q), L, H, Hkv, d, N, M, float(scale),
                                      int(nthreads), out.ctypes.data)
    if rc:
        raise ValueError(f"oracle_score_lastrow failed ({rc})")
    return out


def select(importance, chunk, pool_k, mode, keep_rate=0.0, mass=0.0, boost_first_n=0,
           boost_first_mult=1.0, boost_last_n=0, boost_last_mult=1.0, norm="minmax",
           norm_lo=0.0, norm_hi=0.0, pos_base=0, base_index=0, debug=False):
    """Selection of one prompt from a float32 importance array. norm:
    "minmax", "percentile" (norm_lo, norm_hi: the two quantiles) or "zscore"
    (norm_hi: the clip c in standard deviations).

    Returns (kept_idx int32, pos_ids int32) or, with debug, also a dict of the
    intermediate arrays (v, q, C, key, kept_chunk)."""
    x = np.ascontiguousarray(importance, dtype=np.float32)
    M = x.shape[0]
    mode_i = {"topk": TOPK, "mass": MASS}.get(mode, mode)
    nc = -(-M // chunk) if chunk > 0 else 1
    kept = np.empty(max(M, 1), np.int32)
    pos = np.empty(max(M, 1), np.int32)
    n = np.zeros(1, np.int32)
    v = np.empty(M, np.float32)
    q = np.empty(M, np.uint64)
    C = np.empty(max(nc, 1), np.uint64)
    key = np.empty(max(nc, 1), np.float64)
    kc = np.empty(max(nc, 1), np.uint8)
    rc = _load().oracle_select(x.ctypes.data, M, chunk, pool_k, mode_i, keep_rate, mass,
                               boost_first_n, boost_first_mult, boost_last_n, boost_last_mult,
                               NORMS.get(norm, norm), norm_lo, norm_hi,
                               pos_base, base_index, kept.ctypes.data, pos.ctypes.data,
                               n.ctypes.data, v.ctypes.data, q.ctypes.data, C.ctypes.data,
                               key.ctypes.data, kc.ctypes.data)
    if rc:
        raise ValueError(f"oracle_select rejected its arguments ({rc})")
    k = int(n[0])
    if debug:
        return kept[:k].copy(), pos[:k].copy(), dict(v=v, q=q, C=C[:nc], key=key[:nc],
                                                    kept_chunk=kc[:nc].astype(bool))
    return kept[:k].copy(), pos[:k].copy()


def select_threshold(importance, chunk, keep_rate, min_tok=128, max_keep=0, pos_base=0,
                     base_index=0):
    """Threshold selection of one prompt as the Implementation Guide's program
    performs it (see oracle_select_threshold): (kept_idx int32, pos_ids int32)."""
    x = np.ascontiguousarray(importance, dtype=np.float32)
    M = x.shape[0]
    kept = np.empty(max(M, 1), np.int32)
    pos = np.empty(max(M, 1), np.int32)
    n = np.zeros(1, np.int32)
    rc = _load().oracle_select_threshold(x.ctypes.data, M, int(chunk), float(keep_rate),
                                         int(min_tok), int(max_keep), int(pos_base),
                                         int(base_index), kept.ctypes.data, pos.ctypes.data,
                                         n.ctypes.data)
    if rc:
        raise ValueError(f"oracle_select_threshold rejected its arguments ({rc})")
    k = int(n[0])
    return kept[:k].copy(), pos[:k].copy()


def window_layout(M, window, stride):
    """Sliding windows over M tokens ("SpecPrefill - Implementation Guide",
    Sliding Window: Sliding Window Solution, and Implementation Details:
    Sliding Window Loop (v3.1)): a window starts every stride tokens and spans
    up to window tokens; one that reaches the end of the prompt is the last
    and keeps all its tokens' scores, the others their first stride.
    Returns [(start, length, kept), ...]."""
    if M < 1 or window < 1 or stride < 1 or stride > window:
        raise ValueError("need M, window, stride >= 1 and stride <= window")
    out, pos = [], 0
    while True:
        end = min(pos + window, M)
        if end >= M:
            out.append((pos, end - pos, end - pos))
            return out
        out.append((pos, end - pos, stride))
        pos += stride


def score_windows(Qs, Ks, keeps, scale=0.0, nthreads=0):
    """Importance of a prompt scored window by window: window r's own scores
    (its queries Qs[r] over its keys Ks[r]), of which the first keeps[r] are
    kept, concatenated in window order (each token scored by one window)."""
    parts = [score(Q, K, scale=scale, nthreads=nthreads)[:k] for Q, K, k in zip(Qs, Ks, keeps)]
    return np.concatenate(parts)


def select_params(sel) -> dict:
    """Keyword arguments of select() from a synth.Select."""
    return dict(chunk=sel.chunk, pool_k=sel.pool_k, mode=sel.mode, keep_rate=sel.keep_rate,
                mass=sel.mass, boost_first_n=sel.boost_first_n,
                boost_first_mult=sel.boost_first_mult, boost_last_n=sel.boost_last_n,
                boost_last_mult=sel.boost_last_mult, norm=sel.norm, norm_lo=sel.norm_lo,
                norm_hi=sel.norm_hi)
