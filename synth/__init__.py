"""Seeded synthetic inputs for look-ahead token scoring (shared by the CPU
oracle's tests and the GPU path's tests and benchmark).

Holds no scoring or selection arithmetic: only random draws (``synth.c``) and
their layout. The workloads mirror the pages' setting: a speculator's
look-ahead queries Q[L,H,N,d] and its keys K[L,Hkv,M+N,d] (RoPE already
applied), where a few prompt positions (attention sinks 0-3 and some random
chunks) carry a per-(layer, kv-head) direction that every query also carries,
so those positions draw attention. Values follow N(0,1) noise plus 2*u.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

F32, BF16 = 0, 1
PLANT_SCALE = 2.0


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", _SRC, "-o", tmp,
             "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_direction.argtypes = [u64, i64, i64, i64, i32, vp]
        lib.synth_fill_q.argtypes = [u64, i64, i32, i32, i32, i32, i32, i32, dbl, vp]
        lib.synth_fill_k.argtypes = [u64, i64, i32, i32, i64, i32, i32, dbl, vp, vp, i64, i64]
        lib.synth_uniform_u64.argtypes = [u64, i64, i64, i64, vp]
        lib.synth_choose.argtypes = [u64, i64, i64, i64, vp, vp]
        for f in (lib.synth_direction, lib.synth_fill_q, lib.synth_fill_k, lib.synth_uniform_u64,
                  lib.synth_choose):
            f.restype = None
        _lib = lib
    return _lib


# --------------------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Select:
    """Selection parameters (chunk size, pool width, top-K rate or mass, boosts)."""
    chunk: int
    pool_k: int
    mode: str  # "topk" | "mass"
    keep_rate: float = 0.0
    mass: float = 0.0
    boost_first_n: int = 0
    boost_first_mult: float = 1.0
    boost_last_n: int = 0
    boost_last_mult: float = 1.0
    norm: str = "minmax"  # "minmax" | "percentile" | "zscore"
    norm_lo: float = 0.0
    norm_hi: float = 0.0


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    H: int
    Hkv: int
    d: int
    N: int
    dtype: int
    seed: int
    M: int = 0  # uniform prompt length (R = 1)
    R: int = 1
    len_range: tuple = ()  # ragged: (lo, hi, multiple)
    plant_chunks: int = 0  # fixed count of planted chunks, or
    plant_frac: float = 0.0  # fraction of chunks planted (max(1, round(frac*nc)))
    plant_frac_range: tuple = ()  # ragged: per-request fraction uniform in [lo, hi]
    plant_chunk: int = 32
    selects: tuple = field(default_factory=tuple)

    @property
    def G(self):
        return self.H // self.Hkv


_BOOSTS = dict(boost_first_n=64, boost_first_mult=1.5, boost_last_n=128, boost_last_mult=1.3)

WORKLOADS = {
    # tiny plumbing case, fp32 inputs
    "tiny": Workload("tiny", L=2, H=4, Hkv=2, d=64, N=8, dtype=F32, seed=0, M=1024,
                     plant_chunks=3, plant_chunk=32,
                     selects=(Select(32, 3, "topk", keep_rate=0.3),)),
    # 0.8B-speculator shape
    "spec0.8b_m4608": Workload("spec0.8b_m4608", L=24, H=16, Hkv=8, d=64, N=8, dtype=BF16,
                               seed=1, M=4608, plant_frac=0.05, plant_chunk=32,
                               selects=(Select(32, 5, "mass", mass=0.85, **_BOOSTS),)),
    # 8B-speculator shape, 32K prompt
    "spec8b_m32k": Workload("spec8b_m32k", L=32, H=32, Hkv=8, d=128, N=8, dtype=BF16, seed=2,
                            M=32768, plant_frac=0.02, plant_chunk=32,
                            selects=(Select(32, 13, "topk", keep_rate=0.10),)),
    # 8B-speculator shape, 128K prompt
    "spec8b_m128k": Workload("spec8b_m128k", L=32, H=32, Hkv=8, d=128, N=8, dtype=BF16, seed=3,
                             M=131072, plant_frac=0.005, plant_chunk=64,
                             selects=(Select(64, 13, "topk", keep_rate=0.1),
                                      Select(64, 13, "topk", keep_rate=0.3),
                                      Select(64, 13, "topk", keep_rate=0.5),
                                      Select(64, 13, "mass", mass=0.85))),
    # ragged batch of 16 requests, 4K..64K prompts
    "ragged16_8b": Workload("ragged16_8b", L=32, H=32, Hkv=8, d=128, N=8, dtype=BF16, seed=4,
                            R=16, len_range=(4096, 65536, 64), plant_frac_range=(0.01, 0.10),
                            plant_chunk=32,
                            selects=(Select(32, 13, "mass", mass=0.85, **_BOOSTS),)),
}


def uniform_u64(seed: int, r: int, which: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_uniform_u64(seed, r, which, n, out.ctypes.data)
    return out


def prompt_lengths(w: Workload) -> np.ndarray:
    """Per-request prompt lengths M_r."""
    if w.R == 1 and not w.len_range:
        return np.array([w.M], np.int64)
    lo, hi, mult = w.len_range
    h = uniform_u64(w.seed, 0, 1, w.R)
    span = hi - lo + 1
    m = lo + (h % np.uint64(span)).astype(np.int64)  # uniform integer in [lo, hi]
    return (m // mult) * mult


def planted_fraction(w: Workload, r: int) -> float:
    if w.plant_frac_range:
        lo, hi = w.plant_frac_range
        h = int(uniform_u64(w.seed, r, 2, 1)[0])
        return lo + (hi - lo) * ((h >> 11) * 2.0**-53)
    return w.plant_frac


def planted_mask(w: Workload, r: int, M: int) -> np.ndarray:
    """uint8 mask over the M+N key rows: sinks 0-3 and every token of the chosen
    chunks (look-ahead keys M..M+N-1 are never planted)."""
    nc = -(-M // w.plant_chunk)
    if w.plant_chunks:
        k = w.plant_chunks
    else:
        k = max(1, int(round(planted_fraction(w, r) * nc)))
    k = min(k, nc)
    scratch = np.empty(nc, np.int64)
    chosen = np.empty(max(k, 1), np.int64)
    _load().synth_choose(w.seed, r, nc, k, scratch.ctypes.data, chosen.ctypes.data)
    mask = np.zeros(M + w.N, np.uint8)
    mask[: min(4, M)] = 1
    for c in chosen[:k]:
        mask[c * w.plant_chunk: min((c + 1) * w.plant_chunk, M)] = 1
    return mask


def _np_dtype(dtype):
    return np.float32 if dtype == F32 else np.uint16


def make_q(w: Workload, r: int = 0) -> np.ndarray:
    """Q of request r: [L][H][N][d] (float32, or bf16 bit patterns as uint16)."""
    out = np.empty((w.L, w.H, w.N, w.d), _np_dtype(w.dtype))
    _load().synth_fill_q(w.seed, r, w.L, w.H, w.Hkv, w.N, w.d, w.dtype, PLANT_SCALE,
                         out.ctypes.data)
    return out


def make_k(w: Workload, r: int = 0, M: int | None = None) -> np.ndarray:
    """K of request r: [L][Hkv][M+N][d]."""
    if M is None:
        M = int(prompt_lengths(w)[r])
    mask = planted_mask(w, r, M)
    out = np.empty((w.L, w.Hkv, M + w.N, w.d), _np_dtype(w.dtype))
    _load().synth_fill_k(w.seed, r, w.L, w.Hkv, M + w.N, w.d, w.dtype, PLANT_SCALE,
                         mask.ctypes.data, out.ctypes.data, (M + w.N) * w.d, 0)
    return out


def make_request(w: Workload, r: int = 0):
    """(Q, K, M) of one request."""
    M = int(prompt_lengths(w)[r])
    return make_q(w, r), make_k(w, r, M), M


def make_ragged(w: Workload, lens=None):
    """Packed ragged batch: Q [R][L][H][N][d], K [L][Hkv][T][d] with request r's
    M_r + N key rows at cu_keys[r] (look-ahead keys at the tail of each
    segment), cu_prompt [R+1] offsets of the prompts. lens, if given, are the
    prompt lengths (else those of the workload)."""
    Ms = prompt_lengths(w) if lens is None else np.asarray(lens, np.int64)
    R = len(Ms)
    cu_prompt = np.zeros(R + 1, np.int64)
    cu_prompt[1:] = np.cumsum(Ms)
    cu_keys = np.zeros(R + 1, np.int64)
    cu_keys[1:] = np.cumsum(Ms + w.N)
    T = int(cu_keys[-1])
    Q = np.empty((R, w.L, w.H, w.N, w.d), _np_dtype(w.dtype))
    K = np.empty((w.L, w.Hkv, T, w.d), _np_dtype(w.dtype))
    lib = _load()
    for r in range(R):
        lib.synth_fill_q(w.seed, r, w.L, w.H, w.Hkv, w.N, w.d, w.dtype, PLANT_SCALE,
                         Q[r].ctypes.data)
        mask = planted_mask(w, r, int(Ms[r]))
        lib.synth_fill_k(w.seed, r, w.L, w.Hkv, int(Ms[r]) + w.N, w.d, w.dtype, PLANT_SCALE,
                         mask.ctypes.data, K.ctypes.data, T * w.d, int(cu_keys[r]))
    return Q, K, cu_prompt


def direction(seed: int, r: int, l: int, g: int, d: int) -> np.ndarray:
    u = np.empty(d, np.float64)
    _load().synth_direction(seed, r, l, g, d, u.ctypes.data)
    return u


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)
