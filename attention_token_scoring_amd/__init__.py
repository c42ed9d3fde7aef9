"""Python binding of libspecprefill (SpecPrefill's token-importance estimator on
an AMD Instinct MI355X).

Argument marshalling only: every step of scoring and selection runs in the HIP
kernels of ``libspecprefill.so`` (built in-tree by ``build.py``); torch supplies
device memory and the current stream. There is no CPU fallback: if the
library is missing, or a call fails, an exception says so.

The call names follow the C ABI in ``include/specprefill.h``:
``sp_score``, ``sp_score_varlen``, ``sp_score_windows``, ``sp_window_layout``,
``sp_select``, ``sp_select_varlen``,
``sp_score_workspace_bytes``, ``sp_score_batch_workspace_bytes``, ``sp_select_workspace_bytes``,
``sp_score_plan`` and ``sp_status_string``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecprefill.so")

SP_OK, SP_EINVAL, SP_EUNSUPPORTED, SP_EWORKSPACE, SP_EDEVICE = range(5)
SP_F32, SP_BF16 = 0, 1
SP_SELECT_TOPK, SP_SELECT_MASS, SP_SELECT_THRESHOLD = 0, 1, 2
SP_LAUNCH_RESIDENT, SP_LAUNCH_COOPERATIVE = 0, 1
SP_NORM_MINMAX, SP_NORM_PERCENTILE, SP_NORM_ZSCORE = 0, 1, 2

EXPORTED = ("sp_score", "sp_score_varlen", "sp_select", "sp_select_varlen",
            "sp_score_workspace_bytes", "sp_score_batch_workspace_bytes", "sp_score_batch_plan", "sp_select_workspace_bytes", "sp_score_plan",
            "sp_status_string", "sp_profile_score_kernel", "sp_score_status",
            "sp_score_windows", "sp_window_layout", "sp_gather_rows", "sp_break_even",
            "sp_read_probe", "sp_set_wait_limit", "sp_score_lastrow", "sp_score_noalloc",
            "sp_score_select")


class SpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sp_status_string(status)}")


class ScoreDesc(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("N", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("launch", ctypes.c_int)]


class SelectParams(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("pool_k", ctypes.c_int32), ("mode", ctypes.c_int),
                ("keep_rate", ctypes.c_float), ("mass", ctypes.c_float),
                ("boost_first_n", ctypes.c_int32), ("boost_first_mult", ctypes.c_float),
                ("boost_last_n", ctypes.c_int32), ("boost_last_mult", ctypes.c_float),
                ("min_tok", ctypes.c_int32), ("max_keep", ctypes.c_int32),
                ("norm", ctypes.c_int), ("norm_lo", ctypes.c_float), ("norm_hi", ctypes.c_float)]


_lib = None


def load_library():
    """Loads libspecprefill.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run attention_token_scoring_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    lib.sp_status_string.argtypes = [ctypes.c_int]
    lib.sp_status_string.restype = ctypes.c_char_p
    lib.sp_score_workspace_bytes.argtypes = [P(ScoreDesc), i64]
    lib.sp_score_workspace_bytes.restype = sz
    lib.sp_score_batch_workspace_bytes.argtypes = [P(ScoreDesc), i32, P(ctypes.c_int64)]
    lib.sp_score_batch_workspace_bytes.restype = sz
    lib.sp_score_batch_plan.argtypes = [P(ScoreDesc), i32, P(ctypes.c_int64), sz,
                                        P(ctypes.c_int32), P(ctypes.c_int32)]
    lib.sp_score_plan.argtypes = [P(ScoreDesc), i32, P(ctypes.c_int32)]
    lib.sp_score.argtypes = [P(ScoreDesc), vp, vp, i32, vp, vp, sz, vp]
    lib.sp_score_varlen.argtypes = [P(ScoreDesc), i32, vp, vp, P(ctypes.c_int64), vp, vp, sz, vp]
    lib.sp_select_workspace_bytes.argtypes = [i32, i64, P(SelectParams)]
    lib.sp_select_workspace_bytes.restype = sz
    lib.sp_select.argtypes = [vp, i32, P(SelectParams), i32, vp, vp, vp, vp, sz, vp]
    lib.sp_select_varlen.argtypes = [vp, i32, P(ctypes.c_int64), P(ctypes.c_int32),
                                     P(SelectParams), vp, vp, vp, vp, sz, vp]
    lib.sp_profile_score_kernel.argtypes = [vp, vp]
    lib.sp_score_status.argtypes = [vp, vp, P(ctypes.c_int32)]
    lib.sp_score_windows.argtypes = [P(ScoreDesc), i32, vp, vp, P(ctypes.c_int64),
                                     P(ctypes.c_int64), vp, vp, sz, vp]
    lib.sp_window_layout.argtypes = [i64, i32, i32, P(ctypes.c_int32), P(ctypes.c_int64),
                                     P(ctypes.c_int64), P(ctypes.c_int64), i32]
    lib.sp_gather_rows.argtypes = [vp, i64, vp, vp, i32, P(ctypes.c_int64), vp, vp]
    f32 = ctypes.c_float
    lib.sp_break_even.argtypes = [i64, f32, f32, f32, f32, P(ctypes.c_int32)]
    lib.sp_read_probe.argtypes = [vp, sz, i32, i32, vp, vp]
    lib.sp_set_wait_limit.argtypes = [ctypes.c_uint64]
    lib.sp_score_lastrow.argtypes = [P(ScoreDesc), vp, vp, vp, i32, vp, vp, sz, vp]
    lib.sp_score_noalloc.argtypes = [P(ScoreDesc), vp, vp, i32, vp, vp]
    lib.sp_score_select.argtypes = [P(ScoreDesc), vp, vp, i32, P(SelectParams), i32, vp, vp, vp, vp,
                                    vp, sz, vp]
    for name in ("sp_score_plan", "sp_score", "sp_score_varlen", "sp_select", "sp_select_varlen",
                 "sp_profile_score_kernel", "sp_score_status", "sp_score_windows",
                 "sp_window_layout", "sp_gather_rows", "sp_break_even", "sp_read_probe", "sp_set_wait_limit",
                 "sp_score_lastrow", "sp_score_noalloc", "sp_score_select"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def sp_status_string(status: int) -> str:
    return load_library().sp_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != SP_OK:
        raise SpError(status, where)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SP_BF16
    if t.dtype == torch.float32:
        return SP_F32
    raise TypeError(f"unsupported dtype {t.dtype}: Q and K must be bfloat16 or float32")


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_out(t, dtype, min_numel: int, name: str):
    """A caller-supplied output (or input) tensor the kernels index up to
    min_numel elements: it must be a contiguous CUDA tensor of `dtype` with at
    least that many elements (a smaller one would be written out of bounds)."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def score_desc(L, H, Hkv, d, N, dtype=SP_BF16, scale=0.0, launch=SP_LAUNCH_RESIDENT) -> ScoreDesc:
    return ScoreDesc(int(L), int(H), int(Hkv), int(d), int(N), int(dtype), float(scale), int(launch))


def select_params(chunk=32, pool_k=1, mode="topk", keep_rate=0.0, mass=0.0, boost_first_n=0,
                  boost_first_mult=1.0, boost_last_n=0, boost_last_mult=1.0, min_tok=0,
                  max_keep=0, norm="minmax", norm_lo=0.0, norm_hi=0.0) -> SelectParams:
    m = {"topk": SP_SELECT_TOPK, "mass": SP_SELECT_MASS,
         "threshold": SP_SELECT_THRESHOLD}.get(mode, mode)
    nm = {"minmax": SP_NORM_MINMAX, "percentile": SP_NORM_PERCENTILE,
          "zscore": SP_NORM_ZSCORE}.get(norm, norm)
    return SelectParams(int(chunk), int(pool_k), int(m), float(keep_rate), float(mass),
                        int(boost_first_n), float(boost_first_mult), int(boost_last_n),
                        float(boost_last_mult), int(min_tok), int(max_keep), int(nm),
                        float(norm_lo), float(norm_hi))


def sp_score_workspace_bytes(desc: ScoreDesc, max_prompt_len: int) -> int:
    return int(load_library().sp_score_workspace_bytes(ctypes.byref(desc), int(max_prompt_len)))


def sp_score_batch_workspace_bytes(desc: ScoreDesc, cu_prompt: Sequence[int]) -> int:
    """Workspace with which sp_score_varlen / sp_score_windows pack requests
    into shared launches wherever the planner finds it faster."""
    cu = np.ascontiguousarray(np.asarray(cu_prompt, dtype=np.int64))
    return int(load_library().sp_score_batch_workspace_bytes(
        ctypes.byref(desc), int(cu.shape[0] - 1), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))


def sp_score_batch_plan(desc: ScoreDesc, cu_prompt: Sequence[int], ws_bytes: int) -> np.ndarray:
    """Each request's launch index under sp_score_varlen with a workspace of
    ws_bytes (requests with one index share a launch)."""
    cu = np.ascontiguousarray(np.asarray(cu_prompt, dtype=np.int64))
    R = int(cu.shape[0] - 1)
    out = np.zeros(max(R, 1), np.int32)
    n = ctypes.c_int32(0)
    _check(load_library().sp_score_batch_plan(
        ctypes.byref(desc), R, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(ws_bytes),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(n)), "sp_score_batch_plan")
    return out[:R]


def _batch_workspace(desc: ScoreDesc, cu, maxM: int, device, workspace):
    """A given workspace must hold one request (smaller than the batch's packing
    bound, the batch is scored in turn); else one of the packing bound."""
    if workspace is None:
        nbytes = max(sp_score_batch_workspace_bytes(desc, cu), sp_score_workspace_bytes(desc, maxM))
        return _workspace(nbytes, device)
    return _workspace(sp_score_workspace_bytes(desc, maxM), device, workspace)


def sp_select_workspace_bytes(R: int, total_prompt_len: int, params: SelectParams) -> int:
    return int(load_library().sp_select_workspace_bytes(int(R), int(total_prompt_len),
                                                        ctypes.byref(params)))


def sp_score_plan(desc: ScoreDesc, M: int) -> dict:
    info = (ctypes.c_int32 * 9)()
    _check(load_library().sp_score_plan(ctypes.byref(desc), int(M), info), "sp_score_plan")
    keys = ("grid", "g", "ngroups", "keys_per_wg", "rows", "units", "cus", "defer", "dma")
    return {k: int(info[i]) for i, k in enumerate(keys)}


def sp_profile_score_kernel(before=None, after=None):
    """Profiling aid: record torch.cuda.Event `before`/`after` (already
    recorded once, so that they exist) around each cooperative scoring kernel
    launched by this thread; call with no arguments to stop."""
    b = ctypes.c_void_p(before.cuda_event) if before is not None else None
    a = ctypes.c_void_p(after.cuda_event) if after is not None else None
    _check(load_library().sp_profile_score_kernel(b, a), "sp_profile_score_kernel")


def sp_score_status(workspace, stream=None) -> bool:
    """True if the last scoring call on this workspace timed out in a
    cross-workgroup wait (its importance is then not valid). Waits for the
    stream."""
    _require_cuda(workspace)
    out = ctypes.c_int32(0)
    _check(load_library().sp_score_status(workspace.data_ptr(), _stream(stream),
                                          ctypes.byref(out)), "sp_score_status")
    return bool(out.value)


def sp_set_wait_limit(ticks: int = 0):
    """Testing aid: limit of the bounded waits (the scoring kernel's, and the
    selection's by several workgroups) for this thread's later calls, in
    100 MHz clock ticks (0: the default, 2 s)."""
    _check(load_library().sp_set_wait_limit(int(ticks)), "sp_set_wait_limit")


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise SpError(SP_EWORKSPACE, "workspace")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def sp_score(Q, K, M: Optional[int] = None, scale: float = 0.0, out=None, workspace=None,
             stream=None, launch: int = SP_LAUNCH_RESIDENT):
    """importance [M] float32 of one prompt. Q [L,H,N,d], K [L,Hkv,M+N,d] (bf16 or f32).
    launch: SP_LAUNCH_RESIDENT (ordinary launch) or SP_LAUNCH_COOPERATIVE."""
    torch = _torch()
    _require_cuda(Q, K)
    L, H, N, d = Q.shape
    Hkv = K.shape[1]
    if M is None:
        M = K.shape[2] - N
    desc = score_desc(L, H, Hkv, d, N, _dtype_code(Q), scale, launch)
    if _dtype_code(K) != desc.dtype or K.shape[0] != L or K.shape[3] != d or K.shape[2] != M + N:
        raise ValueError("K must be [L, Hkv, M+N, d] with Q's dtype")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=Q.device)
    _check_out(out, torch.float32, M, "out")
    ws = _workspace(sp_score_workspace_bytes(desc, M), Q.device, workspace)
    st = load_library().sp_score(ctypes.byref(desc), Q.data_ptr(), K.data_ptr(), int(M),
                                 out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check(st, "sp_score")
    return out


def sp_score_lastrow(Q, Q_last, K, M: Optional[int] = None, scale: float = 0.0, out=None,
                     workspace=None, stream=None, launch: int = SP_LAUNCH_RESIDENT):
    """importance [M] float32 with the last prompt token's query row as one
    more step: Q [L,H,N,d], Q_last [L,H,d], K [L,Hkv,M+N,d]."""
    torch = _torch()
    _require_cuda(Q, Q_last, K)
    L, H, N, d = Q.shape
    Hkv = K.shape[1]
    if M is None:
        M = K.shape[2] - N
    desc = score_desc(L, H, Hkv, d, N, _dtype_code(Q), scale, launch)
    if _dtype_code(K) != desc.dtype or K.shape[0] != L or K.shape[3] != d or K.shape[2] != M + N:
        raise ValueError("K must be [L, Hkv, M+N, d] with Q's dtype")
    if _dtype_code(Q_last) != desc.dtype or tuple(Q_last.shape) != (L, H, d):
        raise ValueError("Q_last must be [L, H, d] with Q's dtype")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=Q.device)
    _check_out(out, torch.float32, M, "out")
    ws = _workspace(sp_score_workspace_bytes(desc, M), Q.device, workspace)
    st = load_library().sp_score_lastrow(ctypes.byref(desc), Q.data_ptr(), Q_last.data_ptr(),
                                         K.data_ptr(), int(M), out.data_ptr(), ws.data_ptr(),
                                         ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sp_score_lastrow")
    return out


def sp_score_varlen(Q, K, cu_prompt: Sequence[int], scale: float = 0.0, out=None,
                    workspace=None, stream=None, launch: int = SP_LAUNCH_RESIDENT):
    """importance [sum M_r] float32 of a ragged batch. Q [R,L,H,N,d], K [L,Hkv,T,d]
    with T = sum (M_r + N); cu_prompt: host offsets [R+1]."""
    torch = _torch()
    _require_cuda(Q, K)
    R, L, H, N, d = Q.shape
    Hkv = K.shape[1]
    cu = np.ascontiguousarray(np.asarray(cu_prompt, dtype=np.int64))
    if cu.shape != (R + 1,):
        raise ValueError("cu_prompt must hold R+1 offsets")
    desc = score_desc(L, H, Hkv, d, N, _dtype_code(Q), scale, launch)
    if K.shape[2] != int(cu[-1]) + R * N:
        raise ValueError("K must hold sum(M_r + N) key rows")
    if out is None:
        out = torch.empty(int(cu[-1]), dtype=torch.float32, device=Q.device)
    _check_out(out, torch.float32, int(cu[-1]), "out")
    maxM = int(np.max(np.diff(cu))) if R else 1
    ws = _batch_workspace(desc, cu, maxM, Q.device, workspace)
    st = load_library().sp_score_varlen(
        ctypes.byref(desc), int(R), Q.data_ptr(), K.data_ptr(),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), out.data_ptr(), ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sp_score_varlen")
    return out


def sp_window_layout(M: int, window: int, stride: int):
    """(starts, lens, keeps) int64 arrays of the sliding windows over M tokens."""
    lib = load_library()
    n = ctypes.c_int32(0)
    _check(lib.sp_window_layout(int(M), int(window), int(stride), ctypes.byref(n), None, None,
                                None, 0), "sp_window_layout")
    R = n.value
    starts, lens, keeps = (np.zeros(R, np.int64) for _ in range(3))
    p64 = ctypes.POINTER(ctypes.c_int64)
    _check(lib.sp_window_layout(int(M), int(window), int(stride), ctypes.byref(n),
                                starts.ctypes.data_as(p64), lens.ctypes.data_as(p64),
                                keeps.ctypes.data_as(p64), R), "sp_window_layout")
    return starts, lens, keeps


def sp_score_windows(Q, K, cu_window: Sequence[int], keeps: Sequence[int], scale: float = 0.0,
                     out=None, workspace=None, stream=None, launch: int = SP_LAUNCH_RESIDENT):
    """importance [sum keeps] float32 of R windows: Q [R,L,H,N,d], K [L,Hkv,T,d]
    laid out as for sp_score_varlen (cu_window: host offsets [R+1] of the
    windows' prompt keys); window r contributes its first keeps[r] scores."""
    torch = _torch()
    _require_cuda(Q, K)
    R, L, H, N, d = Q.shape
    Hkv = K.shape[1]
    cu = np.ascontiguousarray(np.asarray(cu_window, dtype=np.int64))
    kp = np.ascontiguousarray(np.asarray(keeps, dtype=np.int64))
    if cu.shape != (R + 1,) or kp.shape != (R,):
        raise ValueError("cu_window must hold R+1 offsets and keeps R counts")
    desc = score_desc(L, H, Hkv, d, N, _dtype_code(Q), scale, launch)
    if K.shape[2] != int(cu[-1]) + R * N:
        raise ValueError("K must hold sum(M_r + N) key rows")
    if out is None:
        out = torch.empty(int(kp.sum()), dtype=torch.float32, device=Q.device)
    _check_out(out, torch.float32, int(kp.sum()), "out")
    maxM = int(np.max(np.diff(cu)))
    ws = _batch_workspace(desc, cu, maxM, Q.device, workspace)
    p64 = ctypes.POINTER(ctypes.c_int64)
    st = load_library().sp_score_windows(
        ctypes.byref(desc), int(R), Q.data_ptr(), K.data_ptr(), cu.ctypes.data_as(p64),
        kp.ctypes.data_as(p64), out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
        _stream(stream))
    _check(st, "sp_score_windows")
    return out


def sp_gather_rows(src, kept_idx, n_kept, cu_prompt: Optional[Sequence[int]] = None, dst=None,
                   stream=None):
    """Rows of the kept tokens in kept order: src [T, ...] (any dtype, rows of a
    multiple of 4 bytes), kept_idx / n_kept as sp_select(_varlen) returns them,
    cu_prompt the request offsets (default: one request over all of src)."""
    torch = _torch()
    _require_cuda(src, kept_idx, n_kept)
    T = src.shape[0]
    cu = np.ascontiguousarray(np.asarray([0, T] if cu_prompt is None else cu_prompt,
                                         dtype=np.int64))
    R = cu.shape[0] - 1
    if dst is None:
        dst = torch.zeros((int(cu[-1]),) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    row_bytes = src[0].numel() * src.element_size() if T else 0
    _require_cuda(dst)
    if dst.numel() * dst.element_size() < int(cu[-1]) * row_bytes:
        raise ValueError(f"dst must hold at least {int(cu[-1])} rows of {row_bytes} bytes")
    _check_out(kept_idx, torch.int32, int(cu[-1]), "kept_idx")
    _check_out(n_kept, torch.int32, R, "n_kept")
    st = load_library().sp_gather_rows(src.data_ptr(), int(row_bytes), kept_idx.data_ptr(),
                                       n_kept.data_ptr(), int(R),
                                       cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                       dst.data_ptr(), _stream(stream))
    _check(st, "sp_gather_rows")
    return dst


def sp_break_even(M: int, keep_fraction: float, spec_tps: float = 600.0,
                  target_tps: float = 270.0, safety: float = 1.2) -> bool:
    """Whether sparse prefill is estimated to save more than safety times the
    scoring time (the Implementation Guide's break-even detection)."""
    run = ctypes.c_int32(0)
    _check(load_library().sp_break_even(int(M), float(keep_fraction), float(spec_tps),
                                        float(target_tps), float(safety), ctypes.byref(run)),
           "sp_break_even")
    return bool(run.value)


def sp_select(importance, params: SelectParams, pos_base: int = 0, kept_idx=None, pos_ids=None,
              n_kept=None, stream=None, workspace=None):
    """(kept_idx [M] int32, pos_ids [M] int32, n_kept [1] int32) on the device; the
    first n_kept entries are valid. workspace: None allocates what
    sp_select_workspace_bytes asks for (several workgroups for long prompts),
    False passes none (one workgroup), or a uint8 device tensor."""
    torch = _torch()
    _require_cuda(importance)
    M = importance.shape[0]
    dev = importance.device
    kept_idx = torch.empty(M, dtype=torch.int32, device=dev) if kept_idx is None else kept_idx
    pos_ids = torch.empty(M, dtype=torch.int32, device=dev) if pos_ids is None else pos_ids
    n_kept = torch.empty(1, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    _check_out(importance, torch.float32, M, "importance")
    _check_out(kept_idx, torch.int32, M, "kept_idx")
    _check_out(pos_ids, torch.int32, M, "pos_ids")
    _check_out(n_kept, torch.int32, 1, "n_kept")
    if workspace is None:
        nbytes = sp_select_workspace_bytes(1, int(M), params)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes > 0 else False
    if workspace is False:
        ws_ptr, ws_bytes = None, 0
    else:
        _check_out(workspace, torch.uint8, 0, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = load_library().sp_select(importance.data_ptr(), int(M), ctypes.byref(params),
                                  int(pos_base), kept_idx.data_ptr(), pos_ids.data_ptr(),
                                  n_kept.data_ptr(), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "sp_select")
    return kept_idx, pos_ids, n_kept


def sp_score_select(Q, K, params: SelectParams, pos_base: int = 0, M: Optional[int] = None,
                    scale: float = 0.0, out=None, kept_idx=None, pos_ids=None, n_kept=None,
                    workspace=None, stream=None, launch: int = SP_LAUNCH_RESIDENT):
    """sp_score and sp_select of one prompt in one launch: (importance [M]
    float32, kept_idx [M] int32, pos_ids [M] int32, n_kept [1] int32)."""
    torch = _torch()
    _require_cuda(Q, K)
    L, H, N, d = Q.shape
    Hkv = K.shape[1]
    if M is None:
        M = K.shape[2] - N
    desc = score_desc(L, H, Hkv, d, N, _dtype_code(Q), scale, launch)
    if _dtype_code(K) != desc.dtype or K.shape[0] != L or K.shape[3] != d or K.shape[2] != M + N:
        raise ValueError("K must be [L, Hkv, M+N, d] with Q's dtype")
    dev = Q.device
    out = torch.empty(M, dtype=torch.float32, device=dev) if out is None else out
    kept_idx = torch.empty(M, dtype=torch.int32, device=dev) if kept_idx is None else kept_idx
    pos_ids = torch.empty(M, dtype=torch.int32, device=dev) if pos_ids is None else pos_ids
    n_kept = torch.empty(1, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    _check_out(out, torch.float32, M, "out")
    _check_out(kept_idx, torch.int32, M, "kept_idx")
    _check_out(pos_ids, torch.int32, M, "pos_ids")
    _check_out(n_kept, torch.int32, 1, "n_kept")
    ws = _workspace(sp_score_workspace_bytes(desc, M), dev, workspace)
    st = load_library().sp_score_select(ctypes.byref(desc), Q.data_ptr(), K.data_ptr(), int(M),
                                        ctypes.byref(params), int(pos_base), out.data_ptr(),
                                        kept_idx.data_ptr(), pos_ids.data_ptr(), n_kept.data_ptr(),
                                        ws.data_ptr(), ws.numel() * ws.element_size(),
                                        _stream(stream))
    _check(st, "sp_score_select")
    return out, kept_idx, pos_ids, n_kept


def sp_select_varlen(importance, cu_prompt: Sequence[int], params: SelectParams,
                     pos_base: Optional[Sequence[int]] = None, kept_idx=None, pos_ids=None,
                     n_kept=None, stream=None):
    """Per-request selection of a ragged batch; request r's outputs start at
    cu_prompt[r]; n_kept [R]."""
    torch = _torch()
    _require_cuda(importance)
    cu = np.ascontiguousarray(np.asarray(cu_prompt, dtype=np.int64))
    R = cu.shape[0] - 1
    total = int(cu[-1])
    dev = importance.device
    kept_idx = torch.empty(total, dtype=torch.int32, device=dev) if kept_idx is None else kept_idx
    pos_ids = torch.empty(total, dtype=torch.int32, device=dev) if pos_ids is None else pos_ids
    n_kept = torch.empty(R, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    _check_out(importance, torch.float32, total, "importance")
    _check_out(kept_idx, torch.int32, total, "kept_idx")
    _check_out(pos_ids, torch.int32, total, "pos_ids")
    _check_out(n_kept, torch.int32, R, "n_kept")
    pb = None
    if pos_base is not None:
        pb_arr = np.ascontiguousarray(np.asarray(pos_base, dtype=np.int32))
        pb = pb_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    st = load_library().sp_select_varlen(
        importance.data_ptr(), int(R), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), pb,
        ctypes.byref(params), kept_idx.data_ptr(), pos_ids.data_ptr(), n_kept.data_ptr(), None,
        0, _stream(stream))
    _check(st, "sp_select_varlen")
    return kept_idx, pos_ids, n_kept


def sp_read_probe(buf, grid: int, depth: int = 8, flag=None, stream=None):
    """Measurement aid: one streaming read of the whole of `buf` (a contiguous
    CUDA tensor) by `grid` workgroups (see the C header). Returns `flag`."""
    torch = _torch()
    _require_cuda(buf)
    if flag is None:
        flag = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check_out(flag, torch.int32, 1, "flag")
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().sp_read_probe(buf.data_ptr(), int(nbytes), int(grid), int(depth),
                                        flag.data_ptr(), _stream(stream)), "sp_read_probe")
    return flag
