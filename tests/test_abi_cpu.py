"""The C-ABI library loads, exports every call the header declares, and rejects
bad arguments synchronously (no GPU needed: every checked error returns before
any device call)."""
import ctypes
import os
import re
import subprocess

import pytest

import attention_token_scoring_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specprefill.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sp.LIB_PATH):
        pytest.skip("libspecprefill.so not built (run __graft_entry__.build())")
    return sp.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(sp.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (sp_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        getattr(lib, name)


def test_status_strings(lib):
    for s in range(5):
        assert sp.sp_status_string(s).startswith("SP_")
    assert "unknown" in sp.sp_status_string(99)


def desc(**kw):
    base = dict(L=2, H=4, Hkv=2, d=64, N=8, dtype=sp.SP_BF16, scale=0.0)
    base.update(kw)
    return sp.score_desc(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(H=3, Hkv=2), sp.SP_EINVAL),
    (dict(L=0), sp.SP_EINVAL),
    (dict(N=0), sp.SP_EINVAL),
    (dict(dtype=7), sp.SP_EINVAL),
    (dict(scale=-1.0), sp.SP_EINVAL),
    (dict(scale=float("inf")), sp.SP_EINVAL),
    (dict(launch=2), sp.SP_EINVAL),
    (dict(launch=-1), sp.SP_EINVAL),
    (dict(d=96), sp.SP_EUNSUPPORTED),
    (dict(H=12, Hkv=4), sp.SP_EUNSUPPORTED),       # G = 3, not a power of two
    (dict(H=32, Hkv=8, N=16), sp.SP_EUNSUPPORTED),  # G*N = 64 > 32
])
def test_score_rejects_descriptors(lib, kw, status):
    d = desc(**kw)
    st = lib.sp_score(ctypes.byref(d), FAKE, FAKE, 100, FAKE, FAKE, 1 << 30, None)
    assert st == status
    assert lib.sp_score_workspace_bytes(ctypes.byref(d), 100) == 0


def test_score_rejects_pointers_and_sizes(lib):
    d = desc()
    assert lib.sp_score(ctypes.byref(d), None, FAKE, 100, FAKE, FAKE, 1 << 30, None) == sp.SP_EINVAL
    assert lib.sp_score(ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, 1 << 30, None) == sp.SP_EINVAL
    mis = ctypes.c_void_p(0x1008)  # not 16-byte aligned
    assert lib.sp_score(ctypes.byref(d), mis, FAKE, 100, FAKE, FAKE, 1 << 30, None) == sp.SP_EINVAL
    assert lib.sp_score(None, FAKE, FAKE, 100, FAKE, FAKE, 1 << 30, None) == sp.SP_EINVAL


def test_varlen_rejects_offsets(lib):
    d = desc()
    for cu in ([1, 10], [0, 10, 10], [0, 5, 3]):
        arr = (ctypes.c_int64 * len(cu))(*cu)
        st = lib.sp_score_varlen(ctypes.byref(d), len(cu) - 1, FAKE, FAKE, arr, FAKE, FAKE,
                                 1 << 30, None)
        assert st == sp.SP_EINVAL, cu
    assert lib.sp_score_varlen(ctypes.byref(d), 0, FAKE, FAKE, None, FAKE, FAKE, 1, None) \
        == sp.SP_EINVAL


def test_workspace_bytes_grows_with_prompt(lib):
    d = desc(L=32, H=32, Hkv=8, d=128)
    a = sp.sp_score_workspace_bytes(d, 1024)
    b = sp.sp_score_workspace_bytes(d, 32768)
    assert 0 < a <= b < (64 << 20)


def test_plan_for_the_8b_shape(lib):
    """At L=32, Hkv=8, d=128, M=32768 the 256 units are shared by groups of
    workgroups that each hold one key slice; the grid (groups plus combiners)
    fits the device, one workgroup per CU."""
    p = sp.sp_score_plan(desc(L=32, H=32, Hkv=8, d=128), 32768)
    assert p["rows"] == 32 and p["units"] == 256
    assert p["g"] * p["keys_per_wg"] >= 32768 and p["keys_per_wg"] <= 1024
    assert p["grid"] <= p["cus"]


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=0), sp.SP_EINVAL),
    (dict(pool_k=4), sp.SP_EINVAL),
    (dict(pool_k=0), sp.SP_EINVAL),
    (dict(keep_rate=0.0), sp.SP_EINVAL),
    (dict(keep_rate=1.01), sp.SP_EINVAL),
    (dict(mode="mass", mass=0.0), sp.SP_EINVAL),
    (dict(mode=5), sp.SP_EINVAL),
    (dict(boost_first_mult=-1.0), sp.SP_EINVAL),
    (dict(boost_last_n=-3), sp.SP_EINVAL),
    (dict(chunk=1), sp.SP_EUNSUPPORTED),            # nc = 10000 > 5120
    (dict(boost_first_mult=3e6), sp.SP_EUNSUPPORTED),  # pooled sums would exceed 2^53
    (dict(min_tok=128), sp.SP_EINVAL),              # threshold-mode fields in top-K mode
    (dict(mode="mass", mass=0.5, max_keep=10), sp.SP_EINVAL),
    (dict(mode="threshold"), sp.SP_EINVAL),         # threshold mode takes no pooling
    (dict(mode="threshold", pool_k=1, boost_first_n=4), sp.SP_EINVAL),  # nor boosts
    (dict(mode="threshold", pool_k=1, min_tok=-1), sp.SP_EINVAL),
    (dict(mode="threshold", pool_k=1, max_keep=-1), sp.SP_EINVAL),
    (dict(mode="threshold", pool_k=1, keep_rate=0.0), sp.SP_EINVAL),
    (dict(mode="threshold", pool_k=1, chunk=1), sp.SP_EUNSUPPORTED),  # nc = 10000 > 4096
    (dict(mode="threshold", pool_k=1, chunk=2), sp.SP_EUNSUPPORTED),  # nc = 5000 > 4096
    (dict(norm=3), sp.SP_EINVAL),
    (dict(norm="minmax", norm_hi=0.5), sp.SP_EINVAL),
    (dict(norm="percentile", norm_lo=0.5, norm_hi=0.5), sp.SP_EINVAL),
    (dict(norm="percentile", norm_lo=-0.1, norm_hi=0.9), sp.SP_EINVAL),
    (dict(norm="percentile", norm_lo=0.1, norm_hi=1.1), sp.SP_EINVAL),
    (dict(norm="zscore", norm_hi=0.0), sp.SP_EINVAL),
    (dict(norm="zscore", norm_lo=0.1, norm_hi=3.0), sp.SP_EINVAL),
    (dict(norm="zscore", norm_hi=float("inf")), sp.SP_EINVAL),
    (dict(mode="threshold", pool_k=1, norm="percentile", norm_lo=0.1, norm_hi=0.9), sp.SP_EINVAL),
])
def test_select_rejects(lib, kw, status):
    base = dict(chunk=32, pool_k=3, mode="topk", keep_rate=0.3)
    base.update(kw)
    p = sp.select_params(**base)
    st = lib.sp_select(FAKE, 10000, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, 0, None)
    assert st == status


@pytest.mark.parametrize("mode,limit", [("topk", 5120), ("mass", 5120), ("threshold", 4096)])
def test_select_chunk_count_limit(lib, mode, limit):
    """One chunk more than the kernels hold is refused before anything runs
    (the largest accepted count is exercised on the GPU)."""
    kw = dict(chunk=32, pool_k=1 if mode == "threshold" else 3, mode=mode, keep_rate=0.3)
    if mode == "mass":
        kw.update(mass=0.85)
    p = sp.select_params(**kw)
    M = limit * 32 + 1
    assert lib.sp_select(FAKE, M, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, 0, None) \
        == sp.SP_EUNSUPPORTED


def test_score_select_rejects(lib):
    """The fused call validates like sp_score and sp_select, and refuses the
    threshold mode; every case fails before anything runs."""
    d = desc()
    ok = sp.select_params(chunk=32, pool_k=3, mode="topk", keep_rate=0.3)
    thr = sp.select_params(chunk=32, pool_k=1, mode="threshold", keep_rate=0.3, min_tok=128)
    bad = sp.select_params(chunk=0, pool_k=3, mode="topk", keep_rate=0.3)

    def call(params, M=1000, kept=FAKE, pos_base=0, ws_bytes=1 << 30, dd=d):
        return lib.sp_score_select(ctypes.byref(dd), FAKE, FAKE, M, ctypes.byref(params), pos_base,
                                   FAKE, kept, FAKE, FAKE, FAKE, ws_bytes, None)

    assert call(thr) == sp.SP_EUNSUPPORTED
    assert call(bad) == sp.SP_EINVAL
    assert call(ok, kept=None) == sp.SP_EINVAL
    assert call(ok, M=0) == sp.SP_EINVAL
    assert call(ok, M=5120 * 32 + 1) == sp.SP_EUNSUPPORTED
    assert call(ok, pos_base=2147483600) == sp.SP_EINVAL
    assert call(ok, dd=desc(N=0)) == sp.SP_EINVAL


def test_select_rejects_null_and_sizes(lib):
    p = sp.select_params(chunk=32, pool_k=3, keep_rate=0.3)
    assert lib.sp_select(None, 100, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, 0, None) \
        == sp.SP_EINVAL
    assert lib.sp_select(FAKE, 0, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, 0, None) \
        == sp.SP_EINVAL
    assert lib.sp_select(FAKE, 100, ctypes.byref(p), 2147483600, FAKE, FAKE, FAKE, None, 0,
                         None) == sp.SP_EINVAL
    cu = (ctypes.c_int64 * 3)(0, 50, 50)
    assert lib.sp_select_varlen(FAKE, 2, cu, None, ctypes.byref(p), FAKE, FAKE, FAKE, None, 0,
                                None) == sp.SP_EINVAL
    assert sp.sp_select_workspace_bytes(1, 100, p) == 0


def test_select_workspace_only_for_long_single_prompts_with_min_max():
    # several workgroups select one prompt of >= 49152 tokens under min-max
    # normalisation (top-K or mass); nothing else asks for a workspace
    need = 8 * (2 * 256 + 2 * 5120)
    topk = sp.select_params(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)
    mass = sp.select_params(chunk=32, pool_k=5, mode="mass", mass=0.85)
    assert sp.sp_select_workspace_bytes(1, 49152, topk) == need
    assert sp.sp_select_workspace_bytes(1, 131072, mass) == need
    assert sp.sp_select_workspace_bytes(1, 49151, topk) == 0
    assert sp.sp_select_workspace_bytes(1, 32768, mass) == 0
    assert sp.sp_select_workspace_bytes(2, 100000, topk) == 0
    pct = sp.select_params(chunk=32, pool_k=13, mode="topk", keep_rate=0.1, norm="percentile",
                           norm_lo=0.01, norm_hi=0.99)
    assert sp.sp_select_workspace_bytes(1, 100000, pct) == 0
    thr = sp.select_params(chunk=32, mode="threshold", keep_rate=0.3, min_tok=64)
    assert sp.sp_select_workspace_bytes(1, 100000, thr) == 0


def test_score_status_rejects_null_pointers(lib):
    out = ctypes.c_int32(7)
    assert lib.sp_score_status(None, None, ctypes.byref(out)) == sp.SP_EINVAL
    assert lib.sp_score_status(FAKE, None, None) == sp.SP_EINVAL
    assert out.value == 7


def test_profile_events_need_both_or_neither(lib):
    assert lib.sp_profile_score_kernel(FAKE, None) == sp.SP_EINVAL
    assert lib.sp_profile_score_kernel(None, FAKE) == sp.SP_EINVAL
    assert lib.sp_profile_score_kernel(None, None) == sp.SP_OK


def test_plan_does_not_depend_on_the_launch_mode(lib):
    for M in (1, 4608, 32768, 131072):
        a = sp.sp_score_plan(desc(L=32, H=32, Hkv=8, d=128), M)
        b = sp.sp_score_plan(desc(L=32, H=32, Hkv=8, d=128, launch=sp.SP_LAUNCH_COOPERATIVE), M)
        assert a == b


@pytest.mark.parametrize("dtype,d,longest", [(sp.SP_BF16, 128, 142792), (sp.SP_BF16, 64, 142792),
                                             (sp.SP_F32, 64, 142792), (sp.SP_F32, 128, 85672)])
def test_plan_longest_prompt(lib, dtype, d, longest):
    """On 256 CUs: 255 workgroups of at most 560 keys (336 for f32 at d = 128)
    hold the M prompt keys and the N = 8 look-ahead keys, and one combiner;
    one key more is rejected."""
    dd = desc(L=1, H=4, Hkv=1, d=d, N=8, dtype=dtype)
    p = sp.sp_score_plan(dd, longest)
    if p["cus"] != 256:
        pytest.skip("the limits below are those of a 256-CU device")
    assert p["g"] == 255 and p["grid"] == 256 and p["g"] * p["keys_per_wg"] >= longest + 8
    with pytest.raises(sp.SpError) as e:
        sp.sp_score_plan(dd, longest + 1)
    assert e.value.status == sp.SP_EUNSUPPORTED
    assert sp.sp_score_workspace_bytes(dd, longest + 1) == 0


def test_score_windows_rejects_keeps(lib):
    d = desc()
    cu = (ctypes.c_int64 * 3)(0, 100, 150)
    for keep in ([0, 50], [101, 50], [100, 51], [-1, 1]):
        kp = (ctypes.c_int64 * 2)(*keep)
        assert lib.sp_score_windows(ctypes.byref(d), 2, FAKE, FAKE, cu, kp, FAKE, FAKE, 1 << 30,
                                    None) == sp.SP_EINVAL, keep
    assert lib.sp_score_windows(ctypes.byref(d), 2, FAKE, FAKE, cu, None, FAKE, FAKE, 1 << 30,
                                None) == sp.SP_EINVAL


def test_plan_cache_returns_each_shapes_own_plan(lib):
    # plans are cached per (shape, M, compute units) in a table of a few
    # hundred slots: more distinct keys than slots, asked for in shuffled
    # order, must each get back the plan their first (uncached) call computed
    import numpy as np
    rng = np.random.default_rng(11)
    shapes = [dict(L=32, H=32, Hkv=8, d=128), dict(L=24, H=16, Hkv=8, d=64),
              dict(L=2, H=4, Hkv=2, d=64, dtype=sp.SP_F32), dict(L=28, H=16, Hkv=4, d=128),
              dict(L=16, H=8, Hkv=8, d=64, N=4)]
    keys = [(i, int(M)) for i in range(len(shapes)) for M in rng.integers(1, 80000, 120)]
    first = {}
    for i, M in keys:
        first[(i, M)] = sp.sp_score_plan(desc(**shapes[i]), M)
    for _ in range(2):
        for x in rng.permutation(len(keys)):
            i, M = keys[x]
            assert sp.sp_score_plan(desc(**shapes[i]), M) == first[(i, M)], (shapes[i], M)
    # and the cached plan of a shape is not served for another at the same M
    a = sp.sp_score_plan(desc(**shapes[0]), 32768)
    b = sp.sp_score_plan(desc(**shapes[3]), 32768)
    assert a != b
