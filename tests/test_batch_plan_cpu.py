"""Host logic of ragged-batch scheduling (no device work): which requests of an
sp_score_varlen / sp_score_windows call share a launch. Every request is in
exactly one launch, a launch holds at most 8 requests whose longest prompt is
at most 4 times the shortest, launches go in order of prompt length, and a
batch of many short prompts of one length is packed."""
import ctypes

import numpy as np
import pytest

import attention_token_scoring_amd as sp

DESC_8B = dict(L=32, H=32, Hkv=8, d=128, N=8)


def _desc(dtype=sp.SP_BF16, **kw):
    a = dict(DESC_8B)
    a.update(kw)
    return sp.score_desc(a["L"], a["H"], a["Hkv"], a["d"], a["N"], dtype, 0.0, 0)


def _cu(lens):
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    return cu


LAYOUTS = [
    ("uniform-16x4k", [4096] * 16),
    ("uniform-12x2k", [2048] * 12),
    ("ragged", [21056, 61248, 5760, 38528, 48384, 55744, 43392, 10496, 17536, 42176, 5120, 13312,
                43584, 25280, 14784, 52544]),
    ("mixed", [4096, 60000, 2048, 30000, 8192, 1000, 50000, 12000, 3000, 40000, 6000, 20000]),
    ("tiny", [1, 2, 3, 5, 1000, 1]),
]


@pytest.mark.parametrize("name,lens", LAYOUTS, ids=[x[0] for x in LAYOUTS])
def test_schedule_is_a_valid_packing(name, lens):
    d = _desc()
    cu = _cu(lens)
    ws = sp.sp_score_batch_workspace_bytes(d, cu)
    assert ws >= sp.sp_score_workspace_bytes(d, max(lens))
    launch = sp.sp_score_batch_plan(d, cu, ws)
    assert launch.shape == (len(lens),)
    nl = int(launch.max()) + 1
    assert sorted(set(launch.tolist())) == list(range(nl))  # every launch index used
    prev_hi = 0
    for l in range(nl):
        m = np.asarray(lens)[launch == l]
        assert 1 <= len(m) <= 8, (name, l)
        assert m.max() <= 4 * m.min(), (name, l, m)
        assert m.min() >= prev_hi, (name, l)  # launches in order of length
        prev_hi = m.max()


def test_uniform_short_prompts_are_packed():
    d = _desc()
    for lens, want in (([4096] * 16, 2), ([2048] * 12, 2), ([1000] * 4, 1), ([1000] * 32, 4)):
        cu = _cu(lens)
        launch = sp.sp_score_batch_plan(d, cu, sp.sp_score_batch_workspace_bytes(d, cu))
        assert int(launch.max()) + 1 == want, lens


def test_long_prompts_keep_a_launch_each():
    # (at 64K tokens a prompt streams at the full rate alone)
    d = _desc()
    cu = _cu([65536, 65536])
    launch = sp.sp_score_batch_plan(d, cu, sp.sp_score_batch_workspace_bytes(d, cu))
    assert launch.tolist() == [0, 1]


def test_single_request_and_errors():
    d = _desc()
    assert sp.sp_score_batch_plan(d, [0, 5000], 1 << 40).tolist() == [0]
    with pytest.raises(sp.SpError):  # below what one request needs alone
        sp.sp_score_batch_plan(d, [0, 5000, 9000], 1024)
    with pytest.raises(sp.SpError):
        sp.sp_score_batch_plan(d, [0, 5000, 5000], 1 << 40)  # an empty request
    lib = sp.load_library()
    cu = np.array([1, 5000], np.int64)  # cu[0] != 0
    n = ctypes.c_int32(0)
    st = lib.sp_score_batch_plan(ctypes.byref(d), 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 1 << 40, None, ctypes.byref(n))
    assert st == sp.SP_EINVAL
    assert sp.sp_score_batch_workspace_bytes(d, cu) == 0
    cu = np.array([0, 4096, 8192], np.int64)
    st = lib.sp_score_batch_plan(ctypes.byref(d), 2, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 1 << 40, None, ctypes.byref(n))  # (launch_of may be NULL)
    assert st == sp.SP_OK and n.value >= 1


@pytest.mark.parametrize("dtype,dd,H,Hkv,N", [(sp.SP_F32, 128, 16, 4, 8), (sp.SP_F32, 64, 16, 4, 8),
                                              (sp.SP_BF16, 64, 8, 8, 4), (sp.SP_BF16, 128, 4, 4, 32)])
def test_schedules_for_other_configurations(dtype, dd, H, Hkv, N):
    d = _desc(dtype, L=4, H=H, Hkv=Hkv, d=dd, N=N)
    lens = [3000, 2000, 2500, 4000, 1, 7]
    cu = _cu(lens)
    launch = sp.sp_score_batch_plan(d, cu, sp.sp_score_batch_workspace_bytes(d, cu))
    for l in range(int(launch.max()) + 1):
        m = np.asarray(lens)[launch == l]
        assert 1 <= len(m) <= 8 and m.max() <= 4 * m.min()


@pytest.mark.parametrize("seed", range(8))
def test_random_batches_schedule_validly(seed):
    """Seeded random batches (1 to 40 requests of 1 to 100000 tokens, some of
    equal length): the schedule's invariants hold, and it is the same on a
    second query (the plans are cached)."""
    rng = np.random.default_rng(seed)
    d = _desc()
    for _ in range(10):
        R = int(rng.integers(1, 41))
        lens = rng.integers(1, 100001, R)
        if R > 4:
            lens[rng.integers(0, R, R // 4)] = int(rng.integers(1, 20000))
        cu = _cu(lens)
        ws = sp.sp_score_batch_workspace_bytes(d, cu)
        assert ws >= sp.sp_score_workspace_bytes(d, int(lens.max()))
        launch = sp.sp_score_batch_plan(d, cu, ws)
        assert np.array_equal(launch, sp.sp_score_batch_plan(d, cu, ws))
        nl = int(launch.max()) + 1
        assert sorted(set(launch.tolist())) == list(range(nl))
        prev_hi = 0
        for l in range(nl):
            m = lens[launch == l]
            assert 1 <= len(m) <= 8 and m.max() <= 4 * m.min()
            assert m.min() >= prev_hi
            prev_hi = m.max()
        # a workspace that fits one request at a time still schedules every request
        one = sp.sp_score_workspace_bytes(d, int(lens.max()))
        small = sp.sp_score_batch_plan(d, cu, one)
        assert int(small.max()) + 1 >= 1 and small.shape == (R,)
