"""sp_score_noalloc (the allocation-free scoring call: its workspace is the
library's static per-device scratch array) against sp_score with a workspace
of its own, through the C ABI: the same kernels and plan, so the scores must
be identical bit for bit. Two calls in a row, the second with a smaller
prompt (the array keeps the first call's contents), then a size the array
cannot hold, which must be refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _noalloc(desc, Q, K, M, out):
    lib = sp.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.sp_score_noalloc(ctypes.byref(desc), Q.data_ptr(), K.data_ptr(), int(M),
                                out.data_ptr(), stream)


CASES = [  # (L, H, Hkv, d, N, M, dtype): the second call is smaller
    (32, 32, 8, 128, 8, 6000, synth.BF16),
    (2, 8, 2, 64, 8, 1000, synth.F32),
]


def test_noalloc_matches_sp_score_on_consecutive_calls():
    for k, (L, H, Hkv, d, N, M, dt) in enumerate(CASES):
        print(f"noalloc call {k}: L={L} H={H} Hkv={Hkv} d={d} N={N} M={M}", flush=True)
        w = synth.Workload("noalloc", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=50 + k, M=M,
                           plant_frac=0.05)
        Qh, Kh, _ = synth.make_request(w)
        Q, K = to_dev(Qh), to_dev(Kh)
        desc = sp.score_desc(L, H, Hkv, d, N, sp.SP_BF16 if dt else sp.SP_F32)
        ref = sp.sp_score(Q, K)
        out = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
        assert _noalloc(desc, Q, K, M, out) == sp.SP_OK
        torch.cuda.synchronize()
        assert torch.equal(out, ref), k
        got = out.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - oracle.score(Qh, Kh))) <= 2e-3


def test_noalloc_refuses_a_plan_larger_than_its_array():
    # 4096 (layer, kv-head) units at 32K keys: the partial statistics alone
    # need more than the array's 64 MiB; refused before any launch (the
    # pointers are never dereferenced)
    desc = sp.score_desc(512, 32, 8, 128, 8, sp.SP_BF16)
    fake = ctypes.c_void_p(0x100000)
    lib = sp.load_library()
    assert lib.sp_score_noalloc(ctypes.byref(desc), fake, fake, 32768, fake, None) \
        == sp.SP_EWORKSPACE
