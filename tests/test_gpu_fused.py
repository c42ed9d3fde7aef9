"""sp_score_select (scoring and selection in one launch) gives, bit for bit,
what sp_score followed by sp_select gives: the same importance, kept indices,
position ids and count, for both operand types, several head-group sizes,
one and many groups per key slice, both selection modes, the robust
normalisations, boosts and position bases; prompts of 16K tokens or more
with min-max normalisation have their chunk masses summed across the
streaming workgroups (the other cases by the selecting workgroup alone). A
forced time-out of the scoring kernel's waits leaves n_kept = -1, and what
the workspace held before does not change the outputs."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402
from test_gpu_parity import to_dev  # noqa: E402

BF, F32 = synth.BF16, synth.F32

CASES = [
    # id, (L, H, Hkv, d, N, M, dtype), selection
    ("tiny-f32", (2, 4, 2, 64, 8, 1024, F32), dict(chunk=32, pool_k=3, mode="topk", keep_rate=0.3)),
    ("0.8b-mass-boosts", (24, 16, 8, 64, 8, 4608, BF),
     dict(chunk=32, pool_k=5, mode="mass", mass=0.85, boost_first_n=64, boost_first_mult=1.5,
          boost_last_n=128, boost_last_mult=1.3)),
    ("8b-small-topk", (4, 32, 8, 128, 8, 20000, BF), dict(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)),
    ("G1-N16-percentile", (2, 4, 4, 128, 16, 3001, BF),
     dict(chunk=16, pool_k=3, mode="mass", mass=0.7, norm="percentile", norm_lo=0.05, norm_hi=0.95)),
    ("G8-N4-zscore", (1, 16, 2, 128, 4, 2000, BF),
     dict(chunk=24, pool_k=1, mode="topk", keep_rate=0.25, norm="zscore", norm_hi=3.0)),
    ("M1", (1, 2, 2, 64, 3, 1, BF), dict(chunk=32, pool_k=3, mode="topk", keep_rate=0.5)),
    ("longer-mass", (8, 32, 8, 128, 8, 40000, BF), dict(chunk=64, pool_k=13, mode="mass", mass=0.85)),
    # summed across workgroups: boosts, a short last chunk, one kv-head plane
    ("large-mass-boosts-ragged-chunk", (8, 16, 8, 64, 8, 24001, BF),
     dict(chunk=24, pool_k=5, mode="mass", mass=0.8, boost_first_n=100, boost_first_mult=1.5,
          boost_last_n=70, boost_last_mult=1.25)),
    ("large-one-plane-f32", (1, 4, 1, 128, 8, 16384, F32), dict(chunk=8, pool_k=3, mode="topk", keep_rate=0.2)),
    # a robust normalisation on a long prompt: the selecting workgroup alone
    ("large-percentile", (4, 32, 8, 128, 8, 20000, BF),
     dict(chunk=32, pool_k=13, mode="topk", keep_rate=0.1, norm="percentile", norm_lo=0.01, norm_hi=0.99)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_score_then_select(case):
    name, (L, H, Hkv, d, N, M, dt), sel = case
    print(f"case {name}", flush=True)
    w = synth.Workload("fused", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=47, M=M,
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    params = sp.select_params(**sel)
    imp = sp.sp_score(Q, K)
    kept, pos, n = sp.sp_select(imp, params, pos_base=11)
    torch.cuda.synchronize()
    for rep in range(2):
        fimp, fkept, fpos, fn = sp.sp_score_select(Q, K, params, pos_base=11)
        torch.cuda.synchronize()
        nk = int(n.cpu()[0])
        assert int(fn.cpu()[0]) == nk, (name, rep)
        assert torch.equal(fimp, imp), (name, rep)
        assert torch.equal(fkept[:nk], kept[:nk]), (name, rep)
        assert torch.equal(fpos[:nk], pos[:nk]), (name, rep)


@pytest.mark.parametrize("M", [6000, 20000], ids=["one-workgroup", "across-workgroups"])
def test_fused_reports_a_timed_out_call(M):
    w = synth.Workload("fused", L=8, H=32, Hkv=8, d=128, N=8, dtype=BF, seed=53, M=M,
                       plant_frac=0.05)
    Qh, Kh, M = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    params = sp.select_params(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)
    ws = torch.empty(sp.sp_score_workspace_bytes(sp.score_desc(8, 32, 8, 128, 8), M),
                     dtype=torch.uint8, device="cuda")
    print("case fused time-out", flush=True)
    try:
        sp.sp_set_wait_limit(1)
        _, _, _, n = sp.sp_score_select(Q, K, params, workspace=ws)
        torch.cuda.synchronize()
        assert sp.sp_score_status(ws) is True
        assert int(n.cpu()[0]) == -1
    finally:
        sp.sp_set_wait_limit(0)
    imp, kept, pos, n = sp.sp_score_select(Q, K, params, workspace=ws)
    torch.cuda.synchronize()
    assert sp.sp_score_status(ws) is False
    ref_kept, _, ref_n = sp.sp_select(sp.sp_score(Q, K), params)
    torch.cuda.synchronize()
    assert int(n.cpu()[0]) == int(ref_n.cpu()[0]) > 0


@pytest.mark.parametrize("M", [6000, 20000], ids=["one-workgroup", "across-workgroups"])
def test_fused_ignores_workspace_contents(M):
    w = synth.Workload("fused", L=4, H=32, Hkv=8, d=128, N=8, dtype=BF, seed=59, M=M, plant_frac=0.05)
    Qh, Kh, _ = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    params = sp.select_params(chunk=32, pool_k=5, mode="mass", mass=0.85)
    nbytes = sp.sp_score_workspace_bytes(sp.score_desc(4, 32, 8, 128, 8), M)
    print(f"case fused workspace M={M}", flush=True)
    ref = sp.sp_score_select(Q, K, params)
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda").manual_seed(61)
    for fill in ("zeros", "ones", "random"):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(255)
        else:
            ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g))
        out = sp.sp_score_select(Q, K, params, workspace=ws)
        torch.cuda.synchronize()
        nk = int(ref[3].cpu()[0])
        assert int(out[3].cpu()[0]) == nk, fill
        assert torch.equal(out[0], ref[0]), fill
        assert torch.equal(out[1][:nk], ref[1][:nk]) and torch.equal(out[2][:nk], ref[2][:nk]), fill
