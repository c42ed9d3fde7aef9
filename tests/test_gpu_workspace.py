"""The scoring workspace needs no initialisation and nothing between calls:
its synchronisation slots carry the epoch of the launch that wrote them, so
whatever a workspace holds (zeros, ones, a fill pattern, random bytes, or the
slots of an earlier call put back) never passes for the current launch's.
Each call here must reproduce, bit for bit, the scores of the same call on a
fresh workspace; calls with different plans (so different slot layouts)
alternate on one workspace."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402
from test_gpu_parity import to_dev  # noqa: E402

# two shapes whose plans differ (groups, slice, units), both with several
# groups per key slice
SHAPES = [(4, 32, 8, 128, 8, 20000, 41), (3, 16, 8, 64, 8, 3000, 43)]


def _inputs(L, H, Hkv, d, N, M, seed):
    w = synth.Workload("ws", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=synth.BF16, seed=seed, M=M,
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_request(w)
    return to_dev(Qh), to_dev(Kh), sp.score_desc(L, H, Hkv, d, N), M


def _reference(Q, K, desc, M):
    ws = torch.zeros(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device="cuda")
    out = sp.sp_score(Q, K, workspace=ws)
    torch.cuda.synchronize()
    return out.clone()


@pytest.mark.parametrize("fill", ["zeros", "ones", "0x5a", "random"])
def test_scores_do_not_depend_on_what_the_workspace_holds(fill):
    Q, K, desc, M = _inputs(*SHAPES[0])
    ref = _reference(Q, K, desc, M)
    assert sp.sp_score_plan(desc, M)["ngroups"] > 1
    n = sp.sp_score_workspace_bytes(desc, M)
    print(f"case fill={fill} M={M}", flush=True)
    if fill == "random":
        g = torch.Generator(device="cuda").manual_seed(7)
        ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
    else:
        ws = torch.full((n,), {"zeros": 0, "ones": 255, "0x5a": 0x5A}[fill], dtype=torch.uint8,
                        device="cuda")
    for rep in range(3):
        out = sp.sp_score(Q, K, out=torch.full((M,), -1.0, device="cuda"), workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (fill, rep)
        assert sp.sp_score_status(ws) is False


def test_an_earlier_calls_slots_put_back_are_not_taken():
    Q, K, desc, M = _inputs(*SHAPES[0])
    ref = _reference(Q, K, desc, M)
    ws = torch.zeros(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device="cuda")
    sp.sp_score(Q, K, workspace=ws)
    torch.cuda.synchronize()
    snapshot = ws.clone()  # every slot tagged with that call's epochs
    for rep in range(3):
        ws.copy_(snapshot)
        print(f"case restored snapshot rep={rep}", flush=True)
        out = sp.sp_score(Q, K, out=torch.full((M,), -1.0, device="cuda"), workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep


def test_plans_alternate_on_one_workspace():
    cases = [_inputs(*s) for s in SHAPES]
    refs = [_reference(*c) for c in cases]
    plans = [sp.sp_score_plan(c[2], c[3]) for c in cases]
    assert plans[0] != plans[1], plans
    n = max(sp.sp_score_workspace_bytes(c[2], c[3]) for c in cases)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for rep in range(4):
        for i, (Q, K, desc, M) in enumerate(cases):
            print(f"case alternate rep={rep} shape={i}", flush=True)
            out = sp.sp_score(Q, K, out=torch.full((M,), -1.0, device="cuda"), workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, refs[i]), (rep, i)
