"""The hot path under HIP graph capture: sp_score + sp_select, or the fused
sp_score_select (both of its ways: the selecting workgroup alone, and the
chunk masses summed across the launch), captured once (torch.cuda.CUDAGraph
on the capture stream) and replayed several times, with eager work that
overwrites the outputs between replays, and the workspace either overwritten
too or left as the previous replay left it; every replay must reproduce the
eager call bit for bit (the scoring kernel is deterministic; a launch's epoch
is fixed into the graph, so a clearing kernel captured before it resets the
workspace's tagged words on every replay, with no memset nodes in the graph:
without it a replay would take the previous replay's slots for its own). At
65536 tokens the eager selection runs on a grid of workgroups and the
captured one on one workgroup (a graph would fix the grid's epoch): the two
must agree."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402
from test_gpu_parity import to_dev  # noqa: E402


@pytest.mark.parametrize("fused", [False, True], ids=["two-calls", "fused"])
@pytest.mark.parametrize("refill", [True, False], ids=["ws-overwritten", "ws-kept"])
@pytest.mark.parametrize("M", [3000, 20000, 65536])
def test_graph_replays_match_eager(M, refill, fused):
    w = synth.Workload("case", L=2, H=8, Hkv=2, d=128, N=8, dtype=synth.BF16, seed=9, M=M,
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_request(w)
    _, Kh2, _ = synth.make_request(synth.Workload("case", L=2, H=8, Hkv=2, d=128, N=8, dtype=synth.BF16, seed=10,
                                                  M=M, plant_frac=0.05, plant_chunk=32))
    Q = to_dev(Qh)
    Ks = [to_dev(Kh), to_dev(Kh2)]  # replays alternate the keys, so a stale slot would be wrong
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N)
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device="cuda")
    params = sp.select_params(chunk=32, pool_k=5, mode="mass", mass=0.8, boost_first_n=16,
                              boost_first_mult=1.5)
    eager = []
    for Kx in Ks:
        imp_e = sp.sp_score(Q, Kx, out=torch.empty(M, dtype=torch.float32, device="cuda"), workspace=ws)
        kept_e, pos_e, n_e = sp.sp_select(imp_e, params, pos_base=3)
        torch.cuda.synchronize()
        eager.append((imp_e, kept_e, pos_e, int(n_e.cpu()[0])))
    assert not torch.equal(eager[0][0], eager[1][0])
    K = Ks[0].clone()  # the graph's key buffer

    imp = torch.empty(M, dtype=torch.float32, device="cuda")
    kept = torch.empty(M, dtype=torch.int32, device="cuda")
    pos = torch.empty(M, dtype=torch.int32, device="cuda")
    nk = torch.empty(1, dtype=torch.int32, device="cuda")

    def body():
        if fused:
            sp.sp_score_select(Q, K, params, pos_base=3, out=imp, kept_idx=kept, pos_ids=pos, n_kept=nk,
                               workspace=ws)
        else:
            sp.sp_score(Q, K, out=imp, workspace=ws)
            sp.sp_select(imp, params, pos_base=3, kept_idx=kept, pos_ids=pos, n_kept=nk)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()  # (a call on the side stream before capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    for rep in range(6):
        # eager work between replays: the next keys, every output overwritten
        # and (refill) the workspace
        K.copy_(Ks[rep % 2])
        imp_e, kept_e, pos_e, ne = eager[rep % 2]
        imp.fill_(-1.0)
        kept.fill_(-1)
        pos.fill_(-1)
        nk.fill_(-1)
        if refill:
            ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"M={M} fused={fused} refill={refill} replay {rep}", flush=True)
        assert torch.equal(imp, imp_e), rep
        assert int(nk.cpu()[0]) == ne, rep
        assert torch.equal(kept[:ne], kept_e[:ne]), rep
        assert torch.equal(pos[:ne], pos_e[:ne]), rep
        assert not sp.sp_score_status(ws), rep
