"""The hot path under HIP graph capture: sp_score + sp_select captured once
(torch.cuda.CUDAGraph on the capture stream) and replayed several times,
with eager work that overwrites the outputs between replays; every replay
must reproduce the eager call bit for bit (the scoring kernel is
deterministic; a launch's epoch is fixed into the graph, so a clearing kernel
captured before it resets the workspace's tagged words on every replay, with
no memset nodes in the graph)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402
from test_gpu_parity import to_dev  # noqa: E402


@pytest.mark.parametrize("M", [3000, 20000])
def test_graph_replays_match_eager(M):
    w = synth.Workload("case", L=2, H=8, Hkv=2, d=128, N=8, dtype=synth.BF16, seed=9, M=M,
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N)
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device="cuda")
    params = sp.select_params(chunk=32, pool_k=5, mode="mass", mass=0.8, boost_first_n=16,
                              boost_first_mult=1.5)
    imp_e = sp.sp_score(Q, K, out=torch.empty(M, dtype=torch.float32, device="cuda"), workspace=ws)
    kept_e, pos_e, n_e = sp.sp_select(imp_e, params, pos_base=3)
    torch.cuda.synchronize()
    ne = int(n_e.cpu()[0])

    imp = torch.empty(M, dtype=torch.float32, device="cuda")
    kept = torch.empty(M, dtype=torch.int32, device="cuda")
    pos = torch.empty(M, dtype=torch.int32, device="cuda")
    nk = torch.empty(1, dtype=torch.int32, device="cuda")

    def body():
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
    for rep in range(4):
        # eager work between replays: overwrite every output and the workspace
        imp.fill_(-1.0)
        kept.fill_(-1)
        pos.fill_(-1)
        nk.fill_(-1)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"M={M} replay {rep}", flush=True)
        assert torch.equal(imp, imp_e), rep
        assert int(nk.cpu()[0]) == ne, rep
        assert torch.equal(kept[:ne], kept_e[:ne]), rep
        assert torch.equal(pos[:ne], pos_e[:ne]), rep
        assert not sp.sp_score_status(ws), rep
