"""Ragged batches whose requests share launches (sp_score_varlen packs requests
of similar length into one launch, each on its own share of the CUs with its
own plan and workspace region). Every request's scores are checked against
the oracle (tolerances as in test_gpu_parity), against sp_score of the same
request alone (bit for bit where the request has a launch to itself; within
the tolerance where it shares one: its split over workgroups differs), and a
packed call captured in a HIP graph must replay bit for bit."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402
from test_gpu_parity import ABS_TOL, check_importance, to_dev  # noqa: E402

BF, F32 = synth.BF16, synth.F32

CASES = [
    # id, L, H, Hkv, d, N, dtype, prompt lengths
    ("bf16-d128-units16", 4, 16, 4, 128, 8, BF, [3000, 2000, 2500, 4000, 1, 5, 9000, 3]),
    ("bf16-d128-units64", 8, 32, 8, 128, 8, BF, [3000, 2000, 2500, 4000, 1, 5, 9000, 12000, 700]),
    ("f32-d128", 4, 16, 4, 128, 8, F32, [3000, 2000, 2500, 4000, 777]),
    ("f32-d64", 4, 16, 4, 64, 8, F32, [3000, 2000, 2500, 4000]),
    ("bf16-d64-G1", 4, 8, 8, 64, 4, BF, [3000, 2000, 2500, 4000]),
    ("bf16-d128-G1-N32", 4, 4, 4, 128, 32, BF, [3000, 2000, 2500, 4000]),
    ("8b-shape", 32, 32, 8, 128, 8, BF, [4096, 3000, 5000, 4500, 1, 2, 3, 6000, 100]),
    # four long prompts in one launch, about 64 CUs each (the 24000-token one
    # needs 43 workgroups per unit: one group)
    ("8b-shape-4x-long", 32, 32, 8, 128, 8, BF, [20000, 18000, 24000, 22000]),
    # eight requests in one launch
    ("8b-shape-8-short", 32, 32, 8, 128, 8, BF, [2048, 2000, 1900, 2100, 2048, 1500, 1800, 2047, 3000]),
    ("bf16-d128-units16-8", 4, 16, 4, 128, 8, BF, [3000, 2000, 2500, 4000, 3500, 2200, 2700, 3900]),
]


def _layout(lens, N):
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    cu_keys = np.concatenate([[0], np.cumsum(np.asarray(lens) + N)])
    return cu, cu_keys


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_packed_batch_matches_oracle_and_single_calls(case):
    name, L, H, Hkv, d, N, dt, lens = case
    print(f"case {name} lens={lens}", flush=True)
    desc = sp.score_desc(L, H, Hkv, d, N, sp.SP_BF16 if dt == BF else sp.SP_F32)
    cu, cu_keys = _layout(lens, N)
    launch = sp.sp_score_batch_plan(desc, cu, sp.sp_score_batch_workspace_bytes(desc, cu))
    shared = [int((launch == launch[r]).sum()) > 1 for r in range(len(lens))]
    assert any(shared), (name, launch)  # (the case must exercise a shared launch)
    w = synth.Workload(name, L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=41, R=len(lens),
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, cu2 = synth.make_ragged(w, lens)
    assert np.array_equal(cu, cu2)
    Q, K = to_dev(Qh), to_dev(Kh)
    ws = torch.empty(sp.sp_score_batch_workspace_bytes(desc, cu), dtype=torch.uint8, device="cuda")
    imp = sp.sp_score_varlen(Q, K, cu, workspace=ws)
    assert not sp.sp_score_status(ws)
    imp_h = imp.cpu().numpy()
    for r, M in enumerate(lens):
        k = np.ascontiguousarray(Kh[:, :, cu_keys[r]:cu_keys[r + 1]])
        got = imp_h[cu[r]:cu[r + 1]]
        check_importance(got, oracle.score(Qh[r], k), f"{name} r={r} M={M} shared={shared[r]}")
        alone = sp.sp_score(Q[r], to_dev(k), M).cpu().numpy()
        if shared[r]:
            assert np.max(np.abs(got.astype(np.float64) - alone)) <= ABS_TOL, r
        else:
            assert np.array_equal(got, alone), r


def test_packed_windows_match_oracle():
    """Windows of one prompt are of one length: they share launches."""
    L, H, Hkv, d, N, M, window, stride = 8, 32, 8, 128, 8, 9000, 2000, 1000
    starts, lens, keeps = sp.sp_window_layout(M, window, stride)
    desc = sp.score_desc(L, H, Hkv, d, N)
    cu, cu_keys = _layout(lens, N)
    launch = sp.sp_score_batch_plan(desc, cu, sp.sp_score_batch_workspace_bytes(desc, cu))
    print(f"windows lens={lens.tolist()} launches={launch.tolist()}", flush=True)
    assert int(launch.max()) + 1 < len(lens)
    w = synth.Workload("win", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=BF, seed=43, R=len(lens),
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_ragged(w, lens)
    Q, K = to_dev(Qh), to_dev(Kh)
    imp = sp.sp_score_windows(Q, K, cu, keeps).cpu().numpy()
    Qs = [Qh[r] for r in range(len(lens))]
    Ks = [np.ascontiguousarray(Kh[:, :, cu_keys[r]:cu_keys[r + 1]]) for r in range(len(lens))]
    check_importance(imp, oracle.score_windows(Qs, Ks, keeps), "packed windows")


@pytest.mark.parametrize("refill", [True, False], ids=["ws-overwritten", "ws-kept"])
def test_packed_batch_graph_replays_match_eager(refill):
    """A packed sp_score_varlen captured once and replayed, the keys alternating
    between two sets and the outputs (and, refill, the workspace) overwritten
    between replays: the clearing kernels captured before the launch reset
    every request's workspace region."""
    L, H, Hkv, d, N = 8, 32, 8, 128, 8
    lens = [3000, 2000, 2500, 4000, 1, 5]
    desc = sp.score_desc(L, H, Hkv, d, N)
    cu, _ = _layout(lens, N)
    launch = sp.sp_score_batch_plan(desc, cu, sp.sp_score_batch_workspace_bytes(desc, cu))
    assert int(launch.max()) + 1 < len(lens)
    mk = lambda seed: synth.make_ragged(synth.Workload("g", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=BF, seed=seed,
                                                       R=len(lens), plant_frac=0.05, plant_chunk=32), lens)
    Qh, Kh1, _ = mk(45)
    _, Kh2, _ = mk(46)
    Q = to_dev(Qh)
    Ks = [to_dev(Kh1), to_dev(Kh2)]
    ws = torch.empty(sp.sp_score_batch_workspace_bytes(desc, cu), dtype=torch.uint8, device="cuda")
    eager = []
    for Kx in Ks:
        e = sp.sp_score_varlen(Q, Kx, cu, workspace=ws)
        torch.cuda.synchronize()
        eager.append(e)
    assert not torch.equal(eager[0], eager[1])
    K = Ks[0].clone()
    imp = torch.empty(int(cu[-1]), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sp.sp_score_varlen(Q, K, cu, out=imp, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp.sp_score_varlen(Q, K, cu, out=imp, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(6):
        K.copy_(Ks[rep % 2])
        imp.fill_(-1.0)
        if refill:
            ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"packed graph refill={refill} replay {rep}", flush=True)
        assert torch.equal(imp, eager[rep % 2]), rep
        assert not sp.sp_score_status(ws), rep


def test_packed_batch_cooperative_launch_matches():
    """The packed launches as cooperative launches: the same schedule and plans,
    so the same scores bit for bit."""
    L, H, Hkv, d, N = 8, 32, 8, 128, 8
    lens = [3000, 2000, 2500, 4000, 1, 5, 9000]
    desc = sp.score_desc(L, H, Hkv, d, N)
    cu, _ = _layout(lens, N)
    launch = sp.sp_score_batch_plan(desc, cu, sp.sp_score_batch_workspace_bytes(desc, cu))
    assert int(launch.max()) + 1 < len(lens)
    w = synth.Workload("coop", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=BF, seed=47, R=len(lens),
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_ragged(w, lens)
    Q, K = to_dev(Qh), to_dev(Kh)
    print("packed batch, cooperative launch", flush=True)
    a = sp.sp_score_varlen(Q, K, cu)
    b = sp.sp_score_varlen(Q, K, cu, launch=sp.SP_LAUNCH_COOPERATIVE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
