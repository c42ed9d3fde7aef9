"""sp_select of one long prompt by several workgroups (given a workspace, at
49152 tokens or more, min-max normalisation) gives, bit for bit, what one
workgroup gives: the kept indices, position ids and count, over score
distributions with ties, both selection modes, boosts, a short last chunk
and the longest prompts; a wait that gives up leaves n_kept = -1, and the
next call is right."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402

CASES = [
    # id, M, selection
    ("49152-topk", 49152, dict(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)),
    ("60001-mass-boosts-short-chunk", 60001,
     dict(chunk=24, pool_k=5, mode="mass", mass=0.85, boost_first_n=100, boost_first_mult=1.5,
          boost_last_n=70, boost_last_mult=1.25)),
    ("65536-topk", 65536, dict(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)),
    ("131072-topk", 131072, dict(chunk=64, pool_k=13, mode="topk", keep_rate=0.1)),
    ("142792-mass-chunk28", 142792, dict(chunk=28, pool_k=3, mode="mass", mass=0.9)),
    # more workgroups (24) than chunks (13): some shares are empty
    ("49153-topk-chunk4096", 49153, dict(chunk=4096, pool_k=3, mode="topk", keep_rate=0.3)),
    ("50000-mass-chunk16", 50000, dict(chunk=16, pool_k=1, mode="mass", mass=0.5)),
]
DISTS = ["powered", "ties", "constant"]


def scores(M, dist, seed):
    rng = np.random.default_rng(seed)
    if dist == "powered":
        x = rng.random(M) ** 4
    elif dist == "ties":
        x = rng.integers(0, 7, M) / 7.0  # few distinct values: many equal chunk keys
    else:
        x = np.full(M, 0.25)
    return torch.from_numpy(x.astype(np.float32)).cuda()


@pytest.mark.parametrize("dist", DISTS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_select_by_several_workgroups_matches_one(case, dist):
    name, M, sel = case
    print(f"case {name} {dist}", flush=True)
    params = sp.select_params(**sel)
    assert sp.sp_select_workspace_bytes(1, M, params) > 0
    x = scores(M, dist, seed=M)
    k1, p1, n1 = sp.sp_select(x, params, pos_base=5, workspace=False)
    torch.cuda.synchronize()
    nk = int(n1.cpu()[0])
    assert nk > 0
    for rep in range(2):
        k2, p2, n2 = sp.sp_select(x, params, pos_base=5)
        torch.cuda.synchronize()
        assert int(n2.cpu()[0]) == nk, (name, dist, rep)
        assert torch.equal(k2[:nk], k1[:nk]), (name, dist, rep)
        assert torch.equal(p2[:nk], p1[:nk]), (name, dist, rep)


def test_select_by_several_workgroups_rejects_non_finite_scores():
    M = 60000
    params = sp.select_params(chunk=32, pool_k=5, mode="topk", keep_rate=0.2)
    for bad in (np.nan, np.inf, -np.inf):
        x = scores(M, "powered", seed=3)
        x[51234] = float(bad)
        _, _, n = sp.sp_select(x, params)
        torch.cuda.synchronize()
        assert int(n.cpu()[0]) == -1, bad


def test_select_by_several_workgroups_wait_limit():
    M = 65536
    params = sp.select_params(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)
    x = scores(M, "powered", seed=4)
    ref_k, _, ref_n = sp.sp_select(x, params, workspace=False)
    torch.cuda.synchronize()
    nk = int(ref_n.cpu()[0])
    print("case select wait limit", flush=True)
    try:
        sp.sp_set_wait_limit(1)  # every wait gives up at once (unless its data is already there)
        for _ in range(3):
            k, _, n = sp.sp_select(x, params)
            torch.cuda.synchronize()
            got = int(n.cpu()[0])
            assert got == -1 or (got == nk and torch.equal(k[:nk], ref_k[:nk]))
    finally:
        sp.sp_set_wait_limit(0)
    k, _, n = sp.sp_select(x, params)
    torch.cuda.synchronize()
    assert int(n.cpu()[0]) == nk and torch.equal(k[:nk], ref_k[:nk])
