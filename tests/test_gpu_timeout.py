"""The time-out path of the scoring kernel's bounded waits, forced from the
host: with a tiny wait limit (sp_set_wait_limit) the waits give up at once and
every kernel still ends normally. The call must then report the time-out
(sp_score_status), its scores must be NaN (not a plausible array), and the
selection must answer n_kept = -1 instead of a kept set. The next call with
the default limit must be complete and correct again. Also: the selection
rejects non-finite scores in every mode."""
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


def _workload(M, seed=31):
    return synth.Workload("timeout", L=8, H=32, Hkv=8, d=128, N=8, dtype=synth.BF16, seed=seed,
                          M=M, plant_frac=0.05)


@pytest.fixture
def restore_limit():
    yield
    sp.sp_set_wait_limit(0)


def test_timed_out_call_is_reported_and_poisoned(restore_limit):
    w = _workload(6000)
    Qh, Kh, M = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    params = sp.select_params(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)
    print("case timeout M=6000 wait limit 1 tick", flush=True)
    sp.sp_set_wait_limit(1)
    ws = torch.empty(sp.sp_score_workspace_bytes(sp.score_desc(8, 32, 8, 128, 8), M),
                     dtype=torch.uint8, device="cuda")
    imp = sp.sp_score(Q, K, workspace=ws)
    assert sp.sp_score_status(ws) is True
    imp_h = imp.cpu().numpy()
    assert np.isnan(imp_h).any()
    _, _, n = sp.sp_select(imp, params)
    assert int(n.cpu()[0]) == -1
    # default limit: complete, finite and right
    sp.sp_set_wait_limit(0)
    imp = sp.sp_score(Q, K, workspace=ws)
    assert sp.sp_score_status(ws) is False
    ref = oracle.score(Qh, Kh)
    got = imp.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) <= 2e-3


def test_timed_out_ragged_call_is_reported(restore_limit):
    """A time-out in any request of a ragged call is reported: the error word is
    tagged with the call's number, which all its requests share."""
    lens = np.array([3000, 2000], np.int64)
    w = synth.Workload("timeout", L=8, H=32, Hkv=8, d=128, N=8, dtype=synth.BF16, seed=33,
                       R=2, len_range=(2000, 3000, 1000), plant_frac=0.05)
    Qh, Kh, cu = synth.make_ragged(w, lens)
    Q, K = to_dev(Qh), to_dev(Kh)
    print("case timeout ragged R=2", flush=True)
    sp.sp_set_wait_limit(1)
    ws = torch.empty(sp.sp_score_workspace_bytes(sp.score_desc(8, 32, 8, 128, 8), 3000),
                     dtype=torch.uint8, device="cuda")
    imp = sp.sp_score_varlen(Q, K, cu, workspace=ws)
    assert sp.sp_score_status(ws) is True
    params = sp.select_params(chunk=32, pool_k=13, mode="mass", mass=0.85)
    _, _, n = sp.sp_select_varlen(imp, cu, params)
    assert (n.cpu().numpy() == -1).any()
    sp.sp_set_wait_limit(0)
    imp = sp.sp_score_varlen(Q, K, cu, workspace=ws)
    assert sp.sp_score_status(ws) is False
    got = imp.cpu().numpy().astype(np.float64)
    for r in range(2):
        ref = oracle.score(Qh[r], Kh[:, :, cu[r] + r * 8: cu[r + 1] + (r + 1) * 8])
        assert np.max(np.abs(got[cu[r]:cu[r + 1]] - ref)) <= 2e-3


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
@pytest.mark.parametrize("mode", ["topk", "mass", "threshold"])
def test_select_rejects_non_finite_scores(bad, mode):
    rng = np.random.default_rng(5)
    x = rng.random(5000).astype(np.float32)
    x[1234] = bad
    kw = dict(chunk=32, pool_k=1 if mode == "threshold" else 5, mode=mode, keep_rate=0.3,
              mass=0.85 if mode == "mass" else 0.0)
    if mode == "threshold":
        kw.update(min_tok=128, max_keep=0)
    params = sp.select_params(**kw)
    xt = torch.from_numpy(x).cuda()
    kept = torch.full((5000,), 7, dtype=torch.int32, device="cuda")
    _, _, n = sp.sp_select(xt, params, kept_idx=kept)
    assert int(n.cpu()[0]) == -1
    assert bool((kept == 7).all().cpu())  # outputs untouched
    # ragged: only the request holding the bad score answers -1
    cu = [0, 1000, 5000]
    _, _, n2 = sp.sp_select_varlen(xt, cu, params)
    assert n2.cpu().numpy().tolist()[0] > 0 and n2.cpu().numpy().tolist()[1] == -1
