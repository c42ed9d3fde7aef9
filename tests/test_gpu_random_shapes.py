"""Parity on seeded random shapes and selection settings, beyond the listed
cases: head-group size, look-ahead steps, head dimension, operand type,
layer and kv-head counts and prompt length drawn at random within what the
kernels implement (G a power of two, G * N <= 32, d in {64, 128}); each
case's importance is compared with the oracle's (the same bounds as the
listed cases) and then selected with random chunking, pooling, mode and
boosts (bit-exact against the oracle on the GPU's importance)."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402
from test_gpu_parity import check_importance, to_dev  # noqa: E402


def _cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        N = int(rng.integers(1, 32 // G + 1)) if G < 32 else 1
        N = min(N, 16)
        d = int(rng.choice([64, 128]))
        dt = synth.BF16 if rng.random() < 0.7 else synth.F32
        L = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 4))
        M = int(np.exp(rng.uniform(0, np.log(4000))))
        sel = dict(chunk=int(rng.choice([8, 16, 32, 64])), pool_k=int(rng.choice([1, 3, 5, 13])),
                   mode=str(rng.choice(["topk", "mass"])), keep_rate=float(rng.uniform(0.05, 0.5)),
                   mass=float(rng.uniform(0.5, 0.95)))
        if rng.random() < 0.5:
            sel.update(boost_first_n=int(rng.integers(0, 80)), boost_first_mult=float(rng.uniform(1, 2)),
                       boost_last_n=int(rng.integers(0, 80)), boost_last_mult=float(rng.uniform(1, 2)))
        out.append((f"r{i}-{'bf16' if dt == synth.BF16 else 'f32'}-d{d}-G{G}-N{N}-L{L}-Hkv{Hkv}-M{M}",
                    L, G * Hkv, Hkv, d, N, M, dt, i, sel))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_shape_score_and_select(case):
    name, L, H, Hkv, d, N, M, dt, seed, sel = case
    print(f"case {name} {sel}", flush=True)
    w = synth.Workload("case", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=100 + seed, M=M,
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, _ = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    check_importance(imp.cpu().numpy(), oracle.score(Qh, Kh), name)
    params = sp.select_params(**sel)
    kept, pos, n = sp.sp_select(imp, params, pos_base=7)
    torch.cuda.synchronize()
    k_ref, p_ref = oracle.select(imp.cpu().numpy(), pos_base=7, **sel)
    nk = int(n.cpu()[0])
    assert nk == len(k_ref), name
    assert np.array_equal(kept[:nk].cpu().numpy(), k_ref), name
    assert np.array_equal(pos[:nk].cpu().numpy(), p_ref), name


def _ragged_cases(n=6, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i, (name, L, H, Hkv, d, N, M, dt, s, sel) in enumerate(_cases(n, seed)):
        R = int(rng.integers(2, 7))
        lens = [int(np.exp(rng.uniform(0, np.log(3000)))) for _ in range(R)]
        out.append((f"ragged{i}-R{R}-" + name.split("-", 1)[1].rsplit("-M", 1)[0], L, H, Hkv, d, N, lens,
                    dt, s, sel))
    return out


RAGGED = _ragged_cases()


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_random_ragged_batch(case):
    """Every request of a random ragged batch (sp_score_varlen, then
    sp_select_varlen with per-request position bases) against the oracle on
    that request's own slices of the packed arrays."""
    name, L, H, Hkv, d, N, lens, dt, seed, sel = case
    print(f"case {name} lens {lens} {sel}", flush=True)
    w = synth.Workload("case", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=200 + seed, M=max(lens),
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, cu = synth.make_ragged(w, lens)
    imp = sp.sp_score_varlen(to_dev(Qh), to_dev(Kh), cu)
    torch.cuda.synchronize()
    imp_h = imp.cpu().numpy()
    ck = np.concatenate([[0], np.cumsum(np.asarray(lens) + N)])
    for r in range(len(lens)):
        ref = oracle.score(Qh[r], np.ascontiguousarray(Kh[:, :, ck[r]:ck[r + 1], :]))
        check_importance(imp_h[cu[r]:cu[r + 1]], ref, f"{name} r={r}")
    pos_base = [(5 * r + 3) % 11 for r in range(len(lens))]
    kept, pos, n = sp.sp_select_varlen(imp, cu, sp.select_params(**sel), pos_base=pos_base)
    torch.cuda.synchronize()
    kept_h, pos_h, n_h = kept.cpu().numpy(), pos.cpu().numpy(), n.cpu().numpy()
    for r in range(len(lens)):
        k_ref, p_ref = oracle.select(imp_h[cu[r]:cu[r + 1]], pos_base=pos_base[r], base_index=int(cu[r]),
                                     **sel)
        off = int(cu[r])
        assert n_h[r] == len(k_ref), (name, r)
        assert np.array_equal(kept_h[off:off + n_h[r]], k_ref), (name, r)
        assert np.array_equal(pos_h[off:off + n_h[r]], p_ref), (name, r)


def _window_cases(n=6, seed=91):
    rng = np.random.default_rng(seed)
    out = []
    for i, (name, L, H, Hkv, d, N, M, dt, s, sel) in enumerate(_cases(n, seed)):
        M = int(rng.integers(1, 6000))
        window = int(rng.integers(1, 2500))
        stride = int(rng.integers(1, window + 1))
        if M // stride > 60:  # (keep the window count, and so the oracle's work, small)
            stride = max(stride, -(-M // 60))
            window = max(window, stride)
        out.append((f"win{i}-M{M}-w{window}-s{stride}-" + name.split("-", 1)[1].rsplit("-M", 1)[0],
                    L, H, Hkv, d, N, M, window, stride, dt, s))
    return out


WINDOWS = _window_cases()


@pytest.mark.parametrize("case", WINDOWS, ids=[c[0] for c in WINDOWS])
def test_random_sliding_windows(case):
    """Random window layouts: the library's layout equals the oracle's, and
    sp_score_windows equals the oracle scoring each window from its own
    arrays and keeping its first keeps[r] scores."""
    name, L, H, Hkv, d, N, M, window, stride, dt, seed = case
    print(f"case {name}", flush=True)
    starts, lens, keeps = sp.sp_window_layout(M, window, stride)
    assert [tuple(x) for x in zip(starts, lens, keeps)] == oracle.window_layout(M, window, stride)
    w = synth.Workload("case", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=300 + seed, R=len(lens),
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, cu = synth.make_ragged(w, lens)
    imp = sp.sp_score_windows(to_dev(Qh), to_dev(Kh), cu, keeps)
    torch.cuda.synchronize()
    ck = np.concatenate([[0], np.cumsum(np.asarray(lens) + N)])
    Qs = [Qh[r] for r in range(len(lens))]
    Ks = [np.ascontiguousarray(Kh[:, :, ck[r]:ck[r + 1], :]) for r in range(len(lens))]
    imp_h = imp.cpu().numpy()
    assert imp_h.shape == (M,)
    check_importance(imp_h, oracle.score_windows(Qs, Ks, keeps), name)
