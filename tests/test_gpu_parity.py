"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same
seeded inputs.

Tolerances. Importance: max-abs <= 2e-3 (the target's stated bound), and in
addition an element-wise relative bound of 1e-3 derived from the arithmetic:
bf16 x bf16 products are exact in fp32, the fp32 MFMA accumulation of d = 128
terms bounds the logit error by about d * 2^-24 * sum|q_t k_t| * scale
(< 1e-4 on these inputs), and p = exp2(s*c - lse) turns an absolute logit
error e into a relative error of about 2e when the row's log-sum-exp carries a
similar error; the hardware exp2/log2 add ~1e-7. 1e-3 leaves a 5x margin and
still catches semantic slips the absolute bound would miss (a softmax over the
wrong number of keys changes every probability by (M+j+1)/(M+N) - 1, which is
~4e-3 at M = 1000). Selection: bit-exact (kept indices, position ids, count)
when the oracle's selection is fed the GPU's float32 importance array.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402

ABS_TOL = 2e-3
REL_TOL = 1e-3


def to_dev(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def check_importance(gpu: np.ndarray, ref: np.ndarray, label: str):
    gpu = gpu.astype(np.float64)
    assert gpu.shape == ref.shape, label
    assert np.all(np.isfinite(gpu)), label
    abs_err = np.max(np.abs(gpu - ref))
    rel = np.abs(gpu - ref) / np.maximum(ref, 1e-30)
    worst = int(np.argmax(rel))
    print(f"[{label}] max-abs {abs_err:.3e}  max-rel {rel[worst]:.3e} at {worst}", flush=True)
    assert abs_err <= ABS_TOL, label
    assert rel[worst] <= REL_TOL, (label, worst, gpu[worst], ref[worst])


def check_selection(imp_gpu_t, sel, label, pos_base=0):
    params = sp.select_params(**oracle.select_params(sel))
    kept, pos, n = sp.sp_select(imp_gpu_t, params, pos_base=pos_base)
    torch.cuda.synchronize()
    imp_h = imp_gpu_t.cpu().numpy()
    k_ref, p_ref = oracle.select(imp_h, pos_base=pos_base, **oracle.select_params(sel))
    nk = int(n.cpu()[0])
    print(f"[{label}] kept {nk} tokens ({sel.mode})", flush=True)
    assert nk == len(k_ref), label
    assert np.array_equal(kept[:nk].cpu().numpy(), k_ref), label
    assert np.array_equal(pos[:nk].cpu().numpy(), p_ref), label
    return nk


def workload(L, H, Hkv, d, N, M, dtype, seed=11, plant_chunk=32):
    return synth.Workload("case", L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dtype, seed=seed, M=M,
                          plant_frac=0.05, plant_chunk=plant_chunk)


BF, F32 = synth.BF16, synth.F32

SMALL_CASES = [
    # id, L, H, Hkv, d, N, M, dtype
    ("bf16-d128-G4-N8-M1000", 2, 8, 2, 128, 8, 1000, BF),
    ("bf16-d128-G4-N8-M4100", 2, 8, 2, 128, 8, 4100, BF),
    ("bf16-d128-G4-N8-M20000", 1, 8, 2, 128, 8, 20000, BF),
    ("bf16-d64-G2-N8-M777", 3, 4, 2, 64, 8, 777, BF),
    ("bf16-d64-G2-N8-M5000", 2, 4, 2, 64, 8, 5000, BF),
    ("f32-d64-G2-N8-M1024", 2, 4, 2, 64, 8, 1024, F32),
    ("f32-d128-G4-N8-M300", 2, 8, 2, 128, 8, 300, F32),
    ("f32-d64-G4-N8-M2100", 1, 8, 2, 64, 8, 2100, F32),
    ("bf16-d128-G1-N16-M513", 2, 4, 4, 128, 16, 513, BF),
    ("bf16-d128-G8-N4-M2000", 1, 16, 2, 128, 4, 2000, BF),
    ("bf16-d64-G16-N2-M900", 1, 16, 1, 64, 2, 900, BF),
    ("bf16-d128-G32-N1-M700", 1, 32, 1, 128, 1, 700, BF),
    ("bf16-d128-G4-N6-M999", 2, 8, 2, 128, 6, 999, BF),
    ("bf16-d64-G1-N3-M1", 1, 2, 2, 64, 3, 1, BF),
    ("bf16-d64-G2-N1-M17", 2, 4, 2, 64, 1, 17, BF),
    ("bf16-d128-G2-N4-M33", 3, 4, 2, 128, 4, 33, BF),
]


# Shapes with many (layer, kv-head) units per group of workgroups, for each
# tile configuration (bf16/f32 x 16/32 query rows, base and deeper slices):
# these exercise the pipeline across units (the K ring running two units
# ahead, parked logits cycling through their LDS banks, deferred finishing),
# which one-unit-per-group shapes never reach.
MULTI_UNIT_CASES = [
    ("multi-bf16-d128-rows32", 32, 32, 8, 128, 8, 4100, BF),
    ("multi-bf16-d64-rows16", 32, 16, 8, 64, 8, 5000, BF),
    ("multi-f32-d64-rows16", 32, 16, 8, 64, 8, 6000, F32),
    ("multi-f32-d128-rows32", 32, 32, 8, 128, 8, 3000, F32),
]


@pytest.mark.parametrize("case", MULTI_UNIT_CASES, ids=[c[0] for c in MULTI_UNIT_CASES])
def test_score_several_units_per_group(case):
    name, L, H, Hkv, d, N, M, dt = case
    print(f"case {name}", flush=True)
    plan = sp.sp_score_plan(sp.score_desc(L, H, Hkv, d, N, sp.SP_BF16 if dt else sp.SP_F32), M)
    assert plan["units"] >= 8 * plan["ngroups"], plan
    w = workload(L, H, Hkv, d, N, M, dt, seed=13)
    Qh, Kh, _ = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    check_importance(imp.cpu().numpy(), oracle.score(Qh, Kh), name)


# Shapes whose cross-group merge takes the batch shapes the other cases do not:
# at least 9 other groups with more than 512 values for some workgroup (4 values
# per thread, 15 groups per batch), and more than 30 other groups (1 value per
# thread, 60 groups per batch). (ngroups, values) follow from the plan: a
# workgroup's share of its slice is ceil(keys / ngroups), times N steps.
MERGE_CASES = [
    ("merge-4x15-bf16-d64-N16", 8, 16, 8, 64, 16, 8192, BF, lambda ng, vals: ng >= 10 and max(vals) > 512),
    ("merge-1x60-bf16-d128", 8, 32, 8, 128, 8, 3000, BF, lambda ng, vals: ng >= 32 and max(vals) <= 512),
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_score_cross_group_merge_shapes(case):
    name, L, H, Hkv, d, N, M, dt, covers = case
    print(f"case {name}", flush=True)
    plan = sp.sp_score_plan(sp.score_desc(L, H, Hkv, d, N, sp.SP_BF16 if dt else sp.SP_F32), M)
    ng, g, kr = plan["ngroups"], plan["g"], plan["keys_per_wg"]
    vals = [N * -(-max(min(r * kr + kr, M + N, M) - r * kr, 0) // ng) for r in range(g)]
    assert covers(ng, vals), (plan, vals)
    w = workload(L, H, Hkv, d, N, M, dt, seed=17)
    Qh, Kh, _ = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    check_importance(imp.cpu().numpy(), oracle.score(Qh, Kh), name)


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_score_small_shapes(case):
    name, L, H, Hkv, d, N, M, dt = case
    print(f"case {name}", flush=True)
    w = workload(L, H, Hkv, d, N, M, dt)
    Qh, Kh, _ = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    check_importance(imp.cpu().numpy(), oracle.score(Qh, Kh), name)


def test_score_peaked_logits_with_explicit_scale():
    """scale = 1 on the planted data gives logits with std ~sqrt(d): rows are
    sharply peaked; the online statistics must stay stable."""
    w = workload(2, 8, 2, 128, 8, 1500, BF, seed=21)
    Qh, Kh, _ = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh), scale=1.0)
    torch.cuda.synchronize()
    ref = oracle.score(Qh, Kh, scale=1.0)
    gpu = imp.cpu().numpy().astype(np.float64)
    big = ref > 1e-6  # relative bound on the probabilities that carry signal
    assert np.max(np.abs(gpu - ref)) <= ABS_TOL
    assert np.max(np.abs(gpu[big] - ref[big]) / ref[big]) <= REL_TOL


def test_score_is_deterministic():
    w = workload(2, 8, 2, 128, 8, 3000, BF, seed=5)
    Qh, Kh, _ = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    a = sp.sp_score(Q, K)
    b = sp.sp_score(Q, K)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


COOP_CASES = [c for c in SMALL_CASES if c[0] in ("bf16-d128-G4-N8-M4100", "f32-d64-G2-N8-M1024",
                                                   "bf16-d64-G1-N3-M1")] + MULTI_UNIT_CASES[:2]


@pytest.mark.parametrize("case", COOP_CASES, ids=[c[0] for c in COOP_CASES])
def test_score_cooperative_launch_matches(case):
    """The two launch modes run the same kernel on the same plan: the scores
    are identical bit for bit, and match the oracle."""
    name, L, H, Hkv, d, N, M, dt = case
    print(f"case {name} (cooperative launch)", flush=True)
    w = workload(L, H, Hkv, d, N, M, dt, seed=17)
    Qh, Kh, _ = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    a = sp.sp_score(Q, K, launch=sp.SP_LAUNCH_COOPERATIVE)
    b = sp.sp_score(Q, K, launch=sp.SP_LAUNCH_RESIDENT)
    torch.cuda.synchronize()
    assert torch.equal(a, b), name
    check_importance(a.cpu().numpy(), oracle.score(Qh, Kh), name)


# The look-ahead keys M..M+N-1 are streamed by the last key slices, with a
# per-row causal mask (step j sees look-ahead keys up to M + j). Prompt
# lengths picked from each shape's plan put them at the slice boundaries:
# a last slice that holds only look-ahead keys, look-ahead keys split over
# two slices, and a slice that ends right after key M.
BOUNDARY_SHAPES = [
    ("bf16-d128-G4-N8", 2, 32, 8, 128, 8, BF),
    ("bf16-d128-G1-N16", 1, 4, 4, 128, 16, BF),
    ("f32-d64-G4-N8", 1, 8, 2, 64, 8, F32),
]


def _boundary_prompts(desc, N):
    """(M, kind) for the three placements, from the plans of M in 600..30000."""
    found = {}
    for M in range(600, 30000):
        p = sp.sp_score_plan(desc, M)
        kr = p["keys_per_wg"]
        for kind, hit in (("tail-only slice", M % kr == 0), ("tail split", M % kr == kr - 3),
                          ("slice ends after key M", (M + 1) % kr == 0)):
            if hit and kind not in found and (M + N + kr - 1) // kr == p["g"]:
                found[kind] = M
        if len(found) == 3:
            break
    return sorted((m, k) for k, m in found.items())


@pytest.mark.parametrize("shape", BOUNDARY_SHAPES, ids=[c[0] for c in BOUNDARY_SHAPES])
def test_score_lookahead_keys_at_slice_boundaries(shape):
    name, L, H, Hkv, d, N, dt = shape
    desc = sp.score_desc(L, H, Hkv, d, N, sp.SP_BF16 if dt else sp.SP_F32)
    cases = _boundary_prompts(desc, N)
    assert len(cases) == 3, cases
    for M, kind in cases:
        label = f"{name}-M{M} ({kind})"
        print(f"case {label}", flush=True)
        w = workload(L, H, Hkv, d, N, M, dt, seed=37)
        Qh, Kh, _ = synth.make_request(w)
        imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
        torch.cuda.synchronize()
        check_importance(imp.cpu().numpy(), oracle.score(Qh, Kh), label)


# The longest prompts the planner accepts: one workgroup per CU but one (the
# combiner's), each holding as many keys as its registers and LDS allow.
LONGEST_CASES = [
    ("longest-bf16-d128", 1, 4, 1, 128, 8, 142792, BF),
    ("longest-f32-d128", 1, 4, 1, 128, 8, 85672, F32),
]


@pytest.mark.parametrize("case", LONGEST_CASES, ids=[c[0] for c in LONGEST_CASES])
def test_score_longest_prompt(case):
    """g = CUs - 1 workgroups share the unit and a single combiner workgroup
    gathers their partials: the largest grid and the smallest combiner."""
    name, L, H, Hkv, d, N, M, dt = case
    print(f"case {name}", flush=True)
    desc = sp.score_desc(L, H, Hkv, d, N, sp.SP_BF16 if dt else sp.SP_F32)
    plan = sp.sp_score_plan(desc, M)
    assert plan["g"] == plan["cus"] - 1 and plan["grid"] == plan["cus"], plan
    with pytest.raises(sp.SpError):
        sp.sp_score_plan(desc, M + 1)
    w = workload(L, H, Hkv, d, N, M, dt, seed=29)
    Qh, Kh, _ = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    check_importance(imp.cpu().numpy(), oracle.score(Qh, Kh), name)


def test_score_status_after_a_normal_call():
    w = workload(2, 8, 2, 128, 8, 2000, BF, seed=6)
    Qh, Kh, M = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N)
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device="cuda")
    ws.fill_(0xff)  # (an error word left in the workspace must not count for this call)
    sp.sp_score(Q, K, workspace=ws)
    assert sp.sp_score_status(ws) is False


def test_score_workspace_too_small_is_rejected():
    w = workload(1, 4, 2, 64, 8, 500, BF)
    Qh, Kh, _ = synth.make_request(w)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(sp.SpError) as e:
        sp.sp_score(to_dev(Qh), to_dev(Kh), workspace=ws)
    assert e.value.status == sp.SP_EWORKSPACE


# ----------------------------------------------------------------------------------------
# the five workloads at full size
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "spec0.8b_m4608", "spec8b_m32k"])
def test_workload_full(name):
    w = synth.WORKLOADS[name]
    print(f"workload {name}: generating", flush=True)
    Qh, Kh, M = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    print(f"workload {name}: oracle", flush=True)
    ref = oracle.score(Qh, Kh)
    check_importance(imp.cpu().numpy(), ref, name)
    for sel in w.selects:
        nk = check_selection(imp, sel, name)
        if sel.mode == "topk" and M % sel.chunk == 0:
            nc = M // sel.chunk
            assert nk == max(1, math.ceil(np.float64(np.float32(sel.keep_rate)) * nc)) * sel.chunk


def test_workload_full_128k():
    w = synth.WORKLOADS["spec8b_m128k"]
    print("workload spec8b_m128k: generating", flush=True)
    Qh, Kh, M = synth.make_request(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    imp = sp.sp_score(Q, K)
    torch.cuda.synchronize()
    del Q, K
    print("workload spec8b_m128k: oracle", flush=True)
    ref = oracle.score(Qh, Kh)
    check_importance(imp.cpu().numpy(), ref, "spec8b_m128k")
    for sel in w.selects:
        check_selection(imp, sel, f"spec8b_m128k {sel.mode} {sel.keep_rate or sel.mass}")


def test_workload_ragged_batch():
    """All 16 requests scored in one varlen call; the oracle recomputes every
    request in full from its slices of the packed arrays (each request is
    independent of the others), and every request's selection is checked bit
    for bit."""
    w = synth.WORKLOADS["ragged16_8b"]
    print("workload ragged16_8b: generating", flush=True)
    Qh, Kh, cu = synth.make_ragged(w)
    Q, K = to_dev(Qh), to_dev(Kh)
    imp = sp.sp_score_varlen(Q, K, cu)
    torch.cuda.synchronize()
    del Q, K
    imp_h = imp.cpu().numpy()
    Ms = np.diff(cu)
    for r in range(len(Ms)):
        print(f"workload ragged16_8b: oracle for request {r} (M={Ms[r]})", flush=True)
        k0 = int(cu[r]) + r * w.N
        k = np.ascontiguousarray(Kh[:, :, k0:k0 + int(Ms[r]) + w.N])
        check_importance(imp_h[cu[r]:cu[r + 1]], oracle.score(Qh[r], k), f"ragged r={r}")
        del k
    del Kh
    assert np.all(np.isfinite(imp_h)) and np.all(imp_h >= 0) and np.all(imp_h <= 1)
    sel = w.selects[0]
    params = sp.select_params(**oracle.select_params(sel))
    pos_base = [(7 * r) % 5 for r in range(len(Ms))]
    kept, pos, n = sp.sp_select_varlen(imp, cu, params, pos_base=pos_base)
    torch.cuda.synchronize()
    kept_h, pos_h, n_h = kept.cpu().numpy(), pos.cpu().numpy(), n.cpu().numpy()
    for r in range(len(Ms)):
        k_ref, p_ref = oracle.select(imp_h[cu[r]:cu[r + 1]], pos_base=pos_base[r],
                                     base_index=int(cu[r]), **oracle.select_params(sel))
        assert n_h[r] == len(k_ref), r
        off = int(cu[r])
        assert np.array_equal(kept_h[off:off + n_h[r]], k_ref), r
        assert np.array_equal(pos_h[off:off + n_h[r]], p_ref), r


# ----------------------------------------------------------------------------------------
# selection on given score arrays (bit-exact against the oracle)
# ----------------------------------------------------------------------------------------
def _select_case(x: np.ndarray, pos_base=0, **kw):
    params = sp.select_params(**kw)
    t = torch.from_numpy(x.astype(np.float32)).cuda()
    kept, pos, n = sp.sp_select(t, params, pos_base=pos_base)
    torch.cuda.synchronize()
    k_ref, p_ref = oracle.select(x.astype(np.float32), pos_base=pos_base, **kw)
    nk = int(n.cpu()[0])
    assert nk == len(k_ref), kw
    assert np.array_equal(kept[:nk].cpu().numpy(), k_ref), kw
    assert np.array_equal(pos[:nk].cpu().numpy(), p_ref), kw
    return k_ref


def test_select_position_id_example():
    x = np.array([0.9, 0.8, 0.1, 0.7, 0.2, 0.3, 0.6, 0.5, 0.05, 0.15])
    k = _select_case(x, chunk=1, pool_k=1, mode="topk", keep_rate=0.5)
    assert k.tolist() == [0, 1, 3, 6, 7]


SELECT_CASES = [
    dict(M=32768, chunk=32, pool_k=13, mode="topk", keep_rate=0.1),
    dict(M=32768, chunk=8, pool_k=5, mode="mass", mass=0.85),       # nc = 4096
    dict(M=163840, chunk=32, pool_k=13, mode="topk", keep_rate=0.1),  # nc = 5120 (maximum)
    dict(M=163835, chunk=32, pool_k=5, mode="mass", mass=0.85),     # nc = 5120, ragged last chunk
    dict(M=142792, chunk=32, pool_k=13, mode="mass", mass=0.85, boost_first_n=64,
         boost_first_mult=1.5, boost_last_n=128, boost_last_mult=1.3),  # the longest scored prompt
    dict(M=4608, chunk=32, pool_k=5, mode="mass", mass=0.85, boost_first_n=64,
         boost_first_mult=1.5, boost_last_n=128, boost_last_mult=1.3),
    dict(M=1000, chunk=24, pool_k=3, mode="topk", keep_rate=0.3),     # chunk not a power of 2
    dict(M=5000, chunk=100, pool_k=7, mode="mass", mass=0.5),         # > 64, not a power of 2
    dict(M=9000, chunk=128, pool_k=3, mode="topk", keep_rate=0.25),   # > 64, power of 2
    dict(M=777, chunk=16, pool_k=41, mode="topk", keep_rate=0.2),     # wide pool
    dict(M=1, chunk=32, pool_k=3, mode="topk", keep_rate=0.1),
    dict(M=64, chunk=64, pool_k=1, mode="mass", mass=1.0),
    dict(M=300, chunk=7, pool_k=1, mode="topk", keep_rate=1.0),
    dict(M=2049, chunk=32, pool_k=3, mode="mass", mass=0.3, boost_first_n=100,
         boost_first_mult=2.0, boost_last_n=2000, boost_last_mult=0.5),
    dict(M=4096, chunk=1, pool_k=9, mode="topk", keep_rate=0.05),    # one token per chunk
    dict(M=200000, chunk=512, pool_k=3, mode="mass", mass=0.9),       # many staged tiles
    dict(M=50000, chunk=20000, pool_k=1, mode="topk", keep_rate=0.5), # three chunks, ragged last
    dict(M=1 << 24, chunk=4096, pool_k=5, mode="topk", keep_rate=0.3),  # the largest prompt
]


@pytest.mark.parametrize("dist", ["uniform", "ties", "constant", "spiky"])
@pytest.mark.parametrize("case", SELECT_CASES,
                         ids=[f"{c['M']}-{c['chunk']}-{c['mode']}" for c in SELECT_CASES])
def test_select_matches_oracle(case, dist):
    kw = dict(case)
    M = kw.pop("M")
    rng = np.random.default_rng(M + len(dist))
    if dist == "uniform":
        x = rng.random(M)
    elif dist == "ties":
        x = rng.integers(0, 4, M) / 3.0
    elif dist == "constant":
        x = np.full(M, 0.125)
    else:
        x = rng.random(M) ** 8 * 1e-3
    _select_case(x, pos_base=3, **kw)


# ----------------------------------------------------------------------------------------
# the last prompt token's query row as one more step (sp_score_lastrow)
# ----------------------------------------------------------------------------------------
def _lastrow_inputs(L, H, Hkv, d, N, M, dt, seed):
    """Q [L,H,N,d], Q_last [L,H,d] (the same generator with one more query row)
    and K [L,Hkv,M+N,d]."""
    wq = workload(L, H, Hkv, d, N + 1, M, dt, seed=seed)
    Qa = synth.make_q(wq)
    w = workload(L, H, Hkv, d, N, M, dt, seed=seed)
    Kh = synth.make_k(w, 0, M)
    return np.ascontiguousarray(Qa[:, :, :N]), np.ascontiguousarray(Qa[:, :, N]), Kh


LASTROW_CASES = [
    ("bf16-d128-G4-N8-M1000", 2, 8, 2, 128, 8, 1000, BF),
    ("bf16-d128-G4-N8-M1", 2, 8, 2, 128, 8, 1, BF),
    ("bf16-d64-G2-N8-M777", 3, 4, 2, 64, 8, 777, BF),
    ("f32-d64-G2-N8-M1024", 2, 4, 2, 64, 8, 1024, F32),
    ("f32-d128-G4-N8-M300", 2, 8, 2, 128, 8, 300, F32),
    ("bf16-d128-G8-N4-M2000", 1, 16, 2, 128, 4, 2000, BF),
    ("bf16-d128-G32-N1-M700", 1, 32, 1, 128, 1, 700, BF),
    ("multi-bf16-d128-rows32", 32, 32, 8, 128, 8, 4100, BF),
    ("multi-bf16-d64-rows16", 24, 16, 8, 64, 8, 4608, BF),
]


@pytest.mark.parametrize("case", LASTROW_CASES, ids=[c[0] for c in LASTROW_CASES])
def test_score_lastrow_matches_oracle(case):
    name, L, H, Hkv, d, N, M, dt = case
    print(f"case lastrow {name}", flush=True)
    Qh, Ql, Kh = _lastrow_inputs(L, H, Hkv, d, N, M, dt, seed=41)
    imp = sp.sp_score_lastrow(to_dev(Qh), to_dev(Ql), to_dev(Kh))
    torch.cuda.synchronize()
    check_importance(imp.cpu().numpy(), oracle.score_lastrow(Qh, Ql, Kh), f"lastrow {name}")


def test_score_lastrow_workload_8b_32k():
    """The 8B shape at M = 32768 with a last-row query: full comparison."""
    w = synth.WORKLOADS["spec8b_m32k"]
    print("lastrow spec8b_m32k: generating", flush=True)
    Qh, Ql, Kh = _lastrow_inputs(w.L, w.H, w.Hkv, w.d, w.N, w.M, w.dtype, seed=w.seed)
    imp = sp.sp_score_lastrow(to_dev(Qh), to_dev(Ql), to_dev(Kh))
    torch.cuda.synchronize()
    print("lastrow spec8b_m32k: oracle", flush=True)
    check_importance(imp.cpu().numpy(), oracle.score_lastrow(Qh, Ql, Kh), "lastrow 8b/32k")


# ----------------------------------------------------------------------------------------
# robust normalisations (percentile clip, clipped z-score): bit-exact against the oracle
# ----------------------------------------------------------------------------------------
NORM_CASES = [
    dict(M=32768, chunk=32, pool_k=13, mode="topk", keep_rate=0.1),
    dict(M=32768, chunk=32, pool_k=13, mode="mass", mass=0.85),
    dict(M=4608, chunk=32, pool_k=5, mode="mass", mass=0.85, boost_first_n=64,
         boost_first_mult=1.5, boost_last_n=128, boost_last_mult=1.3),
    dict(M=1000, chunk=24, pool_k=3, mode="topk", keep_rate=0.3),
    dict(M=1, chunk=32, pool_k=3, mode="topk", keep_rate=0.1),
    dict(M=77, chunk=4, pool_k=1, mode="mass", mass=0.6),
    dict(M=200000, chunk=512, pool_k=3, mode="mass", mass=0.9),
    dict(M=1 << 22, chunk=2048, pool_k=5, mode="topk", keep_rate=0.3),
]
NORMS = [("percentile", 0.01, 0.99), ("percentile", 0.0, 1.0), ("percentile", 0.25, 0.5),
         ("zscore", 0.0, 3.0), ("zscore", 0.0, 0.5)]


@pytest.mark.parametrize("dist", ["uniform", "ties", "constant", "outliers", "signed"])
@pytest.mark.parametrize("norm", NORMS, ids=[f"{n}-{lo}-{hi}" for n, lo, hi in NORMS])
@pytest.mark.parametrize("case", NORM_CASES,
                         ids=[f"{c['M']}-{c['chunk']}-{c['mode']}" for c in NORM_CASES])
def test_select_robust_norms_match_oracle(case, norm, dist):
    kw = dict(case)
    M = kw.pop("M")
    rng = np.random.default_rng(M + 7 * len(dist))
    if dist == "uniform":
        x = rng.random(M)
    elif dist == "ties":
        x = rng.integers(0, 4, M) / 3.0
    elif dist == "constant":
        x = np.full(M, 0.125)
    elif dist == "outliers":
        x = 0.01 + 0.01 * rng.random(M)
        x[rng.integers(0, M, max(1, M // 500))] = rng.random(max(1, M // 500)) * 50.0
    else:  # signed scores spanning many binades (not importance arrays, but valid input)
        x = rng.standard_normal(M) * np.exp2(rng.integers(-30, 30, M))
    n, lo, hi = norm
    _select_case(x, pos_base=5, norm=n, norm_lo=lo, norm_hi=hi, **kw)


def test_select_robust_norms_on_scored_workload():
    """The 0.8B workload's GPU importance under each robust normalisation, in
    both selection modes, and a ragged batch of its slices (per-request
    statistics)."""
    w = synth.WORKLOADS["spec0.8b_m4608"]
    Qh, Kh, M = synth.make_request(w)
    imp = sp.sp_score(to_dev(Qh), to_dev(Kh))
    torch.cuda.synchronize()
    x = imp.cpu().numpy()
    for n, lo, hi in NORMS:
        for kw in (dict(mode="mass", mass=0.85), dict(mode="topk", keep_rate=0.2)):
            _select_case(x, chunk=32, pool_k=5, norm=n, norm_lo=lo, norm_hi=hi,
                         boost_first_n=64, boost_first_mult=1.5, boost_last_n=128,
                         boost_last_mult=1.3, **kw)
    cu = [0, 1000, 1001, 3000, M]
    for n, lo, hi in NORMS:
        sel = dict(chunk=16, pool_k=3, mode="mass", mass=0.8, norm=n, norm_lo=lo, norm_hi=hi)
        kept, pos, nk = sp.sp_select_varlen(imp, cu, sp.select_params(**sel), pos_base=[0, 1, 2, 3])
        torch.cuda.synchronize()
        kh, ph, nh = kept.cpu().numpy(), pos.cpu().numpy(), nk.cpu().numpy()
        for r in range(4):
            k_ref, p_ref = oracle.select(x[cu[r]:cu[r + 1]], pos_base=r, base_index=cu[r], **sel)
            assert nh[r] == len(k_ref), (n, r)
            assert np.array_equal(kh[cu[r]:cu[r] + nh[r]], k_ref), (n, r)
            assert np.array_equal(ph[cu[r]:cu[r] + nh[r]], p_ref), (n, r)


# ----------------------------------------------------------------------------------------
# threshold selection (the Implementation Guide program's chunk selection and cap)
# ----------------------------------------------------------------------------------------
THRESH_CASES = [
    dict(M=10, chunk=1, keep_rate=0.5, min_tok=0, max_keep=0),
    dict(M=32768, chunk=32, keep_rate=0.3, min_tok=128, max_keep=0),
    dict(M=32768, chunk=32, keep_rate=0.3, min_tok=128, max_keep=2000),  # the Guide's defaults
    dict(M=4608, chunk=32, keep_rate=0.1, min_tok=128, max_keep=0),
    dict(M=200, chunk=10, keep_rate=0.05, min_tok=128, max_keep=0),      # the fill
    dict(M=3, chunk=1, keep_rate=0.3, min_tok=0, max_keep=0),
    dict(M=5, chunk=5, keep_rate=0.5, min_tok=0, max_keep=0),
    dict(M=4, chunk=1, keep_rate=0.3, min_tok=128, max_keep=0),         # M <= eff_min
    dict(M=8, chunk=3, keep_rate=0.4, min_tok=128, max_keep=3),
    dict(M=1000, chunk=24, keep_rate=1.0, min_tok=128, max_keep=333),   # everything, capped
    dict(M=131072, chunk=32, keep_rate=0.2, min_tok=128, max_keep=5000),  # nc = 4096
    dict(M=1 << 20, chunk=256, keep_rate=0.5, min_tok=128, max_keep=100000),
    dict(M=50000, chunk=20000, keep_rate=0.5, min_tok=64, max_keep=0),  # three chunks
]


def _threshold_case(x, pos_base=0, **kw):
    params = sp.select_params(mode="threshold", pool_k=1, **kw)
    t = torch.from_numpy(x.astype(np.float32)).cuda()
    kept, pos, n = sp.sp_select(t, params, pos_base=pos_base)
    torch.cuda.synchronize()
    k_ref, p_ref = oracle.select_threshold(x.astype(np.float32), kw["chunk"], kw["keep_rate"],
                                           min_tok=kw["min_tok"], max_keep=kw["max_keep"],
                                           pos_base=pos_base)
    nk = int(n.cpu()[0])
    assert nk == len(k_ref), (kw, nk, len(k_ref))
    assert np.array_equal(kept[:nk].cpu().numpy(), k_ref), kw
    assert np.array_equal(pos[:nk].cpu().numpy(), p_ref), kw


@pytest.mark.parametrize("dist", ["uniform", "ties", "constant", "spiky"])
@pytest.mark.parametrize("case", THRESH_CASES,
                         ids=[f"{c['M']}-{c['chunk']}-{c['keep_rate']}-{c['max_keep']}"
                              for c in THRESH_CASES])
def test_select_threshold_matches_oracle(case, dist):
    kw = dict(case)
    M = kw.pop("M")
    rng = np.random.default_rng(M + 7 * len(dist))
    if dist == "uniform":
        x = rng.random(M)
    elif dist == "ties":
        x = rng.integers(0, 4, M) / 3.0
    elif dist == "constant":
        x = np.full(M, 0.25)
    else:
        x = rng.random(M) ** 12
    _threshold_case(x, pos_base=M % 7, **kw)


def test_select_threshold_varlen():
    rng = np.random.default_rng(3)
    Ms = [5000, 3, 777, 32768, 64, 12000]
    cu = np.concatenate([[0], np.cumsum(Ms)]).astype(np.int64)
    x = (rng.random(int(cu[-1])) ** 4).astype(np.float32)
    kw = dict(chunk=32, keep_rate=0.3, min_tok=128, max_keep=700)
    params = sp.select_params(mode="threshold", pool_k=1, **kw)
    t = torch.from_numpy(x).cuda()
    pos_base = [(11 * r) % 5 for r in range(len(Ms))]
    kept, pos, n = sp.sp_select_varlen(t, cu, params, pos_base=pos_base)
    torch.cuda.synchronize()
    kept_h, pos_h, n_h = kept.cpu().numpy(), pos.cpu().numpy(), n.cpu().numpy()
    for r in range(len(Ms)):
        k_ref, p_ref = oracle.select_threshold(x[cu[r]:cu[r + 1]], pos_base=pos_base[r],
                                               base_index=int(cu[r]), **kw)
        off = int(cu[r])
        assert n_h[r] == len(k_ref), r
        assert np.array_equal(kept_h[off:off + n_h[r]], k_ref), r
        assert np.array_equal(pos_h[off:off + n_h[r]], p_ref), r


# ----------------------------------------------------------------------------------------
# sliding-window scoring
# ----------------------------------------------------------------------------------------
WINDOW_CASES = [
    # id, L, H, Hkv, d, N, M, window, stride, dtype
    ("win-example-4471", 2, 8, 2, 128, 8, 4471, 2000, 1000, BF),
    ("win-one-window", 2, 4, 2, 64, 8, 700, 2000, 1000, BF),
    ("win-f32-nonoverlap", 1, 8, 2, 64, 8, 3000, 1024, 1024, F32),
    ("win-0.8b-shape", 24, 16, 8, 64, 8, 4608, 2000, 1000, BF),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_score_windows_matches_oracle(case):
    name, L, H, Hkv, d, N, M, window, stride, dt = case
    print(f"case {name}", flush=True)
    starts, lens, keeps = sp.sp_window_layout(M, window, stride)
    assert [tuple(x) for x in zip(starts, lens, keeps)] == oracle.window_layout(M, window, stride)
    w = synth.Workload(name, L=L, H=H, Hkv=Hkv, d=d, N=N, dtype=dt, seed=31, R=len(lens),
                       plant_frac=0.05, plant_chunk=32)
    Qh, Kh, cu = synth.make_ragged(w, lens)
    Q, K = to_dev(Qh), to_dev(Kh)
    imp = sp.sp_score_windows(Q, K, cu, keeps)
    full = sp.sp_score_varlen(Q, K, cu)
    torch.cuda.synchronize()
    imp_h, full_h = imp.cpu().numpy(), full.cpu().numpy()
    assert imp_h.shape == (M,)
    # window r's kept scores are the first keeps[r] of its own scores
    got = np.concatenate([full_h[cu[r]:cu[r] + keeps[r]] for r in range(len(lens))])
    assert np.array_equal(imp_h, got), name
    # the oracle scores each window from its own arrays
    Qs, Ks = [], []
    cu_keys = np.concatenate([[0], np.cumsum(np.asarray(lens) + N)])
    for r in range(len(lens)):
        Qs.append(Qh[r])
        Ks.append(np.ascontiguousarray(Kh[:, :, cu_keys[r]:cu_keys[r + 1], :]))
    check_importance(imp_h, oracle.score_windows(Qs, Ks, keeps), name)


# ----------------------------------------------------------------------------------------
# sparse-prefill batch: rows of the kept tokens
# ----------------------------------------------------------------------------------------
def test_gather_token_ids_after_select():
    rng = np.random.default_rng(12)
    M = 32768
    x = torch.from_numpy((rng.random(M) ** 6).astype(np.float32)).cuda()
    tokens = torch.from_numpy(rng.integers(0, 151936, M).astype(np.int32)).cuda()
    params = sp.select_params(chunk=32, pool_k=13, mode="topk", keep_rate=0.1)
    kept, pos, n = sp.sp_select(x, params)
    dst = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    sp.sp_gather_rows(tokens, kept, n, dst=dst)
    torch.cuda.synchronize()
    nk = int(n.cpu()[0])
    k = kept[:nk].cpu().numpy()
    assert np.array_equal(dst[:nk].cpu().numpy(), tokens.cpu().numpy()[k])
    assert np.all(dst[nk:].cpu().numpy() == -7)  # rows past the count untouched


def test_gather_hidden_rows_varlen():
    rng = np.random.default_rng(13)
    Ms = [5000, 3, 777, 12000]
    cu = np.concatenate([[0], np.cumsum(Ms)]).astype(np.int64)
    T = int(cu[-1])
    x = torch.from_numpy((rng.random(T) ** 3).astype(np.float32)).cuda()
    rows = torch.from_numpy(rng.standard_normal((T, 64)).astype(np.float32)).cuda().to(torch.bfloat16)
    params = sp.select_params(chunk=32, pool_k=3, mode="mass", mass=0.6)
    kept, pos, n = sp.sp_select_varlen(x, cu, params)
    dst = sp.sp_gather_rows(rows, kept, n, cu_prompt=cu)
    torch.cuda.synchronize()
    n_h, kept_h = n.cpu().numpy(), kept.cpu().numpy()
    rows_h = rows.view(torch.int16).cpu().numpy()
    dst_h = dst.view(torch.int16).cpu().numpy()
    for r in range(len(Ms)):
        off, nk = int(cu[r]), int(n_h[r])
        assert np.array_equal(dst_h[off:off + nk], rows_h[kept_h[off:off + nk]]), r
