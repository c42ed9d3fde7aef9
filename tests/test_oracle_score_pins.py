"""Pins of the oracle's scoring against what the pages and the mathematics fix.

Each test names the mistake it would catch. Closed forms use inputs whose
values are exact in bf16 and float32, so the expected numbers are derived by
hand from the definition (softmax of the scaled logits of look-ahead row M+j
over its M+j+1 visible keys; max over heads and layers; mean over the N
look-ahead steps), never by calling the oracle twice.

Sources: "Speculative Prefill" review page, Core formulas (attention score
a_ij = Softmax(Q_{M+j} K^T)_i; importance = mean over look-ahead steps of the
max over layers and heads); "SpecPrefill - Implementation Guide", How It Works
(max over heads, then layers, then mean over look-ahead steps).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth


def as_dtype(a32: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32
    bits = a32.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "fixture value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


DTYPES = ["f32", "bf16"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("zero_q", [False, True])
def test_uniform_keys_closed_form(dtype, zero_q):
    """All keys of a (layer, kv-head) equal, or Q = 0: every visible key gets
    1/(M+j+1), so importance_i = (1/N) sum_j 1/(M+j+1) for every prompt key.
    Catches: a denominator over M or M+N keys instead of M+j+1, a missing
    division by N, a sum instead of a max over heads/layers."""
    L, H, Hkv, d, N, M = 3, 4, 2, 8, 5, 37
    rng = np.random.default_rng(7)
    Q = rng.integers(-4, 5, size=(L, H, N, d)).astype(np.float32)
    if zero_q:
        Q[:] = 0
        K = rng.integers(-4, 5, size=(L, Hkv, M + N, d)).astype(np.float32)
    else:
        row = rng.integers(-4, 5, size=(L, Hkv, 1, d)).astype(np.float32)
        K = np.repeat(row, M + N, axis=2)
    imp = oracle.score(as_dtype(Q, dtype), as_dtype(K, dtype))
    expect = sum(1.0 / (M + j + 1) for j in range(N)) / N
    np.testing.assert_allclose(imp, expect, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_planted_key_per_layer_strengths(dtype):
    """Keys are 0 except key i* = c_l * e_a in every kv-head of layer l; every
    query row is e_a. Row j: p_{i*} = e^{c_l s}/(e^{c_l s} + M + j), every other
    visible key 1/(e^{c_l s} + M + j), s = 1/sqrt(d). The max over layers picks the
    largest c_l for i* and the smallest for the others.
    Catches: a mean over layers, a missing or wrong scale, a sign error in the
    exponent, a transposed operand."""
    L, H, Hkv, d, N, M = 3, 4, 2, 16, 4, 50
    istar, a = 17, 5
    cs = [8.0, 2.0, 4.0]  # per layer, exact in bf16
    Q = np.zeros((L, H, N, d), np.float32)
    Q[..., a] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    for l in range(L):
        K[l, :, istar, a] = cs[l]
    imp = oracle.score(as_dtype(Q, dtype), as_dtype(K, dtype))
    s = 1.0 / math.sqrt(d)
    exp_star = np.mean([max(math.exp(c * s) / (math.exp(c * s) + M + j) for c in cs)
                        for j in range(N)])
    exp_other = np.mean([max(1.0 / (math.exp(c * s) + M + j) for c in cs) for j in range(N)])
    assert imp[istar] == pytest.approx(exp_star, rel=1e-14)
    others = np.delete(imp, istar)
    np.testing.assert_allclose(others, exp_other, rtol=1e-14)


def test_explicit_scale_matches_strength():
    """An explicit scale replaces 1/sqrt(d): with scale = 1 the planted key
    gets e^c/(e^c + M + j). Catches an ignored scale argument."""
    L, H, Hkv, d, N, M = 1, 2, 1, 4, 2, 9
    c = 3.0
    Q = np.zeros((L, H, N, d), np.float32)
    Q[..., 0] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[0, 0, 4, 0] = c
    imp = oracle.score(Q, K, scale=1.0)
    expect = np.mean([math.exp(c) / (math.exp(c) + M + j) for j in range(N)])
    assert imp[4] == pytest.approx(expect, rel=1e-14)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gqa_contiguous_head_groups(dtype):
    """H=4, Hkv=2: query heads {0,1} read kv-head 0 and {2,3} read kv-head 1.
    kv-head 0 holds a planted key at i0, kv-head 1 one at i1; only query head 1
    is aligned with them (other heads have Q = 0, i.e. uniform rows).
    Contiguous grouping gives i0 the strong value and i1 only 1/(M+j+1); an
    interleaved mapping (h mod Hkv) would swap them."""
    L, H, Hkv, d, N, M = 1, 4, 2, 8, 3, 40
    i0, i1, c, a = 5, 30, 16.0, 2
    Q = np.zeros((L, H, N, d), np.float32)
    Q[0, 1, :, a] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[0, 0, i0, a] = c
    K[0, 1, i1, a] = c
    imp = oracle.score(as_dtype(Q, dtype), as_dtype(K, dtype))
    s = 1.0 / math.sqrt(d)
    e = math.exp(c * s)
    strong = np.mean([e / (e + M + j) for j in range(N)])
    uniform = np.mean([1.0 / (M + j + 1) for j in range(N)])
    assert imp[i0] == pytest.approx(strong, rel=1e-14)
    assert imp[i1] == pytest.approx(uniform, rel=1e-14)


@pytest.mark.parametrize("t", [0, 2, 4])
def test_causal_lookahead_tail(t):
    """A strong key planted in the look-ahead tail at position M+t counts only in
    the denominators of rows j >= t (row j sees keys up to M+j). Every prompt
    key has logit 0, so importance_i = (1/N) sum_j 1/Z_j with
    Z_j = M+j+1 for j < t and e^{cs} + M + j for j >= t.
    Catches: a non-causal tail (all rows see all N tail keys), a tail that is
    dropped from the denominators, importance reported for tail keys."""
    L, H, Hkv, d, N, M = 2, 2, 1, 4, 5, 23
    c, a = 8.0, 1
    Q = np.zeros((L, H, N, d), np.float32)
    Q[..., a] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[:, :, M + t, a] = c
    imp = oracle.score(Q, K)
    assert imp.shape == (M,)
    e = math.exp(c / math.sqrt(d))
    Z = [(M + j + 1) if j < t else (e + M + j) for j in range(N)]
    expect = np.mean([1.0 / z for z in Z])
    np.testing.assert_allclose(imp, expect, rtol=1e-14)


def test_lookahead_rows_pair_with_their_positions():
    """Row j is the query at position M+j: only row 3 is aligned with a strong
    tail key at M+3, which only row 3 can see. Rows 0-2 (Q = 0) are uniform over
    M+j+1 keys; row 3 has Z = e^{cs} + M + 3. Pairing step j with another
    query row (e.g. N-1-j) moves the aligned query to a row that cannot see the
    key and changes every prompt key's importance."""
    L, H, Hkv, d, N, M = 1, 1, 1, 4, 4, 11
    c, a = 8.0, 0
    Q = np.zeros((L, H, N, d), np.float32)
    Q[0, 0, 3, a] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[0, 0, M + 3, a] = c
    imp = oracle.score(Q, K)
    e = math.exp(c / math.sqrt(d))
    Z = [M + 1, M + 2, M + 3, e + M + 3]
    np.testing.assert_allclose(imp, np.mean([1.0 / z for z in Z]), rtol=1e-14)


def test_rows_sum_to_one_and_nonnegative():
    """Every softmax row over its M+j+1 visible keys sums to 1 (to 1e-12) and
    is non-negative, on the seeded tiny workload."""
    w = synth.WORKLOADS["tiny"]
    Q, K, M = synth.make_request(w)
    for (l, h, j) in [(0, 0, 0), (1, 3, 7), (0, 2, 4), (1, 1, 1)]:
        p = oracle.softmax_row(Q, K, l, h, j)
        assert p.shape == (M + j + 1,)
        assert abs(p.sum() - 1.0) < 1e-12
        assert np.all(p >= 0)


def test_importance_in_unit_interval_and_planted_keys_rank_high():
    """importance lies in [0, 1]; on the planted-direction workload the
    planted positions score higher on average than the rest."""
    w = synth.WORKLOADS["tiny"]
    Q, K, M = synth.make_request(w)
    imp = oracle.score(Q, K)
    assert np.all(imp >= 0) and np.all(imp <= 1)
    mask = synth.planted_mask(w, 0, M)[:M].astype(bool)
    assert imp[mask].mean() > 1.2 * imp[~mask].mean()


def test_permutation_and_duplication_invariance():
    """Permuting layers, permuting query heads inside a GQA group (with their
    Q rows), or duplicating a layer leaves importance bit-identical: the
    reduction over (layer, head) is a max."""
    rng = np.random.default_rng(3)
    L, H, Hkv, d, N, M = 3, 4, 2, 8, 3, 21
    Q = rng.standard_normal((L, H, N, d)).astype(np.float32)
    K = rng.standard_normal((L, Hkv, M + N, d)).astype(np.float32)
    base = oracle.score(Q, K)
    perm = [2, 0, 1]
    assert np.array_equal(oracle.score(Q[perm], K[perm]), base)
    hp = [1, 0, 3, 2]  # swaps inside group 0 and inside group 1
    assert np.array_equal(oracle.score(Q[:, hp], K), base)
    dup = [0, 1, 2, 1]
    assert np.array_equal(oracle.score(Q[dup], K[dup]), base)


def test_thread_count_does_not_change_result():
    w = synth.WORKLOADS["tiny"]
    Q, K, M = synth.make_request(w)
    assert np.array_equal(oracle.score(Q, K, nthreads=1), oracle.score(Q, K, nthreads=4))


def test_single_step_single_head_is_one_softmax_row():
    """N = 1, H = Hkv = L = 1: importance is exactly one softmax row restricted
    to the prompt keys; checked against brute force over the integers
    (logits are small integers times 1/2, p_i = e^{s_i} / sum e^{s_k})."""
    L, H, Hkv, d, N, M = 1, 1, 1, 4, 1, 7
    rng = np.random.default_rng(11)
    Q = rng.integers(-2, 3, size=(L, H, N, d)).astype(np.float32)
    K = rng.integers(-2, 3, size=(L, Hkv, M + N, d)).astype(np.float32)
    imp = oracle.score(Q, K)
    s = [0.5 * sum(int(Q[0, 0, 0, t]) * int(K[0, 0, i, t]) for t in range(d))
         for i in range(M + 1)]
    Z = sum(math.exp(x) for x in s)
    expect = [math.exp(s[i]) / Z for i in range(M)]
    np.testing.assert_allclose(imp, expect, rtol=1e-13)


def test_bf16_and_f32_storage_agree_on_exact_values():
    """Values exact in bf16 give identical importance whether stored as bf16
    or float32 (the oracle widens bf16 exactly)."""
    rng = np.random.default_rng(5)
    L, H, Hkv, d, N, M = 2, 2, 1, 8, 2, 19
    Q = (rng.integers(-8, 9, size=(L, H, N, d)) / 4).astype(np.float32)
    K = (rng.integers(-8, 9, size=(L, Hkv, M + N, d)) / 4).astype(np.float32)
    a = oracle.score(Q, K)
    b = oracle.score(as_dtype(Q, "bf16"), as_dtype(K, "bf16"))
    assert np.array_equal(a, b)


def test_rejects_bad_shapes():
    Q = np.zeros((1, 3, 2, 4), np.float32)
    K = np.zeros((1, 2, 6, 4), np.float32)  # H % Hkv != 0
    with pytest.raises(ValueError):
        oracle.score(Q, K)
