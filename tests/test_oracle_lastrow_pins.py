"""Pins of oracle.score_lastrow: importance with the last prompt token's query
row as one more step ("SpecPrefill - Implementation Guide", How It Works,
Attention Capture (cb_eval)). That row sits at position M-1 and sees the M
prompt keys only, and importance averages the N look-ahead steps and this one.
Closed forms fix the row's key range (the look-ahead keys excluded, itself
included), the 1/(N+1) average and the query-head to kv-head mapping."""
import math

import numpy as np

import oracle


def _uniform_S(M, N):
    return sum(1.0 / (M + j + 1) for j in range(N))


def test_uniform_keys():
    rng = np.random.default_rng(0)
    L, H, Hkv, N, M, d = 2, 4, 2, 5, 300, 16
    Q = rng.standard_normal((L, H, N, d)).astype(np.float32)
    Ql = rng.standard_normal((L, H, d)).astype(np.float32)
    K = np.broadcast_to(rng.standard_normal(d).astype(np.float32), (L, Hkv, M + N, d)).copy()
    got = oracle.score_lastrow(Q, Ql, K)
    np.testing.assert_allclose(got, (_uniform_S(M, N) + 1.0 / M) / (N + 1), rtol=1e-12)


def test_planted_key_for_the_last_row():
    """Look-ahead queries 0 (their rows are uniform), the last row aligned with
    one prompt key of logit a: X = e^a / (e^a + M - 1) there, 1/(e^a + M - 1)
    elsewhere."""
    L, H, Hkv, N, M, d, a, i_star = 1, 2, 1, 3, 200, 4, 4.0, 37
    Q = np.zeros((L, H, N, d), np.float32)
    Ql = np.zeros((L, H, d), np.float32)
    Ql[..., 0] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[0, 0, i_star, 0] = a
    got = oracle.score_lastrow(Q, Ql, K, scale=1.0)
    Z = math.exp(a) + M - 1
    X = np.full(M, 1.0 / Z)
    X[i_star] = math.exp(a) / Z
    np.testing.assert_allclose(got, (_uniform_S(M, N) + X) / (N + 1), rtol=1e-12)


def test_last_row_does_not_see_the_look_ahead_keys():
    """Strong keys in the look-ahead tail only (M..M+N-1), aligned with the last
    row's query: that row must stay uniform over its M keys (X = 1/M), while a
    look-ahead row j that sees t + 1 of them is pulled away from the prompt."""
    L, H, Hkv, N, M, d, a = 1, 1, 1, 4, 100, 4, 5.0
    Q = np.zeros((L, H, N, d), np.float32)
    Q[..., 0] = 1.0
    Ql = np.zeros((L, H, d), np.float32)
    Ql[..., 0] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[0, 0, M:, 0] = a
    got = oracle.score_lastrow(Q, Ql, K, scale=1.0)
    S = sum(1.0 / (M + (j + 1) * math.exp(a)) for j in range(N))
    np.testing.assert_allclose(got, (S + 1.0 / M) / (N + 1), rtol=1e-12)


def test_head_to_kv_head_mapping():
    """G = 2 query heads per kv-head; only kv-head 1 holds a planted key, and
    only the last-row queries of heads 2 and 3 (group 1) align with it. The
    max over heads is then e^a/(e^a + M - 1) at the key and 1/M elsewhere
    (group 0's uniform rows)."""
    L, H, Hkv, N, M, d, a, i_star = 1, 4, 2, 2, 150, 4, 3.0, 99
    Q = np.zeros((L, H, N, d), np.float32)
    Ql = np.zeros((L, H, d), np.float32)
    Ql[0, 2:, 0] = 1.0
    K = np.zeros((L, Hkv, M + N, d), np.float32)
    K[0, 1, i_star, 0] = a
    got = oracle.score_lastrow(Q, Ql, K, scale=1.0)
    X = np.full(M, 1.0 / M)
    X[i_star] = math.exp(a) / (math.exp(a) + M - 1)
    np.testing.assert_allclose(got, (_uniform_S(M, N) + X) / (N + 1), rtol=1e-12)


def test_bf16_matches_widened_f32():
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((2, 4, 3, 8)).astype(np.float32)
    Ql = rng.standard_normal((2, 4, 8)).astype(np.float32)
    K = rng.standard_normal((2, 2, 53, 8)).astype(np.float32)
    to_bf = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
    wid = lambda b: (b.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    a = oracle.score_lastrow(to_bf(Q), to_bf(Ql), to_bf(K))
    b = oracle.score_lastrow(wid(to_bf(Q)), wid(to_bf(Ql)), wid(to_bf(K)))
    assert np.array_equal(a, b)
