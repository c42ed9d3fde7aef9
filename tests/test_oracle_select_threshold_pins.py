"""Pins of the oracle's threshold selection (the chunk selection and the cap on
sparse tokens of the Implementation Guide's own program).

Sources: "SpecPrefill - Implementation Guide", How It Works / Chunk Selection
(32-token chunks ranked by mean score, the first 4 and last 2 tokens always
kept), Configuration Reference (SP_MAX_KEEP) and Full Source Code (the
selection's threshold, fill and cap steps). Expected values below are derived
by hand or from invariants, not by re-running the oracle's own steps.
"""
import numpy as np
import pytest

import oracle


def sel(x, chunk, keep, min_tok=0, max_keep=0, pos_base=0):
    k, p = oracle.select_threshold(np.asarray(x, np.float32), chunk, keep, min_tok=min_tok,
                                   max_keep=max_keep, pos_base=pos_base)
    assert np.array_equal(p, k + pos_base)
    return k.tolist()


X10 = [0.9, 0.8, 0.1, 0.7, 0.2, 0.3, 0.6, 0.5, 0.05, 0.15]


def test_single_token_chunks_hand_derived():
    # K = ceil(10 * 0.5) = 5; the 5th largest score is 0.5, so tokens with
    # score >= 0.5 stay (0, 1, 3, 6, 7), plus the always-kept 0..3 and 8, 9
    assert sel(X10, 1, 0.5) == [0, 1, 2, 3, 6, 7, 8, 9]


def test_two_token_chunks_hand_derived():
    # chunk means 0.85, 0.4, 0.25, 0.55, 0.1; K = ceil(1.5) = 2, threshold 0.55
    # -> chunks 0 and 3; always-kept adds 2, 3, 8, 9
    assert sel(X10, 2, 0.3) == [0, 1, 2, 3, 6, 7, 8, 9]


def test_equal_means_at_the_threshold_are_all_kept():
    # four chunks with means 1, 2, 2, 2: K = ceil(4 * 0.25) = 1 -> threshold 2,
    # and all three chunks at 2 are kept (3 > K)
    x = [1] * 8 + [2] * 24
    got = sel(x, 8, 0.25)
    assert got == [0, 1, 2, 3] + list(range(8, 32))


def test_fill_takes_dropped_chunks_in_index_order():
    # M = 64, chunk 8, chunks 0..7 with means 1..8 except chunk 7 highest;
    # K = ceil(8 * 0.1) = 1 -> chunk 7 (tokens 56..63) plus 0..3 (62, 63 are
    # in it): 12 tokens; min_tok 20 -> eff_min = min(20, max(4, 6)) = 6 <= 12,
    # nothing added. With min_tok large: eff_min = max(4, 64 // 10) = 6.
    x = np.repeat(np.arange(1, 9, dtype=np.float32), 8)
    assert sel(x, 8, 0.1, min_tok=20) == [0, 1, 2, 3] + list(range(56, 64))
    # a prompt of 200 tokens, one hot chunk: eff_min = min(128, max(4, 20)) = 20
    y = np.zeros(200, np.float32)
    y[100:110] = 1.0
    got = sel(y, 10, 0.05, min_tok=128)  # K = 1 -> chunk 10 (tokens 100..109)
    # 10 chunk tokens + 0..3 + 198, 199 = 16 < 20: the 4 lowest free tokens of
    # the dropped chunks, in index order (4, 5, 6, 7)
    assert got == [0, 1, 2, 3, 4, 5, 6, 7] + list(range(100, 110)) + [198, 199]


def test_keep_everything_cases():
    assert sel(X10, 1, 1.0) == list(range(10))
    # M <= eff_min: 10 <= min(128, max(4, 1)) = 4 is false; M = 4 is not
    assert sel([0.5, 0.1, 0.2, 0.3], 1, 0.25, min_tok=128) == [0, 1, 2, 3]


def test_short_prompts_keep_their_first_tokens():
    # M = 3 (the last-two rule needs M > 4): every token is below the floor 4
    assert sel([0.1, 0.9, 0.2], 1, 0.3, min_tok=0) == [0, 1, 2]
    # M = 5: always-kept 0..3 and 3, 4 (overlap at 3 counted once)
    assert sel([0.0, 0.0, 0.0, 0.0, 0.0], 5, 0.5) == [0, 1, 2, 3, 4]


def test_cap_is_a_strided_subsequence_ending_at_the_last_kept_token():
    rng = np.random.default_rng(4)
    x = rng.random(5000).astype(np.float32)
    full = sel(x, 32, 0.5, min_tok=128)
    for cap in (1, 7, 100, len(full) - 1, len(full), len(full) + 5):
        got = sel(x, 32, 0.5, min_tok=128, max_keep=cap)
        if cap >= len(full):
            assert got == full
            continue
        step = len(full) // cap
        assert len(got) == cap
        assert got[:-1] == full[0:(cap - 1) * step:step]
        assert got[-1] == full[-1]


def test_kept_chunks_dominate_dropped_ones():
    rng = np.random.default_rng(9)
    for trial in range(20):
        M = int(rng.integers(5, 3000))
        chunk = int(rng.integers(1, 70))
        keep = float(rng.uniform(0.01, 0.99))
        x = (rng.random(M) ** 3).astype(np.float32)
        got = set(sel(x, chunk, keep))
        nc = -(-M // chunk)
        means = [np.float32(np.sum(x[c * chunk:(c + 1) * chunk], dtype=np.float64) /
                            len(x[c * chunk:(c + 1) * chunk])) for c in range(nc)]
        always = {0, 1, 2, 3} | ({M - 2, M - 1} if M > 4 else set())
        toks = [set(range(c * chunk, min((c + 1) * chunk, M))) for c in range(nc)]
        decided = [c for c in range(nc) if toks[c] - always]  # (not only always-kept tokens)
        kept_c = [c for c in decided if toks[c] <= got]
        dropped = [c for c in decided if not toks[c] <= got]
        K = max(1, int(np.ceil(np.float32(nc) * np.float32(keep))))
        assert len(kept_c) + (nc - len(decided)) >= min(K, nc)
        if kept_c and dropped:
            assert min(means[c] for c in kept_c) >= max(means[c] for c in dropped)
        assert {0, 1, 2, 3} & set(range(M)) <= got
        if M > 4:
            assert {M - 2, M - 1} <= got


def test_rejects_bad_arguments():
    for kw in (dict(chunk=0), dict(keep=0.0), dict(min_tok=-1), dict(max_keep=-2)):
        args = dict(chunk=2, keep=0.5, min_tok=0, max_keep=0)
        args.update(kw)
        with pytest.raises(ValueError):
            oracle.select_threshold(np.ones(10, np.float32), args["chunk"], args["keep"],
                                    min_tok=args["min_tok"], max_keep=args["max_keep"])
