"""Pins of the oracle's selection against the pages, hand derivations and
brute force.

Sources: "Speculative Prefill" review page, Core algorithm (contiguous chunks,
mean score per chunk, top-K chunks, 1-D average pooling across chunks,
position-ID recovery example) and Core formulas (chunk score, top-K);
"SpecPrefill - Implementation Guide", v3 Improvements (cumulative attention
mass, structural boosts), v3.1 item 5 (min-max normalisation) and
Configuration Reference (defaults).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_position_id_example_from_the_pages():
    """The review page's example: of positions 0..9 the kept ones are
    [0, 1, 3, 6, 7] and decoding resumes at 10."""
    g = load("position_ids_example.json")
    imp = np.array(g["importance"], np.float32)
    kept, pos = oracle.select(imp, pos_base=g["pos_base"], **g["select"])
    assert pos.tolist() == g["expected_pos_ids"]
    assert kept.tolist() == g["expected_pos_ids"]
    M = len(imp)
    assert [g["pos_base"] + M + t for t in range(3)] == g["expected_next_decode_positions"]


def test_mass_walk_hand_derived():
    g = load("mass_walk.json")
    imp = np.array(g["importance"], np.float32)
    for case in g["cases"]:
        kept, pos, dbg = oracle.select(imp, g["chunk"], g["pool_k"], "mass", mass=case["mass"],
                                       debug=True)
        assert kept.tolist() == case["kept_tokens"], case
        assert np.nonzero(dbg["kept_chunk"])[0].tolist() == case["kept_chunks"]
        assert dbg["C"].tolist() == [0, 2**33, 2**32, 2**31]


def test_normalisation_endpoints_exact():
    """Min-max normalisation maps the minimum to exactly 0 and the maximum to
    exactly 1 (fp32: (x - min) / (max - min))."""
    rng = np.random.default_rng(1)
    x = rng.random(200).astype(np.float32) * 0.01 + 0.003
    _, _, dbg = oracle.select(x, 8, 1, "topk", keep_rate=0.5, debug=True)
    v = dbg["v"]
    assert v[np.argmax(x)] == 1.0 and v[np.argmin(x)] == 0.0
    assert np.all((v >= 0) & (v <= 1))


@pytest.mark.parametrize("chunk,keep", [(4, 0.3), (8, 0.25), (1, 0.5)])
def test_constant_scores_keep_the_first_chunks(chunk, keep):
    """max == min: every value normalises to 1, every pooled key is equal, and
    the index tie-break keeps chunks 0..K-1, i.e. tokens [0, K*chunk)."""
    M = 64
    x = np.full(M, 0.37, np.float32)
    kept, pos = oracle.select(x, chunk, 3, "topk", keep_rate=keep)
    nc = M // chunk
    K = max(1, math.ceil(keep * nc))
    assert kept.tolist() == list(range(K * chunk))


@pytest.mark.parametrize("M,chunk,keep", [(1024, 32, 0.3), (32768, 32, 0.1), (640, 64, 0.5),
                                          (1000, 32, 0.1)])
def test_topk_keeps_exactly_K_chunks(M, chunk, keep):
    """Top-K keeps max(1, ceil(rate * nc)) chunks: exactly K*chunk tokens when
    chunk divides M (the last, partial chunk counts its own length otherwise)."""
    rng = np.random.default_rng(M)
    x = rng.random(M).astype(np.float32)
    kept, pos, dbg = oracle.select(x, chunk, 13 if M > 2000 else 3, "topk", keep_rate=keep,
                                   debug=True)
    nc = -(-M // chunk)
    K = max(1, math.ceil(np.float64(np.float32(keep)) * nc))
    assert int(dbg["kept_chunk"].sum()) == K
    lens = [min(chunk, M - c * chunk) for c in range(nc)]
    assert len(kept) == sum(l for c, l in enumerate(lens) if dbg["kept_chunk"][c])


def test_pool_closed_form():
    """One chunk at the maximum, all others at the minimum: v = 1 on that
    chunk's tokens and 0 elsewhere, so C = chunk * 2^32 there and 0 elsewhere.
    With pool width 3 the pooled key of the hot chunk and of each neighbour is
    2^32/3 (full window), and at the edge chunk 0 the clipped window [0, 1]
    gives 2^32/2."""
    chunk, nc = 4, 6
    for hot in (0, 3):
        x = np.zeros(chunk * nc, np.float32)
        x[hot * chunk:(hot + 1) * chunk] = 1.0
        _, _, dbg = oracle.select(x, chunk, 3, "topk", keep_rate=0.5, debug=True)
        key = dbg["key"]
        for c in range(nc):
            lo, hi = max(0, c - 1), min(nc - 1, c + 1)
            if lo <= hot <= hi:
                expect = (chunk * 2.0**32) / ((hi - lo + 1) * chunk)
            else:
                expect = 0.0
            assert key[c] == expect, (hot, c, key[c], expect)


def test_pool_width_one_is_chunk_mean():
    """k = 1: the key is the chunk mean of the fixed-point values."""
    x = np.array([0.0, 1.0, 0.5, 0.25, 0.75, 1.0], np.float32)
    _, _, dbg = oracle.select(x, 2, 1, "topk", keep_rate=0.5, debug=True)
    assert dbg["key"].tolist() == [2.0**31, 0.375 * 2**32, 0.875 * 2**32]


def test_boosts_first_then_last_multiply_on_overlap():
    """Boosts multiply the normalised value of the first n tokens, then the
    last n tokens; where the two ranges overlap both factors apply."""
    M = 8
    x = np.full(M, 0.5, np.float32)  # constant: every v is 1
    _, _, dbg = oracle.select(x, 2, 1, "topk", keep_rate=0.5, boost_first_n=2,
                              boost_first_mult=1.5, boost_last_n=3, boost_last_mult=1.25,
                              debug=True)
    assert dbg["v"].tolist() == [1.5, 1.5, 1, 1, 1, 1.25, 1.25, 1.25]
    _, _, dbg = oracle.select(x, 2, 1, "topk", keep_rate=0.5, boost_first_n=6,
                              boost_first_mult=1.5, boost_last_n=4, boost_last_mult=1.25,
                              debug=True)
    assert dbg["v"].tolist() == [1.5, 1.5, 1.5, 1.5, 1.875, 1.875, 1.25, 1.25]


def test_fixed_point_rounds_half_to_even():
    """q = v * 2^32 rounded to nearest, ties to even: v = 2^-33 -> 0,
    3*2^-33 -> 2, 5*2^-33 -> 2, 7*2^-33 -> 4."""
    x = np.array([0.0, 2.0**-33, 3 * 2.0**-33, 5 * 2.0**-33, 7 * 2.0**-33, 1.0], np.float32)
    _, _, dbg = oracle.select(x, 1, 1, "topk", keep_rate=0.5, debug=True)
    assert dbg["q"].tolist() == [0, 0, 2, 2, 4, 2**32]


def _strict_better(key, a, b):
    """a ranks before b: larger pooled key, then smaller index."""
    return key[a] > key[b] or (key[a] == key[b] and a < b)


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed):
    """For nc <= 10 chunks, enumerate every K-subset: exactly one has every
    member ranked before every non-member, and it is the oracle's kept set."""
    rng = np.random.default_rng(seed)
    chunk = 3
    nc = int(rng.integers(2, 11))
    vals = rng.integers(0, 5, size=nc * chunk) / 4.0  # coarse values force ties
    x = vals.astype(np.float32)
    keep = float(rng.choice([0.2, 0.3, 0.5, 0.7, 1.0]))
    pool = int(rng.choice([1, 3, 5]))
    _, _, dbg = oracle.select(x, chunk, pool, "topk", keep_rate=keep, debug=True)
    key = dbg["key"]
    K = max(1, math.ceil(np.float64(np.float32(keep)) * nc))
    winners = []
    for S in itertools.combinations(range(nc), K):
        rest = [c for c in range(nc) if c not in S]
        if all(_strict_better(key, a, b) for a in S for b in rest):
            winners.append(set(S))
    assert len(winners) == 1
    assert set(np.nonzero(dbg["kept_chunk"])[0].tolist()) == winners[0]


@pytest.mark.parametrize("seed", range(12))
def test_mass_brute_force(seed):
    """Mass mode over all subsets: the kept set is the unique set that (a) is
    closed upward in the ranking, (b) reaches the threshold with its own
    (un-pooled) chunk masses, and (c) falls below it without its lowest-ranked
    member."""
    rng = np.random.default_rng(100 + seed)
    chunk = 2
    nc = int(rng.integers(2, 10))
    x = (rng.integers(0, 9, size=nc * chunk) / 8.0).astype(np.float32)
    tau = float(rng.choice([0.3, 0.5, 0.85, 1.0]))
    pool = int(rng.choice([1, 3]))
    _, _, dbg = oracle.select(x, chunk, pool, "mass", mass=tau, debug=True)
    key, C = dbg["key"], [int(c) for c in dbg["C"]]
    thr = float(np.float32(tau)) * float(sum(C))
    found = []
    for r in range(1, nc + 1):
        for S in itertools.combinations(range(nc), r):
            rest = [c for c in range(nc) if c not in S]
            if not all(_strict_better(key, a, b) for a in S for b in rest):
                continue
            if float(sum(C[c] for c in S)) < thr:
                continue
            low = [c for c in S if all(_strict_better(key, o, c) for o in S if o != c)][0]
            if float(sum(C[c] for c in S) - C[low]) >= thr:
                continue
            found.append(set(S))
    assert len(found) == 1
    assert set(np.nonzero(dbg["kept_chunk"])[0].tolist()) == found[0]


def test_mass_one_keeps_every_chunk_with_mass():
    rng = np.random.default_rng(9)
    x = rng.random(300).astype(np.float32)
    _, _, dbg = oracle.select(x, 16, 3, "mass", mass=1.0, debug=True)
    assert np.all(dbg["kept_chunk"][dbg["C"] > 0])


def test_position_ids_ascending_with_offsets():
    """Kept positions are strictly increasing; kept_idx carries the packed
    base index and pos_ids the position base; next decode position = base+M."""
    rng = np.random.default_rng(4)
    M = 500
    x = rng.random(M).astype(np.float32)
    kept, pos = oracle.select(x, 32, 5, "mass", mass=0.85, pos_base=1000, base_index=77)
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(kept - 77, pos - 1000)
    assert pos.min() >= 1000 and pos.max() < 1000 + M


def test_partial_last_chunk():
    """M not a multiple of chunk: the last chunk holds M mod chunk tokens and
    its key averages over those tokens only."""
    x = np.zeros(10, np.float32)
    x[8:] = 1.0  # last chunk (tokens 8, 9) is hot
    kept, _, dbg = oracle.select(x, 4, 1, "topk", keep_rate=0.1, debug=True)
    assert dbg["key"].tolist() == [0.0, 0.0, 2.0**32]
    assert kept.tolist() == [8, 9]


@pytest.mark.parametrize("bad", [dict(chunk=0), dict(pool_k=2), dict(keep_rate=0.0),
                                 dict(keep_rate=1.5)])
def test_rejects_bad_arguments(bad):
    args = dict(chunk=4, pool_k=3, mode="topk", keep_rate=0.5)
    args.update(bad)
    with pytest.raises(ValueError):
        oracle.select(np.ones(16, np.float32), **args)
