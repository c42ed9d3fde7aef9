"""Sliding-window layout: the oracle's and the library's (two separate
implementations) against the Implementation Guide's worked example (section
Sliding Window, Sliding Window Solution: 4471 tokens, window 2000, stride
1000) and the coverage property the v3.1 fix states (every token scored by
exactly one window)."""
import json
import os

import numpy as np
import pytest

import attention_token_scoring_amd as sp
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "window_layout_example.json")


def expected():
    with open(GOLDEN) as f:
        g = json.load(f)
    return g, [(w["start"], w["len"], w["keep"]) for w in g["windows"]]


def lib_layout(M, window, stride):
    starts, lens, keeps = sp.sp_window_layout(M, window, stride)
    return list(zip(starts.tolist(), lens.tolist(), keeps.tolist()))


def test_oracle_layout_matches_the_pages_example():
    g, want = expected()
    assert oracle.window_layout(g["M"], g["window"], g["stride"]) == want


def test_library_layout_matches_the_pages_example():
    g, want = expected()
    assert lib_layout(g["M"], g["window"], g["stride"]) == want


@pytest.mark.parametrize("M,window,stride", [(1, 1, 1), (1500, 2000, 1000), (2000, 2000, 1000),
                                             (2001, 2000, 1000), (4000, 2000, 1000),
                                             (10000, 2048, 2048), (9999, 3000, 7),
                                             (123457, 8192, 4096)])
def test_layouts_cover_every_token_once(M, window, stride):
    lay = lib_layout(M, window, stride)
    assert lay == oracle.window_layout(M, window, stride)
    covered = 0
    for k, (start, length, keep) in enumerate(lay):
        assert start == k * stride and start == covered  # kept ranges are contiguous
        assert 1 <= keep <= length <= window and start + length <= M
        covered += keep
    assert covered == M
    assert lay[-1][0] + lay[-1][1] == M and lay[-1][1] == lay[-1][2]


@pytest.mark.parametrize("M,window,stride", [(0, 10, 5), (10, 0, 1), (10, 5, 0), (10, 5, 6)])
def test_layout_rejects(M, window, stride):
    with pytest.raises(sp.SpError):
        sp.sp_window_layout(M, window, stride)
    with pytest.raises(ValueError):
        oracle.window_layout(M, window, stride)
