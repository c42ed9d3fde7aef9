"""Break-even gate and the sparse batch's argument checks (CPU).

Source: "SpecPrefill - Implementation Guide", v3 Improvements, Break-Even
Detection (scoring ~ M / 600 t/s, saving ~ (M - kept) / 270 t/s, skip when the
saving is below 1.2 x the scoring time) and Configuration Reference
(SP_BREAK_EVEN_SAFETY, SP_SPEC_THROUGHPUT). Both estimates are linear in M, so
the decision depends only on the kept fraction: run iff
keep <= 1 - safety * target / spec (0.46 at the defaults)."""
import ctypes

import numpy as np
import pytest

import attention_token_scoring_amd as sp


@pytest.fixture(scope="module")
def lib():
    return sp.load_library()


@pytest.mark.parametrize("M", [100, 4096, 32768, 10 ** 7])
def test_break_even_boundary_closed_form(lib, M):
    assert sp.sp_break_even(M, 0.3)           # the default keep rate: 0.7 * 600 / 270 = 1.56 >= 1.2
    assert sp.sp_break_even(M, 0.459)
    assert not sp.sp_break_even(M, 0.461)
    assert not sp.sp_break_even(M, 0.85)      # the default mass as a kept fraction
    assert sp.sp_break_even(M, 0.0)
    # a faster speculator moves the boundary: 1 - 1.2 * 270 / 1200 = 0.73
    assert sp.sp_break_even(M, 0.72, spec_tps=1200.0)
    assert not sp.sp_break_even(M, 0.74, spec_tps=1200.0)


@pytest.mark.parametrize("args", [(0, 0.3, 600, 270, 1.2), (10, -0.1, 600, 270, 1.2),
                                  (10, 1.1, 600, 270, 1.2), (10, 0.3, 0, 270, 1.2),
                                  (10, 0.3, 600, -1, 1.2), (10, 0.3, 600, 270, 0)])
def test_break_even_rejects(lib, args):
    with pytest.raises(sp.SpError):
        sp.sp_break_even(*args)


FAKE = ctypes.c_void_p(0x1000)


def test_gather_rejects(lib):
    cu = (ctypes.c_int64 * 2)(0, 10)
    assert lib.sp_gather_rows(FAKE, 6, FAKE, FAKE, 1, cu, FAKE, None) == sp.SP_EUNSUPPORTED
    assert lib.sp_gather_rows(FAKE, 0, FAKE, FAKE, 1, cu, FAKE, None) == sp.SP_EUNSUPPORTED
    assert lib.sp_gather_rows(None, 4, FAKE, FAKE, 1, cu, FAKE, None) == sp.SP_EINVAL
    assert lib.sp_gather_rows(FAKE, 4, FAKE, FAKE, 0, cu, FAKE, None) == sp.SP_EINVAL
    bad = (ctypes.c_int64 * 3)(0, 10, 10)
    assert lib.sp_gather_rows(FAKE, 4, FAKE, FAKE, 2, bad, FAKE, None) == sp.SP_EINVAL
