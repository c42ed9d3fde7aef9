"""The Python binding rejects output (and score) tensors that the kernels would
index out of bounds or misread: wrong dtype, not on the GPU, not contiguous,
or too small. Checked on the CPU (every case fails before any library call)."""
import pytest

torch = pytest.importorskip("torch")

import attention_token_scoring_amd as sp  # noqa: E402


class _FakeCuda:
    """Stands in for a CUDA tensor in the binding's checks (no GPU here)."""

    def __init__(self, t):
        self._t = t
        self.dtype = t.dtype
        self.is_cuda = True

    def is_contiguous(self):
        return self._t.is_contiguous()

    def numel(self):
        return self._t.numel()


def test_check_out_accepts_a_matching_tensor():
    sp._check_out(_FakeCuda(torch.empty(10, dtype=torch.int32)), torch.int32, 10, "x")


@pytest.mark.parametrize("t,dtype,n", [
    (torch.empty(10, dtype=torch.int64), torch.int32, 10),      # wrong dtype
    (torch.empty(10, dtype=torch.float64), torch.float32, 10),  # wrong dtype
    (torch.empty(9, dtype=torch.int32), torch.int32, 10),       # too small
    (torch.empty(0, dtype=torch.float32), torch.float32, 1),    # empty
    (torch.empty(20, dtype=torch.int32)[::2], torch.int32, 10),  # not contiguous
])
def test_check_out_rejects(t, dtype, n):
    with pytest.raises(ValueError):
        sp._check_out(_FakeCuda(t), dtype, n, "x")


def test_check_out_rejects_host_tensors():
    with pytest.raises(ValueError):
        sp._check_out(torch.empty(10, dtype=torch.int32), torch.int32, 10, "x")


def test_select_rejects_host_tensors():
    params = sp.select_params(chunk=32, pool_k=1, mode="topk", keep_rate=0.5)
    with pytest.raises(ValueError):
        sp.sp_select(torch.zeros(64, dtype=torch.float32), params)
    with pytest.raises(ValueError):
        sp.sp_select_varlen(torch.zeros(64, dtype=torch.float32), [0, 32, 64], params)
