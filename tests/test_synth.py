"""The seeded input generator: deterministic, slice-independent, and of the
stated distribution (N(0,1) noise plus 2*u on planted keys and on every
query)."""
import numpy as np

import synth


def small(**kw):
    base = dict(name="t", L=2, H=4, Hkv=2, d=16, N=3, dtype=synth.BF16, seed=9, M=96,
                plant_chunks=2, plant_chunk=8)
    base.update(kw)
    return synth.Workload(**base)


def test_deterministic():
    w = small()
    a = synth.make_request(w)
    b = synth.make_request(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = synth.make_request(small(seed=10))
    assert not np.array_equal(a[1], c[1])


def test_ragged_packing_matches_per_request_generation():
    w = synth.Workload("r", L=2, H=4, Hkv=2, d=16, N=3, dtype=synth.BF16, seed=5, R=3,
                       len_range=(64, 256, 16), plant_frac_range=(0.05, 0.2), plant_chunk=16)
    Q, K, cu = synth.make_ragged(w)
    Ms = np.diff(cu)
    assert np.all(Ms % 16 == 0) and np.all((Ms >= 64) & (Ms <= 256))
    off = 0
    for r in range(3):
        q, k, M = synth.make_request(w, r)
        assert M == Ms[r]
        assert np.array_equal(Q[r], q)
        assert np.array_equal(K[:, :, off:off + M + w.N], k)
        off += M + w.N


def test_planted_mask():
    w = small()
    m = synth.planted_mask(w, 0, w.M)
    assert m.shape == (w.M + w.N,)
    assert m[:4].all() and not m[w.M:].any()
    body = m[4:w.M]
    assert body.sum() >= 2 * w.plant_chunk - 4  # two chunks (one may hold the sinks)


def test_distribution():
    w = small(dtype=synth.F32, d=64, M=4000, plant_chunks=1)
    q, k, M = synth.make_request(w)
    mask = synth.planted_mask(w, 0, M).astype(bool)
    noise = k[:, :, ~mask, :]
    assert abs(noise.mean()) < 0.01 and abs(noise.std() - 1) < 0.01
    for l in range(w.L):
        for g in range(w.Hkv):
            u = synth.direction(w.seed, 0, l, g, w.d)
            assert abs(np.linalg.norm(u) - 1) < 1e-12
            proj_planted = (k[l, g, mask] @ u).mean()
            proj_q = (q[l, g * w.G:(g + 1) * w.G].reshape(-1, w.d) @ u).mean()
            assert 1.0 < proj_planted < 3.0 and 1.0 < proj_q < 3.5


def test_bf16_rounding_is_nearest_even_of_f32():
    a = synth.make_request(small(dtype=synth.F32))[1]
    b = synth.make_request(small(dtype=synth.BF16))[1]
    bits = a.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(rne, b)
