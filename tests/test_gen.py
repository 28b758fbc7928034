"""The seeded input generators produce the workload shapes they promise (CPU)."""
import numpy as np
import pytest

import gtgen


def valid_csr(indptr, indices, N):
    assert indptr[0] == 0 and np.all(np.diff(indptr) >= 0) and indptr[-1] == len(indices)
    assert len(indptr) == N + 1
    assert len(indices) == 0 or (indices.min() >= 0 and indices.max() < N)


def test_counter_generator_is_pure():
    a = [gtgen.lib().gtgen_u64(0, 1, i) for i in range(5)]
    b = [gtgen.lib().gtgen_u64(0, 1, i) for i in range(5)]
    assert a == b and len(set(a)) == 5
    assert gtgen.lib().gtgen_u64(1, 1, 0) != a[0] and gtgen.lib().gtgen_u64(0, 2, 0) != a[0]
    x = gtgen.normal_f32(0, 1, 1001)
    y = gtgen.normal_f32(0, 1, 2000)
    assert np.array_equal(x, y[:1001])


def test_normals_moments():
    x = gtgen.normal_f32(3, 1, 1_000_000).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    b = gtgen.bf16_bits_to_f32(gtgen.normal_bf16(3, 1, 1_000_000, 0.5)).astype(np.float64)
    assert abs(b.std() - 0.5) < 5e-3
    # bf16 values are fp32(N(0,1))*0.5 rounded to 8 significant bits
    f = gtgen.normal_f32(3, 1, 1000) * np.float32(0.5)
    rb = gtgen.bf16_bits_to_f32(gtgen.normal_bf16(3, 1, 1000, 0.5))
    assert np.all(np.abs(rb - f) <= np.abs(f) * 2.0 ** -8)


def test_coo_to_csr_stable():
    src = np.array([5, 1, 2, 7, 3], np.int32)
    dst = np.array([2, 0, 2, 0, 1], np.int32)
    indptr, indices, perm = gtgen.coo_to_csr(3, src, dst, return_perm=True)
    assert indptr.tolist() == [0, 2, 3, 5]
    assert indices.tolist() == [1, 7, 3, 5, 2]
    assert perm.tolist() == [1, 3, 4, 0, 2]


def test_tiny_random():
    w = gtgen.make_workload("tiny_random")
    assert (w["N"], w["E"], w["H"], w["D"]) == (30, 100, 8, 64)
    valid_csr(w["indptr"], w["indices"], 30)
    assert w["Q"].shape == (30, 8, 64) and w["Q"].dtype == np.float32


def test_molecules():
    w = gtgen.make_workload("molecules", with_features=False)
    N, indptr, indices = w["N"], w["indptr"], w["indices"]
    valid_csr(indptr, indices, N)
    assert 128 * 10 <= N <= 128 * 50
    dst = np.repeat(np.arange(N), np.diff(indptr))
    pairs = set(zip(indices.tolist(), dst.tolist()))
    assert len(pairs) == len(indices)  # no duplicates
    assert all((b, a) in pairs for a, b in pairs)  # stored in both directions
    assert np.all(indices != dst)  # no self-loops
    assert np.all(np.diff(indptr) >= 1)


def test_regular16():
    indptr, indices = gtgen.make_graph("regular16")
    valid_csr(indptr, indices, 100_000)
    assert np.all(np.diff(indptr) == 16)


def test_powerlaw_shape():
    indptr, indices = gtgen.make_graph("powerlaw")
    valid_csr(indptr, indices, 1_000_000)
    deg = np.diff(indptr)
    assert indptr[-1] == 16_000_000 and deg.max() == 50_000
    assert 590_000 < (deg > 0).sum() < 620_000
    assert 40 <= (deg == 50_000).sum() <= 100
    # share of edges in rows of degree > 4096 is about half
    assert 0.45 < deg[deg > 4096].sum() / 16e6 < 0.65
    # clipped Zipf(1.8): P(1) = 1/zeta(1.8) ~ 0.531 among drawn rows
    assert abs((deg == 1).sum() / (deg > 0).sum() - 0.531) < 0.01


def test_lognormal_shape():
    deg = gtgen.degrees_lognormal(0, 2_400_000, 60_000_000)
    assert deg.sum() == 60_000_000
    assert 2_000 < deg.max() < 10_000
    assert 0.001 < (deg == 0).mean() < 0.02


def test_source_sorted_is_the_transpose():
    indptr, indices = gtgen.make_graph("tiny_random")
    N = len(indptr) - 1
    tip, tix = gtgen.source_sorted(indptr, indices)
    assert tip[0] == 0 and tip[-1] == len(indices)
    fwd = sorted((int(u), v) for v in range(N) for u in indices[indptr[v]:indptr[v + 1]])
    back = sorted((u, int(v)) for u in range(N) for v in tix[tip[u]:tip[u + 1]])
    assert fwd == back
    # out-edges of a source keep destination-CSR order (stable)
    for u in range(N):
        assert np.all(np.diff(tix[tip[u]:tip[u + 1]]) >= 0)


def test_grad_stream_differs_from_features():
    Q, K, V = gtgen.make_features(10, 2, 4, gtgen.F32, seed=3)
    g = gtgen.make_grad(10, 2, 4, gtgen.F32, seed=3)
    assert g.shape == Q.shape and not np.array_equal(g, Q) and not np.array_equal(g, V)
    assert np.array_equal(g, gtgen.make_grad(10, 2, 4, gtgen.F32, seed=3))
