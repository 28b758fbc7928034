"""Pins of the oracle's graph construction (COO -> destination-sorted CSR and
its source-sorted transpose) to things other than itself (CPU).

* a library sort: numpy's stable lexsort by (destination, COO id) gives the
  CSR order, and searchsorted over the sorted destinations gives indptr;
* invariants: indptr starts at 0, ends at E, never decreases; the multiset of
  (src, dst) pairs is kept; within a row the COO ids increase (stability);
* transposing twice gives back the CSR;
* a hand-worked example under tests/golden/graph/.
test_oracle_graph_mutants.py plants mistakes in copies of oracle.c and shows
each one fails at least one of these checks.
"""
import json
import os

import numpy as np
import pytest

import oracle as oracle_mod
from oracle import Oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "graph")


def random_coo(rng, n_dst, n_src, E):
    return (rng.integers(0, n_src, E).astype(np.int32), rng.integers(0, n_dst, E).astype(np.int32))


def check_library_sort(orc):
    rng = np.random.default_rng(1)
    for n_dst, n_src, E in ((1, 1, 0), (1, 1, 5), (7, 7, 40), (50, 20, 600), (300, 900, 5000), (64, 64, 0)):
        src, dst = random_coo(rng, n_dst, n_src, E)
        indptr, indices, perm = orc.coo_to_csr(n_dst, src, dst, n_src=n_src)
        order = np.lexsort((np.arange(E), dst))
        assert np.array_equal(perm, order)
        assert np.array_equal(indices, src[order])
        assert np.array_equal(indptr, np.searchsorted(dst[order], np.arange(n_dst + 1), side="left"))


def check_invariants(orc):
    rng = np.random.default_rng(2)
    n, E = 200, 3000
    src, dst = random_coo(rng, n, n, E)
    dst[:500] = 17  # a hub row
    indptr, indices, perm = orc.coo_to_csr(n, src, dst)
    assert indptr[0] == 0 and indptr[-1] == E and np.all(np.diff(indptr) >= 0)
    rows = np.repeat(np.arange(n), np.diff(indptr))
    assert sorted(zip(indices.tolist(), rows.tolist())) == sorted(zip(src.tolist(), dst.tolist()))
    for v in range(n):
        assert np.all(np.diff(perm[indptr[v]:indptr[v + 1]]) > 0)
    assert np.array_equal(src[perm], indices) and np.array_equal(dst[perm], rows)


def check_double_transpose(orc):
    rng = np.random.default_rng(3)
    n_dst, n_src, E = 120, 80, 2000
    src, dst = random_coo(rng, n_dst, n_src, E)
    indptr, indices, _ = orc.coo_to_csr(n_dst, src, dst, n_src=n_src)
    t_indptr, t_indices = orc.source_sorted(indptr, indices, n_src=n_src)
    assert len(t_indptr) == n_src + 1
    back_indptr, back_indices = orc.source_sorted(t_indptr, t_indices, n_src=n_dst)
    # the same rows, each now in source order
    rows = np.repeat(np.arange(n_dst), np.diff(indptr))
    assert np.array_equal(back_indptr, indptr)
    assert np.array_equal(back_indices, indices[np.lexsort((indices, rows))])
    # the transpose agrees with numpy's stable argsort of the sources
    assert np.array_equal(t_indices, np.repeat(np.arange(n_dst), np.diff(indptr))[np.argsort(indices, kind="stable")])


def check_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "four_edges.json")))
    indptr, indices, perm = orc.coo_to_csr(g["n"], g["src"], g["dst"])
    assert indptr.tolist() == g["indptr"] and indices.tolist() == g["indices"] and perm.tolist() == g["perm"]
    t_indptr, t_indices = orc.source_sorted(indptr, indices)
    assert t_indptr.tolist() == g["t_indptr"] and t_indices.tolist() == g["t_indices"]


def check_rejects_out_of_range(orc):
    with pytest.raises(ValueError):
        orc.coo_to_csr(3, [0, 3], [1, 1])
    with pytest.raises(ValueError):
        orc.coo_to_csr(3, [0, 1], [1, -1])


ALL_CHECKS = [check_library_sort, check_invariants, check_double_transpose, check_golden, check_rejects_out_of_range]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_graph_pin(check):
    check(Oracle())


def test_module_level_functions():
    indptr, indices, _ = oracle_mod.coo_to_csr(2, [1, 0], [0, 0])
    assert indptr.tolist() == [0, 2, 2] and indices.tolist() == [1, 0]
