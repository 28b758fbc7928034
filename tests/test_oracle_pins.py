"""Pins of the fp64 oracle to things other than itself (CPU only).

Each ``check_*`` takes an oracle object and fails by AssertionError; the
same checks run against deliberately broken copies of oracle.c in
test_oracle_mutants.py, which proves that plausible mistakes are caught.

What pins what:
* whole forward  -- torch's scaled_dot_product_attention (a library routine)
  in float64 on CPU with an additive mask ln(multiplicity), -inf off the graph:
  the dense masked-softmax form of "Graph Transformer theory" (GAT code in the
  implementation section masks non-neighbours with -inf before the softmax);
  the complete graph equals the textbook softmax(QK^T/sqrt(d))V of "Graph
  Transformer in a Nutshell" (section Sparse Multi-head Attention);
  hand-worked golden examples under tests/golden/.
* SDDMM -- basis vectors give exactly delta/sqrt(D); equals the entries of a
  library matrix product Q K^T / sqrt(D) at the edges.
* edge softmax -- scipy.special.softmax per destination; sums to 1; shift
  invariance; two edges give the logistic function; one edge gives 1.
* SpMM -- one in-edge copies the source row exactly; uniform weights give the
  library mean; linearity in V.
* zero in-degree rows are exactly 0; relabelling nodes permutes the output;
  bf16 inputs equal their exact fp32 widening.
"""
import glob
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import gtgen
import oracle

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


# ----------------------------------------------------------------- helpers

def tiny_graph(seed, N, E):
    src, dst = gtgen.random_coo(seed, N, E)
    indptr, indices = gtgen.coo_to_csr(N, src, dst)
    return indptr, indices


def feats(seed, N, H, D, scale=1.0):
    return tuple(gtgen.normal_f32(seed, s, (N, H, D), scale) for s in (1, 2, 3))


def dst_of_edges(indptr):
    return np.repeat(np.arange(len(indptr) - 1), np.diff(indptr))


def sdpa_reference(indptr, indices, Q, K, V):
    """Dense masked attention by torch SDPA (float64, CPU)."""
    N, H, D = Q.shape
    C = np.zeros((N, N))
    np.add.at(C, (dst_of_edges(indptr), indices), 1.0)
    with np.errstate(divide="ignore"):
        mask = torch.from_numpy(np.log(C))  # ln(multiplicity); -inf off the graph
    q = torch.from_numpy(np.asarray(Q, np.float64)).permute(1, 0, 2).contiguous()
    k = torch.from_numpy(np.asarray(K, np.float64)).permute(1, 0, 2).contiguous()
    v = torch.from_numpy(np.asarray(V, np.float64)).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    o = o.permute(1, 0, 2).numpy().copy()
    o[np.diff(indptr) == 0] = 0.0  # the empty sum
    return o


def close(a, b, rtol=1e-12, atol=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite oracle output"
    err = np.abs(a - b) - (atol + rtol * np.abs(b))
    assert np.all(err <= 0), "max excess %.3e at %s" % (err.max(), np.unravel_index(err.argmax(), err.shape))


# ----------------------------------------------------------------- checks

def check_sdpa_random_graphs(orc):
    for seed, N, E, H, D in [(0, 30, 100, 8, 64), (1, 17, 60, 3, 5), (2, 40, 400, 2, 16), (3, 9, 4, 1, 1)]:
        indptr, indices = tiny_graph(seed, N, E)
        Q, K, V = feats(seed, N, H, D)
        close(orc.fwd(indptr, indices, Q, K, V), sdpa_reference(indptr, indices, Q, K, V), 1e-11, 1e-12)


def check_complete_graph_textbook(orc):
    N, H, D = 12, 3, 8
    Q, K, V = feats(7, N, H, D)
    indptr = np.arange(N + 1, dtype=np.int64) * N
    indices = np.tile(np.arange(N, dtype=np.int32), N)
    out = orc.fwd(indptr, indices, Q, K, V)
    for h in range(H):
        q, k, v = (x[:, h, :].astype(np.float64) for x in (Q, K, V))
        ref = scipy.special.softmax(q @ k.T / math.sqrt(D), axis=1) @ v
        close(out[:, h, :], ref, 1e-11, 1e-12)


def check_golden(orc):
    for path in GOLDEN:
        g = json.load(open(path))
        Q, K, V = (np.array(g[k], dtype=np.float64) for k in ("Q", "K", "V"))
        indptr, indices = gtgen.coo_to_csr(g["N"], np.array(g["coo_src"]), np.array(g["coo_dst"]))
        assert indptr.tolist() == g["csr_indptr"] and indices.tolist() == g["csr_indices"], path
        out, s, a = orc.fwd(indptr, indices, Q, K, V, want_edges=True)
        close(out, g["out"], 1e-12, 1e-12)
        close(s, g["scores"], 1e-12, 1e-12)
        close(a, g["alpha"], 1e-12, 1e-12)
        # the unfused stages reach the same values
        s2 = orc.sddmm(indptr, indices, Q, K)
        close(s2, g["scores"], 1e-12, 1e-12)
        close(orc.edge_softmax(indptr, s2), g["alpha"], 1e-12, 1e-12)
        close(orc.spmm(indptr, indices, np.array(g["alpha"]), V), g["out"], 1e-12, 1e-12)


def check_sddmm_basis_vectors(orc):
    N, H, D = 6, 2, 6
    Q = np.zeros((N, H, D), np.float32)
    K = np.zeros((N, H, D), np.float32)
    for n in range(N):
        Q[n, 0, n] = 1.0
        K[n, 0, n] = 1.0
        Q[n, 1, (n + 1) % D] = 1.0
        K[n, 1, n] = 1.0
    indptr, indices = tiny_graph(11, N, 30)
    s = orc.sddmm(indptr, indices, Q, K)
    dst = dst_of_edges(indptr)
    exp0 = (dst == indices) / math.sqrt(D)
    exp1 = (((dst + 1) % D) == indices) / math.sqrt(D)
    assert np.array_equal(s[:, 0], exp0) and np.array_equal(s[:, 1], exp1)


def check_sddmm_vs_dense_product(orc):
    N, H, D = 20, 4, 16
    Q, K, _ = feats(5, N, H, D)
    indptr, indices = tiny_graph(5, N, 150)
    s = orc.sddmm(indptr, indices, Q, K)
    dst = dst_of_edges(indptr)
    for h in range(H):
        dense = Q[:, h, :].astype(np.float64) @ K[:, h, :].astype(np.float64).T / math.sqrt(D)
        close(s[:, h], dense[dst, indices], 1e-12, 1e-13)


def check_softmax_vs_scipy_and_invariants(orc):
    N, H = 25, 3
    indptr, _ = tiny_graph(9, N, 200)
    E = int(indptr[-1])
    s = np.random.default_rng(9).normal(size=(E, H)) * 3
    a = orc.edge_softmax(indptr, s)
    for v in range(N):
        b, e = indptr[v], indptr[v + 1]
        if e > b:
            close(a[b:e], scipy.special.softmax(s[b:e], axis=0), 1e-12, 1e-15)
            close(a[b:e].sum(0), np.ones(H), 1e-13, 0)
            assert np.all(a[b:e] > 0)
    # a per-(destination, head) constant leaves the weights unchanged
    shift = np.random.default_rng(1).normal(size=(N, H)) * 50
    close(orc.edge_softmax(indptr, s + shift[dst_of_edges(indptr)]), a, 1e-10, 1e-14)


def check_softmax_closed_forms(orc):
    # row 0: two edges -> logistic; row 1: one edge -> exactly 1; row 2: empty
    indptr = np.array([0, 2, 3, 3], np.int64)
    s = np.array([[0.3, -2.0], [-1.2, 5.0], [7.0, -7.0]])
    a = orc.edge_softmax(indptr, s)
    logistic = 1.0 / (1.0 + np.exp(s[1] - s[0]))
    close(a[0], logistic, 1e-14, 1e-16)
    close(a[1], 1.0 - logistic, 1e-14, 1e-16)
    assert np.array_equal(a[2], [1.0, 1.0])


def check_spmm_closed_forms(orc):
    N, H, D = 15, 2, 7
    _, _, V = feats(3, N, H, D)
    indptr, indices = tiny_graph(3, N, 60)
    E = len(indices)
    deg = np.diff(indptr)
    dst = dst_of_edges(indptr)
    # uniform weights -> mean of the source rows (multiplicities counted)
    a = np.repeat((1.0 / np.maximum(deg, 1))[:, None], H, 1)[dst]
    out = orc.spmm(indptr, indices, a, V)
    for v in range(N):
        ref = V[indices[indptr[v]:indptr[v + 1]]].astype(np.float64).mean(0) if deg[v] else np.zeros((H, D))
        close(out[v], ref, 1e-13, 1e-14)
    # linearity in V
    w = np.random.default_rng(2).random((E, H))
    V2 = V.astype(np.float64) * 3.0 - 1.0
    lhs = orc.spmm(indptr, indices, w, V2)
    rhs = 3.0 * orc.spmm(indptr, indices, w, V) - orc.spmm(indptr, indices, w, np.ones_like(V2))
    close(lhs, rhs, 1e-12, 1e-12)


def check_single_in_edge_copies_source(orc):
    # every destination has in-degree 1: alpha is exactly 1, out is the source row bit for bit
    N, H, D = 50, 8, 64
    Q, K, V = feats(21, N, H, D, scale=5.0)
    indptr = np.arange(N + 1, dtype=np.int64)
    indices = ((np.arange(N) * 7 + 3) % N).astype(np.int32)
    out, _, a = orc.fwd(indptr, indices, Q, K, V, want_edges=True)
    assert np.array_equal(a, np.ones_like(a))
    assert np.array_equal(out, V[indices].astype(np.float64))


def check_zero_in_degree_rows(orc):
    N, H, D = 40, 2, 4
    src, dst = gtgen.random_coo(4, N, 60)
    keep = dst % 3 != 0  # nodes 0, 3, 6, ... receive nothing
    indptr, indices = gtgen.coo_to_csr(N, src[keep], dst[keep])
    Q, K, V = feats(4, N, H, D)
    out = orc.fwd(indptr, indices, Q, K, V)
    empty = np.diff(indptr) == 0
    assert empty.sum() >= N // 3
    assert np.array_equal(out[empty], np.zeros_like(out[empty]))
    assert np.all(np.abs(out[~empty]).sum(axis=(1, 2)) > 0)


def check_relabel_equivariance(orc):
    N, H, D = 23, 2, 8
    src, dst = gtgen.random_coo(8, N, 90)
    Q, K, V = feats(8, N, H, D)
    perm = np.random.default_rng(8).permutation(N)
    inv = np.argsort(perm)
    out = orc.fwd(*gtgen.coo_to_csr(N, src, dst), Q, K, V)
    # node i is renamed perm[i]
    out_p = orc.fwd(*gtgen.coo_to_csr(N, perm[src], perm[dst]), Q[inv], K[inv], V[inv])
    close(out_p[perm], out, 1e-12, 1e-13)


def check_large_logits(orc):
    N, H, D = 30, 2, 16
    indptr, indices = tiny_graph(12, N, 120)
    Q, K, V = feats(12, N, H, D)
    Qb = Q * np.float32(1000.0)
    out = orc.fwd(indptr, indices, Qb, K, V)
    close(out, sdpa_reference(indptr, indices, Qb, K, V), 1e-10, 1e-10)


def check_bf16_widening(orc):
    N, H, D = 16, 4, 32
    indptr, indices = tiny_graph(13, N, 70)
    Qb, Kb, Vb = (gtgen.normal_bf16(13, s, (N, H, D), 0.5) for s in (1, 2, 3))
    wide = [gtgen.bf16_bits_to_f32(x) for x in (Qb, Kb, Vb)]
    assert np.array_equal(orc.fwd(indptr, indices, Qb, Kb, Vb), orc.fwd(indptr, indices, *wide))
    close(orc.fwd(indptr, indices, Qb, Kb, Vb), sdpa_reference(indptr, indices, *wide), 1e-11, 1e-12)


def check_rows_subset(orc):
    N, H, D = 30, 3, 8
    indptr, indices = tiny_graph(14, N, 100)
    Q, K, V = feats(14, N, H, D)
    full, s, a = orc.fwd(indptr, indices, Q, K, V, want_edges=True)
    rows = np.array([29, 0, 7, 7, 3], np.int64)
    sub, s2, a2 = orc.fwd_rows(indptr, indices, Q, K, V, rows, want_edges=True)
    assert np.array_equal(sub, full[rows])
    sel = np.concatenate([np.arange(indptr[r], indptr[r + 1]) for r in rows])
    assert np.array_equal(s2, s[sel]) and np.array_equal(a2, a[sel])


ALL_CHECKS = [
    check_sdpa_random_graphs,
    check_complete_graph_textbook,
    check_golden,
    check_sddmm_basis_vectors,
    check_sddmm_vs_dense_product,
    check_softmax_vs_scipy_and_invariants,
    check_softmax_closed_forms,
    check_spmm_closed_forms,
    check_single_in_edge_copies_source,
    check_zero_in_degree_rows,
    check_relabel_equivariance,
    check_large_logits,
    check_bf16_widening,
    check_rows_subset,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_oracle_pin(check):
    check(oracle.default())


def test_golden_fixtures_present():
    assert len(GOLDEN) >= 3
    for p in GOLDEN:
        assert "citation" in json.load(open(p)), p
