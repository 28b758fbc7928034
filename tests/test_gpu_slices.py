"""More work items than one launch slice, on the GPU through the C ABI.

A launch covers at most 2^24 work items (rows plus chunks of split rows); a
graph with more is launched in several slices, each with its own item base.
N = 2^24 + 5,000 destinations, each with one in-edge from a uniform source,
except row 0 (1,500 in-edges) and row N - 1 (700 in-edges), which are split
into chunks; H = 1, D = 4, fp32.  The forward (with lse), the three unfused
stages and the backward run over two slices; the oracle checks rows on both
sides of the slice boundary, the split rows, and a random sample, and dK/dV
of sources sampled the same way.
"""
import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.bounds import OutTable, sub_graph
from tests.test_gpu_backward import F32_BTOL, bound_dkv, bound_dq, check_bound, check_lse
from tests.test_gpu_parity import F32_TOL, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

N, H, D = (1 << 24) + 5000, 1, 4
SLICE = 1 << 24


def graph():
    deg = np.ones(N, dtype=np.int64)
    deg[0], deg[N - 1] = 1500, 700
    indptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(deg, out=indptr[1:])
    indices = np.random.default_rng(24).integers(0, N, size=int(indptr[-1]), dtype=np.int32)
    return indptr, indices


def sampled(n_items_before_rows, n, rng):
    """Rows whose items sit on both sides of the slice boundary, the ends, and random rows."""
    b = SLICE - n_items_before_rows  # the first row launched in the second slice
    rows = np.concatenate([np.arange(b - 40, b + 40), [0, 1, n - 2, n - 1], rng.choice(n, 300, replace=False)])
    return np.unique(rows[(rows >= 0) & (rows < n)]).astype(np.int64)


def test_more_items_than_one_slice():
    say("slices: graph of %d rows" % N)
    indptr, indices = graph()
    E = int(indptr[-1])
    Q, K, V = gtgen.make_features(N, H, D, gtgen.F32, 3, 1.0)
    dO = gtgen.make_grad(N, H, D, gtgen.F32, 11)
    chunk = gt.gt_config_chunk_edges(E)
    # the host's upper bound of chunk items, which precede the rows
    max_heavy = min(N, E // (chunk + 1))
    max_chunks = E // chunk + max_heavy
    assert max_chunks + N > SLICE
    rng = np.random.default_rng(5)
    rows = sampled(max_chunks, N, rng)
    d = dev()
    tip, tix = torch.from_numpy(indptr).to(d), torch.from_numpy(indices).to(d)
    tq, tk, tv, tdo = (torch.from_numpy(x).to(d) for x in (Q, K, V, dO))
    rows_t = torch.from_numpy(rows).to(d)

    say("slices: fused forward with lse, E=%d" % E)
    out, lse = gt.gt_sparse_mha_fwd_lse(tip, tix, tq, tk, tv)
    torch.cuda.synchronize()
    rout, rs, ra = oracle.fwd_rows(indptr, indices, Q, K, V, rows, want_edges=True)
    assert_close(host(out[rows_t]), rout, F32_TOL, "out, rows around the slice boundary")
    rlse, rdelta = oracle.row_stats(indptr, indices, Q, K, V, dO)
    check_lse(host(lse[rows_t]), rlse[rows], "lse, rows around the slice boundary")

    say("slices: unfused stages")
    scores = gt.gt_sddmm(tip, tix, tq, tk)
    alpha = gt.gt_edge_softmax(tip, scores)
    out2 = gt.gt_spmm(tip, tix, alpha, tv)
    torch.cuda.synchronize()
    sel = sub_graph(indptr, indices, rows)[2]
    sel_t = torch.from_numpy(sel).to(d)
    assert_close(host(scores[sel_t]), rs, F32_TOL, "scores of the sampled rows")
    assert_close(host(alpha[sel_t]), ra, F32_TOL, "alpha of the sampled rows")
    assert_close(host(out2[rows_t]), rout, F32_TOL, "unfused out of the sampled rows")
    del scores, alpha, out2

    say("slices: backward")
    t_ip, t_ix = gtgen.source_sorted(indptr, indices)
    dq, dk, dv = gt.gt_sparse_mha_bwd(tip, tix, torch.from_numpy(t_ip).to(d), torch.from_numpy(t_ix).to(d), tq, tk,
                                      tv, out, tdo, lse)
    torch.cuda.synchronize()
    w = {"indptr": indptr, "indices": indices, "Q": Q, "K": K, "V": V, "dO": dO, "H": H, "D": D,
         "t_indptr": t_ip, "t_indices": t_ix}
    # sources: the same boundary for the source pass (its chunk bound differs), and random ones
    t_heavy = min(N, E // (chunk + 1))
    srcs = sampled(E // chunk + t_heavy, N, rng)
    need = np.union1d(rows, sub_graph(t_ip, t_ix, srcs)[1])
    outs = OutTable(oracle.fwd_rows(indptr, indices, Q, K, V, need), need)
    rq = oracle.dq_rows(indptr, indices, Q, K, V, dO, rlse, rdelta, rows)
    check_bound(host(dq[rows_t]), rq, bound_dq(w, rlse, outs, rows), F32_BTOL, "dQ around the slice boundary")
    rk, rv = oracle.dkv_sources(t_ip, t_ix, Q, K, V, dO, rlse, rdelta, srcs)
    BK, BV = bound_dkv(w, rlse, outs, srcs)
    srcs_t = torch.from_numpy(srcs).to(d)
    check_bound(host(dk[srcs_t]), rk, BK, F32_BTOL, "dK around the slice boundary")
    check_bound(host(dv[srcs_t]), rv, BV, F32_BTOL, "dV around the slice boundary")
