"""A graph with more than 2^31 edges, on the GPU through the C ABI.

indptr is int64 and the kernels index edges with 64-bit positions; this test
holds them to that.  4,096 destinations share E = 2^31 + 2^21 + 4,097 edges (degrees
differ by at most one, sources uniform over the 4,096 nodes, H = 1, D = 4,
fp32).  The fused forward with lse and the three unfused stages run over the
whole graph; the oracle checks whole rows before, across and after edge
position 2^31: per-edge scores and weights of the unfused stages (a wrong
position reads another edge's source and fails at once), out and lse.
The backward is not run here: its source-sorted graph would have to be built
on the host, and the device builder takes E < 2^31.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.test_gpu_parity import F32_TOL, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

N, H, D = 4096, 1, 4
E = (1 << 31) + (1 << 21) + 4097  # position 2^31 falls a few rows before the last


def graph():
    deg = np.full(N, E // N, dtype=np.int64)
    deg[:E % N] += 1
    indptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(deg, out=indptr[1:])
    indices = np.random.default_rng(31).integers(0, N, size=E, dtype=np.int32)
    return indptr, indices


def test_more_than_2_31_edges():
    say("large: building %d edges on the host" % E)
    indptr, indices = graph()
    assert indptr[-1] == E
    Q, K, V = gtgen.make_features(N, H, D, gtgen.F32, 5, 1.0)
    d = dev()
    t_ip = torch.from_numpy(indptr).to(d)
    t_ix = torch.from_numpy(indices).to(d)
    tq, tk, tv = (torch.from_numpy(x).to(d) for x in (Q, K, V))
    # the rows holding edge positions 2^31 - 1 and 2^31, their neighbours, the first and last rows
    lo, hi = (int(np.searchsorted(indptr, p, side="right")) - 1 for p in ((1 << 31) - 1, 1 << 31))
    rows = np.unique(np.clip([0, lo - 1, lo, hi, hi + 1, N - 1], 0, N - 1)).astype(np.int64)
    assert indptr[lo] <= (1 << 31) - 1 < indptr[lo + 1] and indptr[hi] <= (1 << 31) < indptr[hi + 1]

    say("large: fused forward with lse")
    out, lse = gt.gt_sparse_mha_fwd_lse(t_ip, t_ix, tq, tk, tv)
    torch.cuda.synchronize()
    rout, rs, ra = oracle.fwd_rows(indptr, indices, Q, K, V, rows, want_edges=True)
    rows_t = torch.from_numpy(rows).to(d)
    assert_close(host(out[rows_t]), rout, F32_TOL, "out, rows around 2^31")
    seg = np.concatenate([[0], np.cumsum(indptr[rows + 1] - indptr[rows])])
    rlse = np.stack([logsumexp(rs[seg[i]:seg[i + 1]], axis=0) for i in range(len(rows))])
    glse = host(lse[rows_t])
    assert np.all(np.abs(glse - rlse) <= 1e-5 * (1 + np.abs(rlse))), "lse, rows around 2^31"
    del out, lse

    say("large: unfused stages")
    scores = gt.gt_sddmm(t_ip, t_ix, tq, tk)
    alpha = gt.gt_edge_softmax(t_ip, scores)
    out2 = gt.gt_spmm(t_ip, t_ix, alpha, tv)
    torch.cuda.synchronize()
    for i, v in enumerate(rows):
        b, e = int(indptr[v]), int(indptr[v + 1])
        assert_close(host(scores[b:e]), rs[seg[i]:seg[i + 1]], F32_TOL, "scores of row %d" % v)
        assert_close(host(alpha[b:e]), ra[seg[i]:seg[i + 1]], F32_TOL, "alpha of row %d" % v)
    assert_close(host(out2[rows_t]), rout, F32_TOL, "unfused out, rows around 2^31")
