"""Feature arrays of more than 2^31 elements, on the GPU through the C ABI.

Element offsets into Q, K, V, out and the gradients are 64-bit; this test
holds the kernels to that.  N = 2^22 + 3 nodes of H = 8 heads x D = 64, fp32
(512 elements per node, 8.6 GB per array): the last three nodes start at
element 2^31 and beyond.  Every destination has 4 in-edges from uniform
sources below those three; the last row has 1,500 in-edges, so it is split
into chunks and merged.  A few sampled rows (the first, the last two below
element 2^31, the last three) also take in-edges from the three top nodes,
which have no other out-edges.  The oracle, run on the subgraph of the sampled rows
and their sources, then gives out, scores and weights of the sampled rows,
their dQ, and dK and dV of the three top nodes exactly: the fused forward with
lse, the three unfused stages and the backward on a plan are checked there.
Features are drawn on the device (seeded normal values); only the subgraph's
rows come back to the host.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.bounds import OutTable
from tests.test_gpu_backward import bound_dkv, bound_dq, check_bound, F32_BTOL
from tests.test_gpu_parity import F32_TOL, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

N, H, D = (1 << 22) + 3, 8, 64
TOP = np.arange(N - 3, N, dtype=np.int64)  # first elements at 2^31, 2^31 + 512, 2^31 + 1024
SAMPLED = np.array([0, (1 << 22) - 2, (1 << 22) - 1, N - 3, N - 2, N - 1], dtype=np.int64)
BIG_ROW = N - 1
BIG_DEG = 1500


def graph():
    deg = np.full(N, 4, dtype=np.int64)
    deg[BIG_ROW] = BIG_DEG
    indptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(deg, out=indptr[1:])
    indices = np.random.default_rng(22).integers(0, N - 3, size=int(indptr[-1]), dtype=np.int32)
    # each sampled row takes one in-edge from a top node; the split row takes
    # all three, in its first, a middle and its last chunk
    for i, v in enumerate(SAMPLED):
        indices[indptr[v] + 1] = TOP[i % 3]
    b = indptr[BIG_ROW]
    indices[b + np.array([0, 700, BIG_DEG - 1])] = TOP
    return indptr, indices


def subgraph(indptr, indices):
    """The sampled rows (local ids 0..5) and every source they read, relabelled:
    (local indptr, local indices, global id of each local node)."""
    srcs = np.unique(np.concatenate([indices[indptr[v]:indptr[v + 1]] for v in SAMPLED]).astype(np.int64))
    nodes = np.concatenate([SAMPLED, np.setdiff1d(srcs, SAMPLED)])
    local = {int(g): i for i, g in enumerate(nodes)}
    deg = np.zeros(len(nodes), dtype=np.int64)
    deg[:len(SAMPLED)] = indptr[SAMPLED + 1] - indptr[SAMPLED]
    lip = np.zeros(len(nodes) + 1, dtype=np.int64)
    np.cumsum(deg, out=lip[1:])
    lix = np.concatenate([[local[int(u)] for u in indices[indptr[v]:indptr[v + 1]]] for v in SAMPLED])
    return lip, lix.astype(np.int32), nodes


def test_more_than_2_31_feature_elements():
    say("huge features: graph of %d nodes" % N)
    indptr, indices = graph()
    E = int(indptr[-1])
    d = dev()
    gen = torch.Generator(device=d)
    gen.manual_seed(2024)
    Q, K, V, dO = (torch.randn(N, H, D, device=d, generator=gen) for _ in range(4))
    assert Q.numel() > (1 << 31)
    tip = torch.from_numpy(indptr).to(d)
    tix = torch.from_numpy(indices).to(d)

    lip, lix, nodes = subgraph(indptr, indices)
    nodes_t = torch.from_numpy(nodes).to(d)
    lQ, lK, lV, ldO = (np.ascontiguousarray(host(x[nodes_t]).astype(np.float32)) for x in (Q, K, V, dO))
    rows = np.arange(len(SAMPLED))
    rout, rs, ra = oracle.fwd_rows(lip, lix, lQ, lK, lV, rows, want_edges=True)
    sam_t = torch.from_numpy(SAMPLED).to(d)

    say("huge features: fused forward with lse, E=%d" % E)
    out, lse = gt.gt_sparse_mha_fwd_lse(tip, tix, Q, K, V)
    torch.cuda.synchronize()
    assert_close(host(out[sam_t]), rout, F32_TOL, "out of the sampled rows")
    rlse = np.stack([logsumexp(rs[lip[i]:lip[i + 1]], axis=0) for i in rows])
    glse = host(lse[sam_t])
    assert np.all(np.abs(glse - rlse) <= 1e-5 * (1 + np.abs(rlse))), "lse of the sampled rows"

    say("huge features: unfused stages")
    scores = gt.gt_sddmm(tip, tix, Q, K)
    alpha = gt.gt_edge_softmax(tip, scores)
    out2 = gt.gt_spmm(tip, tix, alpha, V)
    torch.cuda.synchronize()
    for i, v in enumerate(SAMPLED):
        b, e = int(indptr[v]), int(indptr[v + 1])
        assert_close(host(scores[b:e]), rs[lip[i]:lip[i + 1]], F32_TOL, "scores of row %d" % v)
        assert_close(host(alpha[b:e]), ra[lip[i]:lip[i + 1]], F32_TOL, "alpha of row %d" % v)
    assert_close(host(out2[sam_t]), rout, F32_TOL, "unfused out of the sampled rows")
    del scores, alpha, out2

    say("huge features: backward on a plan")
    plan = gt.gt_plan_create(tip, tix, transpose=True)
    dq, dk, dv = gt.gt_sparse_mha_bwd_plan(plan, Q, K, V, out, dO, lse)
    torch.cuda.synchronize()
    plan.destroy()
    w = {"indptr": lip, "indices": lix, "Q": lQ, "K": lK, "V": lV, "dO": ldO, "H": H, "D": D}
    w["t_indptr"], w["t_indices"] = gtgen.source_sorted(lip, lix)
    rq, rk, rv, olse, _ = oracle.bwd(lip, lix, lQ, lK, lV, ldO)
    full_out = oracle.fwd(lip, lix, lQ, lK, lV)
    out_of = OutTable(full_out)
    check_bound(host(dq[sam_t]), rq[rows], bound_dq(w, olse, out_of, rows), F32_BTOL, "dQ of the sampled rows")
    top_local = np.array([np.nonzero(nodes == g)[0][0] for g in TOP])
    BK, BV = bound_dkv(w, olse, out_of, top_local)
    top_t = torch.from_numpy(TOP).to(d)
    check_bound(host(dk[top_t]), rk[top_local], BK, F32_BTOL, "dK of the top nodes")
    check_bound(host(dv[top_t]), rv[top_local], BV, F32_BTOL, "dV of the top nodes")
    del Q, K, V, dO, out, lse, dq, dk, dv
    torch.cuda.empty_cache()
