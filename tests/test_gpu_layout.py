"""The head-innermost feature layout [N][D][H] ("Graph Transformer in a
Nutshell", SparseMHA.forward reshapes q, k, v to [N, dh, nh]) on the GPU.

* Every shape: out and lse against the oracle with the forward tolerances,
  and dQ, dK, dV against the oracle with the backward's bound tolerances,
  whole rows and split rows.  Shapes the head-innermost kernels can take (H a
  multiple of the 16-byte vector with a power-of-two quotient, D*H within
  4 KB) run them or the copies route, whichever the library's cost rule picks.
* Shapes outside that range and the logit options always run the [N][H][D]
  kernels on transposed copies: bit-identical to the [N][H][D] calls.
The oracle works on [N][H][D]; a layout is a permutation of each row, so the
expected values are the oracle's, permuted.
"""
import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.bounds import OutTable
from tests.test_gpu_backward import bound_dkv, bound_dq, btol_of, check_bound, check_lse, to_torch, with_grad
from tests.test_gpu_parity import (assert_close, chunk_edges, custom, dev, host, oracle_inputs, random_graph,
                                   sample_rows, say, say_split, to_dev, tol_of, workload)

pytestmark = pytest.mark.gpu


def ndh(t):
    """[N][H][D] -> [N][D][H] (device tensor)."""
    return t.transpose(1, 2).contiguous()


def nhd(t):
    return t.transpose(1, 2).contiguous()


def takes_kernel(w):
    vn = 4 if w["dtype"] == gtgen.F32 else 8
    hv = w["H"] // vn
    return w["H"] % vn == 0 and hv & (hv - 1) == 0 and w["D"] * hv <= 256


def check_fwd(w):
    say("ndh fwd %s N=%d E=%d H=%d D=%d dtype=%d kernel=%s chunk=%d" % (
        w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"], takes_kernel(w),
        gt.gt_config_chunk_edges(w["E"])))
    t = to_dev(w)
    out, lse = gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]),
                                           layout="ndh", want_lse=True)
    ref_out, ref_lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    torch.cuda.synchronize()
    rout = oracle.fwd(*oracle_inputs(w))
    rlse, _ = oracle.row_stats(*oracle_inputs(w), w["Q"])
    assert_close(host(nhd(out)), rout, tol_of(w), "ndh out " + w["name"])
    check_lse(host(lse), rlse, "ndh lse " + w["name"])
    if not takes_kernel(w):  # transposed copies through the [N][H][D] kernels
        assert torch.equal(nhd(out), ref_out) and torch.equal(lse, ref_lse)


@pytest.mark.parametrize("name", ["molecules", "tiny_random"])
@pytest.mark.parametrize("chunk", [1024, 2, 5])
def test_ndh_workloads(name, chunk):
    with chunk_edges(chunk):
        check_fwd(workload(name))


def test_ndh_molecules_bf16():
    w = dict(workload("molecules"))
    w["dtype"] = gtgen.BF16
    w["Q"], w["K"], w["V"] = gtgen.make_features(w["N"], w["H"], w["D"], gtgen.BF16, 0, 0.5)
    for chunk in (1024, 3):
        with chunk_edges(chunk):
            check_fwd(w)


@pytest.mark.parametrize("H,D", [(4, 16), (16, 4), (64, 1), (8, 8), (32, 2), (4, 1), (8, 10), (3, 5), (2, 7),
                                 (8, 64), (12, 4), (16, 64), (4, 100), (32, 32), (8, 200), (64, 16), (8, 48), (8, 96)])
@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
def test_ndh_shapes(H, D, dtype):
    with chunk_edges(30):
        check_fwd(random_graph(H * 37 + D, 80, 900, H, D, dtype))


def test_ndh_zero_edges_and_hub_row():
    w = custom(20, [], [], 8, 10)
    t = to_dev(w)
    out = torch.full((20, 10, 8), float("nan"), device=dev())
    say("ndh E=0")
    gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]), out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    N, E = 40, 2000
    src = gtgen.random_coo(3, N, E)[0]
    with chunk_edges(64):
        check_fwd(custom(N, src, np.full(E, 5), 8, 10, seed=3))


def check_bwd(w):
    """GPU forward then backward in the head-innermost layout, against the
    oracle's gradients (the backward consumes the GPU's own out and lse)."""
    w = with_grad(w)
    say("ndh bwd %s N=%d E=%d H=%d D=%d dtype=%d kernel=%s chunk=%d" % (
        w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"], takes_kernel(w),
        gt.gt_config_chunk_edges(w["E"])))
    t = to_dev(w)
    d = dev()
    tip, tix = (torch.from_numpy(x).to(d) for x in (w["t_indptr"], w["t_indices"]))
    out, lse = gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]),
                                           layout="ndh", want_lse=True)
    dq, dk, dv, _, _ = gt.gt_sparse_mha_bwd_layout(t["indptr"], t["indices"], tip, tix, None, ndh(t["Q"]),
                                                   ndh(t["K"]), ndh(t["V"]), out, ndh(to_torch(w["dO"])), lse,
                                                   layout="ndh")
    torch.cuda.synchronize()
    rq, rk, rv, rlse, _ = oracle.bwd(*oracle_inputs(w), w["dO"])
    check_lse(host(lse), rlse, "ndh lse " + w["name"])
    outs = OutTable(oracle.fwd(*oracle_inputs(w)))
    allv = np.arange(w["N"])
    BK, BV = bound_dkv(w, rlse, outs, allv)
    tol = btol_of(w)
    check_bound(host(nhd(dq)), rq, bound_dq(w, rlse, outs, allv), tol, "ndh dQ " + w["name"])
    check_bound(host(nhd(dk)), rk, BK, tol, "ndh dK " + w["name"])
    check_bound(host(nhd(dv)), rv, BV, tol, "ndh dV " + w["name"])


@pytest.mark.parametrize("name", ["molecules", "tiny_random"])
@pytest.mark.parametrize("chunk", [1024, 2, 5])
def test_ndh_bwd_workloads(name, chunk):
    with chunk_edges(chunk):
        check_bwd(workload(name))


def test_ndh_bwd_molecules_bf16():
    w = dict(workload("molecules"))
    w["dtype"] = gtgen.BF16
    w["Q"], w["K"], w["V"] = gtgen.make_features(w["N"], w["H"], w["D"], gtgen.BF16, 0, 0.5)
    for chunk in (1024, 3):
        with chunk_edges(chunk):
            check_bwd(w)


@pytest.mark.parametrize("H,D", [(4, 16), (16, 4), (64, 1), (8, 8), (32, 2), (4, 1), (8, 10), (3, 5), (8, 64),
                                 (12, 4), (16, 64), (4, 100), (32, 32), (8, 200), (64, 16), (8, 48), (8, 96)])
@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
def test_ndh_bwd_shapes(H, D, dtype):
    with chunk_edges(30):
        check_bwd(random_graph(H * 41 + D, 80, 900, H, D, dtype))


@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
def test_ndh_bwd_word_shape_large_graph(dtype):
    # 8 x 10 heads on 70 K edges, a hub destination split into chunks: the
    # backward runs on [N][H][D] copies in the word layout, so its gradients
    # are the [N][H][D] call's, bit for bit, given the same out and lse
    N, E = 8000, 70000
    src, dst = gtgen.random_coo(77, N, E)
    dst = np.where(np.arange(E) < 3000, 11, dst)
    w = with_grad(custom(N, src, dst, 8, 10, dtype, seed=77))
    check_bwd(w)
    t = to_dev(w)
    d = dev()
    tip, tix = (torch.from_numpy(x).to(d) for x in (w["t_indptr"], w["t_indices"]))
    out, lse = gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]),
                                           layout="ndh", want_lse=True)
    dO = to_torch(w["dO"])
    g = gt.gt_sparse_mha_bwd_layout(t["indptr"], t["indices"], tip, tix, None, ndh(t["Q"]), ndh(t["K"]),
                                    ndh(t["V"]), out, ndh(dO), lse, layout="ndh")
    ref = gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, t["Q"], t["K"], t["V"], nhd(out), dO, lse)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(nhd(g[i]), ref[i]), "gradient %d" % i


def test_ndh_bwd_zero_edges_and_hub_source():
    w = with_grad(custom(20, [], [], 8, 10))
    t = to_dev(w)
    d = dev()
    tip, tix = (torch.from_numpy(x).to(d) for x in (w["t_indptr"], w["t_indices"]))
    lse = torch.full((20, 8), float("-inf"), device=d)
    z = torch.zeros((20, 10, 8), device=d)
    say("ndh bwd E=0")
    g = gt.gt_sparse_mha_bwd_layout(t["indptr"], t["indices"], tip, tix, None, ndh(t["Q"]), ndh(t["K"]),
                                    ndh(t["V"]), z, ndh(to_torch(w["dO"])), lse, layout="ndh")
    torch.cuda.synchronize()
    assert all(torch.all(x == 0) for x in g[:3])
    # one source feeding every destination many times: a split source row
    N, E = 40, 2000
    dst = np.sort(gtgen.random_coo(5, N, E)[1])
    with chunk_edges(64):
        check_bwd(custom(N, np.full(E, 7), dst, 8, 10, seed=5))


def test_ndh_options_are_the_nhd_calls():
    w = with_grad(workload("molecules"))
    t = to_dev(w)
    d = dev()
    E, H = w["E"], w["H"]
    rng = np.random.default_rng(4)
    opts = dict(bias=torch.from_numpy(rng.normal(0, 1, (E, H)).astype(np.float32)).to(d),
                edge_weight=torch.from_numpy(rng.uniform(0.2, 1, E).astype(np.float32)).to(d),
                dropout_p=0.2, dropout_seed=77)
    tip, tix, tpm = (torch.from_numpy(x).to(d) for x in gtgen.source_sorted(w["indptr"], w["indices"],
                                                                            want_perm=True))
    dO = to_torch(w["dO"])
    say("ndh with options and backward")
    with chunk_edges(4):
        out, lse = gt.gt_sparse_mha_fwd_ex(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], want_lse=True, **opts)
        nout, nlse = gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]),
                                                 layout="ndh", want_lse=True, **opts)
        g = gt.gt_sparse_mha_bwd_ex(t["indptr"], t["indices"], tip, tix, tpm, t["Q"], t["K"], t["V"], out, dO, lse,
                                    want_dbias=True, want_dweight=True, **opts)
        ng = gt.gt_sparse_mha_bwd_layout(t["indptr"], t["indices"], tip, tix, tpm, ndh(t["Q"]), ndh(t["K"]),
                                         ndh(t["V"]), ndh(out), ndh(dO), lse, layout="ndh", want_dbias=True,
                                         want_dweight=True, **opts)
        torch.cuda.synchronize()
    assert torch.equal(nhd(nout), out) and torch.equal(nlse, lse)
    for a, b in zip(ng[:3], g[:3]):
        assert torch.equal(nhd(a), b)
    assert torch.equal(ng[3], g[3]) and torch.equal(ng[4], g[4])


def test_ndh_large_sampled():
    # the power-law workload in the head-innermost layout (8 x 64 fp32: 128 vectors a
    # row, two per lane), sampled rows against the oracle
    w = workload("powerlaw")
    t = to_dev(w)
    say("ndh powerlaw kernel=%s" % takes_kernel(w))
    out, lse = gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]),
                                           want_lse=True)
    torch.cuda.synchronize()
    chunk = gt.gt_config_chunk_edges(w["E"])
    rows = sample_rows(w["indptr"], chunk, n_random=400)
    say_split(w["indptr"], rows, chunk, "ndh powerlaw")
    rows_t = torch.from_numpy(rows).to(dev())
    rout = oracle.fwd_rows(*oracle_inputs(w), rows)
    assert_close(host(nhd(out[rows_t])), rout, tol_of(w), "ndh powerlaw out (%d sampled rows)" % len(rows))
