"""The head-innermost feature layout [N][D][H] ("Graph Transformer in a
Nutshell", SparseMHA.forward reshapes q, k, v to [N, dh, nh]) on the GPU.

* Shapes the head-innermost kernel takes (H a multiple of the 16-byte vector
  with a power-of-two quotient, D*H within 1 KB): out and lse against the
  oracle with the forward tolerances, whole rows and split rows.
* Other shapes, the logit options and the backward run the [N][H][D] kernels
  on transposed copies: bit-identical to the [N][H][D] calls.
The oracle works on [N][H][D]; a layout is a permutation of each row, so the
expected values are the oracle's, permuted.
"""
import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.test_gpu_backward import check_lse, to_torch, with_grad
from tests.test_gpu_parity import (assert_close, chunk_edges, custom, dev, host, oracle_inputs, random_graph, say,
                                   to_dev, tol_of, workload)

pytestmark = pytest.mark.gpu


def ndh(t):
    """[N][H][D] -> [N][D][H] (device tensor)."""
    return t.transpose(1, 2).contiguous()


def nhd(t):
    return t.transpose(1, 2).contiguous()


def takes_kernel(w):
    vn = 4 if w["dtype"] == gtgen.F32 else 8
    hv = w["H"] // vn
    return w["H"] % vn == 0 and hv & (hv - 1) == 0 and w["D"] * hv <= 64


def check_fwd(w):
    say("ndh fwd %s N=%d E=%d H=%d D=%d dtype=%d kernel=%s chunk=%d" % (
        w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"], takes_kernel(w),
        gt.gt_config_get(gt.GT_CFG_CHUNK_EDGES)))
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
                                 (8, 64), (12, 4)])
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


def test_ndh_options_and_backward_are_the_nhd_calls():
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
        plain = gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, t["Q"], t["K"], t["V"], out, dO, lse)
        nplain = gt.gt_sparse_mha_bwd_layout(t["indptr"], t["indices"], tip, tix, None, ndh(t["Q"]), ndh(t["K"]),
                                             ndh(t["V"]), ndh(out), ndh(dO), lse, layout="ndh")
        torch.cuda.synchronize()
    assert torch.equal(nhd(nout), out) and torch.equal(nlse, lse)
    for a, b in zip(ng[:3], g[:3]):
        assert torch.equal(nhd(a), b)
    assert torch.equal(ng[3], g[3]) and torch.equal(ng[4], g[4])
    for a, b in zip(nplain[:3], plain):
        assert torch.equal(nhd(a), b)


def test_ndh_large_sampled():
    # power-law shape in the head-innermost layout (8 x 64 fp32: through the copies)
    w = workload("powerlaw")
    t = to_dev(w)
    say("ndh powerlaw")
    out = gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], ndh(t["Q"]), ndh(t["K"]), ndh(t["V"]))
    ref = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    torch.cuda.synchronize()
    assert torch.equal(nhd(out), ref)
