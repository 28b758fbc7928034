"""Parity of the logit variants (additive bias [E][H], edge weights [E]) and
attention dropout with the fp64 oracle, on the GPU, through the C ABI.

Forward: out with the forward tolerances (fp32 rtol 1e-5, atol 1e-6; bf16
rtol 2e-2, atol 1e-5) and lse to 1e-5 (1 + |lse|).  Backward: as in
test_gpu_backward, relative to the magnitude sums of each gradient, which
with dropout multipliers c_e (0 or 1/(1-p)) and weights w_e read

    B_dQ[v]  = sum over in-edges  alpha_e (c_e |dO_v|.|v_u| + |dO_v|.|out_v|) w_e |k_u| / sqrt(D)
    B_dK[u]  = sum over out-edges alpha_e (c_e |dO_v|.|v_u| + |dO_v|.|out_v|) w_e |q_v| / sqrt(D)
    B_dV[u]  = sum over out-edges alpha_e c_e |dO_v|
    B_db[e]  = alpha_e (c_e |dO_v|.|v_u| + |dO_v|.|out_v|)
    B_dw[e]  = sum over heads B_db[e] |q_v|.|k_u| / sqrt(D)

(rtol 1e-5 for fp32, 2e-2 for bf16).  The dropout mask the bound uses comes
from numpy's Philox4x64-10 generator, independently of both sides.  Neutral
options (zero bias, unit weights, p = 0) must reproduce the plain kernels to
rounding.
"""
import math

import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.bounds import OutTable, dest_bounds, source_bounds, sub_graph
from tests.test_gpu_backward import check_bound, check_lse, to_torch, with_grad
from tests.test_gpu_parity import (BF16_TOL, F32_TOL, assert_close, chunk_edges, dev, host, oracle_inputs,
                                   random_graph, sample_rows, say, say_split, to_dev, workload)

pytestmark = pytest.mark.gpu

F32_BTOL = (1e-5, 1e-7)
BF16_BTOL = (2e-2, 1e-5)


def tols(w):
    return (F32_TOL, F32_BTOL) if w["dtype"] == gtgen.F32 else (BF16_TOL, BF16_BTOL)


def keep_mask(seed, E, H, p):
    """c[e, h] for all edges: 0 or 1/(1-p), from numpy's Philox4x64-10 stream
    (word e*H + h, kept iff its upper 32 bits >= floor(p 2^32)); float32."""
    bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64))
    thresh = np.uint64(math.floor(p * 2.0 ** 32))
    out = np.empty(E * H, dtype=np.float32)
    step = 1 << 24
    for i in range(0, E * H, step):
        n = min(step, E * H - i)
        words = bg.random_raw(n).astype(np.uint64)
        out[i:i + n] = np.where((words >> np.uint64(32)) >= thresh, np.float32(1.0 / (1.0 - p)), np.float32(0.0))
    return out.reshape(E, H)


def make_opts(w, seed, bias=True, weights=True, p=0.0):
    rng = np.random.default_rng(seed)
    E, H = w["E"], w["H"]
    o = dict(bias=rng.normal(0, 1.0, (E, H)).astype(np.float32) if bias else None,
             ew=rng.uniform(0.2, 1.0, E).astype(np.float32) if weights else None,
             drop_p=p, seed=seed * 7919 + 3)
    return o


def gpu_opts(o):
    d = dev()
    return dict(bias=None if o["bias"] is None else torch.from_numpy(o["bias"]).to(d),
                edge_weight=None if o["ew"] is None else torch.from_numpy(o["ew"]).to(d),
                dropout_p=o["drop_p"], dropout_seed=o["seed"])


def oracle_opts(o):
    return dict(bias=o["bias"], ew=o["ew"], drop_p=o["drop_p"], seed=o["seed"])


def run_ex(w, o, t=None):
    t = t or to_dev(w)
    d = dev()
    t["dO"] = to_torch(w["dO"])
    tip, tix, tpm = gtgen.source_sorted(w["indptr"], w["indices"], want_perm=True)
    g = gpu_opts(o)
    out, lse = gt.gt_sparse_mha_fwd_ex(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], want_lse=True, **g)
    res = gt.gt_sparse_mha_bwd_ex(t["indptr"], t["indices"], torch.from_numpy(tip).to(d),
                                  torch.from_numpy(tix).to(d), torch.from_numpy(tpm).to(d), t["Q"], t["K"], t["V"],
                                  out, t["dO"], lse, want_dbias=True, want_dweight=True, **g)
    torch.cuda.synchronize()
    return (out, lse) + tuple(res)


def bound_opts(w, o):
    """The options as the bounds take them (tests.bounds), with the dropout
    multipliers of every edge drawn from numpy's Philox stream."""
    if o["drop_p"] and "c_all" not in o:
        o["c_all"] = keep_mask(o["seed"], w["E"], w["H"], o["drop_p"])
    return dict(ew=o["ew"], bias=o["bias"], c_all=o.get("c_all") if o["drop_p"] else None)


def check_full(w, o):
    say("ex %s N=%d E=%d H=%d D=%d dtype=%d bias=%s ew=%s p=%g chunk=%d" % (
        w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"], o["bias"] is not None, o["ew"] is not None,
        o["drop_p"], gt.gt_config_chunk_edges(w["E"])))
    out, lse, dq, dk, dv, dbias, dw = run_ex(w, o)
    ftol, btol = tols(w)
    kw = oracle_opts(o)
    rout, rlse = oracle.fwd_ex(*oracle_inputs(w), want_lse=True, **kw)
    assert_close(host(out), rout, ftol, "out " + w["name"])
    check_lse(host(lse), rlse, "lse " + w["name"])
    g = oracle.bwd_ex(*oracle_inputs(w), w["dO"], **kw)
    bopts = bound_opts(w, o)
    outs = OutTable(rout)
    allv = np.arange(w["N"])
    tip, tix, tpm = gtgen.source_sorted(w["indptr"], w["indices"], want_perm=True)
    rb = dest_bounds(w, g["lse"], outs, allv, opts=bopts)
    BK, BV = source_bounds(dict(w, t_indptr=tip, t_indices=tix), g["lse"], outs, allv, opts=bopts, t_perm=tpm)
    check_bound(host(dq), g["dq"], rb["dq"], btol, "dQ " + w["name"])
    check_bound(host(dk), g["dk"], BK, btol, "dK " + w["name"])
    check_bound(host(dv), g["dv"], BV, btol, "dV " + w["name"])
    check_bound(host(dbias)[rb["sel"]], g["dbias"][rb["sel"]], rb["db"], btol, "dbias " + w["name"])
    check_bound(host(dw)[rb["sel"]], g["dw"][rb["sel"]], rb["dw"], btol, "dweight " + w["name"])


VARIANTS = {
    "bias": dict(bias=True, weights=False, p=0.0),
    "weights": dict(bias=False, weights=True, p=0.0),
    "dropout": dict(bias=False, weights=False, p=0.25),
    "all": dict(bias=True, weights=True, p=0.4),
}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("name,chunk", [("tiny_random", 1024), ("tiny_random", 2), ("molecules", 1024),
                                        ("molecules", 3)])
def test_variants_small(variant, name, chunk):
    w = with_grad(workload(name))
    with chunk_edges(chunk):
        check_full(w, make_opts(w, 5, **VARIANTS[variant]))


@pytest.mark.parametrize("H,D", [(8, 64), (3, 5), (4, 33), (2, 256), (16, 64), (8, 32), (64, 4), (12, 64),
                                 (24, 64), (16, 32), (4, 128), (8, 16), (4, 64), (2, 64), (16, 16), (8, 128),
                                 (4, 256), (2, 128),
                                 (8, 48), (8, 40), (4, 24), (3, 12), (2, 80), (16, 48), (8, 96)])
@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
@pytest.mark.parametrize("p", [0.3, 0.0])  # the dropout kernels, and those of bias and weights alone
def test_variants_shapes(H, D, dtype, p):
    w = with_grad(random_graph(H * 100 + D, 60, 800, H, D, dtype))
    with chunk_edges(40):
        check_full(w, make_opts(w, H + D, bias=True, weights=True, p=p))


def test_one_hub_row_and_source():
    from tests.test_gpu_parity import custom
    N, E = 40, 2500
    other = gtgen.random_coo(3, N, E)[0]
    with chunk_edges(100):
        for src, dst in ((other, np.full(E, 9)), (np.full(E, 9), other)):
            w = with_grad(custom(N, src, dst, 8, 64, seed=7))
            check_full(w, make_opts(w, 8, bias=True, weights=True, p=0.2))


@pytest.mark.parametrize("name", ["regular16", "molecules"])
def test_neutral_options_match_the_plain_kernels(name):
    w = with_grad(workload(name))
    t = to_dev(w)
    d = dev()
    say("neutral options %s" % name)
    E, H = w["E"], w["H"]
    zeros = torch.zeros((E, H), dtype=torch.float32, device=d)
    ones = torch.ones(E, dtype=torch.float32, device=d)
    tip, tix, tpm = (torch.from_numpy(x).to(d) for x in gtgen.source_sorted(w["indptr"], w["indices"],
                                                                            want_perm=True))
    dO = to_torch(w["dO"])
    with chunk_edges(7):
        out, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        xout, xlse = gt.gt_sparse_mha_fwd_ex(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], want_lse=True,
                                             bias=zeros, edge_weight=ones)
        dq, dk, dv = gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, t["Q"], t["K"], t["V"], out, dO, lse)
        xq, xk, xv, _, _ = gt.gt_sparse_mha_bwd_ex(t["indptr"], t["indices"], tip, tix, tpm, t["Q"], t["K"],
                                                   t["V"], out, dO, lse, bias=zeros, edge_weight=ones,
                                                   want_dbias=True)
        torch.cuda.synchronize()
    # same arithmetic; the two kernel variants differ only in how the compiler
    # contracts multiply-adds around the logit, so agreement is to rounding
    for x, y in ((xout, out), (xlse, lse), (xq, dq), (xk, dk), (xv, dv)):
        assert torch.allclose(x, y, rtol=1e-5, atol=1e-6 * float(y.abs().max()))


def test_plan_with_options_is_bitwise_the_plain_call():
    w = with_grad(workload("regular16"))
    t = to_dev(w)
    o = make_opts(w, 12, bias=True, weights=True, p=0.3)
    g = gpu_opts(o)
    say("plan with options")
    with chunk_edges(5):
        out, lse, dq, dk, dv, db, dw = run_ex(w, o, t)
        plan = gt.gt_plan_create(t["indptr"], t["indices"], transpose=True)
        pout, plse = gt.gt_sparse_mha_fwd_plan(plan, t["Q"], t["K"], t["V"], want_lse=True, **g)
        pq, pk, pv, pb, pw = gt.gt_sparse_mha_bwd_plan(plan, t["Q"], t["K"], t["V"], out, t["dO"], lse,
                                                       want_dbias=True, want_dweight=True, **g)
        torch.cuda.synchronize()
    for x, y in ((pout, out), (plse, lse), (pq, dq), (pk, dk), (pv, dv), (pb, db), (pw, dw)):
        assert torch.equal(x, y)
    plan.destroy()


def test_dropout_is_deterministic_and_seeded():
    w = with_grad(workload("tiny_random"))
    t = to_dev(w)
    o = make_opts(w, 3, bias=False, weights=False, p=0.5)
    a = run_ex(w, o, dict(t))
    b = run_ex(w, o, dict(t))
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c = run_ex(w, dict(o, seed=o["seed"] + 1), dict(t))
    assert not torch.equal(a[0], c[0])


@pytest.mark.parametrize("name,p", [("powerlaw", 0.2), ("lognormal", 0.0)])
def test_variants_large_sampled(name, p):
    w = with_grad(workload(name))
    o = make_opts(w, 21, bias=True, weights=True, p=p)
    say("ex %s sampled N=%d E=%d" % (name, w["N"], w["E"]))
    out, lse, dq, dk, dv, dbias, dw = (host(x) for x in run_ex(w, o))
    ftol, btol = tols(w)
    kw = oracle_opts(o)
    chunk = gt.gt_config_chunk_edges(w["E"])
    rows = sample_rows(w["indptr"], chunk, n_random=600)
    say_split(w["indptr"], rows, chunk, "ex destinations " + name)
    rlse, rdelta = oracle.row_stats_ex(*oracle_inputs(w), w["dO"], **kw)
    check_lse(lse, rlse, "lse " + name)
    tip, tix, tpm = gtgen.source_sorted(w["indptr"], w["indices"], want_perm=True)
    srcs = sample_rows(tip, chunk, n_random=600, seed=1)
    say_split(tip, srcs, chunk, "ex sources " + name)
    need = np.union1d(rows, sub_graph(tip, tix, srcs)[1])
    outs = OutTable(oracle.fwd_ex(*oracle_inputs(w), rows=need, **kw), need)
    assert_close(out[rows], outs.take(rows), ftol, "out %s" % name)
    rdb = np.zeros((w["E"], w["H"]))
    rdw = np.zeros(w["E"])
    rq = oracle.dq_rows_ex(*oracle_inputs(w), w["dO"], rlse, rdelta, rows, dbias=rdb, dw=rdw, **kw)
    bopts = bound_opts(w, o)
    rb = dest_bounds(w, rlse, outs, rows, opts=bopts)
    check_bound(dq[rows], rq, rb["dq"], btol, "dQ %s (%d rows)" % (name, len(rows)))
    eds = rb["sel"]
    check_bound(dbias[eds], rdb[eds], rb["db"], btol, "dbias %s" % name)
    check_bound(dw[eds], rdw[eds], rb["dw"], btol, "dweight %s" % name)
    rk, rv = oracle.dkv_sources_ex(tip, tix, tpm, w["Q"], w["K"], w["V"], w["dO"], rlse, rdelta, srcs, **kw)
    BK, BV = source_bounds(dict(w, t_indptr=tip, t_indices=tix), rlse, outs, srcs, opts=bopts, t_perm=tpm)
    check_bound(dk[srcs], rk, BK, btol, "dK %s (%d sources)" % (name, len(srcs)))
    check_bound(dv[srcs], rv, BV, btol, "dV %s (%d sources)" % (name, len(srcs)))


@pytest.mark.parametrize("H,D,dtype", [(8, 48, gtgen.F32), (8, 96, gtgen.BF16), (6, 64, gtgen.F32), (16, 64, gtgen.F32),
                                       (16, 128, gtgen.BF16), (4, 128, gtgen.F32)])
@pytest.mark.parametrize("p", [0.3, 0.0])
def test_split_rows_every_layout(H, D, dtype, p):
    # a hub destination and a hub source split into chunks, with bias, weights
    # and dropout, for padded heads, rows that end before their last lane
    # group, wide rows and a compile-time layout
    from tests.test_gpu_parity import custom
    N, E = 60, 1500
    src, dst = gtgen.random_coo(H * 10 + D, N, E)
    dst = np.where(np.arange(E) < 500, 5, dst)
    src = np.where((np.arange(E) >= 500) & (np.arange(E) < 900), 9, src)
    w = with_grad(custom(N, src, dst, H, D, dtype, seed=H * D))
    with chunk_edges(37):
        check_full(w, make_opts(w, H + 2 * D, bias=True, weights=True, p=p))
