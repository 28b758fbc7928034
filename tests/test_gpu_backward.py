"""Parity of the HIP backward (gt_sparse_mha_fwd_lse + gt_sparse_mha_bwd, through
the C ABI) with the fp64 oracle, on the GPU.

The backward consumes the GPU forward's own out and lse, as a training step
does.  Tolerances are relative to the magnitude sums of each gradient, which
bound both the gradient and the rounding errors of its terms (ds_e =
alpha_e (da_e - delta_v) never exceeds alpha_e (|dO_v|.|v_u| + |dO_v|.|out_v|)):

    B_dQ[v] = sum over in-edges  alpha_e (|dO_v|.|v_u| + |dO_v|.|out_v|) |k_u| / sqrt(D)
    B_dK[u] = sum over out-edges alpha_e (|dO_v|.|v_u| + |dO_v|.|out_v|) |q_v| / sqrt(D)
    B_dV[u] = sum over out-edges alpha_e |dO_v|

elementwise |gpu - oracle| <= rtol * B + atol, with (rtol, atol) = (1e-5,
1e-7) for fp32 and (2e-2, 1e-5) for bf16 (the forward's rtol applied to the
bound: fp32 accumulation of fp32 terms; bf16 rounds out, which enters delta,
and the stored gradients, each by at most 2^-9 of B).  The forward's
log-sum-exp is checked to 1e-5 (1 + |lse|), and -inf exactly for rows
without in-edges.
"""
import math

import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests import bounds
from tests.bounds import OutTable, sub_graph
from tests.test_gpu_parity import (WORD_SHAPES, check_fused_full, chunk_edges, custom, dev, host, hub_graph,
                                   oracle_inputs, random_graph, sample_rows, say, say_split, to_dev, workload)

pytestmark = pytest.mark.gpu

F32_BTOL = (1e-5, 1e-7)
BF16_BTOL = (2e-2, 1e-5)
LSE_TOL = 1e-5


def btol_of(w):
    return F32_BTOL if w["dtype"] == gtgen.F32 else BF16_BTOL


def widen(x):
    return gtgen.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def to_torch(x):
    d = dev()
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(d).view(torch.bfloat16)
    return torch.from_numpy(x).to(d)


def with_grad(w, seed=None):
    w = dict(w)
    w["dO"] = gtgen.make_grad(w["N"], w["H"], w["D"], w["dtype"], 11 if seed is None else seed)
    w["t_indptr"], w["t_indices"] = gtgen.source_sorted(w["indptr"], w["indices"])
    return w


def run_gpu(w, t=None):
    """GPU forward (out, lse) then backward (dQ, dK, dV), as device tensors."""
    t = t or to_dev(w)
    t["dO"] = to_torch(w["dO"])
    t["t_indptr"] = torch.from_numpy(w["t_indptr"]).to(dev())
    t["t_indices"] = torch.from_numpy(w["t_indices"]).to(dev())
    out, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    dq, dk, dv = gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], t["t_indptr"], t["t_indices"], t["Q"], t["K"],
                                      t["V"], out, t["dO"], lse)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def bound_dq(w, lse, outs, rows):
    """B_dQ of the listed destinations; outs is a bounds.OutTable of the oracle's out."""
    return bounds.dest_bounds(w, lse, outs, rows)["dq"]


def bound_dkv(w, lse, outs, srcs):
    """(B_dK, B_dV) of the listed sources."""
    return bounds.source_bounds(w, lse, outs, srcs)


def check_bound(g, o, B, tol, what):
    rtol, atol = tol
    g = np.asarray(g, np.float64)
    assert g.shape == o.shape == B.shape, (what, g.shape, o.shape, B.shape)
    assert np.all(np.isfinite(g)), what + ": non-finite GPU output"
    err = np.abs(g - o)
    excess = err - (atol + rtol * B)
    bad = int((excess > 0).sum())
    worst = float((err / (B + atol / rtol)).max()) if err.size else 0.0
    say("%s: worst |err| / B = %.3e (rtol %.1e)" % (what, worst, rtol))
    assert bad == 0, "%s: %d elements out of tolerance, worst excess %.3e at %s (gpu %r, oracle %r, B %r)" % (
        what, bad, excess.max(), np.unravel_index(excess.argmax(), excess.shape), g.flat[excess.argmax()],
        o.flat[excess.argmax()], B.flat[excess.argmax()])


def check_lse(g, o, what):
    g = np.asarray(g, np.float64)
    fin = np.isfinite(o)
    assert np.all(g[~fin] == -np.inf), what + ": rows without in-edges must have lse = -inf"
    assert np.all(np.abs(g[fin] - o[fin]) <= LSE_TOL * (1 + np.abs(o[fin]))), what


def check_bwd_full(w, tol=None):
    say("bwd %s N=%d E=%d H=%d D=%d dtype=%d chunk=%d" % (w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"],
                                                          gt.gt_config_chunk_edges(w["E"])))
    res = run_gpu(w)
    _, lse, dq, dk, dv = res
    rq, rk, rv, rlse, _ = oracle.bwd(*oracle_inputs(w), w["dO"])
    check_lse(host(lse), rlse, "lse " + w["name"])
    outs = OutTable(oracle.fwd(*oracle_inputs(w)))
    allv = np.arange(w["N"])
    BK, BV = bound_dkv(w, rlse, outs, allv)
    tol = tol or btol_of(w)
    check_bound(host(dq), rq, bound_dq(w, rlse, outs, allv), tol, "dQ " + w["name"])
    check_bound(host(dk), rk, BK, tol, "dK " + w["name"])
    check_bound(host(dv), rv, BV, tol, "dV " + w["name"])
    return res


def check_bwd_sampled(w, n_random=800):
    """Destinations and sources sampled (split rows, rows at the chunk threshold,
    empty rows, random ones), the oracle computing them one by one."""
    say("bwd %s sampled, N=%d E=%d" % (w["name"], w["N"], w["E"]))
    _, lse, dq, dk, dv = (host(x) for x in run_gpu(w))
    chunk = gt.gt_config_chunk_edges(w["E"])
    rlse, rdelta = oracle.row_stats(*oracle_inputs(w), w["dO"])
    check_lse(lse, rlse, "lse " + w["name"])
    tol = btol_of(w)

    rows = sample_rows(w["indptr"], chunk, n_random=n_random)
    srcs = sample_rows(w["t_indptr"], chunk, n_random=n_random, seed=1)
    say_split(w["indptr"], rows, chunk, "bwd destinations")
    say_split(w["t_indptr"], srcs, chunk, "bwd sources")
    need = np.union1d(rows, sub_graph(w["t_indptr"], w["t_indices"], srcs)[1])
    outs = OutTable(oracle.fwd_rows(*oracle_inputs(w), need), need)

    rq = oracle.dq_rows(*oracle_inputs(w), w["dO"], rlse, rdelta, rows)
    check_bound(dq[rows], rq, bound_dq(w, rlse, outs, rows), tol,
                "dQ %s (%d sampled rows)" % (w["name"], len(rows)))
    rk, rv = oracle.dkv_sources(w["t_indptr"], w["t_indices"], w["Q"], w["K"], w["V"], w["dO"], rlse, rdelta, srcs)
    BK, BV = bound_dkv(w, rlse, outs, srcs)
    check_bound(dk[srcs], rk, BK, tol, "dK %s (%d sampled sources)" % (w["name"], len(srcs)))
    check_bound(dv[srcs], rv, BV, tol, "dV %s (%d sampled sources)" % (w["name"], len(srcs)))


# ------------------------------------------------------------------ forward with lse

@pytest.mark.parametrize("name", ["tiny_random", "molecules"])
@pytest.mark.parametrize("chunk", [1024, 1, 3])
def test_fwd_lse_small(name, chunk):
    w = workload(name)
    t = to_dev(w)
    with chunk_edges(chunk):
        say("fwd_lse %s chunk=%d" % (name, chunk))
        out, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        plain = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        torch.cuda.synchronize()
    assert torch.equal(out, plain), "the lse variant must leave out bit-identical"
    rlse, _ = oracle.row_stats(*oracle_inputs(w), w["Q"])
    check_lse(host(lse), rlse, "lse " + name)


# ------------------------------------------------------------------ backward, whole outputs

@pytest.mark.parametrize("name", ["tiny_random", "molecules"])
@pytest.mark.parametrize("chunk", [1024, 1, 2, 5])
def test_bwd_small_workloads(name, chunk):
    with chunk_edges(chunk):
        check_bwd_full(with_grad(workload(name)))


def test_bwd_regular16_sampled():
    check_bwd_sampled(with_grad(workload("regular16")))


@pytest.mark.parametrize("H,D", [(1, 1), (3, 5), (2, 7), (1, 64), (4, 33), (8, 100), (2, 256), (16, 64),
                                 (5, 16), (64, 4), (3, 128), (12, 64), (3, 256), (24, 64),
                                 (1, 4), (1, 8), (2, 4), (16, 32), (4, 128), (8, 32), (16, 16), (8, 16), (4, 32),
                                 (2, 64), (8, 64), (8, 128), (4, 256), (4, 64), (2, 128),
                                 (8, 48), (8, 40), (4, 24), (3, 12), (2, 80), (16, 48), (8, 96)])
@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
def test_bwd_shapes(H, D, dtype):
    with chunk_edges(40):
        check_bwd_full(with_grad(random_graph(H * 1000 + D, 70, 900, H, D, dtype)))


@pytest.mark.parametrize("chunk", [1024, 100, 7])
def test_bwd_one_destination_and_one_source(chunk):
    # every edge into node 7 (a split row of the destination pass), then every
    # edge out of node 7 (a split row of the source pass)
    N, E = 50, 3000
    other = gtgen.random_coo(3, N, E)[0]
    with chunk_edges(chunk):
        check_bwd_full(with_grad(custom(N, other, np.full(E, 7), 8, 64, seed=3)))
        check_bwd_full(with_grad(custom(N, np.full(E, 7), other, 8, 64, seed=4)))


@pytest.mark.parametrize("chunk", [16, 64])
def test_bwd_degrees_at_threshold(chunk):
    degs = [chunk - 1, chunk, chunk + 1, 2 * chunk, 2 * chunk + 1, 0, 1, 3 * chunk - 1]
    N = 64
    hub = np.concatenate([np.full(d, v) for v, d in enumerate(degs)])
    other = gtgen.random_coo(5, N, len(hub))[0]
    with chunk_edges(chunk):
        for dtype, D in ((gtgen.F32, 64), (gtgen.BF16, 32), (gtgen.F32, 10)):
            check_bwd_full(with_grad(custom(N, other, hub, 8, D, dtype, seed=5)))
            check_bwd_full(with_grad(custom(N, hub, other, 8, D, dtype, seed=6)))


def test_bwd_zero_edges_zero_fill():
    w = with_grad(custom(17, [], [], 8, 64))
    t = to_dev(w)
    t["dO"] = to_torch(w["dO"])
    tip = torch.from_numpy(w["t_indptr"]).to(dev())
    tix = torch.from_numpy(w["t_indices"]).to(dev())
    say("bwd E=0")
    out, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    grads = [torch.full_like(t["Q"], float("nan")) for _ in range(3)]
    gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, t["Q"], t["K"], t["V"], out, t["dO"], lse, *grads)
    torch.cuda.synchronize()
    assert torch.all(lse == -math.inf)
    for g in grads:
        assert torch.all(g == 0)


def test_bwd_single_node_self_loop():
    # alpha = 1, so ds = 0: dQ = dK = 0 and dV = dO (alpha recomputed from
    # lse may differ from 1 in the last bits)
    w = with_grad(custom(1, [0], [0], 8, 64))
    _, _, dq, dk, dv = check_bwd_full(w)
    assert torch.all(dq == 0) and torch.all(dk == 0)
    g = widen(w["dO"])
    assert np.all(np.abs(host(dv) - g) <= 2.0 ** -21 * np.abs(g))


def test_bwd_misaligned_features_use_the_scalar_layout():
    w = with_grad(random_graph(8, 40, 300, 8, 64))
    t = to_dev(w)
    t["dO"] = to_torch(w["dO"])
    shape = t["Q"].shape
    names = ("Q", "K", "V", "dO", "out", "dQ", "dK", "dV")
    bufs = {k: torch.empty(t["Q"].numel() + 1, dtype=torch.float32, device=dev()) for k in names}
    views = {k: bufs[k][1:].view(shape) for k in names}
    for k in ("Q", "K", "V", "dO"):
        views[k].copy_(t[k])
    tip = torch.from_numpy(w["t_indptr"]).to(dev())
    tix = torch.from_numpy(w["t_indices"]).to(dev())
    say("bwd misaligned")
    _, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], views["Q"], views["K"], views["V"],
                                      out=views["out"])
    gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, views["Q"], views["K"], views["V"], views["out"],
                         views["dO"], lse, views["dQ"], views["dK"], views["dV"])
    torch.cuda.synchronize()
    # the scalar layout's gradients against the oracle, at the fp32 backward tolerance
    rq, rk, rv, rlse, _ = oracle.bwd(*oracle_inputs(w), w["dO"])
    check_lse(host(lse), rlse, "misaligned lse")
    outs = OutTable(oracle.fwd(*oracle_inputs(w)))
    allv = np.arange(w["N"])
    BK, BV = bound_dkv(w, rlse, outs, allv)
    check_bound(host(views["dQ"]), rq, bound_dq(w, rlse, outs, allv), F32_BTOL, "misaligned dQ")
    check_bound(host(views["dK"]), rk, BK, F32_BTOL, "misaligned dK")
    check_bound(host(views["dV"]), rv, BV, F32_BTOL, "misaligned dV")
    # and the aligned run (vector layout) too
    check_bwd_full(w)


@pytest.mark.parametrize("H,D,dtype", WORD_SHAPES)
@pytest.mark.parametrize("chunk", [512, 37])
def test_bwd_word_layout_shapes(H, D, dtype, chunk):
    # both passes in the word layout, with a destination hub and a source hub
    # split into chunks at chunk 37
    with chunk_edges(chunk):
        check_bwd_full(with_grad(hub_graph(H, D, dtype, H * 100 + D)))


@pytest.mark.parametrize("H,D,shift", [(2, 64, 2), (4, 10, 1), (8, 10, 2)])
def test_bwd_misaligned_word_layout(H, D, shift):
    w = with_grad(hub_graph(H, D, gtgen.F32, 7 * shift + D))
    t = to_dev(w)
    t["dO"] = to_torch(w["dO"])
    shape = t["Q"].shape
    names = ("Q", "K", "V", "dO", "out", "dQ", "dK", "dV")
    bufs = {k: torch.empty(t["Q"].numel() + shift, dtype=torch.float32, device=dev()) for k in names}
    views = {k: bufs[k][shift:].view(shape) for k in names}
    for k in ("Q", "K", "V", "dO"):
        views[k].copy_(t[k])
    tip = torch.from_numpy(w["t_indptr"]).to(dev())
    tix = torch.from_numpy(w["t_indices"]).to(dev())
    with chunk_edges(37):
        say("bwd misaligned by %d elements H=%d D=%d" % (shift, H, D))
        _, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], views["Q"], views["K"], views["V"],
                                          out=views["out"])
        gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, views["Q"], views["K"], views["V"],
                             views["out"], views["dO"], lse, views["dQ"], views["dK"], views["dV"])
        torch.cuda.synchronize()
    rq, rk, rv, rlse, _ = oracle.bwd(*oracle_inputs(w), w["dO"])
    check_lse(host(lse), rlse, "misaligned lse")
    outs = OutTable(oracle.fwd(*oracle_inputs(w)))
    allv = np.arange(w["N"])
    BK, BV = bound_dkv(w, rlse, outs, allv)
    check_bound(host(views["dQ"]), rq, bound_dq(w, rlse, outs, allv), F32_BTOL, "misaligned dQ")
    check_bound(host(views["dK"]), rk, BK, F32_BTOL, "misaligned dK")
    check_bound(host(views["dV"]), rv, BV, F32_BTOL, "misaligned dV")


def test_bwd_deterministic():
    w = with_grad(workload("regular16"))
    t = to_dev(w)
    with chunk_edges(3):
        say("bwd determinism")
        a = [x.clone() for x in run_gpu(w, t)]
        b = run_gpu(w, t)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ million-node workloads, sampled

@pytest.mark.parametrize("name", ["powerlaw", "lognormal"])
def test_bwd_large_sampled(name):
    check_bwd_sampled(with_grad(workload(name)))


@pytest.mark.parametrize("H,D,dtype", [(8, 48, gtgen.F32), (8, 96, gtgen.BF16), (6, 64, gtgen.F32), (3, 128, gtgen.F32),
                                       (16, 64, gtgen.F32), (16, 128, gtgen.BF16), (24, 64, gtgen.BF16),
                                       (8, 64, gtgen.F32), (8, 32, gtgen.BF16)])
def test_split_rows_every_layout(H, D, dtype):
    # a hub destination and a hub source split into chunks, for padded heads,
    # rows that end before their last lane group and wide rows: the chunk
    # partials are indexed by memory position, not lane slot
    N, E = 60, 1500
    src, dst = gtgen.random_coo(H * 100 + D, N, E)
    dst = np.where(np.arange(E) < 500, 5, dst)
    src = np.where((np.arange(E) >= 500) & (np.arange(E) < 900), 9, src)
    w = custom(N, src, dst, H, D, dtype, seed=H + D)
    with chunk_edges(37):
        check_fused_full(w)
        check_bwd_full(with_grad(w))
