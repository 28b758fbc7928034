"""Properties that hold at any size, checked on every row of the million-node
workloads, in the launch configuration the benchmark times (the library's
default split threshold).  The sampled parity tests compare a few thousand
rows (every split row among them) with the oracle; these cover the rest.

Each property is an identity of the method's exact arithmetic ("Graph
Transformer in a Nutshell", section "Sparse Multi-head Attention": scores at
the edges, a softmax over each destination's in-edges, then the weighted sum
of value rows), so the GPU results must meet it up to fp32 rounding.  The
tolerances are bounds on that rounding, with u = 2^-24:
* a dot product of D terms errs by at most (D + 2) u sum |q_d k_d| <=
  (D + 2) u |q| |k| (Cauchy-Schwarz); scaled by 1/sqrt(D), and doubled when
  two kernels that each round their own dot products are compared;
* a softmax normaliser summed over deg terms errs relatively by at most
  (deg + 8) u (the sum, the exponentials, the division), doubled for margin;
* a bf16 output is rounded to 8 significant bits (relative 2^-9).
Sums over rows are taken in float64 on the GPU.  Each test prints how close
the results come to their bounds.  The per-row properties (weight sums, lse
against the row's scores, outputs within their value rows) come within an
order of magnitude and catch a wrong row anywhere.  The backward's two column
identities add up the worst case of every row, sit far inside their bounds,
and guard against systematic mistakes only; the sampled parity tests check
the gradients element by element.
"""
import math

import numpy as np
import pytest
import torch

import gtgen
import sparse_graph_attention_amd as gt
from tests.test_gpu_backward import to_torch
from tests.test_gpu_parity import dev, say, workload

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
BF16_REL = 2.0 ** -8  # rounding to bf16, with margin


def graph_tensors(w):
    d = dev()
    ip = torch.from_numpy(w["indptr"]).to(d)
    ix = torch.from_numpy(w["indices"]).to(d)
    deg = ip[1:] - ip[:-1]
    rows = torch.repeat_interleave(torch.arange(w["N"], device=d), deg)  # destination of each edge
    return ip, ix, deg, rows


def seg_max(vals, rows, N):
    """Per-row maximum of [E][H] values (rows without edges: -inf)."""
    out = torch.full((N, vals.shape[1]), -math.inf, dtype=vals.dtype, device=vals.device)
    return out.scatter_reduce_(0, rows[:, None].expand_as(vals), vals, "amax", include_self=True)


def seg_sum(vals, rows, N):
    out = torch.zeros((N, vals.shape[1]), dtype=vals.dtype, device=vals.device)
    return out.index_add_(0, rows, vals)


def score_error_bound(Qf, Kf, ix, rows, N, D):
    """Per (row, head): the largest bound over the row's edges on the difference
    between two fp32 evaluations of a score, 2 (D + 2) u |q| |k| / sqrt(D)."""
    qn = torch.linalg.vector_norm(Qf, dim=2)  # [N][H]
    kn = torch.linalg.vector_norm(Kf, dim=2)
    per_edge = qn[rows] * kn[ix.long()]
    return seg_max(per_edge, rows, N).clamp_min(0.0) * (2.0 * (D + 2) * U / math.sqrt(D))


@pytest.mark.parametrize("name", ["powerlaw", "lognormal"])
def test_every_row_softmax_lse_and_output_bounds(name):
    w = workload(name)
    N, E, H, D = w["N"], w["E"], w["H"], w["D"]
    say("properties %s N=%d E=%d" % (name, N, E))
    ip, ix, deg, rows = graph_tensors(w)
    Q, K, V = (to_torch(w[k]) for k in ("Q", "K", "V"))
    has = deg > 0
    degf = deg.double()[:, None]

    # the unfused stages: every row's weights sum to one
    scores = gt.gt_sddmm(ip, ix, Q, K)
    alpha = gt.gt_edge_softmax(ip, scores)
    torch.cuda.synchronize()
    sums = seg_sum(alpha.double(), rows, N)
    tol = 2.0 * (degf + 8.0) * U
    bad = has[:, None] & ((sums - 1.0).abs() > tol)
    assert not bool(bad.any()), "%s: %d (row, head) weight sums off 1, worst %.3e" % (
        name, int(bad.sum()), float((sums - 1.0).abs()[has].max()))
    say("%s: weight sums, largest deviation / bound %.3f" % (name, float(((sums - 1.0).abs() / tol)[has].max())))
    del alpha, sums

    # the fused forward's lse: between the row's largest score and that plus ln(deg)
    out, lse = gt.gt_sparse_mha_fwd_lse(ip, ix, Q, K, V)
    torch.cuda.synchronize()
    Qf, Kf, Vf = Q.double(), K.double(), V.double()
    m = seg_max(scores.double(), rows, N)
    del scores
    eb = score_error_bound(Qf, Kf, ix, rows, N, D)
    lse64 = lse.double()
    tol = eb + 2.0 * (degf + 8.0) * U + 4.0 * U * (lse64.abs() + 1.0) + 1e-6
    low = lse64 < m - tol
    high = lse64 > m + torch.log(degf.clamp_min(1.0)) + tol
    assert not bool((has[:, None] & (low | high)).any()), "%s: lse outside [max score, max + ln deg] at %d places" % (
        name, int((has[:, None] & (low | high)).sum()))
    assert bool(torch.isneginf(lse[~has]).all()), "rows without in-edges must have lse = -inf"
    say("%s: lse - max score in [%.3g, %.3g], ln(max degree) %.3g" % (
        name, float((lse64 - m)[has].min()), float((lse64 - m)[has].max()), math.log(float(deg.max()))))

    # every output row is a convex combination of the row's value rows
    vmax = Vf.abs().amax(dim=2)  # [N][H]: largest |v| of each node's head
    bound = seg_max(vmax[ix.long()], rows, N)
    rel = 2.0 * (degf + 8.0) * U + (BF16_REL if w["dtype"] == gtgen.BF16 else 0.0)
    over = out.double().abs().amax(dim=2) > bound * (1.0 + rel) + 1e-30
    assert not bool((has[:, None] & over).any()), "%s: %d (row, head) outputs outside their value rows' range" % (
        name, int((has[:, None] & over).sum()))
    assert bool((out[~has] == 0).all()), "rows without in-edges must be exactly 0"


@pytest.mark.parametrize("name", ["powerlaw", "lognormal"])
def test_every_row_backward_column_identities(name):
    # dV[u] = sum_v alpha_vu dO_v and the weights of each row sum to one, so
    # sum_u dV[u] = sum of dO over the rows with in-edges; dK[u] = sum_v ds_vu q_v / sqrt(D)
    # with sum_u ds_vu = 0 in each row, so sum_u dK[u] = 0.  Per (head, feature).
    w = workload(name)
    N, E, H, D = w["N"], w["E"], w["H"], w["D"]
    say("backward identities %s N=%d E=%d" % (name, N, E))
    ip, ix, deg, rows = graph_tensors(w)
    tip, tix = gtgen.source_sorted(w["indptr"], w["indices"])
    outdeg_max = int(np.diff(tip).max())
    tip, tix = torch.from_numpy(tip).to(dev()), torch.from_numpy(tix).to(dev())
    Q, K, V = (to_torch(w[k]) for k in ("Q", "K", "V"))
    dO = to_torch(gtgen.make_grad(N, H, D, w["dtype"], 11))
    out, lse = gt.gt_sparse_mha_fwd_lse(ip, ix, Q, K, V)
    dQ, dK, dV = gt.gt_sparse_mha_bwd(ip, ix, tip, tix, Q, K, V, out, dO, lse)
    torch.cuda.synchronize()
    has = deg > 0
    degf = deg.double()[:, None]
    bf16 = w["dtype"] == gtgen.BF16
    Qf, Kf, Vf, dOf = Q.double(), K.double(), V.double(), dO.double()
    eb = score_error_bound(Qf, Kf, ix, rows, N, D)  # [N][H]
    lse64 = torch.where(has[:, None], lse.double(), torch.zeros_like(lse, dtype=torch.float64))
    # how far each row's recomputed weights may sum from one: the scores against
    # the forward's, the normaliser and lse's own rounding, the exponentials
    eps = eb + 2.0 * (degf + 8.0) * U + 4.0 * U * (lse64.abs() + 1.0)
    eps = torch.where(has[:, None], eps, torch.zeros_like(eps))  # [N][H]

    # dV: the weights' sums, then dV's own fp32 sums over each source's
    # out-edges (at most max out-degree + 2 roundings, split sources included)
    adO = dOf.abs() * has[:, None, None]
    diff = (dV.double().sum(0) - (dOf * has[:, None, None]).sum(0)).abs()
    tol = (adO * eps[:, :, None]).sum(0) + (outdeg_max + 2) * U * adO.sum(0) * 1.01
    if bf16:
        tol = tol + BF16_REL * dV.double().abs().sum(0)
    tol = tol + 1e-6
    worst = int((diff / tol).argmax())
    assert bool((diff <= tol).all()), "%s: sum of dV off the sum of dO by %.3e where the bound is %.3e" % (
        name, float(diff.flatten()[worst]), float(tol.flatten()[worst]))
    say("%s: sum of dV - sum of dO, largest deviation / bound %.3f" % (name, float((diff / tol).max())))

    # dK.  Per row, with dp = dO . v_u and delta = dO . out, Cauchy-Schwarz bounds
    # every term by |dO_v| max_u |v_u|: |sum_u ds_vu| <= |dO_v| max|v_u| (3 eps +
    # 2 (D + 2) u + 2 u + r), r the bf16 rounding of the stored out; then dK's fp32
    # sums over each source's out-edges, of terms |ds_vu| |q_v| / sqrt(D) with
    # sum_u |ds_vu| <= 2 |dO_v| max|v_u|.
    don = torch.linalg.vector_norm(dOf, dim=2)
    vn = torch.linalg.vector_norm(Vf, dim=2)
    vmax = seg_max(vn[ix.long()], rows, N).clamp_min(0.0)
    vmax = torch.where(has[:, None], vmax, torch.zeros_like(vmax))
    r = BF16_REL if bf16 else 0.0
    row_err = don * vmax * (3.0 * eps + 2.0 * (D + 2) * U + 2.0 * U + r)
    scale = 1.0 / math.sqrt(D)
    aq = Qf.abs()
    lhs = dK.double().sum(0).abs()
    tol = scale * (aq * row_err[:, :, None]).sum(0)
    tol = tol + (outdeg_max + 2) * U * scale * (aq * (2.0 * 1.01 * don * vmax)[:, :, None]).sum(0)
    if bf16:
        tol = tol + BF16_REL * dK.double().abs().sum(0)
    tol = tol + 1e-6
    worst = int((lhs / tol).argmax())
    assert bool((lhs <= tol).all()), "%s: sum of dK is %.3e where the bound is %.3e" % (
        name, float(lhs.flatten()[worst]), float(tol.flatten()[worst]))
    say("%s: sum of dK, largest value / bound %.3f (largest |sum of dK| %.3e against sum |dK| %.3e)" % (
        name, float((lhs / tol).max()), float(lhs.max()), float(dK.double().abs().sum(0).max())))
