"""Pins of the oracle's backward (dQ, dK, dV, log-sum-exp) to things other than itself (CPU).

* torch autograd (a library routine) through dense masked attention in
  float64: logits QK^T/sqrt(d) + ln(multiplicity), -inf off the graph, the
  dense masked-softmax form of the "Graph Transformer theory" blog's GAT code;
* central finite differences of the oracle's own forward in float64 (the
  forward is pinned separately), along random directions;
* closed forms: a row with one in-edge has dQ = 0; dV = P^T dO; the sum of dK
  over all nodes is 0 (adding one vector to every key shifts each
  destination's scores by a constant); lse is scipy's logsumexp per row;
* a hand-worked example under tests/golden/backward/.
test_oracle_bwd_mutants.py plants mistakes in copies of oracle.c and shows
each one fails at least one of these checks.
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

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "backward", "*.json")))


def graph(seed, N, E, keep_empty=True):
    src, dst = gtgen.random_coo(seed, N, E)
    if keep_empty:
        keep = dst % 5 != 0  # some destinations without in-edges
        src, dst = src[keep], dst[keep]
    return gtgen.coo_to_csr(N, src, dst)


def feats64(seed, N, H, D):
    Q, K, V = (x.astype(np.float64) for x in gtgen.make_features(N, H, D, 0, seed, 1.0))
    dO = gtgen.normal_f32(seed, 9, (N, H, D)).astype(np.float64)
    return Q, K, V, dO


def close(a, b, rtol, atol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)), what + ": non-finite"
    err = np.abs(a - b) - (atol + rtol * np.abs(b))
    assert np.all(err <= 0), "%s: max excess %.3e" % (what, err.max())


def autograd_reference(indptr, indices, Q, K, V, dO):
    N, H, D = Q.shape
    dst = np.repeat(np.arange(N), np.diff(indptr))
    C = np.zeros((N, N))
    np.add.at(C, (dst, indices), 1.0)
    with np.errstate(divide="ignore"):
        logc = torch.from_numpy(np.log(C))
    empty = torch.from_numpy(np.diff(indptr) == 0)
    q, k, v = (torch.tensor(x.transpose(1, 0, 2), requires_grad=True) for x in (Q, K, V))
    logits = q @ k.transpose(1, 2) / math.sqrt(D) + logc
    logits = torch.where(empty[None, :, None], torch.zeros_like(logits), logits)  # finite rows for the softmax
    P = torch.softmax(logits, dim=-1) * (~empty)[None, :, None]
    out = P @ v
    (out * torch.from_numpy(dO.transpose(1, 0, 2))).sum().backward()
    return tuple(t.grad.numpy().transpose(1, 0, 2) for t in (q, k, v))


# ----------------------------------------------------------------- checks

def check_autograd(orc):
    for seed, N, E, H, D in [(0, 30, 140, 2, 8), (1, 12, 50, 3, 5), (2, 25, 300, 1, 16)]:
        indptr, indices = graph(seed, N, E)
        Q, K, V, dO = feats64(seed, N, H, D)
        dq, dk, dv, _, _ = orc.bwd(indptr, indices, Q, K, V, dO)
        rq, rk, rv = autograd_reference(indptr, indices, Q, K, V, dO)
        close(dq, rq, 1e-10, 1e-12, "dQ")
        close(dk, rk, 1e-10, 1e-12, "dK")
        close(dv, rv, 1e-10, 1e-12, "dV")


def check_finite_differences(orc):
    indptr, indices = graph(3, 14, 60)
    N, H, D = 14, 2, 4
    Q, K, V, dO = feats64(3, N, H, D)
    dq, dk, dv, _, _ = orc.bwd(indptr, indices, Q, K, V, dO)
    rng = np.random.default_rng(3)

    def f(q, k, v):
        return float((oracle.fwd(indptr, indices, q, k, v) * dO).sum())

    eps = 1e-5
    for _ in range(3):
        dQ_, dK_, dV_ = (rng.normal(size=(N, H, D)) for _ in range(3))
        num = (f(Q + eps * dQ_, K + eps * dK_, V + eps * dV_) - f(Q - eps * dQ_, K - eps * dK_, V - eps * dV_)) / (2 * eps)
        ana = float((dq * dQ_).sum() + (dk * dK_).sum() + (dv * dV_).sum())
        assert abs(num - ana) <= 1e-7 * max(1.0, abs(ana)), (num, ana)


def check_closed_forms(orc):
    indptr, indices = graph(4, 20, 80)
    N, H, D = 20, 3, 6
    Q, K, V, dO = feats64(4, N, H, D)
    dq, dk, dv, lse, delta = orc.bwd(indptr, indices, Q, K, V, dO)
    # sum of dK over all nodes vanishes, per head and dim
    close(dk.sum(0), np.zeros((H, D)), 0, 1e-12, "sum dK")
    # rows with a single in-edge: alpha = 1, ds = 0, dQ = 0
    one = np.diff(indptr) == 1
    assert one.any()
    close(dq[one], np.zeros_like(dq[one]), 0, 1e-14, "dQ of single-edge rows")
    # lse and dV = P^T dO, from the oracle's own forward weights
    out, s, a = oracle.fwd(indptr, indices, Q, K, V, want_edges=True)
    dst = np.repeat(np.arange(N), np.diff(indptr))
    for v in range(N):
        b, e = indptr[v], indptr[v + 1]
        if e > b:
            close(lse[v], scipy.special.logsumexp(s[b:e], axis=0), 1e-13, 1e-13, "lse")
            close(delta[v], (dO[v] * out[v]).sum(-1), 1e-12, 1e-12, "delta = dO . out")
        else:
            assert np.all(np.isneginf(lse[v])) and np.all(delta[v] == 0)
    ref_dv = np.zeros_like(dv)
    np.add.at(ref_dv, indices, a[:, :, None] * dO[dst])
    close(dv, ref_dv, 1e-12, 1e-13, "dV = P^T dO")


def check_golden(orc):
    assert GOLDEN
    for path in GOLDEN:
        g = json.load(open(path))
        Q, K, V, dO = (np.array(g[k], dtype=np.float64) for k in ("Q", "K", "V", "dO"))
        indptr, indices = gtgen.coo_to_csr(g["N"], np.array(g["coo_src"]), np.array(g["coo_dst"]))
        dq, dk, dv, lse, delta = orc.bwd(indptr, indices, Q, K, V, dO)
        close(dq, g["dQ"], 1e-12, 1e-12, "dQ")
        close(dk, g["dK"], 1e-12, 1e-12, "dK")
        close(dv, g["dV"], 1e-12, 1e-12, "dV")
        close(delta, g["delta"], 1e-12, 1e-12, "delta")
        fin = np.isfinite(lse)
        close(lse[fin], np.array(g["lse"])[fin], 1e-12, 1e-12, "lse")
        assert np.all(np.isneginf(lse[~fin]))


def check_bf16_widening(orc):
    indptr, indices = graph(6, 16, 70)
    N, H, D = 16, 2, 8
    b = [gtgen.normal_bf16(6, s, (N, H, D), 0.5) for s in (1, 2, 3, 9)]
    w = [gtgen.bf16_bits_to_f32(x) for x in b]
    r1 = orc.bwd(indptr, indices, *b)
    r2 = orc.bwd(indptr, indices, *w)
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)


ALL_CHECKS = [check_autograd, check_finite_differences, check_closed_forms, check_golden, check_bf16_widening]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_oracle_bwd_pin(check):
    check(oracle.default())
