"""Pins of the oracle's logit variants (additive bias, edge weights) and
attention dropout to things other than itself (CPU).

* the dropout generator equals numpy's Philox4x64-10 bit generator (a
  library routine) word for word;
* torch autograd in float64 through dense masked attention with the bias
  matrix added to and the weight matrix multiplying the scaled logits, and the
  dropout mask (drawn with numpy's Philox) applied to the softmax: forward,
  lse, dQ, dK, dV, dbias and dw;
* reductions: no bias, unit weights and p = 0 give the base oracle (pinned
  separately); a uniform weight c equals Q scaled by c; a bias constant per
  destination leaves out unchanged and shifts lse by that constant; p close
  to 1 drops (almost) everything, and the kept fraction follows p.
test_oracle_ex_mutants.py plants mistakes in copies of oracle.c and shows
each one fails at least one of these checks.
"""
import math

import numpy as np
import pytest
import torch

import gtgen
from oracle import Oracle
from tests.test_oracle_bwd_pins import close, feats64


def unique_graph(seed, N, E):
    """A graph without duplicate edges (so that a dense matrix holds one bias
    per edge), some destinations without in-edges."""
    src, dst = gtgen.random_coo(seed, N, E)
    pairs = np.unique(np.stack([dst, src], 1), axis=0)
    pairs = pairs[pairs[:, 0] % 5 != 0]
    return gtgen.coo_to_csr(N, pairs[:, 1].astype(np.int32), pairs[:, 0].astype(np.int32))


def numpy_keep(seed, E, H, p):
    """keep[e, h] from numpy's Philox4x64-10: word e*H + h, upper 32 bits >= floor(p 2^32)."""
    words = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64)).random_raw(E * H).astype(np.uint64)
    return ((words >> np.uint64(32)) >= np.uint64(math.floor(p * 2.0 ** 32))).reshape(E, H)


def dense_reference(indptr, indices, Q, K, V, dO, bias=None, ew=None, keep=None, p=0.0):
    """(out, lse, dq, dk, dv, dbias, dw) by torch autograd on dense [H][N][N] matrices."""
    N, H, D = Q.shape
    E = len(indices)
    dst = np.repeat(np.arange(N), np.diff(indptr))
    src = indices.astype(np.int64)
    mask = torch.zeros((N, N), dtype=torch.bool)
    mask[dst, src] = True
    b = torch.zeros((E, H), dtype=torch.float64, requires_grad=True) if bias is None else \
        torch.tensor(np.asarray(bias, np.float64), requires_grad=True)
    w = torch.ones(E, dtype=torch.float64, requires_grad=True) if ew is None else \
        torch.tensor(np.asarray(ew, np.float64), requires_grad=True)
    Bm = torch.zeros((H, N, N), dtype=torch.float64).index_put((torch.arange(H)[:, None], torch.from_numpy(dst)[None],
                                                                torch.from_numpy(src)[None]), b.t())
    Wm = torch.ones((N, N), dtype=torch.float64).index_put((torch.from_numpy(dst), torch.from_numpy(src)), w)
    q, k, v = (torch.tensor(x.transpose(1, 0, 2), requires_grad=True) for x in (Q, K, V))
    logits = Wm[None] * (q @ k.transpose(1, 2).contiguous()) / math.sqrt(D) + Bm
    logits = logits.masked_fill(~mask[None], -math.inf)
    empty = torch.from_numpy(np.diff(indptr) == 0)
    logits = torch.where(empty[None, :, None], torch.zeros_like(logits), logits)
    lse = torch.logsumexp(logits, dim=-1)
    P = torch.softmax(logits, dim=-1) * (~empty)[None, :, None]
    if keep is not None:
        Mm = torch.zeros((H, N, N), dtype=torch.float64).index_put(
            (torch.arange(H)[:, None], torch.from_numpy(dst)[None], torch.from_numpy(src)[None]),
            torch.from_numpy(keep.astype(np.float64)).t())
        P = P * Mm / (1.0 - p)
    out = P @ v
    (out * torch.from_numpy(dO.transpose(1, 0, 2))).sum().backward()
    lse = lse.detach().numpy().T.copy()
    lse[np.diff(indptr) == 0] = -np.inf
    grads = tuple(t.grad.numpy().transpose(1, 0, 2) for t in (q, k, v))
    return (out.detach().numpy().transpose(1, 0, 2), lse, *grads, b.grad.numpy(), w.grad.numpy())


def variant_inputs(seed, E, H):
    rng = np.random.default_rng(seed)
    bias = rng.normal(0, 1.5, (E, H)).astype(np.float32)
    ew = rng.uniform(0.0, 1.0, E).astype(np.float32)
    return bias, ew


# ----------------------------------------------------------------- checks

def check_philox_is_numpy(orc):
    for seed in (0, 1, 12345, 2 ** 63 + 7):
        raw = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64)).random_raw(64)
        assert all(orc.philox_word(seed, i) == int(raw[i]) for i in range(64))
    # far into the stream: numpy's counter starts at the block before
    for i in (2 ** 33 + 5, 10 ** 12 + 2):
        raw = np.random.Philox(key=np.array([99, 0], dtype=np.uint64),
                               counter=np.array([i // 4, 0, 0, 0], dtype=np.uint64)).random_raw(4)
        assert orc.philox_word(99, i) == int(raw[i % 4])


def check_dense_bias_weights(orc):
    indptr, indices = unique_graph(3, 24, 160)
    N, H, D = 24, 3, 8
    Q, K, V, dO = feats64(3, N, H, D)
    bias, ew = variant_inputs(3, len(indices), H)
    for kw in (dict(bias=bias), dict(ew=ew), dict(bias=bias, ew=ew)):
        ref = dense_reference(indptr, indices, Q, K, V, dO, **kw)
        out, lse = orc.fwd_ex(indptr, indices, Q, K, V, want_lse=True, **kw)
        close(out, ref[0], 1e-11, 1e-13, "out")
        fin = np.isfinite(ref[1])
        close(lse[fin], ref[1][fin], 1e-12, 1e-13, "lse")
        assert np.all(lse[~fin] == -np.inf)
        g = orc.bwd_ex(indptr, indices, Q, K, V, dO, **kw)
        for name, r in zip(("dq", "dk", "dv"), ref[2:5]):
            close(g[name], r, 1e-10, 1e-12, name)
        if "bias" in kw:
            close(g["dbias"], ref[5], 1e-10, 1e-12, "dbias")
        close(g["dw"], ref[6], 1e-10, 1e-12, "dw")


def check_dense_dropout(orc):
    indptr, indices = unique_graph(4, 20, 140)
    N, H, D = 20, 2, 6
    Q, K, V, dO = feats64(4, N, H, D)
    bias, ew = variant_inputs(4, len(indices), H)
    for p, seed in ((0.3, 5), (0.75, 2 ** 40 + 1)):
        keep = numpy_keep(seed, len(indices), H, p)
        assert 0 < keep.sum() < keep.size
        ref = dense_reference(indptr, indices, Q, K, V, dO, bias=bias, ew=ew, keep=keep, p=p)
        kw = dict(bias=bias, ew=ew, drop_p=p, seed=seed)
        out = orc.fwd_ex(indptr, indices, Q, K, V, **kw)
        close(out, ref[0], 1e-11, 1e-13, "out")
        g = orc.bwd_ex(indptr, indices, Q, K, V, dO, **kw)
        for name, r in zip(("dq", "dk", "dv", "dbias", "dw"), ref[2:]):
            close(g[name], r, 1e-10, 1e-12, name)


def check_reductions(orc):
    from tests.test_oracle_bwd_pins import graph
    indptr, indices = graph(6, 30, 200)
    N, H, D = 30, 4, 5
    Q, K, V, dO = feats64(6, N, H, D)
    E = len(indices)
    base = orc.fwd(indptr, indices, Q, K, V)
    close(orc.fwd_ex(indptr, indices, Q, K, V), base, 1e-14, 1e-15, "no variant")
    close(orc.fwd_ex(indptr, indices, Q, K, V, bias=np.zeros((E, H)), ew=np.ones(E), drop_p=0.0, seed=3), base,
          1e-14, 1e-15, "neutral variant")
    bq, bk, bv, blse, bdelta = orc.bwd(indptr, indices, Q, K, V, dO)
    g = orc.bwd_ex(indptr, indices, Q, K, V, dO)
    for name, r in (("dq", bq), ("dk", bk), ("dv", bv), ("delta", bdelta)):
        close(g[name], r, 1e-12, 1e-14, name)
    # a uniform weight c: the same as Q scaled by c
    c = 0.375  # exact in float32, as the weights are stored
    out_c, lse_c = orc.fwd_ex(indptr, indices, Q, K, V, ew=np.full(E, c), want_lse=True)
    out_q, lse_q = orc.fwd_ex(indptr, indices, Q * c, K, V, want_lse=True)
    close(out_c, out_q, 1e-12, 1e-14, "uniform weight")
    fin = np.isfinite(lse_q)
    close(lse_c[fin], lse_q[fin], 1e-12, 1e-14, "uniform weight lse")
    # a bias constant per destination row (and head): out unchanged, lse shifted
    shift = np.linspace(-3, 4, N * H).reshape(N, H)
    dst = np.repeat(np.arange(N), np.diff(indptr))
    out_b, lse_b = orc.fwd_ex(indptr, indices, Q, K, V, bias=shift[dst].astype(np.float32), want_lse=True)
    out_0, lse_0 = orc.fwd_ex(indptr, indices, Q, K, V, want_lse=True)
    close(out_b, out_0, 1e-11, 1e-13, "row-constant bias")
    fin = np.isfinite(lse_0)
    close(lse_b[fin], (lse_0 + shift.astype(np.float32))[fin], 1e-12, 1e-12, "row-constant bias lse")


def check_dropout_statistics(orc):
    from tests.test_oracle_bwd_pins import graph
    indptr, indices = graph(8, 400, 20000, keep_empty=False)
    N, H, D = 400, 2, 1
    Q, K, _, _ = feats64(8, N, H, D)
    V = np.ones((N, H, D))
    # with V = 1, out_v = (kept share of alpha) / (1 - p): its mean over rows is about 1
    for p in (0.1, 0.5):
        out = orc.fwd_ex(indptr, indices, Q, K, V, drop_p=p, seed=11)
        assert abs(out.mean() - 1.0) < 0.05, (p, out.mean())
    out = orc.fwd_ex(indptr, indices, Q, K, V, drop_p=1.0 - 2.0 ** -30, seed=11)
    assert np.count_nonzero(out) < 0.01 * out.size
    with pytest.raises(ValueError):
        orc.fwd_ex(indptr, indices, Q, K, V, drop_p=1.0)


ALL_CHECKS = [check_philox_is_numpy, check_dense_bias_weights, check_dense_dropout, check_reductions,
              check_dropout_statistics]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_ex_pin(check):
    check(Oracle())
