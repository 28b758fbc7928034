"""Magnitude bounds behind the backward tolerances, over sub-graphs of listed rows.

A gradient sums terms of both signs, so its rounding error is bounded by the
sum of the terms' magnitudes, not by the gradient itself.  With alpha_e the
softmax weight of edge e = (u -> v), c_e its dropout multiplier (0 or
1/(1 - p); 1 without dropout), w_e its edge weight (1 without weights):

    wt_e    = alpha_e (c_e |dO_v|.|v_u| + |dO_v|.|out_v|)      (per head; bounds |ds_e|)
    B_dQ[v] = sum over in-edges  wt_e w_e |k_u| / sqrt(D)
    B_dK[u] = sum over out-edges wt_e w_e |q_v| / sqrt(D)
    B_dV[u] = sum over out-edges alpha_e c_e |dO_v|
    B_db[e] = wt_e
    B_dw[e] = sum over heads wt_e |q_v|.|k_u| / sqrt(D)

The per-edge dot products and the sums over edges are the oracle's own SDDMM
and SpMM stages (oracle.sddmm, oracle.spmm: pinned, OpenMP over rows) run on
the sub-graph of the listed rows with magnitude features, so that every split
row of the million-node workloads is bounded in seconds.  The magnitudes are
exact: |x| of a float32 is a float32, of a bf16 value its bits without the
sign bit.  Nothing here comes from the GPU path.
"""
import math

import numpy as np

import oracle

# Lines that the test session's summary prints (how many split rows each
# large test checked); filled by tests that sample rows.
REPORT = []


def absf(x):
    """|x| elementwise, exactly, in x's own storage type (float32, float64 or bf16 bits)."""
    if x.dtype == np.uint16:
        return x & np.uint16(0x7FFF)
    return np.abs(x)


def sub_graph(indptr, indices, rows):
    """CSR of the listed rows only (renumbered 0..len(rows)-1, sources kept):
    (sub_indptr, sub_indices, sel) with sel the edges' positions in the full CSR."""
    rows = np.asarray(rows, np.int64)
    starts = indptr[rows]
    deg = indptr[rows + 1] - starts
    sub_ip = np.zeros(len(rows) + 1, dtype=np.int64)
    np.cumsum(deg, out=sub_ip[1:])
    n = int(sub_ip[-1])
    sel = np.arange(n, dtype=np.int64) + np.repeat(starts - sub_ip[:-1], deg)
    return sub_ip, np.ascontiguousarray(indices[sel]), sel


class OutTable:
    """The oracle's out for a set of destinations: take(vs) -> [len(vs)][H][D].
    ids None: values is the whole [N][H][D] array."""

    def __init__(self, values, ids=None):
        self.values = values
        self.ids = None if ids is None else np.asarray(ids, np.int64)

    def take(self, vs):
        vs = np.asarray(vs, np.int64)
        if self.ids is None:
            return self.values[vs]
        pos = np.searchsorted(self.ids, vs)
        assert np.all(self.ids[np.minimum(pos, len(self.ids) - 1)] == vs), "destination without an oracle out"
        return self.values[pos]


def _dabs(w, outs, vs):
    """|dO_v|.|out_v| per head [len(vs)][H]."""
    g = absf(w["dO"][vs])
    g = g.astype(np.float64) if g.dtype != np.uint16 else _widen_bits(g)
    return np.einsum("vhd,vhd->vh", g, np.abs(outs.take(vs)))


def _widen_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _opts_terms(opts, e_ids, shape):
    """(w_e [n][1], bias [n][H] or 0, c_e [n][H]) of the listed CSR edge ids."""
    opts = opts or {}
    ew = opts.get("ew")
    w_e = ew[e_ids].astype(np.float64)[:, None] if ew is not None else np.ones((len(e_ids), 1))
    bias = opts.get("bias")
    b = bias[e_ids].astype(np.float64) if bias is not None else 0.0
    c_all = opts.get("c_all")
    c = c_all[e_ids].astype(np.float64) if c_all is not None else np.ones(shape)
    return w_e, b, c


def dest_bounds(w, lse, outs, rows, opts=None):
    """Bounds for the destination pass over the listed rows' in-edges:
    dict(dq=[len(rows)][H][D], db=[n][H], sel=[n] CSR positions, and with
    opts dw=[n]).  lse [N][H] is the oracle's (fp64); opts (a dict, or None
    for plain logits) holds ew, bias and c_all (the dropout multipliers
    [E][H]), each None when that option is off."""
    D = w["D"]
    sq = math.sqrt(D)
    sub_ip, sub_ix, sel = sub_graph(w["indptr"], w["indices"], rows)
    rows = np.asarray(rows, np.int64)
    deg = np.diff(sub_ip)
    e_dst = np.repeat(rows, deg)
    dot = oracle.sddmm(sub_ip, sub_ix, w["Q"][rows], w["K"])  # <q_v, k_u> / sqrt(D)
    w_e, b, c = _opts_terms(opts, sel, dot.shape)
    alpha = np.exp(dot * w_e + b - lse[e_dst])
    da = oracle.sddmm(sub_ip, sub_ix, absf(w["dO"][rows]), absf(w["V"])) * sq  # |dO_v|.|v_u|
    wt = alpha * (c * da + np.repeat(_dabs(w, outs, rows), deg, axis=0))
    res = dict(sel=sel, db=wt)
    res["dq"] = oracle.spmm(sub_ip, sub_ix, wt * w_e, absf(w["K"])) / sq
    if opts is not None:
        absdot = oracle.sddmm(sub_ip, sub_ix, absf(w["Q"][rows]), absf(w["K"]))  # |q_v|.|k_u| / sqrt(D)
        res["dw"] = (wt * absdot).sum(1)
    return res


def source_bounds(w, lse, outs, srcs, opts=None, t_perm=None):
    """(B_dK, B_dV) [len(srcs)][H][D] for the source pass over the listed
    sources' out-edges (w["t_indptr"], w["t_indices"]: the source-sorted
    graph; t_perm its CSR positions, needed with logit options)."""
    D = w["D"]
    sq = math.sqrt(D)
    sub_ip, sub_dst, sel = sub_graph(w["t_indptr"], w["t_indices"], srcs)
    srcs = np.asarray(srcs, np.int64)
    e_dst = sub_dst.astype(np.int64)
    # roles swapped: the row is the source (its k, v), the gathered node the destination
    dot = oracle.sddmm(sub_ip, sub_dst, w["K"][srcs], w["Q"])
    e_ids = t_perm[sel].astype(np.int64) if t_perm is not None else None
    if opts and e_ids is None:
        raise ValueError("logit options need the transpose's CSR positions")
    w_e, b, c = _opts_terms(opts, e_ids, dot.shape) if opts else (1.0, 0.0, 1.0)
    alpha = np.exp(dot * w_e + b - lse[e_dst])
    da = oracle.sddmm(sub_ip, sub_dst, absf(w["V"][srcs]), absf(w["dO"])) * sq
    uniq, inv = np.unique(e_dst, return_inverse=True)
    wt = alpha * (c * da + _dabs(w, outs, uniq)[inv])
    BK = oracle.spmm(sub_ip, sub_dst, wt * w_e, absf(w["Q"])) / sq
    BV = oracle.spmm(sub_ip, sub_dst, alpha * c, absf(w["dO"]))
    return BK, BV
