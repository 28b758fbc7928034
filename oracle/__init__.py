"""fp64 CPU oracle for sparse multi-head graph attention (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The GPU library
never does, and shares no code with it.

What it computes, and the passages it follows, is stated in ``oracle.c``:
per destination v and head h, scores s_e = <q_v, k_u>/sqrt(D) over the
in-edges u->v (SDDMM), a softmax over those scores, and the weighted sum of
the source V rows (SpMM); zero for a destination with no in-edges.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
things other than itself (library masked attention, closed forms, hand-worked
golden examples, invariants); ``tests/test_oracle_mutants.py`` shows that
plausible mistakes planted in a copy of oracle.c fail those pins.
"""
import ctypes
import os

import numpy as np

from . import _build

F32, BF16, F64 = 0, 1, 2

_LIBS = {}
_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p


def load(path=None):
    """Load liboracle.so (built on first use), or another build of oracle.c at path."""
    path = path or _build.LIB
    if path not in _LIBS:
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_sddmm.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _int]
        L.oracle_edge_softmax.argtypes = [_i64, _i64, _int, _p, _p, _p, _int]
        L.oracle_spmm.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _int]
        L.oracle_fwd_rows.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _p, _i64, _p, _p, _p, _int]
        L.oracle_fwd.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _p, _p, _p, _int]
        L.oracle_max_threads.restype = _int
        _LIBS[path] = L
    return _LIBS[path]


def _p_(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float64:
        return F64
    raise TypeError("features must be float32, float64 or uint16 (bf16 bits), got %s" % x.dtype)


def _csr(indptr, indices):
    return (np.ascontiguousarray(indptr, dtype=np.int64), np.ascontiguousarray(indices, dtype=np.int32))


def _shape(Q):
    if Q.ndim != 3:
        raise ValueError("features are [N][H][D]")
    return Q.shape


class Oracle:
    """Bound to one build of oracle.c (the default, or a test's variant)."""

    def __init__(self, path=None):
        self.L = load(path)

    def max_threads(self):
        return self.L.oracle_max_threads()

    def fwd(self, indptr, indices, Q, K, V, want_edges=False, nthreads=0):
        """Whole forward: out [N][H][D] (fp64); with want_edges also scores and alpha [E][H]."""
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        E = len(indices)
        dt = _dtype_of(Q)
        Q, K, V = (np.ascontiguousarray(x) for x in (Q, K, V))
        out = np.empty((N, H, D), dtype=np.float64)
        s = np.empty((E, H), dtype=np.float64) if want_edges else None
        a = np.empty((E, H), dtype=np.float64) if want_edges else None
        rc = self.L.oracle_fwd(N, E, H, D, dt, _p_(indptr), _p_(indices), _p_(Q), _p_(K), _p_(V),
                               _p_(out), _p_(s), _p_(a), nthreads)
        if rc:
            raise ValueError("oracle_fwd rejected its arguments")
        return (out, s, a) if want_edges else out

    def fwd_rows(self, indptr, indices, Q, K, V, rows, nthreads=0, want_edges=False):
        """Forward for the listed destination rows only: out [len(rows)][H][D]."""
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        E = len(indices)
        dt = _dtype_of(Q)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((len(rows), H, D), dtype=np.float64)
        ne = int((indptr[rows + 1] - indptr[rows]).sum()) if len(rows) else 0
        s = np.empty((ne, H), dtype=np.float64) if want_edges else None
        a = np.empty((ne, H), dtype=np.float64) if want_edges else None
        rc = self.L.oracle_fwd_rows(N, E, H, D, dt, _p_(indptr), _p_(indices), _p_(Q), _p_(K), _p_(V),
                                    _p_(rows), len(rows), _p_(out), _p_(s), _p_(a), nthreads)
        if rc:
            raise ValueError("oracle_fwd_rows rejected its arguments")
        return (out, s, a) if want_edges else out

    def sddmm(self, indptr, indices, Q, K, nthreads=0):
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        E = len(indices)
        Q, K = np.ascontiguousarray(Q), np.ascontiguousarray(K)
        s = np.empty((E, H), dtype=np.float64)
        rc = self.L.oracle_sddmm(N, E, H, D, _dtype_of(Q), _p_(indptr), _p_(indices), _p_(Q), _p_(K), _p_(s),
                                 nthreads)
        if rc:
            raise ValueError("oracle_sddmm rejected its arguments")
        return s

    def edge_softmax(self, indptr, scores, nthreads=0):
        indptr = np.ascontiguousarray(indptr, dtype=np.int64)
        scores = np.ascontiguousarray(scores, dtype=np.float64)
        E, H = scores.shape
        N = len(indptr) - 1
        a = np.empty((E, H), dtype=np.float64)
        rc = self.L.oracle_edge_softmax(N, E, H, _p_(indptr), _p_(scores), _p_(a), nthreads)
        if rc:
            raise ValueError("oracle_edge_softmax rejected its arguments")
        return a

    def spmm(self, indptr, indices, alpha, V, nthreads=0):
        """out [len(indptr)-1][H][D]; V may hold more rows than indptr has (sources index V)."""
        indptr, indices = _csr(indptr, indices)
        _, H, D = _shape(V)
        N = len(indptr) - 1
        E = len(indices)
        alpha = np.ascontiguousarray(alpha, dtype=np.float64)
        V = np.ascontiguousarray(V)
        out = np.empty((N, H, D), dtype=np.float64)
        rc = self.L.oracle_spmm(N, E, H, D, _dtype_of(V), _p_(indptr), _p_(indices), _p_(alpha), _p_(V),
                                _p_(out), nthreads)
        if rc:
            raise ValueError("oracle_spmm rejected its arguments")
        return out


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fwd(*a, **k):
    return default().fwd(*a, **k)


def fwd_rows(*a, **k):
    return default().fwd_rows(*a, **k)


def sddmm(*a, **k):
    return default().sddmm(*a, **k)


def edge_softmax(*a, **k):
    return default().edge_softmax(*a, **k)


def spmm(*a, **k):
    return default().spmm(*a, **k)


# ---------------------------------------------------------------- backward

def _bind_bwd(L):
    if getattr(L, "_bwd_bound", False):
        return L
    L.oracle_row_stats.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _p, _p, _p, _int]
    L.oracle_dq_rows.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _int]
    L.oracle_dkv_sources.argtypes = [_i64, _i64, _int, _int, _int, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _p,
                                     _int]
    L._bwd_bound = True
    return L


def transpose_csr(indptr, indices):
    """Source-sorted view of a destination-sorted CSR: for source u, the destinations
    of its out-edges in edge order (a stable sort of the edges by source)."""
    indptr, indices = _csr(indptr, indices)
    N = len(indptr) - 1
    dst = np.repeat(np.arange(N, dtype=np.int32), np.diff(indptr))
    order = np.argsort(indices, kind="stable")
    t_indptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(np.bincount(indices, minlength=N), out=t_indptr[1:])
    return t_indptr, np.ascontiguousarray(dst[order], dtype=np.int32)


class _Bwd:
    def row_stats(self, indptr, indices, Q, K, V, dO, nthreads=0):
        """(lse, delta), each [N][H]: log-sum-exp of the scores and sum alpha (dO . v)."""
        L = _bind_bwd(self.L)
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        lse = np.empty((N, H))
        delta = np.empty((N, H))
        rc = L.oracle_row_stats(N, len(indices), H, D, _dtype_of(Q), _p_(indptr), _p_(indices), _p_(Q), _p_(K),
                                _p_(V), _p_(dO), _p_(lse), _p_(delta), nthreads)
        if rc:
            raise ValueError("oracle_row_stats rejected its arguments")
        return lse, delta

    def dq_rows(self, indptr, indices, Q, K, V, dO, lse, delta, rows, nthreads=0):
        L = _bind_bwd(self.L)
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        delta = np.ascontiguousarray(delta, dtype=np.float64)
        dq = np.empty((len(rows), H, D))
        rc = L.oracle_dq_rows(N, len(indices), H, D, _dtype_of(Q), _p_(indptr), _p_(indices), _p_(Q), _p_(K),
                              _p_(V), _p_(dO), _p_(lse), _p_(delta), _p_(rows), len(rows), _p_(dq), nthreads)
        if rc:
            raise ValueError("oracle_dq_rows rejected its arguments")
        return dq

    def dkv_sources(self, t_indptr, t_indices, Q, K, V, dO, lse, delta, srcs, nthreads=0):
        L = _bind_bwd(self.L)
        t_indptr, t_indices = _csr(t_indptr, t_indices)
        _, H, D = _shape(Q)
        N = len(t_indptr) - 1  # source nodes (rows of K, V, dK, dV)
        srcs = np.ascontiguousarray(srcs, dtype=np.int64)
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        delta = np.ascontiguousarray(delta, dtype=np.float64)
        dk = np.empty((len(srcs), H, D))
        dv = np.empty((len(srcs), H, D))
        rc = L.oracle_dkv_sources(N, len(t_indices), H, D, _dtype_of(Q), _p_(t_indptr), _p_(t_indices), _p_(Q),
                                  _p_(K), _p_(V), _p_(dO), _p_(lse), _p_(delta), _p_(srcs), len(srcs), _p_(dk),
                                  _p_(dv), nthreads)
        if rc:
            raise ValueError("oracle_dkv_sources rejected its arguments")
        return dk, dv

    def bwd(self, indptr, indices, Q, K, V, dO, nthreads=0):
        """Whole backward: (dQ, dK, dV, lse, delta), all fp64."""
        N = len(indptr) - 1
        lse, delta = self.row_stats(indptr, indices, Q, K, V, dO, nthreads)
        allv = np.arange(N, dtype=np.int64)
        dq = self.dq_rows(indptr, indices, Q, K, V, dO, lse, delta, allv, nthreads)
        t_indptr, t_indices = transpose_csr(indptr, indices)
        dk, dv = self.dkv_sources(t_indptr, t_indices, Q, K, V, dO, lse, delta, allv, nthreads)
        return dq, dk, dv, lse, delta


class _Graph:
    def coo_to_csr(self, n_dst, src, dst, n_src=None):
        """(indptr int64[n_dst+1], indices int32[E], perm int64[E]): stable grouping by destination."""
        L = self.L
        if not getattr(L, "_graph_bound", False):
            L.oracle_coo_to_csr.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p]
            L._graph_bound = True
        src = np.ascontiguousarray(src, dtype=np.int32)
        dst = np.ascontiguousarray(dst, dtype=np.int32)
        if src.shape != dst.shape:
            raise ValueError("src and dst differ in length")
        n_src = n_dst if n_src is None else n_src
        E = len(src)
        indptr = np.empty(n_dst + 1, dtype=np.int64)
        indices = np.empty(E, dtype=np.int32)
        perm = np.empty(E, dtype=np.int64)
        rc = L.oracle_coo_to_csr(n_dst, n_src, E, _p_(src), _p_(dst), _p_(indptr), _p_(indices), _p_(perm))
        if rc:
            raise ValueError("oracle_coo_to_csr rejected its arguments")
        return indptr, indices, perm

    def source_sorted(self, indptr, indices, n_src=None, want_perm=False):
        """The CSR's edges grouped by source (destinations listed in CSR order);
        with want_perm also t_perm, the CSR position of each out-edge."""
        indptr, indices = _csr(indptr, indices)
        n_dst = len(indptr) - 1
        n_src = n_dst if n_src is None else n_src
        dst = np.repeat(np.arange(n_dst, dtype=np.int32), np.diff(indptr))
        t_indptr, t_indices, perm = self.coo_to_csr(n_src, dst, indices, n_src=n_dst)
        return (t_indptr, t_indices, perm.astype(np.int32)) if want_perm else (t_indptr, t_indices)


for _name in ("row_stats", "dq_rows", "dkv_sources", "bwd"):
    setattr(Oracle, _name, getattr(_Bwd, _name))
for _name in ("coo_to_csr", "source_sorted"):
    setattr(Oracle, _name, getattr(_Graph, _name))


_dbl = ctypes.c_double
_u64 = ctypes.c_uint64


def _bind_ex(L):
    if not getattr(L, "_ex_bound", False):
        L.oracle_philox_word.restype = _u64
        L.oracle_philox_word.argtypes = [_u64, _u64]
        L.oracle_fwd_rows_ex.argtypes = [_i64, _i64, _int, _int, _int] + [_p] * 7 + [_dbl, _u64, _p, _i64, _p, _p, _int]
        L.oracle_row_stats_ex.argtypes = [_i64, _i64, _int, _int, _int] + [_p] * 8 + [_dbl, _u64, _p, _p, _int]
        L.oracle_dq_rows_ex.argtypes = ([_i64, _i64, _int, _int, _int] + [_p] * 8 + [_dbl, _u64, _p, _p, _p, _i64]
                                        + [_p] * 3 + [_int])
        L.oracle_dkv_sources_ex.argtypes = ([_i64, _i64, _int, _int, _int] + [_p] * 9 + [_dbl, _u64, _p, _p, _p, _i64]
                                            + [_p] * 2 + [_int])
        L._ex_bound = True
    return L


def _f32_or_none(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float32)


class _Ex:
    """The logit variants (additive bias [E][H], edge weights [E]) and attention
    dropout (probability p, generator seed), as defined in oracle.c."""

    def philox_word(self, seed, i):
        return int(_bind_ex(self.L).oracle_philox_word(seed, i))

    def fwd_ex(self, indptr, indices, Q, K, V, bias=None, ew=None, drop_p=0.0, seed=0, rows=None, want_lse=False,
               nthreads=0):
        L = _bind_ex(self.L)
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        Q, K, V = (np.ascontiguousarray(x) for x in (Q, K, V))
        bias, ew = _f32_or_none(bias), _f32_or_none(ew)
        out = np.empty((len(rows), H, D))
        lse = np.empty((len(rows), H)) if want_lse else None
        rc = L.oracle_fwd_rows_ex(N, len(indices), H, D, _dtype_of(Q), _p_(indptr), _p_(indices), _p_(Q), _p_(K),
                                  _p_(V), _p_(bias), _p_(ew), float(drop_p), seed, _p_(rows), len(rows), _p_(out),
                                  _p_(lse), nthreads)
        if rc:
            raise ValueError("oracle_fwd_rows_ex rejected its arguments")
        return (out, lse) if want_lse else out

    def row_stats_ex(self, indptr, indices, Q, K, V, dO, bias=None, ew=None, drop_p=0.0, seed=0, nthreads=0):
        L = _bind_ex(self.L)
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        bias, ew = _f32_or_none(bias), _f32_or_none(ew)
        lse = np.empty((N, H))
        delta = np.empty((N, H))
        rc = L.oracle_row_stats_ex(N, len(indices), H, D, _dtype_of(Q), _p_(indptr), _p_(indices), _p_(Q), _p_(K),
                                   _p_(V), _p_(dO), _p_(bias), _p_(ew), float(drop_p), seed, _p_(lse), _p_(delta),
                                   nthreads)
        if rc:
            raise ValueError("oracle_row_stats_ex rejected its arguments")
        return lse, delta

    def dq_rows_ex(self, indptr, indices, Q, K, V, dO, lse, delta, rows, bias=None, ew=None, drop_p=0.0, seed=0,
                   dbias=None, dw=None, nthreads=0):
        """dQ of the rows; fills dbias [E][H] / dw [E] (if given) at the rows' edges."""
        L = _bind_ex(self.L)
        indptr, indices = _csr(indptr, indices)
        N, H, D = _shape(Q)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        bias, ew = _f32_or_none(bias), _f32_or_none(ew)
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        delta = np.ascontiguousarray(delta, dtype=np.float64)
        for a in (dbias, dw):
            assert a is None or (a.dtype == np.float64 and a.flags.c_contiguous)
        dq = np.empty((len(rows), H, D))
        rc = L.oracle_dq_rows_ex(N, len(indices), H, D, _dtype_of(Q), _p_(indptr), _p_(indices), _p_(Q), _p_(K),
                                 _p_(V), _p_(dO), _p_(bias), _p_(ew), float(drop_p), seed, _p_(lse), _p_(delta),
                                 _p_(rows), len(rows), _p_(dq), _p_(dbias), _p_(dw), nthreads)
        if rc:
            raise ValueError("oracle_dq_rows_ex rejected its arguments")
        return dq

    def dkv_sources_ex(self, t_indptr, t_indices, t_perm, Q, K, V, dO, lse, delta, srcs, bias=None, ew=None,
                       drop_p=0.0, seed=0, nthreads=0):
        L = _bind_ex(self.L)
        t_indptr, t_indices = _csr(t_indptr, t_indices)
        t_perm = np.ascontiguousarray(t_perm, dtype=np.int32)
        _, H, D = _shape(Q)
        N = len(t_indptr) - 1
        srcs = np.ascontiguousarray(srcs, dtype=np.int64)
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        bias, ew = _f32_or_none(bias), _f32_or_none(ew)
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        delta = np.ascontiguousarray(delta, dtype=np.float64)
        dk = np.empty((len(srcs), H, D))
        dv = np.empty((len(srcs), H, D))
        rc = L.oracle_dkv_sources_ex(N, len(t_indices), H, D, _dtype_of(Q), _p_(t_indptr), _p_(t_indices),
                                     _p_(t_perm), _p_(Q), _p_(K), _p_(V), _p_(dO), _p_(bias), _p_(ew), float(drop_p),
                                     seed, _p_(lse), _p_(delta), _p_(srcs), len(srcs), _p_(dk), _p_(dv), nthreads)
        if rc:
            raise ValueError("oracle_dkv_sources_ex rejected its arguments")
        return dk, dv

    def bwd_ex(self, indptr, indices, Q, K, V, dO, bias=None, ew=None, drop_p=0.0, seed=0, nthreads=0):
        """Whole backward with the variants: dict(dq, dk, dv, dbias, dw, lse, delta), fp64."""
        N = len(indptr) - 1
        E = len(indices)
        H = Q.shape[1]
        kw = dict(bias=bias, ew=ew, drop_p=drop_p, seed=seed, nthreads=nthreads)
        lse, delta = self.row_stats_ex(indptr, indices, Q, K, V, dO, **kw)
        allv = np.arange(N, dtype=np.int64)
        dbias = np.zeros((E, H))
        dw = np.zeros(E)
        dq = self.dq_rows_ex(indptr, indices, Q, K, V, dO, lse, delta, allv, dbias=dbias, dw=dw, **kw)
        t_indptr, t_indices, t_perm = self.source_sorted(indptr, indices, want_perm=True)
        dk, dv = self.dkv_sources_ex(t_indptr, t_indices, t_perm, Q, K, V, dO, lse, delta, allv, **kw)
        return dict(dq=dq, dk=dk, dv=dv, dbias=dbias, dw=dw, lse=lse, delta=delta)


for _name in ("philox_word", "fwd_ex", "row_stats_ex", "dq_rows_ex", "dkv_sources_ex", "bwd_ex"):
    setattr(Oracle, _name, getattr(_Ex, _name))


def fwd_ex(*a, **k):
    return default().fwd_ex(*a, **k)


def bwd_ex(*a, **k):
    return default().bwd_ex(*a, **k)


def row_stats_ex(*a, **k):
    return default().row_stats_ex(*a, **k)


def dq_rows_ex(*a, **k):
    return default().dq_rows_ex(*a, **k)


def dkv_sources_ex(*a, **k):
    return default().dkv_sources_ex(*a, **k)


def philox_word(*a, **k):
    return default().philox_word(*a, **k)


def bwd(*a, **k):
    return default().bwd(*a, **k)


def coo_to_csr(*a, **k):
    return default().coo_to_csr(*a, **k)


def source_sorted(*a, **k):
    return default().source_sorted(*a, **k)


def row_stats(*a, **k):
    return default().row_stats(*a, **k)


def dq_rows(*a, **k):
    return default().dq_rows(*a, **k)


def dkv_sources(*a, **k):
    return default().dkv_sources(*a, **k)
