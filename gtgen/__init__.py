"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

Holds no attention arithmetic: graphs (destination-sorted CSR) and Q/K/V
feature arrays only.  All randomness is counter based (``gtgen.c``), so a
workload is a pure function of its name and seed.

Workloads (shapes after the pages' examples; each a synthetic stand-in):

* ``tiny_random`` -- N=30 nodes, E=100 edges with uniform iid (src, dst),
  duplicates and self-loops kept, H=8, D=64, fp32.  The smoke graph of the
  gist "Efficient Sparse Transformer implementation with DGL's builtin
  operators" (its ``__main__`` block draws a 30-node, 100-edge random graph
  for a layer with 8 heads of 64 dims).
* ``molecules`` -- 128 molecule-like graphs (random recursive tree plus ~10%
  ring-closing edges, stored in both directions) batched block-diagonally,
  H=8, D=10, fp32.  Stands in for the ogbg-molhiv batches of "Graph
  Transformer in a Nutshell" (section Training; hidden 80 = 8 heads x 10).
* ``regular16`` -- N=100,000, every node has in-degree 16 with uniform
  sources, H=8, D=64, fp32.
* ``powerlaw`` -- N=1,000,000, E=16,000,000, in-degrees Zipf(1.8) clipped at
  50,000 assigned in random node order until E is reached, uniform sources,
  H=8, D=64, fp32.
* ``lognormal`` -- N=2,400,000, E=60,000,000, log-normal in-degrees (mean 25,
  log-space sigma 1.2) integerised by largest remainder, uniform sources,
  H=8, D=32, bf16 inputs = bf16(0.5 * N(0,1)).
"""
import ctypes
import os

import numpy as np

from . import _build

_LIB = None

# counter streams
S_GRAPH, S_Q, S_K, S_V, S_PERM, S_DEG, S_SRC, S_DOUT = 0, 1, 2, 3, 4, 5, 6, 7

F32, BF16 = 0, 1

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.gtgen_u64.restype = _u64
        L.gtgen_u64.argtypes = [_u64, _u64, _u64]
        L.gtgen_normal_f32.argtypes = [_u64, _u64, _i64, _dbl, _p]
        L.gtgen_normal_bf16.argtypes = [_u64, _u64, _i64, _dbl, _p]
        L.gtgen_uniform_f64.argtypes = [_u64, _u64, _i64, _dbl, _dbl, _p]
        L.gtgen_random_coo.argtypes = [_u64, _u64, _i64, _i64, _p, _p]
        L.gtgen_coo_to_dst_csr.argtypes = [_i64, _i64, _p, _p, _p, _p, _p]
        L.gtgen_csr_from_degrees.argtypes = [_u64, _u64, _i64, _p, _p, _p]
        L.gtgen_permutation.argtypes = [_u64, _u64, _i64, _p]
        L.gtgen_degrees_zipf.restype = _i64
        L.gtgen_degrees_zipf.argtypes = [_u64, _u64, _u64, _i64, _i64, _dbl, _i64, _p]
        L.gtgen_degrees_lognormal.argtypes = [_u64, _u64, _i64, _i64, _dbl, _dbl, _p]
        L.gtgen_molecules.argtypes = [_u64, _u64, _i64, _i64, _i64, _p, _p, _p, _p]
        _LIB = L
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ---------------------------------------------------------------- features

def normal_f32(seed, stream, shape, scale=1.0):
    out = np.empty(shape, dtype=np.float32)
    lib().gtgen_normal_f32(seed, stream, out.size, scale, _ptr(out))
    return out


def normal_bf16(seed, stream, shape, scale=1.0):
    """bf16 values as raw uint16 bits: bf16_rne(fp32(N(0,1)) * scale)."""
    out = np.empty(shape, dtype=np.uint16)
    lib().gtgen_normal_bf16(seed, stream, out.size, scale, _ptr(out))
    return out


def uniform_f64(seed, stream, n, lo=0.0, hi=1.0):
    out = np.empty(n, dtype=np.float64)
    lib().gtgen_uniform_f64(seed, stream, n, lo, hi, _ptr(out))
    return out


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- graphs

def random_coo(seed, N, E, stream=S_GRAPH):
    src = np.empty(E, dtype=np.int32)
    dst = np.empty(E, dtype=np.int32)
    if E:
        lib().gtgen_random_coo(seed, stream, N, E, _ptr(src), _ptr(dst))
    return src, dst


def permutation(seed, n, stream=S_PERM):
    """A seeded uniform random permutation of range(n) (Fisher-Yates), int64."""
    out = np.empty(n, dtype=np.int64)
    if n:
        lib().gtgen_permutation(seed, stream, n, _ptr(out))
    return out


def coo_to_csr(N, src, dst, return_perm=False):
    """Stable counting sort by destination -> (indptr int64[N+1], indices int32[E])."""
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    E = len(src)
    indptr = np.empty(N + 1, dtype=np.int64)
    indices = np.empty(E, dtype=np.int32)
    perm = np.empty(E, dtype=np.int64) if return_perm else None
    lib().gtgen_coo_to_dst_csr(N, E, _ptr(src), _ptr(dst), _ptr(indptr), _ptr(indices), _ptr(perm))
    return (indptr, indices, perm) if return_perm else (indptr, indices)


def csr_from_degrees(seed, deg, stream=S_SRC):
    deg = np.ascontiguousarray(deg, dtype=np.int64)
    N = len(deg)
    E = int(deg.sum())
    indptr = np.empty(N + 1, dtype=np.int64)
    indices = np.empty(E, dtype=np.int32)
    lib().gtgen_csr_from_degrees(seed, stream, N, _ptr(deg), _ptr(indptr), _ptr(indices))
    return indptr, indices


def degrees_zipf(seed, N, E, alpha=1.8, cap=50000):
    deg = np.empty(N, dtype=np.int64)
    lib().gtgen_degrees_zipf(seed, S_PERM, S_DEG, N, E, alpha, cap, _ptr(deg))
    return deg


def degrees_lognormal(seed, N, E, mean=25.0, sigma=1.2):
    deg = np.empty(N, dtype=np.int64)
    lib().gtgen_degrees_lognormal(seed, S_DEG, N, E, mean, sigma, _ptr(deg))
    return deg


def molecules_coo(seed, ngraphs=128, nmin=10, nmax=50):
    N = ctypes.c_int64()
    E = ctypes.c_int64()
    L = lib()
    L.gtgen_molecules(seed, S_GRAPH, ngraphs, nmin, nmax, ctypes.byref(N), ctypes.byref(E), None, None)
    src = np.empty(E.value, dtype=np.int32)
    dst = np.empty(E.value, dtype=np.int32)
    L.gtgen_molecules(seed, S_GRAPH, ngraphs, nmin, nmax, ctypes.byref(N), ctypes.byref(E), _ptr(src), _ptr(dst))
    return N.value, src, dst


# ---------------------------------------------------------------- workloads

CONFIGS = {
    "tiny_random": dict(H=8, D=64, dtype=F32, scale=1.0),
    "molecules": dict(H=8, D=10, dtype=F32, scale=1.0),
    "regular16": dict(H=8, D=64, dtype=F32, scale=1.0, N=100_000, deg=16),
    "powerlaw": dict(H=8, D=64, dtype=F32, scale=1.0, N=1_000_000, E=16_000_000, alpha=1.8, cap=50_000),
    "lognormal": dict(H=8, D=32, dtype=BF16, scale=0.5, N=2_400_000, E=60_000_000, mean=25.0, sigma=1.2),
}


def make_graph(name, seed=0):
    c = CONFIGS[name]
    if name == "tiny_random":
        N, E = 30, 100
        src, dst = random_coo(seed, N, E)
        indptr, indices = coo_to_csr(N, src, dst)
    elif name == "molecules":
        N, src, dst = molecules_coo(seed)
        indptr, indices = coo_to_csr(N, src, dst)
    elif name == "regular16":
        N = c["N"]
        indptr, indices = csr_from_degrees(seed, np.full(N, c["deg"], dtype=np.int64))
    elif name == "powerlaw":
        indptr, indices = csr_from_degrees(seed, degrees_zipf(seed, c["N"], c["E"], c["alpha"], c["cap"]))
    elif name == "lognormal":
        indptr, indices = csr_from_degrees(seed, degrees_lognormal(seed, c["N"], c["E"], c["mean"], c["sigma"]))
    else:
        raise KeyError(name)
    return indptr, indices


def make_features(N, H, D, dtype, seed=0, scale=1.0):
    """Q, K, V as [N][H][D] arrays: float32, or uint16 bf16 bits when dtype == BF16."""
    gen = normal_f32 if dtype == F32 else normal_bf16
    return tuple(gen(seed, s, (N, H, D), scale) for s in (S_Q, S_K, S_V))


def make_grad(N, H, D, dtype, seed=0, scale=1.0):
    """An upstream gradient dL/dout [N][H][D], drawn like the features (own stream)."""
    gen = normal_f32 if dtype == F32 else normal_bf16
    return gen(seed, S_DOUT, (N, H, D), scale)


def source_sorted(indptr, indices, want_perm=False):
    """The same edges grouped by source: (t_indptr, t_indices) with t_indices holding
    each out-edge's destination, out-edges of a source in destination-CSR order;
    with want_perm also t_perm (int32), each out-edge's destination-CSR position."""
    N = len(indptr) - 1
    dst = np.repeat(np.arange(N, dtype=np.int32), np.diff(indptr))
    if not want_perm:
        return coo_to_csr(N, dst, np.ascontiguousarray(indices, dtype=np.int32))
    t_indptr, t_indices, perm = coo_to_csr(N, dst, np.ascontiguousarray(indices, dtype=np.int32), return_perm=True)
    return t_indptr, t_indices, perm.astype(np.int32)


def make_workload(name, seed=0, with_features=True):
    c = CONFIGS[name]
    indptr, indices = make_graph(name, seed)
    N = len(indptr) - 1
    w = dict(name=name, N=N, E=int(indptr[-1]), H=c["H"], D=c["D"], dtype=c["dtype"],
             indptr=indptr, indices=indices)
    if with_features:
        w["Q"], w["K"], w["V"] = make_features(N, c["H"], c["D"], c["dtype"], seed, c["scale"])
    return w
