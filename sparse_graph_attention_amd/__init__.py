"""Python binding of libgtattn: sparse multi-head graph attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libgtattn.so`` (built from ``csrc/`` for gfx950); PyTorch
supplies device memory and the current stream.  There is no CPU fallback: if
the library is missing or the tensors are not on the GPU, calls fail.

The functions have the names of the C entry points declared in
``include/gtattn.h`` and follow their contracts:

* ``gt_sparse_mha_fwd(indptr, indices, Q, K, V, out=None)`` -- fused forward;
* ``gt_sparse_mha_fwd_noalloc(indptr, indices, Q, K, V, out)`` -- the same with
  no device allocation (for callers that cannot allocate);
* ``gt_sparse_mha_fwd_lse(indptr, indices, Q, K, V, out=None, lse=None)`` --
  fused forward that also returns the per-destination log-sum-exp [N][H];
* ``gt_sparse_mha_bwd(indptr, indices, t_indptr, t_indices, Q, K, V, out, dout,
  lse)`` -- (dQ, dK, dV) given the source-sorted transpose of the graph;
* ``gt_sddmm(indptr, indices, Q, K, scores=None)`` -- scores [E][H] (fp32);
* ``gt_edge_softmax(indptr, scores, alpha=None)`` -- alpha [E][H] (fp32);
* ``gt_spmm(indptr, indices, alpha, V, out=None)`` -- out [N][H][D];
* ``gt_validate_csr(indptr, indices, N)`` -- device-side CSR check;
* ``gt_calib_gather(indices, K, V)`` -- measurement aid: the K and V row
  gathers of the attention alone, with their XOR checksum;
* ``gt_sparse_mha_fwd_ex`` / ``gt_sparse_mha_bwd_ex`` -- with an additive
  logit bias [E][H], edge weights [E] and attention dropout (keyword
  arguments ``bias``, ``edge_weight``, ``dropout_p``, ``dropout_seed``);
* ``gt_sparse_mha_fwd_layout`` / ``gt_sparse_mha_bwd_layout`` -- the same with
  features in the head-innermost layout [N][D][H] (``layout="ndh"``);
* ``gt_coo_to_csr(src, dst, n_dst)`` -- (indptr, indices[, perm]) built on the GPU;
* ``gt_plan_create(indptr, indices)`` / ``gt_plan_create_coo(src, dst, n_dst)``
  -- a reusable graph plan (``GtPlan``), ``gt_plan_destroy``, ``gt_plan_info``,
  ``gt_plan_copy_graph``;
* ``gt_sparse_mha_fwd_plan(plan, Q, K, V)`` / ``gt_sparse_mha_bwd_plan(plan, ...)``;
* ``gt_scratch_release(stream=None)`` / ``gt_scratch_bytes(stream=None)`` -- the
  library's per-stream work buffer;
* ``gt_config_set`` / ``gt_config_get`` / ``gt_config_chunk_edges``, ``gt_profile_begin`` /
  ``gt_profile_end``.

Every tensor must be contiguous and on the current device; calls are
asynchronous on ``stream`` (default: torch's current stream).

Graphs are destination-sorted CSR: ``indptr`` int64 [N+1], ``indices`` int32
[E] holding the source of each in-edge.  Features are [N][H][D] tensors of
dtype float32 or bfloat16.
"""
import ctypes
import os

import torch  # loaded first: libgtattn then binds to the HIP runtime torch already holds

from . import _build

GT_F32, GT_BF16 = 0, 1
GT_OK, GT_EINVAL, GT_EUNSUPPORTED, GT_ENOMEM, GT_EHIP = 0, 1, 2, 3, 4
GT_CFG_CHUNK_EDGES = 0
GT_PLAN_TRANSPOSE = 1
GT_LAYOUT_NHD, GT_LAYOUT_NDH = 0, 1

EXPORTS = (
    "gt_sparse_mha_fwd",
    "gt_sparse_mha_fwd_noalloc",
    "gt_sparse_mha_fwd_lse",
    "gt_sparse_mha_bwd",
    "gt_sparse_mha_fwd_ex",
    "gt_sparse_mha_bwd_ex",
    "gt_sparse_mha_fwd_layout",
    "gt_sparse_mha_bwd_layout",
    "gt_sddmm",
    "gt_edge_softmax",
    "gt_spmm",
    "gt_validate_csr",
    "gt_calib_gather",
    "gt_coo_to_csr",
    "gt_plan_create",
    "gt_plan_create_coo",
    "gt_plan_destroy",
    "gt_plan_info",
    "gt_plan_copy_graph",
    "gt_sparse_mha_fwd_plan",
    "gt_sparse_mha_bwd_plan",
    "gt_status_string",
    "gt_last_error",
    "gt_config_set",
    "gt_config_get",
    "gt_config_chunk_edges",
    "gt_scratch_release",
    "gt_scratch_bytes",
    "gt_profile_begin",
    "gt_profile_end",
)

_lib = None
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class LogitOpts(ctypes.Structure):
    """gt_logit_opts."""
    _fields_ = [("bias", ctypes.c_void_p), ("edge_weight", ctypes.c_void_p), ("dropout_p", ctypes.c_double),
                ("dropout_seed", ctypes.c_uint64)]


class GtError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (%d): %s" % (where, lib().gt_status_string(status).decode(), status,
                                             lib().gt_last_error().decode()))


def lib():
    """The loaded libgtattn.so (compiled on first use if it is not built yet)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.gt_sparse_mha_fwd.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]
        L.gt_sparse_mha_fwd_noalloc.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]
        L.gt_sparse_mha_fwd_lse.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]
        L.gt_sparse_mha_bwd.argtypes = [_p] * 13 + [_i64, _i64, _i32, _i32, _i32, _p]
        _o = ctypes.POINTER(LogitOpts)
        L.gt_sparse_mha_fwd_ex.argtypes = [_p] * 7 + [_i64, _i64, _i32, _i32, _i32, _o, _p]
        L.gt_sparse_mha_bwd_ex.argtypes = [_p] * 16 + [_i64, _i64, _i32, _i32, _i32, _o, _p]
        L.gt_sparse_mha_fwd_layout.argtypes = [_p] * 7 + [_i64, _i64, _i32, _i32, _i32, _i32, _o, _p]
        L.gt_sparse_mha_bwd_layout.argtypes = [_p] * 16 + [_i64, _i64, _i32, _i32, _i32, _i32, _o, _p]
        L.gt_sddmm.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]
        L.gt_edge_softmax.argtypes = [_p, _p, _p, _i64, _i64, _i32, _p]
        L.gt_spmm.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]
        L.gt_validate_csr.argtypes = [_p, _p, _i64, _i64, _p]
        L.gt_calib_gather.argtypes = [_p, _i64, _p, _p, _i64, _i32, _p, _p]
        L.gt_coo_to_csr.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, _p, _p]
        L.gt_plan_create.argtypes = [_p, _p, _i64, _i64, _i64, _i32, _p, ctypes.POINTER(_p)]
        L.gt_plan_create_coo.argtypes = [_p, _p, _i64, _i64, _i64, _i32, _p, ctypes.POINTER(_p)]
        L.gt_plan_destroy.argtypes = [_p]
        L.gt_plan_info.argtypes = [_p] + [ctypes.POINTER(_i64)] * 3 + [ctypes.POINTER(_p)] * 5
        L.gt_plan_copy_graph.argtypes = [_p] * 7
        L.gt_sparse_mha_fwd_plan.argtypes = [_p] * 6 + [_i32, _i32, _i32, ctypes.POINTER(LogitOpts), _p]
        L.gt_sparse_mha_bwd_plan.argtypes = [_p] * 12 + [_i32, _i32, _i32, ctypes.POINTER(LogitOpts), _p]
        L.gt_status_string.restype = ctypes.c_char_p
        L.gt_status_string.argtypes = [ctypes.c_int]
        L.gt_last_error.restype = ctypes.c_char_p
        L.gt_last_error.argtypes = []
        L.gt_config_set.argtypes = [_i32, _i64]
        L.gt_config_get.restype = _i64
        L.gt_config_get.argtypes = [_i32]
        L.gt_config_chunk_edges.restype = _i64
        L.gt_config_chunk_edges.argtypes = [_i64, _i32]
        L.gt_scratch_release.argtypes = [_p]
        L.gt_scratch_release.restype = ctypes.c_int
        L.gt_scratch_bytes.argtypes = [_p]
        L.gt_scratch_bytes.restype = _i64
        L.gt_profile_begin.argtypes = [_i32]
        L.gt_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(_i64)]
        for name in ("gt_coo_to_csr", "gt_plan_create", "gt_plan_create_coo", "gt_plan_destroy", "gt_plan_info",
                     "gt_plan_copy_graph", "gt_sparse_mha_fwd_plan", "gt_sparse_mha_bwd_plan"):
            getattr(L, name).restype = ctypes.c_int
        for name in ("gt_sparse_mha_fwd_ex", "gt_sparse_mha_bwd_ex", "gt_sparse_mha_fwd_layout",
                     "gt_sparse_mha_bwd_layout"):
            getattr(L, name).restype = ctypes.c_int
        for name in ("gt_sparse_mha_fwd", "gt_sparse_mha_fwd_noalloc", "gt_sparse_mha_fwd_lse", "gt_sparse_mha_bwd", "gt_sddmm", "gt_edge_softmax", "gt_spmm", "gt_validate_csr",
                     "gt_calib_gather", "gt_config_set", "gt_profile_begin", "gt_profile_end"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc, where):
    if rc != GT_OK:
        raise GtError(rc, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    elif stream.device.index != torch.cuda.current_device():
        raise ValueError("the stream is on cuda:%d but the current device is cuda:%d" % (
            stream.device.index, torch.cuda.current_device()))
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return GT_F32
    if t.dtype == torch.bfloat16:
        return GT_BF16
    raise TypeError("features must be float32 or bfloat16, got %s" % t.dtype)


def _need_gpu(*ts):
    """Every tensor on the GPU, contiguous, and on the current device: the
    library launches on the current device, where another device's pointers
    would not be valid."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libgtattn works on GPU tensors only; got a %s tensor" % t.device)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device.index
        elif t.device.index != dev:
            raise ValueError("tensors on several devices (cuda:%d and cuda:%d)" % (dev, t.device.index))
    if dev is not None and dev != torch.cuda.current_device():
        raise ValueError("tensors are on cuda:%d but the current device is cuda:%d; call inside "
                         "torch.cuda.device(%d)" % (dev, torch.cuda.current_device(), dev))


def _csr(indptr, indices):
    if indptr.dtype != torch.int64 or indices.dtype != torch.int32:
        raise TypeError("indptr must be int64 and indices int32")
    return indptr.numel() - 1, indices.numel()


def gt_sparse_mha_fwd(indptr, indices, Q, K, V, out=None, stream=None):
    N, E = _csr(indptr, indices)
    if Q.dim() != 3 or Q.shape[0] != N or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must all be [N][H][D] with N = len(indptr) - 1")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    if out is None:
        out = torch.empty_like(Q)
    elif out.shape != Q.shape or out.dtype != Q.dtype:
        raise ValueError("out must match Q in shape and dtype")
    _need_gpu(indptr, indices, Q, K, V, out)
    H, D = Q.shape[1], Q.shape[2]
    _check(lib().gt_sparse_mha_fwd(_ptr(indptr), _ptr(indices), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), N, E, H, D,
                                   _dtype_code(Q), _stream(stream)), "gt_sparse_mha_fwd")
    return out


def gt_sparse_mha_fwd_noalloc(indptr, indices, Q, K, V, out, stream=None):
    """The fused forward into the caller's `out`, with no device allocation: its
    work lists and split-row partials live in the library's static device array."""
    N, E = _csr(indptr, indices)
    if Q.dim() != 3 or Q.shape[0] != N or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must all be [N][H][D] with N = len(indptr) - 1")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    if out is None or out.shape != Q.shape or out.dtype != Q.dtype:
        raise ValueError("out must be given and match Q in shape and dtype")
    _need_gpu(indptr, indices, Q, K, V, out)
    H, D = Q.shape[1], Q.shape[2]
    _check(lib().gt_sparse_mha_fwd_noalloc(_ptr(indptr), _ptr(indices), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), N, E, H,
                                           D, _dtype_code(Q), _stream(stream)), "gt_sparse_mha_fwd_noalloc")
    return out


def _qkv(indptr, indices, Q, K, V):
    N, E = _csr(indptr, indices)
    if Q.dim() != 3 or Q.shape[0] != N or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must all be [N][H][D] with N = len(indptr) - 1")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    return N, E, Q.shape[1], Q.shape[2]


def _like(t, Q, name):
    if t is None:
        return torch.empty_like(Q)
    if t.shape != Q.shape or t.dtype != Q.dtype:
        raise ValueError("%s must match Q in shape and dtype" % name)
    return t


def gt_sparse_mha_fwd_lse(indptr, indices, Q, K, V, out=None, lse=None, stream=None):
    """(out, lse): the fused forward and the log-sum-exp [N][H] (float32) the backward takes."""
    N, E, H, D = _qkv(indptr, indices, Q, K, V)
    out = _like(out, Q, "out")
    if lse is None:
        lse = torch.empty((N, H), dtype=torch.float32, device=Q.device)
    elif lse.shape != (N, H) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [N][H]")
    _need_gpu(indptr, indices, Q, K, V, out, lse)
    _check(lib().gt_sparse_mha_fwd_lse(_ptr(indptr), _ptr(indices), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse),
                                       N, E, H, D, _dtype_code(Q), _stream(stream)), "gt_sparse_mha_fwd_lse")
    return out, lse


def gt_sparse_mha_bwd(indptr, indices, t_indptr, t_indices, Q, K, V, out, dout, lse, dQ=None, dK=None, dV=None,
                      stream=None):
    """(dQ, dK, dV).  (t_indptr, t_indices) is the graph sorted by source, indices holding destinations."""
    N, E, H, D = _qkv(indptr, indices, Q, K, V)
    tN, tE = _csr(t_indptr, t_indices)
    if (tN, tE) != (N, E):
        raise ValueError("the transposed graph must have the same N and E")
    for t, name in ((out, "out"), (dout, "dout")):
        _like(t, Q, name)
    if lse.shape != (N, H) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [N][H]")
    dQ, dK, dV = _like(dQ, Q, "dQ"), _like(dK, Q, "dK"), _like(dV, Q, "dV")
    _need_gpu(indptr, indices, t_indptr, t_indices, Q, K, V, out, dout, lse, dQ, dK, dV)
    _check(lib().gt_sparse_mha_bwd(_ptr(indptr), _ptr(indices), _ptr(t_indptr), _ptr(t_indices), _ptr(Q), _ptr(K),
                                   _ptr(V), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dQ), _ptr(dK), _ptr(dV), N, E, H,
                                   D, _dtype_code(Q), _stream(stream)), "gt_sparse_mha_bwd")
    return dQ, dK, dV


def _opts(E, H, device, bias, edge_weight, dropout_p, dropout_seed):
    """(LogitOpts or None, tensors to keep alive)."""
    if bias is None and edge_weight is None and not dropout_p:
        return None, ()
    if bias is not None and (bias.shape != (E, H) or bias.dtype != torch.float32):
        raise ValueError("bias must be float32 [E][H]")
    if edge_weight is not None and (edge_weight.shape != (E,) or edge_weight.dtype != torch.float32):
        raise ValueError("edge_weight must be float32 [E]")
    _need_gpu(bias, edge_weight)
    o = LogitOpts(None if bias is None else bias.data_ptr(), None if edge_weight is None else edge_weight.data_ptr(),
                  float(dropout_p), int(dropout_seed))
    return o, (bias, edge_weight)


def _optref(o):
    return None if o is None else ctypes.byref(o)


def gt_sparse_mha_fwd_ex(indptr, indices, Q, K, V, out=None, lse=None, want_lse=False, bias=None, edge_weight=None,
                         dropout_p=0.0, dropout_seed=0, stream=None):
    """out (and lse when want_lse or lse is given) with the logit variants and dropout."""
    N, E, H, D = _qkv(indptr, indices, Q, K, V)
    out = _like(out, Q, "out")
    if lse is None and want_lse:
        lse = torch.empty((N, H), dtype=torch.float32, device=Q.device)
    if lse is not None and (lse.shape != (N, H) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [N][H]")
    o, _keep = _opts(E, H, Q.device, bias, edge_weight, dropout_p, dropout_seed)
    _need_gpu(indptr, indices, Q, K, V, out, lse)
    _check(lib().gt_sparse_mha_fwd_ex(_ptr(indptr), _ptr(indices), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse),
                                      N, E, H, D, _dtype_code(Q), _optref(o), _stream(stream)),
           "gt_sparse_mha_fwd_ex")
    return (out, lse) if lse is not None else out


def gt_sparse_mha_bwd_ex(indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse, bias=None,
                         edge_weight=None, dropout_p=0.0, dropout_seed=0, want_dbias=False, want_dweight=False,
                         stream=None):
    """(dQ, dK, dV, dbias or None, dweight or None)."""
    N, E, H, D = _qkv(indptr, indices, Q, K, V)
    tN, tE = _csr(t_indptr, t_indices)
    if (tN, tE) != (N, E):
        raise ValueError("the transposed graph must have the same N and E")
    if t_perm is not None and (t_perm.shape != (E,) or t_perm.dtype != torch.int32):
        raise ValueError("t_perm must be int32 [E]")
    for t, name in ((out, "out"), (dout, "dout")):
        _like(t, Q, name)
    if lse.shape != (N, H) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [N][H]")
    dQ, dK, dV = (torch.empty_like(Q) for _ in range(3))
    dbias = torch.empty((E, H), dtype=torch.float32, device=Q.device) if want_dbias else None
    dweight = torch.empty(E, dtype=torch.float32, device=Q.device) if want_dweight else None
    o, _keep = _opts(E, H, Q.device, bias, edge_weight, dropout_p, dropout_seed)
    _need_gpu(indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse)
    _check(lib().gt_sparse_mha_bwd_ex(_ptr(indptr), _ptr(indices), _ptr(t_indptr), _ptr(t_indices), _ptr(t_perm),
                                      _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dQ), _ptr(dK),
                                      _ptr(dV), _ptr(dbias), _ptr(dweight), N, E, H, D, _dtype_code(Q), _optref(o),
                                      _stream(stream)), "gt_sparse_mha_bwd_ex")
    return dQ, dK, dV, dbias, dweight


def _layout_code(layout):
    codes = {"nhd": GT_LAYOUT_NHD, "ndh": GT_LAYOUT_NDH}
    if layout not in codes:
        raise ValueError("layout must be 'nhd' ([N][H][D]) or 'ndh' ([N][D][H])")
    return codes[layout]


def _heads_dims(Q, layout):
    return (Q.shape[1], Q.shape[2]) if layout == "nhd" else (Q.shape[2], Q.shape[1])


def gt_sparse_mha_fwd_layout(indptr, indices, Q, K, V, layout="ndh", out=None, lse=None, want_lse=False, bias=None,
                             edge_weight=None, dropout_p=0.0, dropout_seed=0, stream=None):
    """gt_sparse_mha_fwd_ex with features [N][D][H] (layout 'ndh') or [N][H][D] ('nhd')."""
    code = _layout_code(layout)
    N, E = _csr(indptr, indices)
    if Q.dim() != 3 or Q.shape[0] != N or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must all be [N][.][.] with N = len(indptr) - 1")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    H, D = _heads_dims(Q, layout)
    out = _like(out, Q, "out")
    if lse is None and want_lse:
        lse = torch.empty((N, H), dtype=torch.float32, device=Q.device)
    if lse is not None and (lse.shape != (N, H) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [N][H]")
    o, _keep = _opts(E, H, Q.device, bias, edge_weight, dropout_p, dropout_seed)
    _need_gpu(indptr, indices, Q, K, V, out, lse)
    _check(lib().gt_sparse_mha_fwd_layout(_ptr(indptr), _ptr(indices), _ptr(Q), _ptr(K), _ptr(V), _ptr(out),
                                          _ptr(lse), N, E, H, D, _dtype_code(Q), code, _optref(o), _stream(stream)),
           "gt_sparse_mha_fwd_layout")
    return (out, lse) if lse is not None else out


def gt_sparse_mha_bwd_layout(indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse, layout="ndh",
                             bias=None, edge_weight=None, dropout_p=0.0, dropout_seed=0, want_dbias=False,
                             want_dweight=False, stream=None):
    """gt_sparse_mha_bwd_ex with features in the given layout: (dQ, dK, dV, dbias or None, dweight or None)."""
    code = _layout_code(layout)
    N, E = _csr(indptr, indices)
    if Q.dim() != 3 or Q.shape[0] != N or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must all be [N][.][.] with N = len(indptr) - 1")
    H, D = _heads_dims(Q, layout)
    for t, name in ((out, "out"), (dout, "dout")):
        _like(t, Q, name)
    if lse.shape != (N, H) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [N][H]")
    dQ, dK, dV = (torch.empty_like(Q) for _ in range(3))
    dbias = torch.empty((E, H), dtype=torch.float32, device=Q.device) if want_dbias else None
    dweight = torch.empty(E, dtype=torch.float32, device=Q.device) if want_dweight else None
    o, _keep = _opts(E, H, Q.device, bias, edge_weight, dropout_p, dropout_seed)
    _need_gpu(indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse)
    _check(lib().gt_sparse_mha_bwd_layout(_ptr(indptr), _ptr(indices), _ptr(t_indptr), _ptr(t_indices),
                                          _ptr(t_perm), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(dout), _ptr(lse),
                                          _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dbias), _ptr(dweight), N, E, H, D,
                                          _dtype_code(Q), code, _optref(o), _stream(stream)),
           "gt_sparse_mha_bwd_layout")
    return dQ, dK, dV, dbias, dweight


def gt_sddmm(indptr, indices, Q, K, scores=None, stream=None):
    N, E = _csr(indptr, indices)
    if Q.dim() != 3 or Q.shape[0] != N or K.shape != Q.shape or Q.dtype != K.dtype:
        raise ValueError("Q and K must both be [N][H][D] of one dtype")
    H, D = Q.shape[1], Q.shape[2]
    if scores is None:
        scores = torch.empty((E, H), dtype=torch.float32, device=Q.device)
    elif scores.shape != (E, H) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [E][H]")
    _need_gpu(indptr, indices, Q, K, scores)
    _check(lib().gt_sddmm(_ptr(indptr), _ptr(indices), _ptr(Q), _ptr(K), _ptr(scores), N, E, H, D, _dtype_code(Q),
                          _stream(stream)), "gt_sddmm")
    return scores


def gt_edge_softmax(indptr, scores, alpha=None, stream=None):
    if indptr.dtype != torch.int64:
        raise TypeError("indptr must be int64")
    N = indptr.numel() - 1
    if scores.dim() != 2 or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [E][H]")
    E, H = scores.shape
    if alpha is None:
        alpha = torch.empty_like(scores)
    elif alpha.shape != scores.shape or alpha.dtype != torch.float32:
        raise ValueError("alpha must be float32 [E][H]")
    _need_gpu(indptr, scores, alpha)
    _check(lib().gt_edge_softmax(_ptr(indptr), _ptr(scores), _ptr(alpha), N, E, H, _stream(stream)),
           "gt_edge_softmax")
    return alpha


def gt_spmm(indptr, indices, alpha, V, out=None, stream=None):
    N, E = _csr(indptr, indices)
    if V.dim() != 3 or V.shape[0] != N:
        raise ValueError("V must be [N][H][D] with N = len(indptr) - 1")
    H, D = V.shape[1], V.shape[2]
    if alpha.shape != (E, H) or alpha.dtype != torch.float32:
        raise ValueError("alpha must be float32 [E][H]")
    if out is None:
        out = torch.empty_like(V)
    elif out.shape != V.shape or out.dtype != V.dtype:
        raise ValueError("out must match V in shape and dtype")
    _need_gpu(indptr, indices, alpha, V, out)
    _check(lib().gt_spmm(_ptr(indptr), _ptr(indices), _ptr(alpha), _ptr(V), _ptr(out), N, E, H, D, _dtype_code(V),
                         _stream(stream)), "gt_spmm")
    return out


def gt_calib_gather(indices, K, V, checksum=None, stream=None):
    """Reads the K and V row of every edge's source as the fused kernel does and
    nothing more (a measurement aid).  K and V are [n_rows][...] with rows of
    512, 1024 or 2048 bytes; returns the int32 device tensor [1] holding the
    XOR of all words read (XORed into `checksum` when one is given)."""
    if indices.dtype != torch.int32 or indices.dim() != 1:
        raise TypeError("indices must be a 1-D int32 tensor")
    if K.shape != V.shape or K.dtype != V.dtype or not K.is_contiguous() or not V.is_contiguous():
        raise ValueError("K and V must be contiguous tensors of one shape and dtype")
    n_rows = K.shape[0]
    row_bytes = K.numel() * K.element_size() // max(n_rows, 1)
    if checksum is None:
        checksum = torch.zeros(1, dtype=torch.int32, device=K.device)
    _need_gpu(indices, K, V, checksum)
    _check(lib().gt_calib_gather(_ptr(indices), indices.numel(), _ptr(K), _ptr(V), n_rows, row_bytes,
                                 _ptr(checksum), _stream(stream)), "gt_calib_gather")
    return checksum


def gt_validate_csr(indptr, indices, N=None, stream=None):
    """True for a valid destination-sorted CSR; False (with the reason in gt_last_error) otherwise."""
    n, E = _csr(indptr, indices)
    N = n if N is None else N
    _need_gpu(indptr, indices)
    rc = lib().gt_validate_csr(_ptr(indptr), _ptr(indices), N, E, _stream(stream))
    if rc == GT_EINVAL:
        return False
    _check(rc, "gt_validate_csr")
    return True


def _coo(src, dst):
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.shape != dst.shape or src.dim() != 1:
        raise TypeError("src and dst must be int32 vectors of one length")
    return src.numel()


def gt_coo_to_csr(src, dst, n_dst, n_src=None, want_perm=False, stream=None):
    """(indptr int64[n_dst+1], indices int32[E][, perm int32[E]]), grouped by destination on the GPU."""
    E = _coo(src, dst)
    n_src = n_dst if n_src is None else n_src
    indptr = torch.empty(n_dst + 1, dtype=torch.int64, device=src.device)
    indices = torch.empty(E, dtype=torch.int32, device=src.device)
    perm = torch.empty(E, dtype=torch.int32, device=src.device) if want_perm else None
    _need_gpu(src, dst, indptr, indices, perm)
    _check(lib().gt_coo_to_csr(_ptr(src), _ptr(dst), n_dst, n_src, E, _ptr(indptr), _ptr(indices), _ptr(perm),
                               _stream(stream)), "gt_coo_to_csr")
    return (indptr, indices, perm) if want_perm else (indptr, indices)


# Plans collected by the garbage collector while a stream capture was under
# way: gt_plan_destroy enqueues the plan's release on the null stream, which a
# capture must not see, so they are destroyed at the next plan call instead.
_deferred = []


def _destroy_deferred():
    if _deferred and not torch.cuda.is_current_stream_capturing():
        while _deferred:
            lib().gt_plan_destroy(_deferred.pop())


class GtPlan:
    """Owner of a gt_plan handle; destroy() (or garbage collection) frees it.
    The release is stream-ordered: it waits on the device, not on the host,
    for the work already enqueued on the plan."""

    def __init__(self, handle):
        self.handle = handle
        self.info = None  # the plan's sizes, read once (a plan never changes)

    def destroy(self):
        if self.handle:
            if torch.cuda.is_current_stream_capturing():
                _deferred.append(self.handle)
            else:
                _destroy_deferred()
                lib().gt_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def gt_plan_create(indptr, indices, n_src=None, transpose=True, stream=None):
    _destroy_deferred()
    n_dst, E = _csr(indptr, indices)
    n_src = n_dst if n_src is None else n_src
    _need_gpu(indptr, indices)
    h = _p()
    _check(lib().gt_plan_create(_ptr(indptr), _ptr(indices), n_dst, n_src, E,
                                GT_PLAN_TRANSPOSE if transpose else 0, _stream(stream), ctypes.byref(h)),
           "gt_plan_create")
    return GtPlan(h.value)


def gt_plan_create_coo(src, dst, n_dst, n_src=None, transpose=True, stream=None):
    _destroy_deferred()
    E = _coo(src, dst)
    n_src = n_dst if n_src is None else n_src
    _need_gpu(src, dst)
    h = _p()
    _check(lib().gt_plan_create_coo(_ptr(src), _ptr(dst), n_dst, n_src, E, GT_PLAN_TRANSPOSE if transpose else 0,
                                    _stream(stream), ctypes.byref(h)), "gt_plan_create_coo")
    return GtPlan(h.value)


def gt_plan_destroy(plan):
    plan.destroy()


def gt_plan_info(plan):
    """dict(n_dst, n_src, E, transpose): the plan's sizes."""
    if plan.info is None:
        n = [_i64() for _ in range(3)]
        tptr = _p()
        _check(lib().gt_plan_info(plan.handle, *[ctypes.byref(x) for x in n], None, None, ctypes.byref(tptr), None,
                                  None), "gt_plan_info")
        plan.info = dict(n_dst=n[0].value, n_src=n[1].value, E=n[2].value, transpose=bool(tptr.value))
    return dict(plan.info)


def gt_plan_copy_graph(plan, device=None, stream=None):
    """The plan's (indptr, indices, t_indptr, t_indices, t_perm) as new device tensors
    (t_* None without a transpose)."""
    info = gt_plan_info(plan)
    device = device or torch.device("cuda", torch.cuda.current_device())
    ip = torch.empty(info["n_dst"] + 1, dtype=torch.int64, device=device)
    ix = torch.empty(info["E"], dtype=torch.int32, device=device)
    tip = torch.empty(info["n_src"] + 1, dtype=torch.int64, device=device) if info["transpose"] else None
    tix = torch.empty(info["E"], dtype=torch.int32, device=device) if info["transpose"] else None
    tpm = torch.empty(info["E"], dtype=torch.int32, device=device) if info["transpose"] else None
    some = info["E"] > 0
    _check(lib().gt_plan_copy_graph(plan.handle, _ptr(ip), _ptr(ix) if some else None, _ptr(tip),
                                    _ptr(tix) if (tix is not None and some) else None,
                                    _ptr(tpm) if (tpm is not None and some) else None, _stream(stream)),
           "gt_plan_copy_graph")
    return ip, ix, tip, tix, tpm


def gt_sparse_mha_fwd_plan(plan, Q, K, V, out=None, lse=None, want_lse=False, bias=None, edge_weight=None,
                           dropout_p=0.0, dropout_seed=0, stream=None):
    """out (and lse when want_lse or lse is given) for the plan's graph; Q/out have n_dst rows, K/V n_src."""
    info = gt_plan_info(plan)
    if Q.dim() != 3 or Q.shape[0] != info["n_dst"] or K.shape != V.shape or K.shape[0] != info["n_src"] or \
            K.shape[1:] != Q.shape[1:]:
        raise ValueError("Q must be [n_dst][H][D], K and V [n_src][H][D]")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    H, D = Q.shape[1], Q.shape[2]
    out = _like(out, Q, "out")
    if lse is None and want_lse:
        lse = torch.empty((info["n_dst"], H), dtype=torch.float32, device=Q.device)
    if lse is not None and (lse.shape != (info["n_dst"], H) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [n_dst][H]")
    o, _keep = _opts(info["E"], H, Q.device, bias, edge_weight, dropout_p, dropout_seed)
    _need_gpu(Q, K, V, out, lse)
    _check(lib().gt_sparse_mha_fwd_plan(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse), H, D,
                                        _dtype_code(Q), _optref(o), _stream(stream)), "gt_sparse_mha_fwd_plan")
    return (out, lse) if lse is not None else out


def gt_sparse_mha_bwd_plan(plan, Q, K, V, out, dout, lse, dQ=None, dK=None, dV=None, bias=None, edge_weight=None,
                           dropout_p=0.0, dropout_seed=0, want_dbias=False, want_dweight=False, stream=None):
    """(dQ, dK, dV) for the plan's graph (built with a transpose); with want_dbias or
    want_dweight also (dbias or None, dweight or None)."""
    info = gt_plan_info(plan)
    if Q.dim() != 3 or Q.shape[0] != info["n_dst"] or K.shape != V.shape or K.shape[0] != info["n_src"] or \
            K.shape[1:] != Q.shape[1:]:
        raise ValueError("Q must be [n_dst][H][D], K and V [n_src][H][D]")
    H, D = Q.shape[1], Q.shape[2]
    for t, name in ((out, "out"), (dout, "dout")):
        _like(t, Q, name)
    if lse.shape != (info["n_dst"], H) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [n_dst][H]")
    dQ, dK, dV = _like(dQ, Q, "dQ"), _like(dK, K, "dK"), _like(dV, K, "dV")
    E = info["E"]
    dbias = torch.empty((E, H), dtype=torch.float32, device=Q.device) if want_dbias else None
    dweight = torch.empty(E, dtype=torch.float32, device=Q.device) if want_dweight else None
    o, _keep = _opts(E, H, Q.device, bias, edge_weight, dropout_p, dropout_seed)
    _need_gpu(Q, K, V, out, dout, lse, dQ, dK, dV)
    _check(lib().gt_sparse_mha_bwd_plan(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(dout), _ptr(lse),
                                        _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dbias), _ptr(dweight), H, D,
                                        _dtype_code(Q), _optref(o), _stream(stream)), "gt_sparse_mha_bwd_plan")
    if want_dbias or want_dweight:
        return dQ, dK, dV, dbias, dweight
    return dQ, dK, dV


def gt_config_set(key, value):
    _check(lib().gt_config_set(key, value), "gt_config_set")


def gt_config_get(key):
    return lib().gt_config_get(key)


def gt_config_chunk_edges(E, softmax=False):
    """The split threshold a call on a graph of E edges uses (that of
    gt_edge_softmax if softmax)."""
    return lib().gt_config_chunk_edges(E, 1 if softmax else 0)


def gt_scratch_release(stream=None):
    """Waits for `stream` (default: torch's current stream), then frees the
    library's scratch buffer for it on the current device."""
    _check(lib().gt_scratch_release(_stream(stream)), "gt_scratch_release")


def gt_scratch_bytes(stream=None):
    """Size of the library's scratch buffer for `stream` (0 if none)."""
    n = lib().gt_scratch_bytes(_stream(stream))
    if n < 0:
        raise GtError(GT_EHIP, "gt_scratch_bytes")
    return n


def gt_profile_begin(capacity):
    _check(lib().gt_profile_begin(capacity), "gt_profile_begin")


def gt_profile_end():
    """(summed attention-kernel ms, summed whole-call ms, calls recorded)."""
    k, c, n = ctypes.c_double(), ctypes.c_double(), _i64()
    _check(lib().gt_profile_end(ctypes.byref(k), ctypes.byref(c), ctypes.byref(n)), "gt_profile_end")
    return k.value, c.value, n.value


def gt_last_error():
    return lib().gt_last_error().decode()


def gt_status_string(status):
    return lib().gt_status_string(status).decode()
