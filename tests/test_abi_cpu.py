"""The C-ABI library loads, exports what include/gtattn.h declares, and rejects
bad arguments before touching the GPU (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

import sparse_graph_attention_amd as gt

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gtattn.h")

NULL = None
S = None  # null stream; never reached by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gt_[a-z_]+)\s*\(", text)))


def test_header_and_exports_agree():
    names = declared_functions()
    assert set(names) == set(gt.EXPORTS), names
    L = gt.lib()
    for n in names:
        assert hasattr(L, n), n


def test_library_is_the_in_tree_build():
    assert os.path.dirname(gt._build.LIB) == os.path.dirname(os.path.abspath(gt.__file__))
    assert os.path.exists(gt._build.LIB)


def test_status_strings():
    assert gt.gt_status_string(0) == "ok"
    assert "invalid" in gt.gt_status_string(1)
    assert "unsupported" in gt.gt_status_string(2)
    assert gt.gt_status_string(99) == "unknown status"


def fwd(N=4, E=4, H=8, D=64, dtype=0, ptr=1):
    p = ctypes.c_void_p(ptr) if ptr else None
    return gt.lib().gt_sparse_mha_fwd(p, p, p, p, p, p, N, E, H, D, dtype, S)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), gt.GT_EINVAL),
    (dict(E=-1), gt.GT_EINVAL),
    (dict(H=0), gt.GT_EINVAL),
    (dict(D=0), gt.GT_EINVAL),
    (dict(N=1 << 31), gt.GT_EINVAL),
    (dict(ptr=0), gt.GT_EINVAL),
    (dict(dtype=7), gt.GT_EUNSUPPORTED),
    (dict(H=65), gt.GT_EUNSUPPORTED),
    (dict(D=257), gt.GT_EUNSUPPORTED),
])
def test_fused_rejects(kw, status):
    assert fwd(**kw) == status
    assert gt.gt_last_error() != ""


def test_zero_nodes_is_a_noop():
    assert fwd(N=0, E=0, ptr=0) == gt.GT_OK


def test_unfused_reject():
    L = gt.lib()
    p = ctypes.c_void_p(1)
    assert L.gt_sddmm(None, p, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_EINVAL
    assert L.gt_sddmm(p, p, p, p, p, 4, 4, 8, 300, 0, S) == gt.GT_EUNSUPPORTED
    assert L.gt_edge_softmax(p, None, p, 4, 4, 8, S) == gt.GT_EINVAL
    assert L.gt_edge_softmax(p, p, p, 4, 4, 0, S) == gt.GT_EINVAL
    assert L.gt_spmm(p, None, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_EINVAL
    assert L.gt_spmm(p, p, p, p, p, 4, 4, 8, 64, 5, S) == gt.GT_EUNSUPPORTED
    assert L.gt_validate_csr(None, p, 4, 4, S) == gt.GT_EINVAL
    assert L.gt_validate_csr(p, p, -1, 4, S) == gt.GT_EINVAL
    # nothing to do: zero edges for the unfused stages that only touch edges
    assert L.gt_sddmm(p, p, p, p, p, 4, 0, 8, 64, 0, S) == gt.GT_OK
    assert L.gt_edge_softmax(p, p, p, 4, 0, 8, S) == gt.GT_OK


def test_calib_gather_rejects():
    L = gt.lib()
    p = ctypes.c_void_p(16)
    assert L.gt_calib_gather(p, -1, p, p, 4, 2048, p, S) == gt.GT_EINVAL
    assert L.gt_calib_gather(p, 4, p, p, 4, 100, p, S) == gt.GT_EUNSUPPORTED
    assert L.gt_calib_gather(None, 4, p, p, 4, 2048, p, S) == gt.GT_EINVAL
    assert L.gt_calib_gather(p, 4, p, p, 4, 2048, None, S) == gt.GT_EINVAL
    assert L.gt_calib_gather(p, 4, ctypes.c_void_p(8), p, 4, 2048, p, S) == gt.GT_EUNSUPPORTED  # misaligned
    assert L.gt_calib_gather(None, 0, None, None, 0, 512, None, S) == gt.GT_OK


def test_config():
    old = gt.gt_config_get(gt.GT_CFG_CHUNK_EDGES)
    assert old == 0  # automatic
    # automatic: 512 edges below 2^23 edges and in the softmax, 2,048 from there
    assert gt.gt_config_chunk_edges(0) == 512
    assert gt.gt_config_chunk_edges(2 ** 23 - 1) == 512
    assert gt.gt_config_chunk_edges(2 ** 23) == 2048
    assert gt.gt_config_chunk_edges(60_000_000) == 2048
    assert gt.gt_config_chunk_edges(60_000_000, softmax=True) == 512
    assert gt.gt_config_chunk_edges(-1) == -1
    try:
        gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, 7)
        assert gt.gt_config_get(gt.GT_CFG_CHUNK_EDGES) == 7
        assert gt.gt_config_chunk_edges(60_000_000) == 7
        assert gt.gt_config_chunk_edges(100, softmax=True) == 7
        gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, 0)
        assert gt.gt_config_chunk_edges(2 ** 23) == 2048
        with pytest.raises(gt.GtError):
            gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, -1)
        with pytest.raises(gt.GtError):
            gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, 2 ** 30 + 1)
        with pytest.raises(gt.GtError):
            gt.gt_config_set(99, 5)
        assert gt.gt_config_get(99) == -1
    finally:
        gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, old)
    assert gt.lib().gt_profile_begin(0) == gt.GT_EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    indptr = torch.zeros(2, dtype=torch.int64)
    indices = torch.zeros(0, dtype=torch.int32)
    Q = torch.zeros(1, 8, 64)
    with pytest.raises(ValueError):
        gt.gt_sparse_mha_fwd(indptr, indices, Q, Q, Q)


def test_graph_and_plan_reject():
    L = gt.lib()
    p = ctypes.c_void_p(1)
    h = ctypes.c_void_p()
    assert L.gt_coo_to_csr(p, p, -1, 4, 4, p, p, None, S) == gt.GT_EINVAL
    assert L.gt_coo_to_csr(p, p, 4, 4, 1 << 31, p, p, None, S) == gt.GT_EUNSUPPORTED
    assert L.gt_coo_to_csr(p, p, 4, 1 << 31, 4, p, p, None, S) == gt.GT_EINVAL
    assert L.gt_coo_to_csr(None, p, 4, 4, 4, p, p, None, S) == gt.GT_EINVAL
    assert L.gt_coo_to_csr(p, p, 4, 4, 4, None, p, None, S) == gt.GT_EINVAL
    assert L.gt_plan_create(p, p, 4, 4, 4, 0, S, None) == gt.GT_EINVAL
    assert L.gt_plan_create(p, p, -4, 4, 4, 0, S, ctypes.byref(h)) == gt.GT_EINVAL
    assert h.value is None
    assert L.gt_plan_create(p, p, 4, 4, 4, 4, S, ctypes.byref(h)) == gt.GT_EINVAL  # unknown flag
    assert L.gt_plan_create(None, p, 4, 4, 4, 0, S, ctypes.byref(h)) == gt.GT_EINVAL
    assert L.gt_plan_create_coo(None, p, 4, 4, 4, 1, S, ctypes.byref(h)) == gt.GT_EINVAL
    assert L.gt_plan_info(None, None, None, None, None, None, None, None, None) == gt.GT_EINVAL
    assert L.gt_plan_destroy(None) == gt.GT_OK
    assert L.gt_plan_copy_graph(None, p, p, None, None, None, S) == gt.GT_EINVAL
    assert L.gt_sparse_mha_fwd_plan(None, p, p, p, p, None, 8, 64, 0, None, S) == gt.GT_EINVAL
    assert L.gt_sparse_mha_bwd_plan(None, p, p, p, p, p, p, p, p, p, None, None, 8, 64, 0, None, S) == gt.GT_EINVAL


def test_logit_options_reject():
    L = gt.lib()
    p = ctypes.c_void_p(1)
    for bad in (-0.1, 1.0, 2.0, float("nan")):
        o = gt.LogitOpts(None, None, bad, 0)
        assert L.gt_sparse_mha_fwd_ex(p, p, p, p, p, p, None, 4, 4, 8, 64, 0, ctypes.byref(o), S) == gt.GT_EINVAL
    # a bias needs the transpose's CSR positions in the backward
    o = gt.LogitOpts(1, None, 0.0, 0)
    assert L.gt_sparse_mha_bwd_ex(p, p, p, p, None, p, p, p, p, p, p, p, p, p, None, None, 4, 4, 8, 64, 0,
                                  ctypes.byref(o), S) == gt.GT_EINVAL
    assert "t_perm" in gt.gt_last_error()


def test_layout_reject():
    L = gt.lib()
    p = ctypes.c_void_p(1)
    assert L.gt_sparse_mha_fwd_layout(p, p, p, p, p, p, None, 4, 4, 8, 64, 0, 2, None, S) == gt.GT_EINVAL
    assert "layout" in gt.gt_last_error()
    assert L.gt_sparse_mha_fwd_layout(p, p, p, p, p, p, None, -1, 4, 8, 64, 0, 1, None, S) == gt.GT_EINVAL
    assert L.gt_sparse_mha_bwd_layout(p, p, p, p, None, p, p, p, p, p, p, p, p, p, None, None, 4, 4, 8, 64, 0, 5,
                                      None, S) == gt.GT_EINVAL
    assert L.gt_sparse_mha_fwd_layout(p, p, p, p, p, p, None, 0, 0, 8, 64, 0, 1, None, S) == gt.GT_OK


class fail_alloc:
    """Sets the GT_TEST_FAIL_ALLOC test hook for the duration of a block."""

    def __enter__(self):
        self.old = os.environ.get("GT_TEST_FAIL_ALLOC")
        os.environ["GT_TEST_FAIL_ALLOC"] = "1"

    def __exit__(self, *a):
        if self.old is None:
            del os.environ["GT_TEST_FAIL_ALLOC"]
        else:
            os.environ["GT_TEST_FAIL_ALLOC"] = self.old


def test_allocation_failure_hook_returns_enomem_before_any_hip_call():
    # with the hook set, the calls that take scratch or allocate a plan stop
    # at the allocation, which comes before every HIP call (there is no device
    # here: a HIP call would fail with GT_EHIP instead), so nothing is enqueued
    L = gt.lib()
    p = ctypes.c_void_p(256)
    with fail_alloc():
        assert fwd(ptr=256) == gt.GT_ENOMEM
        assert "GT_TEST_FAIL_ALLOC" in gt.gt_last_error()
        assert L.gt_sparse_mha_fwd_lse(p, p, p, p, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_ENOMEM
        assert L.gt_sddmm(p, p, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_ENOMEM
        assert L.gt_edge_softmax(p, p, p, 4, 4, 8, S) == gt.GT_ENOMEM
        assert L.gt_spmm(p, p, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_ENOMEM
        assert L.gt_sparse_mha_bwd(p, p, p, p, p, p, p, p, p, p, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_ENOMEM
        assert L.gt_coo_to_csr(p, p, 4, 4, 4, p, p, None, S) == gt.GT_ENOMEM
        h = ctypes.c_void_p()
        assert L.gt_plan_create(p, p, 4, 4, 4, gt.GT_PLAN_TRANSPOSE, S, ctypes.byref(h)) == gt.GT_ENOMEM
        assert h.value is None
        assert L.gt_plan_create_coo(p, p, 4, 4, 4, 0, S, ctypes.byref(h)) == gt.GT_ENOMEM
        assert "plan allocation refused" in gt.gt_last_error()
        # argument errors still come first
        assert fwd(H=0, ptr=256) == gt.GT_EINVAL
    assert gt.gt_status_string(gt.GT_ENOMEM) == "out of device memory"


def test_noalloc_rejects_what_its_static_scratch_cannot_hold():
    # sizes are checked before any HIP call: far too many edges for the static
    # array even at 64 times the split threshold
    L = gt.lib()
    p = ctypes.c_void_p(256)
    assert L.gt_sparse_mha_fwd_noalloc(p, p, p, p, p, p, 1000, 1 << 40, 8, 64, 0, S) == gt.GT_EUNSUPPORTED
    assert "allocation-free forward" in gt.gt_last_error()
    assert L.gt_sparse_mha_fwd_noalloc(p, None, p, p, p, p, 4, 4, 8, 64, 0, S) == gt.GT_EINVAL
    assert L.gt_sparse_mha_fwd_noalloc(None, None, None, None, None, None, 0, 0, 8, 64, 0, S) == gt.GT_OK
