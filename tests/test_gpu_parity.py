"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Tolerances, elementwise |gpu - oracle| <= atol + rtol * |oracle|:
* fp32 inputs: rtol 1e-5, atol 1e-6;
* bf16 inputs (fp32 accumulation, bf16 output): rtol 2e-2, atol 1e-5
  (the bf16 output rounding alone is up to 2^-8 relative);
* scores and alpha from the unfused stages use the fp32 bounds.
Small workloads are compared in full; the million-node workloads on sampled
destination rows (every split row, rows at the chunk threshold, empty rows
and a random sample), which the oracle computes one by one; each such test
prints how many split rows it checked against the graph's count.
"""
import math
import sys

import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests import bounds
from tests.bounds import sub_graph

pytestmark = pytest.mark.gpu

F32_TOL = (1e-5, 1e-6)
BF16_TOL = (2e-2, 1e-5)


def say(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(w):
    d = dev()
    t = dict(indptr=torch.from_numpy(w["indptr"]).to(d), indices=torch.from_numpy(w["indices"]).to(d))
    for k in ("Q", "K", "V"):
        x = w[k]
        if x.dtype == np.uint16:
            t[k] = torch.from_numpy(x.view(np.int16)).to(d).view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(x).to(d)
    return t


def host(x):
    x = x.detach()
    if x.dtype == torch.bfloat16:
        x = x.float()
    return x.cpu().numpy().astype(np.float64)


def assert_close(g, o, tol, what):
    rtol, atol = tol
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.all(np.isfinite(g)), what + ": non-finite GPU output"
    excess = np.abs(g - o) - (atol + rtol * np.abs(o))
    bad = int((excess > 0).sum())
    assert bad == 0, "%s: %d elements out of tolerance, worst excess %.3e at %s (gpu %r, oracle %r)" % (
        what, bad, excess.max(), np.unravel_index(excess.argmax(), excess.shape),
        g.flat[excess.argmax()], o.flat[excess.argmax()])


def tol_of(w):
    return F32_TOL if w["dtype"] == gtgen.F32 else BF16_TOL


def oracle_inputs(w):
    return w["indptr"], w["indices"], w["Q"], w["K"], w["V"]


class chunk_edges:
    """Temporarily set the split threshold (edges per chunk)."""

    def __init__(self, c):
        self.c = c

    def __enter__(self):
        self.old = gt.gt_config_get(gt.GT_CFG_CHUNK_EDGES)
        gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, self.c)

    def __exit__(self, *a):
        gt.gt_config_set(gt.GT_CFG_CHUNK_EDGES, self.old)


def custom(N, src, dst, H, D, dtype=gtgen.F32, seed=0, scale=1.0):
    indptr, indices = gtgen.coo_to_csr(N, np.asarray(src, np.int32), np.asarray(dst, np.int32))
    Q, K, V = gtgen.make_features(N, H, D, dtype, seed, scale)
    return dict(name="custom", N=N, E=len(indices), H=H, D=D, dtype=dtype, indptr=indptr, indices=indices,
                Q=Q, K=K, V=V)


def random_graph(seed, N, E, H, D, dtype=gtgen.F32, scale=1.0):
    src, dst = gtgen.random_coo(seed, N, E)
    return custom(N, src, dst, H, D, dtype, seed, scale)


def run_fused(w, t=None):
    t = t or to_dev(w)
    out = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    torch.cuda.synchronize()
    return out


def check_fused_full(w, tol=None):
    say("fused %s N=%d E=%d H=%d D=%d dtype=%d chunk=%d" % (w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"],
                                                            gt.gt_config_chunk_edges(w["E"])))
    out = run_fused(w)
    ref = oracle.fwd(*oracle_inputs(w))
    assert_close(host(out), ref, tol or tol_of(w), "fused " + w["name"])
    return out


# ------------------------------------------------------------------ workloads

_CACHE = {}


def workload(name):
    if name not in _CACHE:
        _CACHE.clear() if name in ("powerlaw", "lognormal") else None
        _CACHE[name] = gtgen.make_workload(name)
    return _CACHE[name]


def sample_rows(indptr, chunk, n_random=1500, seed=0):
    """Rows checked on the million-node workloads: every split row (more than
    `chunk` in-edges), rows at and around the split threshold, rows without
    in-edges, the first and last row, and a uniform random sample."""
    deg = np.diff(indptr)
    N = len(deg)
    rng = np.random.default_rng(seed)
    heavy = np.nonzero(deg > chunk)[0]
    near = np.nonzero(np.isin(deg, [chunk - 1, chunk, chunk + 1, 2 * chunk, 2 * chunk + 1]))[0][:64]
    empty = np.nonzero(deg == 0)[0][:200]
    rand = rng.choice(N, size=min(n_random, N), replace=False)
    rows = np.unique(np.concatenate([heavy, near, empty, rand, [0, N - 1]]))
    return rows.astype(np.int64)


def say_split(indptr, rows, chunk, what):
    """Prints how many split rows the sample holds, against all split rows of the graph."""
    deg = np.diff(indptr)
    n_split = int((deg > chunk).sum())
    in_sample = int((deg[rows] > chunk).sum())
    line = "%s: %d sampled rows, %d of the graph's %d split rows (%d edges in split rows)" % (
        what, len(rows), in_sample, n_split, int(deg[deg > chunk].sum()))
    say(line)
    bounds.REPORT.append(line)
    assert in_sample == n_split, "every split row must be checked"


# ------------------------------------------------------------------ fused, whole outputs

@pytest.mark.parametrize("name", ["tiny_random", "molecules"])
@pytest.mark.parametrize("chunk", [1024, 1, 2, 3, 5])
def test_fused_small_workloads(name, chunk):
    with chunk_edges(chunk):
        check_fused_full(workload(name))


def test_fused_regular16_full():
    check_fused_full(workload("regular16"))


@pytest.mark.parametrize("name", ["powerlaw", "lognormal"])
def test_fused_large_sampled(name):
    w = workload(name)
    say("fused %s sampled rows, N=%d E=%d" % (name, w["N"], w["E"]))
    out = host(run_fused(w))
    chunk = gt.gt_config_chunk_edges(w["E"])
    rows = sample_rows(w["indptr"], chunk)
    say_split(w["indptr"], rows, chunk, "fused " + name)
    ref = oracle.fwd_rows(*oracle_inputs(w), rows)
    assert_close(out[rows], ref, tol_of(w), "fused %s (%d sampled rows)" % (name, len(rows)))
    deg = np.diff(w["indptr"])
    assert np.all(out[deg == 0] == 0.0), "rows without in-edges must be exactly 0"


# ------------------------------------------------------------------ edge cases

def test_zero_edges_zero_fill():
    w = custom(17, [], [], 8, 64)
    t = to_dev(w)
    out = torch.full_like(t["Q"], float("nan"))
    say("fused E=0")
    gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_single_node_self_loop():
    check_fused_full(custom(1, [0], [0], 8, 64))


@pytest.mark.parametrize("chunk", [1024, 100, 7])
def test_one_row_holds_every_edge(chunk):
    N, E = 50, 3000
    src = gtgen.random_coo(3, N, E)[0]
    with chunk_edges(chunk):
        check_fused_full(custom(N, src, np.full(E, 7), 8, 64, seed=3))


@pytest.mark.parametrize("chunk", [16, 64])
def test_degrees_at_threshold(chunk):
    # rows of degree chunk-1, chunk, chunk+1, 2*chunk, 2*chunk+1, 0, 1
    degs = [chunk - 1, chunk, chunk + 1, 2 * chunk, 2 * chunk + 1, 0, 1, 3 * chunk - 1]
    N = 64
    dst = np.concatenate([np.full(d, v) for v, d in enumerate(degs)])
    src = gtgen.random_coo(5, N, len(dst))[0]
    with chunk_edges(chunk):
        for dtype, D in ((gtgen.F32, 64), (gtgen.BF16, 32), (gtgen.F32, 10)):
            check_fused_full(custom(N, src, dst, 8, D, dtype, seed=5))


@pytest.mark.parametrize("H,D", [(1, 1), (3, 5), (2, 7), (1, 64), (4, 33), (8, 100), (2, 256), (16, 64),
                                 (5, 16), (64, 4), (3, 128), (12, 64), (3, 256), (24, 64),
                                 (1, 4), (1, 8), (2, 4), (16, 32), (4, 128), (8, 32), (16, 16), (8, 16), (4, 32),
                                 (2, 64), (8, 64), (8, 128), (4, 256), (4, 64), (2, 128),
                                 (8, 48), (8, 40), (4, 24), (3, 12), (2, 80), (16, 48), (8, 96)])
@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
def test_shapes(H, D, dtype):
    with chunk_edges(40):
        check_fused_full(random_graph(H * 1000 + D, 70, 900, H, D, dtype))


# Heads of whole 8- or 4-byte words but not 16-byte vectors take the word
# layout (every head of an edge in one lane group): one, three, five, seven,
# fifteen and thirty-one words per head, lane groups of 1 to 64 lanes.
WORD_SHAPES = [(8, 10, gtgen.F32), (8, 10, gtgen.BF16), (6, 10, gtgen.F32), (3, 5, gtgen.F32), (1, 1, gtgen.F32),
               (12, 2, gtgen.F32), (7, 6, gtgen.F32), (4, 14, gtgen.F32), (2, 30, gtgen.F32), (1, 62, gtgen.F32),
               (1, 2, gtgen.BF16), (8, 4, gtgen.BF16), (64, 2, gtgen.BF16), (5, 6, gtgen.BF16), (3, 12, gtgen.BF16),
               (4, 30, gtgen.BF16), (2, 62, gtgen.BF16)]


def hub_graph(H, D, dtype, seed):
    # a destination hub of 500 in-edges and a source hub of 400 out-edges
    N, E = 60, 1500
    src, dst = gtgen.random_coo(seed, N, E)
    dst = np.where(np.arange(E) < 500, 5, dst)
    src = np.where((np.arange(E) >= 500) & (np.arange(E) < 900), 9, src)
    return custom(N, src, dst, H, D, dtype, seed=seed)


@pytest.mark.parametrize("H,D,dtype", WORD_SHAPES)
@pytest.mark.parametrize("chunk", [512, 37])
def test_word_layout_shapes(H, D, dtype, chunk):
    with chunk_edges(chunk):
        check_fused_full(hub_graph(H, D, dtype, H * 100 + D))
        check_fused_full(random_graph(H * 1000 + D, 70, 900, H, D, dtype))


@pytest.mark.parametrize("H,D,shift", [(2, 64, 2), (4, 10, 1), (8, 10, 1), (8, 10, 2)])
def test_misaligned_features_take_word_or_scalar_layouts(H, D, shift):
    # fp32 views `shift` elements into larger buffers: 8-byte aligned rows take
    # 8-byte words (2 x 64 loses the vector layout), 4-byte aligned ones 4-byte
    # words where a head's words fit 32 lane slots (4 x 10), else the scalar layout
    w = hub_graph(H, D, gtgen.F32, 7 * shift + D)
    t = to_dev(w)
    n = t["Q"].numel()
    bufs = {k: torch.empty(n + shift, dtype=torch.float32, device=dev()) for k in ("Q", "K", "V", "out")}
    views = {k: bufs[k][shift:].view(t["Q"].shape) for k in bufs}
    for k in ("Q", "K", "V"):
        views[k].copy_(t[k])
    with chunk_edges(37):
        say("fused misaligned by %d elements H=%d D=%d" % (shift, H, D))
        gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], views["Q"], views["K"], views["V"], out=views["out"])
        torch.cuda.synchronize()
    assert_close(host(views["out"]), oracle.fwd(*oracle_inputs(w)), F32_TOL, "misaligned by %d" % shift)


def test_misaligned_features_use_the_scalar_layout():
    w = random_graph(8, 40, 300, 8, 64)
    t = to_dev(w)
    # views 4 bytes into a larger buffer: not 16-byte aligned
    bufs = {k: torch.empty(t["Q"].numel() + 1, dtype=torch.float32, device=dev()) for k in ("Q", "K", "V", "out")}
    views = {k: bufs[k][1:].view(t["Q"].shape) for k in bufs}
    for k in ("Q", "K", "V"):
        views[k].copy_(t[k])
    say("fused misaligned")
    gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], views["Q"], views["K"], views["V"], out=views["out"])
    torch.cuda.synchronize()
    assert_close(host(views["out"]), oracle.fwd(*oracle_inputs(w)), F32_TOL, "misaligned")


def test_large_logits():
    # Q x 1000: logits of order 1e3.  The fp32 dot product then carries an
    # absolute error up to about (D+4) u sum|q k| / sqrt(D) (u = 2^-24); a
    # weight moves by at most 2 alpha max|ds|, the output by 2 max|ds| max|v|.
    w = random_graph(12, 60, 600, 4, 16, scale=1.0)
    w["Q"] = w["Q"] * np.float32(1000.0)
    say("fused large logits")
    out = host(run_fused(w))
    ref = oracle.fwd(*oracle_inputs(w))
    assert np.all(np.isfinite(out))
    u = 2.0 ** -24
    D = w["D"]
    indptr, indices = w["indptr"], w["indices"]
    Q, K, V = (x.astype(np.float64) for x in (w["Q"], w["K"], w["V"]))
    for v in range(w["N"]):
        b, e = indptr[v], indptr[v + 1]
        if e == b:
            assert np.all(out[v] == 0)
            continue
        src = indices[b:e]
        ds = (D + 4) * u * np.abs(Q[v][None] * K[src]).sum(-1) / math.sqrt(D)  # [deg][H]
        bound = 2 * ds.max(0) * np.abs(V[src]).max(axis=(0, 2))  # [H]
        tol = 1e-6 + 1e-5 * np.abs(ref[v]) + bound[:, None]
        assert np.all(np.abs(out[v] - ref[v]) <= tol), v


def test_deterministic():
    w = workload("regular16")
    t = to_dev(w)
    with chunk_edges(3):
        say("determinism")
        a = run_fused(w, t).clone()
        b = run_fused(w, t)
    assert torch.equal(a, b)


def test_validate_csr():
    w = random_graph(2, 30, 100, 1, 4)
    t = to_dev(w)
    say("validate csr")
    assert gt.gt_validate_csr(t["indptr"], t["indices"])
    bad = t["indices"].clone()
    bad[5] = 30
    assert not gt.gt_validate_csr(t["indptr"], bad)
    assert "outside" in gt.gt_last_error()
    ip = t["indptr"].clone()
    ip[3] = int(ip[4]) + 5  # indptr[3] > indptr[4]: decreasing
    assert not gt.gt_validate_csr(ip, t["indices"])
    assert "decreases" in gt.gt_last_error()


# ------------------------------------------------------------------ unfused stages

def unfused_inputs(w, seed=99):
    """Independent fp32 scores and weights for the softmax and SpMM stages.

    The weights are positive and sum to 1 over each destination's in-edges, as
    softmax weights do; the fp32 bounds hold for outputs of that scale (with
    unnormalised weights the rounding error grows with sum |alpha v|)."""
    E, H = w["E"], w["H"]
    scores = gtgen.normal_f32(seed, 7, (E, H), 2.0)
    raw = gtgen.uniform_f64(seed, 8, E * H, 0.0, 1.0).reshape(E, H)
    dst = np.repeat(np.arange(w["N"]), np.diff(w["indptr"]))
    sums = np.zeros((w["N"], H))
    np.add.at(sums, dst, raw)
    alpha = (raw / sums[dst]).astype(np.float32)
    return scores, alpha


def check_stages(w, rows=None):
    t = to_dev(w)
    tol = tol_of(w)
    say("unfused %s N=%d E=%d" % (w["name"], w["N"], w["E"]))
    s = gt.gt_sddmm(t["indptr"], t["indices"], t["Q"], t["K"])
    sc, al = unfused_inputs(w)
    a = gt.gt_edge_softmax(t["indptr"], torch.from_numpy(sc).to(dev()))
    o = gt.gt_spmm(t["indptr"], t["indices"], torch.from_numpy(al).to(dev()), t["V"])
    # composition of the GPU stages
    comp = gt.gt_spmm(t["indptr"], t["indices"], gt.gt_edge_softmax(t["indptr"], s), t["V"])
    torch.cuda.synchronize()
    s, a, o, comp = host(s), host(a), host(o), host(comp)
    indptr, indices = w["indptr"], w["indices"]
    if rows is None:
        assert_close(s, oracle.sddmm(indptr, indices, w["Q"], w["K"]), F32_TOL, "sddmm")
        assert_close(a, oracle.edge_softmax(indptr, sc.astype(np.float64)), F32_TOL, "edge_softmax")
        assert_close(o, oracle.spmm(indptr, indices, al.astype(np.float64), w["V"]), tol, "spmm")
        assert_close(comp, oracle.fwd(*oracle_inputs(w)), tol, "sddmm->softmax->spmm")
    else:
        ref, rs, _ = oracle.fwd_rows(*oracle_inputs(w), rows, want_edges=True)
        # softmax and SpMM of independent inputs on the same rows, as a sub-CSR of those rows
        sub_indptr, _, sel = sub_graph(indptr, indices, rows)
        assert_close(s[sel], rs, F32_TOL, "sddmm (sampled)")
        assert_close(comp[rows], ref, tol, "sddmm->softmax->spmm (sampled)")
        assert_close(a[sel], oracle.edge_softmax(sub_indptr, sc[sel].astype(np.float64)), F32_TOL,
                     "edge_softmax (sampled)")
        ref_o = oracle.spmm(sub_indptr, indices[sel], al[sel].astype(np.float64), w["V"])
        assert_close(o[rows], ref_o, tol, "spmm (sampled)")


@pytest.mark.parametrize("name", ["tiny_random", "molecules", "regular16"])
@pytest.mark.parametrize("chunk", [1024, 2])
def test_unfused_stages(name, chunk):
    with chunk_edges(chunk):
        check_stages(workload(name))


@pytest.mark.parametrize("dtype,D", [(gtgen.F32, 64), (gtgen.BF16, 32), (gtgen.F32, 10), (gtgen.BF16, 10)])
def test_unfused_split_rows(dtype, D):
    N, E = 40, 2500
    src, dst = gtgen.random_coo(21, N, E)
    dst = np.where(np.arange(E) < 1800, 3, dst)  # one hub row
    with chunk_edges(50):
        check_stages(custom(N, src, dst, 6 if D == 10 else 8, D, dtype, seed=21))


@pytest.mark.parametrize("H,D", [(8, 64), (2, 256), (16, 32), (4, 128), (8, 32), (16, 16), (8, 16), (4, 32), (2, 64),
                                 (8, 128), (4, 256), (4, 64), (2, 128), (3, 128), (5, 16),
                                 (8, 48), (8, 40), (4, 24), (3, 12), (2, 80), (16, 48), (8, 96)])
@pytest.mark.parametrize("dtype", [gtgen.F32, gtgen.BF16])
def test_unfused_shapes(H, D, dtype):
    # every compile-time lane layout of the SDDMM and SpMM, and run-time ones
    with chunk_edges(40):
        check_stages(random_graph(H * 500 + D, 70, 900, H, D, dtype))


@pytest.mark.parametrize("H,D,dtype", [(8, 48, gtgen.F32), (8, 96, gtgen.BF16), (6, 64, gtgen.F32), (16, 64, gtgen.F32),
                                       (8, 64, gtgen.F32), (4, 64, gtgen.BF16)])
def test_unfused_split_rows_every_layout(H, D, dtype):
    # a hub row split into chunks: the SpMM's chunk partials are indexed by
    # memory position (padded heads, early-ending and wide rows)
    N, E = 60, 1500
    src, dst = gtgen.random_coo(H * 7 + D, N, E)
    dst = np.where(np.arange(E) < 500, 5, dst)
    with chunk_edges(37):
        check_stages(custom(N, src, dst, H, D, dtype, seed=D))


def test_softmax_in_place_and_odd_heads():
    w = random_graph(31, 50, 700, 3, 8)
    t = to_dev(w)
    sc, _ = unfused_inputs(w)
    ref = oracle.edge_softmax(w["indptr"], sc.astype(np.float64))
    with chunk_edges(9):
        buf = torch.from_numpy(sc).to(dev())
        say("softmax in place H=3")
        gt.gt_edge_softmax(t["indptr"], buf, alpha=buf)
        torch.cuda.synchronize()
    assert_close(host(buf), ref, F32_TOL, "in-place softmax")


@pytest.mark.parametrize("name", ["powerlaw", "lognormal"])
def test_unfused_large_sampled(name):
    w = workload(name)
    # SDDMM and SpMM split rows at one threshold, the softmax at its own
    chunk = gt.gt_config_chunk_edges(w["E"])
    s_chunk = gt.gt_config_chunk_edges(w["E"], softmax=True)
    rows = np.union1d(sample_rows(w["indptr"], chunk, n_random=500), sample_rows(w["indptr"], s_chunk, n_random=0))
    say_split(w["indptr"], rows, chunk, "unfused " + name)
    say_split(w["indptr"], rows, s_chunk, "unfused softmax " + name)
    check_stages(w, rows)


@pytest.mark.parametrize("H", [1, 4, 8, 16, 64])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("chunk", [512, 20])
def test_softmax_row_blocks(H, in_place, chunk):
    # degrees around the lane/wave cut (16), the rows a wave holds in
    # registers (16 scores a lane: 1024/H edges) and the split threshold (512
    # by default; 20 splits rows that the per-lane path could otherwise take,
    # which in place must not be overwritten before their chunks are read)
    degs = [0, 1, 2, 15, 16, 17, 19, 20, 21, 31, 32, 33, 100, 511, 512, 513, 1300, 0, 5, 64, 65, 7, 127, 128, 129,
            255, 256, 257, 1023, 1024, 1025]
    N = len(degs) + 3
    dst = np.concatenate([np.full(d, v) for v, d in enumerate(degs)])
    src = gtgen.random_coo(41, N, len(dst))[0]
    indptr, indices = gtgen.coo_to_csr(N, src, dst)
    E = len(indices)
    sc = gtgen.normal_f32(41, 7, (E, H), 3.0)
    ref = oracle.edge_softmax(indptr, sc.astype(np.float64))
    ip = torch.from_numpy(indptr).to(dev())
    buf = torch.from_numpy(sc).to(dev())
    say("softmax row blocks H=%d in_place=%s chunk=%d" % (H, in_place, chunk))
    with chunk_edges(chunk):
        a = gt.gt_edge_softmax(ip, buf, alpha=buf if in_place else None)
        torch.cuda.synchronize()
    assert_close(host(a), ref, F32_TOL, "edge_softmax H=%d" % H)


@pytest.mark.parametrize("H", [4, 8, 16])
@pytest.mark.parametrize("in_place", [False, True])
def test_softmax_row_lengths(H, in_place):
    # rows of many lengths (powers of two and one past them, up to the split
    # threshold and far past it, where rows are cut into chunks whose
    # statistics are merged), for 4, 8 and 16 heads, and then a graph of more
    # rows than one plan block lists (8,192), so that several blocks add to the
    # split-row lists
    degs = [1, 7, 8, 9, 31, 32, 33, 127, 128, 129, 255, 256, 257, 300, 511, 512, 513, 0, 2, 1000,
            1024, 1025, 2048, 2049, 4096, 4097, 8192, 8193, 20000]
    N = len(degs) + 2
    dst = np.concatenate([np.full(d, v) for v, d in enumerate(degs)])
    src = gtgen.random_coo(43, N, len(dst))[0]
    cases = [gtgen.coo_to_csr(N, src, dst)]
    rng = np.random.default_rng(H)
    deg2 = rng.choice([0, 1, 3, 8, 9, 20, 33, 70, 130, 260, 400, 520], size=20000)
    dst2 = np.repeat(np.arange(20000), deg2).astype(np.int32)
    cases.append(gtgen.coo_to_csr(20000, rng.integers(0, 20000, len(dst2)).astype(np.int32), dst2))
    for indptr, indices in cases:
        E = len(indices)
        sc = gtgen.normal_f32(47, 7, (E, H), 3.0)
        ref = oracle.edge_softmax(indptr, sc.astype(np.float64))
        ip = torch.from_numpy(indptr).to(dev())
        buf = torch.from_numpy(sc).to(dev())
        say("softmax row lengths H=%d N=%d E=%d in_place=%s" % (H, len(indptr) - 1, E, in_place))
        a = gt.gt_edge_softmax(ip, buf, alpha=buf if in_place else None)
        torch.cuda.synchronize()
        assert_close(host(a), ref, F32_TOL, "edge_softmax row lengths H=%d" % H)


def test_softmax_misaligned_scores():
    # scores 4 bytes into a buffer (not 16-byte aligned), a split row included
    degs = [3, 40, 200, 600, 0, 9]
    N = len(degs)
    dst = np.concatenate([np.full(d, v) for v, d in enumerate(degs)])
    indptr, _ = gtgen.coo_to_csr(N, gtgen.random_coo(44, N, len(dst))[0], dst)
    E, H = len(dst), 8
    sc = gtgen.normal_f32(48, 7, (E, H), 3.0)
    big = torch.empty(E * H + 1, dtype=torch.float32, device=dev())
    view = big[1:].view(E, H)
    view.copy_(torch.from_numpy(sc).to(dev()))
    say("softmax misaligned scores")
    a = gt.gt_edge_softmax(torch.from_numpy(indptr).to(dev()), view)
    torch.cuda.synchronize()
    assert_close(host(a), oracle.edge_softmax(indptr, sc.astype(np.float64)), F32_TOL, "misaligned softmax")
