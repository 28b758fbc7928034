"""The library's calls captured into a HIP graph (torch.cuda.graph) and replayed.

A caller that launches many small calls (a batch of molecules per training
step) can capture them once and replay the graph.  The forward with lse and
the backward (each with its plan kernels, split-row partials and merges), and
the allocation-free forward, make no host synchronisation, no memset and no
allocation once the capturing stream's scratch is sized, which a warm-up call
on that stream does before the capture.  Each graph is replayed several
times, with new inputs written by ordinary kernels and the program's own
synchronisations in between, and every replay is compared bit for bit with
the same calls made eagerly: results do not depend on the order in which the
plan lists split rows, so the two must agree exactly.
"""
import numpy as np
import pytest
import torch

import gtgen
import sparse_graph_attention_amd as gt
from tests.test_gpu_backward import to_torch, with_grad
from tests.test_gpu_parity import custom, dev, say, to_dev

pytestmark = pytest.mark.gpu


def hub_graph(seed, N, E, hubs, H, D, dtype):
    src, dst = gtgen.random_coo(seed, N, E)
    rng = np.random.default_rng(seed)
    dst = np.where(rng.random(E) < 0.3, rng.choice(hubs, E), dst)  # 30% of edges into a few split rows
    return with_grad(custom(N, src, dst.astype(np.int32), H, D, dtype, seed=seed))


def new_inputs(w, r):
    """Features and output gradient of replay r, as device tensors."""
    Q, K, V = gtgen.make_features(w["N"], w["H"], w["D"], w["dtype"], 100 + r, 1.0)
    g = gtgen.make_grad(w["N"], w["H"], w["D"], w["dtype"], seed=200 + r)
    return [to_torch(x) for x in (Q, K, V, g)]


# (seed, nodes, edges, hub rows, H, D, dtype): a graph of one plan block, one
# of several blocks (rows by degree bin), and the molecule shape's word layout
CASES = [(1, 3000, 40000, [0, 2999], 8, 64, gtgen.F32), (2, 20000, 300000, [5, 77, 19999], 8, 32, gtgen.BF16),
         (3, 4000, 9000, [7], 8, 10, gtgen.F32)]


@pytest.mark.parametrize("case", CASES, ids=["one-block", "binned", "word"])
def test_captured_forward_and_backward_replay_bit_for_bit(case):
    w = hub_graph(*case)
    t = to_dev(w)
    d = dev()
    tip, tix = (torch.from_numpy(x).to(d) for x in (w["t_indptr"], w["t_indices"]))
    Q, K, V, dO = (torch.empty_like(t["Q"]) for _ in range(4))
    out, dQ, dK, dV = (torch.empty_like(t["Q"]) for _ in range(4))
    lse = torch.empty((w["N"], w["H"]), dtype=torch.float32, device=d)

    def calls():
        gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], Q, K, V, out=out, lse=lse)
        gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, Q, K, V, out, dO, lse, dQ, dK, dV)

    for x, y in zip((Q, K, V, dO), new_inputs(w, 0)):
        x.copy_(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("capture N=%d E=%d H=%d D=%d dtype=%d" % (w["N"], w["E"], w["H"], w["D"], w["dtype"]))
    with torch.cuda.stream(s):
        calls()  # sizes the capturing stream's scratch: nothing is allocated during the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    for r in range(1, 4):
        for x, y in zip((Q, K, V, dO), new_inputs(w, r)):
            x.copy_(y)
        torch.cuda.synchronize()
        say("replay %d" % r)
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (out, lse, dQ, dK, dV)]
        calls()  # eagerly, on the current stream
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dQ", "dK", "dV"), got, (out, lse, dQ, dK, dV)):
            assert torch.equal(a, b), "replay %d: %s differs from the eager call" % (r, name)
    del g
    torch.cuda.synchronize()


def test_captured_noalloc_forward_replays_bit_for_bit():
    w = hub_graph(4, 20000, 300000, [1, 2, 3], 8, 64, gtgen.F32)
    t = to_dev(w)
    Q, K, V = (torch.empty_like(t["Q"]) for _ in range(3))
    out = torch.empty_like(t["Q"])

    def call():
        gt.gt_sparse_mha_fwd_noalloc(t["indptr"], t["indices"], Q, K, V, out)

    for x, y in zip((Q, K, V), new_inputs(w, 0)[:3]):
        x.copy_(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("capture noalloc N=%d E=%d" % (w["N"], w["E"]))
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(1, 4):
        for x, y in zip((Q, K, V), new_inputs(w, r)[:3]):
            x.copy_(y)
        torch.cuda.synchronize()
        say("replay noalloc %d" % r)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], Q, K, V)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "replay %d differs from gt_sparse_mha_fwd" % r
    del g
    torch.cuda.synchronize()
