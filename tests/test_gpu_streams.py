"""Calls on several HIP streams at once, through the C ABI.

The library keeps one scratch area per (device, stream), so calls enqueued on
different streams may run concurrently.  The kernels are deterministic, so
every result must equal the same call's on the default stream bit for bit:
forward with lse and backward (split rows included), two graphs of different
shapes and dtypes in flight together, and a plan built on one stream and used
on another after a stream wait; and the release of a stream's scratch.
"""
import pytest
import torch

import gtgen
import sparse_graph_attention_amd as gt
from tests.test_gpu_backward import to_torch, with_grad
from tests.test_gpu_parity import chunk_edges, dev, random_graph, say, to_dev

pytestmark = pytest.mark.gpu


def inputs(seed, N, E, H, D, dtype):
    w = with_grad(random_graph(seed, N, E, H, D, dtype))
    t = to_dev(w)
    t["dO"] = to_torch(w["dO"])
    t["tip"] = torch.from_numpy(w["t_indptr"]).to(dev())
    t["tix"] = torch.from_numpy(w["t_indices"]).to(dev())
    return w, t


def run(t):
    out, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    dq, dk, dv = gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], t["tip"], t["tix"], t["Q"], t["K"], t["V"], out,
                                      t["dO"], lse)
    return out, lse, dq, dk, dv


def test_two_streams_match_the_default_stream():
    cases = [inputs(11, 20000, 400000, 8, 64, gtgen.F32), inputs(12, 30000, 300000, 8, 32, gtgen.BF16)]
    with chunk_edges(64):  # rows above 64 edges are split: partials and merges in each stream's scratch
        say("streams: reference calls on the default stream")
        ref = [run(t) for _, t in cases]
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        res = []
        say("streams: 3 rounds on two streams")
        for _ in range(3):
            for (_, t), s in zip(cases, streams):
                with torch.cuda.stream(s):
                    res.append(run(t))
        torch.cuda.synchronize()
    for r, got in enumerate(res):
        for a, b in zip(got, ref[r % 2]):
            assert torch.equal(a, b), "stream result %d differs from the default stream's" % r


def test_plan_built_on_one_stream_used_on_another():
    w, t = inputs(13, 20000, 400000, 8, 64, gtgen.F32)
    with chunk_edges(64):
        ref_out, ref_lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        say("streams: plan on s1, forward on s2")
        with torch.cuda.stream(s1):
            plan = gt.gt_plan_create(t["indptr"], t["indices"], stream=s1)
        s2.wait_stream(s1)
        with torch.cuda.stream(s2):
            out, lse = gt.gt_sparse_mha_fwd_plan(plan, t["Q"], t["K"], t["V"], want_lse=True, stream=s2)
        torch.cuda.synchronize()
        gt.gt_plan_destroy(plan)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_scratch_release_and_reuse():
    """gt_scratch_release frees a stream's buffer; the next call allocates a
    new one and gives the same results bit for bit."""
    _, t = inputs(14, 20000, 400000, 8, 64, gtgen.F32)
    s = torch.cuda.Stream()
    with chunk_edges(64), torch.cuda.stream(s):
        say("streams: scratch release")
        ref = run(t)
        assert gt.gt_scratch_bytes(s) > 0
        gt.gt_scratch_release(s)
        assert gt.gt_scratch_bytes(s) == 0
        gt.gt_scratch_release(s)  # nothing left to free: still OK
        got = run(t)
        assert gt.gt_scratch_bytes(s) > 0
        gt.gt_scratch_release(s)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b), "result after a scratch release differs"
