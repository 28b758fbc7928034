"""Calls on several HIP streams at once, through the C ABI.

The library keeps one scratch area per (device, stream), so calls enqueued on
different streams may run concurrently.  The kernels are deterministic, so
every result must equal the same call's on the default stream bit for bit:
forward with lse and backward (split rows included), two graphs of different
shapes and dtypes in flight together, and a plan built on one stream and used
on another after a stream wait; and the release of a stream's scratch.
Memory is stream-ordered: scratch grows and plans are released without the
host waiting, so results must also hold when a buffer grows, or a plan is
destroyed, behind work that is still queued.  The allocation-failure test hook
must leave every output untouched.
"""
import math
import os

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


def test_scratch_grows_behind_queued_work():
    """A small call, a large one (the stream's buffer grows while the small
    call may still run) and a small one again, with no wait in between."""
    small = inputs(15, 2000, 40000, 8, 64, gtgen.F32)[1]
    large = inputs(16, 40000, 800000, 8, 64, gtgen.F32)[1]
    with chunk_edges(64):
        ref_s, ref_l = run(small), run(large)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        say("streams: scratch growth behind queued work")
        with torch.cuda.stream(s):
            gt.gt_scratch_release(s)
            got = [run(small), run(large), run(small)]
            gt.gt_scratch_release(s)
        torch.cuda.synchronize()
    for g, r in zip(got, (ref_s, ref_l, ref_s)):
        for a, b in zip(g, r):
            assert torch.equal(a, b)


def test_plan_destroyed_behind_queued_work():
    """A plan destroyed right after its forward is enqueued (the host does not
    wait), then a second plan built whose memory may come from the first's:
    the forward must still see the first plan intact."""
    _, t = inputs(17, 40000, 800000, 8, 64, gtgen.F32)
    _, t2 = inputs(18, 40000, 800000, 8, 64, gtgen.F32)
    with chunk_edges(64):
        ref = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        say("streams: plan destroyed behind its queued forward")
        for _ in range(3):
            with torch.cuda.stream(s1):
                plan = gt.gt_plan_create(t["indptr"], t["indices"], stream=s1)
                out = gt.gt_sparse_mha_fwd_plan(plan, t["Q"], t["K"], t["V"], stream=s1)
                plan.destroy()
            with torch.cuda.stream(s2):
                plan2 = gt.gt_plan_create(t2["indptr"], t2["indices"], stream=s2)
                gt.gt_sparse_mha_fwd_plan(plan2, t2["Q"], t2["K"], t2["V"], stream=s2)
                plan2.destroy()
            torch.cuda.synchronize()
            assert torch.equal(out, ref)


def test_allocation_failure_hook_enqueues_nothing():
    """With GT_TEST_FAIL_ALLOC set every call that would allocate returns
    GT_ENOMEM and its outputs keep their contents; unset, the same calls work."""
    w, t = inputs(19, 3000, 60000, 8, 64, gtgen.F32)
    out = torch.full_like(t["Q"], math.nan)
    lse = torch.full((w["N"], w["H"]), math.nan, device=dev())
    grads = [torch.full_like(t["Q"], math.nan) for _ in range(3)]
    say("streams: allocation failure hook")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gt.gt_scratch_release(s)  # a fresh stream: the forward would have to allocate
        os.environ["GT_TEST_FAIL_ALLOC"] = "1"
        try:
            for call in (lambda: gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"],
                                                          out=out, lse=lse),
                         lambda: gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], t["tip"], t["tix"], t["Q"], t["K"],
                                                      t["V"], t["Q"], t["dO"], lse.nan_to_num(0.0), *grads),
                         lambda: gt.gt_plan_create(t["indptr"], t["indices"])):
                with pytest.raises(gt.GtError) as ei:
                    call()
                assert ei.value.status == gt.GT_ENOMEM
        finally:
            del os.environ["GT_TEST_FAIL_ALLOC"]
        torch.cuda.synchronize()
        assert torch.isnan(out).all() and torch.isnan(lse).all()
        for g in grads:
            assert torch.isnan(g).all()
        o2, l2 = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        gt.gt_scratch_release(s)
    torch.cuda.synchronize()
    assert torch.isfinite(o2).all() and not torch.isnan(l2).any()
