"""The allocation-free forward, gt_sparse_mha_fwd_noalloc, through the C ABI,
against the allocating gt_sparse_mha_fwd and the oracle.

Its work lists and split-row partials live in one static device array per
GPU, shared by every call, which keeps the last call's contents.  Calls are
made in a row, each on a smaller input than the one before, so a call that
wrongly read what the last one left (its counters, chunk lists or partials)
would show.  While the split threshold needs no raising, out must equal
gt_sparse_mha_fwd's bit for bit; where it is raised (the log-normal graph
needs twice a threshold of 512 edges to fit), it must equal gt_sparse_mha_fwd
at that threshold bit for bit.  Every case is also held to the oracle (sampled rows,
every split row included, on the million-node graphs).
"""
import math

import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.test_gpu_parity import (assert_close, chunk_edges, custom, dev, host, oracle_inputs, sample_rows, say,
                                   say_split, to_dev, tol_of)

pytestmark = pytest.mark.gpu


def hub_graph(seed, N, E, hubs, dtype, H, D):
    src, dst = gtgen.random_coo(seed, N, E)
    rng = np.random.default_rng(seed)
    dst = np.where(rng.random(E) < 0.3, rng.choice(hubs, E), dst)  # 30% of edges into a few hub rows
    return custom(N, src, dst.astype(np.int32), H, D, dtype, seed=seed)


def check(w, chunk_ref, sampled):
    t = to_dev(w)
    out = torch.full_like(t["Q"], math.nan)
    say("noalloc %s N=%d E=%d H=%d D=%d dtype=%d" % (w["name"], w["N"], w["E"], w["H"], w["D"], w["dtype"]))
    gt.gt_sparse_mha_fwd_noalloc(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out)
    with chunk_edges(chunk_ref):
        ref = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "%s: differs from gt_sparse_mha_fwd at a split threshold of %d" % (
        w["name"], chunk_ref)
    g = host(out)
    if sampled:
        rows = sample_rows(w["indptr"], chunk_ref, n_random=500)
        say_split(w["indptr"], rows, chunk_ref, "noalloc " + w["name"])
        assert_close(g[rows], oracle.fwd_rows(*oracle_inputs(w), rows), tol_of(w), "noalloc " + w["name"])
    else:
        assert_close(g, oracle.fwd(*oracle_inputs(w)), tol_of(w), "noalloc " + w["name"])
    del t, out, ref
    torch.cuda.empty_cache()


def test_noalloc_calls_in_a_row_each_smaller():
    assert gt.gt_config_get(gt.GT_CFG_CHUNK_EDGES) == 0  # automatic
    lognormal = gtgen.make_workload("lognormal")
    # at a configured split threshold of 512 edges the log-normal graph's plan
    # needs 255 MiB of scratch: the call doubles the threshold to 1024 (128 MiB)
    with chunk_edges(512):
        check(lognormal, 1024, True)
    del lognormal
    # the power-law graph's fits at the automatic threshold (2,048 edges: 36 MiB)
    w = gtgen.make_workload("powerlaw")
    assert gt.gt_config_chunk_edges(w["E"]) == 2048
    check(w, 2048, True)
    del w
    # smaller graphs with split rows (automatic threshold 512), then without
    check(hub_graph(3, 20000, 400000, [5, 77, 19999], gtgen.F32, 8, 64), 512, False)
    check(hub_graph(4, 3000, 40000, [0, 2999], gtgen.BF16, 8, 32), 512, False)
    check(hub_graph(5, 500, 6000, [7], gtgen.F32, 8, 10), 512, False)
    check(gtgen.make_workload("tiny_random"), 512, False)


def test_noalloc_threshold_and_empty_graph():
    # a lower configured threshold is kept when the plan fits
    w = hub_graph(6, 4000, 80000, [1, 2, 3], gtgen.F32, 8, 64)
    with chunk_edges(40):
        check(w, 40, False)
    # E = 0: zeros written, nothing read
    e = custom(9, [], [], 8, 64)
    t = to_dev(e)
    out = torch.full_like(t["Q"], math.nan)
    gt.gt_sparse_mha_fwd_noalloc(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
