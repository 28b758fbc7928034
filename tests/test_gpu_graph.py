"""Graph construction and plans on the GPU, through the C ABI.

* gt_coo_to_csr and the plans' CSR and transpose are integer work: compared
  with the oracle's counting sort bit for bit (indptr, indices, perm).
* Attention on a plan runs the same kernels on the same graph: its outputs
  must equal the plan-free calls bit for bit.
* A shard (destination rows [a, b) of a graph, sources over all nodes:
  n_src != n_dst) must reproduce those rows of the whole-graph forward and
  dQ bit for bit; its dK, dV are the shard's share, and the shares of a
  partition add up to the whole-graph gradients (checked against the oracle
  with the backward's tolerances).
"""
import numpy as np
import pytest
import torch

import gtgen
import oracle
import sparse_graph_attention_amd as gt
from tests.bounds import OutTable, sub_graph
from tests.test_gpu_backward import (bound_dkv, btol_of, check_bound, run_gpu, to_torch, widen, with_grad)
from tests.test_gpu_parity import chunk_edges, custom, dev, host, oracle_inputs, say, to_dev, workload

pytestmark = pytest.mark.gpu


def shuffled_coo(indptr, indices, seed):
    """The edges of a CSR as COO arrays in a seeded random order."""
    N = len(indptr) - 1
    dst = np.repeat(np.arange(N, dtype=np.int32), np.diff(indptr))
    order = gtgen.permutation(seed, len(dst)) if len(dst) else np.zeros(0, np.int64)
    return np.ascontiguousarray(indices[order], np.int32), np.ascontiguousarray(dst[order], np.int32)


def check_coo(src, dst, n_dst, n_src=None, what=""):
    n_src = n_dst if n_src is None else n_src
    say("coo_to_csr %s n_dst=%d n_src=%d E=%d" % (what, n_dst, n_src, len(src)))
    d = dev()
    ip, ix, pm = gt.gt_coo_to_csr(torch.from_numpy(src).to(d), torch.from_numpy(dst).to(d), n_dst, n_src,
                                  want_perm=True)
    torch.cuda.synchronize()
    rip, rix, rpm = oracle.coo_to_csr(n_dst, src, dst, n_src=n_src)
    assert np.array_equal(ip.cpu().numpy(), rip), what + ": indptr"
    assert np.array_equal(ix.cpu().numpy(), rix), what + ": indices"
    assert np.array_equal(pm.cpu().numpy().astype(np.int64), rpm), what + ": perm"


@pytest.mark.parametrize("case", ["tiny_random", "molecules", "one_row", "single_node", "empty", "n256", "n257",
                                  "rectangular", "e4096", "e4097", "e16384", "e16385"])
def test_coo_to_csr_small(case):
    rng = np.random.default_rng(7)
    n_src = None
    if case == "tiny_random":
        n = 30
        src, dst = gtgen.random_coo(0, 30, 100)
    elif case == "molecules":
        n, src, dst = gtgen.molecules_coo(0)
    elif case == "one_row":
        n = 50
        src = rng.integers(0, n, 3000).astype(np.int32)
        dst = np.full(3000, 7, np.int32)
    elif case == "single_node":
        n, src, dst = 1, np.zeros(5, np.int32), np.zeros(5, np.int32)
    elif case == "empty":
        n, src, dst = 40, np.zeros(0, np.int32), np.zeros(0, np.int32)
    elif case == "n256":  # 8-bit keys: one pass
        n = 256
        src, dst = gtgen.random_coo(1, n, 20000)
    elif case == "n257":  # 9-bit keys: a second pass of 1 bit
        n = 257
        src, dst = gtgen.random_coo(2, n, 20000)
    elif case.startswith("e"):
        # edge counts around the one-launch sort pass (at most 16,384 keys) and
        # the tiled passes above it; 17-bit ids: three passes, the last of one bit
        n, E = 70000, int(case[1:])
        src = rng.integers(0, n, E).astype(np.int32)
        dst = rng.integers(0, n, E).astype(np.int32)
        dst[: E // 3] = dst[0]  # a long run of one key: stability across waves and tiles
    else:
        n, n_src = 1000, 70000
        src = rng.integers(0, n_src, 50000).astype(np.int32)
        dst = rng.integers(0, n, 50000).astype(np.int32)
    check_coo(np.asarray(src, np.int32), np.asarray(dst, np.int32), n, n_src, case)


@pytest.mark.parametrize("name", ["powerlaw", "lognormal"])
def test_coo_to_csr_large(name):
    w = workload(name)
    src, dst = shuffled_coo(w["indptr"], w["indices"], 5)
    check_coo(src, dst, w["N"], what=name)


def test_coo_to_csr_four_passes():
    # 26-bit destination ids: four 8-bit passes (the last of 2 bits)
    n = (1 << 25) + 12345
    src, dst = gtgen.random_coo(9, n, 3_000_000)
    check_coo(np.asarray(src, np.int32), np.asarray(dst, np.int32), n, what="n=2^25+")


def plan_arrays(plan):
    info = gt.gt_plan_info(plan)
    arrays = gt.gt_plan_copy_graph(plan)
    torch.cuda.synchronize()
    for k, v in zip(("indptr", "indices", "t_indptr", "t_indices", "t_perm"), arrays):
        info[k] = None if v is None else v.cpu().numpy()
    return info


@pytest.mark.parametrize("name", ["tiny_random", "molecules", "powerlaw"])
def test_plan_graph_matches_oracle(name):
    w = workload(name)
    src, dst = shuffled_coo(w["indptr"], w["indices"], 3)
    d = dev()
    say("plan from COO %s" % name)
    plan = gt.gt_plan_create_coo(torch.from_numpy(src).to(d), torch.from_numpy(dst).to(d), w["N"])
    p = plan_arrays(plan)
    rip, rix, _ = oracle.coo_to_csr(w["N"], src, dst)
    assert np.array_equal(p["indptr"], rip) and np.array_equal(p["indices"], rix)
    tip, tix, tpm = oracle.source_sorted(rip, rix, want_perm=True)
    assert np.array_equal(p["t_indptr"], tip) and np.array_equal(p["t_indices"], tix)
    assert np.array_equal(p["t_perm"], tpm)
    plan.destroy()
    say("plan from CSR %s" % name)
    t = to_dev(w)
    plan = gt.gt_plan_create(t["indptr"], t["indices"], transpose=True)
    p = plan_arrays(plan)
    assert np.array_equal(p["indptr"], w["indptr"]) and np.array_equal(p["indices"], w["indices"])
    tip, tix = oracle.source_sorted(w["indptr"], w["indices"])
    assert np.array_equal(p["t_indptr"], tip) and np.array_equal(p["t_indices"], tix)
    assert p["n_dst"] == p["n_src"] == w["N"] and p["E"] == w["E"]
    plan.destroy()
    plan = gt.gt_plan_create(t["indptr"], t["indices"], transpose=False)
    p = plan_arrays(plan)
    assert p["t_indptr"] is None and p["t_indices"] is None
    with pytest.raises(gt.GtError):
        dummy = torch.zeros_like(t["Q"])
        lse = torch.zeros((w["N"], w["H"]), dtype=torch.float32, device=d)
        gt.gt_sparse_mha_bwd_plan(plan, t["Q"], t["K"], t["V"], dummy, dummy, lse)
    plan.destroy()


@pytest.mark.parametrize("n,E", [(300, 16384), (300, 16385), (70000, 12000), (70000, 16385)])
def test_plan_arrays_around_the_one_launch_sort(n, E):
    # both sorts of a plan (by destination from COO, by source for the
    # transpose) on either side of the one-launch sort pass's 16,384-key limit
    rng = np.random.default_rng(n + E)
    src = rng.integers(0, n, E).astype(np.int32)
    dst = rng.integers(0, n, E).astype(np.int32)
    src[: E // 4] = src[0]  # a long run of one source: the transpose's stability
    say("plan arrays n=%d E=%d" % (n, E))
    d = dev()
    plan = gt.gt_plan_create_coo(torch.from_numpy(src).to(d), torch.from_numpy(dst).to(d), n)
    p = plan_arrays(plan)
    rip, rix, _ = oracle.coo_to_csr(n, src, dst)
    assert np.array_equal(p["indptr"], rip) and np.array_equal(p["indices"], rix)
    tip, tix, tpm = oracle.source_sorted(rip, rix, want_perm=True)
    assert np.array_equal(p["t_indptr"], tip) and np.array_equal(p["t_indices"], tix)
    assert np.array_equal(p["t_perm"], tpm)
    plan.destroy()


@pytest.mark.parametrize("lo,hi,n,n_src", [(60000, 61000, 70000, 70000), (0, 100, 70000, 1000),
                                           (3000, 3500, 4000, 250000), (9000, 9001, 200000, 9500)])
def test_plan_with_long_runs_of_empty_rows(lo, hi, n, n_src):
    # destinations and sources confined to narrow ranges, like a row shard of a
    # batch of small graphs: long runs of rows without keys before, between and
    # after the keys, in the CSR and in the transpose (one-launch grouping)
    rng = np.random.default_rng(lo + n)
    E = 5000
    dst = rng.integers(lo, hi, E).astype(np.int32)
    src = rng.integers(max(0, lo - 100), min(n_src, hi + 100), E).astype(np.int32)
    say("plan with empty runs dst [%d, %d) n=%d n_src=%d" % (lo, hi, n, n_src))
    d = dev()
    plan = gt.gt_plan_create_coo(torch.from_numpy(src).to(d), torch.from_numpy(dst).to(d), n, n_src=n_src)
    p = plan_arrays(plan)
    rip, rix, _ = oracle.coo_to_csr(n, src, dst, n_src=n_src)
    assert np.array_equal(p["indptr"], rip) and np.array_equal(p["indices"], rix)
    tip, tix, tpm = oracle.source_sorted(rip, rix, want_perm=True, n_src=n_src)
    assert np.array_equal(p["t_indptr"], tip) and np.array_equal(p["t_indices"], tix)
    assert np.array_equal(p["t_perm"], tpm)
    plan.destroy()
    check_coo(src, dst, n, n_src, "empty runs")


@pytest.mark.parametrize("name,chunk", [("tiny_random", 3), ("molecules", 2), ("regular16", 5), ("powerlaw", 2048),
                                        ("lognormal", 512)])
def test_plan_attention_is_bitwise_the_plain_call(name, chunk):
    w = with_grad(workload(name))
    t = to_dev(w)
    with chunk_edges(chunk):
        say("plan vs plain %s chunk=%d" % (name, chunk))
        plan = gt.gt_plan_create(t["indptr"], t["indices"], transpose=True)
        out, lse, dq, dk, dv = run_gpu(w, t)
        pout, plse = gt.gt_sparse_mha_fwd_plan(plan, t["Q"], t["K"], t["V"], want_lse=True)
        plain_out = gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
        pdq, pdk, pdv = gt.gt_sparse_mha_bwd_plan(plan, t["Q"], t["K"], t["V"], out, t["dO"], lse)
        torch.cuda.synchronize()
    assert torch.equal(pout, out) and torch.equal(plain_out, out) and torch.equal(plse, lse)
    assert torch.equal(pdq, dq) and torch.equal(pdk, dk) and torch.equal(pdv, dv)
    plan.destroy()


def shards(w, t, bounds, srcs_t, full_out, full_lse, full_dq, dk_sum, dv_sum):
    """Each shard of destination rows through its own plan: out, lse and dQ
    equal the whole graph's rows bit for bit; dK and dV are added up over the
    shards at the sampled sources."""
    N = w["N"]
    for a, b in zip(bounds[:-1], bounds[1:]):
        say("shard %s rows [%d, %d)" % (w["name"], a, b))
        ip = w["indptr"][a:b + 1] - w["indptr"][a]
        ix = w["indices"][w["indptr"][a]:w["indptr"][b]]
        d = dev()
        plan = gt.gt_plan_create(torch.from_numpy(ip).to(d), torch.from_numpy(np.ascontiguousarray(ix)).to(d),
                                 n_src=N, transpose=True)
        info = gt.gt_plan_info(plan)
        assert (info["n_dst"], info["n_src"], info["E"]) == (b - a, N, len(ix))
        Qs = t["Q"][a:b].contiguous()
        out, lse = gt.gt_sparse_mha_fwd_plan(plan, Qs, t["K"], t["V"], want_lse=True)
        dOs = t["dO"][a:b].contiguous()
        dq, dk, dv = gt.gt_sparse_mha_bwd_plan(plan, Qs, t["K"], t["V"], out, dOs, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, full_out[a:b]) and torch.equal(lse, full_lse[a:b])
        assert torch.equal(dq, full_dq[a:b])
        dk_sum += host(dk[srcs_t])
        dv_sum += host(dv[srcs_t])
        plan.destroy()


@pytest.mark.parametrize("name,parts", [("regular16", 3), ("powerlaw", 2), ("molecules", 4)])
def test_row_shards(name, parts):
    w = with_grad(workload(name))
    t = to_dev(w)
    N, H = w["N"], w["H"]
    full_out, full_lse, full_dq, _, _ = run_gpu(w, t)
    # split rows so that the shards hold about the same number of edges
    cuts = np.searchsorted(w["indptr"], np.linspace(0, w["E"], parts + 1)[1:-1])
    bounds = [0, *cuts.tolist(), N]
    srcs = np.unique(np.concatenate([np.arange(0, N, max(1, N // 700)), [N - 1]])).astype(np.int64)
    srcs_t = torch.from_numpy(srcs).to(dev())
    dk_sum = np.zeros((len(srcs), H, w["D"]))
    dv_sum = np.zeros((len(srcs), H, w["D"]))
    # the automatic split threshold depends on the edge count, and a shard
    # holds fewer edges than the whole graph: the shards take the whole
    # graph's threshold, so that their rows are split as the whole graph's are
    with chunk_edges(gt.gt_config_chunk_edges(w["E"])):
        shards(w, t, bounds, srcs_t, full_out, full_lse, full_dq, dk_sum, dv_sum)
    rq, rk, rv, rlse, _ = (oracle.bwd(*oracle_inputs(w), w["dO"]) if name == "molecules" else (None,) * 5)
    if rk is None:
        rlse, rdelta = oracle.row_stats(*oracle_inputs(w), w["dO"])
        rk, rv = oracle.dkv_sources(w["t_indptr"], w["t_indices"], w["Q"], w["K"], w["V"], w["dO"], rlse, rdelta,
                                    srcs)
    else:
        rk, rv = rk[srcs], rv[srcs]
    need = np.unique(sub_graph(w["t_indptr"], w["t_indices"], srcs)[1]).astype(np.int64)
    BK, BV = bound_dkv(w, rlse, OutTable(oracle.fwd_rows(*oracle_inputs(w), need), need), srcs)
    check_bound(dk_sum, rk, BK, btol_of(w), "sum of shard dK " + name)
    check_bound(dv_sum, rv, BV, btol_of(w), "sum of shard dV " + name)


def test_shard_without_edges_writes_zeros():
    N = 20
    w = with_grad(custom(N, [], [], 4, 16))
    t = to_dev(w)
    d = dev()
    ip = torch.zeros(6, dtype=torch.int64, device=d)  # 5 destination rows, no edges
    ix = torch.zeros(0, dtype=torch.int32, device=d)
    plan = gt.gt_plan_create(ip, ix, n_src=N, transpose=True)
    Qs = t["Q"][:5].contiguous()
    out, lse = gt.gt_sparse_mha_fwd_plan(plan, Qs, t["K"], t["V"], want_lse=True)
    grads = [torch.full_like(x, float("nan")) for x in (Qs, t["K"], t["V"])]
    say("empty shard")
    gt.gt_sparse_mha_bwd_plan(plan, Qs, t["K"], t["V"], out, to_torch(w["dO"])[:5].contiguous(), lse, *grads)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == -np.inf)
    for g in grads:
        assert torch.all(g == 0)
    plan.destroy()


def test_coo_plan_bf16_is_bitwise_the_plain_call_on_its_graph():
    # a plan built from shuffled COO arrays (rows then list their edges in the
    # shuffled order) against the plain calls on the plan's own CSR and transpose
    w = with_grad(workload("molecules"))
    w = dict(w, dtype=gtgen.BF16)
    for k in ("Q", "K", "V", "dO"):
        f = widen(w[k]).astype(np.float32)
        w[k] = (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 bits will do
    t = to_dev(w)
    dO = to_torch(w["dO"])
    src, dst = shuffled_coo(w["indptr"], w["indices"], 4)
    d = dev()
    plan = gt.gt_plan_create_coo(torch.from_numpy(src).to(d), torch.from_numpy(dst).to(d), w["N"])
    ip, ix, tip, tix, _ = gt.gt_plan_copy_graph(plan)
    say("bf16 plan vs plain on the plan's graph")
    out, lse = gt.gt_sparse_mha_fwd_lse(ip, ix, t["Q"], t["K"], t["V"])
    dq, dk, dv = gt.gt_sparse_mha_bwd(ip, ix, tip, tix, t["Q"], t["K"], t["V"], out, dO, lse)
    pout, plse = gt.gt_sparse_mha_fwd_plan(plan, t["Q"], t["K"], t["V"], want_lse=True)
    pdq, pdk, pdv = gt.gt_sparse_mha_bwd_plan(plan, t["Q"], t["K"], t["V"], out, dO, lse)
    torch.cuda.synchronize()
    assert torch.equal(pout, out) and torch.equal(plse, lse)
    assert torch.equal(pdq, dq) and torch.equal(pdk, dk) and torch.equal(pdv, dv)
    plan.destroy()
