"""Benchmark of the fused sparse multi-head attention forward on one MI355X.

One step = one gt_sparse_mha_fwd call (plan, fused attention kernel, merge of
split rows) over the power-law workload: N=1,000,000 nodes, E=16,000,000
edges, in-degrees Zipf(1.8) clipped at 50,000, uniform sources, H=8 heads of
D=64, fp32; inputs resident in HBM before timing starts.

Prints one JSON line: edge-heads/s of the whole call (and per-call median and
minimum event times, back to back and after an L2 / Infinity Cache flush), the roofline of the
dominant kernels (the fused attention kernel and the merge of split rows, which
writes those rows' outputs, timed with HIP events on their own stream over the
timed region) against MI355X's 8 TB/s HBM peak, the HBM traffic counted by
rocprofv3 (from the committed counter summary, when it matches the current
kernel source), and the CPU oracle timed on a bounded sample of the same
workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--no-stages] [--no-backward] [--no-plan] [--no-variants]
                  [--no-layout] [--no-ceiling] [--no-shards]
                  [--calib-copy] [--calib-windows]

Also reported beside the step: the unfused stages (SDDMM, edge softmax, SpMM),
the backward (gt_sparse_mha_bwd), graph construction (COO to CSR, a plan with
its transpose, the forward on a plan), and the forward and backward with an
additive bias, edge weights and attention dropout, each event-timed on the
same inputs, and the forward with head-innermost [N][D][H] features; and the
achievable ceiling: the K and V row gathers alone (gt_calib_gather) and a
plain device copy; and one GPU's share of an 8-way row-sharded run (each
shard's forward and backward on a plan with all N nodes as sources).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edge-heads/sec + achieved HBM GB/s (% of peak), fused sparse MHA fwd"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_fwd_powerlaw_1M.traffic.txt")
KERNEL_SOURCES = ["sparse_graph_attention_amd/csrc/fused.hip", "sparse_graph_attention_amd/csrc/common.hpp",
                  "sparse_graph_attention_amd/csrc/kernels.hpp"]
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_powerlaw_1M.traffic.txt")
BWD_SOURCES = ["sparse_graph_attention_amd/csrc/bwd.hip", "sparse_graph_attention_amd/csrc/bwd_dq.hip",
               "sparse_graph_attention_amd/csrc/bwd_dkv.hip", "sparse_graph_attention_amd/csrc/plan.hip",
               "sparse_graph_attention_amd/csrc/common.hpp", "sparse_graph_attention_amd/csrc/kernels.hpp"]

DESCRIPTIONS = {
    "powerlaw": "power-law graph: N=1,000,000, E=16,000,000, in-degree Zipf(1.8) clipped at 50,000, "
                "uniform sources, H=8, D=64, fp32",
    "lognormal": "log-normal graph: N=2,400,000, E=60,000,000, in-degree log-normal (mean 25, sigma 1.2), "
                 "uniform sources, H=8, D=32, bf16 in/out, fp32 accumulation",
    "regular16": "in-degree-16 graph: N=100,000, E=1,600,000, uniform sources, H=8, D=64, fp32",
    "molecules": "128 molecule-like graphs batched (N ~ 4,000, E ~ 8,500, symmetric), H=8, D=10, fp32",
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_sha(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for p in sources:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def load_traffic(threshold, path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per call of the timed kernels from a committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE per dispatch, summed over the call's
    kernels and scaled by what the counters read for a plain copy), or None when
    the summary is missing, the kernel sources changed since it was taken, or
    it was taken at another split threshold than `threshold` (edges)."""
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_sha(sources):
        return None, "kernel changed since the counters were taken"
    if kv.get("split_threshold_edges") != str(threshold):
        return None, "counters taken at another split threshold"
    fetch = float(kv["fetch_kib_per_call"]) * 1024 * float(kv["copy_fetch_scale"])
    write = float(kv["write_kib_per_call"]) * 1024 * float(kv["copy_write_scale"])
    return fetch + write, "stored rocprofv3 FETCH_SIZE + WRITE_SIZE (%s), scaled by a plain copy" % (
        os.path.relpath(path, ROOT))


def algorithmic_bytes(w):
    """Bytes the method must move: each edge gathers one K and one V row, Q is read
    once per row with in-edges, out is written once per row, plus the CSR."""
    import numpy as np

    b = 4 if w["dtype"] == 0 else 2
    HD = w["H"] * w["D"]
    nnz = int((np.diff(w["indptr"]) > 0).sum())
    return nnz * HD * b + 2 * w["E"] * HD * b + w["N"] * HD * b + 4 * w["E"] + 8 * (w["N"] + 1)


def stage_bytes(w):
    """Algorithmic bytes of the unfused stages (scores and weights are fp32 [E][H])."""
    import numpy as np

    b = 4 if w["dtype"] == 0 else 2
    N, E, H, HD = w["N"], w["E"], w["H"], w["H"] * w["D"]
    nnz = int((np.diff(w["indptr"]) > 0).sum())
    csr = 4 * E + 8 * (N + 1)
    return {
        "sddmm": nnz * HD * b + E * HD * b + E * H * 4 + csr,
        "edge_softmax": 2 * E * H * 4 + 8 * (N + 1),
        "spmm": E * H * 4 + E * HD * b + N * HD * b + csr,
    }


def time_stages(gt, t, w, steps, warmup):
    """Event-timed unfused stages on the same inputs: ms per call and algorithmic GB/s."""
    import torch

    scores = torch.empty((w["E"], w["H"]), dtype=torch.float32, device=t["Q"].device)
    alpha = torch.empty_like(scores)
    out = torch.empty_like(t["Q"])
    calls = {
        "sddmm": lambda: gt.gt_sddmm(t["indptr"], t["indices"], t["Q"], t["K"], scores=scores),
        "edge_softmax": lambda: gt.gt_edge_softmax(t["indptr"], scores, alpha=alpha),
        "spmm": lambda: gt.gt_spmm(t["indptr"], t["indices"], alpha, t["V"], out=out),
    }
    nbytes = stage_bytes(w)
    res = {}
    for name, fn in calls.items():
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms": ms, "algorithmic_bytes": nbytes[name], "GBps": nbytes[name] / (ms * 1e-3) / 1e9}
        log("stage %s: %.3f ms, %.0f GB/s algorithmic" % (name, ms, res[name]["GBps"]))
    del scores, alpha, out
    return res


def backward_bytes(w):
    """Algorithmic bytes of gt_sparse_mha_bwd: the destination pass gathers K and V
    per edge and reads Q, dO, out, lse of each row with in-edges, writing dQ (all
    rows) and delta; the source pass gathers Q, dO, lse and delta per edge and
    reads K, V of each source with out-edges, writing dK and dV; both CSRs once."""
    import numpy as np

    b = 4 if w["dtype"] == 0 else 2
    N, E, H, HD = w["N"], w["E"], w["H"], w["H"] * w["D"]
    nnz = int((np.diff(w["indptr"]) > 0).sum())
    nsrc = int((np.bincount(w["indices"], minlength=N) > 0).sum())
    csr = 4 * E + 8 * (N + 1)
    dq = E * 2 * HD * b + nnz * (3 * HD * b + 8 * H) + N * HD * b + csr
    dkv = E * (2 * HD * b + 8 * H) + nsrc * 2 * HD * b + N * 2 * HD * b + csr
    return dq + dkv


def time_backward(gt, t, w, steps, warmup):
    """Event-timed gt_sparse_mha_bwd (after a gt_sparse_mha_fwd_lse) on the same inputs."""
    import numpy as np
    import torch

    import gtgen

    dev = t["Q"].device
    tip, tix = gtgen.source_sorted(w["indptr"], w["indices"])
    tip, tix = torch.from_numpy(tip).to(dev), torch.from_numpy(tix).to(dev)
    g = gtgen.make_grad(w["N"], w["H"], w["D"], w["dtype"], seed=11)
    dO = (torch.from_numpy(g.view(np.int16)).to(dev).view(torch.bfloat16) if g.dtype == np.uint16
          else torch.from_numpy(g).to(dev))
    out, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    grads = [torch.empty_like(t["Q"]) for _ in range(3)]

    def call():
        gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, t["Q"], t["K"], t["V"], out, dO, lse, *grads)

    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = backward_bytes(w)
    traffic, note = (load_traffic(gt.gt_config_chunk_edges(w["E"]), BWD_TRAFFIC_FILE, BWD_SOURCES)
                     if w.get("name") == "powerlaw"
                     else (None, "counters are for the power-law workload"))
    res = {"ms": ms, "edge_heads_per_s": w["E"] * w["H"] / (ms * 1e-3),
           # the method's bytes over the call time: can pass the HBM peak, since the
           # source pass re-reads popular destinations' rows from cache
           "algorithmic_bytes": nbytes, "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9,
           "algorithmic_rate_over_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           # HBM bytes counted per call (both passes, merges and work lists) over the call time
           "traffic": traffic, "traffic_source": note,
           "GBps": None if traffic is None else traffic / (ms * 1e-3) / 1e9,
           "frac": None if traffic is None else traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    log("backward: %.3f ms, %.0f GB/s algorithmic; counted traffic: %s" % (
        ms, res["algorithmic_GBps"], "%.0f GB/s (%.0f%% of HBM peak)" % (res["GBps"], 100 * res["frac"])
        if traffic is not None else note))
    del grads, out, lse, dO, tip, tix
    return res


def time_plan(gt, t, w, steps):
    """Graph construction from shuffled COO arrays (gt_coo_to_csr; gt_plan_create_coo with the
    transpose) and the forward on a plan, event-timed on the current stream."""
    import numpy as np
    import torch

    import gtgen

    dev = t["Q"].device
    N = w["N"]
    dst = np.repeat(np.arange(N, dtype=np.int32), np.diff(w["indptr"]))
    order = gtgen.permutation(7, len(dst))
    src_t = torch.from_numpy(np.ascontiguousarray(w["indices"][order])).to(dev)
    dst_t = torch.from_numpy(np.ascontiguousarray(dst[order])).to(dev)
    del dst, order

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        total = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            r = fn()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
            if isinstance(r, gt.GtPlan):
                r.destroy()
        return total / reps

    res = {"coo_to_csr_ms": timed(lambda: gt.gt_coo_to_csr(src_t, dst_t, N), steps),
           "plan_create_coo_ms": timed(lambda: gt.gt_plan_create_coo(src_t, dst_t, N, transpose=True), steps)}
    plan = gt.gt_plan_create_coo(src_t, dst_t, N, transpose=True)
    out = torch.empty_like(t["Q"])
    res["fwd_plan_ms"] = timed(lambda: gt.gt_sparse_mha_fwd_plan(plan, t["Q"], t["K"], t["V"], out=out), steps)
    res["fwd_ms"] = timed(lambda: gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out=out),
                          steps)
    plan.destroy()
    res["edges_per_s_coo_to_csr"] = w["E"] / (res["coo_to_csr_ms"] * 1e-3)
    log("plan: COO->CSR %.3f ms, plan with transpose %.3f ms; forward on a plan %.3f ms vs %.3f ms"
        % (res["coo_to_csr_ms"], res["plan_create_coo_ms"], res["fwd_plan_ms"], res["fwd_ms"]))
    del src_t, dst_t, out
    return res


def time_variants(gt, t, w, steps, warmup=2):
    """Forward and backward with an additive bias [E][H], edge weights [E] and
    attention dropout (p = 0.1), event-timed; algorithmic bytes add the bias
    and weights (and, in the backward, the transpose's CSR positions)."""
    import numpy as np
    import torch

    import gtgen

    dev = t["Q"].device
    E, H = w["E"], w["H"]
    bias = (torch.from_numpy(gtgen.normal_f32(3, 11, (E, H))) * 0.5).to(dev)
    ew = torch.from_numpy(gtgen.uniform_f64(3, 12, E, 0.2, 1.0).astype(np.float32)).to(dev)
    opts = dict(bias=bias, edge_weight=ew, dropout_p=0.1, dropout_seed=1234)
    tip, tix, tpm = (torch.from_numpy(x).to(dev) for x in gtgen.source_sorted(w["indptr"], w["indices"],
                                                                              want_perm=True))
    g = gtgen.make_grad(w["N"], H, w["D"], w["dtype"], seed=11)
    dO = (torch.from_numpy(g.view(np.int16)).to(dev).view(torch.bfloat16) if g.dtype == np.uint16
          else torch.from_numpy(g).to(dev))
    out = torch.empty_like(t["Q"])
    lse = torch.empty((w["N"], H), dtype=torch.float32, device=dev)

    def fwd():
        gt.gt_sparse_mha_fwd_ex(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out=out, lse=lse, **opts)

    def bwd():
        gt.gt_sparse_mha_bwd_ex(t["indptr"], t["indices"], tip, tix, tpm, t["Q"], t["K"], t["V"], out, dO, lse,
                                **opts)

    res = {}
    extra = E * H * 4 + E * 4
    for name, fn, nbytes in (("fwd_ms", fwd, algorithmic_bytes(w) + extra),
                             ("bwd_ms", bwd, backward_bytes(w) + 2 * extra + 4 * E)):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = ms
        res[name.replace("_ms", "_GBps")] = nbytes / (ms * 1e-3) / 1e9
    log("variants (bias, weights, dropout 0.1): forward %.3f ms (%.0f GB/s), backward %.3f ms (%.0f GB/s)"
        % (res["fwd_ms"], res["fwd_GBps"], res["bwd_ms"], res["bwd_GBps"]))
    del bias, ew, tip, tix, tpm, dO, out, lse
    return res


def time_layout(gt, t, w, steps, warmup=3):
    """The forward and the backward with features [N][H][D] (gt_sparse_mha_fwd,
    gt_sparse_mha_bwd) and [N][D][H] (gt_sparse_mha_fwd_layout,
    gt_sparse_mha_bwd_layout: their own kernels where the shape allows, else
    transposed copies), event-timed; algorithmic bytes as for the step and
    for the backward."""
    import numpy as np
    import torch

    import gtgen

    def ndh(x):
        return x.transpose(1, 2).contiguous()

    dev = t["Q"].device
    Qn, Kn, Vn = ndh(t["Q"]), ndh(t["K"]), ndh(t["V"])
    out = torch.empty_like(t["Q"])
    outn = torch.empty_like(Qn)
    tip, tix = (torch.from_numpy(x).to(dev) for x in gtgen.source_sorted(w["indptr"], w["indices"]))
    g = gtgen.make_grad(w["N"], w["H"], w["D"], w["dtype"], seed=11)
    dO = (torch.from_numpy(g.view(np.int16)).to(dev).view(torch.bfloat16) if g.dtype == np.uint16
          else torch.from_numpy(g).to(dev))
    dOn = ndh(dO)
    fo, lse = gt.gt_sparse_mha_fwd_lse(t["indptr"], t["indices"], t["Q"], t["K"], t["V"])
    fon = ndh(fo)
    calls = {
        "nhd": lambda: gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out=out),
        "ndh": lambda: gt.gt_sparse_mha_fwd_layout(t["indptr"], t["indices"], Qn, Kn, Vn, layout="ndh", out=outn),
        "bwd_nhd": lambda: gt.gt_sparse_mha_bwd(t["indptr"], t["indices"], tip, tix, t["Q"], t["K"], t["V"], fo, dO,
                                                lse),
        "bwd_ndh": lambda: gt.gt_sparse_mha_bwd_layout(t["indptr"], t["indices"], tip, tix, None, Qn, Kn, Vn, fon,
                                                       dOn, lse, layout="ndh"),
    }
    res = {}
    for name, fn in calls.items():
        nbytes = backward_bytes(w) if name.startswith("bwd") else algorithmic_bytes(w)
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name + "_ms"] = ms
        res[name + "_GBps"] = nbytes / (ms * 1e-3) / 1e9
    log("layout: forward [N][H][D] %.4f ms, [N][D][H] %.4f ms; backward %.4f ms, %.4f ms" % (
        res["nhd_ms"], res["ndh_ms"], res["bwd_nhd_ms"], res["bwd_ndh_ms"]))
    del Qn, Kn, Vn, out, outn, tip, tix, dO, dOn, fo, fon, lse
    return res


def time_ceiling(gt, t, w, kern_ms, reps=10, copy_gib=1.0):
    """Achievable rates beside the 8 TB/s peak, event-timed on the same inputs:
    gt_calib_gather (the K and V row gathers of every edge, read as the fused
    kernel reads them, and nothing else) and a plain device copy of copy_gib
    GiB.  gather_frac: the fused kernel's K+V gather bytes per its time, over
    the rate of the gathers alone."""
    import torch

    row_bytes = t["K"][0].numel() * t["K"].element_size()
    if row_bytes not in (512, 1024, 2048):
        return None
    sink = torch.zeros(1, dtype=torch.int32, device=t["K"].device)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    g_ms = timed(lambda: gt.gt_calib_gather(t["indices"], t["K"], t["V"], checksum=sink))
    g_bytes = 2 * w["E"] * row_bytes + 4 * w["E"]
    n = int(copy_gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device=t["K"].device)
    b = torch.empty_like(a)
    c_ms = timed(lambda: b.copy_(a))
    del a, b
    res = {
        "gather_ms": g_ms,
        "gather_GBps": g_bytes / (g_ms * 1e-3) / 1e9,
        "gather_bytes": g_bytes,
        "copy_GBps": 2 * n * 4 / (c_ms * 1e-3) / 1e9,
        "gather_frac": (2 * w["E"] * row_bytes / (kern_ms * 1e-3)) / (g_bytes / (g_ms * 1e-3)),
    }
    log("ceiling: K+V gathers alone %.3f ms (%.0f GB/s), device copy %.0f GB/s; fused kernel's gathers at %.0f%% "
        "of the gathers-alone rate" % (g_ms, res["gather_GBps"], res["copy_GBps"], 100 * res["gather_frac"]))
    return res


def time_shards(gt, t, w, parts=8, reps=5):
    """One GPU's share of a row-sharded run: the rows cut into `parts` ranges of
    about E/parts edges each; every shard's plan has its rows as destinations
    and all N nodes as sources (K and V whole, as after an all-gather), and its
    forward (gt_sparse_mha_fwd_plan) and backward (gt_sparse_mha_bwd_plan) are
    event-timed on this GPU at that shape.  The exchange of K/V and of the
    dK/dV shares between GPUs is not included."""
    import numpy as np
    import torch

    import gtgen

    dev = t["Q"].device
    N, E = w["N"], w["E"]
    ip = w["indptr"]
    cuts = np.searchsorted(ip, np.linspace(0, E, parts + 1)[1:-1])
    bounds = [0, *cuts.tolist(), N]
    g = gtgen.make_grad(N, w["H"], w["D"], w["dtype"], seed=11)
    dO = (torch.from_numpy(g.view(np.int16)).to(dev).view(torch.bfloat16) if g.dtype == np.uint16
          else torch.from_numpy(g).to(dev))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    fwd, bwd, edges = [], [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        sip = torch.from_numpy(ip[a:b + 1] - ip[a]).to(dev)
        six = torch.from_numpy(np.ascontiguousarray(w["indices"][ip[a]:ip[b]])).to(dev)
        plan = gt.gt_plan_create(sip, six, n_src=N, transpose=True)
        Qs, dOs = t["Q"][a:b], dO[a:b]
        out, lse = gt.gt_sparse_mha_fwd_plan(plan, Qs, t["K"], t["V"], want_lse=True)
        fwd.append(timed(lambda: gt.gt_sparse_mha_fwd_plan(plan, Qs, t["K"], t["V"], out=out, lse=lse)))
        bwd.append(timed(lambda: gt.gt_sparse_mha_bwd_plan(plan, Qs, t["K"], t["V"], out, dOs, lse)))
        edges.append(int(ip[b] - ip[a]))
        plan.destroy()
        del sip, six, out, lse
    res = {"parts": parts, "edges_per_shard_max": max(edges), "fwd_ms_max": max(fwd), "fwd_ms_mean": sum(fwd) / parts,
           "bwd_ms_max": max(bwd), "bwd_ms_mean": sum(bwd) / parts,
           "fwd_edge_heads_per_s_per_gpu": max(edges) * w["H"] / (max(fwd) * 1e-3)}
    log("shards: %d row ranges of <= %d edges; forward %.3f ms (slowest), backward %.3f ms (slowest)"
        % (parts, max(edges), res["fwd_ms_max"], res["bwd_ms_max"]))
    del dO
    return res


def time_calls(step, reps, flush_gib=1.0):
    """Per-call event times of step(): back to back, and with a write of a
    flush_gib GiB buffer between calls (evicting the L2 and the 256 MB
    Infinity Cache; the write is outside the timed span)."""
    import statistics

    import torch

    junk = torch.empty(int(flush_gib * (1 << 30)) // 4, dtype=torch.float32, device="cuda")
    res = {}
    for name, flush in (("back_to_back", False), ("flushed", True)):
        times = []
        for _ in range(reps):
            if flush:
                junk.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        res[name] = {"median_ms": statistics.median(times), "min_ms": min(times)}
    del junk
    log("per call: back to back median %.3f ms (min %.3f), after a cache flush median %.3f ms (min %.3f)"
        % (res["back_to_back"]["median_ms"], res["back_to_back"]["min_ms"], res["flushed"]["median_ms"],
           res["flushed"]["min_ms"]))
    return res


def cpu_baseline(w, out_gpu, fraction=0.5, seed=0):
    """The oracle as it stands on a fixed random sample of destination rows."""
    import numpy as np

    import oracle

    N = w["N"]
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(N, size=max(1, int(N * fraction)), replace=False)).astype(np.int64)
    ip = w["indptr"]
    edges = int((ip[rows + 1] - ip[rows]).sum())
    threads = oracle.default().max_threads()
    log("cpu baseline: oracle on %d rows (%d edges) with %d threads" % (len(rows), edges, threads))
    t0 = time.perf_counter()
    ref = oracle.fwd_rows(w["indptr"], w["indices"], w["Q"], w["K"], w["V"], rows)
    dt = time.perf_counter() - t0
    g = out_gpu[rows].astype(np.float64)
    log("cpu baseline: %.2f s; GPU vs oracle on the sample: max abs err %.3e" % (dt, float(np.abs(g - ref).max())))
    # one thread, on a tenth of that sample
    rows1 = rows[::10]
    edges1 = int((ip[rows1 + 1] - ip[rows1]).sum())
    t0 = time.perf_counter()
    oracle.fwd_rows(w["indptr"], w["indices"], w["Q"], w["K"], w["V"], rows1, nthreads=1)
    dt1 = time.perf_counter() - t0
    log("cpu baseline, 1 thread: %d rows (%d edges) in %.2f s" % (len(rows1), edges1, dt1))
    return {
        "value": edges * w["H"] / dt,
        "unit": "edge-heads/s",
        "cores": threads,
        "kind": "oracle",
        "host": {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count()},
        "sample": "%d%% of destination rows drawn uniformly (seed %d): %d rows, %d edges, %.1f s wall" % (
            round(fraction * 100), seed, len(rows), edges, dt),
        "single_thread": {
            "value": edges1 * w["H"] / dt1,
            "sample": "every 10th row of that sample: %d rows, %d edges, %.1f s wall" % (len(rows1), edges1, dt1),
        },
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def calib_copy(gib=1.0, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4, "reps": reps}), flush=True)


def calib_windows(E=16_000_000, N=1_000_000, reps=5):
    """The K and V row gathers alone (gt_calib_gather, fp32 rows of 8 x 64,
    2 KB) over E edges whose uniform sources lie in a window of W nodes, for
    K+V footprints from 4 GB down to 4 MB: one JSON line of event-timed rates.
    Under rocprofv3 --pmc FETCH_SIZE the dispatches of each window follow in
    this order (1 warm-up + reps each), which shows whether reads served by the
    Infinity Cache are counted as fetched bytes."""
    import torch

    import sparse_graph_attention_amd as gt

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    K = torch.randn(N, 512, device=dev)
    V = torch.randn(N, 512, device=dev)
    res = []
    for W in (N, 65536, 16384, 1024):
        gen.manual_seed(W)
        idx = torch.randint(0, W, (E,), device=dev, dtype=torch.int32, generator=gen)
        Kw, Vw = K[:W], V[:W]
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        gt.gt_calib_gather(idx, Kw, Vw, checksum=sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gt.gt_calib_gather(idx, Kw, Vw, checksum=sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = 2 * E * 2048 + 4 * E
        res.append({"window_nodes": W, "footprint_bytes": 2 * W * 2048, "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "gather_bytes": nbytes})
        log("window %d nodes (K+V %.1f MB): %.3f ms, %.0f GB/s" % (W, 2 * W * 2048 / 1e6, ms, res[-1]["GBps"]))
        del idx
    print(json.dumps({"calib_windows": res, "reps": reps, "E": E}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="powerlaw", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--calib-windows", action="store_true",
                    help="only the K/V gathers alone over source windows of 4 GB .. 4 MB")
    ap.add_argument("--no-stages", action="store_true", help="skip timing the unfused stages")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward")
    ap.add_argument("--no-plan", action="store_true", help="skip timing graph construction and plans")
    ap.add_argument("--no-variants", action="store_true", help="skip timing the logit variants and dropout")
    ap.add_argument("--no-layout", action="store_true", help="skip timing the head-innermost layout")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the gathers-alone and copy rates")
    ap.add_argument("--no-shards", action="store_true", help="skip timing one GPU's share of 8 row shards")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    if args.calib_windows:
        calib_windows()
        return

    import numpy as np
    import torch

    import gtgen
    import sparse_graph_attention_amd as gt

    log("generating %s" % args.workload)
    t0 = time.perf_counter()
    w = gtgen.make_workload(args.workload)
    log("generated N=%d E=%d in %.1f s" % (w["N"], w["E"], time.perf_counter() - t0))
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(w[k]).to(dev) for k in ("indptr", "indices")}
    for k in ("Q", "K", "V"):
        x = w[k]
        t[k] = (torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) if x.dtype == np.uint16
                else torch.from_numpy(x).to(dev))
    out = torch.empty_like(t["Q"])
    torch.cuda.synchronize()

    def step():
        gt.gt_sparse_mha_fwd(t["indptr"], t["indices"], t["Q"], t["K"], t["V"], out=out)

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    gt.gt_profile_begin(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms, call_ms, calls = gt.gt_profile_end()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_avg_ms = kern_ms / calls
    E, H = w["E"], w["H"]
    alg = algorithmic_bytes(w)
    achieved = alg / (kern_avg_ms * 1e-3) / 1e9
    traffic, traffic_note = (load_traffic(gt.gt_config_chunk_edges(E)) if args.workload == "powerlaw"
                             else (None, "counters are for powerlaw"))
    log("ms/step %.3f (event-timed call %.3f ms, fused kernel + merge %.3f ms); algorithmic %.2f GB -> %.0f GB/s"
        % (ms_per_step, call_ms / calls, kern_avg_ms, alg / 1e9, achieved))
    log("traffic: %s" % traffic_note)

    line = {
        "metric": METRIC,
        "value": E * H / (ms_per_step * 1e-3),
        "unit": "edge-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w["dtype"] == 0 else "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.workload], "N": w["N"], "E": E, "H": H, "D": w["D"],
                   "split_threshold_edges": gt.gt_config_chunk_edges(E)},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_source": traffic_note,
            # HBM bytes counted by rocprofv3 over the same kernels' live average duration
            "traffic_GBps": None if traffic is None else traffic / (kern_avg_ms * 1e-3) / 1e9,
            "kernel": "fused attention kernel + merge of split rows",
            "kernel_ms": kern_avg_ms,
            "algorithmic_bytes": alg,
        },
        "cpu_baseline": None,
        "calls": time_calls(step, max(5, args.steps)),
        "ceiling": None if args.no_ceiling else time_ceiling(gt, t, w, kern_avg_ms),
        "stages": None,
        "backward": None,
        "plan": None,
        "variants": None,
        "layout": None,
        "shards": None,
    }
    out_host = out.float().cpu().numpy() if out.dtype == torch.bfloat16 else out.cpu().numpy()
    if not args.no_stages:
        line["stages"] = time_stages(gt, t, w, max(3, args.steps // 2), 2)
    if not args.no_backward:
        line["backward"] = time_backward(gt, t, w, max(3, args.steps // 2), 2)
    if not args.no_plan:
        line["plan"] = time_plan(gt, t, w, max(3, args.steps // 4))
    if not args.no_variants:
        line["variants"] = time_variants(gt, t, w, max(3, args.steps // 4))
    if not args.no_layout:
        line["layout"] = time_layout(gt, t, w, 200 if w["E"] < 10 ** 6 else max(3, args.steps // 4))
    if not args.no_shards:
        line["shards"] = time_shards(gt, t, w)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, out_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
