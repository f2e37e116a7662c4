"""Throughput of the product-key memory lookup on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload default]

One step = the whole lookup (projection + BN, subkey scoring, per-half top-k,
candidate top-k, softmax, value gather) over one batch of synthetic tokens,
inputs resident in HBM.  Prints one JSON line: tokens/s for the workload,
per-kernel times from HIP events recorded on the stream the library launches
on, the roofline of the dominant kernel and of the value gather, and the fp64
CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

import synthetic

METRIC = "PKM lookups(tokens)/sec + value-gather HBM GB/s, N=1M, k=32, 4 heads"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
# The GEMMs are fp32-accurate products built from three fp16 matrix-core
# products per fp32 product (two-piece fp16 splitting of power-of-two scaled
# rows), so their ceiling is a third of MI355X's dense fp16 matrix peak of
# 2.5 PFLOP/s.
GEMM_PEAK_TFLOPS = 2500.0 / 3
ELT_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1, "int8": 1, "int4": 0.5}
SCALED = ("e4m3", "int8", "int4")  # tables with a per-row fp32 scale
ROOT = os.path.dirname(os.path.abspath(__file__))
# Sources of each kernel: measured HBM traffic is only reported while they
# are unchanged since the counters were taken.
KERNEL_SOURCES = {"exponents": ["gemm_f32.hip"], "query_gemm": ["gemm_f32.hip"], "score_gemm": ["gemm_f32.hip"],
                  "folded_gemm": ["gemm_f32.hip"],
                  "select": ["select.hip", "wave_ops.h"], "gather": ["gather.hip", "gather_dev.h"],
                  "select_gather": ["select.hip", "wave_ops.h", "gather_dev.h"]}


def measured_traffic(workload, kernel):
    """HBM bytes per launch from profiles/traffic.json (rocprofv3 FETCH_SIZE
    and WRITE_SIZE runs, scaled by a plain copy's counts), or None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
        entry = rec["kernels"][kernel]
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "product_key_memory_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return entry["bytes"] if h.hexdigest() == entry["source_sha256"] else None


def per_token_work(wl):
    """Algorithmic work per token (lookups are per token, all heads)."""
    return {
        "query_flop": 2.0 * wl.H * wl.D * wl.D,              # a1: Wq[h] . x for every head
        "score_flop": 2.0 * wl.H * wl.n * wl.D,              # a3: 2 halves x n subkeys x D/2
        "folded_flop": 2.0 * wl.D * 2 * wl.H * wl.n,         # a1-a3 folded: x . M for 2H n folded keys
        "select_bytes": wl.H * (2 * wl.n * 4 + wl.k * 8),    # a4-a6: read half scores, write idx + w
        # a7: the gathered rows (+ one fp32 scale per row for the scaled tables)
        "gather_bytes": wl.H * wl.k * (wl.D * ELT_BYTES[wl.table] + (4 if wl.table in SCALED else 0)),
    }


def fused(wl):
    """Whether the forward runs a4-a7 as one kernel (n_keys 1024 or 2048,
    H k <= 512, table rows longer than 512 bytes)."""
    return wl.n in (1024, 2048) and wl.H * wl.k <= 512 and wl.D * ELT_BYTES[wl.table] > 512


def stage_bytes(wl, prepared=True):
    """Algorithmic HBM bytes of each stage for the whole batch: operands read
    once, results written once.  With the weights prepared (pkm_prepare) the
    exponent pass reads x alone."""
    B, D, H, n, k = wl.B, wl.D, wl.H, wl.n, wl.k
    work = per_token_work(wl)
    return {
        "query_gemm": 4 * (B * D + H * D * D + 4 * H * D + B * H * D),
        "score_gemm": 4 * (B * H * D + H * n * D + B * H * 2 * n),
        # folded: x and the folded matrix (as pieces) read, the scores written
        "folded_gemm": 4 * (B * D + 2 * H * n * D + 2 * H * n + B * H * 2 * n),
        "select": work["select_bytes"] * B,
        "gather": work["gather_bytes"] * B + B * H * k * 8 + B * D * 4,
        # fused: read the scores, write the selection, read the rows, write out
        "select_gather": (work["select_bytes"] + work["gather_bytes"]) * B + B * D * 4,
        # the row exponents: read x (and, unprepared, Wq and the subkeys) once
        "exponents": 4 * (B * D + (0 if prepared else H * D * D + H * n * D)),
    }


def end_to_end(wl, ms):
    """Whole-step tokens/s against two bounds: the value gather alone at HBM
    peak, and the composite roofline sum over stages of max(flop / MFMA peak,
    bytes / HBM peak), with the method's own stages (projection, scoring,
    selection and gather), whichever form the step runs them in."""
    work = per_token_work(wl)
    nbytes = stage_bytes(wl)
    flops = {"query_gemm": work["query_flop"] * wl.B, "score_gemm": work["score_flop"] * wl.B}
    flops.update({"select_gather": 0.0} if fused(wl) else {"select": 0.0, "gather": 0.0})
    ideal = sum(max(flops[s] / (GEMM_PEAK_TFLOPS * 1e12), nbytes[s] / (HBM_PEAK_GBS * 1e9)) for s in flops)
    hbm_only = work["gather_bytes"] * wl.B / (HBM_PEAK_GBS * 1e9)
    value = wl.B / (ms * 1e-3)
    return {"hbm_roofline_tokens_per_s": round(wl.B / hbm_only, 1), "hbm_frac": round(value * hbm_only / wl.B, 4),
            "composite_roofline_tokens_per_s": round(wl.B / ideal, 1),
            "composite_frac": round(value * ideal / wl.B, 4), "composite_ideal_us": round(ideal * 1e6, 2)}


WARM_SECONDS = 1.0   # least warm-up wall time before any timed call
WARM_MAX_SECONDS = 10.0
WARM_SETTLE = 0.02   # warm-up ends once two successive medians agree this well


def warm_up(torch, fn, warmup):
    """At least `warmup` calls and WARM_SECONDS of calls, then calls in
    rounds of 10 until two successive rounds' median call times agree
    within WARM_SETTLE (clocks and caches settled), at most WARM_MAX_SECONDS.
    Returns the number of calls made."""
    calls, t0 = 0, time.perf_counter()
    for _ in range(warmup):
        fn()
        calls += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < WARM_SECONDS:
        fn()
        calls += 1
        torch.cuda.synchronize()
    prev = None
    while time.perf_counter() - t0 < WARM_MAX_SECONDS:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
        ev[0].record()
        for i in range(10):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        calls += 10
        med = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(10)]))
        if prev is not None and abs(med - prev) <= WARM_SETTLE * prev:
            break
        prev = med
    return calls


def timed_steps(torch, fn, steps, warmup, stats=None):
    """Median ms per call of fn over `steps` calls, each bracketed by its own
    pair of events on the current stream (the stream the library launches
    on), after warm_up(); the calls are enqueued back to back and the
    device is synchronised before and after them.  With stats (a dict),
    also records the mean, min, max and the warm-up call count."""
    calls = warm_up(torch, fn, warmup)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    if stats is not None:
        stats.update(mean_ms=round(float(t.mean()), 4), min_ms=round(float(t.min()), 4),
                     max_ms=round(float(t.max()), 4), warmup_calls=calls,
                     total_ms=round(float(ev[0].elapsed_time(ev[steps])), 4))
    return float(np.median(t))


def kernel_times(torch, mem, P, xt, steps, warmup, wl, folded=False):
    """Median ms of each of the forward's own launches (pkm_forward_stage:
    the row exponents, the projection, the scoring, the selection with the
    gather), and of the stand-alone select and gather on the same scores.

    Each launch is timed by difference: an event pair brackets a block of
    launches (the forward's stages 0..s, or nothing, select, select then
    gather), every block runs once per iteration, and a launch's time is
    its block's time minus that of the block without it, taken within the
    iteration and then the median over iterations.  The events' own cost
    cancels, and each forward stage runs right after the one it follows in
    the forward.  (With a chunked forward the projection and scoring are
    timed through the single-step calls instead, which each compute their
    own row exponents.)"""
    B = xt.shape[0]
    q = torch.empty((B, mem.heads, mem.dim), dtype=torch.float32, device=xt.device)
    s = torch.empty((B, mem.heads, 2, mem.n_keys), dtype=torch.float32, device=xt.device)
    idx = torch.empty((B, mem.heads, mem.k), dtype=torch.int32, device=xt.device)
    w = torch.empty((B, mem.heads, mem.k), dtype=torch.float32, device=xt.device)
    idx2, w2 = torch.empty_like(idx), torch.empty_like(w)
    out = torch.empty((B, mem.dim), dtype=torch.float32, device=xt.device)
    out2 = torch.empty_like(out)
    mem.score(P, mem.query(P, xt, q), s)
    mem.select(s, idx2, w2)
    last = "select_gather" if fused(wl) else "select_and_gather"
    if mem.cfg.max_batch >= B and folded:
        # folded: stage 1 is a1-a3 as one contraction, stage 2 launches nothing
        fwd = [lambda st=st: mem.forward_stage(P, xt, st, out, idx, w) for st in (0, 1, 3)]
        fwd_names = ["exponents", "folded_gemm", last]
    elif mem.cfg.max_batch >= B:
        fwd = [lambda st=st: mem.forward_stage(P, xt, st, out, idx, w) for st in range(4)]
        fwd_names = ["exponents", "query_gemm", "score_gemm", last]
    else:
        fwd = [lambda: mem.query(P, xt, q), lambda: mem.score(P, q, s)]
        fwd_names = ["query_gemm", "score_gemm"]
    single = [lambda: mem.select(s, idx2, w2), lambda: mem.gather(P, idx2, w2, out2)]
    # blocks[0] is empty; forward stage j is blocks[j + 1] minus blocks[j];
    # select is the block after the forward's minus the empty one, gather
    # the next minus that
    blocks = [[]] + [fwd[:j + 1] for j in range(len(fwd))] + [single[:1], single]
    pairs = [(j + 1, j) for j in range(len(fwd))] + [(len(fwd) + 1, 0), (len(fwd) + 2, len(fwd) + 1)]
    names = fwd_names + ["select", "gather"]
    if folded:
        # the unfolded scoring from q^ on its own (its own exponent pass
        # included), for the comparison with the flat search
        blocks.append([lambda: mem.score(P, q, s)])
        pairs.append((len(blocks) - 1, 0))
        names.append("score_gemm_unfolded")

    def run(block):
        for f in block:
            f()

    warm_up(torch, lambda: [run(b) for b in blocks], warmup)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in blocks]
          for _ in range(steps)]
    for it in range(steps):
        for b, (e0, e1) in zip(blocks, ev[it]):
            e0.record()
            run(b)
            e1.record()
    torch.cuda.synchronize()
    t = [[e0.elapsed_time(e1) for e0, e1 in ev[it]] for it in range(steps)]
    return {nm: float(np.median([t[it][hi] - t[it][lo] for it in range(steps)]))
            for nm, (hi, lo) in zip(names, pairs)}


def gather_uniform_ms(torch, mem, P, wl, steps, warmup):
    """The gather alone on uniformly random rows (no pipeline locality)."""
    rows, wts = synthetic.uniform_rows(wl, 1, wl.B, wl.H * wl.k)
    idx = torch.from_numpy(rows).cuda()
    w = torch.from_numpy(wts).cuda()
    out = torch.empty((wl.B, wl.D), dtype=torch.float32, device="cuda")
    return timed_steps(torch, lambda: mem.gather(P, idx, w, out), steps, warmup)


def hbm_measured(torch, mem, P, wl, steps, warmup, mib=1024):
    """Streaming references on this machine: torch's device copy of a tensor far
    larger than the caches (read + write bytes), and the gather kernel itself
    on sequential rows (every row read once, in order: the same kernel
    without the random access)."""
    n = mib << 18
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    copy_ms = timed_steps(torch, lambda: b.copy_(a), steps, warmup)
    del a, b
    R = wl.H * wl.k
    rows = (torch.arange(wl.B * R, dtype=torch.int64, device="cuda") % wl.N).to(torch.int32).reshape(wl.B, R)
    w = torch.full((wl.B, R), 1.0 / R, dtype=torch.float32, device="cuda")
    out = torch.empty((wl.B, wl.D), dtype=torch.float32, device="cuda")
    seq_ms = timed_steps(torch, lambda: mem.gather(P, rows, w, out), steps, warmup)
    gathered = per_token_work(wl)["gather_bytes"] * wl.B
    return {"torch_copy_gbs": round(2 * n * 4 / (copy_ms * 1e-3) / 1e9, 1),
            "gather_sequential_rows_gbs": round(gathered / (seq_ms * 1e-3) / 1e9, 1),
            "sample": f"torch copy of {mib} MiB fp32; gather of rows 0..B*H*k-1 in order"}


def flat_vs_product(torch, pk, wl, P, xt, kt, tokens=64, steps=5, warmup=2):
    """The comparison the product keys exist for, measured: the brute-force
    search (every one of the N concatenated keys scored by a D-long dot
    product, exact top-k) against the product search (2 n half-key scores,
    per-half top-k, k^2 candidates), both from the same q^ of `tokens` tokens."""
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=tokens)
    q = mem.query(P, xt[:tokens].contiguous())
    ws = torch.empty(mem.flat_workspace_bytes(tokens), dtype=torch.uint8, device="cuda")
    fidx = torch.empty((tokens, wl.H, wl.k), dtype=torch.int32, device="cuda")
    ftop = torch.empty((tokens, wl.H, wl.k), dtype=torch.float32, device="cuda")
    s = torch.empty((tokens, wl.H, 2, wl.n), dtype=torch.float32, device="cuda")
    pidx = torch.empty_like(fidx)
    pw = torch.empty_like(ftop)
    flat_ms = timed_steps(torch, lambda: mem.flat_search(P, q, fidx, ftop, ws), steps, warmup)
    prod_ms = timed_steps(torch, lambda: (mem.score(P, q, s), mem.select(s, pidx, pw)), 50, 10)
    same = bool((torch.sort(fidx, -1).values == torch.sort(pidx, -1).values).all().item())
    flat_flop = 2.0 * tokens * wl.H * wl.N * wl.D
    full_batch_us = (kt.get("score_gemm", kt.get("score_gemm_unfolded")) + kt["select"]) * 1e3 / wl.B
    return {"tokens": tokens, "flat_ms": round(flat_ms, 4), "product_ms": round(prod_ms, 4),
            "speedup_same_tokens": round(flat_ms / prod_ms, 1),
            "flat_us_per_token": round(flat_ms * 1e3 / tokens, 3),
            "product_us_per_token_full_batch": round(full_batch_us, 5),
            "speedup_per_token": round(flat_ms * 1e3 / tokens / full_batch_us, 1),
            "flat_gemm_tflops": round(flat_flop / (flat_ms * 1e-3) / 1e12, 2),
            "flat_gemm_frac": round(flat_flop / (flat_ms * 1e-3) / 1e12 / GEMM_PEAK_TFLOPS, 4),
            "same_winner_sets": same,
            "key_scores_per_token_head": {"flat": wl.N, "product": 2 * wl.n}, "candidates_per_token_head": wl.k ** 2}


def backward_step(torch, mem, wl, P, xt, idx, wts, dout, fwd_ms, steps, warmup):
    """The gradients of a loss through the same batch (pkm_backward): every
    parameter gradient, dx and the dense fp32 value-table gradient (and
    again with the value gradient's sparse form).  Against a composite
    ideal: the three contractions at the MFMA ceiling plus the step's
    algorithmic HBM bytes at 8 TB/s."""
    grads = {"dx": (wl.B, wl.D), "dwq": (wl.H, wl.D, wl.D), "dbn_gamma": (wl.H, wl.D), "dbn_beta": (wl.H, wl.D),
             "dsubkeys": (wl.H, 2, wl.n, wl.D // 2), "dvalues": (wl.N, wl.D)}
    grads = {name: torch.zeros(shape, dtype=torch.float32, device="cuda") for name, shape in grads.items()}
    ws = torch.empty(mem.backward_workspace_bytes(), dtype=torch.uint8, device="cuda")
    ms = timed_steps(torch, lambda: mem.backward(P, xt, idx, wts, dout, grads, ws), steps, warmup)
    # the same step with the value gradient in its sparse form (touched rows only, written once)
    cap = min(wl.N, wl.B * wl.H * wl.k)
    sparse = {name: t for name, t in grads.items() if name != "dvalues"}
    sparse.update({"dvalues_rows": torch.empty(cap, dtype=torch.int32, device="cuda"),
                   "dvalues_sparse": torch.empty((cap, wl.D), dtype=torch.float32, device="cuda"),
                   "dvalues_count": torch.empty(1, dtype=torch.int64, device="cuda")})
    sparse_ms = timed_steps(torch, lambda: mem.backward(P, xt, idx, wts, dout, sparse, ws), steps, warmup)
    touched = int(sparse["dvalues_count"].item())
    del sparse
    # the same step with training-mode BN (statistics of this batch, running statistics updated)
    out = torch.empty((wl.B, wl.D), dtype=torch.float32, device="cuda")
    running = (torch.zeros((wl.H, wl.D), device="cuda"), torch.ones((wl.H, wl.D), device="cuda"))
    stats = {}

    def fwd_bs():
        stats["r"] = mem.forward_batch_stats(P, xt, out, idx, wts, running=running)

    fwd_bs_ms = timed_steps(torch, fwd_bs, steps, warmup)
    bm, bv = stats["r"][3], stats["r"][4]
    bwd_bs_ms = timed_steps(torch, lambda: mem.backward(P, xt, idx, wts, dout, grads, ws, batch_stats=(bm, bv)),
                            steps, warmup)
    # training with running statistics: the forward that also keeps the
    # projection before BN, and the backward that takes it instead of
    # computing it again
    q = torch.empty((wl.B, wl.H, wl.D), dtype=torch.float32, device="cuda")
    fwd_q_ms = timed_steps(torch, lambda: mem.forward_train(P, xt, out, idx, wts, q), steps, warmup)
    bwd_q_ms = timed_steps(torch, lambda: mem.backward(P, xt, idx, wts, dout, grads, ws, q=q), steps, warmup)
    # GEMM work of the backward: the recomputed q, dWq and dx (2 B H D^2 each)
    flop = 2.0 * wl.B * wl.H * wl.D * wl.D * 3
    B, H, D, n = wl.B, wl.H, wl.D, wl.n
    hbm = (per_token_work(wl)["gather_bytes"] * B  # the selected value rows, for dout . V[row]
           + 2 * touched * D * 4                   # the dense value gradient's touched rows, read and written
           + 2 * H * n * D * 4                     # the subkey gradient, read and written
           + 2 * H * D * D * 4                     # dWq, read and written
           + 2 * B * H * D * 4                     # q recomputed: written, read back
           + 3 * B * D * 4)                        # x and dout read, dx written
    ideal_us = (flop / (GEMM_PEAK_TFLOPS * 1e12) + hbm / (HBM_PEAK_GBS * 1e9)) * 1e6
    # with q given: two contractions, q read once instead of written and read
    ideal_q_us = (flop * 2 / 3 / (GEMM_PEAK_TFLOPS * 1e12) + (hbm - B * H * D * 4) / (HBM_PEAK_GBS * 1e9)) * 1e6
    return {"ms": round(ms, 4), "tokens_per_s": round(wl.B / (ms * 1e-3), 1),
            "composite_ideal_us": round(ideal_us, 1), "composite_frac": round(ideal_us * 1e-3 / ms, 4),
            "hbm_bytes": int(hbm), "gemm_us_at_mfma_ceiling": round(flop / (GEMM_PEAK_TFLOPS * 1e12) * 1e6, 1),
            "forward_backward_tokens_per_s": round(wl.B / ((ms + fwd_ms) * 1e-3), 1),
            "sparse_value_grad_ms": round(sparse_ms, 4), "rows_touched": touched,
            "batch_stats_forward_ms": round(fwd_bs_ms, 4), "batch_stats_backward_ms": round(bwd_bs_ms, 4),
            "batch_stats_forward_backward_tokens_per_s": round(wl.B / ((fwd_bs_ms + bwd_bs_ms) * 1e-3), 1),
            "forward_train_ms": round(fwd_q_ms, 4), "with_saved_q_ms": round(bwd_q_ms, 4),
            "with_saved_q_composite_frac": round(ideal_q_us * 1e-3 / bwd_q_ms, 4),
            "forward_backward_saved_q_tokens_per_s": round(wl.B / ((fwd_q_ms + bwd_q_ms) * 1e-3), 1),
            "gemm_flop": flop, "gemm_tflops_if_all_time": round(flop / (ms * 1e-3) / 1e12, 2),
            "workspace_bytes": mem.backward_workspace_bytes()}


def _ranges(cpus):
    """[0, 1, 2, 5] -> "0-2,5"."""
    out, cpus = [], sorted(cpus)
    i = 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(str(cpus[i]) if i == j else f"{cpus[i]}-{cpus[j]}")
        i = j + 1
    return ",".join(out)


def host_cores():
    """The host's logical CPUs, this process's affinity mask, and the CPU
    time its cgroup allows (cpu.max), if any."""
    aff = sorted(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()
        if q != "max":
            quota = int(q) / int(period)
    except (OSError, ValueError):
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity_count": len(aff), "affinity_mask": _ranges(aff),
            "cgroup_cpu_quota": quota}


def cpu_baseline(wl, params, x, seconds=10.0):
    """The fp64 oracle on every host core this process may use (its
    affinity mask, or the whole CPUs its cgroup quota allows if fewer) over
    a bounded sample of the tokens."""
    import oracle

    hc = host_cores()
    cores = hc["affinity_count"]
    if hc["cgroup_cpu_quota"]:
        cores = max(1, min(cores, int(hc["cgroup_cpu_quota"])))
    model = oracle.Model.from_params(params, wl.k, wl.table)
    probe = min(x.shape[0], 2 * cores)
    t0 = time.perf_counter()
    oracle.run(model, x[:probe], want=("out",), nthreads=cores)
    rate = probe / max(time.perf_counter() - t0, 1e-9)
    sample = int(min(x.shape[0], max(cores, rate * seconds)))
    # when the whole batch takes less than the time budget, pass over it
    # again until the budget is spent (a steadier figure)
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.run(model, x[:sample], want=("out",), nthreads=cores)
        passes += 1
        dt = time.perf_counter() - t0
        if sample < x.shape[0] or dt >= 0.8 * seconds:
            break
    # one core, on a sample a tenth of the time budget long
    one = max(1, min(x.shape[0], int(passes * sample / dt / cores * seconds / 10)))
    t0 = time.perf_counter()
    oracle.run(model, x[:one], want=("out",), nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": passes * sample / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "host": hc,
            "sample": f"{passes} pass(es) over the first {sample} of the {wl.B} tokens of the {wl.name} workload, "
                      f"full lookup in fp64, {dt:.1f} s wall on {cores} threads",
            "single_core_value": one / dt1,
            "single_core_sample": f"first {one} tokens on 1 thread, {dt1:.1f} s wall"}


def cpu_backward_baseline(wl, params, x, dout, seconds=10.0):
    """The fp64 oracle's backward (every gradient, the dense value gradient
    over all N rows included) on the same cores as cpu_baseline, over the
    first tokens of the batch: a one-token call measures the part that does
    not grow with the tokens (the value gradient's N x D fp64 array, zeroed
    per call), a small one the rate per token, and the sample is sized to
    the time budget from the two."""
    import oracle

    hc = host_cores()
    cores = hc["affinity_count"]
    if hc["cgroup_cpu_quota"]:
        cores = max(1, min(cores, int(hc["cgroup_cpu_quota"])))
    model = oracle.Model.from_params(params, wl.k, wl.table)
    t0 = time.perf_counter()
    oracle.backward(model, x[:1], dout[:1], nthreads=cores)
    fixed = time.perf_counter() - t0
    probe = min(x.shape[0], 2 * cores)
    t0 = time.perf_counter()
    oracle.backward(model, x[:probe], dout[:probe], nthreads=cores)
    per_token = max(time.perf_counter() - t0 - fixed, 1e-6) / probe
    sample = int(min(x.shape[0], max(probe, (seconds - fixed) / per_token)))
    t0 = time.perf_counter()
    oracle.backward(model, x[:sample], dout[:sample], nthreads=cores)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {sample} of the {wl.B} tokens of the {wl.name} workload, every gradient in fp64 "
                      f"(the dense value gradient over all {wl.N} rows, {wl.N * wl.D * 8 / 2**30:.1f} GiB, "
                      f"{fixed:.1f} s of each call), {dt:.1f} s wall on {cores} threads"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="default", choices=sorted(synthetic.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target wall time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--max-batch", type=int, default=0, help="tokens per internal chunk (0: the whole batch)")
    ap.add_argument("--no-flat", action="store_true", help="skip the flat (brute-force) search comparison")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward (gradient) timing")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the lookup is data-parallel "
              "over tokens with a replicated table, so N GPUs would run N independent copies).", file=sys.stderr)
        sys.exit(2)

    import torch

    import product_key_memory_amd as pk

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 18
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4}))
        return

    wl = synthetic.WORKLOADS[args.workload]
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)
    P = pk.params_to_device(params, wl.table, "cuda")
    xt = torch.from_numpy(x).cuda()
    max_batch = args.max_batch or wl.B
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=max_batch)
    out = torch.empty((wl.B, wl.D), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.B, wl.H, wl.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((wl.B, wl.H, wl.k), dtype=torch.float32, device="cuda")

    # The weights as they come (split in every call), then prepared once
    # (pkm_prepare: Wq and the subkeys kept as the contractions read them, as
    # a server does once when it loads the layer); the step is timed with the
    # prepared weights, the same bits either way.
    # The weights as they come (split in every call); prepared once as fp16
    # pieces (bit for bit the same step); then, where n_keys <= D, folded
    # (projection, batch-norm with its running statistics and subkeys as one
    # matrix per half of a head), which is what a server does once when it
    # loads the layer and what the step is timed with.
    folded = wl.n <= wl.D
    unprep_stats, split_stats = {}, {}
    unprep_ms = timed_steps(torch, lambda: mem.forward(P, xt, out, idx, wts), args.steps, args.warmup, unprep_stats)
    split_prep_ms = timed_steps(torch, lambda: mem.prepare(P, "split"), 20, 5)
    mem.prepare(P, "split")
    split_ms = timed_steps(torch, lambda: mem.forward(P, xt, out, idx, wts), args.steps, args.warmup, split_stats)
    form = "fold" if folded else "split"
    prep_ms = timed_steps(torch, lambda: mem.prepare(P, form), 5, 2)
    mem.prepare(P, form)
    step_stats = {}
    ms = timed_steps(torch, lambda: mem.forward(P, xt, out, idx, wts), args.steps, args.warmup, step_stats)
    rows = idx.cpu().numpy().ravel()
    distinct = float(np.unique(rows).size) / rows.size
    kt = kernel_times(torch, mem, P, xt, args.steps, args.warmup, wl, folded)
    g_uniform_ms = gather_uniform_ms(torch, mem, P, wl, args.steps, args.warmup)
    hbm = hbm_measured(torch, mem, P, wl, args.steps, args.warmup)

    work = per_token_work(wl)
    B = wl.B
    rl = {
        name: ("mfma", work[flop] * B / (kt[name] * 1e-3) / 1e12, GEMM_PEAK_TFLOPS, "TFLOP/s")
        for name, flop in (("query_gemm", "query_flop"), ("score_gemm", "score_flop"), ("folded_gemm", "folded_flop"))
        if name in kt
    }
    rl.update({
        "select": ("hbm", work["select_bytes"] * B / (kt["select"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
        "gather": ("hbm", work["gather_bytes"] * B / (kt["gather"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
    })
    if "select_gather" in kt:
        rl["select_gather"] = ("hbm", (work["select_bytes"] + work["gather_bytes"]) * B /
                               (kt["select_gather"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")
    if "exponents" in kt:
        rl["exponents"] = ("hbm", stage_bytes(wl)["exponents"] / (kt["exponents"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")
    # the forward's own kernels; the dominant one is the headline roofline
    forward_kernels = ((["exponents"] if "exponents" in kt else []) +
                       (["folded_gemm"] if "folded_gemm" in kt else ["query_gemm", "score_gemm"]) +
                       (["select_gather"] if "select_gather" in kt else ["select", "gather"]))
    dominant = max(forward_kernels, key=kt.get)

    def roof(name):
        bound, achieved, peak, unit = rl[name]
        return {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(wl.name, name),
                "median_ms": round(kt[name], 4)}

    line = {
        "metric": METRIC,
        "value": round(B / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (fp16x3 split)",
        "timing": dict(step_stats, statistic="median of per-step event pairs"),
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": B, "dim": wl.D, "heads": wl.H, "n_keys": wl.n,
                   "rows": wl.N, "k": wl.k, "value_table": wl.table, "seed": 0, "max_batch": max_batch,
                   "weights_prepared": form},
        "roofline": roof(dominant),
        "gather_roofline": roof("gather"),
        "hbm_measured": dict(hbm, gather_frac_of_sequential=round(rl["gather"][1] / hbm["gather_sequential_rows_gbs"],
                                                                    4)),
        "gather_uniform_rows_gbs": round(work["gather_bytes"] * B / (g_uniform_ms * 1e-3) / 1e9, 1),
        "gathered_rows_distinct_frac": round(distinct, 4),
        "end_to_end": end_to_end(wl, ms),
        "prepared_weights": {"form": form, "prepare_ms": round(prep_ms, 4),
                             "unprepared_ms_per_step": round(unprep_ms, 4),
                             "unprepared_tokens_per_s": round(B / (unprep_ms * 1e-3), 1),
                             "unprepared_timing": unprep_stats,
                             "split_prepare_ms": round(split_prep_ms, 4), "split_ms_per_step": round(split_ms, 4),
                             "split_tokens_per_s": round(B / (split_ms * 1e-3), 1), "split_timing": split_stats,
                             "note": "value is timed after pkm_prepare once: 'fold' (n_keys <= D) runs a1-a3 as one "
                                     "contraction of x with the folded projection, running-statistics batch-norm "
                                     "and subkeys (fp32-accurate, checked against the oracle); 'split' keeps Wq and "
                                     "the subkeys as fp16 pieces (bit for bit the unprepared step)"},
        "kernels_ms": {nm: round(v, 4) for nm, v in kt.items()},
        "forward_kernels": forward_kernels,
        "kernel_rooflines": {nm: {"achieved": round(rl[nm][1], 2), "unit": rl[nm][3],
                                  "frac": round(rl[nm][1] / rl[nm][2], 4)} for nm in rl},
    }
    if not args.no_flat:
        line["flat_vs_product"] = flat_vs_product(torch, pk, wl, P, xt, kt)
    if not args.no_backward:
        dout = torch.randn((wl.B, wl.D), dtype=torch.float32, device="cuda",
                           generator=torch.Generator("cuda").manual_seed(1))
        line["backward"] = backward_step(torch, mem, wl, P, xt, idx, wts, dout, ms, max(5, args.steps // 5),
                                         max(2, args.warmup // 5))
        if not args.no_cpu_baseline:
            line["backward"]["cpu_baseline"] = cpu_backward_baseline(wl, params, x, dout.cpu().numpy(),
                                                                     args.cpu_seconds)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, params, x, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
