"""Throughput of the Avey-B ranker + dynamic contextualizer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long] [--no-cpu-baseline]

One step is one pass of the whole path over one batch of synthetic input already resident in
HBM: all-pairs MaxSim, top-k with divide-by-max, weighted gather + (k+1)S -> S compression,
and the dynamic layer's row-normalised cosine mixing. The default workload is the 32K-token
one (batch 2, N = 32768, d = 768, S = 256, k = 3, tail width 1536).

Prints one JSON line: tokens/s over the timed steps, per-kernel times from HIP events on the
launch stream, the MaxSim kernel against the bf16 MFMA roofline, the ceilings measured on the
device (matrix-core and copy probes, the vendor GEMM on the same contraction shapes), and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "tokens/sec for ranker+dynamic layer at N=32K; MaxSim MFMA util %"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attention_free_long_amd", "csrc")

# HBM traffic of one launch of the dominant kernel, from two rocprofv3 --pmc passes (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch, averaged over the dispatches of the run) over this bench on
# the named workload, each scaled by what the same counter reads for a plain 1 GiB device copy
# (FETCH_SIZE read 524302 KiB for 1048576 KiB moved: x1.99995; WRITE_SIZE read 1048576 KiB: x1.0).
# Keyed by the digest of the kernel's sources: once they change the figures no longer apply and
# traffic is reported as null until the counters are taken again.
TRAFFIC = {
    "maxsim": {
        "sources": ("maxsim_bf16.hip", "avey_common.h", "../build.py"),
        "measured": {
            ("4c61ddd2265b4d10", "long"): {"fetch_kib": 1189581.2, "fetch_scale": 1.99995,
                                           "write_kib": 236.8, "write_scale": 1.0},
            ("4c61ddd2265b4d10", "extreme"): {"fetch_kib": 5168265.3, "fetch_scale": 1.99995,
                                              "write_kib": 1147.5, "write_scale": 1.0},
        },
    },
}


def sources_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_bytes(kernel: str, workload: str):
    entry = TRAFFIC[kernel]
    m = entry["measured"].get((sources_digest(entry["sources"]), workload))
    if m is None:
        return None
    return int(round((m["fetch_kib"] * m["fetch_scale"] + m["write_kib"] * m["write_scale"]) * 1024))


def algorithmic(cfg):
    """Algorithmic work per launch of each kernel (FLOPs, bytes)."""
    B, N, d, S, k, m_t = cfg.B, cfg.N, cfg.d, cfg.S, cfg.k, cfg.m_t
    n_s = cfg.n_s
    eb = 2 if cfg.dtype == "bf16" else 4
    pairs = B * n_s * (n_s - 1) // 2
    return {
        # read x once, write its normalised, padded copy once
        "prepare": {"flop": 3.0 * B * N * d, "bytes": B * N * d * eb + B * n_s * S * d * eb},
        # one S x S x d tile per unordered split pair serves both directions; reads the
        # normalised copy once
        "maxsim": {"flop": 2.0 * S * S * d * pairs, "bytes": B * n_s * S * d * eb},
        "topk": {"flop": 0.0, "bytes": B * n_s * n_s * 4 + 2 * B * n_s * k * 4},
        # read X_i and k retrieved splits, write Xhat_i; P once
        "compress": {"flop": 2.0 * B * n_s * S * d * (k + 1) * S,
                     "bytes": (k + 2) * B * N * d * eb + S * (k + 1) * S * eb},
        # read the tail once, write the output once
        "dyn": {"flop": 4.0 * B * n_s * S * S * m_t, "bytes": 2 * B * N * m_t * eb},
        # contextualizer layers outside the step: the tail in, the output out, V and the bias once
        "static_layer": {"flop": 2.0 * B * n_s * S * S * m_t, "bytes": 2 * B * N * m_t * eb + S * S * eb + S * 4},
        "dyn_layer": {"flop": 4.0 * B * n_s * S * S * m_t, "bytes": 2 * B * N * m_t * eb + S * 4},
        # enricher X [M, d] -> Z [M, m]; fuser [Z_h || c] [M, m] -> Y [M, d] (+ X); weights once
        "enrich": {"flop": 2.0 * B * N * d * cfg.m,
                   "bytes": B * N * (d + cfg.m) * eb + d * cfg.m * eb + cfg.m * 4},
        "fuse": {"flop": 2.0 * B * N * cfg.m * d,
                 "bytes": B * N * (cfg.m + 2 * d) * eb + cfg.m * d * eb},
    }


def pipeline_roofline(cfg, value: float, peak_tflops: float) -> dict:
    """The step against the rooflines of the hot path's own work (all-pairs MaxSim, gather +
    compress, dynamic layer; top-k's few KiB are left out): tokens/s the step would reach if every
    kernel ran at its bound, max(FLOP / MFMA peak, bytes / HBM peak) per kernel, and the two
    single-resource figures B N peak / sum(FLOP) and B N BW / sum(bytes). The normalised operand
    copy of the explicit-workspace ranker path is an implementation choice, not work of the method:
    it is not counted."""
    work = algorithmic(cfg)
    names = ("maxsim", "compress", "dyn")
    flop = sum(work[n]["flop"] for n in names)
    byts = sum(work[n]["bytes"] for n in names)
    t_roof = sum(max(work[n]["flop"] / (peak_tflops * 1e12), work[n]["bytes"] / (PEAK_HBM_GBS * 1e9))
                 for n in names)
    tokens = cfg.B * cfg.N
    roof = tokens / t_roof
    mfma = tokens * peak_tflops * 1e12 / flop
    hbm = tokens * PEAK_HBM_GBS * 1e9 / byts
    return {"tokens_per_s": round(roof, 1), "frac": round(value / roof, 4),
            "mfma_tokens_per_s": round(mfma, 1), "mfma_frac": round(value / mfma, 4),
            "hbm_tokens_per_s": round(hbm, 1), "hbm_frac": round(value / hbm, 4),
            "flop_per_step": flop, "bytes_per_step": byts,
            "basis": "sum over maxsim, compress, dyn of max(FLOP/peak, bytes/8 TB/s)"}


def gap_histogram(scores, k: int, edges=(0.0, 1e-6, 1e-4, 1e-3, 1e-2, 1e-1)) -> dict:
    """Histogram of the relative gap between the k-th and (k+1)-th best score of every row of the
    score matrix the GPU computed (the diagonal left out): how close the workload's top-k
    selections are to a tie. Counts per bin [e_i, e_{i+1}), the last bin open-ended."""
    import numpy as np
    s = scores.reshape(-1, scores.shape[-1]).astype(np.float64)
    s = -np.sort(-s, axis=1)   # descending; the diagonal's -inf comes last
    kth, nxt = s[:, k - 1], s[:, k]
    gap = (kth - nxt) / np.abs(kth)
    out = {}
    for lo, hi in zip(edges, list(edges[1:]) + [float("inf")]):
        out[f"[{lo:g},{hi:g})"] = int(((gap >= lo) & (gap < hi)).sum())
    return {"rows": int(len(gap)), "bins": out, "min_gap": float(gap.min()),
            "source": "the GPU's own score matrix of this run"}


def _oracle_worker(args):
    """One process of the CPU baseline: whole target splits of its share, in order, until the
    deadline; the float64 oracle as it stands, with single-threaded BLAS."""
    shard, deadline = args
    from threadpoolctl import threadpool_limits
    from oracle import avey_oracle as O
    inp, xs, Ps = _CPU_STATE
    cfg = inp.cfg
    done = tok = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        for b, i in shard:
            if time.time() >= deadline:
                break
            row = O.score_row(xs[b], cfg.S, i)
            idx, w, _, _ = O.top_k(row, i, cfg.k)
            O.compress_split(xs[b], cfg.S, idx, w, Ps, i)
            rows = slice(i * cfg.S, min((i + 1) * cfg.S, cfg.N))
            O.dyn_context_split(inp.z_tail_f64(b, rows), cfg.S, cfg.eps, 0)
            done += 1
            tok += rows.stop - rows.start
    return done, tok, time.perf_counter() - t0


_CPU_STATE = None


def cpu_baseline(inp, budget_s: float = 12.0):
    """The float64 oracle, as it stands, on whole target splits of the same workload (full score
    row, top-k, compression and dynamic layer of each split), spread over one single-threaded
    process per host core of this process's CPU share (at most 16) until the time budget is
    spent. Runs before anything touches the GPU: the worker processes are forked."""
    import multiprocessing as mp
    global _CPU_STATE
    cfg = inp.cfg
    n_s = cfg.n_s
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    stride = max(1, n_s // 16)
    order = [(b, i) for r in range(stride) for i in range(r, n_s, stride) for b in range(cfg.B)]
    _CPU_STATE = (inp, {b: inp.x_f64(b) for b in range(cfg.B)}, inp.P_f64())
    shards = [order[p::workers] for p in range(workers)]
    t0 = time.perf_counter()
    deadline = time.time() + budget_s
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_oracle_worker, [(sh, deadline) for sh in shards])
    wall = time.perf_counter() - t0
    _CPU_STATE = None
    done = sum(r[0] for r in res)
    tok = sum(r[1] for r in res)
    return {
        "value": tok / wall,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{done} of {cfg.B * n_s} target splits of the {cfg.name} workload (full score row, "
                  f"top-k, compression and dynamic layer per split) in {wall:.1f} s over {workers} "
                  f"single-threaded processes, float64 numpy",
    }


def time_layers(A, cfg, inp, z_tail, work, steps: int, peak: float):
    """The rest of a neural-processor layer on the same workload, timed apart from the step with
    HIP events on the launch stream (not part of the step's throughput): the static and dynamic
    contextualizer layers (bias and ReLU) on the tail, the dynamic layer with each of the other
    row normalisations, the enricher X -> Z (d -> m) and the fuser [Z_h || c] -> Y (m -> d, with
    the residual)."""
    import numpy as np
    import torch
    from synth import layer_params
    V, bias = layer_params(inp)
    if cfg.dtype == "bf16":
        Vd = torch.from_numpy(np.ascontiguousarray(V).view(np.int16)).to("cuda").view(torch.bfloat16)
    else:
        Vd = torch.from_numpy(V).to("cuda")
    bd = torch.from_numpy(bias).to("cuda")
    out = torch.empty((cfg.B, cfg.N, cfg.m_t), device="cuda", dtype=z_tail.dtype)
    from synth import processor_params
    U, bU, Ow = processor_params(cfg, cfg.m, u_std=0.02, o_std=0.02, b_std=0.02)
    dev = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)) \
        if cfg.dtype == "bf16" else (lambda a: torch.from_numpy(a).to("cuda"))
    Ud, Od, bUd = dev(U), dev(Ow), torch.from_numpy(bU).to("cuda")
    x = dev(inp.x)
    zf = torch.empty((cfg.B, cfg.N, cfg.m), device="cuda", dtype=z_tail.dtype)
    y = torch.empty((cfg.B, cfg.N, cfg.d), device="cuda", dtype=z_tail.dtype)
    m_h = cfg.m - cfg.m_t
    calls = {
        "static_layer": lambda: A.avey_static_layer(z_tail, Vd, cfg.S, bd, "relu", out=out),
        "dyn_layer": lambda: A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "relu", out=out),
        # the row normalisations compared beside eq. 6: softmax, RMS, none
        "dyn_layer_softmax": lambda: A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "relu", out=out, norm="softmax"),
        "dyn_layer_rms": lambda: A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "relu", out=out, norm="rms"),
        "dyn_layer_none": lambda: A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "relu", out=out, norm="none"),
        "enrich": lambda: A.avey_enrich(x, Ud, bUd, out=zf),
        "fuse": lambda: A.avey_fuse(zf, m_h, out, Od, x, out=y),
    }
    res = {}
    for name, call in calls.items():
        wk = work[name.split("_softmax")[0].split("_rms")[0].split("_none")[0]]
        for _ in range(5):
            call()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for j in range(steps):
            call()
            ev[j + 1].record()
        torch.cuda.synchronize()
        t = float(np.mean([ev[j].elapsed_time(ev[j + 1]) for j in range(steps)])) * 1e-3
        res[name] = {"avg_us": round(t * 1e6, 3),
                     "hbm_frac": round(wk["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4),
                     "mfma_frac": round(wk["flop"] / t / 1e12 / peak, 4),
                     "launches": steps}
    return res


def time_compress_cold(call, work_bytes: float, reps: int = 10):
    """Gather + compress with a cold last-level cache: before each launch a 512 MiB scratch
    buffer is written on the same stream, which evicts X and P from the 256 MB MALL and the L2s,
    so the X reads come from HBM. Times are from HIP events around the compress call alone."""
    import numpy as np
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ts = []
    for r in range(reps + 2):
        scratch.fill_(r & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(e0.elapsed_time(e1) * 1e-3)
    del scratch
    t = float(np.median(ts))
    return {"median_us": round(t * 1e6, 3), "min_us": round(float(np.min(ts)) * 1e6, 3),
            "hbm_frac": round(work_bytes / t / 1e9 / PEAK_HBM_GBS, 4), "launches": reps,
            "flush": "512 MiB written before each launch"}


def measured_peaks(A, reps: int = 10):
    """The two ceilings measured on this device (include/avey_probe.h), medians of `reps` launches
    timed with HIP events: the bf16 matrix-core rate on register operands that stay fixed or
    change every iteration (as data streamed from memory does), and a 1 GiB device copy."""
    import numpy as np
    import torch

    def timed(call):
        for _ in range(3):
            call()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    iters = 2000
    flops = A.avey_probe_mfma_flops(iters)
    sink = A.avey_probe_mfma_bf16(1, False)
    fixed = flops / timed(lambda: A.avey_probe_mfma_bf16(iters, False, sink)) / 1e12
    changing = flops / timed(lambda: A.avey_probe_mfma_bf16(iters, True, sink)) / 1e12
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    copy_gbs = 2 * n / timed(lambda: A.avey_probe_copy(src, dst)) / 1e9
    del src, dst
    return {"mfma_bf16_tflops_fixed_operands": round(fixed, 1),
            "mfma_bf16_tflops_changing_operands": round(changing, 1),
            "copy_gbs": round(copy_gbs, 1),
            "method": f"avey_probe_mfma_bf16 ({iters} iterations, one 8-wave workgroup per CU) and "
                      f"avey_probe_copy (1 GiB, read + written), median of {reps} launches"}


def library_gemm_rates(cfg, reps: int = 10):
    """The vendor GEMM (hipBLASLt through torch.matmul, bf16 in and out, fp32 accumulation) on the
    contractions of this workload, as a calibration of what the matrix cores sustain here on plain
    GEMMs of the same shapes: MaxSim's all-pairs token product of one sequence ([N, d] x [d, N],
    every ordered pair, no max epilogue), the enricher ([B N, d] x [d, m]) and the fuser
    ([B N, m] x [m, d]). Medians of `reps` launches timed with HIP events; operands are contiguous
    N(0, 1) bf16."""
    import numpy as np
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    shapes = {"maxsim_all_pairs": (cfg.N, cfg.d, cfg.N), "enrich": (cfg.B * cfg.N, cfg.d, cfg.m),
              "fuse": (cfg.B * cfg.N, cfg.m, cfg.d)}
    out = {}
    for name, (M, K, N) in shapes.items():
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=g)
        c = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b, out=c)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(ts))
        tf = 2.0 * M * K * N / t / 1e12
        out[name] = {"shape_mkn": [M, K, N], "median_us": round(t * 1e6, 1), "tflops": round(tf, 1),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del a, b, c
    out["method"] = f"torch.matmul (hipBLASLt) bf16, median of {reps} launches"
    return out


def upload(cfg, inp):
    import numpy as np
    import torch

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    x, P, z = dev(inp.x), dev(inp.P), dev(inp.z)
    return x, P, z, z[..., inp.tail_col:]


def time_workload(A, cfg, inp, steps: int, warmup: int, peak: float):
    """Time `steps` steps of the hot path on one workload after `warmup` untimed ones. Every library
    call enqueues on torch's current stream, on which the events are recorded: each interval
    brackets exactly one call. Returns the measurements and the device tensors."""
    import numpy as np
    import torch

    x, P, z, z_tail = upload(cfg, inp)
    B, N, n_s, S, k = cfg.B, cfg.N, cfg.n_s, cfg.S, cfg.k
    dt = x.dtype
    scores = torch.empty((B, n_s, n_s), device="cuda", dtype=torch.float32)
    idx = torch.empty((B, n_s, k), device="cuda", dtype=torch.int32)
    w = torch.empty((B, n_s, k), device="cuda", dtype=torch.float32)
    xhat = torch.empty((B, N, cfg.d), device="cuda", dtype=dt)
    out = torch.empty((B, N, cfg.m_t), device="cuda", dtype=dt)
    # The ranker through its explicit-workspace path (the faster of the two; the workspace-free
    # avey_split_rank is timed beside it), then gather + compress and the dynamic layer
    ws = A.rank_workspace(x, S)
    names = ("prepare", "maxsim", "topk", "compress", "dyn")
    calls = (
        lambda: A.avey_maxsim_prepare(x, S, ws),
        lambda: A.avey_maxsim_scores(ws, x, S, scores),
        lambda: A.avey_topk_norm(scores, k, idx, w),
        lambda: A.avey_select_compress(x, idx, w, P, S, residual=True, out=xhat),
        lambda: A.avey_dyn_context(z_tail, S, cfg.eps, out=out),
    )

    def step(ev=None):
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record()
            call()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(events[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: [ev[j].elapsed_time(ev[j + 1]) * 1e-3 for ev in events] for j, n in enumerate(names)}
    work = algorithmic(cfg)
    kern = {}
    for n in names:
        t = float(np.mean(per[n]))
        e = {"avg_us": t * 1e6, "median_us": float(np.median(per[n])) * 1e6, "min_us": float(np.min(per[n])) * 1e6}
        if work[n]["flop"]:
            e["tflops"] = work[n]["flop"] / t / 1e12
        e["gbs"] = work[n]["bytes"] / t / 1e9
        kern[n] = {kk: round(v, 3) for kk, v in e.items()}
    value = B * N / (wall / steps)
    ms_t = kern["maxsim"]["avg_us"] * 1e-6
    comp_t = kern["compress"]["avg_us"] * 1e-6
    dyn_t = kern["dyn"]["avg_us"] * 1e-6
    res = {
        "value": value,
        "ms_per_step": wall / steps * 1e3,
        "maxsim_achieved_tflops": work["maxsim"]["flop"] / ms_t / 1e12,
        "compress_hbm_frac": round(work["compress"]["bytes"] / comp_t / 1e9 / PEAK_HBM_GBS, 4),
        "compress_mfma_frac": round(work["compress"]["flop"] / comp_t / 1e12 / peak, 4),
        "dyn_hbm_frac": round(work["dyn"]["bytes"] / dyn_t / 1e9 / PEAK_HBM_GBS, 4),
        "dyn_mfma_frac": round(work["dyn"]["flop"] / dyn_t / 1e12 / peak, 4),
        "kernels": kern,
        "compress_cold": time_compress_cold(calls[3], work["compress"]["bytes"]),
        "pipeline_roofline": pipeline_roofline(cfg, value, peak),
        "gap_histogram": gap_histogram(scores.cpu().numpy(), k),
    }
    res["compress_cold"]["mfma_frac"] = round(work["compress"]["flop"] / (res["compress_cold"]["median_us"] * 1e-6)
                                              / 1e12 / peak, 4)
    res["rank_workspace_free"] = time_workspace_free(A, x, S, k, work, steps, peak)
    return res, (x, z_tail, work)


def time_workspace_free(A, x, S: int, k: int, work, steps: int, peak: float):
    """The workspace-free ranker, avey_split_rank (MaxSim straight from x with the token norms on
    chip, then top-k), beside the step's explicit-workspace one: one HIP-event interval per call
    on the launch stream."""
    import numpy as np
    import torch
    B, N, _ = x.shape
    n_s = -(-N // S)
    scores = torch.empty((B, n_s, n_s), device="cuda", dtype=torch.float32)
    idx = torch.empty((B, n_s, k), device="cuda", dtype=torch.int32)
    w = torch.empty((B, n_s, k), device="cuda", dtype=torch.float32)
    for _ in range(3):
        A.avey_split_rank(x, S, k, scores, idx, w)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        A.avey_split_rank(x, S, k, scores, idx, w)
        e[1].record()
    torch.cuda.synchronize()
    t = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    return {"split_rank_avg_us": round(t * 1e6, 3),
            "maxsim_frac_upper_bound": round(work["maxsim"]["flop"] / t / 1e12 / peak, 4), "launches": steps}


def workload_name(cfg) -> str:
    return f"{cfg.name}: B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S} k={cfg.k} m_t={cfg.m_t} eps={cfg.eps}"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the separate timing of the rest of a layer (static, dynamic, enricher, fuser)")
    ap.add_argument("--no-extreme", action="store_true",
                    help="skip the 96K-token workload timed after the main one")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times (the "
                         "known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path here is the single-GPU kernel set; "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    from synth import CONFIGS, make_inputs

    cfg = None if args.copy_probe_mib > 0 else CONFIGS[args.config]
    inp = None if cfg is None else make_inputs(cfg)
    # The CPU baseline forks its worker processes: it runs before anything touches the GPU.
    cpu = None
    if cfg is not None and not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_budget)
        cpu["value"] = round(cpu["value"], 2)

    import torch

    import attention_free_long_amd as A

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return 0

    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    r, (x, z_tail, work) = time_workload(A, cfg, inp, args.steps, args.warmup, peak)
    achieved = r["maxsim_achieved_tflops"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_bytes("maxsim", cfg.name),
                "traffic_unit": "bytes per launch"}
    result = {
        "metric": METRIC,
        "value": round(r["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": workload_name(cfg), "global_batch": cfg.B, "seq_len": cfg.N,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "pipeline_roofline": r["pipeline_roofline"],
        "maxsim_mfma_util_pct": round(100 * achieved / peak, 2),
    }
    for key in ("compress_hbm_frac", "compress_mfma_frac", "dyn_hbm_frac", "dyn_mfma_frac", "kernels",
                "compress_cold", "rank_workspace_free", "gap_histogram"):
        result[key] = r[key]
    if cfg.dtype == "bf16":
        mp_ = measured_peaks(A)
        result["measured_peaks"] = mp_
        roofline["measured_peak"] = mp_["mfma_bf16_tflops_changing_operands"]
        roofline["frac_measured"] = round(achieved / mp_["mfma_bf16_tflops_changing_operands"], 4)
        comp_t = r["kernels"]["compress"]["avg_us"] * 1e-6
        result["compress_hbm_frac_measured"] = round(work["compress"]["bytes"] / comp_t / 1e9 / mp_["copy_gbs"], 4)
        result["library_gemm"] = library_gemm_rates(cfg)
    if not args.no_layers:
        result["layers"] = time_layers(A, cfg, inp, z_tail, work, max(10, args.steps // 2), peak)
    del x, z_tail
    if not args.no_extreme and cfg.name != "extreme":
        ecfg = CONFIGS["extreme"]
        einp = make_inputs(ecfg)
        e, _ = time_workload(A, ecfg, einp, max(5, args.steps // 5), max(3, args.warmup // 5), PEAK_BF16_TFLOPS)
        result["extreme"] = {
            "workload": workload_name(ecfg),
            "value": round(e["value"], 1), "unit": "tokens/s", "ms_per_step": round(e["ms_per_step"], 4),
            "steps": max(5, args.steps // 5),
            "maxsim": {"achieved": round(e["maxsim_achieved_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(e["maxsim_achieved_tflops"] / PEAK_BF16_TFLOPS, 4),
                       "traffic": traffic_bytes("maxsim", ecfg.name), "traffic_unit": "bytes per launch"},
            "compress_cold": e["compress_cold"],
            "rank_workspace_free": e["rank_workspace_free"],
            "compress_hbm_frac": e["compress_hbm_frac"],
            "dyn_hbm_frac": e["dyn_hbm_frac"], "dyn_mfma_frac": e["dyn_mfma_frac"],
            "pipeline_roofline": e["pipeline_roofline"],
            "kernels": e["kernels"],
            "gap_histogram": e["gap_histogram"],
        }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
