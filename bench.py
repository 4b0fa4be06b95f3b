"""Throughput of the Avey-B ranker + dynamic contextualizer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long] [--no-cpu-baseline]

One step is one pass of the whole path over one batch of synthetic input already resident in
HBM: all-pairs MaxSim, top-k with divide-by-max, weighted gather + (k+1)S -> S compression,
and the dynamic layer's row-normalised cosine mixing. The default workload is the 32K-token
one (batch 2, N = 32768, d = 768, S = 256, k = 3, tail width 1536).

Prints one JSON line: tokens/s over the timed steps, per-kernel times from HIP events on the
launch stream, the MaxSim kernel against the bf16 MFMA roofline, and the CPU oracle timed on a
bounded sample of the same workload.
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
# (FETCH_SIZE read 524300 KiB for 1048576 KiB moved: x2.0; WRITE_SIZE read 1048576 KiB: x1.0).
# Keyed by the digest of the kernel's sources: once they change the figures no longer apply and
# traffic is reported as null until the counters are taken again.
TRAFFIC = {
    "maxsim": {
        "sources": ("maxsim_bf16.hip", "avey_common.h", "../build.py"),
        "measured": {
            ("baf884bcbc72d556", "long"): {"fetch_kib": 1216465.3, "fetch_scale": 1.99995,
                                           "write_kib": 252.6, "write_scale": 1.0},
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


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(inp, budget_s: float = 12.0):
    """The float64 oracle, as it stands, on whole target splits of the same workload until the
    time budget is spent: score row + top-k, compression and dynamic layer of each split."""
    import numpy as np
    from oracle import avey_oracle as O
    cfg = inp.cfg
    n_s = cfg.n_s
    stride = max(1, n_s // 16)
    order = [(b, i) for r in range(stride) for i in range(r, n_s, stride) for b in range(cfg.B)]
    xs, Ps = {}, inp.P_f64()
    done, tok = 0, 0
    t0 = time.perf_counter()
    for b, i in order:
        if b not in xs:
            xs[b] = inp.x_f64(b)
        row = O.score_row(xs[b], cfg.S, i)
        idx, w, _, _ = O.top_k(row, i, cfg.k)
        O.compress_split(xs[b], cfg.S, idx, w, Ps, i)
        rows = slice(i * cfg.S, min((i + 1) * cfg.S, cfg.N))
        O.dyn_context_split(inp.z_tail_f64(b, rows), cfg.S, cfg.eps, 0)
        done += 1
        tok += rows.stop - rows.start
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {
        "value": tok / el,
        "unit": "tokens/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{done} of {cfg.B * n_s} target splits of the {cfg.name} workload (full score row, "
                  f"top-k, compression and dynamic layer per split), {el:.1f} s, float64 numpy",
    }


def time_layers(A, cfg, inp, z_tail, work, steps: int, peak: float):
    """The rest of a neural-processor layer on the same workload, timed apart from the step with
    HIP events on the launch stream (not part of the step's throughput): the static and dynamic
    contextualizer layers (bias and ReLU) on the tail, the enricher X -> Z (d -> m) and the
    fuser [Z_h || c] -> Y (m -> d, with the residual)."""
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
        "enrich": lambda: A.avey_enrich(x, Ud, bUd, out=zf),
        "fuse": lambda: A.avey_fuse(zf, m_h, out, Od, x, out=y),
    }
    res = {}
    for name, call in calls.items():
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
                     "hbm_frac": round(work[name]["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4),
                     "mfma_frac": round(work[name]["flop"] / t / 1e12 / peak, 4),
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
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times (the "
                         "known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path here is the single-GPU kernel set; "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import attention_free_long_amd as A
    from synth import CONFIGS, make_inputs

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
    cfg = CONFIGS[args.config]
    inp = make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    x, P, z = dev(inp.x), dev(inp.P), dev(inp.z)
    z_tail = z[..., inp.tail_col:]
    B, N, n_s, S, k = cfg.B, cfg.N, cfg.n_s, cfg.S, cfg.k
    scores = torch.empty((B, n_s, n_s), device="cuda", dtype=torch.float32)
    idx = torch.empty((B, n_s, k), device="cuda", dtype=torch.int32)
    w = torch.empty((B, n_s, k), device="cuda", dtype=torch.float32)
    ws = A.rank_workspace(x, S)
    xhat = torch.empty((B, N, cfg.d), device="cuda", dtype=dt)
    out = torch.empty((B, N, cfg.m_t), device="cuda", dtype=dt)
    names = ("prepare", "maxsim", "topk", "compress", "dyn")
    calls = (
        lambda: A.avey_maxsim_prepare(x, S, ws),
        lambda: A.avey_maxsim_scores(ws, x, S, scores),
        lambda: A.avey_topk_norm(scores, k, idx, w),
        lambda: A.avey_select_compress(x, idx, w, P, S, residual=True, out=xhat),
        lambda: A.avey_dyn_context(z_tail, S, cfg.eps, out=out),
    )

    def step(ev=None):
        # The events are recorded on torch's current stream, which is the stream every call
        # enqueues its kernels on; each interval brackets exactly one library call.
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record()
            call()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)
    work = algorithmic(cfg)
    kern = {}
    for n in names:
        t = float(np.mean(per[n]))
        entry = {"avg_us": t * 1e6, "median_us": float(np.median(per[n])) * 1e6, "min_us": float(np.min(per[n])) * 1e6}
        if work[n]["flop"]:
            entry["tflops"] = work[n]["flop"] / t / 1e12
        entry["gbs"] = work[n]["bytes"] / t / 1e9
        kern[n] = entry
    ms_per_step = wall / args.steps * 1e3
    value = B * N / (wall / args.steps)

    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    ms_t = kern["maxsim"]["avg_us"] * 1e-6
    achieved = work["maxsim"]["flop"] / ms_t / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_bytes("maxsim", cfg.name),
                "traffic_unit": "bytes per launch"}
    comp_t = kern["compress"]["avg_us"] * 1e-6
    dyn_t = kern["dyn"]["avg_us"] * 1e-6
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} N={N} d={cfg.d} S={S} k={k} m_t={cfg.m_t} eps={cfg.eps}",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "maxsim_mfma_util_pct": round(100 * achieved / peak, 2),
        "compress_hbm_frac": round(work["compress"]["bytes"] / comp_t / 1e9 / PEAK_HBM_GBS, 4),
        "dyn_hbm_frac": round(work["dyn"]["bytes"] / dyn_t / 1e9 / PEAK_HBM_GBS, 4),
        "dyn_mfma_frac": round(work["dyn"]["flop"] / dyn_t / 1e12 / peak, 4),
        "kernels": {n: {kk: round(v, 3) for kk, v in e.items()} for n, e in kern.items()},
    }
    result["compress_cold"] = time_compress_cold(calls[3], work["compress"]["bytes"])
    if cfg.dtype == "bf16":
        mp = measured_peaks(A)
        result["measured_peaks"] = mp
        roofline["measured_peak"] = mp["mfma_bf16_tflops_changing_operands"]
        roofline["frac_measured"] = round(achieved / mp["mfma_bf16_tflops_changing_operands"], 4)
        result["compress_hbm_frac_measured"] = round(work["compress"]["bytes"] / comp_t / 1e9 / mp["copy_gbs"], 4)
    if not args.no_layers:
        result["layers"] = time_layers(A, cfg, inp, z_tail, work, max(10, args.steps // 2), peak)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
        result["cpu_baseline"]["value"] = round(result["cpu_baseline"]["value"], 2)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
