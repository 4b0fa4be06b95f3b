"""Host logic of bench.py, on the CPU: the algorithmic work it divides by (counted here again by
enumeration on small shapes and against the closed forms of the method's steps), the pipeline
roofline, the k-th / (k+1)-th gap histogram and the single-GPU guard. None of it touches a GPU."""
import itertools
import math

import numpy as np
import pytest

import bench
from synth import CONFIGS


def _enumerated_work(cfg):
    """FLOPs and bytes of the three hot-path steps, counted by walking what each step touches
    (one multiply-add = 2 FLOP): every unordered split pair's S x S dot products of length d
    (MaxSim: one tile gives both directions); for every split, the (k + 1) S x S blocks of P
    applied to d features (compress) and two S x S x m_t products (the cosine matrix, then the
    mixing). Bytes: compress reads X_i and k gathered splits and writes Xhat_i, all N tokens
    long, plus P once; the dynamic core reads the tail once and writes it once."""
    eb = 2 if cfg.dtype == "bf16" else 4
    n_s = math.ceil(cfg.N / cfg.S)
    maxsim_flop = 0
    for b in range(cfg.B):
        for i, j in itertools.combinations(range(n_s), 2):
            maxsim_flop += 2 * cfg.S * cfg.S * cfg.d
    compress_flop = 0
    dyn_flop = 0
    for b in range(cfg.B):
        for i in range(n_s):
            for r in range(cfg.k + 1):
                compress_flop += 2 * cfg.S * cfg.S * cfg.d
            dyn_flop += 2 * cfg.S * cfg.S * cfg.m_t   # G = N(Z) N(Z)^T over the tail features
            dyn_flop += 2 * cfg.S * cfg.S * cfg.m_t   # G Z
    compress_bytes = cfg.B * cfg.N * cfg.d * eb * (1 + cfg.k + 1) + cfg.S * (cfg.k + 1) * cfg.S * eb
    dyn_bytes = cfg.B * cfg.N * cfg.m_t * eb * 2
    return {"maxsim": maxsim_flop, "compress": compress_flop, "dyn": dyn_flop,
            "compress_bytes": compress_bytes, "dyn_bytes": dyn_bytes}


@pytest.mark.parametrize("name", ["tiny", "base", "wide"])
def test_algorithmic_work_matches_enumeration(name):
    cfg = CONFIGS[name]
    w = bench.algorithmic(cfg)
    e = _enumerated_work(cfg)
    assert w["maxsim"]["flop"] == e["maxsim"]
    assert w["compress"]["flop"] == e["compress"]
    assert w["dyn"]["flop"] == e["dyn"]
    assert w["compress"]["bytes"] == e["compress_bytes"]
    assert w["dyn"]["bytes"] == e["dyn_bytes"]


def test_long_workload_figures():
    """The 32K-token workload: 2 x 128 splits give 2 x 128 x 127 / 2 = 16256 unordered pairs of
    256 x 256 x 768 dot products, 1.6364e12 FLOP; the gather reads 4 splits and writes one per
    target, 5 x 2 x 32768 x 768 bf16 values plus P (256 x 1024)."""
    cfg = CONFIGS["long"]
    w = bench.algorithmic(cfg)
    assert w["maxsim"]["flop"] == 2 * 256 * 256 * 768 * 16256
    assert abs(w["maxsim"]["flop"] - 1.6364e12) / 1.6364e12 < 1e-4
    assert w["compress"]["bytes"] == 5 * 2 * 32768 * 768 * 2 + 256 * 1024 * 2
    assert w["dyn"]["bytes"] == 2 * 2 * 32768 * 1536 * 2


def test_pipeline_roofline_sums_the_kernel_bounds():
    cfg = CONFIGS["long"]
    w = bench.algorithmic(cfg)
    r = bench.pipeline_roofline(cfg, 1.0e7, bench.PEAK_BF16_TFLOPS)
    t = 0.0
    for n in ("maxsim", "compress", "dyn"):
        t += max(w[n]["flop"] / 2.5e15, w[n]["bytes"] / 8.0e12)
    assert r["tokens_per_s"] == pytest.approx(cfg.B * cfg.N / t, rel=1e-6)
    assert r["frac"] == pytest.approx(1.0e7 / r["tokens_per_s"], abs=1e-4)
    # each kernel's bound is at least its FLOP time and at least its byte time, so neither
    # single-resource figure can be below the pipeline roofline
    assert r["mfma_tokens_per_s"] >= r["tokens_per_s"]
    assert r["hbm_tokens_per_s"] >= r["tokens_per_s"]


def test_gap_histogram_counts_rows():
    inf = float("inf")
    scores = np.array([[[-inf, 4.0, 3.0, 2.0],        # k = 2: 3 vs 2, gap 1/3
                        [10.0, -inf, 9.0, 9.0],       # 9 vs 9: gap 0
                        [1.0, 1.0000005, -inf, 0.5],  # 1.0 vs 0.5: gap 0.5
                        [2.0, 2.0, 2.0 - 4e-3, -inf]]], dtype=np.float32)  # 2 vs 1.996: 2e-3
    h = bench.gap_histogram(scores, 2)
    assert h["rows"] == 4
    assert h["bins"]["[0,1e-06)"] == 1
    assert h["bins"]["[0.001,0.01)"] == 1
    assert h["bins"]["[0.1,inf)"] == 2
    assert sum(h["bins"].values()) == 4
    assert h["min_gap"] == 0.0


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
