"""GPU parity: libavey (through the C ABI) against the float64 CPU oracle on identical inputs.

Small workloads (several tiles, ragged last split) are compared output by output; the full-size
workloads are compared on sampled score rows and sampled splits, in the launch configuration
the bench times.
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_free_long_amd as A
from oracle import avey_oracle as O
from synth import CONFIGS, Config, make_inputs

from helpers import (TOL, check_score_row, check_topk_row, dev_tensor, host_f64, row_rel_err,
                     split_rows_of, upload)

pytestmark = pytest.mark.gpu

SMALL = {
    # 8 splits of 256, last one 208 tokens; 2 sequences
    "small_bf16": Config("small_bf16", B=2, N=2000, d=256, S=256, k=3, m_t=256, m=384, dtype="bf16",
                         x_dist="mixture", n_centroids=16),
    # S = 512: 2 x 2 quadrants per split pair, last split 40 tokens
    "s512_bf16": Config("s512_bf16", B=2, N=2600, d=128, S=512, k=2, m_t=128, m=256, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    # S = 448: the dynamic core's 4 workgroups of 128 tokens per split end with a half-full one,
    # the last split (108 tokens) leaves three of them empty; m_t = 320 ends on a partial
    # 256-feature tile
    "s448_bf16": Config("s448_bf16", B=1, N=1900, d=128, S=448, k=2, m_t=320, m=384, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    # S = 64 < tile: heavy masking inside every tile
    "s64_bf16": Config("s64_bf16", B=1, N=700, d=64, S=64, k=2, m_t=64, m=128, dtype="bf16",
                       x_dist="mixture", n_centroids=8),
    "tiny": CONFIGS["tiny"],
    # S, d and m_t multiples of 16 and 8 only: partial 32-token chunks at the end of every block
    # of X_cat, a partial 64-feature chunk in the dynamic layer, a ragged last split
    "s208_d200": Config("s208_d200", B=2, N=2000, d=200, S=208, k=3, m_t=72, m=136, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    "s48_d72": Config("s48_d72", B=1, N=1000, d=72, S=48, k=4, m_t=40, m=104, dtype="bf16",
                      x_dist="mixture", n_centroids=16),
    # 256 < S <= 512 with S % 64 != 0: the S <= 512 dynamic kernel's partial groups of 128 tokens
    "s400_d136": Config("s400_d136", B=1, N=2100, d=136, S=400, k=2, m_t=200, m=264, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
}


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def run_all(inp, residual=True):
    cfg = inp.cfg
    x, P, z, z_tail = upload(inp)
    scores, idx, w = A.avey_split_rank(x, cfg.S, cfg.k)
    xhat = A.avey_select_compress(x, idx, w, P, cfg.S, residual=residual)
    out = A.avey_dyn_context(z_tail, cfg.S, cfg.eps)
    torch.cuda.synchronize()
    return {
        "scores": scores.cpu().numpy().astype(np.float64),
        "idx": idx.cpu().numpy(),
        "w": w.cpu().numpy(),
        "xhat": host_f64(xhat),
        "out": host_f64(out),
    }


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(gpu_ok, name):
    cfg = SMALL[name]
    tol = TOL[cfg.dtype]
    inp = make_inputs(cfg)
    say(f"{name}: split_rank + select_compress + dyn_context B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S} k={cfg.k}")
    g = run_all(inp)
    x64 = inp.x_f64()
    n_s = cfg.n_s
    ranked = O.split_rank(x64, cfg.S, cfg.k)
    worst = {"scores": 0.0, "xhat": 0.0, "out": 0.0}
    for (b, i), (o_row, o_idx, o_w, gap) in ranked.items():
        worst["scores"] = max(worst["scores"], check_score_row(g["scores"][b, i], o_row, i, tol["scores"]))
        check_topk_row(g["idx"][b, i], g["w"][b, i], o_row, o_idx, gap, i, cfg.k, tol["w"])
    # compression on the GPU's own idx / w (independent of tie effects)
    comp = O.select_compress(x64, cfg.S, g["idx"], g["w"].astype(np.float64), inp.P_f64(), residual=True)
    for (b, i), rows in comp.items():
        err = row_rel_err(g["xhat"][b, split_rows_of(cfg.N, cfg.S, i)], rows)
        assert err <= tol["out"], f"xhat split {(b, i)}: {err:.3e}"
        worst["xhat"] = max(worst["xhat"], err)
    dyn = O.dyn_context(inp.z_tail_f64(), cfg.S, cfg.eps)
    for (b, i), rows in dyn.items():
        err = row_rel_err(g["out"][b, split_rows_of(cfg.N, cfg.S, i)], rows)
        assert err <= tol["out"], f"dyn split {(b, i)}: {err:.3e}"
        worst["out"] = max(worst["out"], err)
    assert n_s == g["scores"].shape[1]
    say(f"{name}: worst relative errors " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))


def test_residual_off_and_k_max(gpu_ok):
    cfg = SMALL["small_bf16"].with_(k=7, B=1)        # k = n_s - 1: every other split is retrieved
    inp = make_inputs(cfg)
    say("residual off, k = n_s - 1")
    g = run_all(inp, residual=False)
    x64 = inp.x_f64()
    ranked = O.split_rank(x64, cfg.S, cfg.k)
    for (b, i), (o_row, o_idx, o_w, gap) in ranked.items():
        assert sorted(g["idx"][b, i].tolist()) == [j for j in range(cfg.n_s) if j != i]
        check_topk_row(g["idx"][b, i], g["w"][b, i], o_row, o_idx, gap, i, cfg.k, TOL["bf16"]["w"])
    comp = O.select_compress(x64, cfg.S, g["idx"], g["w"].astype(np.float64), inp.P_f64(), residual=False)
    for (b, i), rows in comp.items():
        assert row_rel_err(g["xhat"][b, split_rows_of(cfg.N, cfg.S, i)], rows) <= TOL["bf16"]["out"]


def test_padding_rows_never_read_and_determinism(gpu_ok):
    """NaN rows after N must not change any output (they are never loaded); two runs are bitwise equal."""
    cfg = SMALL["small_bf16"].with_(B=1)
    inp = make_inputs(cfg)
    say("NaN sentinels after N, determinism")
    x, P, z, z_tail = upload(inp)
    N, d = cfg.N, cfg.d
    xb = torch.full((1, N + 64, d), float("nan"), device="cuda", dtype=torch.bfloat16)
    xb[:, :N] = x
    zb = torch.full((1, N + 64, cfg.m), float("nan"), device="cuda", dtype=torch.bfloat16)
    zb[:, :N] = z
    outs = []
    for xx, zz in ((x, z), (xb[:, :N], zb[:, :N]), (x, z)):
        s, i_, w_ = A.avey_split_rank(xx, cfg.S, cfg.k)
        xh = A.avey_select_compress(xx, i_, w_, P, cfg.S)
        o = A.avey_dyn_context(zz[..., inp.tail_col:], cfg.S, cfg.eps)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (s, i_, w_, xh, o)])
    for a_, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)
    for a_, b_ in zip(outs[0], outs[2]):
        assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)
    assert torch.isfinite(outs[0][3].float()).all() and torch.isfinite(outs[0][4].float()).all()


def test_empty_inputs(gpu_ok):
    x = torch.empty((0, 1024, 64), device="cuda", dtype=torch.bfloat16)
    s, i_, w_ = A.avey_split_rank(x, 64, 3)
    assert s.numel() == 0
    z = torch.empty((2, 0, 64), device="cuda", dtype=torch.bfloat16)
    assert A.avey_dyn_context(z, 64, 1e-8).numel() == 0


# ------------------------------------------------------------------ full-size workloads
FULL_SAMPLES = {
    "base": [(0, 0), (3, 17), (7, 31)],
    "long": [(0, 0), (0, 77), (1, 127)],
    "extreme": [(0, 0), (0, 200), (0, 383)],
    "wide": [(0, 0), (1, 9), (3, 31)],
}


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_full_size_sampled(gpu_ok, name):
    cfg = CONFIGS[name]
    tol = TOL[cfg.dtype]
    inp = make_inputs(cfg)
    say(f"{name}: full size B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S} k={cfg.k} m_t={cfg.m_t}")
    g = run_all(inp)
    rows = FULL_SAMPLES[name]
    x64_b = {b: inp.x_f64(b) for b in {b for b, _ in rows}}
    worst = 0.0
    for b, i in rows:
        o_row = O.score_row(x64_b[b], cfg.S, i)
        o_idx, _, _, gap = O.top_k(o_row, i, cfg.k)
        worst = max(worst, check_score_row(g["scores"][b, i], o_row, i, tol["scores"]))
        check_topk_row(g["idx"][b, i], g["w"][b, i], o_row, o_idx, gap, i, cfg.k, tol["w"])
        ref = O.compress_split(x64_b[b], cfg.S, g["idx"][b, i], g["w"][b, i].astype(np.float64), inp.P_f64(), i)
        err = row_rel_err(g["xhat"][b, split_rows_of(cfg.N, cfg.S, i)], ref)
        assert err <= tol["out"], f"xhat {(b, i)}: {err:.3e}"
        zt = inp.z_tail_f64(b, split_rows_of(cfg.N, cfg.S, i))
        ref = O.dyn_context_split(zt, cfg.S, cfg.eps, 0)
        err = row_rel_err(g["out"][b, split_rows_of(cfg.N, cfg.S, i)], ref)
        assert err <= tol["out"], f"dyn {(b, i)}: {err:.3e}"
    say(f"{name}: worst score relative error on the sampled rows {worst:.2e}")
    # properties that hold everywhere: w0 == 1, weights in (0, 1], indices valid and not self
    w = g["w"]
    assert (w[..., 0] == 1.0).all() and (w > 0).all() and (w <= 1).all()
    n_s = cfg.n_s
    idx = g["idx"]
    assert (idx >= 0).all() and (idx < n_s).all()
    assert not (idx == np.arange(n_s)[None, :, None]).any()
    assert np.isfinite(g["xhat"]).all() and np.isfinite(g["out"]).all()


@pytest.mark.parametrize("dtype,S", [("bf16", 64), ("bf16", 48), ("f32", 64)])
def test_prepare_normalises_and_pads(gpu_ok, dtype, S):
    """The ranker workspace holds the oracle's N(x) (bf16: rounded, packed block by block in
    chunk planes, a block being a split or, at S = 64 and 128, 256 consecutive tokens; fp32:
    row-major) and zero rows for the padding tokens after N."""
    cfg = Config("prep_" + dtype, B=2, N=1000, d=128, S=S, k=2, m_t=64, m=128, dtype=dtype,
                 x_dist="mixture", n_centroids=8)
    inp = make_inputs(cfg)
    say(f"maxsim_prepare {dtype} B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S}")
    x, _, _, _ = upload(inp)
    x[1, 17].zero_()
    ws = A.avey_maxsim_prepare(x, cfg.S)
    torch.cuda.synchronize()
    d = cfg.d
    P = 256 if dtype == "bf16" and S in (64, 128) else S      # rows per packed block
    n_p = -(-cfg.N // P)
    assert ws.numel() == cfg.B * n_p * P * d * (2 if dtype == "bf16" else 4)
    if dtype == "bf16":
        got = ws[: cfg.B * n_p * P * d * 2].view(torch.bfloat16).float()
        got = got.reshape(cfg.B, n_p, d // 32, P, 32).permute(0, 1, 3, 2, 4).reshape(cfg.B, n_p * P, d)
    else:
        got = ws[: cfg.B * n_p * P * d * 4].view(torch.float32).reshape(cfg.B, n_p * P, d)
    got = got.cpu().numpy().astype(np.float64)
    xs = host_f64(x)
    assert np.all(got[:, cfg.N:] == 0.0)
    assert np.all(got[1, 17] == 0.0)
    rel = 2.0 ** -8 if dtype == "bf16" else 1e-6
    for b in range(cfg.B):
        ref = O.unit_rows(xs[b])
        assert np.all(np.abs(got[b, : cfg.N] - ref) <= rel * np.abs(ref) + 1e-7)


def edge_weights(w, nan_split):
    """Caller-given weights the ranker does not produce but the call accepts: all negative in
    one split, |w| over 50 decades in another, and a NaN at nan_split (that split's outputs must
    be non-finite, as w X is)."""
    B, n_s, k = w.shape
    w[0, 3, :] = -w[0, 3, :]
    w[B - 1, 2, 0] = 1e-30
    w[B - 1, 2, 1:] *= 1e20
    w[nan_split] = np.nan
    return w


def compare_splits(got, ref, N, S, nan_split=None):
    worst = 0.0
    for (b, i), rows in ref.items():
        g = got[b, split_rows_of(N, S, i)]
        if (b, i) == nan_split:
            assert not np.isfinite(g).any(), f"split {(b, i)} with a NaN weight has finite outputs"
            continue
        err = row_rel_err(g, rows)
        assert err <= TOL["bf16"]["out"], f"xhat split {(b, i)}: {err:.3e}"
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("weights", ["positive", "zero_and_negative", "edge"])
def test_compress_given_weights(gpu_ok, weights):
    """select_compress on caller-given idx / w, including a zero and a negative weight (divide-
    by-max of non-positive scores, read as written), weights above 1, and (edge) all-negative,
    widely spread and NaN weights."""
    cfg = SMALL["small_bf16"]
    inp = make_inputs(cfg)
    say(f"select_compress given weights ({weights})")
    x, P, _, _ = upload(inp)
    rng = np.random.default_rng(7)
    B, n_s, k = cfg.B, cfg.n_s, cfg.k
    idx = np.stack([rng.permutation(n_s)[:k] for _ in range(B * n_s)]).reshape(B, n_s, k).astype(np.int32)
    w = rng.uniform(0.05, 3.0, size=(B, n_s, k)).astype(np.float32)
    if weights == "zero_and_negative":
        w[0, 1, 1] = 0.0
        w[1, 2, 0] = -0.75
    nan_split = (0, 5, 1) if weights == "edge" else None
    if nan_split:
        w = edge_weights(w, nan_split)
    g = A.avey_select_compress(x, torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda(), P, cfg.S)
    torch.cuda.synchronize()
    got = host_f64(g)
    ref = O.select_compress(inp.x_f64(), cfg.S, idx, w.astype(np.float64), inp.P_f64(), residual=True)
    worst = compare_splits(got, ref, cfg.N, cfg.S, nan_split[:2] if nan_split else None)
    say(f"given weights ({weights}): worst xhat error {worst:.2e}")


@pytest.mark.parametrize("name", ["small_bf16", "tiny"])
def test_preceding_ranker_parity(gpu_ok, name):
    """Unidirectional ranker: candidates precede the target; short rows end with (-1, 0); the
    compression takes the padded selection (empty blocks are zero rows)."""
    cfg = SMALL[name]
    tol = TOL[cfg.dtype]
    inp = make_inputs(cfg)
    say(f"{name}: split_rank_preceding + select_compress")
    x, P, _, _ = upload(inp)
    scores, idx, w = A.avey_split_rank(x, cfg.S, cfg.k, preceding=True)
    xhat = A.avey_select_compress(x, idx, w, P, cfg.S)
    torch.cuda.synchronize()
    g_s = scores.cpu().numpy().astype(np.float64)
    g_i, g_w = idx.cpu().numpy(), w.cpu().numpy()
    x64 = inp.x_f64()
    ranked = O.split_rank(x64, cfg.S, cfg.k, preceding=True)
    for (b, i), (o_row, o_idx, o_w, gap) in ranked.items():
        check_score_row(g_s[b, i], o_row, i, tol["scores"])
        n_real = min(cfg.k, i)
        gi = [int(v) for v in g_i[b, i]]
        assert gi[n_real:] == [-1] * (cfg.k - n_real) and np.all(g_w[b, i, n_real:] == 0.0)
        real = gi[:n_real]
        assert all(0 <= j < i for j in real) and len(set(real)) == n_real
        if n_real == 0:
            continue
        assert g_w[b, i, 0] == 1.0
        o_real = [int(v) for v in o_idx[:n_real]]
        if gap >= 1e-3:
            assert set(real) == set(o_real), f"row {(b, i)}: {real} vs {o_real}"
        else:
            kth = o_row[o_real[-1]]
            for j in set(real) ^ set(o_real):
                assert abs(o_row[j] - kth) <= 1e-3 * abs(kth)
        ow = np.array([o_row[j] for j in real]) / o_row[real[0]]
        assert np.max(np.abs(g_w[b, i, :n_real] - ow) / np.abs(ow)) <= tol["w"]
    comp = O.select_compress(x64, cfg.S, g_i, g_w.astype(np.float64), inp.P_f64(), residual=True)
    got = host_f64(xhat)
    for (b, i), rows in comp.items():
        err = row_rel_err(got[b, split_rows_of(cfg.N, cfg.S, i)], rows)
        assert err <= tol["out"], f"xhat split {(b, i)}: {err:.3e}"


def test_side_stream_and_workspace_reuse(gpu_ok):
    """Work is enqueued on the caller's current stream, and one workspace serves calls of
    different sizes in a row: results equal the default-stream ones bitwise, on both ranker
    paths."""
    cfg = SMALL["small_bf16"]
    inp = make_inputs(cfg)
    say("side stream, workspace reuse")
    x, P, z, z_tail = upload(inp)
    ref = [t.clone() for t in A.avey_split_rank(x, cfg.S, cfg.k)]
    ref_ws = [t.clone() for t in A.avey_split_rank_ws(x, cfg.S, cfg.k)]
    ref_x = A.avey_select_compress(x, ref[1], ref[2], P, cfg.S)
    ref_o = A.avey_dyn_context(z_tail, cfg.S, cfg.eps)
    torch.cuda.synchronize()
    ws = A.rank_workspace(x, cfg.S)
    small = x[:1, :1100]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        s1 = A.avey_split_rank_ws(small, cfg.S, cfg.k, workspace=ws)   # smaller problem first
        s2 = A.avey_split_rank_ws(x, cfg.S, cfg.k, workspace=ws)
        s3 = A.avey_split_rank(x, cfg.S, cfg.k)
        xh = A.avey_select_compress(x, s3[1], s3[2], P, cfg.S)
        o = A.avey_dyn_context(z_tail, cfg.S, cfg.eps)
    side.synchronize()
    for a_, b_ in zip(ref_ws, s2):
        assert torch.equal(a_, b_)
    for a_, b_ in zip(ref, s3):
        assert torch.equal(a_, b_)
    assert torch.equal(ref_x.view(torch.int16), xh.view(torch.int16))
    assert torch.equal(ref_o.view(torch.int16), o.view(torch.int16))
    s1_ref = A.avey_split_rank_ws(small, cfg.S, cfg.k)
    torch.cuda.synchronize()
    for a_, b_ in zip(s1_ref, s1):
        assert torch.equal(a_, b_)


# The ranker's shape range (S a multiple of 16 up to 512, d a multiple of 8), both paths. The
# d % 32 != 0 cases end every row on a partial 32-feature chunk; S not a multiple of 256 leaves
# rows of every unit past the split; N not a multiple of S leaves a ragged last split.
RANK_SHAPES = {
    "S208_d200": Config("r208", B=2, N=2000, d=200, S=208, k=3, m_t=64, m=64, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    "S48_d72": Config("r48", B=1, N=1000, d=72, S=48, k=4, m_t=64, m=64, dtype="bf16",
                      x_dist="mixture", n_centroids=16),
    "S16_d8": Config("r16", B=2, N=300, d=8, S=16, k=2, m_t=64, m=64, dtype="bf16",
                     x_dist="mixture", n_centroids=8),
    "S400_d776": Config("r400", B=1, N=3000, d=776, S=400, k=2, m_t=64, m=64, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    "S512_d40": Config("r512", B=2, N=2100, d=40, S=512, k=3, m_t=64, m=64, dtype="bf16",
                       x_dist="mixture", n_centroids=16),
    # S = 64 and 128: units of 256 / S splits per side; ragged last split and last group
    "S64_d136": Config("r64", B=2, N=1500, d=136, S=64, k=3, m_t=64, m=64, dtype="bf16",
                       x_dist="mixture", n_centroids=16),
    "S128_d64": Config("r128", B=2, N=1000, d=64, S=128, k=2, m_t=64, m=64, dtype="bf16",
                       x_dist="mixture", n_centroids=16),
    # one group only: every pair inside a single diagonal unit
    "S64_one_group": Config("r64g", B=1, N=200, d=64, S=64, k=2, m_t=64, m=64, dtype="bf16",
                            x_dist="mixture", n_centroids=8),
}


@pytest.mark.parametrize("path", ["rows", "workspace"])
@pytest.mark.parametrize("name", list(RANK_SHAPES))
def test_rank_shape_range(gpu_ok, name, path):
    """Every score, top-k set and weight against the oracle over the ranker's shape range, on the
    workspace-free path (avey_split_rank) and the explicit-workspace path. One token is zero
    (its cosine with everything is 0) and x has a row stride larger than d."""
    cfg = RANK_SHAPES[name]
    tol = TOL[cfg.dtype]
    inp = make_inputs(cfg)
    say(f"rank {path} {name}: B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S} k={cfg.k}")
    xd = dev_tensor(inp.x, cfg.dtype)
    wide = torch.full((cfg.B, cfg.N, cfg.d + 24), float("nan"), device="cuda", dtype=xd.dtype)
    wide[..., : cfg.d] = xd
    x = wide[..., : cfg.d]                          # row stride d + 24, NaN beyond d
    x[cfg.B - 1, 5].zero_()
    x64 = inp.x_f64().copy()
    x64[cfg.B - 1, 5] = 0.0
    if path == "rows":
        scores, idx, w = A.avey_split_rank(x, cfg.S, cfg.k)
    else:
        scores, idx, w = A.avey_split_rank_ws(x, cfg.S, cfg.k)
    torch.cuda.synchronize()
    g_s = scores.cpu().numpy().astype(np.float64)
    g_i, g_w = idx.cpu().numpy(), w.cpu().numpy()
    worst = 0.0
    for (b, i), (o_row, o_idx, o_w, gap) in O.split_rank(x64, cfg.S, cfg.k).items():
        worst = max(worst, check_score_row(g_s[b, i], o_row, i, tol["scores"]))
        check_topk_row(g_i[b, i], g_w[b, i], o_row, o_idx, gap, i, cfg.k, tol["w"])
    say(f"rank {path} {name}: worst score relative error {worst:.2e}")


def test_rank_paths_agree_at_full_size(gpu_ok):
    """The two ranker paths on the 32K-token workload: scores within the score tolerance of each
    other everywhere, the same top-k sets wherever the gap between the k-th and (k+1)-th score
    exceeds twice that tolerance."""
    cfg = CONFIGS["long"]
    inp = make_inputs(cfg)
    say("rank paths at B=2 N=32768 d=768 S=256 k=3")
    x = dev_tensor(inp.x, cfg.dtype)
    s_r, i_r, w_r = [t.cpu().numpy() for t in A.avey_split_rank(x, cfg.S, cfg.k)]
    s_w, i_w, w_w = [t.cpu().numpy() for t in A.avey_split_rank_ws(x, cfg.S, cfg.k)]
    off = ~np.eye(cfg.n_s, dtype=bool)[None].repeat(cfg.B, 0)
    rel = np.abs(s_r[off].astype(np.float64) - s_w[off]) / np.abs(s_w[off])
    assert rel.max() <= 2 * TOL["bf16"]["scores"]
    srt = -np.sort(-np.where(off, s_w, -np.inf), axis=-1)
    gap = (srt[..., cfg.k - 1] - srt[..., cfg.k]) / np.abs(srt[..., cfg.k - 1])
    clear = gap > 4 * TOL["bf16"]["scores"]
    same = np.array([[set(i_r[b, i]) == set(i_w[b, i]) for i in range(cfg.n_s)] for b in range(cfg.B)])
    assert same[clear].all()
    assert (w_r[..., 0] == 1.0).all() and (w_w[..., 0] == 1.0).all()
    say(f"rank paths: max relative score difference {rel.max():.2e}, {int(clear.sum())} clear rows")


# Shapes with at least one 256-feature x 256-token unit per CU (256 CUs), so that compression
# runs on the persistent kernel, small enough for the oracle to check every split.
PERSISTENT = {
    # units = B * n_s * ceil(S / 256) * ceil(d / 256)
    "s256_res": (Config("p256", B=2, N=32668, d=64, S=256, k=3, m_t=64, m=64, dtype="bf16",
                        x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    "s256_nores": (Config("p256", B=2, N=32668, d=64, S=256, k=3, m_t=64, m=64, dtype="bf16",
                          x_dist="mixture", n_centroids=32, z_kind="relu2_x"), False),
    "s512": (Config("p512", B=2, N=32468, d=128, S=512, k=7, m_t=128, m=128, dtype="bf16",
                    x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    "s64": (Config("p64", B=4, N=16374, d=64, S=64, k=2, m_t=64, m=64, dtype="bf16",
                   x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    # 384 units: per XCD one full round of 32 workgroups and 16 units left over
    "tail16": (Config("ptail16", B=1, N=32668, d=768, S=256, k=3, m_t=768, m=768, dtype="bf16",
                         x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    # 448 units: per XCD one full round and 24 units left over
    "tail24": (Config("ptail24", B=1, N=57294, d=512, S=256, k=3, m_t=512, m=512, dtype="bf16",
                         x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    # S = 208 and 400 (cpb rounded up to an even 8 and 14 chunks per block, the last ones
    # partial or empty), d % 32 != 0: 290 and 300 units
    "s208_d200": (Config("p208", B=2, N=30000, d=200, S=208, k=3, m_t=200, m=200, dtype="bf16",
                         x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    "s400_d136": (Config("p400", B=1, N=59950, d=136, S=400, k=3, m_t=136, m=136, dtype="bf16",
                         x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
    # 320 units but k + 1 = 71 blocks, more than the persistent kernel's table holds: the tiled
    # kernel takes it
    "k70": (Config("pk70", B=4, N=5100, d=64, S=64, k=70, m_t=64, m=64, dtype="bf16",
                   x_dist="mixture", n_centroids=32, z_kind="relu2_x"), True),
}


@pytest.mark.parametrize("name", list(PERSISTENT))
def test_compress_persistent_kernel(gpu_ok, name):
    """Every split against the oracle on caller-given idx / w in random order of |w|, with an
    empty block (index -1), a zero weight, the edge weights above and a ragged last split."""
    cfg, residual = PERSISTENT[name]
    inp = make_inputs(cfg)
    say(f"persistent compress {name}: B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S} k={cfg.k} residual={residual}")
    x, P, _, _ = upload(inp)
    rng = np.random.default_rng(3)
    B, n_s, k = cfg.B, cfg.n_s, cfg.k
    idx = np.stack([rng.permutation(n_s)[:k] for _ in range(B * n_s)]).reshape(B, n_s, k).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(B, n_s, k)).astype(np.float32)
    idx[0, 5, k - 1] = -1
    w[0, 5, k - 1] = 0.0
    w[B - 1, n_s - 1, 0] = 0.0
    w = edge_weights(w, (0, 11, k - 1))
    g = A.avey_select_compress(x, torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda(), P, cfg.S,
                               residual=residual)
    torch.cuda.synchronize()
    got = host_f64(g)
    ref = O.select_compress(inp.x_f64(), cfg.S, idx, w.astype(np.float64), inp.P_f64(), residual=residual)
    worst = compare_splits(got, ref, cfg.N, cfg.S, (0, 11))
    say(f"persistent compress {name}: worst xhat error {worst:.2e}")
