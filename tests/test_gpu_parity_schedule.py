"""GPU parity where the persistent MaxSim kernel's workgroups each walk many pair tiles: every
score, every top-k set and every weight against the float64 oracle, then every split of the
compression and the dynamic layer.

MaxSim relevance of every split to every target split, the top-k of each row and its
divide-by-max weights (paperlayer.ai "Avey-B" summary, section 3; papernotes.org Avey-B note,
方法详解/整体框架) are compared output by output at shapes with thousands of pair tiles on the
256 compute units: the cross-tile prefetch of the next unit, the per-XCD range remainder, the
crossing from one sequence of the batch to the next inside a workgroup's range, and (S = 512)
the running column maxima across the 2 x 2 quadrants of a pair.

Each case prints how its rows passed the top-k rule: "exact" (the oracle's k-th and (k+1)-th
scores are at least 1e-3 apart and the sets are equal), "band_same" (closer than that, sets
equal) and "band_differs" (closer than that, the sets differ only by indices inside the band),
and the histogram of the oracle's relative gaps.
"""
import sys
from collections import Counter

import numpy as np
import pytest
import torch

import attention_free_long_amd as A
from oracle import avey_oracle as O
from synth import CONFIGS, Config, make_inputs

from helpers import (TOL, check_score_row, check_topk_row, gap_histogram, host_f64, row_rel_err,
                     split_rows_of, upload)

pytestmark = pytest.mark.gpu

CASES = {
    # the base workload as it is: 8 sequences x 32 splits, 3968 pair tiles (15.5 per CU)
    "base": CONFIGS["base"],
    # the wide workload's split length, k and duplicates with d cut to 256: 496 pairs x 4
    # quadrants per sequence, 7936 units; exact duplicate splits force tied scores
    "wide_d256": CONFIGS["wide"].with_(name="wide_d256", d=256, m_t=256, m=512),
    # 79 splits per sequence, the last one 32 tokens: 9243 tiles over 3 sequences
    "ragged_many": Config("ragged_many", B=3, N=20000, d=128, S=256, k=3, m_t=128, m=256, dtype="bf16",
                          x_dist="mixture", n_centroids=64),
    # S = 64: 4 splits per unit side, 256 splits per sequence (the last one 16 tokens), 64 groups:
    # 4160 units over 2 sequences, 64 of them diagonal
    "s64_many": Config("s64_many", B=2, N=16336, d=128, S=64, k=3, m_t=128, m=256, dtype="bf16",
                       x_dist="mixture", n_centroids=64),
}


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", list(CASES))
def test_all_outputs_many_tiles(gpu_ok, name):
    cfg = CASES[name]
    tol = TOL[cfg.dtype]
    pairs = cfg.B * cfg.n_s * (cfg.n_s - 1) // 2
    if cfg.S in (64, 128):                       # units of 256 / S splits per side, diagonal included
        groups = -(-cfg.N // 256)
        units = cfg.B * groups * (groups + 1) // 2
    else:
        units = pairs * (-(-cfg.S // 256)) ** 2
    say(f"{name}: B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S} k={cfg.k}: {pairs} pairs, {units} MaxSim units")
    inp = make_inputs(cfg)
    x, P, z, z_tail = upload(inp)
    scores, idx, w = A.avey_split_rank(x, cfg.S, cfg.k)
    xhat = A.avey_select_compress(x, idx, w, P, cfg.S, residual=True)
    out = A.avey_dyn_context(z_tail, cfg.S, cfg.eps)
    torch.cuda.synchronize()
    g_s = scores.cpu().numpy().astype(np.float64)
    g_i, g_w = idx.cpu().numpy(), w.cpu().numpy()
    x64 = inp.x_f64()
    say(f"{name}: oracle scores for all {cfg.B * cfg.n_s} rows")
    ranked = O.split_rank(x64, cfg.S, cfg.k)
    worst_s, worst_w = 0.0, 0.0
    how = Counter()
    gaps = []
    for (b, i), (o_row, o_idx, o_w, gap) in ranked.items():
        worst_s = max(worst_s, check_score_row(g_s[b, i], o_row, i, tol["scores"]))
        how[check_topk_row(g_i[b, i], g_w[b, i], o_row, o_idx, gap, i, cfg.k, tol["w"])] += 1
        ow = np.array([o_row[j] for j in g_i[b, i]]) / o_row[g_i[b, i, 0]]
        worst_w = max(worst_w, float(np.max(np.abs(g_w[b, i] - ow) / np.abs(ow))))
        gaps.append(gap)
    say(f"{name}: scores worst rel err {worst_s:.2e}, w worst rel err {worst_w:.2e}; rows {dict(how)}")
    say(f"{name}: oracle k-th vs (k+1)-th relative gap histogram {gap_histogram(gaps)}")
    if inp.meta["dups"]:
        # an exact duplicate pair (s, t) ties in every other row: the oracle scores them equal
        for b, s_, t_ in inp.meta["dups"]:
            r = next(i for i in range(cfg.n_s) if i not in (s_, t_))
            o_row = ranked[(b, r)][0]
            assert o_row[s_] == o_row[t_]
    say(f"{name}: compression and dynamic layer, every split")
    comp = O.select_compress(x64, cfg.S, g_i, g_w.astype(np.float64), inp.P_f64(), residual=True)
    gx = host_f64(xhat)
    worst_x = 0.0
    for (b, i), rows in comp.items():
        err = row_rel_err(gx[b, split_rows_of(cfg.N, cfg.S, i)], rows)
        assert err <= tol["out"], f"xhat split {(b, i)}: {err:.3e}"
        worst_x = max(worst_x, err)
    dyn = O.dyn_context(inp.z_tail_f64(), cfg.S, cfg.eps)
    go = host_f64(out)
    worst_o = 0.0
    for (b, i), rows in dyn.items():
        err = row_rel_err(go[b, split_rows_of(cfg.N, cfg.S, i)], rows)
        assert err <= tol["out"], f"dyn split {(b, i)}: {err:.3e}"
        worst_o = max(worst_o, err)
    say(f"{name}: xhat worst row rel err {worst_x:.2e}, dyn worst row rel err {worst_o:.2e}")
