"""avey_split_rank_noalloc (the ranker with its workspace in the library's own device array)
against the explicit-workspace path it is a variant of: two calls in a row, the second on a
smaller input, then a batch that goes through the array in two passes. The kernels and their
inputs are the same, so scores, indices and weights must be equal bit for bit; the small case is
also checked against the oracle."""
import sys

import numpy as np
import pytest
import torch

import attention_free_long_amd as A
from oracle import avey_oracle as O
from synth import Config, make_inputs

from helpers import TOL, check_score_row, check_topk_row, dev_tensor

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def both_paths(x, S, k):
    ref = [t.clone() for t in A.avey_split_rank_ws(x, S, k)]
    got = A.avey_split_rank_noalloc(x, S, k)
    torch.cuda.synchronize()
    for name, r, g in zip(("scores", "idx", "w"), ref, got):
        assert torch.equal(r, g), f"{name} differs from the explicit-workspace path"
    return got


def test_noalloc_matches_workspace_path(gpu_ok):
    big = Config("na_big", B=3, N=8192, d=768, S=256, k=3, m_t=64, m=64, dtype="bf16",
                 x_dist="mixture", n_centroids=64)
    small = Config("na_small", B=1, N=3000, d=200, S=208, k=4, m_t=64, m=64, dtype="bf16",
                   x_dist="mixture", n_centroids=16)
    say(f"noalloc: B={big.B} N={big.N} d={big.d} S={big.S}, then B={small.B} N={small.N} d={small.d} S={small.S}")
    both_paths(dev_tensor(make_inputs(big).x, "bf16"), big.S, big.k)
    inp = make_inputs(small)
    scores, idx, w = both_paths(dev_tensor(inp.x, "bf16"), small.S, small.k)
    g_s = scores.cpu().numpy().astype(np.float64)
    g_i, g_w = idx.cpu().numpy(), w.cpu().numpy()
    for (b, i), (o_row, o_idx, o_w, gap) in O.split_rank(inp.x_f64(), small.S, small.k).items():
        check_score_row(g_s[b, i], o_row, i, TOL["bf16"]["scores"])
        check_topk_row(g_i[b, i], g_w[b, i], o_row, o_idx, gap, i, small.k, TOL["bf16"]["w"])


def test_noalloc_passes_and_limit(gpu_ok):
    # 157 splits of 256 x 768 features: 61.7 MB per sequence, two sequences per pass of the
    # 160 MiB array, so three sequences take two passes
    cfg = Config("na_pass", B=3, N=40000, d=768, S=256, k=3, m_t=64, m=64, dtype="bf16",
                 x_dist="mixture", n_centroids=64)
    say(f"noalloc in two passes: B={cfg.B} N={cfg.N} d={cfg.d} S={cfg.S}")
    both_paths(dev_tensor(make_inputs(cfg).x, "bf16"), cfg.S, cfg.k)
    # one sequence larger than the array: refused before any launch
    x = torch.zeros((1, 131072, 1024), device="cuda", dtype=torch.bfloat16)
    scores = torch.full((1, 512, 512), 7.0, device="cuda")
    with pytest.raises(A.AveyError) as e:
        A.avey_split_rank_noalloc(x, 256, 3, scores=scores)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((scores == 7.0).all())
