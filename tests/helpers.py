"""Shared pieces of the GPU tests: device transfer of seeded inputs and the comparison rules.

Tolerances (relative): fp32 workloads 1e-5 on everything; bf16 workloads 5e-3 on MaxSim scores
and weights, 2e-2 on the compressed tokens and the dynamic-layer output. Output rows are
compared by ||g - o||_2 / ||o||_2 per token (elementwise relative error is ill-posed near 0).
Top-k sets must match exactly unless the oracle's k-th and (k+1)-th scores are within 1e-3
relative; then every index that differs must score within 1e-3 of the k-th.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import avey_oracle as O

TOL = {
    "f32": {"scores": 1e-5, "w": 1e-5, "out": 1e-5},
    "bf16": {"scores": 5e-3, "w": 5e-3, "out": 2e-2},
}
TIE_GAP = 1e-3


def dev_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Host array (bf16 bits as uint16, or float32) -> device tensor with identical bits."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def upload(inp):
    """x, P, z (full Z) and the z tail view on the device."""
    dt = inp.cfg.dtype
    x = dev_tensor(inp.x, dt)
    P = dev_tensor(inp.P, dt)
    z = dev_tensor(inp.z, dt)
    z_tail = z[..., inp.tail_col:]
    return x, P, z, z_tail


def row_rel_err(g: np.ndarray, o: np.ndarray) -> float:
    num = np.linalg.norm(g - o, axis=-1)
    den = np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
    return float((num / den).max()) if num.size else 0.0


def check_score_row(g_row: np.ndarray, o_row: np.ndarray, i: int, tol: float):
    assert g_row[i] == -math.inf
    mask = np.arange(len(o_row)) != i
    rel = np.abs(g_row[mask] - o_row[mask]) / np.abs(o_row[mask])
    assert rel.max() <= tol, f"score rel err {rel.max():.3e} > {tol}"
    return float(rel.max())


def check_topk_row(g_idx, g_w, o_row, o_idx, gap, i, k, tol_w):
    """Top-k of one row against the oracle under the tie rule. Returns how the row passed:
    "exact" (gap >= TIE_GAP, identical sets), "band_same" (gap < TIE_GAP, identical sets) or
    "band_differs" (gap < TIE_GAP, the sets differ only by indices inside the tie band)."""
    g_idx = [int(v) for v in g_idx]
    assert len(set(g_idx)) == k and i not in g_idx and all(0 <= j < len(o_row) for j in g_idx)
    assert g_w[0] == 1.0, f"w0 = {g_w[0]!r}"
    o_set = set(int(v) for v in o_idx)
    if gap >= TIE_GAP:
        assert set(g_idx) == o_set, f"top-k {g_idx} vs oracle {list(o_idx)} (gap {gap:.2e})"
        how = "exact"
    else:
        kth = o_row[o_idx[-1]]
        for j in set(g_idx) ^ o_set:
            assert abs(o_row[j] - kth) <= TIE_GAP * abs(kth), f"index {j} outside the tie band"
        how = "band_same" if set(g_idx) == o_set else "band_differs"
    # the GPU's ranks are in order of its own scores: non-increasing oracle scores up to the band
    o_sel = np.array([o_row[j] for j in g_idx])
    assert np.all(o_sel[1:] <= o_sel[:-1] + TIE_GAP * np.abs(o_sel[:-1])), f"rank order {g_idx}"
    # weights against the oracle's scores at the GPU's own indices
    ow = o_sel / o_row[g_idx[0]]
    rel = np.abs(np.asarray(g_w, dtype=np.float64) - ow) / np.abs(ow)
    assert rel.max() <= tol_w, f"w rel err {rel.max():.3e}"
    return how


def gap_histogram(gaps, edges=(0.0, 1e-6, 1e-4, 1e-3, 1e-2, 1e-1)):
    """Counts of the oracle's relative k-th vs (k+1)-th score gaps per bin [e_i, e_{i+1}), the last
    bin open-ended; exact ties (gap 0) fall in the first bin."""
    g = np.asarray(list(gaps), dtype=np.float64)
    out = {}
    for lo, hi in zip(edges, list(edges[1:]) + [math.inf]):
        out[f"[{lo:g},{hi:g})"] = int(((g >= lo) & (g < hi)).sum())
    return out


def split_rows_of(N: int, S: int, i: int) -> slice:
    return slice(i * S, min((i + 1) * S, N))


def oracle_rank_rows(x64: np.ndarray, S: int, k: int, rows):
    return O.split_rank(x64, S, k, rows=rows)
