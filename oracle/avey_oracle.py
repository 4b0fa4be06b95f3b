"""CPU oracle for the Avey-B bidirectional ranker and dynamic contextualizer core.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, float64 statement of what the GPU
library computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (``attention_free_long_amd``) never does, and this
module imports nothing from it. Inputs are the exact values the GPU sees (bf16 or fp32 upcast
to float64); every sum is accumulated in float64. Nothing is blocked, fused or reordered
beyond what the definitions below state: the all-pairs score matrix is computed one ordered
pair (i, j) at a time, from scratch.

Sources (the pages' own words are restated, never quoted):

* [notes]   papernotes.org, "Avey-B: 把无注意力架构改造成双向编码器" (ICLR2026 note).
            Section "方法详解 / 整体框架" (ranker: S-token splits with zero padding, MaxSim
            relevance, top-k, division by the largest selected score, weighting and
            concatenation with the current split); "关键设计 2" (dynamic layer mixes Z_t with
            the cosine matrix N(Z_t)N(Z_t)^T); "关键设计 3", eq. 6 (row normalisation
            S~_ij = S_ij / (sum_j S_ij + eps)); "关键设计 4", eq. 8 (X^ = P X_cat with
            P in R^{S x (k+1)S}, plus a residual to the current split's own tokens).
* [summary] paperlayer.ai summary of Avey-B (arXiv 2602.15814v1), section 3 "Background"
            (splits, MaxSim, top-k, normalise-weight-concatenate), section 4.3 "Neural
            compression", appendix H (the compressor residual joins the current split's
            original tokens).
* MaxSim itself is taken as: for target split i and candidate split j, the sum over the
  tokens of i of the largest cosine similarity to any token of j.

Readings where the pages are silent (each is listed, with its reason, in the design notes):
self is never its own candidate; padded tokens are masked (neither a target nor a candidate);
ties in top-k go to the lower split index; X_cat = [current, rank 1, ..., rank k]; the
dynamic layer works within each S-token split on valid tokens only, multiplies the
un-normalised Z_t, and stops at S~ Z_t (no activation, no bias).

Pinned against closed forms, invariants and brute force in ``tests/test_oracle_pins.py``;
no function here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------- splits
def n_splits(N: int, S: int) -> int:
    """[notes] 整体框架: N tokens are cut into S-token splits, the last one zero-padded."""
    return -(-N // S)


def split_rows(N: int, S: int, j: int) -> range:
    """Token positions of split j that hold real tokens (positions >= N are padding)."""
    return range(j * S, min((j + 1) * S, N))


def padded_split(x_b: np.ndarray, S: int, j: int) -> np.ndarray:
    """Split j of one sequence as S rows, padding rows set to zero ([notes] 整体框架)."""
    N, d = x_b.shape
    out = np.zeros((S, d), dtype=np.float64)
    r = split_rows(N, S, j)
    out[: len(r)] = x_b[r.start:r.stop]
    return out


# ----------------------------------------------------------------------------- N(.)
def unit_rows(a: np.ndarray) -> np.ndarray:
    """N(.): each row divided by its L2 norm; a zero row stays zero ([notes] 关键设计 2)."""
    a = np.asarray(a, dtype=np.float64)
    norm = np.sqrt((a * a).sum(axis=-1, keepdims=True))
    out = np.zeros_like(a)
    nz = norm[..., 0] > 0
    out[nz] = a[nz] / norm[nz]
    return out


# ----------------------------------------------------------------------------- ranker
def maxsim(x_b: np.ndarray, S: int, i: int, j: int) -> float:
    """MaxSim relevance of candidate split j to target split i ([summary] 3; [notes] 整体框架).

    Sum over the valid tokens t of split i of max over the valid tokens u of split j of
    cos(x_t, x_u). Padding tokens take part in neither the sum nor the max.
    """
    N = x_b.shape[0]
    ti, tj = split_rows(N, S, i), split_rows(N, S, j)
    ui = unit_rows(x_b[ti.start:ti.stop])
    uj = unit_rows(x_b[tj.start:tj.stop])
    cos = ui @ uj.T                      # [|i|, |j|] cosine similarities
    return float(cos.max(axis=1).sum())


def score_row(x_b: np.ndarray, S: int, i: int) -> np.ndarray:
    """Scores of every candidate j for target split i; the target itself gets -inf."""
    n_s = n_splits(x_b.shape[0], S)
    row = np.empty(n_s, dtype=np.float64)
    for j in range(n_s):
        row[j] = NEG_INF if j == i else maxsim(x_b, S, i, j)
    return row


def score_matrix(x: np.ndarray, S: int) -> np.ndarray:
    """All ordered split pairs: scores[b, i, j] = MaxSim(i <- j), diagonal -inf."""
    B, N, _ = x.shape
    n_s = n_splits(N, S)
    out = np.empty((B, n_s, n_s), dtype=np.float64)
    for b in range(B):
        for i in range(n_s):
            out[b, i] = score_row(x[b], S, i)
    return out


def top_k(row: np.ndarray, i: int, k: int, preceding: bool = False):
    """Top-k candidates of one target split and their divide-by-max weights.

    [notes] 整体框架 / [summary] 3: keep the k most relevant splits, then divide each selected
    score by the largest of them. Order: score descending, ties to the lower index; the
    target itself is never a candidate. Returns (idx[k], w[k], s[k], gap) where gap is the
    relative distance between the k-th and (k+1)-th scores (inf when there is no (k+1)-th).

    preceding=True is the unidirectional ranker: the candidates are the splits before the
    target only ([summary] 3 speaks of the top-k preceding splits; the [summary] pretraining
    ablation and the [notes] training-strategy section find that ranker direction best). When
    fewer than k splits precede the target, the selection is padded with empty blocks:
    index -1, weight 0 (a reading; the pages are silent on it).
    """
    if preceding:
        pool = range(i)
    else:
        pool = (j for j in range(len(row)) if j != i)
    cands = sorted(pool, key=lambda j: (-row[j], j))
    idx = cands[:k]
    s = np.array([row[j] for j in idx], dtype=np.float64)
    w = s / s[0] if len(idx) else s
    if len(cands) > k:
        sk, sk1 = row[cands[k - 1]], row[cands[k]]
        gap = (sk - sk1) / abs(sk) if sk != 0 else (0.0 if sk1 == sk else math.inf)
    else:
        gap = math.inf
    npad = k - len(idx)
    if npad:
        idx = list(idx) + [-1] * npad
        w = np.concatenate([w, np.zeros(npad)])
        s = np.concatenate([s, np.full(npad, NEG_INF)])
    return np.array(idx, dtype=np.int64), w, s, gap


def split_rank(x: np.ndarray, S: int, k: int, rows=None, preceding: bool = False):
    """Score rows, top-k indices and weights for the listed (b, i) target splits (default: all).

    Returns dict {(b, i): (score_row, idx, w, gap)}. preceding selects the unidirectional
    ranker (see top_k).
    """
    B, N, _ = x.shape
    n_s = n_splits(N, S)
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(n_s)]
    out = {}
    for b, i in rows:
        r = score_row(x[b], S, i)
        idx, w, _, gap = top_k(r, i, k, preceding)
        out[(b, i)] = (r, idx, w, gap)
    return out


# ----------------------------------------------------------------------------- compression
def compress_split(x_b: np.ndarray, S: int, idx_i, w_i, P: np.ndarray, i: int, residual: bool = True) -> np.ndarray:
    """X^_i = P X_cat (+ X_i) for target split i, valid rows only.

    [notes] 关键设计 4, eq. 8 and [summary] 4.3: X_cat stacks the current split and its k
    retrieved splits, each retrieved split scaled by its normalised score ([notes] 整体框架);
    P (S x (k+1)S) maps the (k+1)S rows back to S. The residual adds the current split's own
    tokens ([summary] appendix H). Block order: [current, rank 1, ..., rank k]. An index of -1
    is an empty block (S zero rows), as the unidirectional ranker pads its selection.
    """
    N, d = x_b.shape
    blocks = [padded_split(x_b, S, i)]
    for j, wj in zip(idx_i, w_i):
        if int(j) < 0:
            blocks.append(np.zeros((S, d), dtype=np.float64))
        else:
            blocks.append(float(wj) * padded_split(x_b, S, int(j)))
    x_cat = np.concatenate(blocks, axis=0)            # [(k+1)S, d]
    xhat = np.asarray(P, dtype=np.float64) @ x_cat     # [S, d]
    if residual:
        xhat = xhat + blocks[0]
    return xhat[: len(split_rows(N, S, i))]


def select_compress(x: np.ndarray, S: int, idx: np.ndarray, w: np.ndarray, P: np.ndarray,
                    residual: bool = True, splits=None):
    """compress_split over the listed (b, i) splits (default: all). Returns {(b, i): rows}."""
    B, N, _ = x.shape
    n_s = n_splits(N, S)
    if splits is None:
        splits = [(b, i) for b in range(B) for i in range(n_s)]
    return {(b, i): compress_split(x[b], S, idx[b, i], w[b, i], P, i, residual) for b, i in splits}


# ----------------------------------------------------------------------------- dynamic layer
NORMS = ("sum", "softmax", "rms", "none")


def row_normalise(sim: np.ndarray, norm: str, eps: float) -> np.ndarray:
    """Row normalisation of the cosine matrix of one split.

    "sum": eq. 6 of [notes] 关键设计 3, S~_pq = S_pq / (sum_q S_pq + eps). The variants the
    [summary] compares against it (appendix B, normalisation ablation; appendix H, removing the
    row-wise normalisation), in the plainest reading: "softmax" over each row (temperature 1),
    "rms" divides each row by its root mean square, sqrt(mean_q S_pq^2 + eps), and "none" keeps
    S itself. Every row runs over the split's valid tokens only.
    """
    if norm == "sum":
        return sim / (sim.sum(axis=1) + eps)[:, None]
    if norm == "softmax":
        e = np.exp(sim)
        return e / e.sum(axis=1)[:, None]
    if norm == "rms":
        return sim / np.sqrt((sim * sim).mean(axis=1) + eps)[:, None]
    if norm == "none":
        return sim
    raise ValueError(norm)


def dyn_context_split(z_b: np.ndarray, S: int, eps: float, i: int, norm: str = "sum") -> np.ndarray:
    """S~ Z_t for one split, valid rows only.

    [notes] 关键设计 2: the dynamic layer forms the cosine matrix N(Z_t) N(Z_t)^T over the
    tokens of the split and multiplies Z_t by it; 关键设计 3, eq. 6: each row is divided by
    its own sum plus eps (norm="sum"; the other normalisations are row_normalise's). Within-
    split, bidirectional (no mask between valid tokens).
    """
    N = z_b.shape[0]
    r = split_rows(N, S, i)
    zt = np.asarray(z_b[r.start:r.stop], dtype=np.float64)   # [n_valid, m_t]
    nz = unit_rows(zt)
    sim = nz @ nz.T                                            # S = N(Z_t) N(Z_t)^T
    s_tilde = row_normalise(sim, norm, eps)                    # eq. 6 for "sum"
    return s_tilde @ zt


def dyn_context(z: np.ndarray, S: int, eps: float, splits=None, norm: str = "sum"):
    """dyn_context_split over the listed (b, i) splits (default: all). Returns {(b, i): rows}."""
    B, N, _ = z.shape
    n_s = n_splits(N, S)
    if splits is None:
        splits = [(b, i) for b in range(B) for i in range(n_s)]
    return {(b, i): dyn_context_split(z[b], S, eps, i, norm) for b, i in splits}


# ----------------------------------------------------------------------------- contextualizer layers
def activation(a: np.ndarray, act: str) -> np.ndarray:
    """sigma of the contextualizer layers: the pages only ask for a monotone activation
    ([summary] 4, relevance-monotonic updates); this oracle offers identity and ReLU."""
    if act == "identity":
        return a
    if act == "relu":
        return np.maximum(a, 0.0)
    raise ValueError(act)


def static_layer_split(z_b: np.ndarray, S: int, V: np.ndarray, bias: np.ndarray, act: str, i: int) -> np.ndarray:
    """c_static(Z) = sigma(V Z_t + b) for one split, valid rows only ([notes] 关键设计 2: the
    static layer is a learned linear map of the split's tail followed by an activation; V is
    the S x S cross-embedding matrix of [summary] 3, mixing the split's token positions).
    b holds one value per token position of the split (a reading). Padding tokens are zero
    rows of Z_t, so they add nothing to the valid rows."""
    N = z_b.shape[0]
    zt = padded_split(z_b, S, i)                             # [S, m_t], zero padding rows
    y = np.asarray(V, dtype=np.float64) @ zt + np.asarray(bias, dtype=np.float64)[:, None]
    return activation(y, act)[: len(split_rows(N, S, i))]


def dyn_layer_split(z_b: np.ndarray, S: int, eps: float, bias: np.ndarray, act: str, i: int,
                    norm: str = "sum") -> np.ndarray:
    """c_dyn(Z) = sigma(S~ Z_t + b) for one split, valid rows only ([notes] 关键设计 2 and 3):
    the dynamic core of dyn_context_split, plus one bias per token position, then sigma."""
    core = dyn_context_split(z_b, S, eps, i, norm)
    b = np.asarray(bias, dtype=np.float64)[: core.shape[0], None]
    return activation(core + b, act)


def static_layer(z: np.ndarray, S: int, V: np.ndarray, bias: np.ndarray, act: str, splits=None):
    """static_layer_split over the listed (b, i) splits (default: all). Returns {(b, i): rows}."""
    B, N, _ = z.shape
    n_s = n_splits(N, S)
    if splits is None:
        splits = [(b, i) for b in range(B) for i in range(n_s)]
    return {(b, i): static_layer_split(z[b], S, V, bias, act, i) for b, i in splits}


def dyn_layer(z: np.ndarray, S: int, eps: float, bias: np.ndarray, act: str, splits=None, norm: str = "sum"):
    """dyn_layer_split over the listed (b, i) splits (default: all). Returns {(b, i): rows}."""
    B, N, _ = z.shape
    n_s = n_splits(N, S)
    if splits is None:
        splits = [(b, i) for b in range(B) for i in range(n_s)]
    return {(b, i): dyn_layer_split(z[b], S, eps, bias, act, i, norm) for b, i in splits}


# ----------------------------------------------------------------------------- enricher and fuser
def enrich(x: np.ndarray, U: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Z = ReLU(X U + b)^2 row by row ([notes] 整体框架: the enricher is a position-wise map
    Z = sigma(X U + b) from d up to m > d features; [summary] appendix A: its activation is
    ReLU squared, which keeps Z non-negative). x [..., d], U [d, m], b [m] -> [..., m]."""
    h = np.asarray(x, dtype=np.float64) @ np.asarray(U, dtype=np.float64) + np.asarray(b, dtype=np.float64)
    r = np.maximum(h, 0.0)
    return r * r


def fuse(z: np.ndarray, m_h: int, c: np.ndarray, O: np.ndarray, x_res: np.ndarray) -> np.ndarray:
    """Y = [Z_h || c(Z_t)] O + X ([notes] 整体框架: the fuser joins the bypassed head Z_h, the
    first m_h features of Z, with the contextualised tail and projects them back to d, then
    adds the layer's input; [summary] section 3). z [..., m] (only its head is read), c [..., m_t],
    O [m_h + m_t, d], x_res [..., d]."""
    z = np.asarray(z, dtype=np.float64)
    joined = np.concatenate([z[..., :m_h], np.asarray(c, dtype=np.float64)], axis=-1)
    return joined @ np.asarray(O, dtype=np.float64) + np.asarray(x_res, dtype=np.float64)


def neural_layer(x: np.ndarray, S: int, U: np.ndarray, b: np.ndarray, m_h: int, O: np.ndarray,
                 contextualise) -> np.ndarray:
    """One neural-processor layer over whole sequences: enrich, contextualise the tail split by
    split (contextualise(z_tail) -> {(b, i): rows}, e.g. a dynamic or static layer), fuse with
    the residual ([notes] 整体框架; [summary] section 3). x [B, N, d] -> [B, N, d]."""
    B, N, _ = x.shape
    z = enrich(x, U, b)
    c = assemble(contextualise(z[..., m_h:]), B, N, S, z.shape[-1] - m_h)
    return fuse(z, m_h, c, O, x)


def assemble(parts: dict, B: int, N: int, S: int, width: int) -> np.ndarray:
    """Stack per-split results {(b, i): rows} into a [B, N, width] array (NaN where absent)."""
    out = np.full((B, N, width), np.nan)
    for (b, i), rows in parts.items():
        out[b, i * S: i * S + rows.shape[0]] = rows
    return out
