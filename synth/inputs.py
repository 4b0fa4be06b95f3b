"""Seeded synthetic workloads for the Avey-B ranker and dynamic contextualizer.

The workloads stand in for the length sweep the Avey-B efficiency study runs (papernotes.org
ICLR2026 note on Avey-B, section on efficiency experiments: batch 8, lengths from 128 to 96K
tokens on one GPU), at the split size S=256 and top-k=3 that the same note reports as the best
setting (section on losses and training strategy). No dataset is used: every tensor is drawn
here from a numpy PCG64 generator seeded through ``SeedSequence(seed).spawn``.

Layout of what is returned (all host numpy arrays, C-contiguous):

* ``x``   token embeddings X, shape [B, N, d]. For bf16 configs the array holds bf16 bit
  patterns (uint16); for fp32 configs it holds float32 values.
* ``P``   compression matrix, shape [S, (k+1)S], same storage type as ``x``.
* ``z``   the enricher output Z, shape [B, N, m]; only its last ``m_t`` columns (the tail Z_t)
  are meaningful. The head columns hold NaN so that any read of them shows up downstream.

bf16 values are produced from float32 with round-to-nearest-even, and the same bits feed both
the oracle and the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


def n_splits(N: int, S: int) -> int:
    """Number of S-token splits covering N tokens (the last one zero-padded)."""
    return -(-N // S)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns with round-to-nearest-even (NaN stays a quiet NaN)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    N: int
    d: int
    S: int
    k: int
    m_t: int            # width of the tail Z_t fed to the dynamic layer
    m: int              # full enricher width; Z rows have stride m, the tail is the last m_t columns
    dtype: str          # "f32" or "bf16"
    eps: float = 1e-8
    x_dist: str = "iid"         # "iid" N(0,1) or "mixture"
    n_centroids: int = 0
    noise: float = 0.3
    dup_splits: int = 0         # per sequence: this many splits overwritten by copies of others
    p_init: str = "normal"      # "normal" N(0, p_std^2) or "xavier" uniform
    p_std: float = 0.02
    u_std: float = 0.02
    z_kind: str = "relu2_xu"    # "relu2_xu": Z_t = ReLU(X U_t)^2 ; "relu2_x": Z_t = ReLU(X)^2
    seed: int = 0

    @property
    def n_s(self) -> int:
        return n_splits(self.N, self.S)

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads. Tiny is the fp32 parity case; Long is the headline configuration.
CONFIGS: dict[str, Config] = {
    "tiny": Config("tiny", B=1, N=1000, d=64, S=64, k=3, m_t=64, m=64, dtype="f32",
                   p_init="xavier", z_kind="relu2_x"),
    "base": Config("base", B=8, N=8192, d=768, S=256, k=3, m_t=1536, m=3072, dtype="bf16"),
    "long": Config("long", B=2, N=32768, d=768, S=256, k=3, m_t=1536, m=3072, dtype="bf16",
                   x_dist="mixture", n_centroids=128),
    "extreme": Config("extreme", B=1, N=98304, d=768, S=256, k=3, m_t=1536, m=3072, dtype="bf16",
                      x_dist="mixture", n_centroids=128),
    "wide": Config("wide", B=4, N=16384, d=1024, S=512, k=7, m_t=2048, m=4096, dtype="bf16",
                   x_dist="mixture", n_centroids=64, dup_splits=2),
}


@dataclass
class Inputs:
    cfg: Config
    x: np.ndarray                 # [B, N, d]   uint16 bf16 bits or float32
    P: np.ndarray                 # [S, (k+1)S] uint16 bf16 bits or float32
    z: np.ndarray                 # [B, N, m]   uint16 bf16 bits or float32; tail = last m_t columns
    meta: dict = field(default_factory=dict)

    @property
    def tail_col(self) -> int:
        return self.cfg.m - self.cfg.m_t

    def _as_f64(self, a: np.ndarray) -> np.ndarray:
        if self.cfg.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)

    def x_f64(self, b: int | None = None) -> np.ndarray:
        """X (or X[b]) as float64, exactly the values the GPU sees."""
        return self._as_f64(self.x if b is None else self.x[b])

    def P_f64(self) -> np.ndarray:
        return self._as_f64(self.P)

    def z_tail_f64(self, b: int | None = None, rows: slice | None = None) -> np.ndarray:
        """The tail Z_t (or a batch row / token range of it) as float64."""
        z = self.z if b is None else self.z[b]
        if rows is not None:
            z = z[..., rows, :] if b is None else z[rows]
        return self._as_f64(z[..., self.tail_col:])


def _store(cfg: Config, a32: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(a32) if cfg.dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def make_inputs(cfg: Config | str, seed: int | None = None) -> Inputs:
    """Draw the workload ``cfg`` (a Config or a key of CONFIGS) with the given seed (default cfg.seed)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if seed is not None:
        cfg = cfg.with_(seed=seed)
    ss = np.random.SeedSequence(cfg.seed)
    r_x, r_cent, r_assign, r_p, r_u, r_dup = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6))
    B, N, d, S, k = cfg.B, cfg.N, cfg.d, cfg.S, cfg.k

    # Token embeddings X.
    if cfg.x_dist == "iid":
        x32 = r_x.standard_normal((B, N, d), dtype=np.float32)
    elif cfg.x_dist == "mixture":
        cent = r_cent.standard_normal((cfg.n_centroids, d), dtype=np.float32)
        assign = r_assign.integers(0, cfg.n_centroids, size=(B, N))
        x32 = cent[assign]
        x32 += np.float32(cfg.noise) * r_x.standard_normal((B, N, d), dtype=np.float32)
    else:
        raise ValueError(cfg.x_dist)
    x = _store(cfg, x32)
    del x32

    # Exact duplicate splits (copies of whole S-token splits, all four indices distinct).
    dups = []
    if cfg.dup_splits:
        full = N // S  # only whole splits take part
        for b in range(B):
            pick = r_dup.choice(full, size=2 * cfg.dup_splits, replace=False)
            src, dst = pick[: cfg.dup_splits], pick[cfg.dup_splits:]
            for s_, t_ in zip(src, dst):
                x[b, t_ * S:(t_ + 1) * S] = x[b, s_ * S:(s_ + 1) * S]
                dups.append((b, int(s_), int(t_)))

    # Compression matrix P, S x (k+1)S.
    fan_out, fan_in = S, (k + 1) * S
    if cfg.p_init == "xavier":
        a = np.sqrt(6.0 / (fan_in + fan_out))
        p32 = r_p.uniform(-a, a, size=(fan_out, fan_in)).astype(np.float32)
    else:
        p32 = (np.float32(cfg.p_std) * r_p.standard_normal((fan_out, fan_in), dtype=np.float32))
    P = _store(cfg, p32)

    # Enricher output Z [B, N, m]: NaN head, tail Z_t = ReLU(X U_t)^2 (or ReLU(X)^2 for Tiny).
    m, m_t = cfg.m, cfg.m_t
    if cfg.dtype == "bf16":
        z = np.empty((B, N, m), dtype=np.uint16)
        z[..., : m - m_t] = BF16_QNAN
    else:
        z = np.empty((B, N, m), dtype=np.float32)
        z[..., : m - m_t] = np.nan
    xf = bf16_bits_to_f32 if cfg.dtype == "bf16" else (lambda a: a)
    if cfg.z_kind == "relu2_x":
        if m_t != d:
            raise ValueError("relu2_x needs m_t == d")
        t = np.maximum(xf(x), 0.0).astype(np.float32)
        z[..., m - m_t:] = _store(cfg, t * t)
    elif cfg.z_kind == "relu2_xu":
        U = (np.float32(cfg.u_std) * r_u.standard_normal((d, m_t), dtype=np.float32))
        rows = 8192
        for b in range(B):
            for r0 in range(0, N, rows):
                h = xf(x[b, r0:r0 + rows]) @ U
                np.maximum(h, 0.0, out=h)
                h *= h
                z[b, r0:r0 + rows, m - m_t:] = _store(cfg, h)
    else:
        raise ValueError(cfg.z_kind)

    return Inputs(cfg=cfg, x=x, P=P, z=z, meta={"dups": dups})


def layer_params(inp: Inputs) -> tuple[np.ndarray, np.ndarray]:
    """Weights of a static contextualizer layer and one bias vector for either layer.

    * ``V`` [S, S], stored as ``x`` is: a Toeplitz band with signed values, decaying with the
      distance from the diagonal, plus a small dense signed part. Learned static matrices come
      out Toeplitz-like, diagonally dominant and concentrated near the diagonal, with signed
      weights (paperlayer.ai "Avey-B" summary, appendix B).
    * ``bias`` [S] float32, one value per token position of a split: N(0, 1) scaled by the spread
      of the tail values and shifted down by their mean, so that a ReLU after the layer clips a
      good part of each output while leaving the rest (statistics from at most 4096 rows).

    Drawn from the seed's streams 6 and 7, after the six ``make_inputs`` uses.
    """
    cfg = inp.cfg
    S = cfg.S
    r_v, r_b = (np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(cfg.seed).spawn(8)[6:])
    delta = np.arange(S)[:, None] - np.arange(S)[None, :]
    diag = r_v.standard_normal(2 * S - 1).astype(np.float32)
    v32 = np.exp(-np.abs(delta) / 4.0).astype(np.float32) * diag[delta + S - 1]
    v32 += np.float32(0.5 / np.sqrt(S)) * r_v.standard_normal((S, S), dtype=np.float32)
    V = _store(cfg, v32)
    sample = inp.z_tail_f64(0, slice(0, min(cfg.N, 4096)))
    mu, sd = float(sample.mean()), float(sample.std())
    bias = (sd * r_b.standard_normal(S) - mu).astype(np.float32)
    return V, bias


def processor_params(cfg: Config, m: int, u_std: float | None = None, o_std: float | None = None,
                     b_std: float = 0.5, seed: int | None = None):
    """Weights of the enricher and fuser around the contextualizer: U [d, m] and O [m, d] drawn
    N(0, std^2) (defaults 1/sqrt(d) and 1/sqrt(m), so that X U and [Z_h || c] O are of order
    one, as with the N(0, 0.02^2) initialisation at the bf16 workloads' widths they are not),
    b [m] float32 N(0, b_std^2). U and O are stored as ``x`` is. Drawn from the seed's stream 8."""
    d = cfg.d
    s = cfg.seed if seed is None else seed
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence(s).spawn(9)[8]))
    u_std = (1.0 / np.sqrt(d)) if u_std is None else u_std
    o_std = (1.0 / np.sqrt(m)) if o_std is None else o_std
    U = _store(cfg, (np.float32(u_std) * r.standard_normal((d, m), dtype=np.float32)))
    O = _store(cfg, (np.float32(o_std) * r.standard_normal((m, d), dtype=np.float32)))
    b = (b_std * r.standard_normal(m)).astype(np.float32)
    return U, b, O
