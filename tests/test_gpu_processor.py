"""GPU parity of the enricher and fuser (the dense GEMMs of a neural-processor layer) and of a
whole layer X -> Z -> c(Z_t) -> Y, through the C ABI, against the float64 oracle.

Every stage is compared on its own GPU input (the values each kernel actually read), and the
chain end to end against the oracle's unrounded chain. Rows compare by ||g - o|| / ||o||.
"""
import sys

import numpy as np
import pytest
import torch

import attention_free_long_amd as A
from oracle import avey_oracle as O
from synth import CONFIGS, Config, make_inputs, processor_params

from helpers import TOL, dev_tensor, host_f64

pytestmark = pytest.mark.gpu

# (config, m, m_h): the enricher widens d to m; the tail is the last m - m_h columns
CASES = {
    # M = 4000 tokens: 16 token tiles, the last one ragged; m = 576 (2 full feature tiles + 64)
    "small_bf16": (Config("small_bf16", B=2, N=2000, d=256, S=256, k=3, m_t=256, m=576, dtype="bf16",
                          x_dist="mixture", n_centroids=16, z_kind="relu2_x"), 576, 320),
    # no head: the whole of Z goes through the contextualizer
    "nohead_bf16": (Config("nohead_bf16", B=1, N=1100, d=128, S=256, k=2, m_t=128, m=128, dtype="bf16",
                           x_dist="mixture", n_centroids=16, z_kind="relu2_x"), 256, 0),
    "tiny": (CONFIGS["tiny"], 128, 64),
}


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def rows_err(g, o):
    g = g.reshape(-1, g.shape[-1])
    o = o.reshape(-1, o.shape[-1])
    return float((np.linalg.norm(g - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-30)).max())


def as64(a, dtype):
    from synth import bf16_bits_to_f32
    return (bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_enrich_and_fuse(gpu_ok, name):
    cfg, m, m_h = CASES[name]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    U, b, Ow = processor_params(cfg, m)
    say(f"{name}: enrich + fuse, M={cfg.B * cfg.N} d={cfg.d} m={m} m_h={m_h}")
    x = dev_tensor(inp.x, cfg.dtype)
    z = A.avey_enrich(x, dev_tensor(U, cfg.dtype), torch.from_numpy(b).cuda())
    # the contextualised tail: any [B, N, m_t] tensor will do for the fuser; use the dynamic layer
    c = A.avey_dyn_layer(z[..., m_h:], cfg.S, cfg.eps)
    y = A.avey_fuse(z, m_h, c, dev_tensor(Ow, cfg.dtype), x)
    torch.cuda.synchronize()
    x64 = inp.x_f64()
    z_g, c_g, y_g = host_f64(z), host_f64(c), host_f64(y)
    ez = rows_err(z_g, O.enrich(x64, as64(U, cfg.dtype), b.astype(np.float64)))
    assert ez <= tol, f"enrich: {ez:.3e}"
    ey = rows_err(y_g, O.fuse(z_g, m_h, c_g, as64(Ow, cfg.dtype), x64))
    assert ey <= tol, f"fuse: {ey:.3e}"
    say(f"{name}: worst row errors enrich {ez:.2e}, fuse {ey:.2e}")


@pytest.mark.parametrize("name", list(CASES))
def test_neural_layer_chain(gpu_ok, name):
    """X -> enrich -> dynamic layer (ReLU) on the tail -> fuse, end to end against the oracle's
    chain in float64 (intermediates not rounded)."""
    cfg, m, m_h = CASES[name]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    U, b, Ow = processor_params(cfg, m)
    say(f"{name}: neural-processor layer chain")
    x = dev_tensor(inp.x, cfg.dtype)
    z = A.avey_enrich(x, dev_tensor(U, cfg.dtype), torch.from_numpy(b).cuda())
    c = A.avey_dyn_layer(z[..., m_h:], cfg.S, cfg.eps, act="relu")
    y = host_f64(A.avey_fuse(z, m_h, c, dev_tensor(Ow, cfg.dtype), x))
    torch.cuda.synchronize()
    ctx = lambda zt: O.dyn_layer(zt, cfg.S, cfg.eps, np.zeros(cfg.S), "relu")
    ref = O.neural_layer(inp.x_f64(), cfg.S, as64(U, cfg.dtype), b.astype(np.float64), m_h,
                         as64(Ow, cfg.dtype), ctx)
    e = rows_err(y, ref)
    assert e <= tol, f"layer: {e:.3e}"
    say(f"{name}: layer worst row error {e:.2e}")


def test_enrich_fuse_full_size_every_token(gpu_ok):
    """The 2 x 32768-token workload (d = 768, m = 3072, tail 1536): every token of the enricher
    and of the fuser against the oracle (the fuser on the GPU's own Z and c)."""
    cfg = CONFIGS["long"]
    m, m_h = cfg.m, cfg.m - cfg.m_t
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    U, b, Ow = processor_params(cfg, m)
    say(f"long: enrich + fuse, M={cfg.B * cfg.N} d={cfg.d} m={m}, every token")
    x = dev_tensor(inp.x, cfg.dtype)
    z = A.avey_enrich(x, dev_tensor(U, cfg.dtype), torch.from_numpy(b).cuda())
    c = A.avey_dyn_layer(z[..., m_h:], cfg.S, cfg.eps)
    y = A.avey_fuse(z, m_h, c, dev_tensor(Ow, cfg.dtype), x)
    torch.cuda.synchronize()
    U64, O64 = as64(U, cfg.dtype), as64(Ow, cfg.dtype)
    for bb in range(cfg.B):
        xs = inp.x_f64(bb)
        z_b = host_f64(z[bb])
        ez = rows_err(z_b, O.enrich(xs, U64, b.astype(np.float64)))
        assert ez <= tol, f"enrich b={bb}: {ez:.3e}"
        ey = rows_err(host_f64(y[bb]), O.fuse(z_b, m_h, host_f64(c[bb]), O64, xs))
        assert ey <= tol, f"fuse b={bb}: {ey:.3e}"
        say(f"long: sequence {bb}, {cfg.N} tokens: enrich {ez:.2e}, fuse {ey:.2e} (bar {tol})")
        del z_b


def test_gemm_edges(gpu_ok):
    """One partial token tile (100 tokens), the narrowest widths (d = m_h = m_t = 64), no bias;
    and empty inputs, which enqueue nothing."""
    cfg = Config("edge", B=1, N=100, d=64, S=64, k=1, m_t=64, m=64, dtype="bf16", z_kind="relu2_x")
    m, m_h = 128, 64
    inp = make_inputs(cfg)
    U, _, Ow = processor_params(cfg, m)
    say("gemm edges: 100 tokens, d = 64, m = 128, no bias")
    x = dev_tensor(inp.x, cfg.dtype)
    z = A.avey_enrich(x, dev_tensor(U, cfg.dtype))
    c = z[..., m_h:].contiguous()
    y = A.avey_fuse(z, m_h, c, dev_tensor(Ow, cfg.dtype), x)
    torch.cuda.synchronize()
    x64 = inp.x_f64()
    z_g = host_f64(z)
    assert rows_err(z_g, O.enrich(x64, as64(U, cfg.dtype), np.zeros(m))) <= TOL["bf16"]["out"]
    assert rows_err(host_f64(y), O.fuse(z_g, m_h, host_f64(c), as64(Ow, cfg.dtype), x64)) <= TOL["bf16"]["out"]
    e = torch.empty((1, 0, 64), device="cuda", dtype=torch.bfloat16)
    assert A.avey_enrich(e, dev_tensor(U, cfg.dtype)).shape == (1, 0, m)
