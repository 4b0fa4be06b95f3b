"""GPU parity of the two contextualizer layers (static c = act(V Z_t + b), dynamic
c = act(S~ Z_t + b)) against the float64 oracle, through the C ABI.

Rows are compared as in the other parity tests (||g - o||_2 / ||o||_2 per token). With ReLU the
denominator is the oracle's row before the activation: ReLU is 1-Lipschitz, so a pre-activation
error within the tolerance stays within it after the activation, while the clipped row itself
can be arbitrarily small. Where the oracle's pre-activation value lies below minus the
tolerance times its row norm, the GPU output must be exactly zero.
"""
import sys

import numpy as np
import pytest
import torch

import attention_free_long_amd as A
from oracle import avey_oracle as O
from synth import CONFIGS, Config, layer_params, make_inputs

from helpers import TOL, dev_tensor, host_f64, split_rows_of, upload

pytestmark = pytest.mark.gpu

CASES = {
    # 8 splits of 256 (last one 208 tokens), 2 sequences, m_t = 320 (two 128-feature tiles and a 64-feature one)
    "small_bf16": Config("small_bf16", B=2, N=2000, d=256, S=256, k=3, m_t=320, m=384, dtype="bf16",
                         x_dist="mixture", n_centroids=16),
    # S = 512 (two 256-token halves per split), last split 40 tokens
    "s512_bf16": Config("s512_bf16", B=1, N=1576, d=128, S=512, k=2, m_t=192, m=256, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    # S = 64: four splits per workgroup of the dynamic layer, the last group partial
    "s64_bf16": Config("s64_bf16", B=1, N=700, d=64, S=64, k=2, m_t=64, m=128, dtype="bf16",
                       x_dist="mixture", n_centroids=8),
    # S = 128: two splits per workgroup; the last split 4 tokens, alone in a partial group
    "s128_bf16": Config("s128_bf16", B=2, N=900, d=64, S=128, k=2, m_t=136, m=200, dtype="bf16",
                        x_dist="mixture", n_centroids=8),
    "tiny": CONFIGS["tiny"],
    # S = 208 and m_t = 72 (multiples of 16 and 8 only): partial chunks in both layers
    "s208_bf16": Config("s208_bf16", B=1, N=1500, d=64, S=208, k=2, m_t=72, m=136, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    # S = 400: the S <= 512 dynamic kernel with a partial group of 128 tokens
    "s400_bf16": Config("s400_bf16", B=1, N=1300, d=64, S=400, k=2, m_t=200, m=264, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
}


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def check_layer(g, pre, post, cfg, tol, what):
    """g: GPU output [B, N, m_t]; pre / post: oracle rows per split before / after act."""
    worst = 0.0
    for (b, i), o_post in post.items():
        o_pre = pre[(b, i)]
        rows = g[b, split_rows_of(cfg.N, cfg.S, i)]
        num = np.linalg.norm(rows - o_post, axis=-1)
        den = np.maximum(np.linalg.norm(o_pre, axis=-1), 1e-30)
        err = float((num / den).max())
        assert err <= tol, f"{what} split {(b, i)}: {err:.3e}"
        worst = max(worst, err)
        clipped = o_pre < -tol * den[:, None]
        if o_post is not o_pre:
            assert np.all(rows[clipped] == 0.0), f"{what} split {(b, i)}: ReLU left a negative value"
            assert np.all(rows >= 0.0)
    return worst


@pytest.mark.parametrize("act", ["identity", "relu"])
@pytest.mark.parametrize("name", list(CASES))
def test_layers_parity(gpu_ok, name, act):
    cfg = CASES[name]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    V, bias = layer_params(inp)
    say(f"{name}/{act}: static + dynamic layer B={cfg.B} N={cfg.N} S={cfg.S} m_t={cfg.m_t}")
    _, _, _, z_tail = upload(inp)
    Vd = dev_tensor(V, cfg.dtype)
    bd = torch.from_numpy(bias).to("cuda")
    g_s = host_f64(A.avey_static_layer(z_tail, Vd, cfg.S, bd, act))
    g_d = host_f64(A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, act))
    torch.cuda.synchronize()

    z64 = inp.z_tail_f64()
    V64 = inp._as_f64(V)
    b64 = bias.astype(np.float64)
    s_pre = O.static_layer(z64, cfg.S, V64, b64, "identity")
    s_post = s_pre if act == "identity" else O.static_layer(z64, cfg.S, V64, b64, act)
    d_pre = O.dyn_layer(z64, cfg.S, cfg.eps, b64, "identity")
    d_post = d_pre if act == "identity" else O.dyn_layer(z64, cfg.S, cfg.eps, b64, act)
    ws = check_layer(g_s, s_pre, s_post, cfg, tol, "static")
    wd = check_layer(g_d, d_pre, d_post, cfg, tol, "dynamic")
    if act == "relu":
        frac = np.mean([np.mean(v == 0.0) for v in d_post.values()])
        assert 0.05 < frac < 0.95, f"bias leaves ReLU nothing to do: {frac:.2f} of outputs zero"
    say(f"{name}/{act}: worst relative errors static {ws:.2e}, dynamic {wd:.2e}")


@pytest.mark.parametrize("name", ["small_bf16", "s512_bf16", "tiny"])
def test_static_identity_and_permutation_exact(gpu_ok, name):
    """V = I returns Z_t bit for bit; a permutation V moves whole tokens (a slot past the split's
    valid tokens gives a zero row); a bias of zeros with ReLU clips exactly the negatives."""
    cfg = CASES[name]
    inp = make_inputs(cfg)
    say(f"{name}: static layer with identity and permutation V")
    _, _, _, z_tail = upload(inp)
    tdt = z_tail.dtype
    S = cfg.S
    eye = torch.eye(S, dtype=tdt, device="cuda")
    g = A.avey_static_layer(z_tail, eye, S)
    assert torch.equal(g, z_tail)
    perm = np.random.default_rng(5).permutation(S)
    Vp = torch.from_numpy(np.eye(S, dtype=np.float32)[perm]).to("cuda").to(tdt)
    g = host_f64(A.avey_static_layer(z_tail, Vp, S))
    z64 = inp.z_tail_f64()
    for b in range(cfg.B):
        for i in range(cfg.n_s):
            r = split_rows_of(cfg.N, S, i)
            for s_ in range(r.stop - r.start):
                src = i * S + perm[s_]
                want = z64[b, src] if src < cfg.N else np.zeros(cfg.m_t)
                assert np.array_equal(g[b, r.start + s_], want), (b, i, s_)
    neg = -z_tail                                     # exact negation: every value <= 0
    g = A.avey_static_layer(neg, eye, S, torch.zeros(S, device="cuda"), "relu")
    assert torch.count_nonzero(g).item() == 0


@pytest.mark.parametrize("name", ["small_bf16", "s512_bf16", "tiny"])
def test_dyn_layer_defaults_equal_core(gpu_ok, name):
    cfg = CASES[name]
    inp = make_inputs(cfg)
    say(f"{name}: dynamic layer without bias and activation vs the core")
    _, _, _, z_tail = upload(inp)
    core = A.avey_dyn_context(z_tail, cfg.S, cfg.eps)
    lay = A.avey_dyn_layer(z_tail, cfg.S, cfg.eps)
    assert torch.equal(core, lay)


def test_static_then_dynamic(gpu_ok):
    """S -> D: the static layer's output (contiguous, row stride m_t) feeds the dynamic layer.
    Each GPU layer is compared with the oracle on the GPU's own input to that layer."""
    cfg = CASES["small_bf16"]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    V, bias = layer_params(inp)
    say("static (ReLU) -> dynamic (ReLU), small_bf16")
    _, _, _, z_tail = upload(inp)
    bd = torch.from_numpy(bias).to("cuda")
    h = A.avey_static_layer(z_tail, dev_tensor(V, cfg.dtype), cfg.S, bd, "relu")
    out = A.avey_dyn_layer(h, cfg.S, cfg.eps, bd, "relu")
    torch.cuda.synchronize()
    h64, g = host_f64(h), host_f64(out)
    b64 = bias.astype(np.float64)
    pre = O.dyn_layer(h64, cfg.S, cfg.eps, b64, "identity")
    post = O.dyn_layer(h64, cfg.S, cfg.eps, b64, "relu")
    check_layer(g, pre, post, cfg, tol, "S->D dynamic")
    # the static layer's own output, against the oracle on the original tail
    z64 = inp.z_tail_f64()
    V64 = inp._as_f64(V)
    check_layer(h64, O.static_layer(z64, cfg.S, V64, b64, "identity"),
                O.static_layer(z64, cfg.S, V64, b64, "relu"), cfg, tol, "S->D static")


def test_layers_full_size_every_split(gpu_ok):
    """The 2 x 32768-token workload (S = 256, m_t = 1536 at row stride 3072), both layers with
    bias and ReLU, every split against the oracle."""
    cfg = CONFIGS["long"]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    V, bias = layer_params(inp)
    say(f"long: static + dynamic layer, B={cfg.B} N={cfg.N} m_t={cfg.m_t}, every split")
    _, _, _, z_tail = upload(inp)
    bd = torch.from_numpy(bias).to("cuda")
    g_s = A.avey_static_layer(z_tail, dev_tensor(V, cfg.dtype), cfg.S, bd, "relu")
    g_d = A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "relu")
    torch.cuda.synchronize()
    V64 = inp._as_f64(V)
    b64 = bias.astype(np.float64)
    worst = 0.0
    for b in range(cfg.B):
        zb = inp.z_tail_f64(b)
        gs_b, gd_b = host_f64(g_s[b]), host_f64(g_d[b])
        for i in range(cfg.n_s):
            r = split_rows_of(cfg.N, cfg.S, i)
            s_pre = O.static_layer_split(zb, cfg.S, V64, b64, "identity", i)
            d_pre = O.dyn_layer_split(zb, cfg.S, cfg.eps, b64, "identity", i)
            for g, pre, what in ((gs_b[r], s_pre, "static"), (gd_b[r], d_pre, "dynamic")):
                post = np.maximum(pre, 0.0)
                den = np.linalg.norm(pre, axis=-1)
                err = float((np.linalg.norm(g - post, axis=-1) / den).max())
                assert err <= tol, f"{what} split {(b, i)}: {err:.3e}"
                assert np.all(g[pre < -tol * den[:, None]] == 0.0)
                worst = max(worst, err)
        del zb, gs_b, gd_b
    say(f"long: {cfg.B * cfg.n_s} splits of both layers, worst {worst:.2e} (bar {tol})")


def test_static_layer_persistent_kernel(gpu_ok):
    """The static layer at 256 units (2 x 32668 tokens, S = 256, m_t = 64): every split, with
    bias and ReLU, on the persistent kernel."""
    cfg = Config("p256", B=2, N=32668, d=64, S=256, k=0, m_t=64, m=64, dtype="bf16",
                 x_dist="mixture", n_centroids=32, z_kind="relu2_x")
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    V, bias = layer_params(inp)
    say(f"static layer, persistent kernel: B={cfg.B} N={cfg.N} m_t={cfg.m_t}")
    _, _, _, z_tail = upload(inp)
    bd = torch.from_numpy(bias).to("cuda")
    g = host_f64(A.avey_static_layer(z_tail, dev_tensor(V, cfg.dtype), cfg.S, bd, "relu"))
    torch.cuda.synchronize()
    z64 = inp.z_tail_f64()
    V64 = inp._as_f64(V)
    b64 = bias.astype(np.float64)
    w = check_layer(g, O.static_layer(z64, cfg.S, V64, b64, "identity"),
                    O.static_layer(z64, cfg.S, V64, b64, "relu"), cfg, tol, "static")
    say(f"static layer, persistent kernel: worst {w:.2e}")


@pytest.mark.parametrize("norm", ["softmax", "rms", "none"])
@pytest.mark.parametrize("name", list(CASES))
def test_dyn_norm_variants(gpu_ok, name, norm):
    """The dynamic layer with each row normalisation other than eq. 6, with a bias, against the
    oracle on every split (identity activation, so rows compare by their own norm)."""
    cfg = CASES[name]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    _, bias = layer_params(inp)
    say(f"{name}/{norm}: dynamic layer B={cfg.B} N={cfg.N} S={cfg.S} m_t={cfg.m_t}")
    _, _, _, z_tail = upload(inp)
    bd = torch.from_numpy(bias).to("cuda")
    g = host_f64(A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "identity", norm=norm))
    torch.cuda.synchronize()
    ref = O.dyn_layer(inp.z_tail_f64(), cfg.S, cfg.eps, bias.astype(np.float64), "identity", norm=norm)
    w = check_layer(g, ref, ref, cfg, tol, f"dynamic/{norm}")
    say(f"{name}/{norm}: worst relative error {w:.2e}")


# Grids whose last wave is partial: on a 256-CU device the splits (or groups) of that wave are
# each shared by several workgroups, every one computing the split's G and writing its own
# range of feature tiles, beside whole splits of the full wave in the same launch.
WAVE_TAIL = {
    # 300 splits (the last 100 tokens); m_t = 520: five feature tiles, the last one partial;
    # 44 splits in the last wave, four workgroups each (tiles 0 | 1 | 2 | 3-4)
    "tail_s256": Config("tail_s256", B=1, N=76644, d=64, S=256, k=2, m_t=520, m=600, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
    # S = 128: 290 groups of two splits (the last group a single 78-token split), m_t = 392
    "tail_s128": Config("tail_s128", B=1, N=74190, d=64, S=128, k=2, m_t=392, m=456, dtype="bf16",
                        x_dist="mixture", n_centroids=16),
}


@pytest.mark.parametrize("name", list(WAVE_TAIL))
def test_dyn_wave_tail_every_split(gpu_ok, name):
    """The dynamic core, and the dynamic layer with bias, ReLU and softmax weights, on grids with
    a partial last wave: every split against the oracle."""
    cfg = WAVE_TAIL[name]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    _, bias = layer_params(inp)
    say(f"{name}: dynamic core and layer B={cfg.B} N={cfg.N} S={cfg.S} m_t={cfg.m_t}, every split")
    _, _, _, z_tail = upload(inp)
    bd = torch.from_numpy(bias).to("cuda")
    g_core = host_f64(A.avey_dyn_context(z_tail, cfg.S, cfg.eps))
    g_lay = host_f64(A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, bd, "relu", norm="softmax"))
    torch.cuda.synchronize()
    z64 = inp.z_tail_f64()
    b64 = bias.astype(np.float64)
    core = {(0, i): O.dyn_context_split(z64[0], cfg.S, cfg.eps, i) for i in range(cfg.n_s)}
    w1 = check_layer(g_core, core, core, cfg, tol, "dynamic core")
    pre = O.dyn_layer(z64, cfg.S, cfg.eps, b64, "identity", norm="softmax")
    post = O.dyn_layer(z64, cfg.S, cfg.eps, b64, "relu", norm="softmax")
    w2 = check_layer(g_lay, pre, post, cfg, tol, "dynamic layer/softmax")
    say(f"{name}: {cfg.n_s} splits, worst {w1:.2e} (core), {w2:.2e} (layer)")


@pytest.mark.parametrize("norm", ["softmax", "rms"])
def test_dyn_norm_full_size_every_split(gpu_ok, norm):
    """Softmax and RMS normalisation on the 2 x 32768-token workload (m_t = 1536 at row stride
    3072), every split against the oracle."""
    cfg = CONFIGS["long"]
    tol = TOL[cfg.dtype]["out"]
    inp = make_inputs(cfg)
    say(f"long/{norm}: dynamic layer, every split")
    _, _, _, z_tail = upload(inp)
    g = A.avey_dyn_layer(z_tail, cfg.S, cfg.eps, norm=norm)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(cfg.B):
        zb = inp.z_tail_f64(b)
        g_b = host_f64(g[b])
        for i in range(cfg.n_s):
            r = split_rows_of(cfg.N, cfg.S, i)
            o = O.dyn_context_split(zb, cfg.S, cfg.eps, i, norm)
            err = float((np.linalg.norm(g_b[r] - o, axis=-1) / np.linalg.norm(o, axis=-1)).max())
            assert err <= tol, f"{norm} split {(b, i)}: {err:.3e}"
            worst = max(worst, err)
        del zb, g_b
    say(f"long/{norm}: {cfg.B * cfg.n_s} splits, worst {worst:.2e} (bar {tol})")
