"""Avey-B bidirectional ranker and dynamic contextualizer core on MI355X (gfx950).

Thin ctypes binding over libavey.so (see include/avey.h): argument marshalling only, every step
runs in the library's HIP kernels. torch supplies device memory and the current stream.

    scores, idx, w = avey_split_rank(x, S, k)        # no workspace: token norms on chip
    xhat = avey_select_compress(x, idx, w, P, S, residual=True)
    out = avey_dyn_context(z_tail, S, eps)
    out = avey_dyn_layer(z_tail, S, eps, bias, act="relu")       # sigma(S~ Z_t + b)
    out = avey_static_layer(z_tail, V, S, bias, act="identity")  # sigma(V Z_t + b)
    z = avey_enrich(x, U, b)                                    # ReLU(X U + b)^2
    y = avey_fuse(z, m_h, c, O, x)                              # [Z_h || c] O + X

Tensors are [B, N, width] with unit stride along width and any row stride (ld); bf16 or fp32.
There is no fallback: if libavey.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libavey.so")

AVEY_F32, AVEY_BF16 = 0, 1
AVEY_ACT = {"identity": 0, "relu": 1}
AVEY_NORM = {"sum": 0, "softmax": 1, "rms": 2, "none": 3}
AVEY_ABI_VERSION = 2

EXPORTS = (
    "avey_abi_version",
    "avey_status_str",
    "avey_maxsim",
    "avey_rank_workspace_bytes",
    "avey_maxsim_prepare",
    "avey_maxsim_scores",
    "avey_topk_norm",
    "avey_topk_norm_preceding",
    "avey_split_rank",
    "avey_split_rank_preceding",
    "avey_split_rank_noalloc",
    "avey_select_compress",
    "avey_dyn_context",
    "avey_dyn_layer",
    "avey_static_layer",
    "avey_enrich",
    "avey_fuse",
    "avey_probe_mfma_flops",
    "avey_probe_mfma_bf16",
    "avey_probe_copy",
)


class AveyError(RuntimeError):
    """A libavey call returned a non-zero status (or the library could not be loaded)."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libavey.so once and declare the C signatures. Raises AveyError if it is missing."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise AveyError("load_library", -100, f"{path} not found; build it with `python -m attention_free_long_amd.build`")
    lib = ctypes.CDLL(path)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    lib.avey_abi_version.restype = i32
    lib.avey_abi_version.argtypes = []
    lib.avey_status_str.restype = ctypes.c_char_p
    lib.avey_status_str.argtypes = [i32]
    lib.avey_rank_workspace_bytes.restype = i64
    lib.avey_rank_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.avey_maxsim_prepare.restype = i32
    lib.avey_maxsim_prepare.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, vp]
    lib.avey_maxsim_scores.restype = i32
    lib.avey_maxsim_scores.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp]
    lib.avey_topk_norm.restype = i32
    lib.avey_topk_norm.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.avey_topk_norm_preceding.restype = i32
    lib.avey_topk_norm_preceding.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.avey_maxsim.restype = i32
    lib.avey_maxsim.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, vp]
    for fn in (lib.avey_split_rank, lib.avey_split_rank_preceding, lib.avey_split_rank_noalloc):
        fn.restype = i32
        fn.argtypes = [vp, i32, i64, i64, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.avey_select_compress.restype = i32
    lib.avey_select_compress.argtypes = [vp, i32, i64, i64, i64, i64, i32, i32, vp, vp, vp, i32, vp, i64, vp]
    lib.avey_dyn_context.restype = i32
    lib.avey_dyn_context.argtypes = [vp, i32, i64, i64, i64, i64, i32, f32, vp, i64, vp]
    lib.avey_dyn_layer.restype = i32
    lib.avey_dyn_layer.argtypes = [vp, i32, i64, i64, i64, i64, i32, f32, i32, vp, i32, vp, i64, vp]
    lib.avey_enrich.restype = i32
    lib.avey_enrich.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp]
    lib.avey_fuse.restype = i32
    lib.avey_fuse.argtypes = [vp, i32, i64, i64, i64, vp, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.avey_static_layer.restype = i32
    lib.avey_static_layer.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, vp, i32, vp, i64, vp]
    lib.avey_probe_mfma_flops.restype = i64
    lib.avey_probe_mfma_flops.argtypes = [i64]
    lib.avey_probe_mfma_bf16.restype = i32
    lib.avey_probe_mfma_bf16.argtypes = [i64, i32, vp, vp]
    lib.avey_probe_copy.restype = i32
    lib.avey_probe_copy.argtypes = [vp, vp, i64, vp]
    ver = lib.avey_abi_version()
    if ver != AVEY_ABI_VERSION:
        raise AveyError("load_library", -101, f"ABI version {ver}, expected {AVEY_ABI_VERSION}")
    _lib_handle = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise AveyError(fn, status, load_library().avey_status_str(status).decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return AVEY_BF16
    if t.dtype == torch.float32:
        return AVEY_F32
    raise AveyError("dtype", -3, f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _rows(t, name: str):
    """(B, N, width, ld) of a [B, N, width] tensor with unit inner stride and batch stride N*ld."""
    if t.dim() != 3:
        raise AveyError(name, -2, f"{name} must be [B, N, width], got {tuple(t.shape)}")
    B, N, w = t.shape
    if not t.is_cuda:
        raise AveyError(name, -1, f"{name} must be a device tensor")
    if w > 0 and t.stride(2) != 1:
        raise AveyError(name, -2, f"{name} must have unit stride along its last axis")
    ld = t.stride(1) if N > 1 else max(w, t.stride(1))
    if B > 1 and N > 0 and t.stride(0) != N * ld:
        raise AveyError(name, -2, f"{name} batch stride must be N * row stride")
    return B, N, w, ld


def _arg(t, fn: str, name: str, like, dtype, shape=None):
    """Check a tensor argument before any launch: a contiguous device tensor on `like`'s device,
    of dtype `dtype` and (when given) exactly `shape`; raises AveyError otherwise."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise AveyError(fn, -1, f"{name} must be a torch tensor")
    if not t.is_cuda or t.device != like.device:
        raise AveyError(fn, -1, f"{name} must be a device tensor on {like.device}, got {t.device}")
    if t.dtype != dtype:
        raise AveyError(fn, -3, f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise AveyError(fn, -2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise AveyError(fn, -2, f"{name} must be contiguous")
    return t


def _out_rows(t, fn: str, name: str, like, shape):
    """An output [B, N, width] tensor (any row stride): device and dtype of `like`, exact shape."""
    if not t.is_cuda or t.device != like.device:
        raise AveyError(fn, -1, f"{name} must be a device tensor on {like.device}, got {t.device}")
    if t.dtype != like.dtype:
        raise AveyError(fn, -3, f"{name} must have dtype {like.dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise AveyError(fn, -2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return _rows(t, name)


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def n_splits(N: int, S: int) -> int:
    return -(-N // S)


def avey_rank_workspace_bytes(dtype_code: int, B: int, N: int, d: int, S: int) -> int:
    """Bytes of the ranker workspace for this shape; raises AveyError if the shape is rejected."""
    n = load_library().avey_rank_workspace_bytes(dtype_code, B, N, d, S)
    if n < 0:
        _check("avey_rank_workspace_bytes", int(n))
    return int(n)


def rank_workspace(x, S: int):
    """A device byte buffer large enough to be the ranker workspace for x [B, N, d]."""
    import torch
    B, N, d, _ = _rows(x, "x")
    n = avey_rank_workspace_bytes(_dtype_code(x), B, N, d, S)
    return torch.empty((max(n, 16),), device=x.device, dtype=torch.uint8)


def _workspace_arg(fn: str, workspace, x, S: int):
    """The caller's ranker workspace: a contiguous uint8 device tensor on x's device, at least
    avey_rank_workspace_bytes(...) bytes long."""
    import torch
    B, N, d, _ = _rows(x, "x")
    need = avey_rank_workspace_bytes(_dtype_code(x), B, N, d, S)
    _arg(workspace, fn, "workspace", x, torch.uint8)
    if workspace.numel() < need:
        raise AveyError(fn, -2, f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace


def _scores_arg(fn: str, scores, x, B: int, n_s: int):
    import torch
    if scores is None:
        return torch.empty((B, n_s, n_s), device=x.device, dtype=torch.float32)
    return _arg(scores, fn, "scores", x, torch.float32, (B, n_s, n_s))


def _topk_args(fn: str, idx, w, like, B: int, n_s: int, k: int):
    import torch
    if idx is None:
        idx = torch.empty((B, n_s, k), device=like.device, dtype=torch.int32)
    if w is None:
        w = torch.empty((B, n_s, k), device=like.device, dtype=torch.float32)
    _arg(idx, fn, "idx", like, torch.int32, (B, n_s, k))
    _arg(w, fn, "w", like, torch.float32, (B, n_s, k))
    return idx, w


def avey_maxsim_prepare(x, S: int, workspace=None):
    """Fill (and return) the ranker workspace from x [B, N, d]."""
    B, N, d, ld = _rows(x, "x")
    if workspace is None:
        workspace = rank_workspace(x, S)
    _workspace_arg("avey_maxsim_prepare", workspace, x, S)
    _check("avey_maxsim_prepare", load_library().avey_maxsim_prepare(
        x.data_ptr(), _dtype_code(x), B, N, d, ld, S, workspace.data_ptr(), _stream(x)))
    return workspace


def avey_maxsim_scores(workspace, x, S: int, scores=None):
    """All-pairs MaxSim scores [B, n_s, n_s] (fp32, diagonal -inf) from a workspace that
    avey_maxsim_prepare filled for x (x supplies the shape and dtype only)."""
    B, N, d, _ = _rows(x, "x")
    n_s = n_splits(N, S)
    _workspace_arg("avey_maxsim_scores", workspace, x, S)
    scores = _scores_arg("avey_maxsim_scores", scores, x, B, n_s)
    _check("avey_maxsim_scores", load_library().avey_maxsim_scores(
        workspace.data_ptr(), _dtype_code(x), B, N, d, S, scores.data_ptr(), _stream(x)))
    return scores


def avey_topk_norm(scores, k: int, idx=None, w=None, preceding: bool = False):
    """Top-k indices [B, n_s, k] (int32) and divide-by-max weights (fp32) of a score matrix.

    preceding=True: candidates of row i are the splits j < i; short rows end with (-1, 0)."""
    import torch
    if not isinstance(scores, torch.Tensor) or scores.dim() != 3 or scores.shape[1] != scores.shape[2]:
        raise AveyError("avey_topk_norm", -2, "scores must be a [B, n_s, n_s] tensor")
    B, n_s, _ = scores.shape
    _arg(scores, "avey_topk_norm", "scores", scores, torch.float32)
    idx, w = _topk_args("avey_topk_norm", idx, w, scores, B, n_s, k)
    lib = load_library()
    fn = lib.avey_topk_norm_preceding if preceding else lib.avey_topk_norm
    _check("avey_topk_norm", fn(scores.data_ptr(), B, n_s, k, idx.data_ptr(), w.data_ptr(), _stream(scores)))
    return idx, w


def avey_maxsim(x, S: int, scores=None):
    """All-pairs MaxSim scores [B, n_s, n_s] (fp32, diagonal -inf) straight from x [B, N, d], with
    no workspace (token norms on chip)."""
    B, N, d, ld = _rows(x, "x")
    n_s = n_splits(N, S)
    scores = _scores_arg("avey_maxsim", scores, x, B, n_s)
    _check("avey_maxsim", load_library().avey_maxsim(
        x.data_ptr(), _dtype_code(x), B, N, d, ld, S, scores.data_ptr(), _stream(x)))
    return scores


def avey_split_rank(x, S: int, k: int, scores=None, idx=None, w=None, preceding: bool = False):
    """(scores, idx, w) of the ranker for x [B, N, d], with no workspace: bidirectional (every
    other split is a candidate), or with preceding=True unidirectional (only earlier splits)."""
    B, N, d, ld = _rows(x, "x")
    n_s = n_splits(N, S)
    fn_name = "avey_split_rank_preceding" if preceding else "avey_split_rank"
    scores = _scores_arg(fn_name, scores, x, B, n_s)
    idx, w = _topk_args(fn_name, idx, w, x, B, n_s, k)
    lib = load_library()
    fn = lib.avey_split_rank_preceding if preceding else lib.avey_split_rank
    _check(fn_name, fn(
        x.data_ptr(), _dtype_code(x), B, N, d, ld, S, k, scores.data_ptr(), idx.data_ptr(), w.data_ptr(),
        _stream(x)))
    return scores, idx, w


def avey_split_rank_noalloc(x, S: int, k: int, scores=None, idx=None, w=None):
    """(scores, idx, w) of the bidirectional ranker through the explicit-workspace path with the
    workspace in the library's own device array (the call allocates no device memory; outputs
    are allocated here only when not given)."""
    B, N, d, ld = _rows(x, "x")
    n_s = n_splits(N, S)
    fn_name = "avey_split_rank_noalloc"
    scores = _scores_arg(fn_name, scores, x, B, n_s)
    idx, w = _topk_args(fn_name, idx, w, x, B, n_s, k)
    _check(fn_name, load_library().avey_split_rank_noalloc(
        x.data_ptr(), _dtype_code(x), B, N, d, ld, S, k, scores.data_ptr(), idx.data_ptr(), w.data_ptr(),
        _stream(x)))
    return scores, idx, w


def avey_split_rank_ws(x, S: int, k: int, workspace=None, scores=None, idx=None, w=None, preceding: bool = False):
    """The same ranker through the explicit-workspace path: avey_maxsim_prepare, avey_maxsim_scores
    and the top-k call on the current stream (allocates the workspace if not given)."""
    B, N, d, _ = _rows(x, "x")
    n_s = n_splits(N, S)
    fn_name = "avey_split_rank_ws"
    if workspace is None:
        workspace = rank_workspace(x, S)
    _workspace_arg(fn_name, workspace, x, S)
    scores = _scores_arg(fn_name, scores, x, B, n_s)
    idx, w = _topk_args(fn_name, idx, w, x, B, n_s, k)
    avey_maxsim_prepare(x, S, workspace)
    avey_maxsim_scores(workspace, x, S, scores)
    avey_topk_norm(scores, k, idx, w, preceding=preceding)
    return scores, idx, w


def avey_select_compress(x, idx, w, P, S: int, residual: bool = True, out=None):
    """Xhat [B, N, d] = P X_cat (+ X_i) per split, X_cat gathered through idx and weighted by w."""
    import torch
    fn = "avey_select_compress"
    B, N, d, ld = _rows(x, "x")
    if not isinstance(idx, torch.Tensor) or idx.dim() != 3:
        raise AveyError(fn, -2, "idx must be a [B, n_s, k] tensor")
    k = idx.shape[-1]
    n_s = n_splits(N, S)
    _arg(idx, fn, "idx", x, torch.int32, (B, n_s, k))
    _arg(w, fn, "w", x, torch.float32, (B, n_s, k))
    _arg(P, fn, "P", x, x.dtype, (S, (k + 1) * S))
    if out is None:
        out = torch.empty((B, N, d), device=x.device, dtype=x.dtype)
    _, _, _, ld_out = _out_rows(out, fn, "out", x, (B, N, d))
    _check(fn, load_library().avey_select_compress(
        x.data_ptr(), _dtype_code(x), B, N, d, ld, S, k, idx.data_ptr(), w.data_ptr(), P.data_ptr(),
        1 if residual else 0, out.data_ptr(), ld_out, _stream(x)))
    return out


def avey_dyn_context(z_tail, S: int, eps: float, out=None):
    """S~ Z_t per split for z_tail [B, N, m_t] (may be a column slice of Z with row stride m)."""
    import torch
    B, N, m_t, ld = _rows(z_tail, "z_tail")
    if out is None:
        out = torch.empty((B, N, m_t), device=z_tail.device, dtype=z_tail.dtype)
    _, _, _, ld_out = _out_rows(out, "avey_dyn_context", "out", z_tail, (B, N, m_t))
    _check("avey_dyn_context", load_library().avey_dyn_context(
        z_tail.data_ptr(), _dtype_code(z_tail), B, N, m_t, ld, S, float(eps), out.data_ptr(), ld_out,
        _stream(z_tail)))
    return out


def _layer_args(fn: str, z_tail, S: int, bias, act: str):
    """Shared marshalling of the two contextualizer layers: (bias pointer or 0, act code)."""
    import torch
    if act not in AVEY_ACT:
        raise AveyError(fn, -2, f"act must be one of {sorted(AVEY_ACT)}")
    if bias is None:
        return 0, AVEY_ACT[act]
    _arg(bias, fn, "bias", z_tail, torch.float32, (S,))
    return bias.data_ptr(), AVEY_ACT[act]


def avey_dyn_layer(z_tail, S: int, eps: float, bias=None, act: str = "identity", out=None, norm: str = "sum"):
    """act(S~ Z_t + bias[slot]) per split: the dynamic layer with its bias and activation; norm
    selects the row normalisation of the cosine matrix ("sum", "softmax", "rms" or "none")."""
    import torch
    fn = "avey_dyn_layer"
    B, N, m_t, ld = _rows(z_tail, "z_tail")
    bptr, code = _layer_args(fn, z_tail, S, bias, act)
    if norm not in AVEY_NORM:
        raise AveyError(fn, -2, f"norm must be one of {sorted(AVEY_NORM)}")
    if out is None:
        out = torch.empty((B, N, m_t), device=z_tail.device, dtype=z_tail.dtype)
    _, _, _, ld_out = _out_rows(out, fn, "out", z_tail, (B, N, m_t))
    _check(fn, load_library().avey_dyn_layer(
        z_tail.data_ptr(), _dtype_code(z_tail), B, N, m_t, ld, S, float(eps), AVEY_NORM[norm], bptr, code,
        out.data_ptr(), ld_out, _stream(z_tail)))
    return out


def avey_static_layer(z_tail, V, S: int, bias=None, act: str = "identity", out=None):
    """act(V Z_t + bias[slot]) per split, V [S, S] mixing the split's token positions."""
    import torch
    fn = "avey_static_layer"
    B, N, m_t, ld = _rows(z_tail, "z_tail")
    bptr, code = _layer_args(fn, z_tail, S, bias, act)
    _arg(V, fn, "V", z_tail, z_tail.dtype, (S, S))
    if out is None:
        out = torch.empty((B, N, m_t), device=z_tail.device, dtype=z_tail.dtype)
    _, _, _, ld_out = _out_rows(out, fn, "out", z_tail, (B, N, m_t))
    _check(fn, load_library().avey_static_layer(
        z_tail.data_ptr(), _dtype_code(z_tail), B, N, m_t, ld, S, V.data_ptr(), bptr, code, out.data_ptr(),
        ld_out, _stream(z_tail)))
    return out


def avey_enrich(x, U, b=None, out=None):
    """Z [B, N, m] = ReLU(X U + b)^2 for x [B, N, d], U [d, m], b [m] float32 (or None)."""
    import torch
    fn = "avey_enrich"
    B, N, d, ld = _rows(x, "x")
    if not isinstance(U, torch.Tensor) or U.dim() != 2:
        raise AveyError(fn, -2, "U must be a [d, m] tensor")
    m = U.shape[1]
    _arg(U, fn, "U", x, x.dtype, (d, m))
    if b is not None:
        _arg(b, fn, "b", x, torch.float32, (m,))
    if out is None:
        out = torch.empty((B, N, m), device=x.device, dtype=x.dtype)
    _, _, _, ld_out = _out_rows(out, fn, "out", x, (B, N, m))
    _check(fn, load_library().avey_enrich(
        x.data_ptr(), _dtype_code(x), B * N, d, ld, U.data_ptr(), m, b.data_ptr() if b is not None else 0,
        out.data_ptr(), ld_out, _stream(x)))
    return out


def avey_fuse(z, m_h: int, c, O, x, out=None):
    """Y [B, N, d] = [Z_h || C] O + X: z [B, N, >= m_h] (head = its first m_h columns), c [B, N, m_t],
    O [m_h + m_t, d], x [B, N, d] the layer's input."""
    import torch
    fn = "avey_fuse"
    B, N, d, ld_x = _rows(x, "x")
    _, _, m_t, ld_c = _rows(c, "c")
    _, _, wz, ld_z = _rows(z, "z")
    if tuple(c.shape[:2]) != (B, N) or tuple(z.shape[:2]) != (B, N):
        raise AveyError(fn, -2, f"z and c must have the leading shape [B, N] = [{B}, {N}] of x")
    if z.device != x.device or c.device != x.device:
        raise AveyError(fn, -1, "z, c and x must be on one device")
    if wz < m_h:
        raise AveyError(fn, -2, f"z has {wz} columns, fewer than m_h = {m_h}")
    if z.dtype != x.dtype or c.dtype != x.dtype:
        raise AveyError(fn, -3, "z, c, O and x must share one dtype")
    _arg(O, fn, "O", x, x.dtype, (m_h + m_t, d))
    if out is None:
        out = torch.empty((B, N, d), device=x.device, dtype=x.dtype)
    _, _, _, ld_y = _out_rows(out, fn, "out", x, (B, N, d))
    _check(fn, load_library().avey_fuse(
        z.data_ptr(), _dtype_code(x), B * N, m_h, ld_z, c.data_ptr(), m_t, ld_c, O.data_ptr(), d,
        x.data_ptr(), ld_x, out.data_ptr(), ld_y, _stream(x)))
    return out


# ---- peak micro-benchmarks (include/avey_probe.h): the measured ceilings, not the hot path

def avey_probe_mfma_flops(iters: int) -> int:
    """bf16 FLOPs one avey_probe_mfma_bf16 launch of `iters` iterations performs on this device."""
    n = load_library().avey_probe_mfma_flops(int(iters))
    if n < 0:
        _check("avey_probe_mfma_flops", int(n))
    return int(n)


def avey_probe_mfma_bf16(iters: int, changing: bool, sink=None):
    """Enqueue the matrix-core probe on the current stream (register operands, no memory traffic;
    `changing` replaces the operands every iteration). Returns the sink buffer it was given or
    allocated (one float per compute unit)."""
    import torch
    if sink is None:
        sink = torch.zeros(4096, device="cuda", dtype=torch.float32)
    if not sink.is_cuda or sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < 4096:
        raise AveyError("avey_probe_mfma_bf16", -2, "sink must be a contiguous float32 device tensor of >= 4096 values")
    st = torch.cuda.current_stream().cuda_stream
    _check("avey_probe_mfma_bf16",
           load_library().avey_probe_mfma_bf16(int(iters), 1 if changing else 0, sink.data_ptr(), st))
    return sink


def avey_probe_copy(src, dst) -> None:
    """Enqueue dst <- src (same number of bytes, contiguous, 16-byte aligned) on the current stream."""
    import torch
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.device == dst.device):
        raise AveyError("avey_probe_copy", -1, "src and dst must be device tensors on one device")
    if not (src.is_contiguous() and dst.is_contiguous()) or dst.numel() * dst.element_size() != nbytes:
        raise AveyError("avey_probe_copy", -2, "src and dst must be contiguous and of the same size in bytes")
    st = torch.cuda.current_stream().cuda_stream
    _check("avey_probe_copy", load_library().avey_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, st))
