"""libavey.so loads on the host, exports every function include/*.h declares, and rejects bad
arguments before any HIP call (CPU only: every call here fails validation or is empty work)."""
import ctypes
import os
import re

import pytest

import attention_free_long_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP = 0, -1, -2, -3, -4, -5
P16 = 0x10000          # fake, 16-byte aligned device address: never dereferenced by these calls
P4 = 0x10004           # 4-byte aligned, not 16-byte aligned


def declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(avey_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return A.load_library()


def test_exports_match_header(lib):
    decl = declared_functions()
    assert set(decl) == set(A.EXPORTS)
    so = ctypes.CDLL(A.LIB_PATH)
    for name in decl:
        assert hasattr(so, name), name
    assert lib.avey_abi_version() == A.AVEY_ABI_VERSION == 2


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, -6):
        assert lib.avey_status_str(code).decode().startswith("AVEY_")
    assert lib.avey_status_str(12345) == b"unknown avey status"


def test_split_rank_validation(lib):
    f = lib.avey_split_rank
    # (x, dt, B, N, d, ld, S, k, scores, idx, w, stream): no workspace
    assert f(P16, 7, 1, 1024, 64, 64, 64, 3, P16, P16, P16, None) == DTYPE
    assert f(P16, 1, -1, 1024, 64, 64, 64, 3, P16, P16, P16, None) == SHAPE
    assert f(P16, 1, 1, 1024, 64, 64, 0, 3, P16, P16, P16, None) == SHAPE
    assert f(P16, 1, 1, 1024, 64, 64, 1024, 3, P16, P16, P16, None) == SHAPE      # S > 512
    assert f(None, 1, 0, 1024, 64, 64, 64, 3, None, None, None, None) == OK       # B == 0: no work
    assert f(None, 1, 1, 0, 64, 64, 64, 3, None, None, None, None) == OK          # N == 0: no work
    assert f(None, 1, 1, 1024, 64, 64, 64, 3, P16, P16, P16, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, None, P16, P16, None) == NULL        # scores
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16, None, P16, None) == NULL        # idx
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16, P16, None, None) == NULL        # w
    assert f(P16, 1, 1, 1024, 64, 64, 64, 16, P16, P16, P16, None) == SHAPE       # k > n_s - 1
    assert f(P16, 1, 1, 1024, 64, 64, 64, 0, P16, P16, P16, None) == SHAPE
    assert f(P16, 1, 1, 64, 64, 64, 64, 1, P16, P16, P16, None) == SHAPE          # a single split
    assert f(P16, 1, 1, 1024, 64, 32, 64, 3, P16, P16, P16, None) == SHAPE        # ld < d
    assert f(P16, 1, 1, 1024, 100, 104, 64, 3, P16, P16, P16, None) == UNSUP      # bf16 d % 8
    assert f(P16, 1, 1, 1000, 64, 64, 100, 3, P16, P16, P16, None) == UNSUP       # bf16 S % 16
    assert f(P16, 1, 1, 1024, 64, 68, 64, 3, P16, P16, P16, None) == ALIGN        # bf16 ld % 8
    assert f(P4, 1, 1, 1024, 64, 64, 64, 3, P16, P16, P16, None) == ALIGN         # bf16 x alignment
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16 + 2, P16, P16, None) == ALIGN    # scores alignment
    assert f(P16, 0, 1, 1000, 64, 64, 64, 3, P16, P16 + 2, P16, None) == ALIGN    # idx alignment
    assert f(P16, 1, 1, 1 << 25, 64, 64, 256, 3, P16, P16, P16, None) == UNSUP    # > 2^30 elements
    assert f(P16, 1, 1, 1024, 64, 1 << 20, 64, 3, P16, P16, P16, None) == UNSUP   # (N + 512) ld >= 2^30


def test_maxsim_validation(lib):
    f = lib.avey_maxsim
    # (x, dt, B, N, d, ld, S, scores, stream)
    assert f(None, 1, 0, 1024, 64, 64, 64, None, None) == OK
    assert f(None, 1, 1, 1024, 64, 64, 64, P16, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, None, None) == NULL
    assert f(P16, 1, 1, 64, 64, 64, 64, P16, None) == SHAPE                # a single split
    assert f(P16, 1, 1, 1024, 64, 64, 40, P16, None) == UNSUP              # bf16 S % 16
    assert f(P16, 1, 1, 1024, 12, 16, 64, P16, None) == UNSUP              # bf16 d % 8
    assert f(P16, 0, 1, 1024, 12, 12, 40, P16 + 1, None) == ALIGN          # f32: any S, d; scores 4-aligned
    assert f(P16, 9, 1, 1024, 64, 64, 64, P16, None) == DTYPE


def test_workspace_prepare_and_scores_validation(lib):
    n = lib.avey_rank_workspace_bytes
    assert n(1, 2, 32768, 768, 256) == 2 * 128 * 256 * 768 * 2
    assert n(1, 1, 1000, 72, 64) == 1 * 16 * 64 * 96 * 2                # bf16 d padded to 32
    assert n(1, 1, 1100, 64, 64) == 1 * 5 * 256 * 64 * 2                 # bf16 S = 64: blocks of 256 tokens
    assert n(1, 1, 1100, 64, 128) == 1 * 5 * 256 * 64 * 2                # bf16 S = 128 likewise
    assert n(1, 1, 1100, 64, 48) == 1 * 23 * 48 * 64 * 2                 # other S: blocks of one split
    assert n(0, 1, 1100, 64, 64) == 1 * 18 * 64 * 64 * 4                 # fp32: splits
    assert n(0, 1, 1000, 72, 64) == 1 * 16 * 64 * 72 * 4                 # fp32 d as it is
    assert n(0, 1, 1000, 64, 64) == 1 * 16 * 64 * 64 * 4                 # padded to whole splits
    assert n(1, 0, 1000, 64, 64) == 0
    assert n(1, 1, 1000, 64, 100) == UNSUP                               # bf16 S % 16
    assert n(1, 1, 1000, 60, 64) == UNSUP                                # bf16 d % 8
    assert n(9, 1, 1000, 64, 64) == DTYPE
    assert n(1, 1, 64, 64, 64) == SHAPE                                  # a single split
    p = lib.avey_maxsim_prepare
    # (x, dt, B, N, d, ld, S, workspace, stream)
    assert p(None, 1, 0, 1024, 64, 64, 64, None, None) == OK
    assert p(P16, 1, 1, 1024, 64, 64, 64, None, None) == NULL
    assert p(None, 1, 1, 1024, 64, 64, 64, P16, None) == NULL
    assert p(P16, 1, 1, 1024, 64, 32, 64, P16, None) == SHAPE
    assert p(P16, 1, 1, 1024, 64, 64, 64, P4, None) == ALIGN
    assert p(P16, 1, 1, 1024, 100, 104, 64, P16, None) == UNSUP
    m = lib.avey_maxsim_scores
    # (workspace, dt, B, N, d, S, scores, stream)
    assert m(None, 1, 1, 0, 64, 64, None, None) == OK
    assert m(None, 1, 1, 1024, 64, 64, P16, None) == NULL
    assert m(P16, 1, 1, 1024, 64, 64, None, None) == NULL
    assert m(P16, 1, 1, 64, 64, 64, P16, None) == SHAPE                  # a single split
    assert m(P16, 1, 1, 1024, 64, 72, P16, None) == UNSUP                # bf16 S % 16
    assert m(P16, 1, 1, 1024, 100, 64, P16, None) == UNSUP               # bf16 d % 8
    assert m(P16, 0, 1, 1024, 64, 64, P16 + 1, None) == ALIGN


@pytest.mark.parametrize("fn", ["avey_topk_norm", "avey_topk_norm_preceding"])
def test_topk_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(P16, 0, 16, 3, P16, P16, None) == OK
    assert f(None, 1, 16, 3, P16, P16, None) == NULL
    assert f(P16, 1, 16, 16, P16, P16, None) == SHAPE
    assert f(P16, 1, 1, 1, P16, P16, None) == SHAPE
    assert f(P16 + 1, 1, 16, 3, P16, P16, None) == ALIGN


def test_split_rank_preceding_validation(lib):
    f = lib.avey_split_rank_preceding
    # same argument list and checks as avey_split_rank
    assert f(None, 1, 0, 1024, 64, 64, 64, 3, None, None, None, None) == OK
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, None, P16, P16, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, 16, P16, P16, P16, None) == SHAPE
    assert f(P16, 1, 1, 1024, 100, 104, 64, 3, P16, P16, P16, None) == UNSUP


def test_select_compress_validation(lib):
    f = lib.avey_select_compress
    # (x, dt, B, N, d, ld_x, S, k, idx, w, P, residual, xhat, ld_out, stream)
    assert f(None, 1, 0, 1024, 64, 64, 64, 3, None, None, None, 1, None, 64, None) == OK
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, None, P16, P16, 1, P16, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16, P16, P16, 1, None, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16, P16, P16, 2, P16, 64, None) == SHAPE   # residual flag
    assert f(P16, 1, 1, 1024, 64, 64, 64, 0, P16, P16, P16, 1, P16, 64, None) == SHAPE
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16, P16, P16, 1, P16, 60, None) == SHAPE   # ld_out < d
    assert f(P16, 1, 1, 1024, 64, 64, 64, 3, P16, P16, P4, 1, P16, 64, None) == ALIGN    # P alignment
    assert f(P16, 1, 1, 1024, 64, 64, 40, 3, P16, P16, P16, 1, P16, 64, None) == UNSUP   # bf16 S % 16
    assert f(P16, 1, 1, 1024, 60, 64, 64, 3, P16, P16, P16, 1, P16, 64, None) == UNSUP   # bf16 d % 8
    assert f(P16, 1, 1, 1 << 20, 64, 64, 64, 600, P16, P16, P16, 1, P16, 64, None) == UNSUP   # bf16 k + 1 > 512


def test_dyn_context_validation(lib):
    f = lib.avey_dyn_context
    # (z_tail, dt, B, N, m_t, ld_z, S, eps, out, ld_out, stream)
    assert f(None, 1, 0, 1024, 64, 64, 64, 1e-8, None, 64, None) == OK
    assert f(None, 1, 1, 1024, 64, 64, 64, 1e-8, P16, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, 1e-8, None, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 100, 104, 64, 1e-8, P16, 104, None) == UNSUP    # bf16 m_t % 8
    assert f(P16, 1, 1, 1024, 64, 64, 72, 1e-8, P16, 64, None) == UNSUP       # bf16 S % 16
    assert f(P16, 1, 1, 1024, 64, 64, 600, 1e-8, P16, 64, None) == SHAPE      # S > 512
    assert f(P16 + 8, 1, 1, 1024, 64, 64, 64, 1e-8, P16, 64, None) == ALIGN
    assert f(P16, 9, 1, 1024, 64, 64, 64, 1e-8, P16, 64, None) == DTYPE


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(A.AveyError):
        A.avey_split_rank(torch.zeros(1, 1024, 64, dtype=torch.bfloat16), 64, 3)


def test_dyn_layer_validation(lib):
    f = lib.avey_dyn_layer
    # (z_tail, dt, B, N, m_t, ld_z, S, eps, norm, bias, act, out, ld_out, stream)
    assert f(None, 1, 0, 1024, 64, 64, 64, 1e-8, 0, None, 0, None, 64, None) == OK
    assert f(None, 1, 1, 1024, 64, 64, 64, 1e-8, 0, None, 0, P16, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, 1e-8, 0, None, 2, P16, 64, None) == SHAPE     # unknown act
    assert f(P16, 1, 1, 1024, 64, 64, 64, 1e-8, 0, None, -1, P16, 64, None) == SHAPE
    assert f(P16, 1, 1, 1024, 64, 64, 64, 1e-8, 4, None, 0, P16, 64, None) == SHAPE     # unknown norm
    assert f(P16, 1, 1, 1024, 64, 64, 64, 1e-8, -1, None, 0, P16, 64, None) == SHAPE
    assert f(P16, 1, 1, 1024, 64, 64, 64, 1e-8, 1, P16 + 2, 1, P16, 64, None) == ALIGN  # bias not 4-aligned
    assert f(P16, 1, 1, 1024, 64, 64, 88, 1e-8, 2, None, 1, P16, 64, None) == UNSUP    # bf16 S % 16
    assert f(P16, 9, 1, 1024, 64, 64, 64, 1e-8, 3, None, 0, P16, 64, None) == DTYPE


def test_static_layer_validation(lib):
    f = lib.avey_static_layer
    # (z_tail, dt, B, N, m_t, ld_z, S, V, bias, act, out, ld_out, stream)
    assert f(None, 1, 0, 1024, 64, 64, 64, None, None, 0, None, 64, None) == OK
    assert f(P16, 1, 1, 1024, 64, 64, 64, None, None, 0, P16, 64, None) == NULL      # V
    assert f(None, 1, 1, 1024, 64, 64, 64, P16, None, 0, P16, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, P16, None, 0, None, 64, None) == NULL
    assert f(P16, 1, 1, 1024, 64, 64, 64, P16, None, 5, P16, 64, None) == SHAPE     # unknown act
    assert f(P16, 1, 1, 1024, 64, 64, 64, P16 + 8, None, 0, P16, 64, None) == ALIGN  # bf16 V 16-aligned
    assert f(P16, 0, 1, 1024, 64, 64, 64, P16 + 2, None, 0, P16, 64, None) == ALIGN  # f32 V 4-aligned
    assert f(P16, 1, 1, 1024, 64, 64, 64, P16, P16 + 1, 0, P16, 64, None) == ALIGN   # bias
    assert f(P16, 1, 1, 1024, 64, 64, 40, P16, None, 0, P16, 64, None) == UNSUP     # bf16 S % 16
    assert f(P16, 1, 1, 1024, 12, 16, 64, P16, None, 0, P16, 16, None) == UNSUP     # bf16 m_t % 8
    assert f(P16, 1, 1, 1024, 64, 32, 64, P16, None, 0, P16, 64, None) == SHAPE     # ld_z < m_t
    assert f(P16, 1, 1, 1024, 64, 64, 0, P16, None, 0, P16, 64, None) == SHAPE      # S < 1


def test_enrich_validation(lib):
    f = lib.avey_enrich
    # (x, dt, M, d, ld_x, U, m, b, z, ld_z, stream)
    assert f(None, 1, 0, 64, 64, None, 128, None, None, 128, None) == OK
    assert f(P16, 1, 100, 64, 64, None, 128, None, P16, 128, None) == NULL      # U
    assert f(P16, 1, 100, 64, 64, P16, 128, None, None, 128, None) == NULL      # z
    assert f(P16, 1, 100, 96, 96, P16, 128, None, P16, 128, None) == UNSUP      # bf16 d % 64
    assert f(P16, 1, 100, 64, 64, P16 + 8, 128, None, P16, 128, None) == ALIGN  # bf16 U 16-aligned
    assert f(P16, 1, 100, 64, 64, P16, 128, P16 + 2, P16, 128, None) == ALIGN   # b 4-aligned
    assert f(P16, 1, 100, 64, 64, P16, 8192, P16, P16, 8192, None) == UNSUP     # bf16 m > 4096 with b
    assert f(P16, 1, 100, 64, 32, P16, 128, None, P16, 128, None) == SHAPE      # ld_x < d
    assert f(P16, 1, -1, 64, 64, P16, 128, None, P16, 128, None) == SHAPE
    assert f(P16, 7, 100, 64, 64, P16, 128, None, P16, 128, None) == DTYPE


def test_fuse_validation(lib):
    f = lib.avey_fuse
    # (z, dt, M, m_h, ld_z, c, m_t, ld_c, O, d, x, ld_x, y, ld_y, stream)
    assert f(None, 1, 0, 64, 128, None, 64, 64, None, 64, None, 64, None, 64, None) == OK
    assert f(P16, 1, 10, 64, 128, P16, 64, 64, None, 64, P16, 64, P16, 64, None) == NULL    # O
    assert f(None, 1, 10, 64, 128, P16, 64, 64, P16, 64, P16, 64, P16, 64, None) == NULL    # z with a head
    assert f(None, 1, 10, 0, 0, P16, 64, 64, P16 + 8, 64, P16, 64, P16, 64, None) == ALIGN  # no head: z unused
    assert f(P16, 1, 10, 32, 128, P16, 64, 64, P16, 64, P16, 64, P16, 64, None) == UNSUP    # bf16 m_h % 64
    assert f(P16, 1, 10, -64, 128, P16, 64, 64, P16, 64, P16, 64, P16, 64, None) == SHAPE
    assert f(P16, 1, 10, 64, 128, P16, 64, 64, P16 + 8, 64, P16, 64, P16, 64, None) == ALIGN
    assert f(P16, 1, 10, 64, 128, P16, 64, 64, P16, 64, P16, 32, P16, 64, None) == SHAPE    # ld_x < d
    assert f(P16, 0, 10, 64, 128, P16, 64, 64, P16 + 2, 64, P16, 64, P16, 64, None) == ALIGN


def test_probe_validation(lib):
    f = lib.avey_probe_mfma_flops
    assert f(0) == SHAPE
    m = lib.avey_probe_mfma_bf16
    # (iters, changing, sink, stream)
    assert m(0, 0, P16, None) == SHAPE
    assert m(10, 0, None, None) == NULL
    assert m(10, 1, P16 + 2, None) == ALIGN
    c = lib.avey_probe_copy
    # (src, dst, bytes, stream)
    assert c(P16, P16 + 4096, 0, None) == OK            # nothing to copy
    assert c(P16, P16 + 4096, -16, None) == SHAPE
    assert c(P16, P16 + 4096, 24, None) == SHAPE         # not a multiple of 16
    assert c(None, P16, 32, None) == NULL
    assert c(P4, P16, 32, None) == ALIGN
    assert c(P16, P4, 32, None) == ALIGN
