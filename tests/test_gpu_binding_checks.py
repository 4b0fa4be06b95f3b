"""The Python binding refuses every ill-formed tensor argument before any launch: a host tensor,
a tensor on another device, a wrong dtype, a wrong shape, a non-contiguous tensor, a workspace
that is too small. Each refusal raises AveyError and leaves the output buffer untouched."""
import pytest
import torch

import attention_free_long_amd as A

pytestmark = pytest.mark.gpu

B, N, d, S, k = 2, 1000, 128, 256, 2
n_s = -(-N // S)
BF = torch.bfloat16


def dev(*shape, dtype=BF, fill=0.5):
    return torch.full(shape, fill, device="cuda", dtype=dtype)


def refused(call, out=None):
    sentinel = None if out is None else out.clone()
    with pytest.raises(A.AveyError):
        call()
    torch.cuda.synchronize()
    if out is not None:
        assert torch.equal(out, sentinel), "a refused call wrote its output"


def test_split_rank_checks(gpu_ok):
    x = dev(B, N, d)
    scores = dev(B, n_s, n_s, dtype=torch.float32, fill=7.0)
    idx = torch.zeros(B, n_s, k, device="cuda", dtype=torch.int32)
    w = dev(B, n_s, k, dtype=torch.float32)
    good = dict(scores=scores, idx=idx, w=w)
    bad = [
        dict(good, scores=scores.cpu()),
        dict(good, scores=dev(B, n_s, n_s + 1, dtype=torch.float32)),
        dict(good, scores=dev(B, n_s, n_s, dtype=torch.float64)),
        dict(good, scores=dev(B, n_s, 2 * n_s, dtype=torch.float32)[..., ::2]),
        dict(good, idx=idx.long()),
        dict(good, idx=idx[:, :, :1]),
        dict(good, w=w.cpu()),
        dict(good, w=w[:1]),
    ]
    for kw in bad:
        refused(lambda: A.avey_split_rank(x, S, k, **kw), scores)
    ws = A.rank_workspace(x, S)
    refused(lambda: A.avey_maxsim_prepare(x, S, ws[:-16]))
    refused(lambda: A.avey_maxsim_prepare(x, S, ws.view(torch.int16)))
    refused(lambda: A.avey_maxsim_scores(ws[:1024], x, S, scores), scores)
    refused(lambda: A.avey_maxsim_scores(ws.cpu(), x, S, scores), scores)
    refused(lambda: A.avey_topk_norm(scores.cpu(), k))
    refused(lambda: A.avey_topk_norm(scores, k, idx=idx[:, :1]))
    refused(lambda: A.avey_topk_norm(scores.half(), k))


def test_select_compress_checks(gpu_ok):
    x = dev(B, N, d)
    idx = torch.zeros(B, n_s, k, device="cuda", dtype=torch.int32)
    w = dev(B, n_s, k, dtype=torch.float32)
    P = dev(S, (k + 1) * S)
    out = dev(B, N, d, fill=3.0)
    good = dict(idx=idx, w=w, P=P)
    bad = [
        dict(good, idx=idx.cpu()),
        dict(good, idx=idx[:1]),
        dict(good, idx=idx.long()),
        dict(good, w=w.cpu()),
        dict(good, w=w.double()),
        dict(good, w=w[:, :-1]),
        dict(good, P=P.cpu()),
        dict(good, P=P.float()),
        dict(good, P=P[:, :-S]),
        dict(good, P=dev((k + 1) * S, S).t()),
    ]
    for kw in bad:
        refused(lambda: A.avey_select_compress(x, kw["idx"], kw["w"], kw["P"], S, out=out), out)
    refused(lambda: A.avey_select_compress(x, idx, w, P, S, out=out.cpu()))
    refused(lambda: A.avey_select_compress(x, idx, w, P, S, out=dev(B, N, d, dtype=torch.float32)))
    refused(lambda: A.avey_select_compress(x, idx, w, P, S, out=dev(B, N - 1, d)))


def test_layer_checks(gpu_ok):
    z = dev(B, N, 64)
    out = dev(B, N, 64, fill=3.0)
    bias = dev(S, dtype=torch.float32)
    refused(lambda: A.avey_dyn_context(z, S, 1e-8, out=out.cpu()))
    refused(lambda: A.avey_dyn_context(z, S, 1e-8, out=dev(B, N, 128)))
    refused(lambda: A.avey_dyn_layer(z, S, 1e-8, bias=bias.cpu(), out=out), out)
    refused(lambda: A.avey_dyn_layer(z, S, 1e-8, bias=bias[:-1], out=out), out)
    refused(lambda: A.avey_dyn_layer(z, S, 1e-8, bias=bias.double(), out=out), out)
    V = dev(S, S)
    refused(lambda: A.avey_static_layer(z, V.cpu(), S, out=out), out)
    refused(lambda: A.avey_static_layer(z, V[:, :-1], S, out=out), out)
    refused(lambda: A.avey_static_layer(z, V.t(), S, out=out), out)
    refused(lambda: A.avey_static_layer(z, V.float(), S, out=out), out)


def test_enrich_fuse_checks(gpu_ok):
    x = dev(B, N, d)
    m, m_h = 256, 128
    U = dev(d, m)
    b = dev(m, dtype=torch.float32)
    z = dev(B, N, m, fill=3.0)
    refused(lambda: A.avey_enrich(x, U.cpu(), b, out=z), z)
    refused(lambda: A.avey_enrich(x, dev(d + 64, m), b, out=z), z)
    refused(lambda: A.avey_enrich(x, U.t().contiguous().t(), b, out=z), z)
    refused(lambda: A.avey_enrich(x, U, b.cpu(), out=z), z)
    refused(lambda: A.avey_enrich(x, U, b[:-1], out=z), z)
    refused(lambda: A.avey_enrich(x, U, b, out=dev(B, N, m + 64)))
    c = dev(B, N, m - m_h)
    O = dev(m, d)
    y = dev(B, N, d, fill=3.0)
    refused(lambda: A.avey_fuse(z, m_h, c, O.cpu(), x, out=y), y)
    refused(lambda: A.avey_fuse(z, m_h, c, O[:-64], x, out=y), y)
    refused(lambda: A.avey_fuse(z, m_h, c, O.float(), x, out=y), y)
    refused(lambda: A.avey_fuse(z, m_h, c[:1], O, x, out=y), y)
    refused(lambda: A.avey_fuse(z, m_h, c, O, x, out=y.cpu()))
