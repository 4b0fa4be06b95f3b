"""Pins of the CPU oracle against facts other than itself (CPU only).

Each test is chosen so that a plausible slip in the oracle fails it: the MaxSim direction
(target sum vs candidate max), missing normalisation, unmasked padding, the top-k order and
tie rule, the X_cat block order and weighting, the residual, eq. 6's denominator and the
within-split scope of the dynamic layer.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import avey_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


# ----------------------------------------------------------------------------- hand-worked
def test_hand_worked_maxsim_and_topk():
    g = GOLD["maxsim"]
    x = np.array(g["x"], dtype=np.float64)
    S, k = g["S"], g["k"]
    sc = O.score_matrix(x[None], S)[0]
    for i, row in enumerate(g["scores"]):
        for j, v in enumerate(row):
            if v is None:
                assert sc[i, j] == -math.inf
            else:
                assert sc[i, j] == pytest.approx(v, abs=1e-14)
    ranked = O.split_rank(x[None], S, k)
    for i in range(3):
        _, idx, w, _ = ranked[(0, i)]
        assert list(idx) == g["idx"][i]
        np.testing.assert_allclose(w, g["w"][i], rtol=1e-14)


def test_hand_worked_compress():
    g = GOLD["compress"]
    x = np.array(g["x"], dtype=np.float64)[None]
    S = g["S"]
    for case in g["cases"]:
        idx = np.array(case["idx"])[None]
        w = np.array(case["w"])[None]
        P = np.array(case["P"], dtype=np.float64)
        parts = O.select_compress(x, S, idx, w, P, residual=case["residual"])
        if "xhat" in case:
            got = O.assemble(parts, 1, x.shape[1], S, 2)[0]
            np.testing.assert_allclose(got, case["xhat"], atol=1e-14)
        else:
            np.testing.assert_allclose(parts[(0, case["only_split"])], case["xhat_split0"], atol=1e-14)


def test_hand_worked_dyn():
    g = GOLD["dyn"]
    z = np.array(g["z"], dtype=np.float64)[None]
    out = O.dyn_context(z, g["S"], g["eps"])[(0, 0)]
    np.testing.assert_allclose(out, g["out"], atol=1e-15)


# ----------------------------------------------------------------------------- MaxSim
def _one_hot(codes, d):
    x = np.zeros((len(codes), d))
    x[np.arange(len(codes)), codes] = 1.0
    return x


def test_maxsim_one_hot_counts():
    """One-hot tokens: cosines are 0/1, so MaxSim(i<-j) counts the tokens of i whose code occurs in j."""
    rng = np.random.default_rng(1)
    S, d, n_s = 8, 12, 6
    codes = rng.integers(0, d, size=S * n_s - 3)          # ragged: last split has 5 tokens
    x = _one_hot(codes, d)
    sc = O.score_matrix(x[None], S)[0]
    N = len(codes)
    for i in range(n_s):
        ci = codes[i * S: min((i + 1) * S, N)]
        for j in range(n_s):
            if i == j:
                continue
            cj = set(codes[j * S: min((j + 1) * S, N)].tolist())
            assert sc[i, j] == sum(1 for c in ci if c in cj)
    # direction: a target with repeated codes versus a candidate with distinct codes
    x2 = _one_hot([0, 0, 0, 1, 0, 2, 3, 4], 5)
    s2 = O.score_matrix(x2[None], 4)[0]
    assert s2[0, 1] == 3 and s2[1, 0] == 1


def test_maxsim_scale_and_permutation_invariance():
    rng = np.random.default_rng(2)
    S, d, N = 7, 5, 31
    x = rng.standard_normal((N, d))
    base = O.score_matrix(x[None], S)[0]
    scaled = x * rng.uniform(0.1, 10.0, size=(N, 1))
    np.testing.assert_allclose(O.score_matrix(scaled[None], S)[0], base, rtol=1e-12)
    perm = x.copy()
    for j in range(O.n_splits(N, S)):
        r = O.split_rows(N, S, j)
        perm[r.start:r.stop] = x[r.start:r.stop][rng.permutation(len(r))]
    np.testing.assert_allclose(O.score_matrix(perm[None], S)[0], base, rtol=1e-12)


def test_maxsim_duplicate_split_closed_form():
    rng = np.random.default_rng(3)
    S, d, n_s = 6, 4, 5
    x = rng.standard_normal((S * n_s, d))
    x[4 * S:5 * S] = x[1 * S:2 * S]                      # split 4 is an exact copy of split 1
    sc = O.score_matrix(x[None], S)[0]
    assert sc[1, 4] == pytest.approx(S, abs=1e-12) and sc[4, 1] == pytest.approx(S, abs=1e-12)
    for i in (0, 2, 3):
        assert sc[i, 1] == sc[i, 4]                      # identical computation -> identical bits
    # no other candidate can beat a copy: each term is at most 1
    assert np.all(sc[1][[0, 2, 3]] <= S + 1e-12)


def test_maxsim_padding_is_masked():
    """A padded candidate whose valid tokens are all anti-parallel gives -(#target tokens).

    Were the zero padding rows candidates (cosine 0), every term would be 0 instead.
    """
    d, S = 3, 4
    tgt = np.tile([1.0, 0.0, 0.0], (S, 1))
    cand = np.array([[-2.0, 0.0, 0.0]])                  # one valid token, three padding slots
    x = np.concatenate([tgt, cand])
    sc = O.score_matrix(x[None], S)[0]
    assert sc[0, 1] == pytest.approx(-4.0, abs=1e-15)
    assert sc[1, 0] == pytest.approx(-1.0, abs=1e-15)    # only the one valid target token counts
    # Appending rows after N changes nothing: they are never part of any split's valid tokens.
    more = np.concatenate([x, np.full((2, d), 7.0)])
    sc2 = O.score_matrix(more[None, :5], S)[0]
    np.testing.assert_array_equal(sc2, sc)


def test_maxsim_brute_force_tiny():
    """Scalar loops with math.sqrt, per token pair, on many random tiny shapes."""
    rng = np.random.default_rng(4)
    for trial in range(40):
        S = int(rng.integers(1, 6))
        d = int(rng.integers(1, 6))
        N = int(rng.integers(S + 1, 4 * S + 2))
        x = rng.standard_normal((N, d))
        if trial % 5 == 0:
            x[rng.integers(0, N)] = 0.0                  # a zero token: cosine 0 with everything
        sc = O.score_matrix(x[None], S)[0]
        n_s = -(-N // S)
        for i in range(n_s):
            for j in range(n_s):
                if i == j:
                    continue
                total = 0.0
                for t in range(i * S, min(i * S + S, N)):
                    best = -math.inf
                    for u in range(j * S, min(j * S + S, N)):
                        dot = sum(x[t, c] * x[u, c] for c in range(d))
                        nt = math.sqrt(sum(x[t, c] ** 2 for c in range(d)))
                        nu = math.sqrt(sum(x[u, c] ** 2 for c in range(d)))
                        cos = 0.0 if nt == 0 or nu == 0 else dot / (nt * nu)
                        best = max(best, cos)
                    total += best
                assert sc[i, j] == pytest.approx(total, abs=1e-12)


# ----------------------------------------------------------------------------- top-k
def test_topk_worked_ties():
    row = np.array([5.0, 3.0, 3.0, 9.0, -math.inf])
    idx, w, s, gap = O.top_k(row, 4, 3)
    assert list(idx) == [3, 0, 1]                        # tie 3.0 at j=1 and j=2 -> lower index
    assert w[0] == 1.0 and w[1] == 5.0 / 9.0 and w[2] == 3.0 / 9.0
    assert gap == 0.0                                    # k-th and (k+1)-th are tied


@pytest.mark.parametrize("seed", range(20))
def test_topk_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 40))
    i = int(rng.integers(0, n))
    k = int(rng.integers(1, n))
    row = rng.integers(1, 6, size=n).astype(np.float64) * rng.choice([1.0, 0.5])  # many ties
    row[i] = -math.inf
    idx, w, s, _ = O.top_k(row, i, k)
    assert len(set(idx.tolist())) == k and i not in idx and all(0 <= j < n for j in idx)
    assert w[0] == 1.0
    assert np.all(np.diff(s) <= 0) and np.all((w > 0) & (w <= 1))
    kth = s[-1]
    for j in range(n):
        if j == i or j in idx:
            continue
        assert row[j] < kth or (row[j] == kth and j > max(jj for jj in idx if row[jj] == kth))
    for a, b in zip(idx[:-1], idx[1:]):
        assert row[a] > row[b] or (row[a] == row[b] and a < b)


def test_preceding_topk_hand_worked():
    """Unidirectional ranker on the hand-worked scores: candidates precede the target; missing
    candidates are empty blocks (index -1, weight 0)."""
    g = GOLD["maxsim"]
    x = np.array(g["x"], dtype=np.float64)
    ranked = O.split_rank(x[None], g["S"], 2, preceding=True)
    _, idx0, w0, _ = ranked[(0, 0)]
    _, idx1, w1, _ = ranked[(0, 1)]
    _, idx2, w2, _ = ranked[(0, 2)]
    assert list(idx0) == [-1, -1] and list(w0) == [0.0, 0.0]
    assert list(idx1) == [0, -1] and list(w1) == [1.0, 0.0]
    # s(2<-0) = 0.6 and s(2<-1) = -0.28 from the golden file
    assert list(idx2) == [0, 1]
    np.testing.assert_allclose(w2, [1.0, -0.28 / 0.6], rtol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_preceding_topk_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 30))
    i = int(rng.integers(0, n))
    k = int(rng.integers(1, n))
    row = rng.integers(1, 6, size=n).astype(np.float64)
    row[i] = -math.inf
    idx, w, s, _ = O.top_k(row, i, k, preceding=True)
    real = [j for j in idx.tolist() if j >= 0]
    assert len(idx) == k and len(real) == min(k, i)
    assert all(j < i for j in real) and idx.tolist()[len(real):] == [-1] * (k - len(real))
    assert np.all(w[len(real):] == 0.0)
    brute = sorted(range(i), key=lambda j: (-row[j], j))[:k]
    assert real == brute
    if real:
        assert w[0] == 1.0


def test_compress_empty_block_is_zero():
    """Index -1 contributes nothing, whatever its weight: same result as weight 0 on a real
    split."""
    rng = np.random.default_rng(8)
    S, d, k = 4, 3, 2
    x, idx, w, N, n_s = _rand_setup(rng, S, d, 5, N=18, k=k)
    P = rng.standard_normal((S, (k + 1) * S))
    idx_e, w_e = idx.copy(), w.copy()
    idx_e[0, 2, 1] = -1
    w_e[0, 2, 1] = 0.0
    w_z = w.copy()
    w_z[0, 2, 1] = 0.0
    a = O.select_compress(x, S, idx_e, w_e, P)
    b = O.select_compress(x, S, idx, w_z, P)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], atol=1e-14)


# ----------------------------------------------------------------------------- compression
def _rand_setup(rng, S=4, d=3, n_s=5, N=None, k=2):
    N = N or S * n_s
    x = rng.standard_normal((1, N, d))
    n_s = -(-N // S)
    idx = np.stack([rng.permutation([j for j in range(n_s) if j != i])[:k] for i in range(n_s)])[None]
    w = rng.uniform(0.2, 1.0, size=(1, n_s, k))
    w[..., 0] = 1.0
    return x, idx, w, N, n_s


def test_compress_block_order_and_weights():
    rng = np.random.default_rng(5)
    S, d, k = 4, 3, 2
    x, idx, w, N, n_s = _rand_setup(rng, S, d, 6, N=22, k=k)   # last split has 2 valid tokens
    eye = np.eye(S)
    for r in range(k + 1):
        P = np.zeros((S, (k + 1) * S))
        P[:, r * S:(r + 1) * S] = eye
        got = O.select_compress(x, S, idx, w, P, residual=False)
        for i in range(n_s):
            n_i = len(O.split_rows(N, S, i))
            src = i if r == 0 else int(idx[0, i, r - 1])
            scale = 1.0 if r == 0 else w[0, i, r - 1]
            want = scale * O.padded_split(x[0], S, src)[:n_i]
            np.testing.assert_allclose(got[(0, i)], want, atol=1e-15)
    # residual adds exactly the current split's own tokens
    P = rng.standard_normal((S, (k + 1) * S))
    a = O.select_compress(x, S, idx, w, P, residual=True)
    b = O.select_compress(x, S, idx, w, P, residual=False)
    for i in range(n_s):
        r_ = O.split_rows(N, S, i)
        np.testing.assert_allclose(a[(0, i)] - b[(0, i)], x[0, r_.start:r_.stop], atol=1e-12)


def test_compress_padding_rows_are_zero_and_linear_in_P():
    rng = np.random.default_rng(6)
    S, d, k = 4, 3, 1
    x, idx, w, N, n_s = _rand_setup(rng, S, d, 5, N=17, k=k)   # split 4 holds one token
    last = n_s - 1
    idx[0, 0, 0] = last
    P = np.zeros((S, 2 * S))
    P[:, S:] = np.eye(S)                                  # output = w * (retrieved split)
    out = O.select_compress(x, S, idx, w, P, residual=False)[(0, 0)]
    np.testing.assert_allclose(out[0], w[0, 0, 0] * x[0, 16], atol=1e-15)
    assert np.all(out[1:] == 0.0)                         # padding slots of the retrieved split
    P1, P2 = rng.standard_normal((2, S, 2 * S))
    o1 = O.select_compress(x, S, idx, w, P1, residual=False)
    o2 = O.select_compress(x, S, idx, w, P2, residual=False)
    o3 = O.select_compress(x, S, idx, w, 2.0 * P1 - 3.0 * P2, residual=False)
    for key in o1:
        np.testing.assert_allclose(o3[key], 2.0 * o1[key] - 3.0 * o2[key], atol=1e-12)


def test_compress_brute_force_tiny():
    rng = np.random.default_rng(7)
    S, d, k = 3, 2, 2
    x, idx, w, N, n_s = _rand_setup(rng, S, d, 4, N=11, k=k)
    P = rng.standard_normal((S, (k + 1) * S))
    got = O.select_compress(x, S, idx, w, P, residual=True)
    for i in range(n_s):
        for s in range(len(O.split_rows(N, S, i))):
            for f in range(d):
                acc = 0.0
                for blk in range(k + 1):
                    src = i if blk == 0 else int(idx[0, i, blk - 1])
                    wt = 1.0 if blk == 0 else w[0, i, blk - 1]
                    for slot in range(S):
                        t = src * S + slot
                        if t < N:
                            acc += P[s, blk * S + slot] * wt * x[0, t, f]
                acc += x[0, i * S + s, f]
                assert got[(0, i)][s, f] == pytest.approx(acc, abs=1e-12)


# ----------------------------------------------------------------------------- dynamic layer
def test_dyn_constant_and_orthogonal_splits():
    eps = 1e-3                                           # large enough to see in the closed forms
    S, m = 5, 4
    z = np.tile(np.array([0.5, 2.0, 0.0, 1.0]), (S, 1))[None]
    out = O.dyn_context(z, S, eps)[(0, 0)]
    np.testing.assert_allclose(out, S * z[0] / (S + eps), rtol=1e-14)
    z2 = (np.eye(4) * np.array([3.0, 1.0, 2.0, 5.0]))[None]   # orthogonal tokens -> S~ = I/(1+eps)
    out2 = O.dyn_context(z2, 4, eps)[(0, 0)]
    np.testing.assert_allclose(out2, z2[0] / (1 + eps), rtol=1e-14)


def test_dyn_two_token_closed_form_and_padding():
    eps = 1e-8
    rng = np.random.default_rng(8)
    z1, z2 = rng.uniform(0, 1, size=(2, 6))
    c = z1 @ z2 / (np.linalg.norm(z1) * np.linalg.norm(z2))
    # split 0 = {z1, z2}; split 1 = {z1} alone (N=3, S=2: one padding slot)
    z = np.stack([z1, z2, z1])[None]
    res = O.dyn_context(z, 2, eps)
    np.testing.assert_allclose(res[(0, 0)][0], (z1 + c * z2) / (1 + c + eps), rtol=1e-13)
    np.testing.assert_allclose(res[(0, 0)][1], (c * z1 + z2) / (1 + c + eps), rtol=1e-13)
    assert res[(0, 1)].shape == (1, 6)
    np.testing.assert_allclose(res[(0, 1)][0], z1 / (1 + eps), rtol=1e-14)


def test_dyn_row_stochastic_bounds_scaling_and_scope():
    rng = np.random.default_rng(9)
    S, m, N = 8, 5, 29
    z = np.maximum(rng.standard_normal((1, N, m)), 0) ** 2
    res = O.dyn_context(z, S, 1e-8)
    for (b, i), out in res.items():
        r = O.split_rows(N, S, i)
        zi = z[0, r.start:r.stop]
        assert np.all(out >= -1e-15) and np.all(out <= zi.max(axis=0) + 1e-12)   # sub-convex mix
    res2 = O.dyn_context(3.5 * z, S, 1e-8)
    for key in res:
        np.testing.assert_allclose(res2[key], 3.5 * res[key], rtol=1e-9)
    # only tokens of the same split mix: changing split 2 leaves split 0 unchanged
    z3 = z.copy()
    z3[0, 2 * S:3 * S] += 1.0
    np.testing.assert_array_equal(O.dyn_context(z3, S, 1e-8)[(0, 0)], res[(0, 0)])


def test_dyn_monotonic_in_similarity():
    """[summary] appendix A: raising one token's similarity to the target weakly raises its
    normalised weight and weakly lowers the others. Moving z_q toward z_p raises G_pq only."""
    rng = np.random.default_rng(10)
    m = 6
    zp = rng.uniform(0.1, 1, m)
    others = rng.uniform(0.1, 1, (3, m))
    def weights(zq):
        zs = np.vstack([zp, zq, others])
        n = O.unit_rows(zs)
        g = n @ n.T
        return g[0] / (g[0].sum() + 1e-8)
    zq0 = rng.uniform(0.1, 1, m)
    w0 = weights(zq0)
    w1 = weights(0.5 * zq0 + 0.5 * zp / np.linalg.norm(zp) * np.linalg.norm(zq0))
    assert w1[1] > w0[1] and np.all(w1[[0, 2, 3, 4]] <= w0[[0, 2, 3, 4]] + 1e-15)
    # and the oracle's output equals the explicit weighted sum with these weights
    zs = np.vstack([zp, zq0, others])
    out = O.dyn_context(zs[None], 5, 1e-8)[(0, 0)]
    np.testing.assert_allclose(out[0], w0 @ zs, rtol=1e-13)


def test_dyn_brute_force_tiny():
    rng = np.random.default_rng(11)
    S, m, N, eps = 3, 4, 8, 1e-8
    z = np.maximum(rng.standard_normal((1, N, m)), 0)
    z[0, 4] = 0.0                                         # zero token: no similarity to anything
    res = O.dyn_context(z, S, eps)
    for i in range(-(-N // S)):
        toks = list(range(i * S, min(i * S + S, N)))
        for a, p in enumerate(toks):
            np_ = math.sqrt(sum(v * v for v in z[0, p]))
            g = []
            for q in toks:
                nq = math.sqrt(sum(v * v for v in z[0, q]))
                dot = sum(z[0, p, c] * z[0, q, c] for c in range(m))
                g.append(0.0 if np_ == 0 or nq == 0 else dot / (np_ * nq))
            den = sum(g) + eps
            for c in range(m):
                want = sum(g[bq] * z[0, q, c] for bq, q in enumerate(toks)) / den
                assert res[(0, i)][a, c] == pytest.approx(want, abs=1e-12)


# ----------------------------------------------------------------------------- contextualizer layers
def test_static_layer_closed_forms():
    """V = I gives Z_t back; a permutation V permutes the split's tokens (padding rows are
    zero, so a valid row that draws from a padding slot is zero); the bias adds one value per
    token position; ReLU clips the identity result at 0."""
    rng = np.random.default_rng(21)
    S, m = 4, 3
    z = rng.standard_normal((1, 10, m))                 # splits of 4, 4, 2 valid tokens
    zero_b = np.zeros(S)
    out = O.static_layer(z, S, np.eye(S), zero_b, "identity")
    for (b, i), rows in out.items():
        r = O.split_rows(10, S, i)
        np.testing.assert_array_equal(rows, z[0, r.start:r.stop])
    perm = [2, 0, 3, 1]
    V = np.eye(S)[perm]                                 # row s of V picks token perm[s]
    out = O.static_layer(z, S, V, zero_b, "identity")
    for i in range(3):
        r = O.split_rows(10, S, i)
        for s_, src in enumerate(perm[: len(r)]):
            want = z[0, i * S + src] if i * S + src < 10 else np.zeros(m)
            np.testing.assert_array_equal(out[(0, i)][s_], want)
    bias = rng.standard_normal(S)
    a = O.static_layer(z, S, V, bias, "identity")
    c = O.static_layer(z, S, V, bias, "relu")
    for key in a:
        n = a[key].shape[0]
        base = O.static_layer(z, S, V, zero_b, "identity")[key]
        np.testing.assert_allclose(a[key] - base, np.repeat(bias[:n, None], m, axis=1), atol=1e-15)
        np.testing.assert_array_equal(c[key], np.where(a[key] > 0, a[key], 0.0))


def test_dyn_layer_reduces_to_core():
    """With b = 0 and the identity the layer is the core S~ Z_t; ReLU output is
    non-negative and equals the clipped identity result."""
    rng = np.random.default_rng(22)
    S, m = 5, 4
    z = rng.standard_normal((2, 13, m))
    zero_b = np.zeros(S)
    core = O.dyn_context(z, S, 1e-8)
    lay = O.dyn_layer(z, S, 1e-8, zero_b, "identity")
    for key in core:
        np.testing.assert_array_equal(lay[key], core[key])
    bias = rng.standard_normal(S)
    a = O.dyn_layer(z, S, 1e-8, bias, "identity")
    c = O.dyn_layer(z, S, 1e-8, bias, "relu")
    for key in a:
        assert np.all(c[key] >= 0)
        np.testing.assert_array_equal(c[key], np.where(a[key] > 0, a[key], 0.0))


# ----------------------------------------------------------------------------- normalisation variants
def test_norm_variants_closed_forms():
    """Orthogonal tokens (G = I on the n valid tokens): softmax weights e / (e + n - 1) on the
    diagonal and 1 / (e + n - 1) elsewhere; rms weight sqrt(n / (1 + n eps)) on the diagonal;
    none gives Z back; sum gives Z / (1 + eps). A constant split (G = all ones): softmax 1 / n,
    rms 1 / sqrt(1 + eps), none 1, sum 1 / (n + eps), each times the shared token."""
    eps = 1e-3
    n, m = 3, 5
    z = np.zeros((1, n, m))
    z[0, 0, 0], z[0, 1, 1], z[0, 2, 4] = 2.0, -1.5, 0.5           # pairwise orthogonal
    e = math.e
    soft = O.dyn_context(z, n, eps, norm="softmax")[(0, 0)]
    want = np.array([[(e if p == q else 1.0) / (e + n - 1) for q in range(n)] for p in range(n)]) @ z[0]
    np.testing.assert_allclose(soft, want, rtol=1e-14, atol=1e-15)
    rms = O.dyn_context(z, n, eps, norm="rms")[(0, 0)]
    np.testing.assert_allclose(rms, math.sqrt(n / (1 + n * eps)) * z[0], rtol=1e-14)
    np.testing.assert_allclose(O.dyn_context(z, n, eps, norm="none")[(0, 0)], z[0], rtol=1e-15)
    np.testing.assert_allclose(O.dyn_context(z, n, eps, norm="sum")[(0, 0)], z[0] / (1 + eps), rtol=1e-15)
    c = np.tile(np.array([0.3, -1.0, 2.0, 0.0, 0.7]), (1, 4, 1))
    for norm, f in (("softmax", 4 * (1 / 4)), ("rms", 4 / math.sqrt(1 + eps)), ("none", 4.0),
                    ("sum", 4 / (4 + eps))):
        out = O.dyn_context(c, 4, eps, norm=norm)[(0, 0)]
        np.testing.assert_allclose(out, f * c[0], rtol=1e-13, err_msg=norm)


def test_norm_variants_row_properties_and_padding():
    """Softmax rows sum to 1 and stay positive with signed cosines; rms rows have unit mean
    square up to eps; padding tokens take part in no row (ragged split equals the same tokens
    alone); the default is the sum normalisation."""
    rng = np.random.default_rng(31)
    S, m = 6, 4
    z = rng.standard_normal((1, 10, m))                 # splits of 6 and 4 valid tokens
    for i in range(2):
        r = O.split_rows(10, S, i)
        nz = O.unit_rows(z[0, r.start:r.stop])
        sim = nz @ nz.T
        sm = O.row_normalise(sim, "softmax", 1e-8)
        np.testing.assert_allclose(sm.sum(axis=1), 1.0, rtol=1e-14)
        assert np.all(sm > 0)
        rm = O.row_normalise(sim, "rms", 0.0)
        np.testing.assert_allclose((rm * rm).mean(axis=1), 1.0, rtol=1e-13)
        for norm in O.NORMS:
            alone = O.dyn_context(z[:, r.start:r.stop], S, 1e-8, norm=norm)[(0, 0)]
            np.testing.assert_allclose(O.dyn_context(z, S, 1e-8, norm=norm)[(0, i)], alone, rtol=1e-14)
    np.testing.assert_array_equal(O.dyn_context(z, S, 1e-8)[(0, 1)], O.dyn_context(z, S, 1e-8, norm="sum")[(0, 1)])
    with pytest.raises(ValueError):
        O.row_normalise(np.eye(2), "l1", 1e-8)


# ----------------------------------------------------------------------------- enricher and fuser
def test_enrich_closed_forms():
    """U = I and b = 0 give ReLU(x)^2; a one-hot column of U picks a feature; the bias shifts
    before the activation; the output is never negative."""
    x = np.array([[1.5, -2.0, 0.25], [-0.5, 3.0, 0.0]])
    np.testing.assert_array_equal(O.enrich(x, np.eye(3), np.zeros(3)), np.maximum(x, 0) ** 2)
    U = np.zeros((3, 4))
    U[2, 0] = 1.0
    U[0, 3] = -2.0
    b = np.array([0.5, -1.0, 0.0, 1.0])
    want = np.stack([np.maximum(x[:, 2] + 0.5, 0) ** 2, np.zeros(2), np.zeros(2),
                     np.maximum(-2 * x[:, 0] + 1.0, 0) ** 2], axis=1)
    np.testing.assert_allclose(O.enrich(x, U, b), want, rtol=1e-15)
    rng = np.random.default_rng(41)
    assert np.all(O.enrich(rng.standard_normal((5, 6)), rng.standard_normal((6, 9)), rng.standard_normal(9)) >= 0)


def test_fuse_closed_forms():
    """O = I returns the joined head and contextualised tail plus the residual; the head part of
    O only sees Z_h (the tail of z is never read) and its tail part only sees c."""
    rng = np.random.default_rng(42)
    m_h, m_t, d = 3, 2, 5
    z = rng.standard_normal((4, m_h + m_t))
    c = rng.standard_normal((4, m_t))
    xr = rng.standard_normal((4, d))
    np.testing.assert_allclose(O.fuse(z, m_h, c, np.eye(d), xr), np.concatenate([z[:, :m_h], c], 1) + xr, rtol=1e-15)
    Oh = np.zeros((m_h + m_t, d))
    Oh[:m_h] = rng.standard_normal((m_h, d))
    z2 = z.copy()
    z2[:, m_h:] = 1e6                                    # the tail of Z is not read
    np.testing.assert_allclose(O.fuse(z2, m_h, c, Oh, 0 * xr), z[:, :m_h] @ Oh[:m_h], rtol=1e-14)
    Ot = np.zeros((m_h + m_t, d))
    Ot[m_h:] = rng.standard_normal((m_t, d))
    np.testing.assert_allclose(O.fuse(z, m_h, c, Ot, 0 * xr), c @ Ot[m_h:], rtol=1e-14)


def test_neural_layer_reduces_to_parts():
    """With U = I (m = d), b = 0, no head and O = I the layer is X + c(ReLU(X)^2); with a zero O
    it is the residual alone."""
    rng = np.random.default_rng(43)
    S, d = 4, 3
    x = rng.standard_normal((1, 10, d))
    ctx = lambda zt: O.dyn_context(zt, S, 1e-8)
    y = O.neural_layer(x, S, np.eye(d), np.zeros(d), 0, np.eye(d), ctx)
    c = O.assemble(O.dyn_context(np.maximum(x, 0) ** 2, S, 1e-8), 1, 10, S, d)
    np.testing.assert_allclose(y, x + c, rtol=1e-14)
    np.testing.assert_array_equal(O.neural_layer(x, S, np.eye(d), np.zeros(d), 1, np.zeros((d, d)), ctx), x)
