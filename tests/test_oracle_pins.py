"""Pins for the fp64 oracle: each test checks it against something other than itself.

- mpmath brute force at 50 digits on tiny inputs (definition of KL between two softmaxes),
- scipy's logsumexp / rel_entr,
- torch CPU float64 log_softmax + kl_div + autograd (independent library, stop-gradient on the
  fixed side) for both backward settings,
- central finite differences of the (separately pinned) forward,
- closed forms (two-key Bernoulli KL, uniform rows, KL to uniform = ln n - entropy) and the
  invariants the mathematics fixes (KL >= 0, identical inputs give exactly 0, the pages'
  identity KL = sum P1 (S1 - S2) - LSE1 + LSE2 from gist.science/pt "Metodologia" section 1,
  key-permutation invariance, query-permutation equivariance, power-of-two scale invariance,
  zero row sums of dS hence zero column sums of dK, causal row 0).
"""
import math

import mpmath
import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
from oracle.reference import forward_slice, backward_slice, dk_rows_slice


def rand_slice(nq, nk, d, seed, std=1.0):
    r = np.random.default_rng(seed)
    return [std * r.standard_normal((n, d)) for n in (nq, nk, nq, nk)]


# ------------------------------------------------------------------ mpmath brute force
def mp_forward(q1, k1, q2, k2, scale, causal):
    mpmath.mp.dps = 50
    nq, nk = q1.shape[0], k1.shape[0]
    out = []
    for i in range(nq):
        js = [j for j in range(nk) if (not causal or j <= i)]
        s1 = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                              for a, b in zip(q1[i], k1[j])) for j in js]
        s2 = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                              for a, b in zip(q2[i], k2[j])) for j in js]
        z1 = mpmath.fsum(mpmath.exp(x) for x in s1)
        z2 = mpmath.fsum(mpmath.exp(x) for x in s2)
        p1 = [mpmath.exp(x) / z1 for x in s1]
        p2 = [mpmath.exp(x) / z2 for x in s2]
        kl = mpmath.fsum(a * mpmath.log(a / b) for a, b in zip(p1, p2))
        out.append((float(kl), float(mpmath.log(z1)), float(mpmath.log(z2))))
    return np.array(out).T


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(3, 5, 4), (6, 6, 3), (1, 7, 2)])
def test_forward_vs_mpmath(causal, shape):
    nq, nk, d = shape
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=nq * 100 + nk, std=1.5)
    scale = 1 / math.sqrt(d)
    ref = mp_forward(q1, k1, q2, k2, scale, causal)
    got = np.array(forward_slice(q1, k1, q2, k2, scale, causal))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ scipy
@pytest.mark.parametrize("causal", [False, True])
def test_forward_vs_scipy(causal):
    nq, nk, d = 70, 90, 16
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=7)
    scale = 0.25
    kl, lse1, lse2 = forward_slice(q1, k1, q2, k2, scale, causal)
    for i in range(nq):
        n = min(nk, i + 1) if causal else nk
        s1 = scale * np.array([q1[i] @ k1[j] for j in range(n)])
        s2 = scale * np.array([q2[i] @ k2[j] for j in range(n)])
        np.testing.assert_allclose(lse1[i], sps.logsumexp(s1), rtol=1e-13)
        np.testing.assert_allclose(lse2[i], sps.logsumexp(s2), rtol=1e-13)
        np.testing.assert_allclose(kl[i], sps.rel_entr(sps.softmax(s1), sps.softmax(s2)).sum(),
                                   rtol=1e-10, atol=1e-14)


# ------------------------------------------------------------------ torch autograd
def torch_kl(q1, k1, q2, k2, scale, causal):
    s1 = scale * q1 @ k1.T
    s2 = scale * q2 @ k2.T
    if causal:
        vis = torch.arange(k1.shape[0])[None, :] <= torch.arange(q1.shape[0])[:, None]
        # a finite fill keeps autograd free of 0 * inf; exp(-1e4) is exactly 0 in float64
        s1 = s1.masked_fill(~vis, -1e4)
        s2 = s2.masked_fill(~vis, -1e4)
    lp1 = torch.log_softmax(s1, dim=-1)
    lp2 = torch.log_softmax(s2, dim=-1)
    terms = torch.nn.functional.kl_div(lp2, lp1, reduction="none", log_target=True)
    if causal:
        terms = torch.where(vis, terms, torch.zeros_like(terms))
    return terms.sum(-1), torch.logsumexp(s1, -1), torch.logsumexp(s2, -1)


@pytest.mark.parametrize("setting", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(40, 40, 8), (33, 57, 16), (57, 33, 16)])
def test_backward_vs_torch_autograd(setting, causal, shape):
    nq, nk, d = shape
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=nq + 3 * nk + setting)
    g = np.random.default_rng(1).random(nq)
    scale = 1 / math.sqrt(d)
    T = [torch.tensor(x, dtype=torch.float64) for x in (q1, k1, q2, k2)]
    free = (2, 3) if setting == 1 else (0, 1)
    for i in free:
        T[i].requires_grad_(True)
    kl, lse1, lse2 = torch_kl(*T, scale, causal)
    (kl * torch.tensor(g)).sum().backward()
    dq_ref, dk_ref = T[free[0]].grad.numpy(), T[free[1]].grad.numpy()

    fk, fl1, fl2 = forward_slice(q1, k1, q2, k2, scale, causal)
    np.testing.assert_allclose(fk, kl.detach().numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(fl1, lse1.detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(fl2, lse2.detach().numpy(), rtol=1e-13)
    dq, dk = backward_slice(setting, q1, k1, q2, k2, g, scale, causal)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(dk, dk_ref, rtol=1e-9, atol=1e-13)
    # column-wise dK and row-sampled dQ agree with the full backward
    keys = np.array([0, nk // 2, nk - 1])
    np.testing.assert_allclose(dk_rows_slice(setting, q1, k1, q2, k2, g, scale, causal, keys),
                               dk[keys], rtol=1e-10, atol=1e-14)
    rows = np.array([nq - 1, 0, nq // 3])
    dqr, _ = backward_slice(setting, q1, k1, q2, k2, g, scale, causal, rows=rows, want_dk=False)
    np.testing.assert_allclose(dqr, dq[rows], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ finite differences
@pytest.mark.parametrize("setting", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_vs_finite_differences(setting, causal):
    nq, nk, d = 12, 15, 6
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=11 + setting)
    g = np.random.default_rng(5).random(nq) + 0.5
    scale = 1 / math.sqrt(d)
    dq, dk = backward_slice(setting, q1, k1, q2, k2, g, scale, causal)
    r = np.random.default_rng(9)
    vq, vk = r.standard_normal(q1.shape), r.standard_normal(k1.shape)
    h = 1e-6

    def loss(t):
        a = [q1, k1, q2, k2]
        fi = (2, 3) if setting == 1 else (0, 1)
        a[fi[0]] = a[fi[0]] + t * vq
        a[fi[1]] = a[fi[1]] + t * vk
        return float(g @ forward_slice(*a, scale, causal)[0])

    fd = (loss(h) - loss(-h)) / (2 * h)
    an = float((dq * vq).sum() + (dk * vk).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


# ------------------------------------------------------------------ closed forms
def test_two_key_bernoulli_closed_form():
    # d = 1, keys [0, x]: P = (1 - sigmoid(s), sigmoid(s)) with s = scale * q * x
    scale = 1.0
    q1, q2 = np.array([[0.7]]), np.array([[-1.3]])
    k = np.array([[0.0], [2.0]])
    kl, lse1, lse2 = forward_slice(q1, k, q2, k, scale, False)
    a = 1 / (1 + math.exp(-0.7 * 2.0))
    b = 1 / (1 + math.exp(1.3 * 2.0))
    want = a * math.log(a / b) + (1 - a) * math.log((1 - a) / (1 - b))
    assert abs(kl[0] - want) < 1e-14
    assert abs(lse1[0] - math.log(1 + math.exp(1.4))) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_rows_and_kl_to_uniform(causal):
    nq, nk, d = 20, 24, 8
    q1, k1, _, k2 = rand_slice(nq, nk, d, seed=3)
    zero = np.zeros((nq, d))
    scale = 0.5
    kl, lse1, lse2 = forward_slice(q1, k1, zero, k2, scale, causal)
    n = np.minimum(np.arange(nq) + 1, nk) if causal else np.full(nq, nk)
    np.testing.assert_array_equal(lse2, np.log(n))          # constant logits: LSE = ln n exactly
    # KL(P || uniform) = ln n - H(P)
    for i in range(nq):
        s = scale * q1[i] @ k1[: n[i]].T
        p = sps.softmax(s)
        assert abs(kl[i] - (math.log(n[i]) + (p * np.log(p)).sum())) < 1e-12


def test_memory_figure_from_the_pages():
    # gist.science/pt "Definicao do Problema": two 64K x 64K distributions x 32 heads in BF16
    # take ~512 GB. 2 distributions * 32 heads * 65536^2 * 2 bytes = 512 GiB exactly.
    assert 2 * 32 * 65536 ** 2 * 2 == 512 * 2 ** 30


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    nq, nk, d = 48, 64, 16
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=21)
    g = np.random.default_rng(2).random(nq)
    scale = 1 / math.sqrt(d)
    kl, lse1, lse2 = forward_slice(q1, k1, q2, k2, scale, causal)
    assert (kl >= -1e-15).all()                                   # Gibbs
    # identical distributions: exactly zero KL and zero gradients
    z, a, b = forward_slice(q1, k1, q1, k1, scale, causal)
    assert (z == 0).all() and (a == b).all()
    for s in (1, 2):
        dq0, dk0 = backward_slice(s, q1, k1, q1, k1, g, scale, causal)
        assert (dq0 == 0).all() and (dk0 == 0).all()
    # the pages' identity: KL = sum_j P1 (S1 - S2) - LSE1 + LSE2
    for i in range(nq):
        n = min(nk, i + 1) if causal else nk
        s1 = scale * q1[i] @ k1[:n].T
        s2 = scale * q2[i] @ k2[:n].T
        p1 = sps.softmax(s1)
        assert abs(kl[i] - ((p1 * (s1 - s2)).sum() - lse1[i] + lse2[i])) < 1e-12
    # power-of-two scale invariance: (scale, Q) and (scale/2, 2Q) give identical logits
    kl2, l12, l22 = forward_slice(2 * q1, k1, 2 * q2, k2, scale / 2, causal)
    np.testing.assert_array_equal(kl2, kl)
    np.testing.assert_array_equal(l12, lse1)
    # query permutation equivariance (non-causal) / causal row 0
    if not causal:
        p = np.random.default_rng(0).permutation(nq)
        klp, _, _ = forward_slice(q1[p], k1, q2[p], k2, scale, causal)
        np.testing.assert_allclose(klp, kl[p], rtol=1e-12, atol=1e-15)
        # key permutation invariance; dK permutes with the keys
        pk = np.random.default_rng(1).permutation(nk)
        klk, _, _ = forward_slice(q1, k1[pk], q2, k2[pk], scale, causal)
        np.testing.assert_allclose(klk, kl, rtol=1e-11, atol=1e-14)
        _, dk = backward_slice(1, q1, k1, q2, k2, g, scale, causal)
        _, dkp = backward_slice(1, q1, k1[pk], q2, k2[pk], g, scale, causal)
        np.testing.assert_allclose(dkp, dk[pk], rtol=1e-10, atol=1e-14)
    else:
        assert kl[0] == 0.0
        assert abs(lse1[0] - scale * q1[0] @ k1[0]) < 1e-14
    # rows of dS sum to zero in both settings, so dK columns sum to zero
    for s in (1, 2):
        _, dk = backward_slice(s, q1, k1, q2, k2, g, scale, causal)
        assert np.abs(dk.sum(0)).max() < 1e-12


def test_slice_independence():
    B, H, nq, nk, d = 2, 3, 17, 23, 8
    r = np.random.default_rng(4)
    q1, q2 = r.standard_normal((2, B, H, nq, d))
    k1, k2 = r.standard_normal((2, B, H, nk, d))
    g = r.random((B, H, nq))
    kl, l1, l2 = oracle.forward(q1, k1, q2, k2, 0.3, True, workers=3)
    dq, dk = oracle.backward(2, q1, k1, q2, k2, g, 0.3, True, workers=2)
    for b in range(B):
        for h in range(H):
            a = forward_slice(q1[b, h], k1[b, h], q2[b, h], k2[b, h], 0.3, True)
            np.testing.assert_array_equal(kl[b, h], a[0])
            e = backward_slice(2, q1[b, h], k1[b, h], q2[b, h], k2[b, h], g[b, h], 0.3, True)
            np.testing.assert_array_equal(dq[b, h], e[0])
            np.testing.assert_array_equal(dk[b, h], e[1])


@pytest.mark.parametrize("causal", [False, True])
def test_dk_rows_slice_with_a_row_range_matches_the_all_rows_backward(causal):
    """dk_rows_slice, the column-by-column dK that checks sampled keys at full sizes, against
    the row-block backward over all rows: with rows = r0 .. n_q - 1 (causal) it must give the
    complete dK of every key >= r0 (no row before r0 sees such a key), and with every row
    (non-causal) the complete dK of any key; both settings."""
    from oracle.reference import backward_slice, dk_rows_slice
    rng = np.random.default_rng(21)
    nq, nk, d = 90, 90, 16
    q1, k1, q2, k2 = (rng.standard_normal((n, d)) for n in (nq, nk, nq, nk))
    g = rng.uniform(0.2, 1.0, nq)
    scale = d ** -0.5
    r0 = 57 if causal else 0
    keys = np.arange(r0, nk)[::3]
    rows = np.arange(r0, nq)
    for setting in (1, 2):
        _, dk = backward_slice(setting, q1, k1, q2, k2, g, scale, causal)
        got = dk_rows_slice(setting, q1, k1, q2, k2, g, scale, causal, keys, rows=rows)
        np.testing.assert_allclose(got, dk[keys], rtol=1e-10, atol=1e-13)
    if causal:
        # a key before r0 is also seen by rows < r0: the truncated sum must differ there
        _, dk = backward_slice(1, q1, k1, q2, k2, g, scale, causal)
        early = dk_rows_slice(1, q1, k1, q2, k2, g, scale, causal, np.array([3]), rows=rows)
        assert np.abs(early - dk[[3]]).max() > 1e-6
