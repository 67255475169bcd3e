"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins notice.

Each mutant replaces one internal function of `oracle.reference` with a subtly wrong copy (a
sign flip, a dropped term, the wrong weights, an off-by-one mask, a transposed operand); the
independent pins (mpmath brute force, torch float64 autograd) must then disagree.
"""
import math

import numpy as np
import pytest
import torch

import oracle.reference as R
from test_oracle_pins import mp_forward, rand_slice, torch_kl


def _torch_grads(setting, q1, k1, q2, k2, g, scale, causal):
    T = [torch.tensor(x, dtype=torch.float64) for x in (q1, k1, q2, k2)]
    free = (2, 3) if setting == 1 else (0, 1)
    for i in free:
        T[i].requires_grad_(True)
    kl, _, _ = torch_kl(*T, scale, causal)
    (kl * torch.tensor(g)).sum().backward()
    return T[free[0]].grad.numpy(), T[free[1]].grad.numpy()


def mutant_sign(setting, S1, S2, vis, g_rows):
    _, lp1 = R._log_softmax(S1)
    _, lp2 = R._log_softmax(S2)
    return g_rows[:, None] * (np.exp(lp1) - np.exp(lp2))


def mutant_dropped_kl(setting, S1, S2, vis, g_rows):
    _, lp1 = R._log_softmax(S1)
    _, lp2 = R._log_softmax(S2)
    with np.errstate(invalid="ignore"):
        return g_rows[:, None] * np.exp(lp1) * np.where(vis, lp1 - lp2, 0.0)


def mutant_weights(logp1, logp2, vis):
    with np.errstate(invalid="ignore"):
        diff = np.where(vis, logp1 - logp2, 0.0)
    p2 = np.exp(logp2)
    return (p2 * diff).sum(axis=1), np.exp(logp1), diff


_orig_logits = R.logits_block


def mutant_mask(q, k, scale, causal, rows):
    S, vis = _orig_logits(q, k, scale, causal, rows)
    if causal:
        off = np.arange(S.shape[1])[None, :] == np.asarray(rows)[:, None]
        vis = vis & ~off
        vis[:, 0] = True
        S = np.where(vis, S, -np.inf)
    return S, vis


@pytest.mark.parametrize("setting,name", [(1, "sign"), (2, "dropped_kl")])
def test_gradient_mutants_are_caught(monkeypatch, setting, name):
    nq, nk, d = 24, 24, 8
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=17)
    g = np.random.default_rng(3).random(nq) + 0.1
    scale = 1 / math.sqrt(d)
    ref = _torch_grads(setting, q1, k1, q2, k2, g, scale, False)
    monkeypatch.setattr(R, "_dS_block", {"sign": mutant_sign, "dropped_kl": mutant_dropped_kl}[name])
    dq, dk = R.backward_slice(setting, q1, k1, q2, k2, g, scale, False)
    assert not np.allclose(dq, ref[0], rtol=1e-6, atol=1e-9)


def test_transposed_operand_is_caught(monkeypatch):
    nq = nk = 16
    d = 16
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=19)
    g = np.ones(nq)
    scale = 0.25
    ref = _torch_grads(1, q1, k1, q2, k2, g, scale, False)
    orig = R._dS_block
    monkeypatch.setattr(R, "_dS_block", lambda *a: orig(*a).T)
    dq, _ = R.backward_slice(1, q1, k1, q2, k2, g, scale, False)
    assert not np.allclose(dq, ref[0], rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_mutants_are_caught(monkeypatch, causal):
    nq, nk, d = 5, 6, 3
    q1, k1, q2, k2 = rand_slice(nq, nk, d, seed=23, std=1.5)
    scale = 1 / math.sqrt(d)
    ref = mp_forward(q1, k1, q2, k2, scale, causal)
    monkeypatch.setattr(R, "_kl_rows", mutant_weights)
    got = np.array(R.forward_slice(q1, k1, q2, k2, scale, causal))
    assert not np.allclose(got[0], ref[0], rtol=1e-9, atol=1e-12)
    monkeypatch.undo()
    if causal:
        monkeypatch.setattr(R, "logits_block", mutant_mask)
        got = np.array(R.forward_slice(q1, k1, q2, k2, scale, causal))
        assert not np.allclose(got, ref, rtol=1e-9, atol=1e-12)
