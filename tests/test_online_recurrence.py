"""The online five-scalar recurrence, modelled in numpy, against the fp64 oracle.

The pages give the forward as five running per-row scalars (m1, l1, m2, l2, acc) updated per
key tile and finalised as KL = acc / l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t
(gist.science/pt "Metodologia" section 1). The agents-report.net pseudocode updates l1, l2 and
acc without rescaling them when a running max grows; the reading adopted here rescales all
three by exp(m_old - m_new) as in online softmax (hackmd lecture notes, section 4 on the
FlashAttention correction factor), with acc sharing l1's factor. This file shows that the
rescaled recurrence equals the definition for any tiling, including causal tile skipping and
a ragged last tile, that partial states over disjoint key subsets merge associatively (which
the GPU kernel relies on: each lane keeps its own partial state), and that the literal
no-rescale pseudocode does not.
"""
import math

import numpy as np
import pytest

from oracle.reference import forward_slice


def online_rows(q1, k1, q2, k2, scale, causal, tile, rescale=True, key_subset=None):
    nq, nk = q1.shape[0], k1.shape[0]
    out = np.empty((3, nq))
    states = []
    for i in range(nq):
        m1 = m2 = -np.inf
        l1 = l2 = acc = 0.0
        last = min(nk, i + 1) if causal else nk           # tiles past the frontier are skipped
        keys = np.arange(last) if key_subset is None else np.array(
            [j for j in key_subset if j < last], dtype=int)
        for t0 in range(0, keys.shape[0], tile):
            js = keys[t0:t0 + tile]
            s1 = scale * (k1[js] @ q1[i])
            s2 = scale * (k2[js] @ q2[i])
            n1, n2 = max(m1, s1.max()), max(m2, s2.max())
            if rescale:
                a1, a2 = math.exp(m1 - n1), math.exp(m2 - n2)
                l1, acc, l2 = l1 * a1, acc * a1, l2 * a2
            m1, m2 = n1, n2
            p1 = np.exp(s1 - m1)
            l1 += p1.sum()
            l2 += np.exp(s2 - m2).sum()
            acc += (p1 * (s1 - s2)).sum()
        states.append((m1, l1, m2, l2, acc))
        if l1 == 0.0:                 # empty key subset: no visible key, state stays empty
            out[:, i] = np.nan
            continue
        lse1, lse2 = m1 + math.log(l1), m2 + math.log(l2)
        out[:, i] = (acc / l1 + lse2 - lse1, lse1, lse2)
    return out, states


def merge(a, b):
    """Associative merge of two partial states over disjoint key sets."""
    m1, m2 = max(a[0], b[0]), max(a[2], b[2])
    fa1, fb1 = math.exp(a[0] - m1), math.exp(b[0] - m1)
    fa2, fb2 = math.exp(a[2] - m2), math.exp(b[2] - m2)
    return (m1, a[1] * fa1 + b[1] * fb1, m2, a[3] * fa2 + b[3] * fb2, a[4] * fa1 + b[4] * fb1)


def rand(nq, nk, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((n, d)) * 1.5 for n in (nq, nk, nq, nk)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 7, 16, 64, 1000])
def test_rescaled_recurrence_equals_definition(causal, tile):
    nq, nk, d = 37, 53, 16
    q1, k1, q2, k2 = rand(nq, nk, d, 1)
    scale = 1 / math.sqrt(d)
    got, _ = online_rows(q1, k1, q2, k2, scale, causal, tile)
    ref = np.array(forward_slice(q1, k1, q2, k2, scale, causal))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_partial_states_merge(causal):
    nq, nk, d = 20, 64, 8
    q1, k1, q2, k2 = rand(nq, nk, d, 2)
    scale = 0.4
    # two "lanes" own interleaved groups of 4 keys, as the two halves of a 32x32 MFMA tile do
    ids = np.arange(nk)
    half_a = ids[(ids // 4) % 2 == 0]
    half_b = ids[(ids // 4) % 2 == 1]
    _, sa = online_rows(q1, k1, q2, k2, scale, causal, 8, key_subset=half_a)
    _, sb = online_rows(q1, k1, q2, k2, scale, causal, 8, key_subset=half_b)
    ref = np.array(forward_slice(q1, k1, q2, k2, scale, causal))
    for i in range(nq):
        # rows 0..3 (causal): lane b holds no visible key, its state is empty and merges as 0
        m1, l1, m2, l2, acc = merge(sa[i], sb[i])
        lse1, lse2 = m1 + math.log(l1), m2 + math.log(l2)
        np.testing.assert_allclose([acc / l1 + lse2 - lse1, lse1, lse2], ref[:, i], rtol=1e-12,
                                   atol=1e-12)


def test_literal_pseudocode_without_rescale_is_wrong():
    nq, nk, d = 37, 53, 16
    q1, k1, q2, k2 = rand(nq, nk, d, 3)
    scale = 1 / math.sqrt(d)
    got, _ = online_rows(q1, k1, q2, k2, scale, False, 7, rescale=False)
    ref = np.array(forward_slice(q1, k1, q2, k2, scale, False))
    assert np.abs(got[0] - ref[0]).max() > 1e-2
