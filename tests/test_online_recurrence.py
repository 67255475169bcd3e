"""The online five-scalar state, modelled in numpy from its definition, against the fp64 oracle.

The pages describe the forward as five running per-row scalars (m1, l1, m2, l2, acc) carried
over the key tiles and finished as KL = acc / l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t
(gist.science/pt "Resumo Tecnico: StreamKL", "Metodologia" section 1, "Formulacao Online").
Here the state of any set T of keys of one query row is defined directly:

    m_t = max_{j in T} S_t[j],   l_t = sum_{j in T} exp(S_t[j] - m_t),
    acc = sum_{j in T} exp(S1[j] - m1) (S1[j] - S2[j]),

and the state of a union of two disjoint sets follows from the states of the parts (`merge`:
the larger maximum wins, the other part's sums are multiplied by exp(m_part - m), acc with
side 1's factor; the correction factor of online softmax, hackmd lecture notes on
FlashAttention, section 4). Streaming the keys is then folding tile states with `merge`, which is
what the kernels do per lane, and the two lanes of a row merge their partial states at the end.

Shown here: folding tile states equals the definition for any tiling (with causal tile
skipping and a ragged last tile), disjoint interleaved key subsets merge to the same result,
and adding a new tile's sums without rescaling the old ones (taking the pages' simplified
forward pseudocode on agents-report.net, section on the simplified forward, literally) is wrong
on a hand-built two-tile row.
"""
import math

import numpy as np
import pytest

from oracle.reference import forward_slice

EMPTY = (-math.inf, 0.0, -math.inf, 0.0, 0.0)


def set_state(s1, s2):
    """The state (m1, l1, m2, l2, acc) of a non-empty key set with logits s1, s2, by definition."""
    m1, m2 = float(s1.max()), float(s2.max())
    p1 = np.exp(s1 - m1)
    return (m1, float(p1.sum()), m2, float(np.exp(s2 - m2).sum()), float((p1 * (s1 - s2)).sum()))


def merge(a, b):
    """State of the union of two disjoint key sets from the states of the parts."""
    if a[1] == 0.0:
        return b
    if b[1] == 0.0:
        return a
    m1, m2 = max(a[0], b[0]), max(a[2], b[2])
    fa1, fb1 = math.exp(a[0] - m1), math.exp(b[0] - m1)
    fa2, fb2 = math.exp(a[2] - m2), math.exp(b[2] - m2)
    return (m1, a[1] * fa1 + b[1] * fb1, m2, a[3] * fa2 + b[3] * fb2, a[4] * fa1 + b[4] * fb1)


def finish(st):
    m1, l1, m2, l2, acc = st
    lse1, lse2 = m1 + math.log(l1), m2 + math.log(l2)
    return acc / l1 + lse2 - lse1, lse1, lse2


def streamed_row_states(q1, k1, q2, k2, scale, causal, tile, key_subset=None):
    """Per query row: the state folded over tiles of `tile` visible keys (optionally only the
    keys in key_subset), tiles past the causal frontier skipped."""
    nk = k1.shape[0]
    states = []
    for i in range(q1.shape[0]):
        last = min(nk, i + 1) if causal else nk
        keys = np.arange(last) if key_subset is None else np.array(
            [j for j in key_subset if j < last], dtype=int)
        st = EMPTY
        for t0 in range(0, keys.shape[0], tile):
            js = keys[t0:t0 + tile]
            st = merge(st, set_state(scale * (k1[js] @ q1[i]), scale * (k2[js] @ q2[i])))
        states.append(st)
    return states


def rand(nq, nk, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((n, d)) * 1.5 for n in (nq, nk, nq, nk)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 7, 16, 64, 1000])
def test_folded_tile_states_equal_definition(causal, tile):
    nq, nk, d = 37, 53, 16
    q1, k1, q2, k2 = rand(nq, nk, d, 1)
    scale = 1 / math.sqrt(d)
    got = np.array([finish(st) for st in streamed_row_states(q1, k1, q2, k2, scale, causal,
                                                             tile)]).T
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
    sa = streamed_row_states(q1, k1, q2, k2, scale, causal, 8, key_subset=half_a)
    sb = streamed_row_states(q1, k1, q2, k2, scale, causal, 8, key_subset=half_b)
    ref = np.array(forward_slice(q1, k1, q2, k2, scale, causal))
    for i in range(nq):
        # rows 0..3 (causal): lane b holds no visible key, its state is empty
        np.testing.assert_allclose(finish(merge(sa[i], sb[i])), ref[:, i], rtol=1e-12,
                                   atol=1e-12)


def test_sums_without_rescaling_are_wrong():
    """One row, two one-key tiles with logits (S1, S2) = (0, 0) then (5, 1). By definition
    l1 = exp(0 - 5) + 1 relative to m1 = 5; adding the second tile's exp(5 - 5) = 1 to the first
    tile's l1 = 1 (taken relative to m1 = 0) without rescaling gives l1 = 2, and LSE1 and KL go
    wrong by O(1)."""
    s1 = np.array([0.0, 5.0])
    s2 = np.array([0.0, 1.0])
    exact = finish(merge(set_state(s1[:1], s2[:1]), set_state(s1[1:], s2[1:])))
    lse = lambda s: math.log(np.exp(s).sum())  # noqa: E731
    p1 = np.exp(s1 - lse(s1))
    kl = float((p1 * ((s1 - lse(s1)) - (s2 - lse(s2)))).sum())
    np.testing.assert_allclose(exact, (kl, lse(s1), lse(s2)), rtol=1e-13)
    # no rescale: the running maxima move to the new tile's, the old sums are kept as they are
    m1, l1, m2, l2, acc = set_state(s1[:1], s2[:1])
    m1, m2 = max(m1, s1[1]), max(m2, s2[1])
    l1 += math.exp(s1[1] - m1)
    l2 += math.exp(s2[1] - m2)
    acc += math.exp(s1[1] - m1) * (s1[1] - s2[1])
    naive = finish((m1, l1, m2, l2, acc))
    assert abs(naive[1] - exact[1]) > 0.5 and abs(naive[0] - exact[0]) > 0.5
