"""GPU parity of the adaptive entry points (streamkl_fwd, streamkl_bwd_fixP1, streamkl_bwd_fixP2),
which choose their kernels from the sizes: at every query-row count they match the fp64 oracle,
and they run exactly the path their plan names (bitwise equal to the explicit entry point of
that path: split-K or one-pass forward; fused, key-split dQ + dK, or one-kernel dQ + dK)."""
import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
import oracle
from oracle.reference import backward_slice, forward_slice
from parity_util import assert_grad_close, assert_rows_close, grad_atol, to_np
from test_gpu_parity import check_grads, make, shape_id

pytestmark = pytest.mark.gpu

# (batch, heads, n_q, n_k, head_dim, causal): query-row counts on both sides of the fused limit
# (64) and of the split plans
SHAPES = [(1, 4, nq, 4096, 128, False) for nq in (1, 33, 64, 65, 300, 512)] + [
    (2, 2, 40, 3000, 64, True), (1, 3, 200, 2500, 64, True), (1, 2, 1000, 1000, 128, True)]


def explicit_forward(d, w):
    if skl.streamkl_fwd_workspace_size(d["q1"], d["k1"], causal=w.causal) > 0:
        return skl.streamkl_fwd_splitk(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    return skl.streamkl_fwd_one_pass(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)


def explicit_backward(setting, d, w, l1, l2, kl):
    args = (setting, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl, d["g"])
    if w.n_q <= 64:
        return skl.streamkl_bwd_fused(*args, causal=w.causal)
    dk = skl.streamkl_bwd_dk(*args, causal=w.causal)
    if skl.streamkl_bwd_dq_splitk_workspace_size(d["q1"], d["k1"], causal=w.causal) > 0:
        return skl.streamkl_bwd_dq_splitk(*args, causal=w.causal), dk
    return skl.streamkl_bwd_dq(*args, causal=w.causal), dk


def plain_backward(setting, d, w, l1, l2, kl):
    if setting == 1:
        return skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, d["g"],
                                      causal=w.causal)
    return skl.streamkl_bwd_fixP2(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl, d["g"],
                                  causal=w.causal)


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
def test_adaptive_paths_match_oracle_and_their_plan(shape):
    print(f"adaptive {shape_id(shape)}", flush=True)
    w, d, r = make(shape, "perturb")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    assert_rows_close(to_np(kl), rk, "KL")
    assert_rows_close(to_np(l1), r1, "LSE1")
    assert_rows_close(to_np(l2), r2, "LSE2")
    for a, b in zip((kl, l1, l2), explicit_forward(d, w)):
        assert torch.equal(a, b)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        dq, dk = plain_backward(setting, d, w, l1, l2, kl)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        check_grads(w, r, setting, dq, dk, rdq, rdk, lmax, tag="adaptive ")
        eq, ek = explicit_backward(setting, d, w, l1, l2, kl)
        assert torch.equal(dq, eq) and torch.equal(dk, ek)


@pytest.mark.parametrize("nq", [1, 64, 65, 512])
def test_adaptive_paths_at_64k_keys(nq):
    """The few-query-row bench shape (32 heads, 64K keys, d = 128): plain entry points against
    their plan's explicit path (every output) and two heads against the oracle (every output)."""
    print(f"adaptive 64k nq={nq}", flush=True)
    shape = (1, 32, nq, 65536, 128, False)
    w, d, r = make(shape, "perturb")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"])
    for a, b in zip((kl, l1, l2), explicit_forward(d, w)):
        assert torch.equal(a, b)
    dq, dk = plain_backward(1, d, w, l1, l2, kl)
    eq, ek = explicit_backward(1, d, w, l1, l2, kl)
    assert torch.equal(dq, eq) and torch.equal(dk, ek)
    kl_h, l1_h, l2_h, dq_h, dk_h = (to_np(t) for t in (kl, l1, l2, dq, dk))
    for hd in (0, 31):
        a = {n: r[n][0, hd] for n in ("q1", "k1", "q2", "k2")}
        rk, r1, r2 = forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], w.scale, False)
        assert_rows_close(kl_h[0, hd], rk, f"head {hd} KL")
        assert_rows_close(l1_h[0, hd], r1, f"head {hd} LSE1")
        assert_rows_close(l2_h[0, hd], r2, f"head {hd} LSE2")
        lmax = max(np.abs(r1).max(), np.abs(r2).max())
        rdq, rdk = backward_slice(1, a["q1"], a["k1"], a["q2"], a["k2"], r["g"][0, hd], w.scale,
                                  False)
        aq = grad_atol(w.scale, r["g"], lmax, a["k2"])
        ak = grad_atol(w.scale, r["g"], lmax, a["q2"], mass=w.n_q / w.n_k)
        assert_grad_close(dq_h[0, hd], rdq, f"head {hd} dQ", aq)
        assert_grad_close(dk_h[0, hd], rdk, f"head {hd} dK", ak)


def test_adaptive_caller_workspace():
    """A caller-provided workspace of exactly the reported size, filled with NaN, gives the same
    bits as the binding's own allocation; one byte short is rejected."""
    print("adaptive workspace", flush=True)
    w, d, r = make((1, 4, 33, 4096, 128, False), "perturb")
    nf = skl.streamkl_fwd_workspace_size(d["q1"], d["k1"])
    nb = skl.streamkl_bwd_workspace_size(d["q1"], d["k1"])
    assert nf > 0 and nb > 0
    a = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"])
    wsf = torch.full((nf,), 255, dtype=torch.uint8, device="cuda")
    b = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], workspace=wsf)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    g1 = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], a[1], a[2], d["g"])
    wsb = torch.full((nb,), 255, dtype=torch.uint8, device="cuda")
    g2 = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], a[1], a[2], d["g"],
                                workspace=wsb)
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])
    with pytest.raises(skl.StreamKLError):
        skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], a[1], a[2], d["g"],
                               workspace=wsb[: nb - 1])
    with pytest.raises(skl.StreamKLError):
        skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], workspace=wsf[: nf - 1])
