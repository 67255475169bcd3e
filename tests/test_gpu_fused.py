"""GPU parity of the fused few-query backward (one key-major pass for dQ and dK, n_q <= 64)
against the fp64 oracle, and against the separate dQ / dK kernels."""
import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
import oracle
from parity_util import assert_grad_close, grad_atol, to_np
from test_gpu_parity import bf16_ds_bound, check_grads, make, shape_id, signed_g

pytestmark = pytest.mark.gpu

# (batch, heads, n_q, n_k, head_dim, causal)
SHAPES = [
    (1, 2, 1, 4096, 128, False),
    (1, 3, 17, 5000, 64, False),
    (2, 2, 64, 3000, 128, True),
    (1, 1, 33, 1, 64, False),
    (1, 2, 40, 700, 128, True),
    (1, 2, 64, 1030, 128, False),
    (1, 1, 5, 600, 64, True),
]


def run(setting, w, d, l1, l2, kl):
    return skl.streamkl_bwd_fused(setting, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2,
                                  kl if setting == 2 else None, d["g"], causal=w.causal)


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
@pytest.mark.parametrize("recipe", ["iid", "perturb", "shared_k"])
def test_fused_matches_oracle_and_separate(shape, recipe):
    print(f"fused {shape_id(shape)} {recipe}", flush=True)
    w, d, r = make(shape, recipe)
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    _, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        dq, dk = run(setting, w, d, l1, l2, kl)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        check_grads(w, r, setting, dq, dk, rdq, rdk, lmax, tag="fused ")
        # the one-kernel dQ and dK passes (what the adaptive entry points run at large n_q)
        sq = skl.streamkl_bwd_dq(setting, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl, d["g"],
                                 causal=w.causal)
        sk = skl.streamkl_bwd_dk(setting, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl, d["g"],
                                 causal=w.causal)
        # the same dS in float32 on both paths, other summation order, both rounded to bf16;
        # the float32 floor of the oracle comparison covers rows whose gradient is rounding
        # noise (e.g. a causal row that sees one key)
        qf, kf = (r["q2"], r["k2"]) if setting == 1 else (r["q1"], r["k1"])
        aq = grad_atol(w.scale, r["g"], lmax, kf)
        ak = grad_atol(w.scale, r["g"], lmax, qf, mass=w.n_q / w.n_k)
        assert_grad_close(to_np(dq), to_np(sq).astype(np.float64), "fused vs separate dQ", aq)
        assert_grad_close(to_np(dk), to_np(sk).astype(np.float64), "fused vs separate dK", ak)


@pytest.mark.parametrize("shape", [(1, 2, 40, 1300, 128, False), (2, 1, 64, 900, 64, True)],
                         ids=shape_id)
def test_fused_signed_upstream_gradient(shape):
    print(f"fused signed g {shape_id(shape)}", flush=True)
    w, d, r = make(shape, "perturb")
    g = signed_g(*shape[:3], seed=9)
    d["g"], r["g"] = torch.from_numpy(g).cuda(), g.astype(np.float64)
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    _, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        dq, dk = run(setting, w, d, l1, l2, kl)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        check_grads(w, r, setting, dq, dk, rdq, rdk, lmax, tag="fused signed ",
                    extra=bf16_ds_bound(setting, r, w.scale, w.causal))


def test_fused_deterministic_and_ignores_workspace_contents():
    print("fused determinism", flush=True)
    w, d, r = make((1, 3, 20, 2500, 128, False), "perturb")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"])
    nbytes = skl.streamkl_bwd_fused_workspace_size(d["q1"], d["k1"])
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    a = skl.streamkl_bwd_fused(1, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, None, d["g"],
                               workspace=ws.view(torch.uint8))
    for _ in range(2):
        ws.fill_(float("inf"))
        b = skl.streamkl_bwd_fused(1, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, None, d["g"],
                                   workspace=ws.view(torch.uint8))
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fused_identical_inputs_give_zeros():
    print("fused identical", flush=True)
    w, d, r = make((1, 2, 9, 1500, 64, False), "iid")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q1"], d["k1"])
    for setting in (1, 2):
        dq, dk = skl.streamkl_bwd_fused(setting, d["q1"], d["k1"], d["q1"], d["k1"], l1, l2, kl,
                                        d["g"])
        assert torch.all(dq == 0) and torch.all(dk == 0)


def test_fused_rejects_too_many_query_rows():
    print("fused n_q limit", flush=True)
    w, d, r = make((1, 1, 65, 128, 64, False), "iid")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"])
    with pytest.raises(skl.StreamKLError) as e:
        skl.streamkl_bwd_fused(1, d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, None, d["g"])
    assert e.value.status == 2


@pytest.mark.parametrize("shape", [(1, 32, 3, 16461, 64, False), (1, 16, 20, 20000, 128, True)],
                         ids=shape_id)
def test_fused_many_key_groups_per_block(shape):
    """Shapes where each block walks several 32-key groups per wave (the operands of the next
    group are fetched during the current one), with a ragged last block."""
    print(f"fused groups {shape_id(shape)}", flush=True)
    w, d, r = make(shape, "perturb")
    nbytes = skl.streamkl_bwd_fused_workspace_size(d["q1"], d["k1"], causal=w.causal)
    B, H, nq, nk, D = shape[:5]
    steps = -(-nk // 128)
    assert nbytes < -(-nk // 128) * B * H * nq * D * 4  # more than one group per wave
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    _, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        dq, dk = run(setting, w, d, l1, l2, kl)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        check_grads(w, r, setting, dq, dk, rdq, rdk, lmax, tag="fused groups ")
    assert steps > 1


def test_fused_at_64k_keys_sampled_slices():
    """32 heads, 64K keys, 16 query rows (the few-query-row bench shape): every output of three
    slices against the oracle."""
    print("fused 64k", flush=True)
    shape = (1, 32, 16, 65536, 128, False)
    w, d, r = make(shape, "perturb")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"])
    dq, dk = run(1, w, d, l1, l2, kl)
    dq_h, dk_h = to_np(dq), to_np(dk)
    from oracle.reference import backward_slice, forward_slice
    for hd in (0, 13, 31):
        a = {n: r[n][0, hd] for n in ("q1", "k1", "q2", "k2")}
        _, r1, r2 = forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], w.scale, False)
        lmax = max(np.abs(r1).max(), np.abs(r2).max())
        rdq, rdk = backward_slice(1, a["q1"], a["k1"], a["q2"], a["k2"], r["g"][0, hd], w.scale,
                                  False)
        aq = grad_atol(w.scale, r["g"], lmax, a["k2"])
        ak = grad_atol(w.scale, r["g"], lmax, a["q2"], mass=w.n_q / w.n_k)
        assert_grad_close(dq_h[0, hd], rdq, f"64k head {hd} dQ", aq)
        assert_grad_close(dk_h[0, hd], rdk, f"64k head {hd} dK", ak)
