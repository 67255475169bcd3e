"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element, at
sizes the oracle finishes in seconds that still span several tiles and ragged tails."""
import sys

import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
import oracle
from parity_util import assert_grad_close, assert_rows_close, dev_bf16, f64, grad_atol, to_np
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

# (batch, heads, n_q, n_k, head_dim, causal)
SHAPES = [
    (1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 128, True),
    (1, 2, 17, 33, 64, False),
    (1, 1, 64, 64, 128, True),
    (2, 1, 65, 65, 64, True),
    (1, 1, 255, 257, 128, False),
    (1, 2, 257, 255, 128, True),
    (1, 1, 1000, 1000, 64, True),
    (1, 1, 300, 700, 128, True),
    (1, 1, 700, 300, 64, True),
    (1, 1, 129, 1024, 128, False),
    (1, 3, 384, 384, 128, False),
    # many slices: the block -> (slice, row block) mapping over 128 slices
    (8, 16, 70, 90, 64, True),
    # a multiple of 8 slices with several row blocks each: every XCD runs whole slices, their
    # row blocks in order (ragged last blocks on both sides)
    (2, 4, 600, 520, 128, True),
    (1, 8, 1000, 1000, 64, False),
]


def shape_id(s):
    return "B{}H{}_q{}_k{}_d{}_{}".format(*s[:5], "causal" if s[5] else "full")


def make(shape, recipe="iid", seed=123, g_mode="uniform"):
    B, H, nq, nk, d, causal = shape
    w = Workload("test", B, H, nq, nk, d, causal, (1, 2), seed, recipe, sigma=0.3,
                 g_mode=g_mode)
    x = make_inputs(w)
    dev = {n: dev_bf16(x[n]) for n in ("q1", "k1", "q2")}
    dev["k2"] = dev["k1"] if x["k2"] is x["k1"] else dev_bf16(x["k2"])
    dev["g"] = torch.from_numpy(x["g"]).cuda()
    ref = {n: f64(x[n]) for n in ("q1", "k1", "q2", "k2")}
    ref["g"] = x["g"].astype(np.float64)
    return w, dev, ref


def check_grads(w, r, setting, dq, dk, rdq, rdk, lse_max, tag="", extra=(None, None)):
    qf, kf = (r["q2"], r["k2"]) if setting == 1 else (r["q1"], r["k1"])
    aq = grad_atol(w.scale, r["g"], lse_max, kf)
    ak = grad_atol(w.scale, r["g"], lse_max, qf, mass=w.n_q / w.n_k)
    assert_grad_close(to_np(dq), rdq, f"{tag}setting {setting} dQ", aq, extra[0])
    assert_grad_close(to_np(dk), rdk, f"{tag}setting {setting} dK", ak, extra[1])


def bf16_ds_bound(setting, r, scale, causal):
    """Per-element bound on what rounding dS to bf16 (relative error <= 2^-9, doubled for the
    fp32 error of forming dS) can change dQ = scale dS K_f and dK = scale dS^T Q_f, from the
    oracle's own dS: 2^-8 scale |dS| |K_f| and 2^-8 scale |dS|^T |Q_f|."""
    from oracle.reference import _dS_block, logits_block
    qf, kf = (r["q2"], r["k2"]) if setting == 1 else (r["q1"], r["k1"])
    bq, bk = np.zeros(qf.shape), np.zeros(kf.shape)
    B, H, nq = qf.shape[:3]
    for b in range(B):
        for h in range(H):
            rows = np.arange(nq)
            S1, vis = logits_block(r["q1"][b, h], r["k1"][b, h], scale, causal, rows)
            S2, _ = logits_block(r["q2"][b, h], r["k2"][b, h], scale, causal, rows)
            ads = np.abs(_dS_block(setting, S1, S2, vis, r["g"][b, h]))
            nc = ads.shape[1]
            bq[b, h] = 2.0 ** -8 * scale * (ads @ np.abs(kf[b, h][:nc]))
            bk[b, h][:nc] = 2.0 ** -8 * scale * (ads.T @ np.abs(qf[b, h]))
    return bq, bk


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
@pytest.mark.parametrize("recipe", ["iid", "perturb", "shared_k"])
def test_forward_and_backward(shape, recipe):
    announce(f"parity {shape_id(shape)} {recipe}")
    w, d, r = make(shape, recipe)
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    assert_rows_close(to_np(kl), rk, "KL")
    assert_rows_close(to_np(l1), r1, "LSE1")
    assert_rows_close(to_np(l2), r2, "LSE2")
    for setting in (1, 2):
        if setting == 1:
            dq, dk = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, d["g"],
                                            causal=w.causal)
        else:
            dq, dk = skl.streamkl_bwd_fixP2(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl,
                                            d["g"], causal=w.causal)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        check_grads(w, r, setting, dq, dk, rdq, rdk, max(np.abs(r1).max(), np.abs(r2).max()))


@pytest.mark.parametrize("shape", [SHAPES[5], SHAPES[7]], ids=shape_id)
def test_backward_from_oracle_state(shape):
    """The backward fed with the oracle's own LSE / KL (rounded to fp32), isolating it from
    forward error."""
    announce(f"bwd-from-oracle {shape_id(shape)}")
    w, d, r = make(shape, "perturb")
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    t = [torch.from_numpy(a.astype(np.float32)).cuda() for a in (rk, r1, r2)]
    dq, dk = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], t[1], t[2], d["g"],
                                    causal=w.causal)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    rdq, rdk = oracle.backward(1, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale, w.causal)
    check_grads(w, r, 1, dq, dk, rdq, rdk, lmax)
    dq, dk = skl.streamkl_bwd_fixP2(d["q1"], d["k1"], d["q2"], d["k2"], t[1], t[2], t[0], d["g"],
                                    causal=w.causal)
    rdq, rdk = oracle.backward(2, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale, w.causal)
    check_grads(w, r, 2, dq, dk, rdq, rdk, lmax)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_inputs_give_exact_zeros(causal):
    announce(f"identical causal={causal}")
    w, d, r = make((1, 2, 300, 300, 128, causal))
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q1"], d["k1"], causal=causal)
    assert torch.all(kl == 0) and torch.equal(l1, l2)
    dq, dk = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q1"], d["k1"], l1, l2, d["g"],
                                    causal=causal)
    assert torch.all(dq == 0) and torch.all(dk == 0)
    dq, dk = skl.streamkl_bwd_fixP2(d["q1"], d["k1"], d["q1"], d["k1"], l1, l2, kl, d["g"],
                                    causal=causal)
    assert torch.all(dq == 0) and torch.all(dk == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_rows(causal):
    """Q1 = Q2 = 0: every visible logit is 0, so both distributions are uniform over the row's
    visible keys: LSE = log(n_visible) (n_k, or min(i + 1, n_k) with the causal mask), KL = 0
    and every gradient vanishes. Also Q1 = 0 against a random Q2, against the oracle (the KL of
    a uniform row to P2)."""
    announce(f"zero queries causal={causal}")
    w, d, r = make((1, 2, 300, 257, 64, causal), "perturb")
    z = torch.zeros_like(d["q1"])
    kl, l1, l2 = skl.streamkl_fwd(z, d["k1"], z, d["k2"], causal=causal)
    nvis = np.minimum(np.arange(300) + 1, 257) if causal else np.full(300, 257)
    ref = np.broadcast_to(np.log(nvis.astype(np.float64)), (1, 2, 300))
    assert_rows_close(to_np(l1), ref, "LSE1 of uniform rows")
    assert_rows_close(to_np(l2), ref, "LSE2 of uniform rows")
    assert torch.all(kl == 0)
    for dq, dk in (skl.streamkl_bwd_fixP1(z, d["k1"], z, d["k2"], l1, l2, d["g"], causal=causal),
                   skl.streamkl_bwd_fixP2(z, d["k1"], z, d["k2"], l1, l2, kl, d["g"],
                                          causal=causal)):
        assert torch.all(dq == 0) and torch.all(dk == 0)
    rz = np.zeros_like(r["q1"])
    kl, l1, l2 = skl.streamkl_fwd(z, d["k1"], d["q2"], d["k2"], causal=causal)
    rk, r1, r2 = oracle.forward(rz, r["k1"], r["q2"], r["k2"], w.scale, causal)
    assert_rows_close(to_np(kl), rk, "KL(uniform || P2)")
    assert_rows_close(to_np(l1), r1, "LSE1 (uniform)")
    assert_rows_close(to_np(l2), r2, "LSE2")


def test_forward_is_deterministic():
    announce("determinism")
    w, d, r = make((1, 4, 1000, 1000, 128, True), "perturb")
    a = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=True)
    for _ in range(3):
        b = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=True)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    g1 = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], a[1], a[2], d["g"], causal=True)
    g2 = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], a[1], a[2], d["g"], causal=True)
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])


def test_strided_inputs():
    """[B, N, H, d] storage viewed as [B, H, N, d]: strides (N*H*d, d, H*d)."""
    announce("strided")
    B, H, nq, nk, dd = 2, 3, 200, 150, 64
    w, d, r = make((B, H, nq, nk, dd, True), "perturb")
    sd = {n: d[n].transpose(1, 2).contiguous().transpose(1, 2) for n in ("q1", "k1", "q2", "k2")}
    assert sd["q1"].stride() == (nq * H * dd, dd, H * dd, 1)
    kl, l1, l2 = skl.streamkl_fwd(sd["q1"], sd["k1"], sd["q2"], sd["k2"], causal=True)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, True)
    assert_rows_close(to_np(kl), rk, "KL")
    dq, dk = skl.streamkl_bwd_fixP1(sd["q1"], sd["k1"], sd["q2"], sd["k2"], l1, l2, d["g"],
                                    causal=True)
    rdq, rdk = oracle.backward(1, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale, True)
    check_grads(w, r, 1, dq, dk, rdq, rdk, max(np.abs(r1).max(), np.abs(r2).max()))


def test_invalid_call_raises():
    announce("invalid")
    w, d, r = make((1, 1, 64, 64, 64, False))
    bad = torch.empty((1, 1, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(skl.StreamKLError) as e:
        skl.streamkl_fwd(bad, bad, bad, bad)
    assert e.value.status == 2
    # tensors that are not on the inputs' device are refused by the binding before any call:
    # an output, a row vector or a workspace in host memory would hand the kernels a host address
    q1, k1, q2, k2, g = d["q1"], d["k1"], d["q2"], d["k2"], d["g"]
    kl, l1, l2 = skl.streamkl_fwd(q1, k1, q2, k2)
    host_bf16 = torch.empty(q2.shape, dtype=torch.bfloat16)
    for call in (
            lambda: skl.streamkl_bwd_dq(1, q1, k1, q2, k2, l1, l2, None, g, out=host_bf16),
            lambda: skl.streamkl_bwd_dk(1, q1, k1, q2, k2, l1, l2, None, g, out=host_bf16),
            lambda: skl.streamkl_bwd_dq_splitk(1, q1, k1, q2, k2, l1, l2, None, g,
                                               out=host_bf16),
            lambda: skl.streamkl_bwd_fused(1, q1, k1, q2, k2, l1, l2, None, g,
                                           out=(host_bf16, torch.empty_like(k2))),
            lambda: skl.streamkl_bwd_fixP1(q1, k1, q2, k2, l1, l2, g.cpu()),
            lambda: skl.streamkl_fwd(q1, k1, q2, k2, out=(kl.cpu(), l1, l2)),
            lambda: skl.streamkl_fwd_splitk(q1, k1, q2, k2,
                                            workspace=torch.empty(1 << 20, dtype=torch.uint8)),
            lambda: skl.streamkl_fwd(q1.cpu(), k1, q2, k2)):
        with pytest.raises(ValueError):
            call()


def spiky_inputs(B, H, nq, nk, d, boost, seed):
    """Queries aligned with one direction v and small random keys, except for three keys whose
    logits exceed the rest by about boost * |4 v| (unscaled): each is boost * u (u = v / |v|) plus
    its own component of length 2 boost orthogonal to v, so that the gradient products over
    these keys do not reduce to a cancellation of nearly parallel vectors. The other side is iid."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B, H, 1, d)).astype(np.float32)
    u = v / np.sqrt((v ** 2).sum(-1, keepdims=True))
    q1 = 4 * v + 0.3 * rng.standard_normal((B, H, nq, d)).astype(np.float32)
    k1 = 0.1 * rng.standard_normal((B, H, nk, d)).astype(np.float32)
    for pos, f in ((40, 1.0), (150, 0.99), (nk - 10, 1.01)):
        n = rng.standard_normal((B, H, d)).astype(np.float32)
        n -= (n * u[:, :, 0]).sum(-1, keepdims=True) * u[:, :, 0]
        n /= np.sqrt((n ** 2).sum(-1, keepdims=True))
        k1[:, :, pos] = boost * (f * u[:, :, 0] + 2.0 * n)
    q2 = rng.standard_normal((B, H, nq, d)).astype(np.float32)
    k2 = rng.standard_normal((B, H, nk, d)).astype(np.float32)
    g = rng.uniform(0, 1, (B, H, nq)).astype(np.float32)
    bits = {n: f32_to_bf16_bits(a) for n, a in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2))}
    dev = {n: dev_bf16(b) for n, b in bits.items()}
    ref = {n: f64(b) for n, b in bits.items()}
    dev["g"], ref["g"] = torch.from_numpy(g).cuda(), g.astype(np.float64)
    return dev, ref


@pytest.mark.parametrize("boost", [16.0, 30.0], ids=["wide", "overflow"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_logit_range(boost, causal):
    """Rows whose largest logits lie far above every logit of the first key tile: about 2^90
    (wide) and 2^170 (overflow) in exp2 units relative to the first tile's maximum. Both must
    match the oracle: the second cannot be accumulated against the first tile's maximum in fp32
    and has to take the exact path."""
    announce(f"large logit range boost={boost} causal={causal}")
    B, H, nq, nk, d = 1, 2, (300 if causal else 100), (300 if causal else 333), 64
    d_, r = spiky_inputs(B, H, nq, nk, d, boost, seed=11)
    scale = d ** -0.5
    kl, l1, l2 = skl.streamkl_fwd(d_["q1"], d_["k1"], d_["q2"], d_["k2"], causal=causal)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], scale, causal)
    assert rk.max() > 1.0 and r1.max() > 40.0   # the spikes dominate P1
    assert_rows_close(to_np(kl), rk, "KL")
    assert_rows_close(to_np(l1), r1, "LSE1")
    assert_rows_close(to_np(l2), r2, "LSE2")
    w = Workload("spiky", B, H, nq, nk, d, causal, (1, 2), 11, "iid")
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        if setting == 1:
            dq, dk = skl.streamkl_bwd_fixP1(d_["q1"], d_["k1"], d_["q2"], d_["k2"], l1, l2,
                                            d_["g"], causal=causal)
        else:
            dq, dk = skl.streamkl_bwd_fixP2(d_["q1"], d_["k1"], d_["q2"], d_["k2"], l1, l2, kl,
                                            d_["g"], causal=causal)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], scale,
                                   causal)
        # the spike keys make some dK rows a near-cancellation of large terms (every query lies
        # along v): there the rounding of dS to bf16, not the kernel, sets the error
        check_grads(w, r, setting, dq, dk, rdq, rdk, lmax,
                    extra=bf16_ds_bound(setting, r, scale, causal))


def signed_g(B, H, nq, seed):
    """Upstream gradients of both signs and of very different sizes, laid out so that query tiles
    of 32 rows come in every kind: all positive, one negative row, all zero, all negative, mixed
    with zeros. Magnitudes are log-uniform over [1e-3, 1e3]."""
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-3, 3, (B, H, nq))
    sign = np.where(rng.random((B, H, nq)) < 0.5, -1.0, 1.0)
    g = mag * sign
    kinds = ["pos", "one_neg", "zero", "neg", "mixed"] * (nq // 160 + 1)
    for t0, kind in zip(range(0, nq, 32), kinds):
        blk = slice(t0, min(nq, t0 + 32))
        if kind == "pos":
            g[..., blk] = np.abs(g[..., blk])
        elif kind == "one_neg":
            g[..., blk] = np.abs(g[..., blk])
            g[..., t0 + min(5, nq - 1 - t0)] *= -1
        elif kind == "zero":
            g[..., blk] = 0.0
        elif kind == "neg":
            g[..., blk] = -np.abs(g[..., blk])
        else:
            g[..., t0:min(nq, t0 + 32):7] = 0.0
    g[..., nq - 3:] = 0.0
    return g.astype(np.float32)


@pytest.mark.parametrize("shape", [(1, 2, 300, 257, 128, True), (1, 1, 257, 400, 64, False),
                                   (2, 1, 640, 640, 128, True)], ids=shape_id)
def test_signed_upstream_gradient(shape):
    """Both backward settings with g of both signs, zeros and six decades of magnitude (the dK
    kernel folds log2 |g| into its exponents and applies the sign only on tiles that need it)."""
    announce(f"signed g {shape_id(shape)}")
    w, d, r = make(shape, "perturb")
    g = signed_g(*shape[:3], seed=5)
    d["g"], r["g"] = torch.from_numpy(g).cuda(), g.astype(np.float64)
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        if setting == 1:
            dq, dk = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, d["g"],
                                            causal=w.causal)
        else:
            dq, dk = skl.streamkl_bwd_fixP2(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl,
                                            d["g"], causal=w.causal)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        # rows of opposite sign cancel in dK: the bf16 rounding of dS bounds that error
        check_grads(w, r, setting, dq, dk, rdq, rdk, lmax,
                    extra=bf16_ds_bound(setting, r, w.scale, w.causal))


@pytest.mark.parametrize("shape", [(1, 2, 300, 500, 128, False), (1, 2, 300, 300, 64, True),
                                   (1, 2, 40, 700, 128, False)], ids=shape_id)
def test_nan_input_row_leaves_other_rows_unaffected(shape):
    """Non-finite inputs: the outputs that depend on them are unspecified, the others are not
    affected. A NaN in one element of query row i of q1 (slice 1) may change KL, LSE and the dQ
    row of that query only: every other query row's KL, LSE1, LSE2 and dQ (both settings) still
    match the oracle on the clean inputs, and the other slice's dK too."""
    announce(f"nan row {shape_id(shape)}")
    w, d, r = make(shape, "perturb")
    i = shape[2] // 2
    q1 = d["q1"].clone()
    q1[0, 1, i, 5] = float("nan")
    kl, l1, l2 = skl.streamkl_fwd(q1, d["k1"], d["q2"], d["k2"], causal=w.causal)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    keep = np.ones(shape[:3], dtype=bool)
    keep[0, 1, i] = False
    assert_rows_close(to_np(kl)[keep], rk[keep], "KL (other rows)")
    assert_rows_close(to_np(l1)[keep], r1[keep], "LSE1 (other rows)")
    assert_rows_close(to_np(l2)[keep], r2[keep], "LSE2 (other rows)")
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        if setting == 1:
            dq, dk = skl.streamkl_bwd_fixP1(q1, d["k1"], d["q2"], d["k2"], l1, l2, d["g"],
                                            causal=w.causal)
        else:
            dq, dk = skl.streamkl_bwd_fixP2(q1, d["k1"], d["q2"], d["k2"], l1, l2, kl, d["g"],
                                            causal=w.causal)
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   w.causal)
        qf, kf = (r["q2"], r["k2"]) if setting == 1 else (r["q1"], r["k1"])
        aq = grad_atol(w.scale, r["g"], lmax, kf)
        ak = grad_atol(w.scale, r["g"], lmax, qf, mass=w.n_q / w.n_k)
        assert_grad_close(to_np(dq)[keep], rdq[keep], f"setting {setting} dQ (other rows)", aq)
        # dK of slice 0 (slice 1's dK sums the NaN row and is unspecified)
        assert_grad_close(to_np(dk)[0, 0], rdk[0, 0], f"setting {setting} dK (clean slice)", ak)
