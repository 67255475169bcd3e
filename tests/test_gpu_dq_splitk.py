"""GPU parity of the key-range split dQ (few query rows): against the fp64 oracle and against
the one-kernel dQ."""
import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
import oracle
from parity_util import assert_grad_close, dev_bf16, f64, grad_atol, to_np
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 4, 1, 4096, 128, False),
    (2, 3, 7, 5000, 64, False),
    (1, 2, 40, 3000, 128, True),
    (1, 2, 100, 257, 128, False),
    (1, 1, 300, 2000, 64, True),
    (1, 2, 600, 1200, 128, False),
    (1, 32, 16, 16384, 128, False),
]


def shape_id(s):
    return "B{}H{}_q{}_k{}_d{}_{}".format(*s[:5], "causal" if s[5] else "full")


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
@pytest.mark.parametrize("recipe", ["perturb", "shared_k"])
def test_dq_splitk(shape, recipe):
    print(f"dq splitk {shape_id(shape)} {recipe}", flush=True)
    B, H, nq, nk, d, causal = shape
    w = Workload("dqsplit", B, H, nq, nk, d, causal, (1, 2), 77, recipe, sigma=0.3,
                 g_mode="uniform")
    x = make_inputs(w)
    dv = {n: dev_bf16(x[n]) for n in ("q1", "k1", "q2")}
    dv["k2"] = dv["k1"] if x["k2"] is x["k1"] else dev_bf16(x["k2"])
    g = torch.from_numpy(x["g"]).cuda()
    r = {n: f64(x[n]) for n in ("q1", "k1", "q2", "k2")}
    kl, l1, l2 = skl.streamkl_fwd(dv["q1"], dv["k1"], dv["q2"], dv["k2"], causal=causal)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, causal)
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        kf = r["k2"] if setting == 1 else r["k1"]
        rdq = np.stack([np.stack([oracle.reference.backward_slice(
            setting, r["q1"][b, h], r["k1"][b, h], r["q2"][b, h], r["k2"][b, h],
            x["g"][b, h].astype(np.float64), w.scale, causal, want_dk=False)[0]
            for h in range(H)]) for b in range(B)])
        one = skl.streamkl_bwd_dq(setting, dv["q1"], dv["k1"], dv["q2"], dv["k2"], l1, l2, kl, g,
                                  causal=causal)
        aq = grad_atol(w.scale, x["g"], lmax, kf)
        for n_splits in (0, 2, 5, 1000):
            dq = skl.streamkl_bwd_dq_splitk(setting, dv["q1"], dv["k1"], dv["q2"], dv["k2"], l1,
                                            l2, kl, g, causal=causal, n_splits=n_splits)
            assert_grad_close(to_np(dq), rdq, f"setting {setting} n_splits={n_splits} dQ", aq)
            # the one-kernel dQ: same float32 terms summed in another order, rounded once;
            # at most a couple of bf16 steps apart
            a, b = to_np(dq), to_np(one)
            assert np.all(np.abs(a - b) <= 2 ** -6 * np.abs(b) + 4 * aq + 1e-30), \
                f"setting {setting} n_splits={n_splits}: split vs one-kernel dQ"


def test_dq_splitk_deterministic():
    B, H, nq, nk, d = 1, 2, 50, 3000, 128
    w = Workload("dqsplit", B, H, nq, nk, d, False, (1,), 5, "perturb", sigma=0.3)
    x = make_inputs(w)
    dv = {n: dev_bf16(x[n]) for n in ("q1", "k1", "q2", "k2")}
    g = torch.from_numpy(x["g"]).cuda()
    kl, l1, l2 = skl.streamkl_fwd(dv["q1"], dv["k1"], dv["q2"], dv["k2"])
    nbytes = skl.streamkl_bwd_dq_splitk_workspace_size(dv["q1"], dv["k1"], n_splits=6)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    a = skl.streamkl_bwd_dq_splitk(1, dv["q1"], dv["k1"], dv["q2"], dv["k2"], l1, l2, kl, g,
                                   n_splits=6, workspace=ws.view(torch.uint8))
    ws.fill_(float("inf"))
    b = skl.streamkl_bwd_dq_splitk(1, dv["q1"], dv["k1"], dv["q2"], dv["k2"], l1, l2, kl, g,
                                   n_splits=6, workspace=ws.view(torch.uint8))
    assert torch.equal(a, b)
