"""GPU parity of the fp8 e4m3 forward against the fp64 oracle on the dequantised inputs (the
codes decoded exactly and divided by their power-of-two gains)."""
import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
import oracle
from parity_util import assert_rows_close, oracle_forward_rows, to_np
from workloads import WORKLOADS, Workload, fp8_e4m3_bits_to_f32, fp8_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 1, 1, 1, 128, False),
    (1, 2, 17, 33, 64, False),
    (1, 1, 64, 64, 128, True),
    (2, 1, 65, 65, 64, True),
    (1, 1, 255, 257, 128, False),
    (1, 2, 257, 255, 128, True),
    (1, 1, 1000, 1000, 64, True),
    (1, 3, 384, 384, 128, False),
]
GAIN = (4.0, 4.0, 2.0, 2.0)


def shape_id(s):
    return "B{}H{}_q{}_k{}_d{}_{}".format(*s[:5], "causal" if s[5] else "full")


def dev_fp8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).cuda()


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
@pytest.mark.parametrize("recipe", ["iid", "perturb", "shared_k"])
def test_fp8_forward(shape, recipe):
    print(f"fp8 {shape_id(shape)} {recipe}", flush=True)
    B, H, nq, nk, d, causal = shape
    w = Workload("fp8", B, H, nq, nk, d, causal, (1,), 99, recipe, sigma=0.3)
    gain = (GAIN[0], GAIN[1], GAIN[2], GAIN[1] if recipe == "shared_k" else GAIN[3])
    x = fp8_inputs(w, gain)
    dv = {n: dev_fp8(x[n]) for n in ("q1", "k1", "q2")}
    dv["k2"] = dv["k1"] if x["k2"] is x["k1"] else dev_fp8(x["k2"])
    ref = {n: fp8_e4m3_bits_to_f32(x[n]).astype(np.float64) / gn
           for n, gn in zip(("q1", "k1", "q2", "k2"), gain)}
    kl, l1, l2 = skl.streamkl_fwd_fp8(dv["q1"], dv["k1"], dv["q2"], dv["k2"], x["descale1"],
                                      x["descale2"], causal=causal)
    rk, r1, r2 = oracle.forward(ref["q1"], ref["k1"], ref["q2"], ref["k2"], w.scale, causal)
    assert_rows_close(to_np(kl), rk, "KL")
    assert_rows_close(to_np(l1), r1, "LSE1")
    assert_rows_close(to_np(l2), r2, "LSE2")


def test_fp8_identical_sides_give_zero():
    w = Workload("fp8", 1, 2, 300, 300, 128, True, (1,), 5, "iid")
    x = fp8_inputs(w)
    q, k = dev_fp8(x["q1"]), dev_fp8(x["k1"])
    kl, l1, l2 = skl.streamkl_fwd_fp8(q, k, q, k, 0.25, 0.25, causal=True)
    assert torch.all(kl == 0) and torch.equal(l1, l2)


def test_fp8_rejects_bad_descale_and_stride():
    w = Workload("fp8", 1, 1, 64, 64, 64, False, (1,), 5, "iid")
    x = fp8_inputs(w)
    q, k = dev_fp8(x["q1"]), dev_fp8(x["k1"])
    with pytest.raises(skl.StreamKLError):
        skl.streamkl_fwd_fp8(q, k, q, k, 0.0, 1.0)
    with pytest.raises(skl.StreamKLError):
        skl.streamkl_fwd_fp8(q, k, q, k, float("inf"), 1.0)


@pytest.mark.parametrize("name", ["nc_4k_d128", "causal_64k_d128"])
def test_fp8_full_size(name):
    """The fp8 forward on a whole workload (its inputs scaled by the gains and rounded to e4m3,
    as bench.py --fp8 times it): every row of slice (0, 0) and sampled rows of two more slices
    against the oracle on the exactly decoded inputs."""
    w = WORKLOADS[name]
    print(f"fp8 full size {name}: generating inputs", flush=True)
    x = fp8_inputs(w, GAIN)
    dv = {n: dev_fp8(x[n]) for n in ("q1", "k1", "q2")}
    dv["k2"] = dv["k1"] if x["k2"] is x["k1"] else dev_fp8(x["k2"])
    kl, l1, l2 = skl.streamkl_fwd_fp8(dv["q1"], dv["k1"], dv["q2"], dv["k2"], x["descale1"],
                                      x["descale2"], causal=w.causal)
    kl_h, l1_h, l2_h = to_np(kl), to_np(l1), to_np(l2)
    rng = np.random.default_rng(11)
    B, H = w.batch, w.heads
    slices = [(0, 0)] + sorted({(B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))}
                               - {(0, 0)})
    for b, h in slices:
        print(f"fp8 full size {name}: oracle on slice ({b}, {h})", flush=True)
        a = {n: fp8_e4m3_bits_to_f32(x[n][b, h]).astype(np.float64) / gn
             for n, gn in zip(("q1", "k1", "q2", "k2"), GAIN)}
        if (b, h) == (0, 0):
            rows = np.arange(w.n_q)
        else:
            rows = np.unique(np.concatenate([[0, 1, w.n_q // 2, w.n_q - 2, w.n_q - 1],
                                             rng.integers(0, w.n_q, 24)]))
        rk, r1, r2 = oracle_forward_rows(a, w.scale, w.causal, rows)
        assert_rows_close(kl_h[b, h, rows], rk, f"{name} fp8 KL ({b}, {h})")
        assert_rows_close(l1_h[b, h, rows], r1, f"{name} fp8 LSE1 ({b}, {h})")
        assert_rows_close(l2_h[b, h, rows], r2, f"{name} fp8 LSE2 ({b}, {h})")
