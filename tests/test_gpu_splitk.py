"""GPU parity of the split-K forward (few query rows, keys cut into ranges whose partial online
states are merged) against the fp64 oracle and against the one-pass forward."""
import sys

import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
import oracle
from parity_util import assert_rows_close, dev_bf16, f64, to_np
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

# (batch, heads, n_q, n_k, head_dim, causal)
SHAPES = [
    (1, 4, 1, 4096, 128, False),
    (2, 3, 7, 5000, 64, False),
    (1, 2, 40, 3000, 128, True),
    (1, 1, 33, 1, 64, False),
    (1, 2, 100, 257, 128, False),
    (1, 1, 70, 70, 64, True),
    (1, 32, 16, 65536, 128, False),
    (1, 2, 32, 3000, 128, True),
    # more than 32 query rows: ranges run as blocks of the LDS-staged forward kernel
    (1, 2, 300, 1000, 128, True),
    (2, 2, 513, 777, 64, False),
    (1, 3, 65, 2000, 128, False),
    (1, 1, 700, 300, 64, True),
]


def shape_id(s):
    return "B{}H{}_q{}_k{}_d{}_{}".format(*s[:5], "causal" if s[5] else "full")


def make(shape, recipe, seed=321):
    B, H, nq, nk, d, causal = shape
    w = Workload("splitk", B, H, nq, nk, d, causal, (1,), seed, recipe, sigma=0.3)
    x = make_inputs(w)
    dev = {n: dev_bf16(x[n]) for n in ("q1", "k1", "q2")}
    dev["k2"] = dev["k1"] if x["k2"] is x["k1"] else dev_bf16(x["k2"])
    ref = {n: f64(x[n]) for n in ("q1", "k1", "q2", "k2")}
    return w, dev, ref


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
@pytest.mark.parametrize("recipe", ["iid", "perturb", "shared_k"])
def test_splitk_matches_oracle(shape, recipe):
    print(f"splitk {shape_id(shape)} {recipe}", flush=True)
    w, d, r = make(shape, recipe)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, w.causal)
    base = skl.streamkl_fwd_one_pass(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    for n_splits in (0, 1, 3, 64, 65, 1000):
        kl, l1, l2 = skl.streamkl_fwd_splitk(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal,
                                             n_splits=n_splits)
        tag = f"n_splits={n_splits} "
        assert_rows_close(to_np(kl), rk, tag + "KL")
        assert_rows_close(to_np(l1), r1, tag + "LSE1")
        assert_rows_close(to_np(l2), r2, tag + "LSE2")
        # and the one-pass forward (same float32 arithmetic, other summation order)
        for a, b, what in zip((kl, l1, l2), base, ("KL", "LSE1", "LSE2")):
            assert_rows_close(to_np(a), to_np(b), tag + what + " vs one-pass")


@pytest.mark.parametrize("nq", [9, 100])
def test_splitk_deterministic_and_ignores_workspace_contents(nq):
    print(f"splitk determinism nq={nq}", flush=True)
    w, d, r = make((1, 4, nq, 3000, 128, False), "perturb")
    nbytes = skl.streamkl_fwd_splitk_workspace_size(d["q1"], d["k1"], n_splits=5)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    a = skl.streamkl_fwd_splitk(d["q1"], d["k1"], d["q2"], d["k2"], n_splits=5,
                                workspace=ws.view(torch.uint8))
    for _ in range(2):
        ws.fill_(float("inf"))
        b = skl.streamkl_fwd_splitk(d["q1"], d["k1"], d["q2"], d["k2"], n_splits=5,
                                    workspace=ws.view(torch.uint8))
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_splitk_identical_inputs_give_zero():
    print("splitk identical", flush=True)
    w, d, r = make((1, 2, 5, 2000, 64, False), "iid")
    kl, l1, l2 = skl.streamkl_fwd_splitk(d["q1"], d["k1"], d["q1"], d["k1"], n_splits=7)
    assert torch.all(kl == 0) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_splitk_large_logit_range(causal):
    """Spiky keys far above every logit of a range's first tile: ranges that overflow against
    that maximum must be recomputed exactly."""
    from test_gpu_parity import spiky_inputs
    print(f"splitk large logit range causal={causal}", flush=True)
    B, H, nq, nk, d = 1, 2, (300 if causal else 100), (300 if causal else 333), 64
    dv, r = spiky_inputs(B, H, nq, nk, d, 30.0, seed=11)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], d ** -0.5, causal)
    for n_splits in (1, 3):
        kl, l1, l2 = skl.streamkl_fwd_splitk(dv["q1"], dv["k1"], dv["q2"], dv["k2"],
                                             causal=causal, n_splits=n_splits)
        assert_rows_close(to_np(kl), rk, f"n_splits={n_splits} KL")
        assert_rows_close(to_np(l1), r1, f"n_splits={n_splits} LSE1")
        assert_rows_close(to_np(l2), r2, f"n_splits={n_splits} LSE2")


def test_splitk_too_small_workspace_raises():
    w, d, r = make((1, 1, 4, 640, 64, False), "iid")
    nbytes = skl.streamkl_fwd_splitk_workspace_size(d["q1"], d["k1"], n_splits=4)
    ws = torch.empty(nbytes - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(skl.StreamKLError) as e:
        skl.streamkl_fwd_splitk(d["q1"], d["k1"], d["q2"], d["k2"], n_splits=4, workspace=ws)
    assert e.value.status == 1


def test_splitk_blocks_at_64k_keys():
    """The key-range blocks at the small-N bench shape (32 heads, 512 query rows, 64K keys):
    every row against the one-pass forward, sampled rows of sampled slices against the oracle."""
    from oracle.reference import forward_slice
    print("splitk blocks 32x512x65536", flush=True)
    B, H, nq, nk, d = 1, 32, 512, 65536, 128
    w = Workload("splitk_64k", B, H, nq, nk, d, False, (1,), 9, "perturb", sigma=0.5)
    x = make_inputs(w)
    dv = {n: dev_bf16(x[n]) for n in ("q1", "k1", "q2", "k2")}
    assert skl.streamkl_fwd_splitk_default_splits(dv["q1"], dv["k1"]) > 1
    kl, l1, l2 = skl.streamkl_fwd_splitk(dv["q1"], dv["k1"], dv["q2"], dv["k2"])
    base = skl.streamkl_fwd_one_pass(dv["q1"], dv["k1"], dv["q2"], dv["k2"])
    for a, b, what in zip((kl, l1, l2), base, ("KL", "LSE1", "LSE2")):
        assert_rows_close(to_np(a), to_np(b), what + " vs one-pass")
    rng = np.random.default_rng(3)
    rows = np.array(sorted({0, 255, 256, nq - 1} | set(rng.integers(0, nq, 12).tolist())))
    for h in (0, 17, H - 1):
        a = {n: f64(x[n][0, h]) for n in ("q1", "k1", "q2", "k2")}
        rk, r1, r2 = forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], w.scale, False, rows=rows)
        assert_rows_close(to_np(kl)[0, h, rows], rk, f"head {h} KL")
        assert_rows_close(to_np(l1)[0, h, rows], r1, f"head {h} LSE1")
        assert_rows_close(to_np(l2)[0, h, rows], r2, f"head {h} LSE2")
