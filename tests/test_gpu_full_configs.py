"""GPU parity at the full workload sizes, in the launch configuration bench.py times (the C ABI
entry points on the full tensors), checked on sampled outputs the oracle computes one by one:

- KL, LSE1, LSE2 of sampled query rows (first, last, spread, ragged) of sampled slices;
- dQ rows of those query rows (each needs only its own row of logits);
- dK rows of sampled keys: non-causal, any key (the oracle forms all rows' LSE of that slice);
  causal, keys in the last 256 positions (seen only by the last rows, whose LSE is cheap);
- everywhere: the column sums of dK vanish (every row of dS sums to zero), checked against the
  size of the gradient.
"""
import sys

import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
from oracle.reference import backward_slice, dk_rows_slice, forward_slice
from parity_util import assert_grad_close, assert_rows_close, dev_bf16, f64, grad_atol
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sampled_rows(n, rng, k=24):
    base = {0, 1, n - 1, n - 2, n // 2}
    base |= set(rng.integers(0, n, size=k).tolist())
    return np.array(sorted(x for x in base if 0 <= x < n))


@pytest.mark.parametrize("name", ["nc_4k_d128", "causal_16k_sharedk_d128", "causal_64k_d128",
                                  "asym_2k_32k_d64"])
def test_full_size(name):
    w = WORKLOADS[name]
    announce(f"[full] {name}: generating inputs")
    x = make_inputs(w)
    d = {n: dev_bf16(x[n]) for n in ("q1", "k1", "q2")}
    d["k2"] = d["k1"] if x["k2"] is x["k1"] else dev_bf16(x["k2"])
    g = torch.from_numpy(x["g"]).cuda()
    announce(f"[full] {name}: GPU forward + backward {w.settings}")
    kl, l1, l2 = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    grads = {}
    for s in w.settings:
        if s == 1:
            grads[s] = skl.streamkl_bwd_fixP1(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, g,
                                              causal=w.causal)
        else:
            grads[s] = skl.streamkl_bwd_fixP2(d["q1"], d["k1"], d["q2"], d["k2"], l1, l2, kl, g,
                                              causal=w.causal)
    torch.cuda.synchronize()
    kl_h, l1_h, l2_h = (t.cpu().numpy().astype(np.float64) for t in (kl, l1, l2))

    rng = np.random.default_rng(7)
    B, H = w.batch, w.heads
    slices = sorted({(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))})
    for (b, h) in slices:
        announce(f"[full] {name}: oracle samples of slice ({b}, {h})")
        a = {n: f64(x[n][b, h]) for n in ("q1", "k1", "q2", "k2")}
        gs = x["g"][b, h].astype(np.float64)
        rows = sampled_rows(w.n_q, rng)
        rk, r1, r2 = forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], w.scale, w.causal, rows=rows)
        assert_rows_close(kl_h[b, h, rows], rk, f"{name} KL")
        assert_rows_close(l1_h[b, h, rows], r1, f"{name} LSE1")
        assert_rows_close(l2_h[b, h, rows], r2, f"{name} LSE2")
        lse_max = max(np.abs(r1).max(), np.abs(r2).max())
        # keys whose dK the oracle can form here, and the query rows that see them
        if w.causal:
            keys = np.arange(w.n_k - 256, w.n_k)[::17]
            frows = np.arange(int(keys.min()), w.n_q)
        else:
            keys = sampled_rows(w.n_k, rng, k=6)
            frows = np.arange(w.n_q)
        ffwd = forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], w.scale, w.causal, rows=frows)
        for s in w.settings:
            dq, dk = (t[b, h].float().cpu().numpy().astype(np.float64) for t in grads[s])
            qf, kf = (a["q2"], a["k2"]) if s == 1 else (a["q1"], a["k1"])
            rdq, _ = backward_slice(s, a["q1"], a["k1"], a["q2"], a["k2"], gs, w.scale, w.causal,
                                    rows=rows, want_dk=False)
            aq = grad_atol(w.scale, gs, lse_max, kf)
            assert_grad_close(dq[rows], rdq, f"{name} setting {s} dQ rows", aq)
            rdk = dk_rows_slice(s, a["q1"], a["k1"], a["q2"], a["k2"], gs, w.scale, w.causal,
                                keys, fwd=ffwd, rows=frows)
            ak = grad_atol(w.scale, gs, lse_max, qf, mass=w.n_q / w.n_k)
            assert_grad_close(dk[keys], rdk, f"{name} setting {s} dK rows", ak)
            # column sums of dK vanish: each row of dS sums to zero
            colsum = np.abs(dk.sum(0)).max()
            scale = np.abs(dk).sum(0).max()
            assert colsum <= 2e-2 * scale + 1e-6, f"{name} setting {s}: dK column sum {colsum}"

