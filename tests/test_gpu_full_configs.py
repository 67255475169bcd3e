"""GPU parity at the full workload sizes, in the launch configuration bench.py times (the C ABI
entry points on the full tensors), against the fp64 oracle:

- one whole slice, (0, 0), element by element: KL, LSE1, LSE2 of every query row, dQ of every
  query row and dK of every key (key 0 of the 64K causal slice sums all 65,536 rows). The oracle
  runs over row blocks in a thread pool (the rows of a block are independent for KL, LSE and dQ;
  the dK contributions of the blocks are added up);
- sampled query rows (first, last, spread, ragged) of two more slices: KL, LSE1, LSE2 and dQ;
- every slice: the column sums of dK vanish (every row of dS sums to zero), against the size of
  the gradient.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import online_attention_kl_amd as skl
from oracle.reference import backward_slice, forward_slice
from parity_util import (assert_grad_close, assert_rows_close, dev_bf16, f64, grad_atol,
                         row_chunks)
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sampled_rows(n, rng, k=24):
    base = {0, 1, n - 1, n - 2, n // 2}
    base |= set(rng.integers(0, n, size=k).tolist())
    return np.array(sorted(x for x in base if 0 <= x < n))


def oracle_whole_slice(a, g, scale, causal, settings):
    """KL, LSE1, LSE2 of every row and (dQ, dK) of each setting for one slice, from the oracle's
    functions over row blocks in a thread pool (BLAS one thread per worker)."""
    n_q, d = a["q1"].shape
    n_k = a["k1"].shape[0]
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = row_chunks(n_q, n_k, causal, 8 * workers)
    fwd = np.empty((3, n_q))
    dq = {s: np.empty((n_q, d)) for s in settings}
    dk = {s: np.zeros((n_k, d)) for s in settings}

    def run(rows):
        f = forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], scale, causal, rows=rows)
        b = {s: backward_slice(s, a["q1"], a["k1"], a["q2"], a["k2"], g, scale, causal, rows=rows)
             for s in settings}
        return rows, f, b

    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)
    except Exception:  # pragma: no cover
        ctx = None
    try:
        with ThreadPoolExecutor(workers) as ex:
            for rows, f, b in ex.map(run, chunks):
                fwd[:, rows] = np.stack(f)
                for s in settings:
                    dq[s][rows] = b[s][0]
                    dk[s] += b[s][1]
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    return fwd, dq, dk


# each workload with the backward settings it names, and two more: setting 2 at the 64K causal
# size and setting 1 on the shared-key workload
CASES = [(n, None) for n in ("tiny_256_d64", "nc_4k_d128", "causal_16k_sharedk_d128",
                             "causal_64k_d128", "asym_2k_32k_d64")]
CASES += [("causal_64k_d128", (2,)), ("causal_16k_sharedk_d128", (1,))]


@pytest.mark.parametrize("name,settings", CASES,
                         ids=[n + ("" if st is None else f"_setting{st[0]}") for n, st in CASES])
def test_full_size(name, settings):
    w = WORKLOADS[name]
    if settings is not None:
        import dataclasses
        w = dataclasses.replace(w, settings=settings)
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
    gr_h = {s: tuple(t.float().cpu().numpy().astype(np.float64) for t in grads[s])
            for s in w.settings}

    # every slice: the column sums of dK vanish
    for s in w.settings:
        dk = gr_h[s][1]
        colsum = np.abs(dk.sum(2)).max(axis=-1)
        size = np.abs(dk).sum(2).max(axis=-1)
        assert (colsum <= 2e-2 * size + 1e-6).all(), f"{name} setting {s}: dK column sums"

    # slice (0, 0): every output against the oracle
    announce(f"[full] {name}: oracle over the whole slice (0, 0)")
    a = {n: f64(x[n][0, 0]) for n in ("q1", "k1", "q2", "k2")}
    gs = x["g"][0, 0].astype(np.float64)
    (rk, r1, r2), rdq, rdk = oracle_whole_slice(a, gs, w.scale, w.causal, w.settings)
    assert_rows_close(kl_h[0, 0], rk, f"{name} KL")
    assert_rows_close(l1_h[0, 0], r1, f"{name} LSE1")
    assert_rows_close(l2_h[0, 0], r2, f"{name} LSE2")
    lse_max = max(np.abs(r1).max(), np.abs(r2).max())
    for s in w.settings:
        qf, kf = (a["q2"], a["k2"]) if s == 1 else (a["q1"], a["k1"])
        aq = grad_atol(w.scale, gs, lse_max, kf)
        ak = grad_atol(w.scale, gs, lse_max, qf, mass=w.n_q / w.n_k)
        assert_grad_close(gr_h[s][0][0, 0], rdq[s], f"{name} setting {s} dQ (all rows)", aq)
        assert_grad_close(gr_h[s][1][0, 0], rdk[s], f"{name} setting {s} dK (all keys)", ak)

    # sampled rows of two more slices
    rng = np.random.default_rng(7)
    B, H = w.batch, w.heads
    slices = sorted({(B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))} - {(0, 0)})
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
        for s in w.settings:
            kf = a["k2"] if s == 1 else a["k1"]
            rdq, _ = backward_slice(s, a["q1"], a["k1"], a["q2"], a["k2"], gs, w.scale, w.causal,
                                    rows=rows, want_dk=False)
            aq = grad_atol(w.scale, gs, lse_max, kf)
            assert_grad_close(gr_h[s][0][b, h, rows], rdq, f"{name} setting {s} dQ rows", aq)
