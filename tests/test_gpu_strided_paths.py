"""The few-query-row paths (split-K forward, key-split dQ, fused backward) on strided inputs:
[B, N, H, d] storage viewed as [B, H, N, d] (row stride H*d), against the fp64 oracle."""
import numpy as np
import pytest

import online_attention_kl_amd as skl
import oracle
from parity_util import assert_rows_close, to_np
from test_gpu_parity import check_grads, make

pytestmark = pytest.mark.gpu


def strided(t):
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("nq", [21, 50, 100])
@pytest.mark.parametrize("causal", [False, True])
def test_few_query_paths_on_strided_inputs(causal, nq):
    """21 rows: wavefront split-K items; 50 and 100: key ranges on the LDS-staged forward kernel;
    the fused backward only up to 64 rows."""
    print(f"strided few-query paths causal={causal} nq={nq}", flush=True)
    B, H, nk, dd = 2, 3, 1500, 64
    w, d, r = make((B, H, nq, nk, dd, causal), "perturb")
    sd = {n: strided(d[n]) for n in ("q1", "k1", "q2", "k2")}
    assert sd["q1"].stride() == (nq * H * dd, dd, H * dd, 1)
    rk, r1, r2 = oracle.forward(r["q1"], r["k1"], r["q2"], r["k2"], w.scale, causal)
    kl, l1, l2 = skl.streamkl_fwd_splitk(sd["q1"], sd["k1"], sd["q2"], sd["k2"], causal=causal,
                                         n_splits=5)
    assert_rows_close(to_np(kl), rk, "split-K KL")
    assert_rows_close(to_np(l1), r1, "split-K LSE1")
    assert_rows_close(to_np(l2), r2, "split-K LSE2")
    lmax = max(np.abs(r1).max(), np.abs(r2).max())
    for setting in (1, 2):
        rdq, rdk = oracle.backward(setting, r["q1"], r["k1"], r["q2"], r["k2"], r["g"], w.scale,
                                   causal)
        dq = skl.streamkl_bwd_dq_splitk(setting, sd["q1"], sd["k1"], sd["q2"], sd["k2"], l1, l2,
                                        kl, d["g"], causal=causal, n_splits=4)
        if nq <= 64:
            dq_f, dk_f = skl.streamkl_bwd_fused(setting, sd["q1"], sd["k1"], sd["q2"], sd["k2"],
                                                l1, l2, kl, d["g"], causal=causal)
            check_grads(w, r, setting, dq, dk_f, rdq, rdk, lmax,
                        tag="strided split dQ / fused dK ")
            check_grads(w, r, setting, dq_f, dk_f, rdq, rdk, lmax, tag="strided fused ")
        else:
            dk = skl.streamkl_bwd_dk(setting, sd["q1"], sd["k1"], sd["q2"], sd["k2"], l1, l2, kl,
                                     d["g"], causal=causal)
            check_grads(w, r, setting, dq, dk, rdq, rdk, lmax, tag="strided split dQ / dK ")
