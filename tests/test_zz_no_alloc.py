"""GPU test of the allocation-free forward (streamkl_fwd_noalloc, through the C ABI): it gives
the same bits as streamkl_fwd with a caller workspace, on two calls in a row that both take the
split-K path through the library's scratch, the second with a smaller input (different plan,
fewer ranges and rows), then on a one-pass shape and the split shape again."""
import sys

import pytest
import torch

import online_attention_kl_amd as skl
from test_gpu_parity import make, shape_id

pytestmark = pytest.mark.gpu


def run_both(shape):
    print(f"noalloc {shape_id(shape)}", flush=True)
    sys.stdout.flush()
    w, d, r = make(shape, "perturb")
    ref = skl.streamkl_fwd(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    got = skl.streamkl_fwd_noalloc(d["q1"], d["k1"], d["q2"], d["k2"], causal=w.causal)
    torch.cuda.synchronize()
    for a, b, what in zip(got, ref, ("KL", "LSE1", "LSE2")):
        assert torch.equal(a, b), f"{shape_id(shape)} {what}"
    return w, d


def test_noalloc_matches_streamkl_fwd_on_consecutive_calls():
    cap = skl.lib().streamkl_fwd_noalloc_max_workspace()
    big = (1, 32, 64, 65536, 128, False)     # key ranges on the LDS-staged kernel
    small = (1, 8, 5, 4096, 64, False)       # wavefront work items, fewer ranges and rows
    for shape in (big, small):
        w, d = make(shape, "perturb")[:2]
        need = skl.streamkl_fwd_workspace_size(d["q1"], d["k1"], causal=w.causal)
        assert 0 < need <= cap, (shape, need)
    run_both(big)
    run_both(small)
    # a one-pass shape (no scratch) and the split shape again after it
    one_pass = (2, 40, 900, 900, 64, True)
    w, d = make(one_pass, "perturb")[:2]
    assert skl.streamkl_fwd_workspace_size(d["q1"], d["k1"], causal=True) == 0
    run_both(one_pass)
    run_both(small)
