"""The seeded input generator: bf16 rounding, determinism, slice independence, shapes."""
import numpy as np
import pytest
import torch

from workloads import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, slice_inputs,
                       visible_pairs)


def test_bf16_rne_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), want)
    back = bf16_bits_to_f32(want)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_deterministic_and_independent():
    w = WORKLOADS["tiny_256_d64"].with_(batch=2, heads=3)
    a = make_inputs(w, threads=4)
    b = make_inputs(w, threads=1)
    for k in ("q1", "k1", "q2", "k2", "g"):
        np.testing.assert_array_equal(a[k], b[k])
    s = slice_inputs(w, 1, 2)
    np.testing.assert_array_equal(s["q2"], a["q2"][1, 2])
    assert not np.array_equal(a["q1"][0, 0], a["q1"][0, 1])


def test_recipes():
    w = WORKLOADS["causal_16k_sharedk_d128"].with_(n_q=64, n_k=64, batch=1, heads=1)
    s = slice_inputs(w, 0, 0)
    assert s["k2"] is s["k1"]
    w = WORKLOADS["nc_4k_d128"].with_(n_q=512, n_k=512, heads=1)
    s = slice_inputs(w, 0, 0)
    diff = bf16_bits_to_f32(s["q2"]) - bf16_bits_to_f32(s["q1"])
    assert abs(diff.std() - 0.3) < 0.01
    assert 0 <= s["g"].min() and s["g"].max() < 1
    w = WORKLOADS["asym_2k_32k_d64"].with_(n_q=256, n_k=256, batch=1, heads=1)
    s = slice_inputs(w, 0, 0)
    assert abs(bf16_bits_to_f32(s["q1"]).std() - 2.0) < 0.05


def test_visible_pairs():
    assert visible_pairs(WORKLOADS["causal_64k_d128"]) == 32 * 65536 * 65537 // 2
    assert visible_pairs(WORKLOADS["asym_2k_32k_d64"]) == 4 * 32 * 2048 * 32768
    w = WORKLOADS["tiny_256_d64"].with_(n_q=5, n_k=3, causal=True)
    assert visible_pairs(w) == 1 + 2 + 3 + 3 + 3


def test_fp8_e4m3_codes_match_torch():
    """The generator's e4m3 rounding (ties to even) and decoding agree with PyTorch's own
    float8_e4m3fn conversion on random values, every representable value and every midpoint."""
    import torch
    from workloads import f32_to_fp8_e4m3_bits, fp8_e4m3_bits_to_f32
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s
                        for s in (1e-3, 0.1, 1.0, 10.0, 100.0)])
    x = x[np.abs(x) < 448]
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8_e4m3_bits_to_f32(codes)
    pos = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, pos, -pos, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_fp8_e4m3_bits(x), ref)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.all((vals == dec) | (np.isnan(vals) & np.isnan(dec)))
    with pytest.raises(ValueError):
        f32_to_fp8_e4m3_bits(np.array([470.0], np.float32))
