"""Seeded synthetic inputs for StreamKL, shared by the HIP path's tests/bench and the oracle.

This module holds no part of the method's arithmetic: it only draws random numbers, rounds
them to bfloat16 or fp8 e4m3 bit patterns (round-to-nearest-even) and decodes those bit patterns
back to float32. Both sides (oracle and GPU) read the same bytes produced here.

Workload shapes follow the pages' setting: attention distillation over contexts of 4K-512K
tokens with 32 heads (gist.science/pt "Resultados Experimentais"; 64K x 32 heads in BF16 in
"Definicao do Problema"). The pages evaluate on synthetic context lengths only and name no
dataset, so nothing is stood in for.

Every (tensor, b, h) slice is drawn from its own PCG64 stream keyed by (seed, b, h), so any
single head can be regenerated without generating the whole tensor. Within a slice the draw
order is fixed: Q1, K1, Q2 (or its noise), K2 (or its noise), g.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "slice_inputs", "make_inputs", "visible_pairs", "f32_to_fp8_e4m3_bits",
    "fp8_e4m3_bits_to_f32", "fp8_inputs",
]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n_q: int
    n_k: int
    head_dim: int
    causal: bool
    settings: tuple          # backward settings exercised: 1 = P1 fixed, 2 = P2 fixed
    seed: int
    recipe: str              # "iid" | "perturb" | "shared_k" | "sharp_teacher"
    sigma: float = 0.0       # perturbation std for recipe "perturb"
    teacher_q_std: float = 1.0
    g_mode: str = "one"      # "one" | "uniform"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def shared_k(self) -> bool:
        return self.recipe == "shared_k"

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workload shapes. Seeds 1-4 and the unstated details (K1 of the sharpened-teacher
# workload, g where unstated) are readings listed in the design notes.
WORKLOADS = {
    "tiny_256_d64": Workload("tiny_256_d64", 1, 1, 256, 256, 64, False, (1,), 0, "iid"),
    "nc_4k_d128": Workload("nc_4k_d128", 1, 32, 4096, 4096, 128, False, (1,), 1, "perturb",
                           sigma=0.3, g_mode="uniform"),
    "causal_16k_sharedk_d128": Workload("causal_16k_sharedk_d128", 2, 32, 16384, 16384, 128,
                                        True, (2,), 2, "shared_k"),
    "causal_64k_d128": Workload("causal_64k_d128", 1, 32, 65536, 65536, 128, True, (1,), 3,
                                "perturb", sigma=0.5),
    "asym_2k_32k_d64": Workload("asym_2k_32k_d64", 4, 32, 2048, 32768, 64, False, (1, 2), 4,
                                "sharp_teacher", teacher_q_std=2.0),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def visible_pairs(w: Workload) -> int:
    """Number of visible (query, key) pairs over all slices (top-left causal: key j <= query i)."""
    if not w.causal:
        per = w.n_q * w.n_k
    else:
        n = min(w.n_q, w.n_k)
        per = n * (n + 1) // 2 + max(0, w.n_q - w.n_k) * w.n_k
    return w.batch * w.heads * per


# ---------------------------------------------------------------- bf16 encoding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even. Finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- drawing
def _rng(w: Workload, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=w.seed, spawn_key=(b, h))))


def slice_inputs(w: Workload, b: int, h: int, g_mode: str | None = None) -> dict:
    """Inputs of one (b, h) slice: q1,k1,q2,k2 as bf16 bits [N, d] (uint16) and g float32 [N_Q].

    With a shared-K workload, k2 is the same array object as k1.
    """
    g_mode = w.g_mode if g_mode is None else g_mode
    rng = _rng(w, b, h)
    nq, nk, d = w.n_q, w.n_k, w.head_dim

    def normal(n):
        return rng.standard_normal((n, d), dtype=np.float32)

    if w.recipe == "iid":
        q1 = f32_to_bf16_bits(normal(nq))
        k1 = f32_to_bf16_bits(normal(nk))
        q2 = f32_to_bf16_bits(normal(nq))
        k2 = f32_to_bf16_bits(normal(nk))
    elif w.recipe == "perturb":
        # student = bf16(teacher_bf16 + sigma * N(0,1)), the sum taken in float32
        q1 = f32_to_bf16_bits(normal(nq))
        k1 = f32_to_bf16_bits(normal(nk))
        nzq = normal(nq)
        q2 = f32_to_bf16_bits(bf16_bits_to_f32(q1).reshape(nq, d) + np.float32(w.sigma) * nzq)
        del nzq
        nzk = normal(nk)
        k2 = f32_to_bf16_bits(bf16_bits_to_f32(k1).reshape(nk, d) + np.float32(w.sigma) * nzk)
        del nzk
    elif w.recipe == "shared_k":
        q1 = f32_to_bf16_bits(normal(nq))
        k1 = f32_to_bf16_bits(normal(nk))
        q2 = f32_to_bf16_bits(normal(nq))
        k2 = k1
    elif w.recipe == "sharp_teacher":
        q1 = f32_to_bf16_bits(np.float32(w.teacher_q_std) * normal(nq))
        k1 = f32_to_bf16_bits(normal(nk))
        q2 = f32_to_bf16_bits(normal(nq))
        k2 = f32_to_bf16_bits(normal(nk))
    else:
        raise ValueError(f"unknown recipe {w.recipe!r}")

    if g_mode == "one":
        g = np.ones(nq, dtype=np.float32)
    elif g_mode == "uniform":
        g = rng.random(nq, dtype=np.float32)
    else:
        raise ValueError(f"unknown g_mode {g_mode!r}")
    k1v = k1.reshape(nk, d)
    k2v = k1v if k2 is k1 else k2.reshape(nk, d)
    return {"q1": q1.reshape(nq, d), "k1": k1v, "q2": q2.reshape(nq, d), "k2": k2v, "g": g}


def make_inputs(w: Workload, g_mode: str | None = None, threads: int | None = None) -> dict:
    """All slices: q1,q2 uint16 [B,H,N_Q,d], k1,k2 uint16 [B,H,N_K,d], g float32 [B,H,N_Q].

    Slices are drawn in parallel threads (numpy's generators release the GIL); the result does
    not depend on the thread count. With a shared-K workload, k2 is k1 (same object).
    """
    B, H = w.batch, w.heads
    q1 = np.empty((B, H, w.n_q, w.head_dim), np.uint16)
    q2 = np.empty_like(q1)
    k1 = np.empty((B, H, w.n_k, w.head_dim), np.uint16)
    k2 = k1 if w.shared_k else np.empty_like(k1)
    g = np.empty((B, H, w.n_q), np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        s = slice_inputs(w, b, h, g_mode)
        q1[b, h], k1[b, h], q2[b, h], g[b, h] = s["q1"], s["k1"], s["q2"], s["g"]
        if not w.shared_k:
            k2[b, h] = s["k2"]

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or B * H == 1:
        for bh in range(B * H):
            fill(bh)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(B * H)))
    return {"q1": q1, "k1": k1, "q2": q2, "k2": k2, "g": g}


# ---------------------------------------------------------------- fp8 e4m3 (OCP, "fn" variant)
# 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; subnormals below 2^-6 in steps of 2^-9;
# no infinities; the largest finite value is 448 = 1.75 * 2^8.
FP8_E4M3_MAX = 448.0


def f32_to_fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest e4m3 code (ties to even). Values that would round
    past 448 are rejected (no saturation, no NaN codes are produced)."""
    x = np.asarray(x, np.float32)
    a = np.abs(x).astype(np.float64)
    if np.any(~np.isfinite(a)) or np.any(a >= 464.0):  # 464 = halfway from 448 to 512
        raise ValueError("value outside the e4m3 range")
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -9)))
    e = np.clip(e, -6, 8)                   # binade; -6 also covers the subnormals
    quantum = np.exp2(e - 3)                # spacing of the 8 mantissa steps in that binade
    m = np.rint(a / quantum) * quantum      # round half to even
    # re-encode (a carry into the next binade stays exact)
    e2 = np.floor(np.log2(np.maximum(m, 2.0 ** -9)))
    normal = m >= 2.0 ** -6
    exp_field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, m / np.exp2(e2) - 1.0, m / 2.0 ** -9) * np.where(normal, 8.0, 1.0)
    mant = np.where(m == 0, 0, mant)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def fp8_e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode e4m3 codes to float32 (exact); NaN codes (0x7f, 0xff) decode to NaN."""
    b = np.asarray(b, np.uint8).astype(np.int64)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((b & 0x7F) == 0x7F, np.nan, v)
    return np.where(b & 0x80, -v, v).astype(np.float32)


def fp8_inputs(w: Workload, gain: tuple = (4.0, 4.0, 2.0, 2.0), threads: int | None = None) -> dict:
    """The workload's bf16 inputs (same seed and draws) multiplied by per-tensor power-of-two
    gains and rounded to e4m3 codes: q1, k1, q2, k2 as uint8 arrays plus g. Side t's
    dequantisation factor is 1 / (gain_q gain_k), returned as "descale1", "descale2"."""
    x = make_inputs(w, threads=threads)
    out = {"g": x["g"]}
    names = ("q1", "k1", "q2", "k2")
    for n, gn in zip(names, gain):
        if n == "k2" and x["k2"] is x["k1"] and gain[3] == gain[1]:
            out["k2"] = out["k1"]
            continue
        f = bf16_bits_to_f32(x[n]).reshape(x[n].shape)
        out[n] = f32_to_fp8_e4m3_bits(f * np.float32(gn))
    out["descale1"] = 1.0 / (gain[0] * gain[1])
    out["descale2"] = 1.0 / (gain[2] * gain[3])
    return out
