"""Helpers shared by the GPU parity tests: moving the generator's bf16 bits to the device and the
tolerance checks.

Tolerances: per-row KL and LSE must satisfy |gpu - ref| <= 1e-4 + 1e-3 |ref| elementwise.
Gradients (bf16 outputs) must satisfy, elementwise, |gpu - ref| <= 2e-2 (|ref| + rms_row(ref)) +
atol and, normwise, ||gpu - ref|| <= 2e-2 ||ref|| + atol sqrt(n). Pure elementwise relative
error is meaningless near the zeros of a gradient, so each element is measured against the rms
of its own output row (the head_dim vector dQ[i] or dK[j]): the GEMM operand dS is rounded to
bf16, and that rounding error scales with the row's own dS magnitude, which varies by orders of
magnitude between rows (a causal row with few visible keys has a large, peaked dS). A CPU
emulation of bf16-rounded dS against the exact gradient uses at most ~0.008 of the 0.02 budget
under this rule on every test shape. atol is the float32 floor of
the computation: dS is formed in float32 from logits and LSEs of magnitude up to max(1, |LSE|),
so its absolute error is about 1e-6 max(1, |LSE|) |g| times the probability mass, and the
gradient GEMM multiplies that by scale * (row norm of the contracted operand) and by the mass
that one output row sums (1 for dQ, about n_q / n_k for dK). It only matters where the exact
gradient vanishes (a single visible key, identical distributions).
"""
import numpy as np
import torch

from workloads import bf16_bits_to_f32

KL_ATOL, KL_RTOL = 1e-4, 1e-3
GRAD_RTOL = 2e-2


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).reshape(bits.shape).astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_rows_close(got, ref, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = KL_ATOL + KL_RTOL * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} rows out of tolerance; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r}")


def grad_atol(scale, g, lse_max, other, mass=1.0):
    """float32 floor for a gradient whose GEMM contracts `other` (rows = contracted operand)."""
    row = np.sqrt((np.asarray(other, np.float64) ** 2).sum(-1)).max()
    return 1e-6 * scale * float(np.abs(g).max()) * max(1.0, float(lse_max)) * row * max(1.0, mass)


def assert_grad_close(got, ref, what, atol=0.0, extra=None):
    """`extra` (optional, per element) widens the elementwise bound by an error bound derived
    for the case at hand, e.g. the most that rounding dS to bf16 can change the product."""
    got = np.asarray(got, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    err = np.abs(got - ref)
    bound = GRAD_RTOL * (np.abs(ref) + rms) + atol
    if extra is not None:
        bound = bound + extra
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; worst "
                             f"at {i}: got {got[i]!r} ref {ref[i]!r} (row rms {rms[i[:-1]][0]:.3e})")
    nerr, nref = np.linalg.norm(got - ref), np.linalg.norm(ref)
    assert nerr <= GRAD_RTOL * nref + atol * np.sqrt(ref.size), \
        f"{what}: normwise error {nerr:.3e} vs reference norm {nref:.3e}"


def row_chunks(n_q, n_k, causal, n_chunks):
    """Contiguous row ranges with about equal numbers of visible pairs."""
    pairs = np.minimum(np.arange(n_q) + 1, n_k) if causal else np.full(n_q, n_k)
    cum = np.cumsum(pairs)
    cuts = np.searchsorted(cum, np.linspace(0, cum[-1], n_chunks + 1)[1:-1])
    edges = np.unique(np.concatenate([[0], cuts, [n_q]]))
    return [np.arange(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def oracle_forward_rows(a, scale, causal, rows=None):
    """The oracle's KL, LSE1, LSE2 ([3, len(rows)]) of one slice (a: q1, k1, q2, k2 in float64)
    for the given query rows (default: all), over row blocks in a thread pool with BLAS at one
    thread per worker (the rows of a block are independent)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from oracle.reference import forward_slice

    n_q, n_k = a["q1"].shape[0], a["k1"].shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    if len(rows) == n_q:
        chunks = row_chunks(n_q, n_k, causal, 8 * workers)
    else:
        chunks = np.array_split(rows, max(1, min(len(rows), workers)))
    out = np.empty((3, n_q))

    def run(r):
        return r, forward_slice(a["q1"], a["k1"], a["q2"], a["k2"], scale, causal, rows=r)

    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)
    except Exception:  # pragma: no cover
        ctx = None
    try:
        with ThreadPoolExecutor(workers) as ex:
            for r, f in ex.map(run, chunks):
                out[:, r] = np.stack(f)
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    return out[:, rows]
