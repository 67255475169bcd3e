"""fp64 reference implementation of StreamKL by definition.  TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s `cpu_baseline` leg may use this
module; the product path must never route through it.

Sources (the pages are secondary summaries of the StreamKL paper, arXiv 2606.20005):
  [PT]  gist.science/pt/paper/2606.20005, "Resumo Tecnico: StreamKL":
        "Definicao do Problema" (KL between two materialised attention distributions),
        "Metodologia" section 1 (online formulation: L = acc/l1 + LSE2 - LSE1, LSE_t = m_t + log l_t),
        section 2 (saved state KL, LSE1, LSE2; regeneration P_i = exp(S_i - LSE_i); the two
        gradient settings), section 3 ("Estabilidade Numerica": log-ratio from logit
        differences and saved LSEs).
  [HI]  gist.science/hi/paper/2606.20005, technical summary (same content as [PT]).
  [ZH]  agents-report.net StreamKL article, simplified forward pseudocode.

What is computed, per (batch, head) slice, for query rows i and key columns j:
  S_t[i, j]  = scale * <Q_t[i], K_t[j]>; with `causal`, key j is visible to query i iff
               j <= i (top-left alignment), masked entries are -inf.
  LSE_t[i]   = log sum_j exp(S_t[i, j])                  (natural log, max-shifted)
  logP_t     = S_t - LSE_t[:, None],  P_t = exp(logP_t)    (masked entries: P = 0)
  KL[i]      = sum_j P1[i, j] * (logP1[i, j] - logP2[i, j])  over visible j
The gradients are not printed on the pages; they are the derivatives of sum_i g_i * KL[i]
with the fixed side held constant (stop-gradient), derived by hand:
  setting 1 (P1 fixed, P2 free):  dS2 = g_i * (P2 - P1)
  setting 2 (P2 fixed, P1 free):  dS1 = g_i * P1 * (logP1 - logP2 - KL[i])
and then, for the free side f:  dQ_f = scale * dS @ K_f,   dK_f = scale * dS^T @ Q_f.

Everything here is float64 from the exact (bf16-representable) inputs. The only blocking is
over query rows, so that one block of logits fits in memory; with `causal`, columns past the
last visible key of a block are not formed (they are masked for every row of the block).
Setting 2 uses the oracle's own float64 KL.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_ELEMS_PER_BLOCK = 1 << 23   # logits elements per row block (64 MiB per float64 matrix)


def _rows_per_block(n_k: int) -> int:
    return max(1, min(4096, _ELEMS_PER_BLOCK // max(1, n_k)))


def logits_block(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, rows: np.ndarray):
    """S = scale * q[rows] @ k^T in float64 with causal entries (j > i) set to -inf.

    Returns (S, visible) where `visible` is the boolean mask of visible entries ([PT]
    "Definicao do Problema": the attention logits of one distribution; causal masking as read
    from "Metodologia" section 1: whole key tiles past the causal frontier are skipped).
    With causal, only columns 0..max(rows) are formed.
    """
    rows = np.asarray(rows)
    n_k = k.shape[0]
    ncols = min(n_k, int(rows.max()) + 1) if causal else n_k
    S = scale * (np.asarray(q[rows], np.float64) @ np.asarray(k[:ncols], np.float64).T)
    if causal:
        visible = np.arange(ncols)[None, :] <= rows[:, None]
        S = np.where(visible, S, -np.inf)
    else:
        visible = np.ones(S.shape, dtype=bool)
    return S, visible


def _log_softmax(S: np.ndarray):
    """Row-wise LSE and log-probabilities, max-shifted ([PT] section 1: LSE_t = m_t + log l_t)."""
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return lse, S - lse[:, None]


def _kl_rows(logp1: np.ndarray, logp2: np.ndarray, visible: np.ndarray):
    """KL[i] = sum over visible j of P1 * (logP1 - logP2) ([PT] "Definicao do Problema")."""
    with np.errstate(invalid="ignore"):
        diff = np.where(visible, logp1 - logp2, 0.0)
    p1 = np.exp(logp1)           # exactly 0 on masked entries (exp(-inf))
    return (p1 * diff).sum(axis=1), p1, diff


def forward_slice(q1, k1, q2, k2, scale: float, causal: bool, rows=None):
    """KL, LSE1, LSE2 (float64) for the requested query rows of one slice (all rows if None).

    q*: [N_Q, d], k*: [N_K, d] (any real dtype; used as float64).
    """
    n_q = q1.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    kl = np.empty(rows.shape[0])
    lse1 = np.empty(rows.shape[0])
    lse2 = np.empty(rows.shape[0])
    bs = _rows_per_block(k1.shape[0])
    for s in range(0, rows.shape[0], bs):
        r = rows[s:s + bs]
        S1, vis = logits_block(q1, k1, scale, causal, r)
        S2, _ = logits_block(q2, k2, scale, causal, r)
        a, logp1 = _log_softmax(S1)
        b, logp2 = _log_softmax(S2)
        kl[s:s + bs], _, _ = _kl_rows(logp1, logp2, vis)
        lse1[s:s + bs], lse2[s:s + bs] = a, b
    return kl, lse1, lse2


def _dS_block(setting: int, S1, S2, vis, g_rows):
    """dS of the free side for one row block ([PT] "Metodologia" section 2, two settings)."""
    _, logp1 = _log_softmax(S1)
    _, logp2 = _log_softmax(S2)
    kl, p1, diff = _kl_rows(logp1, logp2, vis)
    if setting == 1:
        p2 = np.exp(logp2)
        return g_rows[:, None] * (p2 - p1)
    if setting == 2:
        return g_rows[:, None] * p1 * np.where(vis, diff - kl[:, None], 0.0)
    raise ValueError("setting must be 1 or 2")


def backward_slice(setting: int, q1, k1, q2, k2, g, scale: float, causal: bool, rows=None,
                   want_dk: bool = True):
    """(dQ_free, dK_free) in float64 for one slice.

    setting 1: free side is 2 (returns dQ2, dK2); setting 2: free side is 1 (dQ1, dK1).
    With `rows`, dQ is returned only for those query rows (in that order) and dK sums only
    their contributions (pass want_dk=False to skip it).
    """
    n_q, d = q1.shape
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    qf, kf = (q2, k2) if setting == 1 else (q1, k1)
    kf64 = np.asarray(kf, np.float64)
    dq = np.zeros((rows.shape[0], d))
    dk = np.zeros((kf.shape[0], d)) if want_dk else None
    g = np.asarray(g, np.float64)
    bs = _rows_per_block(k1.shape[0])
    for s in range(0, rows.shape[0], bs):
        r = rows[s:s + bs]
        S1, vis = logits_block(q1, k1, scale, causal, r)
        S2, _ = logits_block(q2, k2, scale, causal, r)
        dS = _dS_block(setting, S1, S2, vis, g[r])
        nc = dS.shape[1]
        dq[s:s + bs] = scale * (dS @ kf64[:nc])
        if want_dk:
            dk[:nc] += scale * (dS.T @ np.asarray(qf[r], np.float64))
    return dq, dk


def dk_rows_slice(setting: int, q1, k1, q2, k2, g, scale: float, causal: bool, keys,
                  fwd=None, rows=None):
    """dK_free[keys] (float64) of one slice, formed column by column.

    Sums the contributions of query rows `rows` (all rows if None). Needs LSE1, LSE2 (and KL
    for setting 2) of those rows: taken from `fwd` (= forward_slice(..., rows=rows)) or computed
    here. With causal, a key j is seen only by rows i >= j, so for keys >= rows[0] a row set
    that runs from rows[0] to the end gives the complete dK of those keys.
    """
    keys = np.asarray(keys)
    n_q = q1.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    if fwd is None:
        fwd = forward_slice(q1, k1, q2, k2, scale, causal, rows=rows)
    kl, lse1, lse2 = fwd
    qf = q2 if setting == 1 else q1
    S1 = scale * (np.asarray(q1[rows], np.float64) @ np.asarray(k1[keys], np.float64).T)
    S2 = scale * (np.asarray(q2[rows], np.float64) @ np.asarray(k2[keys], np.float64).T)
    if causal:
        vis = keys[None, :] <= rows[:, None]
    else:
        vis = np.ones(S1.shape, dtype=bool)
    with np.errstate(invalid="ignore"):
        logp1 = np.where(vis, S1 - lse1[:, None], -np.inf)
        logp2 = np.where(vis, S2 - lse2[:, None], -np.inf)
        p1 = np.exp(logp1)
        gr = np.asarray(g, np.float64)[rows][:, None]
        if setting == 1:
            dS = gr * (np.exp(logp2) - p1)
        else:
            dS = gr * p1 * np.where(vis, logp1 - logp2 - kl[:, None], 0.0)
    return scale * (dS.T @ np.asarray(qf[rows], np.float64))


# ---------------------------------------------------------------- whole tensors
def pool_map(fn, items, workers: int):
    """Map fn over items in a thread pool of `workers` threads, BLAS limited to one thread each."""
    if workers <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        ctx = None
    try:
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))
    finally:
        if ctx is not None:
            ctx.restore_original_limits()


def default_workers() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def forward(q1, k1, q2, k2, scale: float, causal: bool, workers: int = 1):
    """KL, LSE1, LSE2 float64 [B, H, N_Q] for [B, H, N, d] inputs (slices in a thread pool)."""
    B, H = q1.shape[:2]
    items = [(b, h) for b in range(B) for h in range(H)]
    res = pool_map(lambda bh: forward_slice(q1[bh], k1[bh], q2[bh], k2[bh], scale, causal),
                    items, workers)
    out = np.empty((3, B, H, q1.shape[2]))
    for (b, h), (kl, l1, l2) in zip(items, res):
        out[0, b, h], out[1, b, h], out[2, b, h] = kl, l1, l2
    return out[0], out[1], out[2]


def backward(setting: int, q1, k1, q2, k2, g, scale: float, causal: bool, workers: int = 1):
    """(dQ_free, dK_free) float64 [B, H, N, d] for [B, H, N, d] inputs."""
    B, H = q1.shape[:2]
    items = [(b, h) for b in range(B) for h in range(H)]
    res = pool_map(lambda bh: backward_slice(setting, q1[bh], k1[bh], q2[bh], k2[bh], g[bh],
                                              scale, causal), items, workers)
    dq = np.empty(q1.shape)
    dk = np.empty(k1.shape)
    for (b, h), (a, c) in zip(items, res):
        dq[b, h], dk[b, h] = a, c
    return dq, dk
