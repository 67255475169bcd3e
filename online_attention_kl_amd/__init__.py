"""StreamKL for AMD Instinct MI355X: a thin Python binding of libstreamkl.so.

The binding only marshals arguments: it checks shapes and dtypes, allocates outputs with
PyTorch (device memory is PyTorch's job) and passes raw pointers and the current HIP stream to
the C ABI declared in include/streamkl.h. Every step of the computation runs in the library's
HIP kernels; there is no fallback. If the library has not been built, `lib()` raises.

Functions (names follow the C ABI):
  streamkl_fwd(q1, k1, q2, k2, scale=None, causal=False)           -> (kl, lse1, lse2); adaptive
  streamkl_fwd_workspace_size(q1, k1, ...), streamkl_bwd_workspace_size(q1, k1, ...)
  streamkl_fwd_one_pass(q1, k1, q2, k2, ...)                        -> (kl, lse1, lse2)
  streamkl_fwd_noalloc(q1, k1, q2, k2, ...)      -> (kl, lse1, lse2), library scratch, no allocation
  streamkl_fwd_fp8(q1, k1, q2, k2, descale1=1, descale2=1, ...)   -> (kl, lse1, lse2), fp8 inputs
  streamkl_fwd_splitk(q1, k1, q2, k2, n_splits=0, ...)             -> (kl, lse1, lse2)
  streamkl_fwd_splitk_default_splits(q1, k1, ...), streamkl_fwd_splitk_workspace_size(...)
  streamkl_bwd_fixP1(q1, k1, q2, k2, lse1, lse2, grad_kl, ...)      -> (dq2, dk2); adaptive
  streamkl_bwd_fixP2(q1, k1, q2, k2, lse1, lse2, kl, grad_kl, ...)  -> (dq1, dk1); adaptive
  streamkl_bwd_dq(setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, ...) -> dq (one kernel)
  streamkl_bwd_dk(setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, ...) -> dk (one kernel)
  streamkl_bwd_dq_splitk(setting, ..., n_splits=0)                 -> dq (key ranges + sum)
  streamkl_bwd_fused(setting, ...)                                  -> (dq, dk), n_q <= 64
The adaptive entry points take an optional `workspace` (a uint8 CUDA tensor); when it is needed
and not given, it is allocated here with PyTorch (the library itself never allocates).
Inputs are bfloat16 CUDA tensors [B, H, N, d] (the d axis contiguous, any other strides that
are multiples of 8 elements); kl / lse / grad_kl are float32 [B, H, N_Q].
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstreamkl.so")

STATUS = {0: "STREAMKL_SUCCESS", 1: "STREAMKL_ERROR_INVALID_VALUE",
          2: "STREAMKL_ERROR_NOT_SUPPORTED", 3: "STREAMKL_ERROR_HIP"}

EXPORTS = ("streamkl_fwd", "streamkl_fwd_workspace_size", "streamkl_fwd_one_pass",
           "streamkl_fwd_noalloc", "streamkl_fwd_noalloc_max_workspace",
           "streamkl_fwd_fp8", "streamkl_fwd_splitk", "streamkl_fwd_splitk_default_splits",
           "streamkl_fwd_splitk_workspace_size", "streamkl_bwd_workspace_size",
           "streamkl_bwd_fixP1", "streamkl_bwd_fixP2",
           "streamkl_bwd_dq", "streamkl_bwd_dk", "streamkl_bwd_dq_splitk",
           "streamkl_bwd_dq_splitk_default_splits", "streamkl_bwd_dq_splitk_workspace_size",
           "streamkl_bwd_fused", "streamkl_bwd_fused_workspace_size",
           "streamkl_status_string", "streamkl_last_error")


class StreamKLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("n_q", ctypes.c_int64),
                ("n_k", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32)]


_lib = None


def lib(path: str | None = None) -> ctypes.CDLL:
    """Load libstreamkl.so (once). Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libstreamkl.so not found at {p}; build it with "
                          "`python -m online_attention_kl_amd.build`")
    L = ctypes.CDLL(p)
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    pp = ctypes.POINTER(Problem)
    L.streamkl_fwd.argtypes = [pp, vp, vp, vp, vp, fp, fp, fp, vp, ctypes.c_size_t, vp]
    L.streamkl_fwd_workspace_size.argtypes = [pp]
    L.streamkl_fwd_workspace_size.restype = ctypes.c_size_t
    L.streamkl_fwd_one_pass.argtypes = [pp, vp, vp, vp, vp, fp, fp, fp, vp]
    L.streamkl_fwd_one_pass.restype = ctypes.c_int
    L.streamkl_bwd_workspace_size.argtypes = [pp]
    L.streamkl_bwd_workspace_size.restype = ctypes.c_size_t
    L.streamkl_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, fp, fp, fp, vp]
    L.streamkl_fwd_noalloc.restype = ctypes.c_int
    L.streamkl_fwd_noalloc_max_workspace.argtypes = []
    L.streamkl_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    L.streamkl_fwd_fp8.argtypes = [pp, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp, fp, fp, fp,
                                   vp]
    L.streamkl_fwd_fp8.restype = ctypes.c_int
    L.streamkl_fwd_splitk.argtypes = [pp, vp, vp, vp, vp, fp, fp, fp, ctypes.c_int32, vp,
                                      ctypes.c_size_t, vp]
    L.streamkl_fwd_splitk.restype = ctypes.c_int
    L.streamkl_fwd_splitk_default_splits.argtypes = [pp]
    L.streamkl_fwd_splitk_default_splits.restype = ctypes.c_int32
    L.streamkl_fwd_splitk_workspace_size.argtypes = [pp, ctypes.c_int32]
    L.streamkl_fwd_splitk_workspace_size.restype = ctypes.c_size_t
    L.streamkl_bwd_fixP1.argtypes = [pp, vp, vp, vp, vp, fp, fp, fp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    L.streamkl_bwd_fixP2.argtypes = [pp, vp, vp, vp, vp, fp, fp, fp, fp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    for name in ("streamkl_bwd_dq", "streamkl_bwd_dk"):
        getattr(L, name).argtypes = [pp, ctypes.c_int32, vp, vp, vp, vp, fp, fp, fp, fp, vp, vp]
    L.streamkl_bwd_dq_splitk.argtypes = [pp, ctypes.c_int32, vp, vp, vp, vp, fp, fp, fp, fp, vp,
                                         ctypes.c_int32, vp, ctypes.c_size_t, vp]
    L.streamkl_bwd_dq_splitk_default_splits.argtypes = [pp]
    L.streamkl_bwd_dq_splitk_default_splits.restype = ctypes.c_int32
    L.streamkl_bwd_dq_splitk_workspace_size.argtypes = [pp, ctypes.c_int32]
    L.streamkl_bwd_dq_splitk_workspace_size.restype = ctypes.c_size_t
    L.streamkl_bwd_fused.argtypes = [pp, ctypes.c_int32, vp, vp, vp, vp, fp, fp, fp, fp, vp, vp,
                                     vp, ctypes.c_size_t, vp]
    L.streamkl_bwd_fused_workspace_size.argtypes = [pp]
    L.streamkl_bwd_fused_workspace_size.restype = ctypes.c_size_t
    for name in ("streamkl_fwd", "streamkl_bwd_fixP1", "streamkl_bwd_fixP2", "streamkl_bwd_dq",
                 "streamkl_bwd_dk", "streamkl_bwd_dq_splitk", "streamkl_bwd_fused"):
        getattr(L, name).restype = ctypes.c_int
    L.streamkl_status_string.argtypes = [ctypes.c_int]
    L.streamkl_status_string.restype = ctypes.c_char_p
    L.streamkl_last_error.argtypes = []
    L.streamkl_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = L
    return L


def _check(status: int):
    if status != 0:
        msg = lib().streamkl_last_error().decode()
        raise StreamKLError(status, msg)


def _run(t, fn, *args):
    """Calls a library entry point with t's device current, as the launch context of its
    kernels, and raises on an error status."""
    import torch
    with torch.cuda.device(t.device):
        status = fn(*args)
    _check(status)


def _same_device(dev, *named):
    for name, t in named:
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"{name} must be a CUDA tensor on {dev}, the device of q1")


def make_problem(q1, k1, scale, causal) -> Problem:
    B, H, nq, d = q1.shape
    nk = k1.shape[2]
    p = Problem()
    p.batch, p.heads, p.n_q, p.n_k, p.head_dim = B, H, nq, nk, d
    for i in range(3):
        p.q_stride[i] = q1.stride(i)
        p.k_stride[i] = k1.stride(i)
    p.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    p.causal = 1 if causal else 0
    return p


def _check_inputs(q1, k1, q2, k2):
    import torch
    for name, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a bfloat16 CUDA tensor [B, H, N, d] with a "
                             "contiguous last dimension")
    if q1.shape != q2.shape or q1.stride() != q2.stride():
        raise ValueError("q1 and q2 must have the same shape and strides")
    if k1.shape != k2.shape or k1.stride() != k2.stride():
        raise ValueError("k1 and k2 must have the same shape and strides")
    if k1.shape[:2] != q1.shape[:2] or k1.shape[3] != q1.shape[3]:
        raise ValueError("q and k must agree on batch, heads and head_dim")
    _same_device(q1.device, ("k1", k1), ("q2", q2), ("k2", k2))


def _rowvec(t, name, shape, dev):
    import torch
    if not t.is_cuda or t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape {shape}")
    _same_device(dev, (name, t))


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(need, workspace, device):
    """The caller's workspace tensor (checked) or, when none is given and `need` > 0, a new one.
    Returns (pointer or None, size in bytes, tensor kept alive by the caller)."""
    import torch
    if workspace is None:
        if need == 0:
            return None, 0, None
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    _same_device(device, ("workspace", workspace))
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def _fwd_out(q1, out):
    import torch
    B, H, nq, _ = q1.shape
    if out is None:
        out = tuple(torch.empty((B, H, nq), dtype=torch.float32, device=q1.device)
                    for _ in range(3))
    for n, t in zip(("kl", "lse1", "lse2"), out):
        _rowvec(t, n, (B, H, nq), q1.device)
    return out


def streamkl_fwd_workspace_size(q1, k1, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_fwd_workspace_size(ctypes.byref(p)))


def streamkl_fwd(q1, k1, q2, k2, scale=None, causal=False, out=None, workspace=None):
    """Per-row KL(P1 || P2), LSE1, LSE2 (float32 [B, H, N_Q]); the library picks one pass or the
    split-K path from the sizes."""
    _check_inputs(q1, k1, q2, k2)
    out = _fwd_out(q1, out)
    p = make_problem(q1, k1, scale, causal)
    need = int(lib().streamkl_fwd_workspace_size(ctypes.byref(p)))
    wp, wn, _keep = _workspace(need, workspace, q1.device)
    _run(q1, lib().streamkl_fwd, ctypes.byref(p), q1.data_ptr(), k1.data_ptr(), q2.data_ptr(),
         k2.data_ptr(), out[0].data_ptr(), out[1].data_ptr(),
         out[2].data_ptr(), wp, wn, _stream(q1))
    return out


def streamkl_fwd_noalloc(q1, k1, q2, k2, scale=None, causal=False, out=None):
    """streamkl_fwd with any split-K workspace taken from the library's static device scratch
    (no allocation by the library; `out` may be given to allocate nothing here either)."""
    _check_inputs(q1, k1, q2, k2)
    out = _fwd_out(q1, out)
    p = make_problem(q1, k1, scale, causal)
    _run(q1, lib().streamkl_fwd_noalloc, ctypes.byref(p), q1.data_ptr(), k1.data_ptr(),
         q2.data_ptr(), k2.data_ptr(), out[0].data_ptr(),
         out[1].data_ptr(), out[2].data_ptr(), _stream(q1))
    return out


def streamkl_fwd_one_pass(q1, k1, q2, k2, scale=None, causal=False, out=None):
    """The one-pass forward kernel whatever the sizes (no workspace)."""
    _check_inputs(q1, k1, q2, k2)
    out = _fwd_out(q1, out)
    p = make_problem(q1, k1, scale, causal)
    _run(q1, lib().streamkl_fwd_one_pass, ctypes.byref(p), q1.data_ptr(), k1.data_ptr(),
         q2.data_ptr(), k2.data_ptr(), out[0].data_ptr(),
         out[1].data_ptr(), out[2].data_ptr(), _stream(q1))
    return out


def streamkl_fwd_fp8(q1, k1, q2, k2, descale1=1.0, descale2=1.0, scale=None, causal=False,
                     out=None):
    """Forward with float8_e4m3fn inputs: side t's logits are scale * descale_t * Q_t K_t^T."""
    import torch
    for name, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2)):
        if not t.is_cuda or t.dtype != torch.float8_e4m3fn or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a float8_e4m3fn CUDA tensor [B, H, N, d] with a "
                             "contiguous last dimension")
    if q1.shape != q2.shape or q1.stride() != q2.stride() or k1.shape != k2.shape \
            or k1.stride() != k2.stride() or k1.shape[:2] != q1.shape[:2] \
            or k1.shape[3] != q1.shape[3]:
        raise ValueError("q1/q2 and k1/k2 must match in shape and strides; q and k in batch, "
                         "heads and head_dim")
    B, H, nq, _ = q1.shape
    if out is None:
        out = tuple(torch.empty((B, H, nq), dtype=torch.float32, device=q1.device)
                    for _ in range(3))
    for n, t in zip(("kl", "lse1", "lse2"), out):
        _rowvec(t, n, (B, H, nq), q1.device)
    p = make_problem(q1, k1, scale, causal)
    _run(q1, lib().streamkl_fwd_fp8, ctypes.byref(p), float(descale1), float(descale2),
         q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(),
         out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
         _stream(q1))
    return out


def streamkl_fwd_splitk_default_splits(q1, k1, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_fwd_splitk_default_splits(ctypes.byref(p)))


def streamkl_fwd_splitk_workspace_size(q1, k1, n_splits=0, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_fwd_splitk_workspace_size(ctypes.byref(p), int(n_splits)))


def streamkl_fwd_splitk(q1, k1, q2, k2, scale=None, causal=False, n_splits=0, workspace=None,
                        out=None):
    """Split-K forward for few query rows: the same (kl, lse1, lse2) as streamkl_fwd. The
    workspace (a uint8 CUDA tensor of at least streamkl_fwd_splitk_workspace_size bytes) is
    allocated here when not given."""
    import torch
    _check_inputs(q1, k1, q2, k2)
    B, H, nq, _ = q1.shape
    if out is None:
        out = tuple(torch.empty((B, H, nq), dtype=torch.float32, device=q1.device)
                    for _ in range(3))
    for n, t in zip(("kl", "lse1", "lse2"), out):
        _rowvec(t, n, (B, H, nq), q1.device)
    p = make_problem(q1, k1, scale, causal)
    need = int(lib().streamkl_fwd_splitk_workspace_size(ctypes.byref(p), int(n_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    _same_device(q1.device, ("workspace", workspace))
    nbytes = workspace.numel() * workspace.element_size()
    _run(q1, lib().streamkl_fwd_splitk, ctypes.byref(p), q1.data_ptr(), k1.data_ptr(),
         q2.data_ptr(), k2.data_ptr(), out[0].data_ptr(),
         out[1].data_ptr(), out[2].data_ptr(), int(n_splits),
         workspace.data_ptr(), nbytes, _stream(q1))
    return out


def _grad_out(q, k, out):
    import torch
    if out is None:
        out = (torch.empty(q.shape, dtype=torch.bfloat16, device=q.device),
               torch.empty(k.shape, dtype=torch.bfloat16, device=k.device))
    for n, t, ref in (("dq", out[0], q), ("dk", out[1], k)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.shape != ref.shape \
                or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous bfloat16 CUDA tensor of shape {tuple(ref.shape)}")
        _same_device(q.device, (n, t))
    return out


def streamkl_bwd_workspace_size(q1, k1, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_bwd_workspace_size(ctypes.byref(p)))


def streamkl_bwd_fixP1(q1, k1, q2, k2, lse1, lse2, grad_kl, scale=None, causal=False, out=None,
                       workspace=None):
    """Setting 1 (P1 fixed): gradients (dq2, dk2) of sum g_i KL_i, bfloat16; the library picks
    the kernels from the sizes."""
    _check_inputs(q1, k1, q2, k2)
    B, H, nq, _ = q1.shape
    for n, t in (("lse1", lse1), ("lse2", lse2), ("grad_kl", grad_kl)):
        _rowvec(t, n, (B, H, nq), q1.device)
    out = _grad_out(q2, k2, out)
    p = make_problem(q1, k1, scale, causal)
    need = int(lib().streamkl_bwd_workspace_size(ctypes.byref(p)))
    wp, wn, _keep = _workspace(need, workspace, q1.device)
    _run(q1, lib().streamkl_bwd_fixP1, ctypes.byref(p), q1.data_ptr(), k1.data_ptr(), q2.data_ptr(),
         k2.data_ptr(), lse1.data_ptr(), lse2.data_ptr(),
         grad_kl.data_ptr(), out[0].data_ptr(), out[1].data_ptr(),
         wp, wn, _stream(q1))
    return out


def streamkl_bwd_fixP2(q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale=None, causal=False,
                       out=None, workspace=None):
    """Setting 2 (P2 fixed): gradients (dq1, dk1) of sum g_i KL_i, bfloat16; the library picks
    the kernels from the sizes."""
    _check_inputs(q1, k1, q2, k2)
    B, H, nq, _ = q1.shape
    for n, t in (("lse1", lse1), ("lse2", lse2), ("kl", kl), ("grad_kl", grad_kl)):
        _rowvec(t, n, (B, H, nq), q1.device)
    out = _grad_out(q1, k1, out)
    p = make_problem(q1, k1, scale, causal)
    need = int(lib().streamkl_bwd_workspace_size(ctypes.byref(p)))
    wp, wn, _keep = _workspace(need, workspace, q1.device)
    _run(q1, lib().streamkl_bwd_fixP2, ctypes.byref(p), q1.data_ptr(), k1.data_ptr(), q2.data_ptr(),
         k2.data_ptr(), lse1.data_ptr(), lse2.data_ptr(),
         kl.data_ptr(), grad_kl.data_ptr(), out[0].data_ptr(),
         out[1].data_ptr(), wp, wn, _stream(q1))
    return out


def _bwd_one(which, setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale, causal, out):
    import torch
    _check_inputs(q1, k1, q2, k2)
    B, H, nq, _ = q1.shape
    vecs = [("lse1", lse1), ("lse2", lse2), ("grad_kl", grad_kl)]
    if setting == 2:
        vecs.append(("kl", kl))
    for n, t in vecs:
        _rowvec(t, n, (B, H, nq), q1.device)
    ref = (q2 if setting == 1 else q1) if which == "dq" else (k2 if setting == 1 else k1)
    if out is None:
        out = torch.empty(ref.shape, dtype=torch.bfloat16, device=ref.device)
    if out.dtype != torch.bfloat16 or out.shape != ref.shape or not out.is_contiguous():
        raise ValueError(f"{which} must be a contiguous bfloat16 tensor of shape {tuple(ref.shape)}")
    _same_device(q1.device, (which, out))
    p = make_problem(q1, k1, scale, causal)
    fn = lib().streamkl_bwd_dq if which == "dq" else lib().streamkl_bwd_dk
    _run(q1, fn, ctypes.byref(p), setting, q1.data_ptr(), k1.data_ptr(), q2.data_ptr(),
         k2.data_ptr(), lse1.data_ptr(), lse2.data_ptr(),
         kl.data_ptr() if kl is not None else None, grad_kl.data_ptr(), out.data_ptr(),
         _stream(q1))
    return out


def streamkl_bwd_dq(setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale=None, causal=False,
                    out=None):
    """dQ of the free side only (one kernel): dq2 for setting 1, dq1 for setting 2."""
    return _bwd_one("dq", setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale, causal, out)


def streamkl_bwd_dk(setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale=None, causal=False,
                    out=None):
    """dK of the free side only (one kernel): dk2 for setting 1, dk1 for setting 2."""
    return _bwd_one("dk", setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale, causal, out)


def streamkl_bwd_dq_splitk_default_splits(q1, k1, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_bwd_dq_splitk_default_splits(ctypes.byref(p)))


def streamkl_bwd_dq_splitk_workspace_size(q1, k1, n_splits=0, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), int(n_splits)))


def streamkl_bwd_dq_splitk(setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale=None,
                           causal=False, n_splits=0, workspace=None, out=None):
    """dQ of the free side with the keys split into ranges (few query rows); the workspace (a
    uint8 CUDA tensor of at least streamkl_bwd_dq_splitk_workspace_size bytes) is allocated
    here when not given."""
    import torch
    _check_inputs(q1, k1, q2, k2)
    B, H, nq, _ = q1.shape
    vecs = [("lse1", lse1), ("lse2", lse2), ("grad_kl", grad_kl)]
    if setting == 2:
        vecs.append(("kl", kl))
    for n, t in vecs:
        _rowvec(t, n, (B, H, nq), q1.device)
    ref = q2 if setting == 1 else q1
    if out is None:
        out = torch.empty(ref.shape, dtype=torch.bfloat16, device=ref.device)
    if out.dtype != torch.bfloat16 or out.shape != ref.shape or not out.is_contiguous():
        raise ValueError(f"dq must be a contiguous bfloat16 tensor of shape {tuple(ref.shape)}")
    _same_device(q1.device, ("dq", out))
    p = make_problem(q1, k1, scale, causal)
    need = int(lib().streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), int(n_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    _same_device(q1.device, ("workspace", workspace))
    nbytes = workspace.numel() * workspace.element_size()
    _run(q1, lib().streamkl_bwd_dq_splitk, ctypes.byref(p), setting, q1.data_ptr(), k1.data_ptr(),
         q2.data_ptr(), k2.data_ptr(), lse1.data_ptr(),
         lse2.data_ptr(), kl.data_ptr() if kl is not None else None,
         grad_kl.data_ptr(), out.data_ptr(), int(n_splits),
         workspace.data_ptr(), nbytes, _stream(q1))
    return out


def streamkl_bwd_fused_workspace_size(q1, k1, scale=None, causal=False) -> int:
    p = make_problem(q1, k1, scale, causal)
    return int(lib().streamkl_bwd_fused_workspace_size(ctypes.byref(p)))


def streamkl_bwd_fused(setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, scale=None,
                       causal=False, workspace=None, out=None):
    """(dQ, dK) of the free side from one key-major pass (n_q <= 64); the workspace (a uint8
    CUDA tensor of at least streamkl_bwd_fused_workspace_size bytes) is allocated here when
    not given."""
    import torch
    _check_inputs(q1, k1, q2, k2)
    B, H, nq, _ = q1.shape
    vecs = [("lse1", lse1), ("lse2", lse2), ("grad_kl", grad_kl)]
    if setting == 2:
        vecs.append(("kl", kl))
    for n, t in vecs:
        _rowvec(t, n, (B, H, nq), q1.device)
    qf, kf = (q2, k2) if setting == 1 else (q1, k1)
    if out is None:
        out = (torch.empty(qf.shape, dtype=torch.bfloat16, device=qf.device),
               torch.empty(kf.shape, dtype=torch.bfloat16, device=kf.device))
    for t, ref, name in ((out[0], qf, "dq"), (out[1], kf, "dk")):
        if t.dtype != torch.bfloat16 or t.shape != ref.shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor of shape "
                             f"{tuple(ref.shape)}")
        _same_device(q1.device, (name, t))
    p = make_problem(q1, k1, scale, causal)
    need = int(lib().streamkl_bwd_fused_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    _same_device(q1.device, ("workspace", workspace))
    nbytes = workspace.numel() * workspace.element_size()
    _run(q1, lib().streamkl_bwd_fused, ctypes.byref(p), setting, q1.data_ptr(), k1.data_ptr(),
         q2.data_ptr(), k2.data_ptr(), lse1.data_ptr(),
         lse2.data_ptr(), kl.data_ptr() if kl is not None else None,
         grad_kl.data_ptr(), out[0].data_ptr(), out[1].data_ptr(),
         workspace.data_ptr(), nbytes, _stream(q1))
    return out
