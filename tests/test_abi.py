"""C ABI contract, on the CPU: the library loads, exports every function the header declares,
and rejects invalid calls with the documented status before touching the GPU."""
import ctypes
import os
import re

import pytest

import online_attention_kl_amd as skl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamkl.h")

pytestmark = pytest.mark.skipif(not os.path.exists(skl.LIB_PATH),
                                reason="libstreamkl.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(streamkl_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(skl.EXPORTS)
    L = skl.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = skl.lib()
    for code, name in skl.STATUS.items():
        assert L.streamkl_status_string(code).decode() == name
    assert L.streamkl_status_string(99).decode() == "STREAMKL_UNKNOWN_STATUS"


def good_problem(d=128):
    p = skl.Problem()
    p.batch, p.heads, p.n_q, p.n_k, p.head_dim = 1, 2, 64, 80, d
    for i, s in enumerate((2 * 64 * d, 64 * d, d)):
        p.q_stride[i] = s
    for i, s in enumerate((2 * 80 * d, 80 * d, d)):
        p.k_stride[i] = s
    p.scale = 0.125
    p.causal = 0
    return p


# Fake, never-dereferenced device addresses: validation returns before any launch.
Q1, K1, Q2, K2 = 0x10000000, 0x20000000, 0x30000000, 0x40000000
O1, O2, O3 = 0x50000000, 0x60000000, 0x70000000


def fwd(p, q1=Q1, k1=K1, q2=Q2, k2=K2, o=(O1, O2, O3), ws=None, nbytes=0):
    return skl.lib().streamkl_fwd(ctypes.byref(p) if p is not None else None, q1, k1, q2, k2,
                                  *o, ws, nbytes, None)


def last_error():
    return skl.lib().streamkl_last_error().decode()


def test_invalid_problem_values():
    assert fwd(None) == 1
    p = good_problem()
    p.n_q = 0
    assert fwd(p) == 1 and "n_q" in last_error()
    p = good_problem(d=96)
    for i in range(3):
        p.q_stride[i] = p.k_stride[i] = 96
    assert fwd(p) == 2 and "head_dim" in last_error()
    p = good_problem()
    p.scale = float("nan")
    assert fwd(p) == 1
    p = good_problem()
    p.scale = -1.0
    assert fwd(p) == 1
    p = good_problem()
    p.causal = 2
    assert fwd(p) == 1
    p = good_problem()
    p.q_stride[2] = 100
    assert fwd(p) == 1 and "stride" in last_error()
    p = good_problem()
    p.k_stride[2] = 64
    assert fwd(p) == 1
    # row strides of 16 MiB or more are not supported (32-bit offsets within a staged tile)
    p = good_problem()
    p.k_stride[2] = 1 << 23
    p.k_stride[1] = 80 << 23
    p.k_stride[0] = 160 << 23
    assert fwd(p) == 2 and "16 MiB" in last_error()
    p.k_stride[2] = (1 << 23) - 8
    # accepted by the stride check; the (fake) outputs then fall inside the 2.6 GB key span,
    # so the call still stops in validation, before any launch
    assert fwd(p) == 1 and "overlap" in last_error()


def test_sizes_and_strides_that_overflow():
    # each of batch and heads is bounded before their product is formed
    p = good_problem()
    p.batch, p.heads = 1 << 40, 1 << 40
    assert fwd(p) == 1 and "too large" in last_error()
    # the size queries plan from the sizes: out-of-range sizes give 0, not a plan
    L, pp = skl.lib(), ctypes.byref(p)
    assert L.streamkl_fwd_workspace_size(pp) == 0
    assert L.streamkl_bwd_workspace_size(pp) == 0
    assert L.streamkl_fwd_splitk_default_splits(pp) == 0
    assert L.streamkl_fwd_splitk_workspace_size(pp, 0) == 0
    assert L.streamkl_bwd_dq_splitk_default_splits(pp) == 0
    assert L.streamkl_bwd_dq_splitk_workspace_size(pp, 0) == 0
    assert L.streamkl_bwd_fused_workspace_size(pp) == 0
    q = good_problem()
    # each size in range, the grid not: 1024 slices x (2^29 / 128 + 1) blocks >= 2^31
    q.heads, q.n_q, q.n_k = 1024, 1 << 29, 1 << 29
    assert L.streamkl_fwd_workspace_size(ctypes.byref(q)) == 0
    assert fwd(q) == 1 and "grid" in last_error()
    p = good_problem()
    p.batch = 1 << 31
    assert fwd(p) == 1 and "too large" in last_error()
    # a batch stride whose extent does not fit in 62 bits
    p = good_problem()
    p.batch = 4
    p.k_stride[0] = 1 << 61
    assert fwd(p) == 1 and "extent" in last_error()
    p = good_problem()
    p.batch = 3
    p.q_stride[0] = (1 << 63) - 8
    assert fwd(p) == 1 and "extent" in last_error()
    # an input whose extent would wrap past the top of the address space
    p = good_problem()
    assert fwd(p, k2=(1 << 64) - 4096) == 1 and "wraps" in last_error()
    # an output that wraps
    assert fwd(p, o=(O1, O2, (1 << 64) - 16)) == 1 and "wraps" in last_error()


def test_invalid_pointers():
    p = good_problem()
    assert fwd(p, q1=0) == 1
    assert fwd(p, k2=K2 + 8) == 1 and "aligned" in last_error()
    assert fwd(p, o=(O1, 0, O3)) == 1
    assert fwd(p, o=(Q1 + 64, O2, O3)) == 1 and "overlap" in last_error()
    assert fwd(p, o=(O1, O1 + 16, O3)) == 1
    L = skl.lib()
    # backward: outputs overlapping the lse / grad vectors are rejected
    WS = 0x7A000000
    r = L.streamkl_bwd_fixP1(ctypes.byref(p), Q1, K1, Q2, K2, O1, O2, O3, O1, 0x7F000000, WS,
                             1 << 30, None)
    assert r == 1
    r = L.streamkl_bwd_fixP2(ctypes.byref(p), Q1, K1, Q2, K2, O1, O2, None, O3, 0x7E000000,
                             0x7F000000, WS, 1 << 30, None)
    assert r == 1


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        skl.lib(str(tmp_path / "nope.so"))


def splitk(p, ws, nbytes, n_splits=0, o=(O1, O2, O3)):
    return skl.lib().streamkl_fwd_splitk(ctypes.byref(p), Q1, K1, Q2, K2, *o, n_splits, ws,
                                         nbytes, None)


def test_splitk_plan_and_workspace_size():
    L = skl.lib()
    assert L.streamkl_fwd_splitk_default_splits(None) == 0
    assert L.streamkl_fwd_splitk_workspace_size(None, 4) == 0
    for nq, nk in ((1, 65536), (16, 4096), (64, 80), (300, 33), (7, 1), (33, 4096), (65, 4096),
                   (512, 65536), (2000, 1000)):
        p = good_problem()
        p.n_q, p.n_k = nq, nk
        # key granules of a range: 32 keys for wave work items (n_q <= 32), else one stage of
        # the LDS-staged kernel (128 keys without the causal mask; good_problem is non-causal)
        ntiles = (nk + 31) // 32 if nq <= 32 else (nk + 127) // 128
        per_range = 2 * nq * 5 * 4  # batch * heads * n_q * 5 floats
        d = L.streamkl_fwd_splitk_default_splits(ctypes.byref(p))
        assert 1 <= d <= ntiles
        # the default keeps at least 8 key tiles per range unless there are fewer tiles
        assert d == 1 or -(-ntiles // d) >= 8
        assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 0) == d * per_range
        for req in (1, 2, 3, 5, 64, 10 ** 6):
            used = L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), req) // per_range
            assert 1 <= used <= min(req, ntiles, 4096)
            tiles_per = -(-ntiles // used)
            assert -(-ntiles // tiles_per) == used  # no range is empty
            # as many ranges as the request allows, up to ceil(ntiles / ceil(ntiles / req))
            r = min(req, ntiles, 4096)
            assert used == -(-ntiles // -(-ntiles // r))


def test_splitk_invalid_workspace():
    p = good_problem()
    need = skl.lib().streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 1)
    WS = 0x7A000000
    assert splitk(p, 0, need, 1) == 1
    assert splitk(p, WS, need - 4, 1) == 1 and "workspace too small" in last_error()
    assert splitk(p, WS + 8, need, 1) == 1 and "aligned" in last_error()
    assert splitk(p, Q1 + 64, need, 1) == 1 and "overlap" in last_error()
    assert splitk(p, WS, need, 1, o=(O1, WS + 16, O3)) == 1


def test_dq_splitk_plan_and_workspace():
    L = skl.lib()
    assert L.streamkl_bwd_dq_splitk_default_splits(None) == 0
    assert L.streamkl_bwd_dq_splitk_workspace_size(None, 4) == 0
    for nq, nk, causal in ((1, 65536, 0), (128, 65536, 0), (300, 5000, 1), (64, 80, 0),
                           (40000, 40000, 0)):
        p = good_problem()
        p.n_q, p.n_k, p.causal = nq, nk, causal
        nvis = min(nq, nk) if causal else nk
        ntiles = (nvis + 31) // 32
        per_range = 2 * nq * 128 * 4
        d = L.streamkl_bwd_dq_splitk_default_splits(ctypes.byref(p))
        assert 1 <= d <= ntiles
        blocks = 2 * -(-nq // 256)
        if blocks >= 256:
            assert d == 1
        ws0 = L.streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), 0)
        assert ws0 == (d * per_range if d > 1 else 0)
        for req in (1, 2, 7, 10 ** 6):
            ws = L.streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), req)
            used = ws // per_range if ws else 1
            r = min(req, ntiles, 1024)
            assert used == -(-ntiles // -(-ntiles // r))


def test_dq_splitk_invalid_workspace():
    p = good_problem()
    p.n_k = 4096
    L = skl.lib()
    need = L.streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), 4)
    assert need > 0
    WS = 0x7A000000

    def call(ws, nbytes, n=4):
        return L.streamkl_bwd_dq_splitk(ctypes.byref(p), 1, Q1, K1, Q2, K2, O1, O2, None, O3,
                                        0x7C000000, n, ws, nbytes, None)
    assert call(WS, need - 4) == 1 and "workspace too small" in last_error()
    assert call(0, need) == 1
    assert call(WS + 8, need) == 1 and "aligned" in last_error()
    assert call(K1 + 64, need) == 1 and "overlap" in last_error()
    # one range: no workspace needed, validation passes up to the launch (no GPU here)
    assert L.streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), 1) == 0


def test_fused_workspace_and_limits():
    L = skl.lib()
    assert L.streamkl_bwd_fused_workspace_size(None) == 0
    for nq, nk, d, heads in ((1, 65536, 128, 32), (64, 80, 128, 2), (17, 513, 64, 2),
                             (64, 1, 64, 2), (3, 4096, 128, 32), (5, 300000, 64, 8)):
        p = good_problem(d)
        p.n_q, p.n_k, p.heads = nq, nk, heads
        steps = -(-nk // 128)
        groups = max(1, min(64, steps, steps * heads // 256))
        nkb = -(-nk // (128 * groups))
        assert L.streamkl_bwd_fused_workspace_size(ctypes.byref(p)) == nkb * heads * nq * d * 4
    p = good_problem()
    p.n_q = 65
    assert L.streamkl_bwd_fused_workspace_size(ctypes.byref(p)) == 0
    WS = 0x7A000000

    def call(p, setting=1, ws=WS, nbytes=1 << 30):
        return L.streamkl_bwd_fused(ctypes.byref(p), setting, Q1, K1, Q2, K2, O1, O2, O3,
                                    0x7C000000, 0x7D000000, 0x7E000000, ws, nbytes, None)
    # n_q past the fused path's limit: valid but not supported
    assert call(p) == 2 and "n_q" in last_error()
    p = good_problem()
    need = L.streamkl_bwd_fused_workspace_size(ctypes.byref(p))
    assert call(p, nbytes=need - 4) == 1 and "workspace too small" in last_error()
    assert call(p, ws=0, nbytes=need) == 1
    assert call(p, ws=WS + 8, nbytes=need) == 1 and "aligned" in last_error()
    assert call(p, ws=K1 + 64, nbytes=need) == 1 and "overlap" in last_error()
    assert call(p, setting=3, nbytes=need) == 1
    # setting 2 needs kl
    r = L.streamkl_bwd_fused(ctypes.byref(p), 2, Q1, K1, Q2, K2, O1, O2, None, 0x7C000000,
                             0x7D000000, 0x7E000000, WS, need, None)
    assert r == 1


def test_adaptive_workspace_sizes_follow_the_plans():
    """streamkl_fwd / streamkl_bwd_fixP1 / _fixP2 choose their kernels from the sizes; the
    workspace they need is the chosen path's: split-K forward while its default plan has more
    than one range, else none; fused backward for n_q <= 64, key-split dQ while its default plan
    has more than one range, else none."""
    L = skl.lib()
    assert L.streamkl_fwd_workspace_size(None) == 0
    assert L.streamkl_bwd_workspace_size(None) == 0
    cases = ((1, 65536, 128, 32, 0), (16, 4096, 64, 2, 1), (64, 80, 128, 2, 0),
             (65, 65536, 128, 32, 0), (512, 65536, 128, 32, 1), (4096, 4096, 128, 32, 0),
             (65536, 65536, 128, 32, 1), (2048, 32768, 64, 128, 0), (300, 33, 64, 1, 1))
    for nq, nk, d, heads, causal in cases:
        p = good_problem(d)
        p.n_q, p.n_k, p.heads, p.causal = nq, nk, heads, causal
        ns = L.streamkl_fwd_splitk_default_splits(ctypes.byref(p))
        fws = L.streamkl_fwd_workspace_size(ctypes.byref(p))
        assert fws == (L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 0) if ns > 1 else 0)
        bws = L.streamkl_bwd_workspace_size(ctypes.byref(p))
        if nq <= 64:
            assert bws == L.streamkl_bwd_fused_workspace_size(ctypes.byref(p)) > 0
        else:
            assert bws == L.streamkl_bwd_dq_splitk_workspace_size(ctypes.byref(p), 0)
    # the headline shape (32 heads x 64K rows) needs no workspace at all
    p = good_problem()
    p.n_q = p.n_k = 65536
    p.heads, p.causal = 32, 1
    assert L.streamkl_fwd_workspace_size(ctypes.byref(p)) == 0
    assert L.streamkl_bwd_workspace_size(ctypes.byref(p)) == 0
    p.head_dim = 96
    assert L.streamkl_bwd_workspace_size(ctypes.byref(p)) == 0


def test_adaptive_entry_points_check_the_workspace():
    L = skl.lib()
    WS = 0x7A000000
    p = good_problem()
    p.n_q, p.n_k, p.heads = 1, 65536, 32
    for i, s in enumerate((32 * 65536 * 128, 65536 * 128, 128)):
        p.k_stride[i] = s
    for i, s in enumerate((32 * 128, 128, 128)):
        p.q_stride[i] = s
    # keys span 512 MiB from K1 and K2: put the outputs and the workspace past them
    q1, q2, k1, k2 = 0x1000000000, 0x1100000000, 0x1200000000, 0x1300000000
    o = (0x1400000000, 0x1400010000, 0x1400020000)
    need = L.streamkl_fwd_workspace_size(ctypes.byref(p))
    assert need > 0
    ws = 0x1500000000

    def f(ws, nbytes):
        return L.streamkl_fwd(ctypes.byref(p), q1, k1, q2, k2, *o, ws, nbytes, None)
    assert f(None, 0) == 1 and "workspace too small" in last_error()
    assert f(ws, need - 4) == 1 and "workspace too small" in last_error()
    assert f(ws + 8, need) == 1 and "aligned" in last_error()
    assert f(k1 + 64, need) == 1 and "overlap" in last_error()
    assert f(o[1], need) == 1 and "overlap" in last_error()
    bneed = L.streamkl_bwd_workspace_size(ctypes.byref(p))
    assert bneed > 0
    g = 0x1400030000
    dq, dk = 0x1600000000, 0x1700000000

    def b1(ws, nbytes):
        return L.streamkl_bwd_fixP1(ctypes.byref(p), q1, k1, q2, k2, o[1], o[2], g, dq, dk, ws,
                                    nbytes, None)

    def b2(ws, nbytes, kl=o[0]):
        return L.streamkl_bwd_fixP2(ctypes.byref(p), q1, k1, q2, k2, o[1], o[2], kl, g, dq, dk,
                                    ws, nbytes, None)
    assert b1(None, 0) == 1 and "workspace too small" in last_error()
    assert b1(ws, bneed - 1) == 1 and "workspace too small" in last_error()
    assert b1(ws + 4, bneed) == 1 and "aligned" in last_error()
    assert b1(dk + 64, bneed) == 1 and "overlap" in last_error()
    assert b2(ws, bneed, kl=None) == 1
    assert b2(None, 0) == 1 and "workspace too small" in last_error()
    # one-pass forward: never a workspace; its own validation still applies
    assert L.streamkl_fwd_one_pass(ctypes.byref(p), q1, k1, q2, k2, o[0], o[0], o[2], None) == 1
    assert "overlap" in last_error()


def test_noalloc_forward_scratch_covers_every_plan_and_validates():
    """streamkl_fwd_noalloc: the library's 4 MiB scratch holds the split-K partial states of the
    default plan at every size (swept here), and invalid calls are refused before any device
    call."""
    L = skl.lib()
    cap = L.streamkl_fwd_noalloc_max_workspace()
    assert cap == 4 << 20
    worst = 0
    for bh in (1, 2, 3, 7, 8, 32, 100, 255, 256, 257, 1024):
        for nq in (1, 16, 32, 33, 64, 200, 256, 257, 511, 4096):
            for nk in (1, 100, 4096, 65536, 1 << 22):
                for causal in (0, 1):
                    p = good_problem()
                    p.heads, p.n_q, p.n_k, p.causal = bh, nq, nk, causal
                    worst = max(worst, L.streamkl_fwd_workspace_size(ctypes.byref(p)))
    assert 3 << 20 < worst <= cap
    assert L.streamkl_fwd_noalloc(None, Q1, K1, Q2, K2, O1, O2, O3, None) == 1
    p = good_problem()
    p.n_q, p.n_k = 1, 4096
    assert 0 < L.streamkl_fwd_workspace_size(ctypes.byref(p)) <= cap
    assert L.streamkl_fwd_noalloc(ctypes.byref(p), Q1, K1, Q2, K2, O1, O1, O3, None) == 1
    assert "overlap" in last_error()
    assert L.streamkl_fwd_noalloc(ctypes.byref(p), Q1, K1 + 8, Q2, K2, O1, O2, O3, None) == 1
    assert "aligned" in last_error()
