"""The C-ABI boundary on the CPU: the library loads, exports every declared
entry point, and rejects bad arguments with the right status before any
launch.  No call here reaches a kernel."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")
LIB = os.path.join(ROOT, "dynamic_block_sparse_amd", "lib", "libprism.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libprism.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) >= {"prism_audio_norm_map", "prism_zone_shapes", "prism_block_permute", "prism_select", "prism_sparse_attn_fwd",
                          "prism_sparse_attn_bwd", "prism_workspace_size", "prism_status_string",
                          "prism_last_error", "prism_candidate_shapes"}
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (prism_\w+)", out))
    assert set(names) <= exported


def test_binding_names_match_the_header():
    from dynamic_block_sparse_amd import prism as P
    assert sorted(P.EXPORTS) == _declared()
    for n in P.EXPORTS:
        assert callable(getattr(P, n))


def test_candidate_table_matches_the_oracle():
    from dynamic_block_sparse_amd import prism as P
    from oracle import prism_oracle as orc
    assert P.prism_candidate_shapes() == orc.candidate_shapes()


def test_status_strings():
    from dynamic_block_sparse_amd import prism as P
    for s in range(7):
        assert P.prism_status_string(s) and P.prism_status_string(s) != "unknown status"


# ---------------------------------------------------------------- argument checks
# Fake device addresses: non-null and 256-byte aligned, never dereferenced
# because every call below fails its host-side checks first.

A = 0x10000
B = 0x20000
Cc = 0x30000


def _lib():
    lib = ctypes.CDLL(LIB)
    from dynamic_block_sparse_amd import prism as P   # sets argtypes on its own handle
    return P._lib, P


def test_zone_shapes_rejects_bad_grids_and_args():
    lib, P = _lib()
    ws_need = P.prism_workspace_size(P.OP_ZONE_SHAPES, 8 * 16 * 16, 1, 64, 0, 0)
    assert ws_need > 0
    call = lambda T=8, H=16, W=16, v=A, dt=0, C=64, ld=64, a=B, zs=Cc, bo=A, nb=B, ws=Cc, wsb=ws_need: \
        lib.prism_zone_shapes(T, H, W, v, dt, C, ld, a, None, zs, bo, nb, None, None, ws, wsb, None, None)
    assert call(T=12) == 2
    assert call(H=0) == 2
    assert call(W=-8) == 2
    assert call(dt=7) == 3
    assert call(v=None) == 1
    assert call(a=None) == 1
    assert call(C=0) == 1
    assert call(ld=32) == 1
    assert call(ws=None) == 5
    assert call(wsb=ws_need - 1) == 5
    assert "workspace" in P.prism_last_error()


def test_zone_shapes_rejects_bad_thresholds():
    lib, P = _lib()
    ws_need = P.prism_workspace_size(P.OP_ZONE_SHAPES, 512, 1, 64, 0, 0)
    bad = P.PrismShapeParams(0.2, 0.5, 1e-6)      # tau256 above tau128
    st = lib.prism_zone_shapes(8, 8, 8, A, 0, 64, 64, B, ctypes.byref(bad), Cc, A, B, None, None, Cc, ws_need, None,
                               None)
    assert st == 1
    bad = P.PrismShapeParams(0.5, 0.25, 0.0)      # eps must be positive
    st = lib.prism_zone_shapes(8, 8, 8, A, 0, 64, 64, B, ctypes.byref(bad), Cc, A, B, None, None, Cc, ws_need, None,
                               None)
    assert st == 1


def test_block_permute_rejects():
    lib, P = _lib()
    f = lambda T=8, zs=A, x=B, y=Cc, dt=1, re_=128, xl=128, yl=128, inv=0: \
        lib.prism_block_permute(T, 8, 8, zs, x, y, dt, re_, xl, yl, inv, None, None)
    assert f(T=4) == 2
    assert f(zs=None) == 1
    assert f(dt=5) == 3
    assert f(re_=0) == 1
    assert f(xl=64) == 1
    assert f(inv=2) == 1
    assert f(x=B, y=B + 64) == 1                   # overlapping buffers
    assert "overlap" in P.prism_last_error()


def test_block_permute_heads_rejects():
    lib, P = _lib()
    X, Y = 0x1000000, 0x2000000                    # 16 MiB apart: the 8x8x8 spans do not meet
    f = lambda T=8, zs=A, x=X, y=Y, dt=1, heads=2, d=128, xl=256, xh=128, yl=128, yh=512 * 128, inv=0: \
        lib.prism_block_permute_heads(T, 8, 8, zs, x, y, dt, heads, d, xl, xh, yl, yh, inv, None, None)
    assert f(T=12) == 2
    assert f(zs=None) == 1
    assert f(y=None) == 1
    assert f(dt=7) == 3
    assert f(heads=0) == 1
    assert f(d=0) == 1
    assert f(xh=-128) == 1
    assert f(inv=3) == 1
    assert f(d=100) == 4                           # 200 bytes: not a 16-byte multiple
    assert f(xl=260) == 4
    assert f(y=Y + 8) == 4                         # misaligned
    assert f(x=X, y=X + 4096) == 1                 # overlapping spans
    assert "overlap" in P.prism_last_error()


def test_select_rejects():
    lib, P = _lib()
    N, heads, d, nb = 2048, 1, 64, 24
    cap = nb * nb
    need = P.prism_workspace_size(P.OP_SELECT, N, heads, d, nb, cap)
    f = lambda q=A, dt=0, N=N, heads=heads, d=d, ld=64, hs=64, nb=nb, k=4, p=0.9, cap=cap, ws=Cc, wsb=need: \
        lib.prism_select(q, B, dt, N, heads, d, ld, hs, Cc, nb, k, p, 0.125, A, B, cap, Cc, None, ws, wsb, None)
    assert f(dt=3) == 3
    assert f(N=100) == 1
    assert f(heads=0) == 1
    assert f(d=96) == 4
    assert f(ld=60) == 1
    assert f(ld=66) == 4                           # not a multiple of 4 fp32 elements
    assert f(ld=1 << 24) == 4                      # 64 rows would span 4 GiB: beyond 32-bit tile offsets
    assert f(nb=0) == 1
    assert f(nb=N // 64 + 1) == 1
    assert f(N=64 * 32769, nb=32769) == 4          # above the 32768-block limit
    assert "32768" in P.prism_last_error()
    assert f(k=-1) == 1
    assert f(p=1.5) == 1
    assert f(p=float("nan")) == 1
    assert f(cap=0) == 1
    assert f(q=None) == 1
    assert f(q=A + 8) == 4                         # misaligned
    assert f(ws=None) == 5
    assert f(wsb=need - 1) == 5


def test_select_subblock_rejects():
    lib, P = _lib()
    N, heads, d, nb = 2048, 2, 64, 24
    cap = nb * nb
    need = P.prism_workspace_size(P.OP_SELECT_SUB, N, heads, d, nb, cap)
    assert need >= heads * (N // 64) ** 2 * 8 + 2 * heads * (N // 64) * d * 8   # run-pair scores and run means
    f = lambda q=A, dt=0, N=N, heads=heads, d=d, nb=nb, k=4, p=0.9, cap=cap, ws=Cc, wsb=need: \
        lib.prism_select_subblock(q, B, dt, N, heads, d, 128, 64, Cc, nb, k, p, 0.125, A, B, cap, Cc, None, ws, wsb,
                                  None)
    assert f(dt=3) == 3
    assert f(N=100) == 1
    assert f(N=2048 + 32) == 1                     # not a multiple of 64
    assert f(heads=0) == 1
    assert f(d=96) == 4
    assert f(nb=0) == 1
    assert f(k=-1) == 1
    assert f(p=-0.5) == 1
    assert f(q=None) == 1
    assert f(q=A + 8) == 4
    assert f(ws=None) == 5
    assert f(wsb=need - 1) == 5
    assert "workspace" in P.prism_last_error()


def test_attention_rejects():
    import ctypes
    lib, P = _lib()
    N, heads, d, nb = 2048, 2, 128, 24
    cap = nb * nb
    fneed = P.prism_workspace_size(P.OP_ATTN_FWD, N, heads, d, nb, cap)
    assert fneed >= 4 * heads * (N // 64)          # at least the tile order
    good = P.PrismRasterLayout(8, 16, 16, Cc, None, heads * d, d)
    fwd = lambda q=A, dt=1, d=d, o=Cc, ws=B, wsb=fneed, lay=None, res=None: lib.prism_sparse_attn_fwd(
        q, B, Cc, o, A, res, dt, N, heads, d, 256, 128, B, nb, Cc, A, cap, 0.088,
        ctypes.byref(lay) if lay is not None else None, ws, wsb, None)
    assert fwd(dt=2) == 3
    assert fwd(d=32) == 4
    assert fwd(q=None) == 1
    assert fwd(o=Cc + 8) == 4                      # misaligned
    assert fwd(ws=None) == 5
    assert fwd(wsb=fneed - 16) == 5
    assert fwd(res=B + 8) == 4                     # misaligned residual
    assert fwd(res=B, dt=0) == 1                   # residual of an fp32 output
    assert fwd(res=B, ws=None) == 5                # an aligned bf16 residual passes its checks
    # raster placement of the outputs: grid, token count, zone shapes, strides
    assert fwd(lay=P.PrismRasterLayout(8, 16, 12, Cc, None, heads * d, d)) == 2     # W not a multiple of 8
    assert fwd(lay=P.PrismRasterLayout(8, 16, 8, Cc, None, heads * d, d)) == 1      # 1024 tokens, not N
    assert fwd(lay=P.PrismRasterLayout(8, 16, 16, None, None, heads * d, d)) == 1   # no zone shapes
    assert fwd(lay=P.PrismRasterLayout(8, 16, 16, Cc, None, heads * d + 4, d)) == 4  # 8-byte stride (bf16)
    assert fwd(lay=P.PrismRasterLayout(8, 16, 16, Cc, None, 0, d)) == 4
    assert fwd(lay=P.PrismRasterLayout(8, 16, 16, Cc, None, heads * d, -8)) == 4
    assert fwd(lay=good, ws=None) == 5             # a valid layout passes its checks
    need = P.prism_workspace_size(P.OP_ATTN_BWD, N, heads, d, nb, cap)
    assert need > 0
    bwd = lambda ws=A, wsb=need, dq=A, lay=None, res=None: lib.prism_sparse_attn_bwd(
        A, B, Cc, A, res, B, Cc, dq, B, Cc, 1, N, heads, d, 256, 128, A, nb, B, Cc, cap, 0.088,
        ctypes.byref(lay) if lay is not None else None, ws, wsb, None)
    assert bwd(ws=None) == 5
    assert bwd(wsb=need - 16) == 5
    assert bwd(dq=None) == 1
    assert bwd(res=Cc + 4) == 4
    assert bwd(lay=P.PrismRasterLayout(16, 16, 16, Cc, None, heads * d, d)) == 1     # 4096 tokens, not N
    assert bwd(lay=good, ws=None) == 5


def test_workspace_sizes_grow_with_the_problem():
    from dynamic_block_sparse_amd import prism as P
    a = P.prism_workspace_size(P.OP_SELECT, 4096, 1, 64, 16, 256)
    b = P.prism_workspace_size(P.OP_SELECT, 4096, 2, 64, 16, 256)
    c = P.prism_workspace_size(P.OP_SELECT, 4096, 1, 64, 32, 1024)
    assert 0 < a < b and a < c
    f1 = P.prism_workspace_size(P.OP_ATTN_FWD, 4096, 1, 64, 16, 256)
    assert 0 < f1 < P.prism_workspace_size(P.OP_ATTN_FWD, 4096, 2, 64, 16, 256)
    assert P.prism_workspace_size(P.OP_ZONE_SHAPES, 512, 1, 3072, 0, 0) >= 16 * 8


def test_norm_map_rejects():
    lib, P = _lib()
    need = P.prism_workspace_size(P.OP_NORM_MAP, 1000, 0, 0, 0, 0)
    assert need >= 8 * 1000
    f = lambda h=A, dt=1, N=1000, C=64, ld=64, a=B, ws=Cc, wsb=need: lib.prism_audio_norm_map(h, dt, N, C, ld, a, None,
                                                                                          ws, wsb, None)
    assert f(dt=2) == 3
    assert f(h=None) == 1
    assert f(a=None) == 1
    assert f(N=0) == 1
    assert f(C=0) == 1
    assert f(ld=63) == 1
    assert f(ws=None) == 5
    assert f(wsb=need - 8) == 5


def test_flat_route_and_routed_forward_reject():
    lib, P = _lib()
    heads, nb = 2, 24
    need = P.prism_workspace_size(P.OP_FLAT_ROUTE, 0, heads, 0, nb, 0)
    assert need >= 8 * heads * nb
    r = lambda L=A, h=heads, n=nb, ratio=0.5, fl=B, M=None, ws=Cc, wsb=need: lib.prism_flat_route(L, h, n, ratio, fl, M,
                                                                                                 ws, wsb, None)
    assert r(L=None) == 1
    assert r(fl=None) == 1
    assert r(h=0) == 1
    assert r(n=0) == 1
    assert r(ratio=1.5) == 1
    assert r(ratio=float("nan")) == 1
    assert r(ws=None) == 5
    assert r(wsb=need - 8) == 5
    N, d = 2048, 128
    cap = nb * nb
    fneed = P.prism_workspace_size(P.OP_ROUTED_FWD, N, heads, d, nb, cap)
    assert fneed >= 2 * 4 * heads * nb * d + 4 * heads * (N // 64)   # block means and the tile order
    f = lambda fl=B, ws=Cc, wsb=fneed, dt=1: lib.prism_routed_attn_fwd(A, B, Cc, Cc, A, None, dt, N, heads, d, 256, 128,
                                                                       B, nb, Cc, A, cap, fl, 0.088, ws, wsb, None)
    assert f(dt=2) == 3
    assert f(fl=None) == 1
    assert f(ws=None) == 5
    assert f(wsb=fneed - 16) == 5


def test_routed_backward_rejects():
    lib, P = _lib()
    N, heads, d, nb = 2048, 2, 128, 24
    cap = nb * nb
    need = P.prism_workspace_size(P.OP_ROUTED_BWD, N, heads, d, nb, cap)
    assert need >= 4 * 4 * heads * nb * d + 4 * heads * N     # block-mean gradients and the row dots
    f = lambda fl=B, ws=A, wsb=need, dq=A: lib.prism_routed_attn_bwd(A, B, Cc, A, None, B, Cc, dq, B, Cc, 1, N, heads, d,
                                                                     256, 128, A, nb, B, Cc, cap, fl, 0.088, ws, wsb,
                                                                     None)
    assert f(dq=None) == 1
    assert f(fl=None) == 1
    assert f(ws=None) == 5
    assert f(wsb=need - 16) == 5


@pytest.mark.parametrize("grid", [(8, 8, 8), (16, 16, 16), (64, 64, 64), (64, 72, 128), (24, 40, 16), (120, 72, 128)])
def test_hilbert_zone_order_matches_the_oracle(grid):
    """The library's host Hilbert order (its own implementation of Skilling's
    transform) against the oracle's, on cubes and on the workloads' grids."""
    from dynamic_block_sparse_amd import prism as P
    from oracle import prism_oracle as orc
    T, H, W = grid
    assert P.prism_hilbert_zone_order(T, H, W) == orc.hilbert_zone_order(T, H, W).tolist()


def test_hilbert_zone_order_rejects():
    lib, P = _lib()
    buf = (ctypes.c_int32 * 8)()
    assert lib.prism_hilbert_zone_order(12, 8, 8, buf) == 2
    assert lib.prism_hilbert_zone_order(8, 8, 8, None) == 1


def test_zone_shapes_noalloc_rejects_before_any_launch():
    """The no-allocation zone shapes call checks its arguments like
    prism_zone_shapes and rejects a grid whose scratch exceeds the fixed
    array (PRISM_E_WORKSPACE) before it looks up the array or launches."""
    lib, P = _lib()
    f = lambda T=8, H=8, W=8, v=A, C_=128, a=B, zs=Cc: lib.prism_zone_shapes_noalloc(
        T, H, W, v, 1, C_, C_, a, None, zs, Cc, Cc, None, None, None, None)
    assert f(T=12) == 2
    assert f(v=None) == 1
    assert f(C_=0) == 1
    # 64 x 64 x 64 zones at 3072 channels: about 109 MB of scratch
    big = P.prism_workspace_size(P.OP_ZONE_SHAPES, 512 ** 3, 0, 3072, 0, 0)
    assert big > P.ZONE_SCRATCH_BYTES
    assert f(T=512, H=512, W=512, C_=3072) == 5
    assert "no-allocation" in P.prism_last_error()
    # the 2K workload's grid fits
    assert P.prism_workspace_size(P.OP_ZONE_SHAPES, 64 * 72 * 128, 0, 3072, 0, 0) <= P.ZONE_SCRATCH_BYTES
