"""ctypes binding of libprism.so (the C ABI of include/prism.h).

The functions carry the ABI's names and only marshal arguments: torch tensors
become device pointers, the current torch stream becomes the hipStream_t, and
a non-OK status raises PrismError with the library's message.  Every step of
the path runs in the library's HIP kernels; PyTorch only provides device
memory and the stream.  There is no fallback: if the library was not built,
importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libprism.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m dynamic_block_sparse_amd.build`")
_lib = C.CDLL(_LIB_PATH)

PRISM_F32, PRISM_BF16 = 0, 1
(OP_ZONE_SHAPES, OP_SELECT, OP_ATTN_FWD, OP_ATTN_BWD, OP_NORM_MAP, OP_FLAT_ROUTE, OP_ROUTED_FWD,
 OP_ROUTED_BWD, OP_SELECT_SUB) = range(9)
ZS_STRIDE = 16
STATUS = {0: "PRISM_OK", 1: "PRISM_E_ARG", 2: "PRISM_E_GRID", 3: "PRISM_E_DTYPE",
          4: "PRISM_E_UNSUPPORTED", 5: "PRISM_E_WORKSPACE", 6: "PRISM_E_HIP"}

EXPORTS = ["prism_hilbert_zone_order", "prism_audio_norm_map", "prism_zone_shapes", "prism_zone_shapes_noalloc",
           "prism_block_permute", "prism_block_permute_heads", "prism_select",
           "prism_select_subblock", "prism_sparse_attn_fwd", "prism_flat_route", "prism_routed_attn_fwd", "prism_routed_attn_bwd",
           "prism_sparse_attn_bwd", "prism_workspace_size", "prism_status_string", "prism_last_error",
           "prism_candidate_shapes"]


class PrismShapeParams(C.Structure):
    _fields_ = [("tau128", C.c_double), ("tau256", C.c_double), ("eps", C.c_double)]


class PrismRasterLayout(C.Structure):
    """prism_raster_layout: attention outputs written straight to raster order."""
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("W", C.c_int32), ("zone_shape", C.c_void_p),
                ("zone_order", C.c_void_p), ("ld", C.c_int64), ("hs", C.c_int64)]


class PrismError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_vp, _i32, _i64, _f32, _f64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_size_t
_lib.prism_zone_shapes.argtypes = [_i32, _i32, _i32, _vp, _i32, _i64, _i64, _vp, C.POINTER(PrismShapeParams), _vp,
                                   _vp, _vp, C.POINTER(_i32), _vp, _vp, _sz, _vp, _vp]
_lib.prism_zone_shapes_noalloc.argtypes = [_i32, _i32, _i32, _vp, _i32, _i64, _i64, _vp, C.POINTER(PrismShapeParams),
                                           _vp, _vp, _vp, C.POINTER(_i32), _vp, _vp, _vp]
_lib.prism_block_permute.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp]
_lib.prism_block_permute_heads.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i64, _i64,
                                           _i32, _vp, _vp]
_lib.prism_hilbert_zone_order.argtypes = [_i32, _i32, _i32, C.POINTER(_i32)]
_lib.prism_hilbert_zone_order.restype = C.c_int
_lib.prism_select.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _vp, _i32, _i32, _f64, _f32, _vp, _vp,
                              _i64, _vp, _vp, _vp, _sz, _vp]
_lib.prism_select_subblock.argtypes = _lib.prism_select.argtypes
_lib.prism_sparse_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _vp, _i32, _vp,
                                       _vp, _i64, _f32, C.POINTER(PrismRasterLayout), _vp, _sz, _vp]
_lib.prism_sparse_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64,
                                       _i64, _vp, _i32, _vp, _vp, _i64, _f32, C.POINTER(PrismRasterLayout), _vp, _sz,
                                       _vp]
_lib.prism_audio_norm_map.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]
_lib.prism_flat_route.argtypes = [_vp, _i32, _i32, _f64, _vp, _vp, _vp, _sz, _vp]
_lib.prism_routed_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _vp, _i32, _vp,
                                       _vp, _i64, _vp, _f32, _vp, _sz, _vp]
_lib.prism_routed_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64,
                                       _i64, _vp, _i32, _vp, _vp, _i64, _vp, _f32, _vp, _sz, _vp]
for _f in ("prism_zone_shapes_noalloc", "prism_flat_route", "prism_routed_attn_fwd", "prism_routed_attn_bwd", "prism_audio_norm_map", "prism_zone_shapes", "prism_block_permute", "prism_block_permute_heads", "prism_select",
           "prism_select_subblock", "prism_sparse_attn_fwd", "prism_sparse_attn_bwd"):
    getattr(_lib, _f).restype = C.c_int
_lib.prism_workspace_size.argtypes = [_i32, _i64, _i32, _i32, _i32, _i64]
_lib.prism_workspace_size.restype = _sz
_lib.prism_status_string.argtypes = [C.c_int]
_lib.prism_status_string.restype = C.c_char_p
_lib.prism_last_error.argtypes = []
_lib.prism_last_error.restype = C.c_char_p
_lib.prism_candidate_shapes.argtypes = [C.POINTER(_i32 * 3)]
_lib.prism_candidate_shapes.restype = None


def library_path():
    return _LIB_PATH


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dt(t):
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    if t.dtype == torch.float32:
        return PRISM_F32
    return 99   # rejected by the library with PRISM_E_DTYPE


def _check(st):
    if st != 0:
        raise PrismError(st, prism_last_error())


def prism_status_string(status):
    return _lib.prism_status_string(status).decode()


def prism_last_error():
    return _lib.prism_last_error().decode()


def prism_candidate_shapes():
    out = (_i32 * 3 * 16)()
    _lib.prism_candidate_shapes(out)
    return [tuple(int(x) for x in row) for row in out]


def prism_workspace_size(op, N, heads, d, nb, cap):
    return int(_lib.prism_workspace_size(op, N, heads, d, nb, cap))


def prism_zone_shapes(T, H, W, v, C_, v_ld, a_map, zone_shape, block_offsets, nb_dev, ws, prm=None,
                      zone_stats=None, want_nb=True, stream=None, dtype=None, zone_order=None):
    """v: raster [N, C] (any view with token stride v_ld); returns NB when want_nb."""
    nb_host = _i32(-1)
    p = PrismShapeParams(*prm) if prm is not None else None
    st = _lib.prism_zone_shapes(T, H, W, _ptr(v), _dt(v) if dtype is None else dtype, C_, v_ld, _ptr(a_map),
                                C.byref(p) if p is not None else None, _ptr(zone_shape), _ptr(block_offsets),
                                _ptr(nb_dev), C.byref(nb_host) if want_nb else None, _ptr(zone_stats), _ptr(ws),
                                ws.numel() * ws.element_size() if ws is not None else 0, _ptr(zone_order),
                                _stream(stream))
    _check(st)
    return int(nb_host.value) if want_nb else None


def prism_zone_shapes_noalloc(T, H, W, v, C_, v_ld, a_map, zone_shape, block_offsets, nb_dev, prm=None,
                              zone_stats=None, want_nb=True, stream=None, dtype=None, zone_order=None):
    """prism_zone_shapes with its scratch in the library's fixed device array
    (no workspace, nothing allocated); returns NB when want_nb."""
    nb_host = _i32(-1)
    p = PrismShapeParams(*prm) if prm is not None else None
    st = _lib.prism_zone_shapes_noalloc(T, H, W, _ptr(v), _dt(v) if dtype is None else dtype, C_, v_ld, _ptr(a_map),
                                        C.byref(p) if p is not None else None, _ptr(zone_shape), _ptr(block_offsets),
                                        _ptr(nb_dev), C.byref(nb_host) if want_nb else None, _ptr(zone_stats),
                                        _ptr(zone_order), _stream(stream))
    _check(st)
    return int(nb_host.value) if want_nb else None


ZONE_SCRATCH_BYTES = 8 << 20   # PRISM_ZONE_SCRATCH_BYTES


def prism_block_permute(T, H, W, zone_shape, x, y, row_elems, x_ld, y_ld, inverse, stream=None, dtype=None,
                        zone_order=None):
    st = _lib.prism_block_permute(T, H, W, _ptr(zone_shape), _ptr(x), _ptr(y), _dt(x) if dtype is None else dtype,
                                  row_elems, x_ld, y_ld, int(inverse), _ptr(zone_order), _stream(stream))
    _check(st)


def prism_block_permute_heads(T, H, W, zone_shape, x, y, heads, d, x_ld, x_hs, y_ld, y_hs, inverse, stream=None,
                              dtype=None, zone_order=None):
    st = _lib.prism_block_permute_heads(T, H, W, _ptr(zone_shape), _ptr(x), _ptr(y), _dt(x) if dtype is None else dtype,
                                        heads, d, x_ld, x_hs, y_ld, y_hs, int(inverse), _ptr(zone_order),
                                        _stream(stream))
    _check(st)


def prism_hilbert_zone_order(T, H, W):
    """Host list: order[pos] = raster zone index along the 3D Hilbert curve."""
    nZ = (T // 8) * (H // 8) * (W // 8)
    buf = (_i32 * max(nZ, 1))()
    _check(_lib.prism_hilbert_zone_order(T, H, W, buf))
    return [int(buf[i]) for i in range(nZ)]


def prism_audio_norm_map(h, N, C, ld, a, ws, norms=None, stream=None, dtype=None):
    st = _lib.prism_audio_norm_map(_ptr(h), _dt(h) if dtype is None else dtype, N, C, ld, _ptr(a), _ptr(norms),
                                   _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                   _stream(stream))
    _check(st)


def prism_select(q, k, N, heads, d, ld, hs, block_offsets, nb, top_k, top_p, scale, sel_offsets, sel_idx, cap,
                 sel_total, ws, logits=None, stream=None, dtype=None):
    st = _lib.prism_select(_ptr(q), _ptr(k), _dt(q) if dtype is None else dtype, N, heads, d, ld, hs,
                           _ptr(block_offsets), nb, top_k, float(top_p), float(scale), _ptr(sel_offsets),
                           _ptr(sel_idx), cap, _ptr(sel_total), _ptr(logits), _ptr(ws),
                           ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st)


def prism_select_subblock(q, k, N, heads, d, ld, hs, block_offsets, nb, top_k, top_p, scale, sel_offsets, sel_idx,
                          cap, sel_total, ws, logits=None, stream=None, dtype=None):
    """prism_select with sub-block scores (64-token runs pooled and scored in pairs)."""
    st = _lib.prism_select_subblock(_ptr(q), _ptr(k), _dt(q) if dtype is None else dtype, N, heads, d, ld, hs,
                                    _ptr(block_offsets), nb, top_k, float(top_p), float(scale), _ptr(sel_offsets),
                                    _ptr(sel_idx), cap, _ptr(sel_total), _ptr(logits), _ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st)


def prism_sparse_attn_fwd(q, k, v, o, lse, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, cap, scale,
                          ws=None, stream=None, dtype=None, layout=None, o_res=None):
    """layout: None (o block-major with q's strides) or a PrismRasterLayout.
    o_res: None or a tensor laid out like o that receives the bf16 residual of O."""
    st = _lib.prism_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o_res),
                                    _dt(q) if dtype is None else dtype,
                                    N, heads, d, ld, hs, _ptr(block_offsets), nb, _ptr(sel_offsets), _ptr(sel_idx), cap,
                                    float(scale), C.byref(layout) if layout is not None else None, _ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st)


def prism_flat_route(logits, heads, nb, flat_ratio, flat, sharpness=None, ws=None, stream=None):
    st = _lib.prism_flat_route(_ptr(logits), heads, nb, float(flat_ratio), _ptr(flat), _ptr(sharpness), _ptr(ws),
                               ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st)


def prism_routed_attn_fwd(q, k, v, o, lse, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, cap, flat,
                          scale, ws, stream=None, dtype=None, o_res=None):
    st = _lib.prism_routed_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o_res),
                                    _dt(q) if dtype is None else dtype,
                                    N, heads, d, ld, hs, _ptr(block_offsets), nb, _ptr(sel_offsets), _ptr(sel_idx),
                                    cap, _ptr(flat), float(scale), _ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st)


def prism_routed_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, N, heads, d, ld, hs, block_offsets, nb, sel_offsets,
                          sel_idx, cap, flat, scale, ws, stream=None, dtype=None, o_res=None):
    st = _lib.prism_routed_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_res), _ptr(dout), _ptr(lse), _ptr(dq),
                                    _ptr(dk),
                                    _ptr(dv), _dt(q) if dtype is None else dtype, N, heads, d, ld, hs,
                                    _ptr(block_offsets), nb, _ptr(sel_offsets), _ptr(sel_idx), cap, _ptr(flat),
                                    float(scale), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                    _stream(stream))
    _check(st)


def prism_sparse_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, N, heads, d, ld, hs, block_offsets, nb, sel_offsets,
                          sel_idx, cap, scale, ws, stream=None, dtype=None, layout=None, o_res=None):
    """layout: None (o, dq, dk, dv block-major with q's strides) or a PrismRasterLayout.
    o_res: None or the forward's residual of O (laid out like o)."""
    st = _lib.prism_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_res), _ptr(dout), _ptr(lse), _ptr(dq),
                                    _ptr(dk),
                                    _ptr(dv), _dt(q) if dtype is None else dtype, N, heads, d, ld, hs,
                                    _ptr(block_offsets), nb, _ptr(sel_offsets), _ptr(sel_idx), cap, float(scale),
                                    C.byref(layout) if layout is not None else None, _ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st)
