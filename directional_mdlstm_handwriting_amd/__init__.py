"""Python binding of libmdlstm (example-packed 4-direction 2D MDLSTM on MI355X).

Argument marshalling only: each function has the name of the C entry point it
calls (``include/mdlstm.h``) and passes device pointers and a HIP stream
through; every step of the computation runs in the library's HIP kernels.
Device arguments may be torch tensors (their ``data_ptr()`` is passed) or
plain integer addresses. ``stream`` defaults to torch's current stream.

The library is built in-tree (``python directional_mdlstm_handwriting_amd/build.py``
or ``__graft_entry__.build()``); importing this package without it raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

# torch is imported before the library is loaded: its HIP runtime then is the one
# libamdhip64 dependency the library binds to, so the device pointers and stream
# handles torch hands over belong to the same runtime instance as the library's
# own HIP calls (a second runtime loaded first finds no device it can use).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmdlstm.so")

MDL_OK = 0
MDL_EINVAL = -1
MDL_ENOMEM = -2
MDL_EOVERFLOW = -3
MDL_ESIZE = -4
MDL_EHIP = -5
MDL_EUNSUPPORTED = -6

MDL_PACK_ALG1 = 0
MDL_PACK_PADDED = 1
MDL_PACK_EXACT = 2
MDL_F32 = 0
MDL_BF16 = 1
MDL_CELL_MDLSTM = 0
MDL_CELL_LEAKY_LP = 1

INFO_KEYS = ("n", "canvas_h", "canvas_w", "rows", "real_pixels", "computed_cells", "max_depth", "max_diag", "mode",
             "wg_groups")

# every exported entry point: (name, restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SIGS = [
    ("mdl_pack", _I32, [_P, _P, _I32, _I32, _I32, _I32, ctypes.POINTER(_P)]),
    ("mdl_pack_level", _I32, [_P, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_P)]),
    ("mdl_layout_free", None, [_P]),
    ("mdl_layout_info", _I32, [_P, _P]),
    ("mdl_layout_rects", _I32, [_P, _P, _P]),
    ("mdl_layout_rows", _I32, [_P, _P, _P]),
    ("mdl_layout_maps", _I32, [_P, _P, _P]),
    ("mdl_layout_units", _I32, [_P, _P, ctypes.POINTER(_SZ)]),
    ("mdl_layout_device_size", _I32, [_P, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    ("mdl_layout_upload", _I32, [_P, _P, _SZ, _P]),
    ("mdl_workspace_size", _I32, [_P, _I32, _I32, ctypes.POINTER(_SZ)]),
    ("mdl_scatter", _I32, [_P, _P, _P, _I32, _I32, _P, _P]),
    ("mdl_forward", _I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("mdl_forward_dirsum", _I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("mdl_dirsum_unpack", _I32, [_P, _P, _P, _I32, _P, _P]),
    ("mdl_skewed_workspace_size", _I32, [_P, _I32, _I32, ctypes.POINTER(_SZ)]),
    ("mdl_forward_skewed", _I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("mdl_backward_skewed", _I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _SZ, _P]),
    ("mdl_backward", _I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                            _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("mdl_blockconv_forward", _I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _I32, _P, _P]),
    ("mdl_blockconv_workspace_size", _I32, [_P, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    ("mdl_blockconv_backward", _I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _P, _P, _SZ,
                                      _P]),
    ("mdl_blockconv_backward_noalloc", _I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _P, _P]),
    ("mdl_ctc_workspace_size", _I32, [_P, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    ("mdl_ctc_head", _I32, [_P, _P, _P, _I32, _P, _P, _I32, _P, _P, ctypes.c_int64, _I32, _P, _P, _P, _P, _P,
                            _SZ, _P]),
    ("mdl_timing", _I32, [_I32]),
    ("mdl_set_wgrad_overlap", _I32, [_I32]),
    ("mdl_timing_only", _I32, [ctypes.c_char_p]),
    ("mdl_timing_report", _I32, [_I32, _P, _P, _P, ctypes.POINTER(_I32)]),
    ("mdl_last_error", ctypes.c_char_p, []),
]
EXPORTED = tuple(name for name, _, _ in _SIGS)


class MdlError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmdlstm error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python directional_mdlstm_handwriting_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in _SIGS:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library():
    return _lib


def _check(rc: int):
    if rc != MDL_OK:
        raise MdlError(rc, _lib.mdl_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    raise TypeError(f"cannot take the address of {type(t)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


class Layout:
    """Owns an mdl_layout* (host object)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        info = np.zeros(len(INFO_KEYS), dtype=np.int64)
        _check(_lib.mdl_layout_info(self._h, info.ctypes.data))
        self.info = {k: int(v) for k, v in zip(INFO_KEYS, info)}

    @property
    def handle(self):
        return self._h

    def free(self):
        # _lib is None during interpreter shutdown, when the process releases everything anyway
        if getattr(self, "_h", None) is not None and self._h.value and _lib is not None:
            _lib.mdl_layout_free(self._h)
        self._h = None

    def __del__(self):
        self.free()

    n = property(lambda s: s.info["n"])
    Hc = property(lambda s: s.info["canvas_h"])
    Wc = property(lambda s: s.info["canvas_w"])


def mdl_pack(heights, widths, canvas_w_min: int, sep: int = 1, mode: int = MDL_PACK_ALG1) -> Layout:
    h = np.ascontiguousarray(heights, dtype=np.int32)
    w = np.ascontiguousarray(widths, dtype=np.int32)
    out = ctypes.c_void_p()
    _check(_lib.mdl_pack(h.ctypes.data, w.ctypes.data, len(h), canvas_w_min, sep, mode, ctypes.byref(out)))
    return Layout(out.value)


def mdl_pack_level(lk: Layout, kh: int, kw: int, canvas_w_min: int, sep: int = 1,
                   mode: int = MDL_PACK_ALG1) -> Layout:
    out = ctypes.c_void_p()
    _check(_lib.mdl_pack_level(lk.handle, kh, kw, canvas_w_min, sep, mode, ctypes.byref(out)))
    return Layout(out.value)


def mdl_layout_free(layout: Layout):
    layout.free()


def mdl_layout_info(layout: Layout) -> dict:
    info = np.zeros(len(INFO_KEYS), dtype=np.int64)
    _check(_lib.mdl_layout_info(layout.handle, info.ctypes.data))
    return {k: int(v) for k, v in zip(INFO_KEYS, info)}


def mdl_layout_rects(layout: Layout):
    n = layout.n
    rects = np.zeros((n, 4), np.int32)
    real = np.zeros((n, 4), np.int32)
    _check(_lib.mdl_layout_rects(layout.handle, rects.ctypes.data, real.ctypes.data))
    return rects, real


def mdl_layout_rows(layout: Layout):
    starts = np.zeros(layout.info["rows"] + 1, np.int32)
    ex = np.zeros(layout.n, np.int32)
    _check(_lib.mdl_layout_rows(layout.handle, starts.ctypes.data, ex.ctypes.data))
    return [ex[starts[r]:starts[r + 1]].tolist() for r in range(layout.info["rows"])]


def mdl_layout_units(layout: Layout):
    """(units int32 [4n], byte offset of that array in the device descriptor)."""
    units = np.zeros(4 * layout.info["n"], dtype=np.int32)
    off = _SZ()
    _check(_lib.mdl_layout_units(layout.handle, units.ctypes.data, ctypes.byref(off)))
    return units, int(off.value)


def mdl_layout_maps(layout: Layout):
    eid = np.zeros((layout.Hc, layout.Wc), np.int32)
    border = np.zeros((layout.Hc, layout.Wc), np.uint8)
    _check(_lib.mdl_layout_maps(layout.handle, eid.ctypes.data, border.ctypes.data))
    return eid, border


def mdl_layout_device_size(layout: Layout):
    b, e, o = _SZ(), _SZ(), _SZ()
    _check(_lib.mdl_layout_device_size(layout.handle, ctypes.byref(b), ctypes.byref(e), ctypes.byref(o)))
    return b.value, e.value, o.value


def mdl_layout_upload(layout: Layout, d_desc, nbytes: int, stream=None):
    _check(_lib.mdl_layout_upload(layout.handle, _ptr(d_desc), nbytes, _stream(stream)))


def mdl_workspace_size(layout: Layout, C: int, H: int) -> int:
    b = _SZ()
    _check(_lib.mdl_workspace_size(layout.handle, C, H, ctypes.byref(b)))
    return b.value


def mdl_scatter(layout: Layout, d_desc, x_flat, C: int, dtype: int, x_canvas, stream=None):
    _check(_lib.mdl_scatter(layout.handle, _ptr(d_desc), _ptr(x_flat), C, dtype, _ptr(x_canvas), _stream(stream)))


def mdl_forward(layout: Layout, d_desc, x_canvas, x_dtype: int, C: int, H: int, cell: int, Wx, Ul, Uu, b, Vl, Vu,
                h_dirs, ws, ws_bytes: int, stream=None):
    _check(_lib.mdl_forward(layout.handle, _ptr(d_desc), _ptr(x_canvas), x_dtype, C, H, cell, _ptr(Wx), _ptr(Ul),
                            _ptr(Uu), _ptr(b), _ptr(Vl), _ptr(Vu), _ptr(h_dirs), _ptr(ws), ws_bytes,
                            _stream(stream)))


def mdl_forward_dirsum(layout: Layout, d_desc, x_canvas, x_dtype: int, C: int, H: int, cell: int, Wx, Ul, Uu, b, Vl,
                       Vu, h_dirs, y_flat, ws, ws_bytes: int, stream=None):
    _check(_lib.mdl_forward_dirsum(layout.handle, _ptr(d_desc), _ptr(x_canvas), x_dtype, C, H, cell, _ptr(Wx),
                                   _ptr(Ul), _ptr(Uu), _ptr(b), _ptr(Vl), _ptr(Vu), _ptr(h_dirs), _ptr(y_flat),
                                   _ptr(ws), ws_bytes, _stream(stream)))


def mdl_skewed_workspace_size(layout: Layout, C: int, H: int) -> int:
    b = _SZ()
    _check(_lib.mdl_skewed_workspace_size(layout.handle, C, H, ctypes.byref(b)))
    return int(b.value)


def mdl_forward_skewed(layout: Layout, d_desc, x_canvas, x_dtype: int, C: int, H: int, Wx, Ul, Uu, b, h_dirs, ws,
                       ws_bytes: int, stream=None):
    _check(_lib.mdl_forward_skewed(layout.handle, _ptr(d_desc), _ptr(x_canvas), x_dtype, C, H, _ptr(Wx), _ptr(Ul),
                                   _ptr(Uu), _ptr(b), _ptr(h_dirs), _ptr(ws), ws_bytes, _stream(stream)))


def mdl_backward_skewed(layout: Layout, d_desc, x_canvas, x_dtype: int, C: int, H: int, Wx, Ul, Uu, h_dirs, dy_flat,
                        dh_dirs, dx_flat, dx_canvas, dWx, dUl, dUu, db, ws, ws_bytes: int, stream=None):
    _check(_lib.mdl_backward_skewed(layout.handle, _ptr(d_desc), _ptr(x_canvas), x_dtype, C, H, _ptr(Wx), _ptr(Ul),
                                    _ptr(Uu), _ptr(h_dirs), _ptr(dy_flat), _ptr(dh_dirs), _ptr(dx_flat),
                                    _ptr(dx_canvas), _ptr(dWx), _ptr(dUl), _ptr(dUu), _ptr(db), _ptr(ws), ws_bytes,
                                    _stream(stream)))


def mdl_dirsum_unpack(layout: Layout, d_desc, h_dirs, H: int, y_flat, stream=None):
    _check(_lib.mdl_dirsum_unpack(layout.handle, _ptr(d_desc), _ptr(h_dirs), H, _ptr(y_flat), _stream(stream)))


def mdl_backward(layout: Layout, d_desc, x_canvas, x_dtype: int, C: int, H: int, cell: int, Wx, Ul, Uu, Vl, Vu,
                 h_dirs, dy_flat, dh_dirs, dx_flat, dx_canvas, dWx, dUl, dUu, db, dVl, dVu, ws, ws_bytes: int,
                 stream=None):
    _check(_lib.mdl_backward(layout.handle, _ptr(d_desc), _ptr(x_canvas), x_dtype, C, H, cell, _ptr(Wx), _ptr(Ul),
                             _ptr(Uu), _ptr(Vl), _ptr(Vu), _ptr(h_dirs), _ptr(dy_flat), _ptr(dh_dirs),
                             _ptr(dx_flat), _ptr(dx_canvas), _ptr(dWx), _ptr(dUl), _ptr(dUu), _ptr(db), _ptr(dVl),
                             _ptr(dVu), _ptr(ws), ws_bytes, _stream(stream)))


def mdl_blockconv_forward(lk: Layout, d_desc_k, lk1: Layout, d_desc_k1, h_dirs_k, H: int, kh: int, kw: int, Wc, bc,
                          Cout: int, x_canvas_k1, stream=None):
    _check(_lib.mdl_blockconv_forward(lk.handle, _ptr(d_desc_k), lk1.handle, _ptr(d_desc_k1), _ptr(h_dirs_k), H, kh,
                                      kw, _ptr(Wc), _ptr(bc), Cout, _ptr(x_canvas_k1), _stream(stream)))


def mdl_ctc_workspace_size(layout: Layout, H: int, K: int, max_label: int) -> int:
    b = _SZ()
    _check(_lib.mdl_ctc_workspace_size(layout.handle, H, K, max_label, ctypes.byref(b)))
    return b.value


def mdl_ctc_head(layout: Layout, d_desc, y_flat, H: int, Wfc, bfc, K: int, labels, label_off, n_labels: int,
                 max_label: int, loss, dy_flat, dWfc, dbfc, ws, ws_bytes: int, stream=None):
    _check(_lib.mdl_ctc_head(layout.handle, _ptr(d_desc), _ptr(y_flat), H, _ptr(Wfc), _ptr(bfc), K, _ptr(labels),
                             _ptr(label_off), n_labels, max_label, _ptr(loss), _ptr(dy_flat), _ptr(dWfc),
                             _ptr(dbfc), _ptr(ws), ws_bytes, _stream(stream)))


def mdl_blockconv_workspace_size(lk1: Layout, H: int, kh: int, kw: int, Cout: int) -> int:
    b = _SZ()
    _check(_lib.mdl_blockconv_workspace_size(lk1.handle, H, kh, kw, Cout, ctypes.byref(b)))
    return b.value


def mdl_blockconv_backward(lk: Layout, d_desc_k, lk1: Layout, d_desc_k1, h_dirs_k, H: int, kh: int, kw: int, Wc,
                           Cout: int, dx_canvas_k1, dh_dirs_k, dWc, dbc, ws, ws_bytes: int, stream=None):
    _check(_lib.mdl_blockconv_backward(lk.handle, _ptr(d_desc_k), lk1.handle, _ptr(d_desc_k1), _ptr(h_dirs_k), H, kh,
                                       kw, _ptr(Wc), Cout, _ptr(dx_canvas_k1), _ptr(dh_dirs_k), _ptr(dWc), _ptr(dbc),
                                       _ptr(ws), ws_bytes, _stream(stream)))


def mdl_blockconv_backward_noalloc(lk: Layout, d_desc_k, lk1: Layout, d_desc_k1, h_dirs_k, H: int, kh: int, kw: int,
                                   Wc, Cout: int, dx_canvas_k1, dh_dirs_k, dWc, dbc, stream=None):
    _check(_lib.mdl_blockconv_backward_noalloc(lk.handle, _ptr(d_desc_k), lk1.handle, _ptr(d_desc_k1), _ptr(h_dirs_k),
                                               H, kh, kw, _ptr(Wc), Cout, _ptr(dx_canvas_k1), _ptr(dh_dirs_k),
                                               _ptr(dWc), _ptr(dbc), _stream(stream)))


def mdl_set_wgrad_overlap(mode):
    """Weight-gradient overlap with the reverse wavefront: True / 1 on, False / 0 off, 2 on with every task
    given up beside the wavefront (the path of a wait that runs out of time)."""
    _check(_lib.mdl_set_wgrad_overlap(int(mode)))


def mdl_timing(enable: bool):
    _check(_lib.mdl_timing(1 if enable else 0))


def mdl_timing_only(group=None):
    _check(_lib.mdl_timing_only(group.encode() if group else None))


def mdl_timing_report(max_groups: int = 32):
    """{kernel group: (total ms, launches)} of the launches recorded since the last report."""
    names = ctypes.create_string_buffer(32 * max_groups)
    ms = np.zeros(max_groups, np.float64)
    cnt = np.zeros(max_groups, np.int64)
    k = _I32()
    _check(_lib.mdl_timing_report(max_groups, names, ms.ctypes.data, cnt.ctypes.data, ctypes.byref(k)))
    out = {}
    for i in range(k.value):
        nm = names.raw[32 * i:32 * (i + 1)].split(b"\0", 1)[0].decode()
        out[nm] = (float(ms[i]), int(cnt[i]))
    return out


def mdl_last_error() -> str:
    return _lib.mdl_last_error().decode()
