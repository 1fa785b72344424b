"""Device-side orchestration of the C ABI with torch-allocated buffers.

torch supplies device memory and the stream; every computation is a libmdlstm
kernel. ``PackedLayer`` holds one layout's descriptor and a layer's workspace
and runs scatter -> forward -> direction sum/un-pack, and the backward.
``PackedStack`` chains three levels with block-strided convolutions, each
level re-packed from the previous level's output sizes ("No Padding Please",
§V-A: packing happens just before each MDLSTM layer). ``CTCHead`` runs the
model head (height collapse, shared fully-connected layer, CTC loss) on the
last level's output.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import (MDL_BF16, MDL_CELL_LEAKY_LP, MDL_CELL_MDLSTM, MDL_F32, MDL_PACK_ALG1, MDL_PACK_EXACT, MDL_PACK_PADDED, Layout, mdl_backward,
               mdl_blockconv_backward, mdl_blockconv_forward, mdl_blockconv_workspace_size, mdl_dirsum_unpack, mdl_forward, mdl_forward_dirsum,
               mdl_layout_device_size, mdl_layout_rects, mdl_layout_upload, mdl_pack, mdl_pack_level, mdl_scatter, mdl_workspace_size,
               mdl_ctc_head, mdl_ctc_workspace_size)


def _dev(a, device, dtype=torch.float32):
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dtype, device=device).contiguous()


@dataclasses.dataclass
class DeviceParams:
    """A layer's weights on the device; Vl, Vu (the memory-state projections) only for the Leaky LP cell."""
    Wx: torch.Tensor
    Ul: torch.Tensor
    Uu: torch.Tensor
    b: torch.Tensor
    Vl: Optional[torch.Tensor] = None
    Vu: Optional[torch.Tensor] = None

    @staticmethod
    def from_host(P, device) -> "DeviceParams":
        V = [_dev(getattr(P, n), device) if getattr(P, n, None) is not None else None for n in ("Vl", "Vu")]
        return DeviceParams(_dev(P.Wx, device), _dev(P.Ul, device), _dev(P.Uu, device), _dev(P.b, device), *V)

    @property
    def cell(self):
        return MDL_CELL_MDLSTM if self.Vl is None else MDL_CELL_LEAKY_LP

    @property
    def C(self):
        return int(self.Wx.shape[1])

    @property
    def H(self):
        return int(self.Ul.shape[1])


PACK_MODES = {"packed": MDL_PACK_ALG1, "padded": MDL_PACK_PADDED, "exact": MDL_PACK_EXACT}


class DeviceLayout:
    """A packed layout plus its uploaded device descriptor."""

    def __init__(self, heights, widths, canvas_w_min: int, sep: int = 1, mode: str = "packed",
                 device: str = "cuda", stream=None, layout: Optional[Layout] = None):
        """Packs (heights, widths), or takes an already built `layout` (heights and widths then unused)."""
        if layout is None:
            if mode not in PACK_MODES:
                raise ValueError(f"unknown packing mode {mode!r}; one of {sorted(PACK_MODES)}")
            layout = mdl_pack(heights, widths, canvas_w_min, sep, PACK_MODES[mode])
        self.layout: Layout = layout
        self.device = device
        nbytes, self.eid_off, self.border_off = mdl_layout_device_size(self.layout)
        self.desc = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.desc_bytes = nbytes
        mdl_layout_upload(self.layout, self.desc, nbytes, stream)

    @property
    def info(self):
        return self.layout.info

    def sizes(self):
        """(heights, widths) of the examples, input order."""
        _, real = mdl_layout_rects(self.layout)
        return real[:, 2].copy(), real[:, 3].copy()

    def device_maps(self):
        Hc, Wc = self.layout.Hc, self.layout.Wc
        P = Hc * Wc
        eid = self.desc[self.eid_off:self.eid_off + 4 * P].view(torch.int32).reshape(Hc, Wc)
        border = self.desc[self.border_off:self.border_off + P].reshape(Hc, Wc)
        return eid, border


class PackedLayer:
    """One 4-direction MDLSTM layer on one device layout."""

    def __init__(self, dl: DeviceLayout, C: int, H: int, x_dtype: str = "f32"):
        self.dl, self.C, self.H = dl, C, H
        self.x_dtype = MDL_BF16 if x_dtype == "bf16" else MDL_F32
        info = dl.info
        dev = dl.device
        self.ws_bytes = mdl_workspace_size(dl.layout, C, H)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        tdt = torch.bfloat16 if self.x_dtype == MDL_BF16 else torch.float32
        self.x_canvas = torch.empty(info["canvas_h"], info["canvas_w"], C, dtype=tdt, device=dev)
        self.h_dirs = torch.empty(4, info["canvas_h"], info["canvas_w"], H, dtype=torch.float32, device=dev)
        self.y = torch.empty(info["real_pixels"] * H, dtype=torch.float32, device=dev)

    def scatter(self, x_flat: torch.Tensor, stream=None):
        mdl_scatter(self.dl.layout, self.dl.desc, x_flat, self.C, self.x_dtype, self.x_canvas, stream)

    def forward(self, P: DeviceParams, stream=None):
        """The cell follows the parameters: the Leaky LP cell when they carry Vl, Vu."""
        mdl_forward(self.dl.layout, self.dl.desc, self.x_canvas, self.x_dtype, self.C, self.H, P.cell, P.Wx, P.Ul,
                    P.Uu, P.b, P.Vl, P.Vu, self.h_dirs, self.ws, self.ws_bytes, stream)

    def dirsum(self, stream=None):
        mdl_dirsum_unpack(self.dl.layout, self.dl.desc, self.h_dirs, self.H, self.y, stream)

    def forward_dirsum(self, P: DeviceParams, stream=None):
        """forward() and dirsum() in one call, the direction sum overlapping the wavefront where it can."""
        mdl_forward_dirsum(self.dl.layout, self.dl.desc, self.x_canvas, self.x_dtype, self.C, self.H, P.cell, P.Wx,
                           P.Ul, P.Uu, P.b, P.Vl, P.Vu, self.h_dirs, self.y, self.ws, self.ws_bytes, stream)

    def backward(self, P: DeviceParams, grads: "LayerGrads", dy_flat=None, dh_dirs=None, dx_flat=None,
                 dx_canvas=None, stream=None):
        mdl_backward(self.dl.layout, self.dl.desc, self.x_canvas, self.x_dtype, self.C, self.H, P.cell, P.Wx, P.Ul,
                     P.Uu, P.Vl, P.Vu, self.h_dirs, dy_flat, dh_dirs, dx_flat, dx_canvas, grads.dWx, grads.dUl,
                     grads.dUu, grads.db, grads.dVl, grads.dVu, self.ws, self.ws_bytes, stream)


@dataclasses.dataclass
class LayerGrads:
    """Weight gradients; dVl, dVu for the Leaky LP cell only."""
    dWx: torch.Tensor
    dUl: torch.Tensor
    dUu: torch.Tensor
    db: torch.Tensor
    dVl: Optional[torch.Tensor] = None
    dVu: Optional[torch.Tensor] = None

    @staticmethod
    def like(P: DeviceParams) -> "LayerGrads":
        V = [torch.empty_like(t) if t is not None else None for t in (P.Vl, P.Vu)]
        return LayerGrads(torch.empty_like(P.Wx), torch.empty_like(P.Ul), torch.empty_like(P.Uu),
                          torch.empty_like(P.b), *V)


def flat_input(xs: Sequence[np.ndarray], x_dtype: str, device) -> torch.Tensor:
    """Concatenate per-example [h][w][C] tensors (bf16-exact values for 'bf16')."""
    flat = np.concatenate([np.asarray(x, np.float32).reshape(-1) for x in xs])
    t = torch.as_tensor(flat, device=device)
    return t.to(torch.bfloat16) if x_dtype == "bf16" else t


class PackedStack:
    """MDLSTM -> block conv -> MDLSTM -> block conv -> MDLSTM, re-packed per level."""

    def __init__(self, heights, widths, C: int, Hs: Sequence[int], couts: Sequence[int], canvas_w_min: Sequence[int],
                 sep: int = 1, kh: int = 2, kw: int = 4, device: str = "cuda"):
        self.kh, self.kw = kh, kw
        self.levels: List[PackedLayer] = []
        c_in = C
        dl = DeviceLayout(heights, widths, canvas_w_min[0], sep, "packed", device)
        for lvl, H in enumerate(Hs):
            self.levels.append(PackedLayer(dl, c_in, H))
            if lvl + 1 < len(Hs):
                # the next level's examples: the block conv's output sizes, packed again (the library's rule)
                nxt = mdl_pack_level(dl.layout, kh, kw, canvas_w_min[lvl + 1], sep, MDL_PACK_ALG1)
                dl = DeviceLayout(None, None, 0, device=device, layout=nxt)
                c_in = couts[lvl]
        self.couts = list(couts)
        self.conv_ws = []
        self.dx_canvas = []
        self.dh_dirs = []
        for lvl in range(len(Hs) - 1):
            lk, lk1 = self.levels[lvl], self.levels[lvl + 1]
            nb = mdl_blockconv_workspace_size(lk1.dl.layout, lk.H, kh, kw, self.couts[lvl])
            self.conv_ws.append((torch.empty(max(nb, 4), dtype=torch.uint8, device=device), nb))
            self.dx_canvas.append(torch.empty_like(lk1.x_canvas, dtype=torch.float32))
            self.dh_dirs.append(torch.empty_like(lk.h_dirs))

    @property
    def level_sizes(self):
        """Per level, the (heights, widths) of its examples."""
        return [lay.dl.sizes() for lay in self.levels]

    def forward(self, x_flat, params: Sequence[DeviceParams], convs, stream=None):
        L0 = self.levels[0]
        L0.scatter(x_flat, stream)
        for lvl, lay in enumerate(self.levels):
            lay.forward(params[lvl], stream)
            if lvl + 1 < len(self.levels):
                nxt = self.levels[lvl + 1]
                W, b = convs[lvl]
                mdl_blockconv_forward(lay.dl.layout, lay.dl.desc, nxt.dl.layout, nxt.dl.desc, lay.h_dirs, lay.H,
                                      self.kh, self.kw, W, b, self.couts[lvl], nxt.x_canvas, stream)
        self.levels[-1].dirsum(stream)
        return self.levels[-1].y

    def backward(self, params, convs, dy_flat, lgrads: Sequence[LayerGrads], cgrads, dx_flat=None, stream=None):
        n = len(self.levels)
        for lvl in range(n - 1, -1, -1):
            lay = self.levels[lvl]
            kwargs = {}
            if lvl == n - 1:
                kwargs["dy_flat"] = dy_flat
            else:
                kwargs["dh_dirs"] = self.dh_dirs[lvl]
            if lvl > 0:
                kwargs["dx_canvas"] = self.dx_canvas[lvl - 1]
            else:
                kwargs["dx_flat"] = dx_flat
            lay.backward(params[lvl], lgrads[lvl], stream=stream, **kwargs)
            if lvl > 0:
                prev = self.levels[lvl - 1]
                W, _ = convs[lvl - 1]
                dW, db = cgrads[lvl - 1]
                wsb, nb = self.conv_ws[lvl - 1]
                mdl_blockconv_backward(prev.dl.layout, prev.dl.desc, lay.dl.layout, lay.dl.desc, prev.h_dirs, prev.H,
                                       self.kh, self.kw, W, self.couts[lvl - 1], self.dx_canvas[lvl - 1],
                                       self.dh_dirs[lvl - 1], dW, db, wsb, nb, stream)


class CTCHead:
    """The model head on a layout's direction-summed output: rows summed into frames, one fully-connected layer
    to K classes (0 = blank), CTC loss per example and the gradients of their sum (mdl_ctc_head). Labels are
    fixed at construction: one sequence of classes 1..K-1 per example of the layout, in input order."""

    def __init__(self, dl: DeviceLayout, H: int, K: int, labels: Sequence[Sequence[int]],
                 max_label: Optional[int] = None):
        n = dl.info["n"]
        if len(labels) != n:
            raise ValueError(f"need one label per example ({n}), got {len(labels)}")
        self.dl, self.K, self.H = dl, K, H
        flat = np.array([c for lab in labels for c in lab], dtype=np.int32)
        off = np.zeros(n + 1, dtype=np.int32)
        off[1:] = np.cumsum([len(lab) for lab in labels])
        self.max_label = int(max(len(lab) for lab in labels)) if max_label is None else int(max_label)
        dev = dl.device
        self.n_labels = int(flat.size)
        self.labels = torch.as_tensor(flat if flat.size else np.zeros(1, np.int32), device=dev)
        self.label_off = torch.as_tensor(off, device=dev)
        self.ws_bytes = mdl_ctc_workspace_size(dl.layout, H, K, self.max_label)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.loss = torch.empty(n, dtype=torch.float32, device=dev)
        self.dy = torch.empty(dl.info["real_pixels"] * H, dtype=torch.float32, device=dev)

    def run(self, y_flat: torch.Tensor, Wfc: torch.Tensor, bfc: torch.Tensor, dWfc: Optional[torch.Tensor] = None,
            dbfc: Optional[torch.Tensor] = None, want_dy: bool = True, stream=None):
        """Loss per example into self.loss, the gradient of the summed loss with respect to y_flat into self.dy
        (if want_dy), dWfc / dbfc if given."""
        mdl_ctc_head(self.dl.layout, self.dl.desc, y_flat, self.H, Wfc, bfc, self.K, self.labels, self.label_off,
                     self.n_labels, self.max_label, self.loss, self.dy if want_dy else None, dWfc, dbfc, self.ws,
                     self.ws_bytes, stream)
        return self.loss
