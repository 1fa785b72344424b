"""Three-level MDLSTM / block-conv stack on re-packed canvases, oracle form (test infrastructure only).

"No Padding Please", §II/Fig. 1: MDLSTM layers alternate with block-strided
convolutions; §V-A: packing happens just before each MDLSTM layer from that
layer's list of input tensors, and un-packing right after it; §V-B: the
convolutions run on tensor-list chunks. The direction sum is taken after the
last MDLSTM level only (between levels the convolution consumes all four
directions' outputs as channels).
"""

from __future__ import annotations

from typing import List

import numpy as np

from . import blockconv, canvas, mdlstm, pack


def _per_example_dirs(layout, hd):
    out = []
    for (y0, x0, h, w) in layout.real:
        out.append(np.array(hd[:, y0:y0 + h, x0:x0 + w, :]))
    return out


def stack_forward(heights, widths, xs: List[np.ndarray], layers, convs, canvas_w_min, sep=1):
    """Returns (ys, caches): ys[e] = direction sum of the last level's output."""
    hs = [int(v) for v in heights]
    ws = [int(v) for v in widths]
    inputs = [np.asarray(x, np.float64) for x in xs]
    caches = []
    ys = None
    for lvl, P in enumerate(layers):
        lay = pack.pack_alg1(hs, ws, canvas_w_min[lvl], sep)
        xc = canvas.scatter(lay, inputs)
        hd, cd, gd = mdlstm.forward_vec(xc, lay.rects, P)
        entry = {"layout": lay, "cache": (xc, hd, cd, gd), "sizes": (list(hs), list(ws))}
        if lvl == len(layers) - 1:
            ys = canvas.dirsum_unpack(lay, hd)
        else:
            conv = convs[lvl]
            hd_list = _per_example_dirs(lay, hd)
            inputs = blockconv.conv_chunked(hd_list, conv.W, conv.b, conv.kh, conv.kw)
            entry["hd_list"] = hd_list
            hs = [o.shape[0] for o in inputs]
            ws = [o.shape[1] for o in inputs]
        caches.append(entry)
    return ys, caches


def stack_backward(layers, convs, caches, dys: List[np.ndarray]):
    """Returns (dxs, layer_grads [(dWx, dUl, dUu, db)] per level, conv_grads [(dW, db)] per conv)."""
    layer_grads = [None] * len(layers)
    conv_grads = [None] * len(convs)
    dhd = None
    dxs = None
    for lvl in range(len(layers) - 1, -1, -1):
        entry = caches[lvl]
        lay = entry["layout"]
        if lvl == len(layers) - 1:
            res = mdlstm.layer_backward(lay, layers[lvl], entry["cache"], dys=dys)
        else:
            res = mdlstm.layer_backward(lay, layers[lvl], entry["cache"], dhd=dhd)
        dxs_l = res[0]
        layer_grads[lvl] = tuple(res[1:5])
        if lvl > 0:
            conv = convs[lvl - 1]
            prev = caches[lvl - 1]
            dhd_list, dWc, dbc = blockconv.conv_chunked_backward(prev["hd_list"], conv.W, dxs_l, conv.kh, conv.kw)
            conv_grads[lvl - 1] = (dWc, dbc)
            play = prev["layout"]
            H = prev["cache"][1].shape[-1]
            dhd = np.zeros((4, play.Hc, play.Wc, H))
            for e, (y0, x0, h, w) in enumerate(play.real):
                dhd[:, y0:y0 + h, x0:x0 + w, :] = dhd_list[e]
        else:
            dxs = dxs_l
    return dxs, layer_grads, conv_grads
