"""4-direction 2D MDLSTM layer, forward and 2D BPTT, oracle form (test infrastructure only).

What is computed
----------------
"No Padding Please", §III (and Fig. 2/4a): a 2D MDLSTM cell receives a
<hidden, state> pair from each of its two predecessors in the scan direction
(the one to its left and the one above it, "as defined by the scanning
direction", §IV-A) plus its input; two forget gates weigh the two predecessor
states. Four such MDLSTMs, one per scan direction, each with its own weights,
make the 4-directional layer. RETURNN (§4.2) states the same dependency:
h(u,v) needs h(u-1,v) and h(u,v-1). The cell equations sat in a figure that
the extracted text lost; the cell used here is the one the task states:

    a   = x.Wx[d] + b[d] + h_left.Ul[d] + h_up.Uu[d]        (5H: i, f_l, f_u, o, g)
    i, f_l, f_u, o = sigmoid(.),  g = tanh(.)
    c   = f_l * c_left + f_u * c_up + i * g
    h   = o * tanh(c)
    y   = sum over the four directions of h

§V: a binary mask blocks hidden and memory state coming from predecessors
that are padding or separator cells; such a predecessor reads as (0, 0).

Directions (sy, sx): 0 = (+1,+1) from the top-left, 1 = (+1,-1) from the
top-right, 2 = (-1,+1) from the bottom-left, 3 = (-1,-1) from the bottom-right.
The left predecessor of (y, x) is (y, x - sx), the upper one (y - sy, x).

Backward (2D BPTT): the general rule of the single-stream generalised-LSTM
paper (backward pass in reverse topological order; weight gradient = sum over
frames of activation times delta) applied to this cell, derived by hand:

    tc = tanh(c); do = dh*tc; dc = dc_in + dh*o*(1-tc^2)
    da = [dc*g*i(1-i), dc*c_l*f_l(1-f_l), dc*c_u*f_u(1-f_u), do*o(1-o), dc*i*(1-g^2)]
    left  predecessor: dh += da.Ul^T, dc += dc*f_l;   upper: dh += da.Uu^T, dc += dc*f_u
    dWx += x^T da, dUl += h_l^T da, dUu += h_u^T da, db += da, dx += da.Wx^T

Forms
-----
* ``forward_canvas_brute`` / ``backward_canvas_brute``: the definition. Scan the
  whole canvas cell by cell in each direction's scan order; predecessor
  validity comes from the packer's border map.
* ``forward_example_brute``: one example alone (validity from its bounds).
* ``forward_vec`` / ``backward_vec``: the same arithmetic, all cells of one
  local anti-diagonal of every example at once (the diagonal parallelism of
  §I / RETURNN §4.2); checked against the brute forms.
All arithmetic in float64. The per-diagonal forms also take a numeric context
(``num``): the floating-point type of every array and the elementary functions
(exponential, tanh, division). The default is float64 with NumPy's functions;
a float32 context evaluates the same formulas in single precision, which the
tests use to measure how far valid fp32 evaluations scatter around the exact
result and the CPU timing uses as the float32 form.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .pack import BIT_D, BIT_L, BIT_R, BIT_U

DIRS = ((+1, +1), (+1, -1), (-1, +1), (-1, -1))


class Num:
    """Numeric context of the per-diagonal forms: array type and elementary functions."""

    def __init__(self, dtype=np.float64):
        self.dtype = np.dtype(dtype)

    def exp(self, z):
        return np.exp(z)

    def tanh(self, z):
        return np.tanh(z)

    def div(self, a, b):
        return a / b


F64 = Num(np.float64)


def _p64(P, dtype=np.float64):
    return (np.asarray(P.Wx, dtype), np.asarray(P.Ul, dtype),
            np.asarray(P.Uu, dtype), np.asarray(P.b, dtype))


def sigmoid(z, num=F64):
    return num.div(1.0, 1.0 + num.exp(-z))


def _pred_bits(d):
    sy, sx = DIRS[d]
    return (BIT_L if sx > 0 else BIT_R), (BIT_U if sy > 0 else BIT_D)


def _cell(xv, hl, cl, hu, cu, Wx, Ul, Uu, b, H, num=F64):
    a = xv @ Wx + b + hl @ Ul + hu @ Uu
    i = sigmoid(a[..., 0:H], num)
    fl = sigmoid(a[..., H:2 * H], num)
    fu = sigmoid(a[..., 2 * H:3 * H], num)
    o = sigmoid(a[..., 3 * H:4 * H], num)
    g = num.tanh(a[..., 4 * H:5 * H])
    c = fl * cl + fu * cu + i * g
    h = o * num.tanh(c)
    return h, c, np.concatenate([i, fl, fu, o, g], axis=-1)


def _cell_grad(dh, dc_in, gates, c, cl, cu, H, num=F64):
    i, fl, fu, o, g = (gates[..., k * H:(k + 1) * H] for k in range(5))
    tc = num.tanh(c)
    do = dh * tc
    dc = dc_in + dh * o * (1.0 - tc * tc)
    da = np.concatenate([dc * g * i * (1.0 - i),
                         dc * cl * fl * (1.0 - fl),
                         dc * cu * fu * (1.0 - fu),
                         do * o * (1.0 - o),
                         dc * i * (1.0 - g * g)], axis=-1)
    return da, dc, fl, fu


# ----------------------------------------------------------------------------------------------
# definition: cell-by-cell scan of the canvas, validity from the border map
# ----------------------------------------------------------------------------------------------

def _scan(Hc, Wc, d, reverse=False):
    sy, sx = DIRS[d]
    ys = list(range(Hc)) if sy > 0 else list(range(Hc - 1, -1, -1))
    xs = list(range(Wc)) if sx > 0 else list(range(Wc - 1, -1, -1))
    order = [(y, x) for y in ys for x in xs]
    return order[::-1] if reverse else order


def forward_canvas_brute(xc, eid, border, P):
    """xc [Hc][Wc][C] -> (h_dirs, c_dirs, gates) each [4][Hc][Wc][.]; zero where eid < 0."""
    Wx, Ul, Uu, b = _p64(P)
    xc = np.asarray(xc, np.float64)
    Hc, Wc, _ = xc.shape
    H = Ul.shape[1]
    hd = np.zeros((4, Hc, Wc, H))
    cd = np.zeros((4, Hc, Wc, H))
    gd = np.zeros((4, Hc, Wc, 5 * H))
    zero = np.zeros(H)
    for d in range(4):
        sy, sx = DIRS[d]
        lbit, ubit = _pred_bits(d)
        for (y, x) in _scan(Hc, Wc, d):
            if eid[y, x] < 0:
                continue
            if border[y, x] & lbit:
                hl, cl = hd[d, y, x - sx], cd[d, y, x - sx]
            else:
                hl, cl = zero, zero
            if border[y, x] & ubit:
                hu, cu = hd[d, y - sy, x], cd[d, y - sy, x]
            else:
                hu, cu = zero, zero
            h, c, g = _cell(xc[y, x], hl, cl, hu, cu, Wx[d], Ul[d], Uu[d], b[d], H)
            hd[d, y, x], cd[d, y, x], gd[d, y, x] = h, c, g
    return hd, cd, gd


def backward_canvas_brute(xc, eid, border, P, hd, cd, gd, dhd):
    """Reverse scan. dhd [4][Hc][Wc][H] = dL/dh of each direction's output.

    Returns (dxc [Hc][Wc][C], dWx, dUl, dUu, db)."""
    Wx, Ul, Uu, b = _p64(P)
    xc = np.asarray(xc, np.float64)
    Hc, Wc, C = xc.shape
    H = Ul.shape[1]
    dxc = np.zeros((Hc, Wc, C))
    dWx, dUl, dUu, db = (np.zeros_like(a) for a in (Wx, Ul, Uu, b))
    zero = np.zeros(H)
    for d in range(4):
        sy, sx = DIRS[d]
        lbit, ubit = _pred_bits(d)
        dh_acc = np.array(dhd[d], np.float64)
        dc_acc = np.zeros((Hc, Wc, H))
        for (y, x) in _scan(Hc, Wc, d, reverse=True):
            if eid[y, x] < 0:
                continue
            vl = bool(border[y, x] & lbit)
            vu = bool(border[y, x] & ubit)
            hl, cl = (hd[d, y, x - sx], cd[d, y, x - sx]) if vl else (zero, zero)
            hu, cu = (hd[d, y - sy, x], cd[d, y - sy, x]) if vu else (zero, zero)
            da, dc, fl, fu = _cell_grad(dh_acc[y, x], dc_acc[y, x], gd[d, y, x], cd[d, y, x], cl, cu, H)
            if vl:
                dh_acc[y, x - sx] += Ul[d] @ da
                dc_acc[y, x - sx] += dc * fl
            if vu:
                dh_acc[y - sy, x] += Uu[d] @ da
                dc_acc[y - sy, x] += dc * fu
            dWx[d] += np.outer(xc[y, x], da)
            dUl[d] += np.outer(hl, da)
            dUu[d] += np.outer(hu, da)
            db[d] += da
            dxc[y, x] += Wx[d] @ da
    return dxc, dWx, dUl, dUu, db


def forward_example_brute(x, P):
    """One example alone, x [h][w][C]; predecessors outside [0,h)x[0,w) read as zero.

    Returns h_dirs [4][h][w][H]."""
    Wx, Ul, Uu, b = _p64(P)
    x = np.asarray(x, np.float64)
    h_, w_, _ = x.shape
    H = Ul.shape[1]
    hd = np.zeros((4, h_, w_, H))
    cd = np.zeros((4, h_, w_, H))
    zero = np.zeros(H)
    for d in range(4):
        sy, sx = DIRS[d]
        for (y, xx) in _scan(h_, w_, d):
            inl = 0 <= xx - sx < w_
            inu = 0 <= y - sy < h_
            hl, cl = (hd[d, y, xx - sx], cd[d, y, xx - sx]) if inl else (zero, zero)
            hu, cu = (hd[d, y - sy, xx], cd[d, y - sy, xx]) if inu else (zero, zero)
            h, c, _ = _cell(x[y, xx], hl, cl, hu, cu, Wx[d], Ul[d], Uu[d], b[d], H)
            hd[d, y, xx], cd[d, y, xx] = h, c
    return hd


# ----------------------------------------------------------------------------------------------
# per-diagonal form: all cells of one local anti-diagonal (of every example) at once
# ----------------------------------------------------------------------------------------------

def diagonals(rects, d):
    """For direction d: list over local diagonal s of (Y, X, left_valid, up_valid).

    An example's cell with direction-local coordinates (a, b) (a counted along
    the scan's rows, b along its columns) lies on diagonal s = a + b."""
    sy, sx = DIRS[d]
    per_s = {}
    for (y0, x0, h, w) in np.asarray(rects, np.int64):
        for s in range(h + w - 1):
            a = np.arange(max(0, s - w + 1), min(h - 1, s) + 1)
            bb = s - a
            Y = y0 + (a if sy > 0 else h - 1 - a)
            X = x0 + (bb if sx > 0 else w - 1 - bb)
            per_s.setdefault(s, []).append((Y, X, bb > 0, a > 0))
    out = []
    for s in sorted(per_s):
        parts = per_s[s]
        out.append(tuple(np.concatenate([p[k] for p in parts]) for k in range(4)))
    return out


def forward_vec(xc, rects, P, num=F64):
    """Same as forward_canvas_brute, one local diagonal at a time."""
    ft = num.dtype
    Wx, Ul, Uu, b = _p64(P, ft)
    xc = np.asarray(xc, ft)
    Hc, Wc, _ = xc.shape
    H = Ul.shape[1]
    hd = np.zeros((4, Hc, Wc, H), ft)
    cd = np.zeros((4, Hc, Wc, H), ft)
    gd = np.zeros((4, Hc, Wc, 5 * H), ft)
    for d in range(4):
        sy, sx = DIRS[d]
        for (Y, X, VL, VU) in diagonals(rects, d):
            m = len(Y)
            hl = np.zeros((m, H), ft); cl = np.zeros((m, H), ft)
            hu = np.zeros((m, H), ft); cu = np.zeros((m, H), ft)
            hl[VL] = hd[d, Y[VL], X[VL] - sx]
            cl[VL] = cd[d, Y[VL], X[VL] - sx]
            hu[VU] = hd[d, Y[VU] - sy, X[VU]]
            cu[VU] = cd[d, Y[VU] - sy, X[VU]]
            h, c, g = _cell(xc[Y, X], hl, cl, hu, cu, Wx[d], Ul[d], Uu[d], b[d], H, num)
            hd[d, Y, X], cd[d, Y, X], gd[d, Y, X] = h, c, g
    return hd, cd, gd


def backward_vec(xc, rects, P, hd, cd, gd, dhd, num=F64):
    """Same as backward_canvas_brute, one local diagonal at a time, in reverse."""
    ft = num.dtype
    Wx, Ul, Uu, b = _p64(P, ft)
    xc = np.asarray(xc, ft)
    Hc, Wc, C = xc.shape
    H = Ul.shape[1]
    dxc = np.zeros((Hc, Wc, C), ft)
    dWx, dUl, dUu, db = (np.zeros_like(a) for a in (Wx, Ul, Uu, b))
    for d in range(4):
        sy, sx = DIRS[d]
        dh_acc = np.array(dhd[d], ft)
        dc_acc = np.zeros((Hc, Wc, H), ft)
        for (Y, X, VL, VU) in reversed(diagonals(rects, d)):
            m = len(Y)
            hl = np.zeros((m, H), ft); cl = np.zeros((m, H), ft)
            hu = np.zeros((m, H), ft); cu = np.zeros((m, H), ft)
            hl[VL] = hd[d, Y[VL], X[VL] - sx]
            cl[VL] = cd[d, Y[VL], X[VL] - sx]
            hu[VU] = hd[d, Y[VU] - sy, X[VU]]
            cu[VU] = cd[d, Y[VU] - sy, X[VU]]
            gates = gd[d, Y, X]
            da, dc, fl, fu = _cell_grad(dh_acc[Y, X], dc_acc[Y, X], gates, cd[d, Y, X], cl, cu, H, num)
            # the left predecessors of distinct cells are distinct, likewise the upper ones
            dh_acc[Y[VL], X[VL] - sx] += da[VL] @ Ul[d].T
            dc_acc[Y[VL], X[VL] - sx] += dc[VL] * fl[VL]
            dh_acc[Y[VU] - sy, X[VU]] += da[VU] @ Uu[d].T
            dc_acc[Y[VU] - sy, X[VU]] += dc[VU] * fu[VU]
            xv = xc[Y, X]
            dWx[d] += xv.T @ da
            dUl[d] += hl.T @ da
            dUu[d] += hu.T @ da
            db[d] += da.sum(axis=0)
            dxc[Y, X] += da @ Wx[d].T
    return dxc, dWx, dUl, dUu, db


# ----------------------------------------------------------------------------------------------
# whole layer on a packed canvas: per-example inputs in, per-example outputs out
# ----------------------------------------------------------------------------------------------

def layer_forward(layout, xs: Sequence[np.ndarray], P, brute=False, num=F64):
    """Scatter -> 4-direction forward -> (direction sum, un-pack).

    Returns (ys, cache) with ys[e] [h][w][H]. ``num`` applies to the per-diagonal form."""
    from .canvas import scatter, dirsum_unpack
    xc = scatter(layout, xs)
    if brute:
        hd, cd, gd = forward_canvas_brute(xc, layout.eid, layout.border, P)
    else:
        hd, cd, gd = forward_vec(xc, layout.rects, P, num)
    return dirsum_unpack(layout, hd), (xc, hd, cd, gd)


def layer_backward(layout, P, cache, dys: Sequence[np.ndarray] = None, dhd=None, brute=False, num=F64):
    """Backward of layer_forward for per-example output gradients ``dys`` (each
    direction receives the same gradient through the direction sum), or for a
    per-direction canvas gradient ``dhd`` [4][Hc][Wc][H].

    Returns (dxs, dWx, dUl, dUu, db)."""
    from .canvas import scatter, unpack
    xc, hd, cd, gd = cache
    if dhd is None:
        dyc = scatter(layout, dys)
        dhd = np.broadcast_to(dyc, (4,) + dyc.shape)
    if brute:
        res = backward_canvas_brute(xc, layout.eid, layout.border, P, hd, cd, gd, dhd)
    else:
        res = backward_vec(xc, layout.rects, P, hd, cd, gd, dhd, num)
    return (unpack(layout, res[0]),) + tuple(res[1:])
