"""4-direction 2D Leaky-LP layer, forward and 2D BPTT, oracle form (test infrastructure only).

What is computed
----------------
"No Padding Please", §III and Figure 4(b): the Leaky LP cell is a stable
variant of the 2D MDLSTM cell. Where the plain cell adds its two predecessor
memory states through two forget gates (whose sum can exceed one, so the
state can grow without bound), a lambda gate forms a weighted sum of the two
predecessor states with weights that sum to one. The pages use a variant in
which the two output gates take the previous memory state as their memory
input instead of the newly computed one. §IX-A counts the matrices: five for
each of the two predecessor hidden states H1, H2 and three for each of the two
predecessor memory states S1, S2. The figure with the equations was lost and
the cited paper [10] is not at hand, so the cell below is a reading of those
statements (the pages fix no more):

    a    = x.Wx + b + h_l.Ul + h_u.Uu                  (5H: f, lam, o1, o2, g)
    a[lam, o1, o2] += s_l.Vl + s_u.Vu                  (3H: the memory-state projections)
    f, lam, o1, o2 = sigmoid(.),  g = tanh(.)
    sbar = lam * s_l + (1 - lam) * s_u                 (lambda gate: a convex combination)
    s    = f * sbar + (1 - f) * g                      (leaky: a convex combination again)
    h    = o1 * tanh(s) + o2 * s                       (the two output gates)

Every state is a convex combination of earlier states and g in (-1, 1), so
|s| < 1 everywhere: the cell is stable by construction. A predecessor outside
the example reads as (h, s) = (0, 0) (§V's mask), as for the plain cell.
Directions, the direction sum and the layout are those of oracle.mdlstm.

Backward (2D BPTT, derived by hand, reverse topological order):

    ts = tanh(s);  ds = ds_in + dh*(o2 + o1*(1 - ts^2))
    da = [ds*(sbar - g)*f(1-f), dsbar*(s_l - s_u)*lam(1-lam), dh*ts*o1(1-o1), dh*s*o2(1-o2), ds*(1-f)*(1-g^2)]
         with dsbar = ds*f
    left  predecessor: dh += da.Ul^T;  ds += dsbar*lam     + da[lam,o1,o2].Vl^T
    upper predecessor: dh += da.Uu^T;  ds += dsbar*(1-lam) + da[lam,o1,o2].Vu^T
    dWx += x^T da, dUl += h_l^T da, dUu += h_u^T da, db += da,
    dVl += s_l^T da[lam,o1,o2], dVu += s_u^T da[lam,o1,o2], dx += da.Wx^T

Forms: ``forward_canvas_brute`` / ``backward_canvas_brute`` scan the canvas
cell by cell (the definition); ``forward_vec`` / ``backward_vec`` take one
local anti-diagonal of every example at a time. All arithmetic in float64.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .mdlstm import DIRS, _pred_bits, _scan, diagonals

GATES = ("f", "lam", "o1", "o2", "g")  # order along the 5H axis; lam, o1, o2 take the memory states


def _p64(P):
    """P: Wx[d][C][5H], Ul, Uu [d][H][5H], b [d][5H] (gates f, lam, o1, o2, g), Vl, Vu [d][H][3H] (lam, o1, o2)."""
    return tuple(np.asarray(a, np.float64) for a in (P.Wx, P.Ul, P.Uu, P.b, P.Vl, P.Vu))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _cell(xv, hl, sl, hu, su, Wx, Ul, Uu, b, Vl, Vu, H):
    a = xv @ Wx + b + hl @ Ul + hu @ Uu
    a[..., H:4 * H] = a[..., H:4 * H] + sl @ Vl + su @ Vu
    f = sigmoid(a[..., 0:H])
    lam = sigmoid(a[..., H:2 * H])
    o1 = sigmoid(a[..., 2 * H:3 * H])
    o2 = sigmoid(a[..., 3 * H:4 * H])
    g = np.tanh(a[..., 4 * H:5 * H])
    sbar = lam * sl + (1.0 - lam) * su
    s = f * sbar + (1.0 - f) * g
    h = o1 * np.tanh(s) + o2 * s
    return h, s, np.concatenate([f, lam, o1, o2, g], axis=-1)


def _cell_grad(dh, ds_in, gates, s, sl, su, H):
    f, lam, o1, o2, g = (gates[..., k * H:(k + 1) * H] for k in range(5))
    ts = np.tanh(s)
    ds = ds_in + dh * (o2 + o1 * (1.0 - ts * ts))
    sbar = lam * sl + (1.0 - lam) * su
    dsbar = ds * f
    da = np.concatenate([ds * (sbar - g) * f * (1.0 - f),
                         dsbar * (sl - su) * lam * (1.0 - lam),
                         dh * ts * o1 * (1.0 - o1),
                         dh * s * o2 * (1.0 - o2),
                         ds * (1.0 - f) * (1.0 - g * g)], axis=-1)
    return da, dsbar * lam, dsbar * (1.0 - lam)


# ---------------------------------------------------------------------------------------------- definition

def forward_canvas_brute(xc, eid, border, P):
    """xc [Hc][Wc][C] -> (h_dirs, s_dirs, gates), each [4][Hc][Wc][.]; zero where eid < 0."""
    Wx, Ul, Uu, b, Vl, Vu = _p64(P)
    xc = np.asarray(xc, np.float64)
    Hc, Wc, _ = xc.shape
    H = Ul.shape[1]
    hd = np.zeros((4, Hc, Wc, H))
    sd = np.zeros((4, Hc, Wc, H))
    gd = np.zeros((4, Hc, Wc, 5 * H))
    zero = np.zeros(H)
    for d in range(4):
        sy, sx = DIRS[d]
        lbit, ubit = _pred_bits(d)
        for (y, x) in _scan(Hc, Wc, d):
            if eid[y, x] < 0:
                continue
            hl, sl = (hd[d, y, x - sx], sd[d, y, x - sx]) if border[y, x] & lbit else (zero, zero)
            hu, su = (hd[d, y - sy, x], sd[d, y - sy, x]) if border[y, x] & ubit else (zero, zero)
            h, s, g = _cell(xc[y, x], hl, sl, hu, su, Wx[d], Ul[d], Uu[d], b[d], Vl[d], Vu[d], H)
            hd[d, y, x], sd[d, y, x], gd[d, y, x] = h, s, g
    return hd, sd, gd


def backward_canvas_brute(xc, eid, border, P, hd, sd, gd, dhd):
    """Reverse scan; dhd [4][Hc][Wc][H] = dL/dh per direction. Returns (dxc, dWx, dUl, dUu, db, dVl, dVu)."""
    Wx, Ul, Uu, b, Vl, Vu = _p64(P)
    xc = np.asarray(xc, np.float64)
    Hc, Wc, C = xc.shape
    H = Ul.shape[1]
    dxc = np.zeros((Hc, Wc, C))
    grads = [np.zeros_like(a) for a in (Wx, Ul, Uu, b, Vl, Vu)]
    zero = np.zeros(H)
    for d in range(4):
        sy, sx = DIRS[d]
        lbit, ubit = _pred_bits(d)
        dh_acc = np.array(dhd[d], np.float64)
        ds_acc = np.zeros((Hc, Wc, H))
        for (y, x) in _scan(Hc, Wc, d, reverse=True):
            if eid[y, x] < 0:
                continue
            vl, vu = bool(border[y, x] & lbit), bool(border[y, x] & ubit)
            hl, sl = (hd[d, y, x - sx], sd[d, y, x - sx]) if vl else (zero, zero)
            hu, su = (hd[d, y - sy, x], sd[d, y - sy, x]) if vu else (zero, zero)
            da, ds_l, ds_u = _cell_grad(dh_acc[y, x], ds_acc[y, x], gd[d, y, x], sd[d, y, x], sl, su, H)
            da3 = da[H:4 * H]
            if vl:
                dh_acc[y, x - sx] += Ul[d] @ da
                ds_acc[y, x - sx] += ds_l + Vl[d] @ da3
            if vu:
                dh_acc[y - sy, x] += Uu[d] @ da
                ds_acc[y - sy, x] += ds_u + Vu[d] @ da3
            grads[0][d] += np.outer(xc[y, x], da)
            grads[1][d] += np.outer(hl, da)
            grads[2][d] += np.outer(hu, da)
            grads[3][d] += da
            grads[4][d] += np.outer(sl, da3)
            grads[5][d] += np.outer(su, da3)
            dxc[y, x] += Wx[d] @ da
    return (dxc,) + tuple(grads)


# ---------------------------------------------------------------------------------------------- per diagonal

def forward_vec(xc, rects, P):
    """Same as forward_canvas_brute, one local diagonal at a time."""
    Wx, Ul, Uu, b, Vl, Vu = _p64(P)
    xc = np.asarray(xc, np.float64)
    Hc, Wc, _ = xc.shape
    H = Ul.shape[1]
    hd = np.zeros((4, Hc, Wc, H))
    sd = np.zeros((4, Hc, Wc, H))
    gd = np.zeros((4, Hc, Wc, 5 * H))
    for d in range(4):
        sy, sx = DIRS[d]
        for (Y, X, VL, VU) in diagonals(rects, d):
            m = len(Y)
            hl, sl, hu, su = (np.zeros((m, H)) for _ in range(4))
            hl[VL], sl[VL] = hd[d, Y[VL], X[VL] - sx], sd[d, Y[VL], X[VL] - sx]
            hu[VU], su[VU] = hd[d, Y[VU] - sy, X[VU]], sd[d, Y[VU] - sy, X[VU]]
            h, s, g = _cell(xc[Y, X], hl, sl, hu, su, Wx[d], Ul[d], Uu[d], b[d], Vl[d], Vu[d], H)
            hd[d, Y, X], sd[d, Y, X], gd[d, Y, X] = h, s, g
    return hd, sd, gd


def backward_vec(xc, rects, P, hd, sd, gd, dhd):
    """Same as backward_canvas_brute, one local diagonal at a time, in reverse."""
    Wx, Ul, Uu, b, Vl, Vu = _p64(P)
    xc = np.asarray(xc, np.float64)
    Hc, Wc, C = xc.shape
    H = Ul.shape[1]
    dxc = np.zeros((Hc, Wc, C))
    grads = [np.zeros_like(a) for a in (Wx, Ul, Uu, b, Vl, Vu)]
    for d in range(4):
        sy, sx = DIRS[d]
        dh_acc = np.array(dhd[d], np.float64)
        ds_acc = np.zeros((Hc, Wc, H))
        for (Y, X, VL, VU) in reversed(diagonals(rects, d)):
            m = len(Y)
            hl, sl, hu, su = (np.zeros((m, H)) for _ in range(4))
            hl[VL], sl[VL] = hd[d, Y[VL], X[VL] - sx], sd[d, Y[VL], X[VL] - sx]
            hu[VU], su[VU] = hd[d, Y[VU] - sy, X[VU]], sd[d, Y[VU] - sy, X[VU]]
            da, ds_l, ds_u = _cell_grad(dh_acc[Y, X], ds_acc[Y, X], gd[d, Y, X], sd[d, Y, X], sl, su, H)
            da3 = da[:, H:4 * H]
            # the left predecessors of distinct cells are distinct, likewise the upper ones
            dh_acc[Y[VL], X[VL] - sx] += da[VL] @ Ul[d].T
            ds_acc[Y[VL], X[VL] - sx] += ds_l[VL] + da3[VL] @ Vl[d].T
            dh_acc[Y[VU] - sy, X[VU]] += da[VU] @ Uu[d].T
            ds_acc[Y[VU] - sy, X[VU]] += ds_u[VU] + da3[VU] @ Vu[d].T
            grads[0][d] += xc[Y, X].T @ da
            grads[1][d] += hl.T @ da
            grads[2][d] += hu.T @ da
            grads[3][d] += da.sum(axis=0)
            grads[4][d] += sl.T @ da3
            grads[5][d] += su.T @ da3
            dxc[Y, X] += da @ Wx[d].T
    return (dxc,) + tuple(grads)


# ---------------------------------------------------------------------------------------------- whole layer

def layer_forward(layout, xs: Sequence[np.ndarray], P, brute=False):
    """Scatter -> 4-direction Leaky-LP forward -> (direction sum, un-pack). Returns (ys, cache)."""
    from .canvas import scatter, dirsum_unpack
    xc = scatter(layout, xs)
    if brute:
        hd, sd, gd = forward_canvas_brute(xc, layout.eid, layout.border, P)
    else:
        hd, sd, gd = forward_vec(xc, layout.rects, P)
    return dirsum_unpack(layout, hd), (xc, hd, sd, gd)


def layer_backward(layout, P, cache, dys: Sequence[np.ndarray] = None, dhd=None, brute=False):
    """Backward of layer_forward. Returns (dxs, dWx, dUl, dUu, db, dVl, dVu)."""
    from .canvas import scatter, unpack
    xc, hd, sd, gd = cache
    if dhd is None:
        dyc = scatter(layout, dys)
        dhd = np.broadcast_to(dyc, (4,) + dyc.shape)
    if brute:
        res = backward_canvas_brute(xc, layout.eid, layout.border, P, hd, sd, gd, dhd)
    else:
        res = backward_vec(xc, layout.rects, P, hd, sd, gd, dhd)
    return (unpack(layout, res[0]),) + tuple(res[1:])
