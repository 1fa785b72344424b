"""Pins of the oracle MDLSTM forward and 2D BPTT.

None of the pages prints an MDLSTM activation or gradient, so the oracle is
pinned by what the mathematics fixes:
  * a height-1 (width-1) example reduces each direction to a 1-D LSTM along
    its row (column): compared with torch.nn.LSTM, forward and autograd;
  * with zero recurrent weights the memory state has a closed form: a sum over
    source cells of (i*g) times the sum over monotone lattice paths of the
    product of the receiving cells' forget gates; with constant gates the path
    sum is a binomial double sum;
  * all-zero parameters give zero output;
  * flipping the image maps direction d onto direction 0 ("No Padding Please"
    §III: four MDLSTMs, one per scanning direction);
  * packed == alone: on the canvas, an example's outputs do not depend on its
    neighbours (the binary mask of §V blocks separator and padding state);
  * central finite differences of the forward give the backward;
  * weight gradients of a packed batch are the sum of per-example ones;
  * the per-diagonal form equals the per-cell scan.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import canvas, mdlstm, pack
from workloads import LayerParams, make_workload, random_layer, random_images, cotangent

# the direction numbering (a convention of this library, written out here rather than imported):
# d0 scans from the top-left, d1 from the top-right, d2 from the bottom-left, d3 from the bottom-right
DIRS = ((+1, +1), (+1, -1), (-1, +1), (-1, -1))


def _p(seed, C, H, scale=0.1):
    return random_layer(seed, C, H, scale)


def _alone(x, P):
    return mdlstm.forward_example_brute(x, P)


# ------------------------------------------------------------------------------------ reductions

def _torch_lstm_from(P, d, H, axis):
    """torch.nn.LSTM (gate rows i, f, g, o) built from direction d of the 2D cell.

    axis 'x': forget gate = f_left, recurrent weights = Ul; axis 'y': f_up, Uu."""
    C = P.Wx.shape[1]
    lstm = torch.nn.LSTM(C, H, batch_first=True).double()
    fcol = slice(H, 2 * H) if axis == "x" else slice(2 * H, 3 * H)
    U = P.Ul if axis == "x" else P.Uu
    cols = [slice(0, H), fcol, slice(4 * H, 5 * H), slice(3 * H, 4 * H)]   # i, f, g, o
    with torch.no_grad():
        lstm.weight_ih_l0.copy_(torch.tensor(np.concatenate([np.asarray(P.Wx[d][:, c], np.float64).T for c in cols])))
        lstm.weight_hh_l0.copy_(torch.tensor(np.concatenate([np.asarray(U[d][:, c], np.float64).T for c in cols])))
        lstm.bias_ih_l0.copy_(torch.tensor(np.concatenate([np.asarray(P.b[d][c], np.float64) for c in cols])))
        lstm.bias_hh_l0.zero_()
    return lstm, cols


@pytest.mark.parametrize("axis", ["x", "y"])
def test_reduces_to_1d_lstm(axis):
    H, C = 5, 3
    P = _p(11, C, H, scale=0.6)
    L = 9
    x = np.random.default_rng(3).random((1, L, C) if axis == "x" else (L, 1, C))
    hd = _alone(x, P)
    for d, (sy, sx) in enumerate(DIRS):
        step = sx if axis == "x" else sy
        order = list(range(L)) if step > 0 else list(range(L - 1, -1, -1))
        seq = x[0, order, :] if axis == "x" else x[order, 0, :]
        lstm, _ = _torch_lstm_from(P, d, H, axis)
        out, _ = lstm(torch.tensor(seq[None]))
        ref = out[0].detach().numpy()
        got = hd[d, 0, order, :] if axis == "x" else hd[d, order, 0, :]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("axis", ["x", "y"])
def test_backward_matches_torch_autograd_1d(axis):
    H, C = 4, 2
    P = _p(12, C, H, scale=0.6)
    L = 7
    x = np.random.default_rng(4).random((1, L, C) if axis == "x" else (L, 1, C))
    R = np.random.default_rng(5).standard_normal((4, x.shape[0], x.shape[1], H))
    lay = pack.pack_alg1([x.shape[0]], [x.shape[1]], 1, 0)
    xc = canvas.scatter(lay, [x])
    hd, cd, gd = mdlstm.forward_vec(xc, lay.rects, P)
    for d, (sy, sx) in enumerate(DIRS):
        dhd = np.zeros_like(R)
        dhd[d] = R[d]
        dxc, dWx, dUl, dUu, db = mdlstm.backward_vec(xc, lay.rects, P, hd, cd, gd, dhd)
        step = sx if axis == "x" else sy
        order = list(range(L)) if step > 0 else list(range(L - 1, -1, -1))
        seq = torch.tensor((x[0, order, :] if axis == "x" else x[order, 0, :])[None], requires_grad=True)
        lstm, cols = _torch_lstm_from(P, d, H, axis)
        out, _ = lstm(seq)
        r = R[d, 0, order, :] if axis == "x" else R[d, order, 0, :]
        (out[0] * torch.tensor(r)).sum().backward()
        gx = seq.grad[0].numpy()
        got_dx = dxc[0, order, :] if axis == "x" else dxc[order, 0, :]
        np.testing.assert_allclose(got_dx, gx, rtol=1e-10, atol=1e-12)
        U = dUl if axis == "x" else dUu
        Uother = dUu if axis == "x" else dUl
        gih = lstm.weight_ih_l0.grad.numpy()
        ghh = lstm.weight_hh_l0.grad.numpy()
        gb = lstm.bias_ih_l0.grad.numpy()
        for k, c in enumerate(cols):
            np.testing.assert_allclose(dWx[d][:, c].T, gih[k * H:(k + 1) * H], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(U[d][:, c].T, ghh[k * H:(k + 1) * H], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(db[d][c], gb[k * H:(k + 1) * H], rtol=1e-10, atol=1e-12)
        assert np.all(Uother[d] == 0)   # the other predecessor never exists
        other_f = slice(2 * H, 3 * H) if axis == "x" else slice(H, 2 * H)
        assert np.all(dWx[d][:, other_f] == 0) and np.all(db[d][other_f] == 0)


# ------------------------------------------------------------------------------------ closed forms

def _gates_from_bias(b, H):
    sig = lambda z: 1 / (1 + np.exp(-z))
    return (sig(b[0:H]), sig(b[H:2 * H]), sig(b[2 * H:3 * H]), sig(b[3 * H:4 * H]), np.tanh(b[4 * H:5 * H]))


def _local(d, h, w, y, x):
    sy, sx = DIRS[d]
    return (y if sy > 0 else h - 1 - y), (x if sx > 0 else w - 1 - x)


def test_constant_gates_binomial_closed_form():
    H, C, h, w = 3, 2, 5, 6
    rng = np.random.default_rng(7)
    P = LayerParams(np.zeros((4, C, 5 * H)), np.zeros((4, H, 5 * H)), np.zeros((4, H, 5 * H)),
                    rng.normal(0, 1.0, (4, 5 * H)))
    x = rng.random((h, w, C))
    hd = _alone(x, P)
    for d in range(4):
        i, fl, fu, o, g = _gates_from_bias(np.asarray(P.b[d], np.float64), H)
        for y in range(h):
            for xx in range(w):
                a, bb = _local(d, h, w, y, xx)
                s = sum(math.comb(p + q, p) * fu ** p * fl ** q for p in range(a + 1) for q in range(bb + 1))
                c = i * g * s
                np.testing.assert_allclose(hd[d, y, xx], o * np.tanh(c), rtol=1e-12, atol=1e-14)


def _paths(a0, b0, a1, b1):
    """All monotone lattice paths from (a0,b0) to (a1,b1) as lists of (step, receiving cell)."""
    if (a0, b0) == (a1, b1):
        yield []
        return
    if a0 < a1:
        for rest in _paths(a0 + 1, b0, a1, b1):
            yield [("up", (a0 + 1, b0))] + rest
    if b0 < b1:
        for rest in _paths(a0, b0 + 1, a1, b1):
            yield [("left", (a0, b0 + 1))] + rest


def test_zero_recurrence_path_enumeration():
    """Ul = Uu = 0: gates depend on the pixel only; c is a sum over source cells and paths."""
    H, C, h, w = 2, 3, 4, 4
    P0 = _p(21, C, H, scale=1.0)
    P = LayerParams(P0.Wx, np.zeros_like(P0.Ul), np.zeros_like(P0.Uu), P0.b)
    x = np.random.default_rng(8).random((h, w, C))
    hd = _alone(x, P)
    sig = lambda z: 1 / (1 + np.exp(-z))
    for d in range(4):
        sy, sx = DIRS[d]
        # gates at direction-local coordinates
        G = {}
        for y in range(h):
            for xx in range(w):
                a = x[y, xx] @ np.asarray(P.Wx[d], np.float64) + np.asarray(P.b[d], np.float64)
                G[_local(d, h, w, y, xx)] = (sig(a[:H]), sig(a[H:2 * H]), sig(a[2 * H:3 * H]),
                                            sig(a[3 * H:4 * H]), np.tanh(a[4 * H:]))
        for y in range(h):
            for xx in range(w):
                A, B = _local(d, h, w, y, xx)
                c = np.zeros(H)
                for a0 in range(A + 1):
                    for b0 in range(B + 1):
                        i0, _, _, _, g0 = G[(a0, b0)]
                        tot = np.zeros(H)
                        for path in _paths(a0, b0, A, B):
                            prod = np.ones(H)
                            for step, cell in path:
                                prod = prod * (G[cell][1] if step == "left" else G[cell][2])
                            tot = tot + prod
                        c = c + i0 * g0 * tot
                o = G[(A, B)][3]
                np.testing.assert_allclose(hd[d, y, xx], o * np.tanh(c), rtol=1e-12, atol=1e-14)


def test_direction_start_corners():
    """Each direction's first cell has no predecessor: h = o * tanh(i * g) from its own pixel."""
    H, C, h, w = 3, 2, 4, 5
    P = _p(51, C, H, scale=1.0)
    x = np.random.default_rng(2).random((h, w, C))
    hd = _alone(x, P)
    corners = {0: (0, 0), 1: (0, w - 1), 2: (h - 1, 0), 3: (h - 1, w - 1)}
    sig = lambda z: 1 / (1 + np.exp(-z))
    for d, (y, xx) in corners.items():
        a = x[y, xx] @ np.asarray(P.Wx[d], np.float64) + np.asarray(P.b[d], np.float64)
        ref = sig(a[3 * H:4 * H]) * np.tanh(sig(a[:H]) * np.tanh(a[4 * H:]))
        np.testing.assert_allclose(hd[d, y, xx], ref, rtol=1e-13)
        for (y2, x2) in corners.values():
            if (y2, x2) != (y, xx):
                a2 = x[y2, x2] @ np.asarray(P.Wx[d], np.float64) + np.asarray(P.b[d], np.float64)
                ref2 = sig(a2[3 * H:4 * H]) * np.tanh(sig(a2[:H]) * np.tanh(a2[4 * H:]))
                assert np.max(np.abs(hd[d, y2, x2] - ref2)) > 1e-6


def test_zero_parameters_give_zero():
    H, C = 3, 2
    P = LayerParams(np.zeros((4, C, 5 * H)), np.zeros((4, H, 5 * H)), np.zeros((4, H, 5 * H)), np.zeros((4, 5 * H)))
    x = np.random.default_rng(1).random((4, 5, C))
    assert np.all(_alone(x, P) == 0)


def test_flip_symmetry():
    H, C, h, w = 3, 2, 4, 6
    P = _p(31, C, H, scale=0.8)
    x = np.random.default_rng(9).random((h, w, C))
    hd = _alone(x, P)
    for d, (sy, sx) in enumerate(DIRS):
        xf = x[::sy, ::sx]
        Pd = LayerParams(*(np.repeat(np.asarray(a)[d:d + 1], 4, axis=0) for a in (P.Wx, P.Ul, P.Uu, P.b)))
        h0 = _alone(xf, Pd)[0]
        np.testing.assert_allclose(hd[d], h0[::sy, ::sx], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------------ canvas forms

def _tiny(seed=0):
    wl = make_workload("tiny", seed)
    lay = pack.pack_alg1(wl.heights, wl.widths, wl.canvas_w_min[0], wl.sep)
    return wl, lay


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_equals_alone(seed):
    wl, lay = _tiny(seed)
    P = wl.layers[0]
    xc = canvas.scatter(lay, wl.xs)
    hd, cd, gd = mdlstm.forward_canvas_brute(xc, lay.eid, lay.border, P)
    assert np.all(hd[:, lay.eid < 0] == 0)
    for e, x in enumerate(wl.xs):
        y0, x0, h, w = lay.rects[e]
        np.testing.assert_allclose(hd[:, y0:y0 + h, x0:x0 + w], _alone(x, P), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("seed", [0, 3])
def test_vec_equals_brute(seed):
    wl, lay = _tiny(seed)
    P = wl.layers[0]
    xc = canvas.scatter(lay, wl.xs)
    b = mdlstm.forward_canvas_brute(xc, lay.eid, lay.border, P)
    v = mdlstm.forward_vec(xc, lay.rects, P)
    for u, w_ in zip(b, v):
        np.testing.assert_allclose(w_, u, rtol=1e-12, atol=1e-14)
    R = np.random.default_rng(seed).standard_normal(b[0].shape)
    gb = mdlstm.backward_canvas_brute(xc, lay.eid, lay.border, P, *b, R)
    gv = mdlstm.backward_vec(xc, lay.rects, P, *v, R)
    for u, w_ in zip(gb, gv):
        np.testing.assert_allclose(w_, u, rtol=1e-11, atol=1e-13)


def _loss_grads(lay, xs, P, dys):
    ys, cache = mdlstm.layer_forward(lay, xs, P)
    return mdlstm.layer_backward(lay, P, cache, dys=dys)


def test_finite_differences_all_entries():
    """Central differences for every parameter and every pixel of a small packed batch."""
    heights, widths = [3, 2, 3], [4, 3, 2]
    H, C = 3, 2
    lay = pack.pack_alg1(heights, widths, 6, 1)
    P = _p(41, C, H, scale=0.7)
    P = LayerParams(*(np.asarray(a, np.float64) for a in (P.Wx, P.Ul, P.Uu, P.b)))
    xs = [np.asarray(x, np.float64) for x in random_images(5, heights, widths, C)]
    dys = [np.asarray(r, np.float64) for r in cotangent(5, heights, widths, H)]

    def loss(P_, xs_):
        ys, _ = mdlstm.layer_forward(lay, xs_, P_)
        return sum(float(np.sum(y * r)) for y, r in zip(ys, dys))

    dxs, dWx, dUl, dUu, db = _loss_grads(lay, xs, P, dys)
    eps = 1e-6
    for name, g in (("Wx", dWx), ("Ul", dUl), ("Uu", dUu), ("b", db)):
        arr = getattr(P, name)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps; lp = loss(P, xs)
            arr[idx] = old - eps; lm = loss(P, xs)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 + 1e-6 * abs(g[idx]), (name, idx, fd, g[idx])
    for e, x in enumerate(xs):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps; lp = loss(P, xs)
            x[idx] = old - eps; lm = loss(P, xs)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - dxs[e][idx]) <= 1e-7 + 1e-6 * abs(dxs[e][idx]), (e, idx)


def test_finite_differences_tiny_workload_sample():
    wl, lay = _tiny(1)
    P = LayerParams(*(np.asarray(a, np.float64) for a in (wl.layers[0].Wx, wl.layers[0].Ul,
                                                          wl.layers[0].Uu, wl.layers[0].b)))
    xs = [np.asarray(x, np.float64) for x in wl.xs]
    ones = [np.ones(x.shape[:2] + (wl.H,)) for x in xs]   # sum-of-outputs loss

    def loss(P_):
        ys, _ = mdlstm.layer_forward(lay, xs, P_)
        return sum(float(np.sum(y)) for y in ys)

    _, dWx, dUl, dUu, db = _loss_grads(lay, xs, P, ones)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, g in (("Wx", dWx), ("Ul", dUl), ("Uu", dUu), ("b", db)):
        arr = getattr(P, name)
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps; lp = loss(P)
            arr[idx] = old - eps; lm = loss(P)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 + 1e-6 * abs(g[idx]), (name, idx, fd, g[idx])


def test_gradient_additivity_and_packed_dx():
    wl, lay = _tiny(2)
    P = wl.layers[0]
    dys = cotangent(2, wl.heights, wl.widths, wl.H)
    dxs, dWx, dUl, dUu, db = _loss_grads(lay, wl.xs, P, dys)
    acc = [np.zeros_like(a, dtype=np.float64) for a in (dWx, dUl, dUu, db)]
    for e in range(wl.n):
        h, w = int(wl.heights[e]), int(wl.widths[e])
        single = pack.pack_alg1([h], [w], 1, 0)
        r = _loss_grads(single, [wl.xs[e]], P, [dys[e]])
        np.testing.assert_allclose(dxs[e], r[0][0], rtol=1e-12, atol=1e-14)
        for k in range(4):
            acc[k] += r[1 + k]
    for a, b in zip(acc, (dWx, dUl, dUu, db)):
        np.testing.assert_allclose(b, a, rtol=1e-11, atol=1e-13)


def test_zero_cotangent():
    wl, lay = _tiny(0)
    zeros = [np.zeros(x.shape[:2] + (wl.H,)) for x in wl.xs]
    res = _loss_grads(lay, wl.xs, wl.layers[0], zeros)
    assert all(np.all(x == 0) for x in res[0])
    assert all(np.all(a == 0) for a in res[1:])


def test_padded_mode_is_zero_padded_images():
    wl = make_workload("tiny", 4)
    lay = pack.pack_padded(wl.heights, wl.widths)
    P = wl.layers[0]
    ys, _ = mdlstm.layer_forward(lay, wl.xs, P)
    Hm, Wm = int(max(wl.heights)), int(max(wl.widths))
    for e, x in enumerate(wl.xs):
        h, w = x.shape[:2]
        xp = np.zeros((Hm, Wm, x.shape[2]))
        xp[:h, :w] = x
        ref = _alone(xp, P).sum(axis=0)[:h, :w]
        np.testing.assert_allclose(ys[e], ref, rtol=1e-12, atol=1e-14)
