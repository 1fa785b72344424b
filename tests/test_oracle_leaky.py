"""Pins of the Leaky-LP oracle (oracle/leaky.py).

The pages print no activation of the cell and its defining figure is lost, so
the oracle is pinned by what the mathematics fixes for the cell as read:
  * with the lambda gate held at 1 and the output gates at (0, 1) by saturated
    biases, a one-row example reduces to a gated recurrent unit whose reset
    gate is held at 1 (the state update f*s_prev + (1-f)*g is the GRU's
    update with z = f, n = g): torch.nn.GRU, forward and autograd;
  * with constant gates, s at direction-local cell (a, b) is
    (1-f) g sum_{i<=a, j<=b} C(i+j, i) (f(1-lam))^i (f lam)^j (monotone lattice
    paths from each source cell, weight f*lam per step along the row and
    f*(1-lam) per step across rows);
  * the memory state stays inside (-1, 1) for any weights (every update is a
    convex combination), where the plain cell's grows without bound;
  * central finite differences give the backward (every parameter, Vl and Vu
    included, and every input pixel);
  * packed == alone, flip symmetry, the per-diagonal form equals the per-cell
    scan, additivity of the weight gradients.
"""

import math

import numpy as np
import pytest
import torch

from oracle import canvas, leaky, mdlstm, pack
from workloads import LeakyLayerParams, cotangent, random_images, random_leaky_layer

DIRS = ((+1, +1), (+1, -1), (-1, +1), (-1, -1))
BIG = 800.0  # a bias whose sigmoid is exactly 1 (or, negated, exactly 0) in float64


def _layer(h, w, xs, P, cw=None, dys=None, brute=False):
    lay = pack.pack(h, w, cw or max(max(w), 8), 1, "packed")
    ys, cache = leaky.layer_forward(lay, xs, P, brute=brute)
    res = leaky.layer_backward(lay, P, cache, dys=dys, brute=brute) if dys is not None else None
    return lay, ys, cache, res


def test_vec_equals_brute():
    h, w = [5, 3, 7, 2], [6, 9, 4, 8]
    P = random_leaky_layer(1, 3, 5)
    xs = random_images(2, h, w, 3)
    dys = cotangent(3, h, w, 5)
    _, yb, cb, rb = _layer(h, w, xs, P, dys=dys, brute=True)
    _, yv, cv, rv = _layer(h, w, xs, P, dys=dys)
    for a, b in zip(cb[1:], cv[1:]):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    for a, b in zip(rb[1:], rv[1:]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    for a, b in zip(rb[0], rv[0]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_packed_equals_alone_and_additivity():
    h, w = [4, 6, 3], [7, 5, 9]
    P = random_leaky_layer(4, 2, 4)
    xs = random_images(5, h, w, 2)
    dys = cotangent(6, h, w, 4)
    _, ys, _, res = _layer(h, w, xs, P, cw=24, dys=dys)
    dW = [np.zeros_like(a) for a in res[1:]]
    for e in range(3):
        _, ye, _, re = _layer([h[e]], [w[e]], [xs[e]], P, dys=[dys[e]])
        np.testing.assert_allclose(ys[e], ye[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(res[0][e], re[0][0], rtol=0, atol=1e-13)
        dW = [a + b for a, b in zip(dW, re[1:])]
    for a, b in zip(res[1:], dW):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_finite_differences_every_entry():
    h, w, C, H = [3, 2], [4, 5], 2, 3
    P = random_leaky_layer(7, C, H, scale=0.5)
    xs = random_images(8, h, w, C)
    R = cotangent(9, h, w, H)
    lay = pack.pack(h, w, 8, 1, "packed")

    def loss(Pp, xsp):
        ys, _ = leaky.layer_forward(lay, xsp, Pp)
        return sum(float(np.sum(r * y)) for r, y in zip(R, ys))

    ys, cache = leaky.layer_forward(lay, xs, P)
    res = leaky.layer_backward(lay, P, cache, dys=R)
    eps = 1e-6
    names = ("Wx", "Ul", "Uu", "b", "Vl", "Vu")
    P64 = LeakyLayerParams(*(np.asarray(getattr(P, n), np.float64) for n in names))
    for k, n in enumerate(names):
        arr = getattr(P64, n)
        g = res[1 + k]
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(P64, xs)
            arr[idx] = old - eps
            lm = loss(P64, xs)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (n, idx, fd, g[idx])
    xs64 = [np.asarray(x, np.float64) for x in xs]
    for e in range(len(xs)):
        for idx in np.ndindex(xs64[e].shape):
            old = xs64[e][idx]
            xs64[e][idx] = old + eps
            lp = loss(P64, xs64)
            xs64[e][idx] = old - eps
            lm = loss(P64, xs64)
            xs64[e][idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - res[0][e][idx]) <= 1e-6 * max(1.0, abs(fd)), ("x", e, idx)


def _gru_from(P, d, H):
    """torch.nn.GRU (float64) whose update gate is the Leaky-LP f gate and whose candidate is g, reset held at 1."""
    C = P.Wx.shape[1]
    gru = torch.nn.GRU(C, H, batch_first=True).double()
    f, g = slice(0, H), slice(4 * H, 5 * H)
    Wx, Ul, b = (np.asarray(a[d], np.float64) for a in (P.Wx, P.Ul, P.b))
    with torch.no_grad():
        gru.weight_ih_l0.copy_(torch.tensor(np.concatenate([np.zeros((H, C)), Wx[:, f].T, Wx[:, g].T])))
        gru.weight_hh_l0.copy_(torch.tensor(np.concatenate([np.zeros((H, H)), Ul[:, f].T, Ul[:, g].T])))
        gru.bias_ih_l0.copy_(torch.tensor(np.concatenate([np.full(H, BIG), b[f], b[g]])))
        gru.bias_hh_l0.zero_()
    return gru


@pytest.mark.parametrize("d", range(4))
def test_one_row_reduces_to_gru(d):
    C, H, w = 3, 4, 9
    P = random_leaky_layer(11, C, H, scale=0.5)
    b = np.array(P.b, np.float64)
    b[:, H:2 * H] = BIG        # lambda = 1: the left predecessor's state only
    b[:, 2 * H:3 * H] = -BIG   # o1 = 0
    b[:, 3 * H:4 * H] = BIG    # o2 = 1: h = s
    P = LeakyLayerParams(P.Wx, P.Ul, P.Uu, b, P.Vl, P.Vu)
    x = random_images(12, [1], [w], C)[0]
    R = cotangent(13, [1], [w], H)[0]
    with np.errstate(over="ignore"):
        lay = pack.pack([1], [w], w, 1, "packed")
        _, cache = leaky.layer_forward(lay, [x], P)
        hd = cache[1][d, 0]                                        # [w][H] of direction d
        dhd = np.zeros((4, 1, w, H))
        dhd[d, 0] = R
        res = leaky.layer_backward(lay, P, cache, dhd=dhd)
    sx = DIRS[d][1]
    order = slice(None) if sx > 0 else slice(None, None, -1)
    gru = _gru_from(P, d, H)
    xt = torch.tensor(np.ascontiguousarray(np.asarray(x[0], np.float64)[order])[None], requires_grad=True)
    out, _ = gru(xt)
    np.testing.assert_allclose(out[0].detach().numpy(), hd[order], rtol=1e-12, atol=1e-13)
    (out[0] * torch.tensor(np.ascontiguousarray(R[0][order]))).sum().backward()
    np.testing.assert_allclose(xt.grad[0].numpy(), res[0][0][0][order], rtol=1e-10, atol=1e-12)
    f, g = slice(0, H), slice(4 * H, 5 * H)
    gi, gh = gru.weight_ih_l0.grad.numpy(), gru.weight_hh_l0.grad.numpy()
    np.testing.assert_allclose(res[1][d][:, f], gi[H:2 * H].T, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res[1][d][:, g], gi[2 * H:].T, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res[2][d][:, f], gh[H:2 * H].T, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res[2][d][:, g], gh[2 * H:].T, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res[4][d][f], gru.bias_ih_l0.grad.numpy()[H:2 * H], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res[4][d][g], gru.bias_ih_l0.grad.numpy()[2 * H:], rtol=1e-10, atol=1e-12)
    # the saturated gates have zero slope: no gradient reaches their parameters
    assert np.all(res[1][d][:, H:4 * H] == 0) and np.all(res[5][d] == 0) and np.all(res[6][d] == 0)


def test_constant_gates_closed_form():
    C, H, h, w = 2, 3, 4, 5
    rng = np.random.default_rng(14)
    b = rng.normal(0, 1.0, (4, 5 * H))
    z = lambda *s: np.zeros(s)
    P = LeakyLayerParams(z(4, C, 5 * H), z(4, H, 5 * H), z(4, H, 5 * H), b, z(4, H, 3 * H), z(4, H, 3 * H))
    x = random_images(15, [h], [w], C)[0]
    lay = pack.pack([h], [w], w, 1, "packed")
    _, cache = leaky.layer_forward(lay, [x], P)
    sig = lambda v: 1 / (1 + math.exp(-v))
    for d, (sy, sx) in enumerate(DIRS):
        for k in range(H):
            f, lam = sig(b[d, k]), sig(b[d, H + k])
            o1, o2, g = sig(b[d, 2 * H + k]), sig(b[d, 3 * H + k]), math.tanh(b[d, 4 * H + k])
            for a in range(h):
                for bb in range(w):
                    s = (1 - f) * g * sum(math.comb(i + j, i) * (f * (1 - lam)) ** i * (f * lam) ** j
                                          for i in range(a + 1) for j in range(bb + 1))
                    y = a if sy > 0 else h - 1 - a
                    xx = bb if sx > 0 else w - 1 - bb
                    assert abs(cache[2][d, y, xx, k] - s) < 1e-13
                    assert abs(cache[1][d, y, xx, k] - (o1 * math.tanh(s) + o2 * s)) < 1e-13


def test_flip_symmetry():
    C, H = 2, 3
    P = random_leaky_layer(16, C, H)
    x = random_images(17, [5], [6], C)[0]
    lay = pack.pack([5], [6], 6, 1, "packed")
    _, cache = leaky.layer_forward(lay, [x], P)
    for d, (sy, sx) in enumerate(DIRS):
        Pd = LeakyLayerParams(*(np.repeat(np.asarray(a)[d:d + 1], 4, axis=0) for a in (P.Wx, P.Ul, P.Uu, P.b, P.Vl, P.Vu)))
        xf = x[::sy, ::sx]
        _, cf = leaky.layer_forward(lay, [np.ascontiguousarray(xf)], Pd)
        np.testing.assert_allclose(cache[1][d], cf[1][0][::sy, ::sx], rtol=0, atol=1e-14)


def test_state_bounded_where_the_plain_cell_grows():
    """Weights 30x larger than the workloads' (N(0, 3)): the Leaky-LP state stays within [-1, 1] on a 32 x 200
    chain (a saturated tanh(g) rounds to exactly 1), the plain cell's memory state under the same Wx, Ul, Uu, b
    grows far beyond 1 (to about 3e30)."""
    C, H, h, w = 4, 8, 32, 200
    P = random_leaky_layer(18, C, H, scale=3.0)
    x = random_images(19, [h], [w], C)[0]
    lay = pack.pack([h], [w], w, 1, "packed")
    _, cache = leaky.layer_forward(lay, [x], P)
    s, hh = cache[2], cache[1]
    assert np.all(np.abs(s) <= 1.0) and np.all(np.abs(hh) <= 2.0)
    from workloads import LayerParams
    _, pc = mdlstm.layer_forward(lay, [x], LayerParams(P.Wx, P.Ul, P.Uu, P.b))
    assert np.max(np.abs(pc[2])) > 1e3


def test_zero_cotangent_and_zero_parameters():
    h, w, C, H = [3, 4], [5, 2], 2, 3
    P = random_leaky_layer(20, C, H)
    xs = random_images(21, h, w, C)
    zeros = [np.zeros((a, b, H)) for a, b in zip(h, w)]
    _, _, _, res = _layer(h, w, xs, P, dys=zeros)
    assert all(np.all(np.asarray(g) == 0) for g in res[1:]) and all(np.all(d == 0) for d in res[0])
    z = lambda *s: np.zeros(s)
    Pz = LeakyLayerParams(z(4, C, 5 * H), z(4, H, 5 * H), z(4, H, 5 * H), z(4, 5 * H), z(4, H, 3 * H), z(4, H, 3 * H))
    _, ys, _, _ = _layer(h, w, xs, Pz)
    assert all(np.all(y == 0) for y in ys)
