"""Pins of the oracle block-strided convolution and the three-level stack.

"No Padding Please" §V-B states the invariant: the chunked computation equals
the block-strided convolution of each input tensor separately. The
per-example convolution is in turn checked against torch's conv2d (CPU,
float64) with stride equal to the kernel, and the backward against autograd.
The stack is checked end to end with finite differences.
"""

import numpy as np
import pytest
import torch

from oracle import blockconv, stack
from workloads import ConvParams, LayerParams, make_workload, random_layer, random_images, cotangent


def _torch_conv(hd_e, W, b, kh=2, kw=4):
    D, h, w, H = hd_e.shape
    ho, wo = -(-h // kh), -(-w // kw)
    x = np.zeros((1, D * H, ho * kh, wo * kw))
    x[0, :, :h, :w] = np.asarray(hd_e, np.float64).transpose(0, 3, 1, 2).reshape(D * H, h, w)
    Wt = np.asarray(W, np.float64).reshape(W.shape[0], D * H, kh, kw)
    out = torch.nn.functional.conv2d(torch.tensor(x), torch.tensor(Wt), torch.tensor(np.asarray(b, np.float64)),
                                     stride=(kh, kw))
    return out[0].numpy().transpose(1, 2, 0)


def _rand_list(seed, sizes, H):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((4, h, w, H)) for (h, w) in sizes]


SIZES = [(1, 1), (2, 4), (3, 5), (5, 9), (4, 8), (7, 3)]


def test_example_conv_matches_torch():
    H, Cout = 3, 5
    rng = np.random.default_rng(0)
    W = rng.standard_normal((Cout, 4, H, 2, 4))
    b = rng.standard_normal(Cout)
    for hd_e in _rand_list(1, SIZES, H):
        np.testing.assert_allclose(blockconv.conv_example(hd_e, W, b), _torch_conv(hd_e, W, b), rtol=1e-12, atol=1e-12)


def test_chunked_equals_per_example():
    H, Cout = 2, 6
    rng = np.random.default_rng(2)
    W = rng.standard_normal((Cout, 4, H, 2, 4))
    b = rng.standard_normal(Cout)
    lst = _rand_list(3, SIZES, H)
    outs = blockconv.conv_chunked(lst, W, b)
    for hd_e, o in zip(lst, outs):
        np.testing.assert_allclose(o, blockconv.conv_example(hd_e, W, b), rtol=1e-12, atol=1e-12)


def test_chunked_backward_matches_autograd():
    H, Cout = 2, 3
    rng = np.random.default_rng(4)
    W = rng.standard_normal((Cout, 4, H, 2, 4))
    b = rng.standard_normal(Cout)
    lst = _rand_list(5, SIZES, H)
    douts = [rng.standard_normal((-(-h // 2), -(-w // 4), Cout)) for (h, w) in SIZES]
    dhd, dW, db = blockconv.conv_chunked_backward(lst, W, douts)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    total = 0
    xts = []
    for hd_e, g in zip(lst, douts):
        D, h, w, _ = hd_e.shape
        xt = torch.tensor(hd_e, requires_grad=True)
        xts.append(xt)
        ho, wo = -(-h // 2), -(-w // 4)
        x = torch.nn.functional.pad(xt.permute(0, 3, 1, 2).reshape(1, D * H, h, w), (0, wo * 4 - w, 0, ho * 2 - h))
        out = torch.nn.functional.conv2d(x, Wt.reshape(Cout, D * H, 2, 4), bt, stride=(2, 4))
        total = total + (out[0].permute(1, 2, 0) * torch.tensor(g)).sum()
    total.backward()
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-11, atol=1e-11)
    for a, xt in zip(dhd, xts):
        np.testing.assert_allclose(a, xt.grad.numpy(), rtol=1e-11, atol=1e-11)


def _small_stack(seed=0):
    heights, widths = [3, 5, 2, 4], [6, 9, 3, 5]
    rng = np.random.default_rng(seed)
    layers = [random_layer(seed + 1, 2, 2, 0.6), random_layer(seed + 2, 3, 3, 0.6), random_layer(seed + 3, 4, 2, 0.6)]
    convs = [ConvParams(rng.normal(0, 0.4, (3, 4, 2, 2, 4)), rng.normal(0, 0.4, 3)),
             ConvParams(rng.normal(0, 0.4, (4, 4, 3, 2, 4)), rng.normal(0, 0.4, 4))]
    layers = [LayerParams(*(np.asarray(a, np.float64) for a in (p.Wx, p.Ul, p.Uu, p.b))) for p in layers]
    xs = [np.asarray(x, np.float64) for x in random_images(seed + 9, heights, widths, 2)]
    return heights, widths, xs, layers, convs, [8, 4, 2]


def test_stack_finite_differences():
    heights, widths, xs, layers, convs, cw = _small_stack()
    ys, caches = stack.stack_forward(heights, widths, xs, layers, convs, cw)
    rng = np.random.default_rng(11)
    dys = [rng.standard_normal(y.shape) for y in ys]
    dxs, lgrads, cgrads = stack.stack_backward(layers, convs, caches, dys)

    def loss():
        y2, _ = stack.stack_forward(heights, widths, xs, layers, convs, cw)
        return sum(float(np.sum(a * r)) for a, r in zip(y2, dys))

    eps = 1e-6
    checks = []
    for lvl, P in enumerate(layers):
        for k, name in enumerate(("Wx", "Ul", "Uu", "b")):
            checks.append((getattr(P, name), lgrads[lvl][k]))
    for j, cv in enumerate(convs):
        checks.append((cv.W, cgrads[j][0]))
        checks.append((cv.b, cgrads[j][1]))
    for e in range(len(xs)):
        checks.append((xs[e], dxs[e]))
    for arr, g in checks:
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps; lp = loss()
            arr[idx] = old - eps; lm = loss()
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 + 1e-5 * abs(g[idx]), (idx, fd, g[idx])


def test_stack_level_sizes_word_workload():
    wl = make_workload("stack", 0)
    sizes = [(int(h), int(w)) for h, w in zip(wl.heights, wl.widths)]
    l2 = [blockconv.out_size(h, w) for h, w in sizes]
    l3 = [blockconv.out_size(h, w) for h, w in l2]
    assert all(1 <= h <= 20 and 1 <= w <= 50 for h, w in l2)
    assert all(1 <= h <= 10 and 1 <= w <= 13 for h, w in l3)
