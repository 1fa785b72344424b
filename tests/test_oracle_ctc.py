"""Pins of the model-head oracle (oracle/ctc.py): the CTC loss of "No Padding Please" §II (reference [13]
of the pages, Graves et al. 2006) and the head in front of it.

The recursion is checked against (a) the definition written out as a sum over every path (brute force),
(b) closed forms for uniform logits, (c) the identity sum_s alpha_t(s) beta_t(s) / y_t(l'_s) = p at every
frame, (d) torch's own CTC loss and its gradient (an independent library implementation), (e) central
finite differences, and (f) the head's gradients against torch autograd of the same composition.
"""

import math

import numpy as np
import pytest
import torch

from oracle import ctc


def _rand_case(rng, T, K, U):
    z = rng.normal(0.0, 1.5, (T, K))
    lab = [int(v) for v in rng.integers(1, K, U)]
    return z, lab


@pytest.mark.parametrize("seed", range(10))
def test_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    for T in range(1, 6):
        K = 2 + seed % 2
        for U in range(0, 4):
            z, lab = _rand_case(rng, T, K, U)
            loss, _, _, _ = ctc.ctc(z, lab)
            ref = ctc.ctc_brute(z, lab)
            if math.isinf(ref):
                assert math.isinf(loss)
            else:
                assert abs(loss - ref) <= 1e-12 * max(1.0, abs(ref)), (T, K, lab)


def test_repeated_labels_need_a_blank():
    # [1, 1] needs three frames (1, blank, 1); [1, 2] needs two
    z = np.zeros((2, 3))
    assert math.isinf(ctc.ctc(z, [1, 1])[0]) and math.isinf(ctc.ctc_brute(z, [1, 1]))
    loss, dz, _, _ = ctc.ctc(z, [1, 1])
    assert not dz.any()
    assert math.isfinite(ctc.ctc(z, [1, 2])[0])
    assert math.isfinite(ctc.ctc(np.zeros((3, 3)), [1, 1])[0])


@pytest.mark.parametrize("T,K", [(1, 2), (4, 3), (7, 5), (12, 80)])
def test_uniform_logits_closed_forms(T, K):
    z = np.zeros((T, K))
    # empty label: the all-blank path only
    assert abs(ctc.ctc(z, [])[0] - T * math.log(K)) < 1e-10
    # one label: blank^a c^b blank^(T-a-b) with b >= 1, T (T + 1) / 2 paths
    assert abs(ctc.ctc(z, [1])[0] - (T * math.log(K) - math.log(T * (T + 1) / 2))) < 1e-10
    # two distinct labels over T frames: the paths are words blank* c1+ blank* c2+ blank*, i.e. C(T + 2, 4)
    if T >= 2:
        n = math.comb(T + 2, 4)
        assert abs(ctc.ctc(z, [1, 2])[0] - (T * math.log(K) - math.log(n))) < 1e-10


@pytest.mark.parametrize("seed", range(5))
def test_alpha_beta_identity(seed):
    rng = np.random.default_rng(100 + seed)
    z, lab = _rand_case(rng, 9, 6, 3)
    loss, _, la, lb = ctc.ctc(z, lab)
    logy = ctc.log_softmax(z)
    lp = ctc.extended(lab)
    for t in range(z.shape[0]):
        terms = [la[t, s] + lb[t, s] - logy[t, lp[s]] for s in range(len(lp))]
        assert abs(np.logaddexp.reduce(terms) + loss) < 1e-10


@pytest.mark.parametrize("seed", range(6))
def test_against_torch_ctc(seed):
    rng = np.random.default_rng(200 + seed)
    T, K = int(rng.integers(3, 20)), int(rng.integers(2, 30))
    U = int(rng.integers(0, (T + 1) // 2 + 1))
    z, lab = _rand_case(rng, T, K, U)
    loss, dz, _, _ = ctc.ctc(z, lab)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    lp = torch.log_softmax(zt, dim=-1)
    ref = torch.nn.functional.ctc_loss(lp[:, None, :], torch.tensor([lab], dtype=torch.long),
                                       torch.tensor([T]), torch.tensor([U]), blank=0, reduction="sum")
    ref.backward()
    assert abs(loss - ref.item()) < 1e-9 * max(1.0, abs(loss))
    assert np.allclose(dz, zt.grad.numpy(), rtol=1e-8, atol=1e-10)


@pytest.mark.parametrize("seed", range(4))
def test_gradient_finite_differences(seed):
    rng = np.random.default_rng(300 + seed)
    z, lab = _rand_case(rng, 6, 4, 2)
    _, dz, _, _ = ctc.ctc(z, lab)
    eps = 1e-6
    num = np.zeros_like(z)
    for t in range(z.shape[0]):
        for k in range(z.shape[1]):
            zp, zm = z.copy(), z.copy()
            zp[t, k] += eps
            zm[t, k] -= eps
            num[t, k] = (ctc.ctc(zp, lab)[0] - ctc.ctc(zm, lab)[0]) / (2 * eps)
    assert np.allclose(dz, num, atol=1e-7)
    # softmax gradients sum to zero in every frame
    assert np.allclose(dz.sum(axis=1), 0.0, atol=1e-12)


def test_head_against_torch_autograd():
    rng = np.random.default_rng(400)
    H, K = 5, 7
    sizes = [(3, 6), (1, 4), (4, 9)]
    ys = [rng.normal(0, 0.5, (h, w, H)) for h, w in sizes]
    Wfc = rng.normal(0, 0.3, (H, K))
    bfc = rng.normal(0, 0.3, K)
    labels = [[1, 3], [], [2, 2, 5]]
    losses, dys, dW, db = ctc.head_forward_backward(ys, Wfc, bfc, labels)
    Wt = torch.tensor(Wfc, requires_grad=True)
    bt = torch.tensor(bfc, requires_grad=True)
    yts = [torch.tensor(y, requires_grad=True) for y in ys]
    total = 0
    for e, (yt, lab) in enumerate(zip(yts, labels)):
        zt = yt.sum(dim=0) @ Wt + bt
        lp = torch.log_softmax(zt, dim=-1)
        le = torch.nn.functional.ctc_loss(lp[:, None, :], torch.tensor([lab], dtype=torch.long),
                                          torch.tensor([zt.shape[0]]), torch.tensor([len(lab)]), blank=0,
                                          reduction="sum")
        assert abs(le.item() - losses[e]) < 1e-9 * max(1.0, losses[e])
        total = total + le
    total.backward()
    assert np.allclose(dW, Wt.grad.numpy(), rtol=1e-8, atol=1e-10)
    assert np.allclose(db, bt.grad.numpy(), rtol=1e-8, atol=1e-10)
    for dy, yt in zip(dys, yts):
        assert np.allclose(dy, yt.grad.numpy(), rtol=1e-8, atol=1e-10)
