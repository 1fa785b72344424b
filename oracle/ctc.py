"""Model head and CTC loss, oracle form (test infrastructure only).

"No Padding Please", §II and Figure 1: the network ends in a fully-connected
layer shared across the four scan directions, whose per-frame character
probabilities are trained with connectionist temporal classification (CTC,
the pages' reference [13]: Graves, Fernandez, Gomez and Schmidhuber, ICML
2006). The figure itself is lost, so the head is read as follows:

  * input: the last MDLSTM level's direction sum y_e[h][w][H] of example e
    (one shared fully-connected layer applied to each direction and added is
    the same linear map of the direction sum; its bias is counted once);
  * the image's height is collapsed by summing the rows, which turns the 2D
    output into a sequence of T = w frames, Y[t] = sum_r y_e[r][t];
  * logits z[t][k] = sum_j Y[t][j] Wfc[j][k] + b[k] over K classes, class 0
    being CTC's blank, then a softmax over k in each frame;
  * the loss of example e is -ln p(l | x) with p the CTC probability of its
    label sequence l (labels in 1..K-1); the batch loss is the plain sum over
    examples; an example whose label cannot be aligned to its frames (p = 0)
    gets loss +inf and contributes no gradient.

p(l | x) is by definition the sum, over all frame-wise paths pi in
{0..K-1}^T that reduce to l when repeats are merged and blanks dropped, of
prod_t y_t(pi_t). ``ctc_brute`` writes exactly that sum out (tiny T only).
``ctc`` computes it with the forward-backward recursion of the CTC paper
(§4.1 there): the label padded with blanks, l' = (0, l1, 0, l2, ..., lU, 0),
alpha over prefixes and beta over suffixes of l', in log space, and the
gradient of -ln p with respect to the logits,
    dz_t(k) = y_t(k) - (1 / (p y_t(k))) * sum over s with l'_s = k of alpha_t(s) beta_t(s),
both alpha_t(s) and beta_t(s) including the factor y_t(l'_s).
Everything is float64.
"""

from __future__ import annotations

import itertools
from typing import List, Sequence

import numpy as np

NEG = -np.inf


def head_logits(y: np.ndarray, Wfc: np.ndarray, bfc: np.ndarray) -> np.ndarray:
    """y [h][w][H] (direction sum) -> logits [w][K]: rows summed, then the shared fully-connected layer."""
    Y = np.asarray(y, np.float64).sum(axis=0)
    return Y @ np.asarray(Wfc, np.float64) + np.asarray(bfc, np.float64)


def log_softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))


def extended(label: Sequence[int]) -> List[int]:
    """l' = blank, l1, blank, l2, ..., lU, blank."""
    out = [0]
    for c in label:
        out += [int(c), 0]
    return out


def ctc(z: np.ndarray, label: Sequence[int]):
    """(loss, dz, log_alpha, log_beta) of one example from its logits z [T][K]."""
    logy = log_softmax(z)
    T, K = logy.shape
    lp = extended(label)
    S = len(lp)
    la = np.full((T, S), NEG)
    lb = np.full((T, S), NEG)
    # alpha: paths through the first t + 1 frames ending in state s
    la[0, 0] = logy[0, lp[0]]
    if S > 1:
        la[0, 1] = logy[0, lp[1]]
    for t in range(1, T):
        for s in range(S):
            acc = la[t - 1, s]
            if s >= 1:
                acc = np.logaddexp(acc, la[t - 1, s - 1])
            if s >= 2 and lp[s] != 0 and lp[s] != lp[s - 2]:
                acc = np.logaddexp(acc, la[t - 1, s - 2])
            la[t, s] = acc + logy[t, lp[s]]
    # beta: paths through frames t .. T-1 starting in state s
    lb[T - 1, S - 1] = logy[T - 1, lp[S - 1]]
    if S > 1:
        lb[T - 1, S - 2] = logy[T - 1, lp[S - 2]]
    for t in range(T - 2, -1, -1):
        for s in range(S):
            acc = lb[t + 1, s]
            if s + 1 < S:
                acc = np.logaddexp(acc, lb[t + 1, s + 1])
            if s + 2 < S and lp[s] != 0 and lp[s] != lp[s + 2]:
                acc = np.logaddexp(acc, lb[t + 1, s + 2])
            lb[t, s] = acc + logy[t, lp[s]]
    logp = la[T - 1, S - 1] if S == 1 else np.logaddexp(la[T - 1, S - 1], la[T - 1, S - 2])
    if not np.isfinite(logp):
        return np.inf, np.zeros((T, K)), la, lb
    dz = np.exp(logy)
    for t in range(T):
        for k in range(K):
            terms = [la[t, s] + lb[t, s] for s in range(S) if lp[s] == k]
            if terms:
                dz[t, k] -= np.exp(np.logaddexp.reduce(terms) - logp - logy[t, k])
    return -logp, dz, la, lb


def ctc_brute(z: np.ndarray, label: Sequence[int]) -> float:
    """-ln p(l | x) as the plain sum over all K^T paths (tiny T and K only)."""
    y = np.exp(log_softmax(z))
    T, K = y.shape
    target = [int(c) for c in label]
    p = 0.0
    for path in itertools.product(range(K), repeat=T):
        merged = [c for i, c in enumerate(path) if i == 0 or c != path[i - 1]]
        if [c for c in merged if c != 0] == target:
            p += float(np.prod([y[t, path[t]] for t in range(T)]))
    return -np.log(p) if p > 0 else np.inf


def head_forward_backward(ys: List[np.ndarray], Wfc: np.ndarray, bfc: np.ndarray, labels: List[Sequence[int]]):
    """Losses [n], gradients of the summed loss: dys (one [h][w][H] per example), dWfc [H][K], dbfc [K]."""
    Wfc = np.asarray(Wfc, np.float64)
    bfc = np.asarray(bfc, np.float64)
    losses, dys = [], []
    dW = np.zeros_like(Wfc)
    db = np.zeros_like(bfc)
    for y, lab in zip(ys, labels):
        y = np.asarray(y, np.float64)
        Y = y.sum(axis=0)
        loss, dz, _, _ = ctc(Y @ Wfc + bfc, lab)
        losses.append(loss)
        dW += Y.T @ dz
        db += dz.sum(axis=0)
        dY = dz @ Wfc.T
        # the rows were summed: each row receives the frame's gradient
        dys.append(np.broadcast_to(dY[None], y.shape).copy())
    return np.array(losses), dys, dW, db
