"""Block-strided convolution between MDLSTM levels, oracle form (test infrastructure only).

"No Padding Please", §V-B: a block-strided convolution has a stride equal to
its kernel size, so kernel applications never overlap. Tensor-list chunking
cuts every example into blocks of the kernel size, stacks all blocks on the
batch axis, runs one convolution over the stack, and de-chunking puts each
example's outputs back together from the original sizes; the result equals
the per-example convolution.

Readings where the pages are silent: the kernel is (rows 2, cols 4); its input is
the four directions' hidden outputs stacked as 4H channels (channel d*H + k),
so no direction sum happens between levels; partial blocks at the bottom and
right edge are zero padded (output size ceil(h/2) x ceil(w/4)); no activation
follows the convolution.
"""

from __future__ import annotations

from typing import List

import numpy as np


def out_size(h: int, w: int, kh: int = 2, kw: int = 4):
    return -(-h // kh), -(-w // kw)


def conv_example(hd_e: np.ndarray, W: np.ndarray, b: np.ndarray, kh: int = 2, kw: int = 4) -> np.ndarray:
    """hd_e [4][h][w][H] -> out [ceil(h/kh)][ceil(w/kw)][Cout], by explicit sums per output pixel."""
    hd_e = np.asarray(hd_e, np.float64)
    W = np.asarray(W, np.float64)
    D, h, w, H = hd_e.shape
    ho, wo = out_size(h, w, kh, kw)
    Cout = W.shape[0]
    out = np.zeros((ho, wo, Cout))
    for r in range(ho):
        for c in range(wo):
            acc = np.array(b, np.float64)
            for i in range(kh):
                for j in range(kw):
                    y, x = kh * r + i, kw * c + j
                    if y < h and x < w:
                        # W[o][d][k][i][j] * hd_e[d][y][x][k], summed over d and k
                        acc = acc + np.einsum("odk,dk->o", W[:, :, :, i, j], hd_e[:, y, x, :])
            out[r, c] = acc
    return out


def _chunks(hd_e, kh, kw):
    """Zero-pad to whole blocks and cut into blocks [nblocks][4][kh][kw][H]."""
    D, h, w, H = hd_e.shape
    ho, wo = out_size(h, w, kh, kw)
    pad = np.zeros((D, ho * kh, wo * kw, H))
    pad[:, :h, :w, :] = hd_e
    blocks = pad.reshape(D, ho, kh, wo, kw, H).transpose(1, 3, 0, 2, 4, 5)  # [ho][wo][D][kh][kw][H]
    return blocks.reshape(ho * wo, D, kh, kw, H)


def conv_chunked(hd_list: List[np.ndarray], W, b, kh: int = 2, kw: int = 4) -> List[np.ndarray]:
    """Tensor-list chunking: all blocks of all examples stacked, one contraction, de-chunked."""
    W = np.asarray(W, np.float64)
    stacks, shapes = [], []
    for hd_e in hd_list:
        hd_e = np.asarray(hd_e, np.float64)
        shapes.append(out_size(hd_e.shape[1], hd_e.shape[2], kh, kw))
        stacks.append(_chunks(hd_e, kh, kw))
    allb = np.concatenate(stacks, axis=0)                       # [B][D][kh][kw][H]
    Wm = W.transpose(0, 1, 3, 4, 2)                              # [Cout][D][kh][kw][H]
    res = np.einsum("bdijk,odijk->bo", allb, Wm) + np.asarray(b, np.float64)
    out, pos = [], 0
    for (ho, wo) in shapes:
        out.append(res[pos:pos + ho * wo].reshape(ho, wo, -1))
        pos += ho * wo
    return out


def conv_chunked_backward(hd_list: List[np.ndarray], W, douts: List[np.ndarray], kh: int = 2, kw: int = 4):
    """Gradients of conv_chunked: (d hd_list, dW, db)."""
    W = np.asarray(W, np.float64)
    Wm = W.transpose(0, 1, 3, 4, 2)                              # [Cout][D][kh][kw][H]
    dW = np.zeros_like(Wm)
    db = np.zeros(W.shape[0])
    dhd = []
    for hd_e, dout in zip(hd_list, douts):
        hd_e = np.asarray(hd_e, np.float64)
        D, h, w, H = hd_e.shape
        ho, wo = out_size(h, w, kh, kw)
        blocks = _chunks(hd_e, kh, kw)
        g = np.asarray(dout, np.float64).reshape(ho * wo, -1)    # [B][Cout]
        dW += np.einsum("bo,bdijk->odijk", g, blocks)
        db += g.sum(axis=0)
        dblocks = np.einsum("bo,odijk->bdijk", g, Wm)            # [B][D][kh][kw][H]
        pad = dblocks.reshape(ho, wo, D, kh, kw, H).transpose(2, 0, 3, 1, 4, 5).reshape(D, ho * kh, wo * kw, H)
        dhd.append(pad[:, :h, :w, :].copy())
    return dhd, dW.transpose(0, 1, 4, 2, 3), db
