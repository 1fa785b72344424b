"""Canvas scatter, direction sum and un-packing, oracle form (test infrastructure only).

"No Padding Please", §V-A: un-packing is packing in reverse; using the original
example indices and sizes, each example's activations are cut out of the packed
tensor and the separator pixels are dropped. §III: the 4-directional layer
combines the outputs of four MDLSTMs, one per scan direction; the combination
used here is their sum (the stacked outputs summed over the direction axis).
"""

from __future__ import annotations

from typing import List

import numpy as np


def scatter(layout, xs: List[np.ndarray]) -> np.ndarray:
    """Per-example tensors [h][w][C] -> canvas [Hc][Wc][C], zero outside the real pixels."""
    C = xs[0].shape[2]
    out = np.zeros((layout.Hc, layout.Wc, C), dtype=np.float64)
    for e, x in enumerate(xs):
        y0, x0, h, w = (int(v) for v in layout.real[e])
        assert x.shape[:2] == (h, w)
        out[y0:y0 + h, x0:x0 + w, :] = x
    return out


def unpack(layout, canvas: np.ndarray) -> List[np.ndarray]:
    """Canvas [Hc][Wc][K] -> per-example tensors [h][w][K], input order."""
    out = []
    for e in range(len(layout.real)):
        y0, x0, h, w = (int(v) for v in layout.real[e])
        out.append(np.array(canvas[y0:y0 + h, x0:x0 + w, :]))
    return out


def dirsum_unpack(layout, h_dirs: np.ndarray) -> List[np.ndarray]:
    """h_dirs [4][Hc][Wc][H] -> per-example sum over the four directions [h][w][H]."""
    total = h_dirs[0] + h_dirs[1] + h_dirs[2] + h_dirs[3]
    return unpack(layout, total)


def flat(xs: List[np.ndarray]) -> np.ndarray:
    return np.concatenate([np.asarray(x).reshape(-1) for x in xs])
