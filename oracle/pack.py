"""Example packing, oracle form (test infrastructure only).

Follows "No Padding Please", §V (tile examples in a 2D grid, separator pixels
between them, a binary mask), §V-A (bucket by height, fill rows greedily with
the widest still-fitting example, tile rows with separators) and §IX-B
(packing algorithm details, Algorithm 1: the packing loop). The skew of §IV-A / Algorithm 1's last step is
an implementation device for convolution-based MDLSTMs and does not change any
cell's value, so the canvas here stays unskewed.

Readings where the pages leave a step open:
  * bucket visiting order: tallest height first;
  * ties between equally wide fitting examples: lowest input index;
  * a row is closed only when nothing of the current bucket fits (as the loop
    is printed), so a row may continue into the next, shorter bucket; its
    height is that of its first example, and examples are top-aligned;
  * the row still open when the loop ends is kept;
  * one separator pixel (``sep``) between neighbours in a row and between
    rows;
  * canvas width = max(canvas_w_min, widest example).

The padded mode is the "last-minute batch-padding" baseline of §VII-C: every
example gets a slot of max-height x max-width, stacked vertically, the real
pixels top-left, the rest zero padding that is computed like real cells.

The exact-height mode is the other reading of the same section: §V requires
that the examples of one packed row share one height (so that the rows can be
skewed and un-skewed for the column-parallel computation of §IV-A), and step 2
of §V-A fills rows inside each height bucket. Here a row is therefore also
closed when its bucket runs out; everything else (bucket order, greedy choice,
ties, separators) is as in the Algorithm 1 reading. ``skew`` / ``unskew`` and
``skew_stats`` give the input-skewing trick of §IV-A (Figure 3; Algorithm 1's
last step applies it to the whole packed tensor and mask): image row i is
shifted right by i pixels, so that column k of the skewed grid holds exactly
the cells on the canvas's global anti-diagonal y + x = k and depends only on
column k - 1. A pass over the skewed canvas then takes Hc + Wc - 1 dependent
column steps and computes every cell of the Hc x (Wc + Hc - 1) grid.
"""

from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

BIT_L, BIT_R, BIT_U, BIT_D = 1, 2, 4, 8   # neighbour (y,x-1), (y,x+1), (y-1,x), (y+1,x) in same example


@dataclasses.dataclass
class Layout:
    Hc: int
    Wc: int
    rects: np.ndarray        # int32 [n][4] (y0, x0, h, w) of the computed region, input order
    real: np.ndarray         # int32 [n][4] (y0, x0, h, w) of the real pixels, input order
    rows: List[List[int]]    # original example indices per packed row, left to right
    eid: np.ndarray          # int32 [Hc][Wc], example id of the computed region, -1 elsewhere
    border: np.ndarray       # uint8 [Hc][Wc], BIT_* set where that neighbour is the same example
    mode: str


def _check(heights, widths, canvas_w_min, sep):
    heights = [int(v) for v in heights]
    widths = [int(v) for v in widths]
    if len(heights) != len(widths) or len(heights) < 1:
        raise ValueError("need n >= 1 examples with one height and one width each")
    if min(heights) < 1 or min(widths) < 1:
        raise ValueError("example sizes must be positive")
    if sep < 0 or canvas_w_min < 1:
        raise ValueError("sep must be >= 0 and canvas_w_min >= 1")
    return heights, widths


def _maps(Hc, Wc, rects):
    eid = np.full((Hc, Wc), -1, dtype=np.int32)
    for e, (y0, x0, h, w) in enumerate(rects):
        region = eid[y0:y0 + h, x0:x0 + w]
        if (region != -1).any():
            raise AssertionError("overlapping rectangles")
        region[...] = e
    border = np.zeros((Hc, Wc), dtype=np.uint8)
    same = eid >= 0
    # neighbour to the left / right / above / below belongs to the same example
    border[:, 1:] |= np.where(same[:, 1:] & (eid[:, 1:] == eid[:, :-1]), BIT_L, 0).astype(np.uint8)
    border[:, :-1] |= np.where(same[:, :-1] & (eid[:, :-1] == eid[:, 1:]), BIT_R, 0).astype(np.uint8)
    border[1:, :] |= np.where(same[1:, :] & (eid[1:, :] == eid[:-1, :]), BIT_U, 0).astype(np.uint8)
    border[:-1, :] |= np.where(same[:-1, :] & (eid[:-1, :] == eid[1:, :]), BIT_D, 0).astype(np.uint8)
    return eid, border


def pack_alg1(heights, widths, canvas_w_min: int, sep: int = 1) -> Layout:
    """Shelf packing by Algorithm 1 (literal reading, see module docstring)."""
    return _shelf(heights, widths, canvas_w_min, sep, exact=False)


def pack_exact(heights, widths, canvas_w_min: int, sep: int = 1) -> Layout:
    """Shelf packing with exact-height rows (§V, §V-A prose reading): a row also closes when its bucket empties."""
    return _shelf(heights, widths, canvas_w_min, sep, exact=True)


def _shelf(heights, widths, canvas_w_min: int, sep: int, exact: bool) -> Layout:
    heights, widths = _check(heights, widths, canvas_w_min, sep)
    n = len(heights)
    Wc = max(int(canvas_w_min), max(widths))

    # §V-A step 1: buckets of equal height, filled tallest first.
    # §V-A step 2: a row takes the widest example of the bucket that still fits (lowest index among equal
    # widths). Ordered widest first, that is the first example of the bucket, in this order, that fits; a row
    # only grows, so an example the scan passes over cannot fit later in the same row. One scan over the rest
    # of the bucket therefore fills the current row, and the row is full if the scan leaves anything. A scan
    # that empties the bucket leaves the row open for the next, shorter bucket (the loop as the pages print it).
    rows: List[List[int]] = []
    row: List[int] = []
    x_of = [0] * n
    x_end = 0
    for hgt in sorted(set(heights), reverse=True):
        queue = sorted((e for e in range(n) if heights[e] == hgt), key=lambda e: (-widths[e], e))
        while queue:
            passed = []
            for e in queue:
                off = x_end + sep if row else 0
                if off + widths[e] <= Wc:
                    row.append(e)
                    x_of[e] = off
                    x_end = off + widths[e]
                else:
                    passed.append(e)
            queue = passed
            if queue:
                rows.append(row)
                row = []
                x_end = 0
        if exact and row:
            # exact-height rows: the bucket is used up, so is its row
            rows.append(row)
            row = []
            x_end = 0
    if row:
        rows.append(row)

    # step 3: tile the rows vertically with separator rows in between
    y_of = [0] * n
    y = 0
    Hc = 0
    for k, r in enumerate(rows):
        for e in r:
            y_of[e] = y
        Hc = y + heights[r[0]]
        y = Hc + sep
    rects = np.array([[y_of[e], x_of[e], heights[e], widths[e]] for e in range(n)], dtype=np.int32)
    if Hc * Wc >= 2 ** 31:
        raise OverflowError("canvas too large")
    eid, border = _maps(Hc, Wc, rects)
    return Layout(Hc, Wc, rects, rects.copy(), rows, eid, border, "exact" if exact else "packed")


def pack_padded(heights, widths) -> Layout:
    """Minimal per-batch padding: slot b at (b*Hmax, 0), Hmax x Wmax, no separator."""
    heights, widths = _check(heights, widths, 1, 0)
    n = len(heights)
    Hm, Wm = max(heights), max(widths)
    rects = np.array([[b * Hm, 0, Hm, Wm] for b in range(n)], dtype=np.int32)
    real = np.array([[b * Hm, 0, heights[b], widths[b]] for b in range(n)], dtype=np.int32)
    Hc, Wc = n * Hm, Wm
    if Hc * Wc >= 2 ** 31:
        raise OverflowError("canvas too large")
    eid, border = _maps(Hc, Wc, rects)
    return Layout(Hc, Wc, rects, real, [[b] for b in range(n)], eid, border, "padded")


def pack(heights, widths, canvas_w_min: int, sep: int = 1, mode: str = "packed") -> Layout:
    if mode == "packed":
        return pack_alg1(heights, widths, canvas_w_min, sep)
    if mode == "padded":
        return pack_padded(heights, widths)
    if mode == "exact":
        return pack_exact(heights, widths, canvas_w_min, sep)
    raise ValueError(mode)


def waste(layout: Layout, heights, widths) -> dict:
    """Padding figures: canvas waste, computed-cell padding fraction, zero-padding ratio."""
    N = int(np.sum(np.asarray(heights, np.int64) * np.asarray(widths, np.int64)))
    computed = int(np.sum(layout.rects[:, 2].astype(np.int64) * layout.rects[:, 3]))
    return {
        "real_pixels": N,
        "computed_cells": computed,
        "canvas_pixels": layout.Hc * layout.Wc,
        "canvas_waste": 1.0 - N / (layout.Hc * layout.Wc),
        "padded_cell_fraction": 1.0 - N / computed,
        "zpr": (computed - N) / N,
    }


def skew(canvas: np.ndarray) -> np.ndarray:
    """Input-skewing trick (§IV-A, Figure 3): row i of an Hc x Wc (x ...) canvas moves right by i pixels into
    an Hc x (Wc + Hc - 1) grid of zeros."""
    Hc, Wc = canvas.shape[0], canvas.shape[1]
    out = np.zeros((Hc, Wc + Hc - 1) + canvas.shape[2:], dtype=canvas.dtype)
    for i in range(Hc):
        out[i, i:i + Wc] = canvas[i]
    return out


def unskew(skewed: np.ndarray, Wc: int) -> np.ndarray:
    """Inverse of ``skew``: row i is read back from columns i .. i + Wc - 1."""
    Hc = skewed.shape[0]
    out = np.zeros((Hc, Wc) + skewed.shape[2:], dtype=skewed.dtype)
    for i in range(Hc):
        out[i] = skewed[i, i:i + Wc]
    return out


def skew_stats(layout: Layout, heights, widths) -> dict:
    """Work and depth of one direction's pass over the skewed canvas (§IV-A) next to the per-example local
    diagonals: the skewed grid's cells are all computed (the mask zeroes the invalid ones), one column per
    dependent step."""
    h = np.asarray(heights, np.int64)
    w = np.asarray(widths, np.int64)
    N = int(np.sum(h * w))
    Hc, Wc = layout.Hc, layout.Wc
    cells = Hc * (Wc + Hc - 1)
    return {
        "canvas": [Hc, Wc],
        "canvas_waste": 1.0 - N / (Hc * Wc),
        "skewed_cells": cells,
        "skewed_padding_fraction": 1.0 - N / cells,
        "global_depth": Hc + Wc - 1,
        "local_depth": int(np.max(h + w - 1)),
        "cells_per_column": Hc,
        "widest_local_diagonal": int(np.max(np.minimum(h, w))),
    }
