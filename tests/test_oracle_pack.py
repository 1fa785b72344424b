"""Pins of the oracle packer ("No Padding Please", §V, §V-A, §IX-B (packing algorithm details, Algorithm 1)) and of the
input-skewing trick (§IV-A, Figure 3).

The packer is checked against (a) hand-worked runs of the loop, (b) an
independent replay verifier that re-derives every greedy choice and every row
break from the rules, (c) geometric invariants (disjoint, separated, inside),
(d) special cases with known answers, and (e) brute-force per-pixel maps.
"""

import json
import os

import numpy as np
import pytest

from oracle import pack
from workloads import make_sizes_only

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_worked.json")


def _replay_verify(heights, widths, lay, sep):
    """Re-derive the greedy choices from the layout alone."""
    n = len(heights)
    Wc = lay.Wc
    seq = [e for row in lay.rows for e in row]
    assert sorted(seq) == list(range(n)), "every example placed exactly once"
    hs = [heights[e] for e in seq]
    assert all(hs[k] >= hs[k + 1] for k in range(n - 1)), "buckets visited tallest first"
    placed = set()
    for r, row in enumerate(lay.rows):
        x_end = None
        for pos, e in enumerate(row):
            off = 0 if pos == 0 else x_end + sep
            assert lay.rects[e][1] == off
            bucket = [q for q in range(n) if heights[q] == heights[e] and q not in placed]
            fitting = [q for q in bucket if off + widths[q] <= Wc]
            best = sorted(fitting, key=lambda q: (-widths[q], q))[0]
            assert best == e, (r, pos, e, best)
            placed.add(e)
            x_end = off + widths[e]
        if r + 1 < len(lay.rows):
            nxt = lay.rows[r + 1][0]
            if heights[nxt] == heights[row[-1]]:
                # the row closed inside a bucket: nothing of that bucket fitted any more
                bucket = [q for q in range(n) if heights[q] == heights[nxt] and q not in placed]
                assert all(x_end + sep + widths[q] > Wc for q in bucket)
            else:
                # a row never closes on a bucket change alone; if it closed, the next bucket did not fit
                bucket = [q for q in range(n) if heights[q] == heights[nxt] and q not in placed]
                assert all(x_end + sep + widths[q] > Wc for q in bucket)


def _replay_verify_exact(heights, widths, lay, sep):
    """Exact-height rows: the same greedy choices as Algorithm 1, every row of a single height, and a row
    closes either because nothing of its bucket fits any more or because the bucket is used up."""
    n = len(heights)
    Wc = lay.Wc
    seq = [e for row in lay.rows for e in row]
    assert sorted(seq) == list(range(n))
    hs = [heights[e] for e in seq]
    assert all(hs[k] >= hs[k + 1] for k in range(n - 1)), "buckets visited tallest first"
    placed = set()
    for r, row in enumerate(lay.rows):
        assert len({heights[e] for e in row}) == 1, "one height per row"
        x_end = None
        for pos, e in enumerate(row):
            off = 0 if pos == 0 else x_end + sep
            assert lay.rects[e][1] == off
            bucket = [q for q in range(n) if heights[q] == heights[e] and q not in placed]
            best = sorted([q for q in bucket if off + widths[q] <= Wc], key=lambda q: (-widths[q], q))[0]
            assert best == e, (r, pos, e, best)
            placed.add(e)
            x_end = off + widths[e]
        rest = [q for q in range(n) if heights[q] == heights[row[0]] and q not in placed]
        assert all(x_end + sep + widths[q] > Wc for q in rest), "closed although an example of the bucket fitted"


def _geometry(heights, widths, lay, sep):
    n = len(heights)
    R = lay.rects.astype(int)
    for e in range(n):
        y0, x0, h, w = R[e]
        assert (h, w) == (heights[e], widths[e])
        assert 0 <= y0 and y0 + h <= lay.Hc and 0 <= x0 and x0 + w <= lay.Wc
    for a in range(n):
        for b in range(a + 1, n):
            ya, xa, ha, wa = R[a]
            yb, xb, hb, wb = R[b]
            hgap = max(xb - (xa + wa), xa - (xb + wb))
            vgap = max(yb - (ya + ha), ya - (yb + hb))
            assert hgap >= sep or vgap >= sep, (a, b)
    for row in lay.rows:
        assert R[row[-1]][1] + R[row[-1]][3] <= lay.Wc
        ys = {R[e][0] for e in row}
        assert len(ys) == 1, "examples of one row are top-aligned"
        assert all(heights[e] <= heights[row[0]] for e in row)


def _brute_maps(lay):
    Hc, Wc = lay.Hc, lay.Wc
    eid = -np.ones((Hc, Wc), np.int32)
    for e, (y0, x0, h, w) in enumerate(lay.rects):
        for y in range(y0, y0 + h):
            for x in range(x0, x0 + w):
                eid[y, x] = e
    border = np.zeros((Hc, Wc), np.uint8)
    for y in range(Hc):
        for x in range(Wc):
            e = eid[y, x]
            if e < 0:
                continue
            if x > 0 and eid[y, x - 1] == e:
                border[y, x] |= 1
            if x + 1 < Wc and eid[y, x + 1] == e:
                border[y, x] |= 2
            if y > 0 and eid[y - 1, x] == e:
                border[y, x] |= 4
            if y + 1 < Hc and eid[y + 1, x] == e:
                border[y, x] |= 8
    return eid, border


def test_hand_worked_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        lay = pack.pack_alg1(c["heights"], c["widths"], c["canvas_w_min"], c["sep"])
        assert (lay.Hc, lay.Wc) == (c["Hc"], c["Wc"])
        assert lay.rows == c["rows"]
        assert lay.rects.tolist() == c["rects"]


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("kind", ["tiny", "word", "line"])
def test_replay_and_geometry(kind, seed):
    h, w = make_sizes_only(kind, seed)
    cw = {"tiny": 8, "word": 1024, "line": 2048}[kind]
    lay = pack.pack_alg1(h, w, cw, 1)
    _replay_verify(list(h), list(w), lay, 1)
    _geometry(list(h), list(w), lay, 1)


@pytest.mark.parametrize("seed", range(6))
def test_adversarial_sizes(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 40))
    h = rng.integers(1, 6, n)
    w = rng.integers(1, 15, n)
    for sep in (0, 1, 2):
        lay = pack.pack_alg1(h, w, 16, sep)
        _replay_verify(list(h), list(w), lay, sep)
        _geometry(list(h), list(w), lay, sep)
        eid, border = _brute_maps(lay)
        assert np.array_equal(eid, lay.eid)
        assert np.array_equal(border, lay.border)


def test_special_cases():
    lay = pack.pack_alg1([5], [7], 3, 1)
    assert lay.rects.tolist() == [[0, 0, 5, 7]] and (lay.Hc, lay.Wc) == (5, 7)
    # every example as wide as the canvas: one per row
    lay = pack.pack_alg1([2, 3, 2], [9, 9, 9], 9, 1)
    assert lay.rows == [[1], [0], [2]]
    assert lay.rects.tolist() == [[4, 0, 2, 9], [0, 0, 3, 9], [7, 0, 2, 9]]
    # one bucket: widest first, rows of what fits
    lay = pack.pack_alg1([4] * 4, [5, 2, 5, 3], 10, 1)
    assert lay.rows == [[0, 3], [2, 1]]
    # all of width 1 on a canvas of width 1 with no separator: a column
    lay = pack.pack_alg1([1, 1, 1], [1, 1, 1], 1, 0)
    assert lay.Hc == 3 and lay.rects[:, 0].tolist() == [0, 1, 2]


def test_maps_word():
    h, w = make_sizes_only("tiny", 3)
    lay = pack.pack_alg1(h, w, 8, 1)
    eid, border = _brute_maps(lay)
    assert np.array_equal(eid, lay.eid)
    assert np.array_equal(border, lay.border)


def test_padded_layout():
    h, w = make_sizes_only("word", 0)
    lay = pack.pack_padded(h, w)
    Hm, Wm = int(max(h)), int(max(w))
    assert (lay.Hc, lay.Wc) == (len(h) * Hm, Wm)
    for b in range(len(h)):
        assert lay.rects[b].tolist() == [b * Hm, 0, Hm, Wm]
        assert lay.real[b].tolist() == [b * Hm, 0, h[b], w[b]]
    assert (lay.eid >= 0).all()
    eid, border = _brute_maps(lay)
    assert np.array_equal(border, lay.border)
    f = pack.waste(lay, h, w)
    assert 0.5 < f["padded_cell_fraction"] < 0.85


def test_errors():
    with pytest.raises(ValueError):
        pack.pack_alg1([], [], 8, 1)
    with pytest.raises(ValueError):
        pack.pack_alg1([0], [3], 8, 1)
    with pytest.raises(ValueError):
        pack.pack_alg1([3], [3], 8, -1)
    with pytest.raises(OverflowError):
        pack.pack_alg1([2 ** 16], [2 ** 15], 1, 1)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kind", ["tiny", "word", "line"])
def test_exact_height_replay_and_geometry(kind, seed):
    h, w = make_sizes_only(kind, seed)
    cw = {"tiny": 8, "word": 1024, "line": 2048}[kind]
    lay = pack.pack_exact(h, w, cw, 1)
    _replay_verify_exact(list(h), list(w), lay, 1)
    _geometry(list(h), list(w), lay, 1)
    eid, border = _brute_maps(lay)
    assert np.array_equal(eid, lay.eid) and np.array_equal(border, lay.border)


@pytest.mark.parametrize("seed", range(6))
def test_exact_height_adversarial(seed):
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 40))
    h = rng.integers(1, 6, n)
    w = rng.integers(1, 15, n)
    for sep in (0, 1, 2):
        lay = pack.pack_exact(h, w, 16, sep)
        _replay_verify_exact(list(h), list(w), lay, sep)
        _geometry(list(h), list(w), lay, sep)


def test_exact_height_special_cases():
    # worked by hand: Wc = 10; bucket 3 = {0}: e0 at x 0 and the bucket is used up, so its row closes even
    # though e1 (3 wide) would still fit after it; bucket 2: e1 at (4, 0); Hc = 3 + 1 + 2
    lay = pack.pack_exact([3, 2], [2, 3], 10, 1)
    assert lay.rows == [[0], [1]] and lay.Hc == 6
    assert lay.rects.tolist() == [[0, 0, 3, 2], [4, 0, 2, 3]]
    # the Algorithm 1 reading lets that row run on into the shorter bucket
    assert pack.pack_alg1([3, 2], [2, 3], 10, 1).rows == [[0, 1]]
    # one height: both readings are the same loop (the line batch)
    for seed in range(4):
        h, w = make_sizes_only("line", seed)
        a, b = pack.pack_alg1(h, w, 2048, 1), pack.pack_exact(h, w, 2048, 1)
        assert a.rows == b.rows and np.array_equal(a.rects, b.rects)
    # exact-height rows never fill less canvas height than the mixed rows
    for seed in range(4):
        h, w = make_sizes_only("word", seed)
        assert pack.pack_exact(h, w, 1024, 1).Hc >= pack.pack_alg1(h, w, 1024, 1).Hc


def test_skew_columns_are_global_antidiagonals():
    # §IV-A: after the skew, column k holds the canvas cells with y + x = k, and every dependency of a cell
    # (its left and upper neighbour) sits in column k - 1, so a column can be computed at once
    Hc, Wc = 5, 7
    ys, xs = np.meshgrid(np.arange(Hc), np.arange(Wc), indexing="ij")
    idx = np.stack([ys, xs], axis=-1) + 1      # +1 so that the zero fill is told apart from cell (0, 0)
    sk = pack.skew(idx)
    assert sk.shape == (Hc, Wc + Hc - 1, 2)
    for k in range(Wc + Hc - 1):
        cells = {(int(a) - 1, int(b) - 1) for a, b in sk[:, k] if a > 0}
        assert cells == {(y, k - y) for y in range(Hc) if 0 <= k - y < Wc}
        for (y, x) in cells:
            for (py, px) in ((y, x - 1), (y - 1, x)):
                if py >= 0 and px >= 0:
                    assert py + px == k - 1
    assert np.array_equal(pack.unskew(sk, Wc), idx)


def test_skew_stats_word_batch():
    h, w = make_sizes_only("word", 0)
    for lay in (pack.pack_alg1(h, w, 1024, 1), pack.pack_exact(h, w, 1024, 1)):
        st = pack.skew_stats(lay, h, w)
        N = int(np.sum(np.asarray(h, np.int64) * np.asarray(w, np.int64)))
        mask = (lay.eid >= 0).astype(np.int64)
        sk = pack.skew(mask)
        # the skewed grid's size, and its mask still counts every real pixel once
        assert sk.size == st["skewed_cells"] and int(sk.sum()) == N
        assert st["global_depth"] == sk.shape[1] == lay.Hc + lay.Wc - 1
        assert st["local_depth"] == int(np.max(np.asarray(h) + np.asarray(w) - 1)) < st["global_depth"]
        assert 0.0 < st["canvas_waste"] < st["skewed_padding_fraction"] < 1.0
