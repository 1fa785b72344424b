"""Seeded synthetic inputs for the packed 4-direction 2D MDLSTM workloads.

This module only draws numbers: example sizes, pixel tensors, layer parameters
and cotangents. It holds none of the method's arithmetic (no packing, no cell
equations), so both the CPU oracle under ``oracle/`` and the HIP path (tests,
bench) can take their inputs from it without sharing any computation.

The five workloads stand in for the IAM word and line strips that
"No Padding Please: Efficient Neural Handwriting Recognition" trains on
(§VII-A); the pages print no size distribution, so the sizes below are a stated
synthetic recipe:

* ``tiny``   4 single-channel images, h ~ U{4..8}, w ~ U{4..12}, H = 4,
             canvas at least 8 wide.
* ``word``   64 images of 4 channels (2x2 blocks of grey pixels), h ~ U{12..40},
             w = clip(rint(h * LogNormal(1, 0.5)), 8, 200), H = 16, canvas 1024 wide.
* ``word_padded``  the same 64 images, laid out as a minimal-padding stack.
* ``line``   32 images of 4 channels, h = 32, w ~ U{256..1024}, pixels stored as
             bfloat16, H = 32, canvas 2048 wide.
* ``stack``  128 word-like images through MDLSTM(H=2) -> 2x4 block conv to 6 ->
             MDLSTM(H=10) -> 2x4 block conv to 20 -> MDLSTM(H=50).

Draw order for one seed (``numpy.random.default_rng(seed)``, PCG64): heights,
then the log-normal factors (or the widths), then each example's pixels in
index order, then per MDLSTM layer ``Wx, Ul, Uu, b`` and per block conv
``W, b``, all ``N(0, 0.1)`` cast to float32. Pixels are ``U(0, 1)`` float32.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

GATES = 5  # gate pre-activations per hidden unit: i, f_left, f_up, o, g
DIRECTIONS = 4

CONFIG_NAMES = ("tiny", "word", "word_padded", "line", "stack")


@dataclasses.dataclass
class LayerParams:
    """Parameters of one 4-direction MDLSTM layer (float32).

    Wx[d][C][5H], Ul[d][H][5H], Uu[d][H][5H], b[d][5H]; along the 5H axis the
    gate blocks are ordered (i, f_left, f_up, o, g), each H wide.
    """

    Wx: np.ndarray
    Ul: np.ndarray
    Uu: np.ndarray
    b: np.ndarray

    @property
    def C(self) -> int:
        return int(self.Wx.shape[1])

    @property
    def H(self) -> int:
        return int(self.Ul.shape[1])


@dataclasses.dataclass
class LeakyLayerParams:
    """Parameters of one 4-direction Leaky-LP layer (float32).

    Wx[d][C][5H], Ul[d][H][5H], Uu[d][H][5H], b[d][5H] with the gate blocks ordered (f, lambda, o1, o2, g),
    each H wide; Vl[d][H][3H], Vu[d][H][3H] project the left and upper predecessors' memory states onto the
    gates (lambda, o1, o2).
    """

    Wx: np.ndarray
    Ul: np.ndarray
    Uu: np.ndarray
    b: np.ndarray
    Vl: np.ndarray
    Vu: np.ndarray

    @property
    def C(self) -> int:
        return int(self.Wx.shape[1])

    @property
    def H(self) -> int:
        return int(self.Ul.shape[1])


@dataclasses.dataclass
class ConvParams:
    """Block-strided conv between MDLSTM levels: W[Cout][4][H][kh][kw], b[Cout]."""

    W: np.ndarray
    b: np.ndarray
    kh: int = 2
    kw: int = 4


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    heights: np.ndarray            # int32 [n]
    widths: np.ndarray             # int32 [n]
    xs: List[np.ndarray]           # per example float32 [h][w][C] (bf16-exact when dtype == "bf16")
    x_dtype: str                   # "f32" or "bf16": how the pixels are stored
    layers: List[LayerParams]
    convs: List[ConvParams]
    canvas_w_min: List[int]        # per MDLSTM level
    sep: int
    mode: str                      # "packed" or "padded"

    @property
    def n(self) -> int:
        return int(len(self.heights))

    @property
    def C(self) -> int:
        return self.layers[0].C

    @property
    def H(self) -> int:
        return self.layers[0].H

    def x_flat(self) -> np.ndarray:
        """All pixels, example after example, each example row-major [h][w][C]."""
        return np.concatenate([x.reshape(-1) for x in self.xs]).astype(np.float32)


def _round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32.

    Storage conversion of the inputs only (the line workload keeps its pixels
    in bfloat16); both sides then see the same exact values.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-exact float32 values (the bfloat16 encoding)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _layer(rng: np.random.Generator, C: int, H: int) -> LayerParams:
    def draw(shape):
        return rng.normal(0.0, 0.1, shape).astype(np.float32)

    Wx = draw((DIRECTIONS, C, GATES * H))
    Ul = draw((DIRECTIONS, H, GATES * H))
    Uu = draw((DIRECTIONS, H, GATES * H))
    b = draw((DIRECTIONS, GATES * H))
    return LayerParams(Wx, Ul, Uu, b)


def _conv(rng: np.random.Generator, H: int, cout: int) -> ConvParams:
    W = rng.normal(0.0, 0.1, (cout, DIRECTIONS, H, 2, 4)).astype(np.float32)
    b = rng.normal(0.0, 0.1, (cout,)).astype(np.float32)
    return ConvParams(W, b)


def _word_sizes(rng: np.random.Generator, n: int):
    h = rng.integers(12, 41, n)
    f = rng.lognormal(1.0, 0.5, n)
    w = np.clip(np.rint(h * f), 8, 200)
    return h.astype(np.int32), w.astype(np.int32)


def _pixels(rng: np.random.Generator, heights, widths, C: int) -> List[np.ndarray]:
    return [rng.random((int(h), int(w), C), dtype=np.float32) for h, w in zip(heights, widths)]


def _leaky(rng: np.random.Generator, C: int, H: int) -> LeakyLayerParams:
    """Wx, Ul, Uu, b drawn as for the plain cell, then the memory-state projections Vl, Vu."""
    P = _layer(rng, C, H)
    Vl = rng.normal(0.0, 0.1, (DIRECTIONS, H, 3 * H)).astype(np.float32)
    Vu = rng.normal(0.0, 0.1, (DIRECTIONS, H, 3 * H)).astype(np.float32)
    return LeakyLayerParams(P.Wx, P.Ul, P.Uu, P.b, Vl, Vu)


def random_leaky_layer(seed: int, C: int, H: int, scale: float = 0.1) -> LeakyLayerParams:
    """Stand-alone random Leaky-LP layer parameters."""
    rng = np.random.default_rng(seed)
    p = _leaky(rng, C, H)
    if scale != 0.1:
        p = LeakyLayerParams(*(a * np.float32(scale / 0.1) for a in (p.Wx, p.Ul, p.Uu, p.b, p.Vl, p.Vu)))
    return p


def make_workload(name: str, seed: int = 0, cell: str = "mdlstm") -> Workload:
    """Build one of the five named workloads for ``seed``. cell = "leaky": the single-layer workloads (tiny,
    word, word_padded, line) with a Leaky-LP layer, drawn from the same stream (the same sizes, pixels and
    Wx, Ul, Uu, b, then Vl, Vu)."""
    if cell == "leaky":
        if name == "stack":
            raise ValueError("the Leaky-LP cell is offered for the single-layer workloads")
        wl = make_workload(name, seed)
        rng = np.random.default_rng(seed)
        # replay the draws up to the layer, then draw the layer as a Leaky-LP one
        if name == "tiny":
            rng.integers(4, 9, 4); rng.integers(4, 13, 4)
        elif name in ("word", "word_padded"):
            _word_sizes(rng, 64)
        else:
            rng.integers(256, 1025, 32)
        _pixels(rng, wl.heights, wl.widths, wl.C)
        wl.layers = [_leaky(rng, wl.C, wl.H)]
        wl.name = name
        return wl
    if cell != "mdlstm":
        raise ValueError(f"unknown cell {cell!r}")
    rng = np.random.default_rng(seed)
    if name == "tiny":
        h = rng.integers(4, 9, 4).astype(np.int32)
        w = rng.integers(4, 13, 4).astype(np.int32)
        xs = _pixels(rng, h, w, 1)
        return Workload(name, seed, h, w, xs, "f32", [_layer(rng, 1, 4)], [], [8], 1, "packed")
    if name in ("word", "word_padded"):
        h, w = _word_sizes(rng, 64)
        xs = _pixels(rng, h, w, 4)
        mode = "padded" if name == "word_padded" else "packed"
        return Workload(name, seed, h, w, xs, "f32", [_layer(rng, 4, 16)], [], [1024], 1, mode)
    if name == "line":
        h = np.full(32, 32, dtype=np.int32)
        w = rng.integers(256, 1025, 32).astype(np.int32)
        xs = [_round_bf16(x) for x in _pixels(rng, h, w, 4)]
        return Workload(name, seed, h, w, xs, "bf16", [_layer(rng, 4, 32)], [], [2048], 1, "packed")
    if name == "stack":
        h, w = _word_sizes(rng, 128)
        xs = _pixels(rng, h, w, 4)
        l1 = _layer(rng, 4, 2)
        c1 = _conv(rng, 2, 6)
        l2 = _layer(rng, 6, 10)
        c2 = _conv(rng, 10, 20)
        l3 = _layer(rng, 20, 50)
        return Workload(name, seed, h, w, xs, "f32", [l1, l2, l3], [c1, c2],
                        [1024, 256, 64], 1, "packed")
    raise ValueError(f"unknown workload {name!r}; expected one of {CONFIG_NAMES}")


def make_sizes_only(kind: str, seed: int, n: Optional[int] = None):
    """Just the (heights, widths) draw of a workload family, for packer tests."""
    rng = np.random.default_rng(seed)
    if kind == "word":
        return _word_sizes(rng, n or 64)
    if kind == "line":
        w = rng.integers(256, 1025, n or 32).astype(np.int32)
        return np.full(len(w), 32, dtype=np.int32), w
    if kind == "tiny":
        h = rng.integers(4, 9, n or 4).astype(np.int32)
        w = rng.integers(4, 13, n or 4).astype(np.int32)
        return h, w
    raise ValueError(kind)


def random_layer(seed: int, C: int, H: int, scale: float = 0.1) -> LayerParams:
    """Stand-alone random layer parameters (parity cases at other sizes)."""
    rng = np.random.default_rng(seed)
    p = _layer(rng, C, H)
    if scale != 0.1:
        p = LayerParams(*(a * np.float32(scale / 0.1) for a in (p.Wx, p.Ul, p.Uu, p.b)))
    return p


def random_images(seed: int, heights, widths, C: int) -> List[np.ndarray]:
    rng = np.random.default_rng(seed)
    return _pixels(rng, heights, widths, C)


def cotangent(seed: int, heights, widths, H: int) -> List[np.ndarray]:
    """Seeded N(0, 1) output gradient per example, float32 [h][w][H]."""
    rng = np.random.default_rng(seed + 7919)
    return [rng.standard_normal((int(h), int(w), H)).astype(np.float32)
            for h, w in zip(heights, widths)]


CTC_CLASSES = 80  # 79 symbols and the CTC blank: the size of the IAM character set the pages train on


def head_params(seed: int, H: int, K: int = CTC_CLASSES):
    """Seeded N(0, 0.1) float32 weights [H][K] and bias [K] of the model head's fully-connected layer."""
    rng = np.random.default_rng(seed + 104729)
    W = rng.normal(0.0, 0.1, (H, K)).astype(np.float32)
    b = rng.normal(0.0, 0.1, K).astype(np.float32)
    return W, b


def ctc_labels(seed: int, frames, K: int = CTC_CLASSES) -> List[List[int]]:
    """One synthetic label per example with T = frames[e] frames: length U ~ U{1..(T+1)//2} (so every label,
    repeats included, can be aligned), classes ~ U{1..K-1}."""
    rng = np.random.default_rng(seed + 130363)
    out = []
    for T in frames:
        U = int(rng.integers(1, (int(T) + 1) // 2 + 1))
        out.append([int(c) for c in rng.integers(1, K, U)])
    return out
