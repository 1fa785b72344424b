"""GPU parity of the Leaky-LP cell (MDL_CELL_LEAKY_LP) against the oracle (oracle/leaky.py), element by element:
h_dirs (the whole canvas), y, dx and every weight gradient, dVl and dVu included, under the tolerance and
conditioning criterion of test_gpu_parity. Workspace and outputs are filled with NaN first. Cases: the tiny
workload, ragged shape sets at every instantiated hidden size (several tiles, ragged tails, 1-pixel rows and
columns, the widest diagonals the kernels take), bf16 input, the full word and line batches with every example
compared, and the cell's stability on the line batch (|s| <= 1, where the plain cell's state is ~1e10)."""

import numpy as np
import pytest
import torch

from test_gpu_parity import (BF16_TOL, DEV, F32_TOL, Lazy, _cat, _np, assert_close, perturbed, poison)
from oracle import leaky as olk, pack as opack
from workloads import LeakyLayerParams, cotangent, make_workload, random_images, random_leaky_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import directional_mdlstm_handwriting_amd as M
    from directional_mdlstm_handwriting_amd.layer import DeviceLayout, DeviceParams, LayerGrads, PackedLayer, flat_input

NAMES = ("dWx", "dUl", "dUu", "db", "dVl", "dVu")


def oracle_leaky(heights, widths, xs, P, canvas_w_min, dys, sep=1):
    lay = opack.pack(heights, widths, canvas_w_min, sep, "packed")

    def run(xs_, P_, dys_):
        ys, cache = olk.layer_forward(lay, xs_, P_)
        res = olk.layer_backward(lay, P_, cache, dys=dys_)
        return {"ys": ys, "hd": cache[1], "sd": cache[2], "dxs": res[0], "dW": res[1:]}

    out = run(xs, P, dys)

    def response():
        rng = np.random.default_rng(12345)
        Pp = LeakyLayerParams(*(perturbed(getattr(P, n), rng) for n in ("Wx", "Ul", "Uu", "b", "Vl", "Vu")))
        q = run([perturbed(x, rng) for x in xs], Pp, [perturbed(d, rng) for d in dys])
        return {"hd": q["hd"] - out["hd"], "ys": [a - b for a, b in zip(q["ys"], out["ys"])],
                "dxs": [a - b for a, b in zip(q["dxs"], out["dxs"])], "dW": [a - b for a, b in zip(q["dW"], out["dW"])]}

    out["sens"] = Lazy(response)
    return out


def run_leaky(heights, widths, xs, P, canvas_w_min, dys, x_dtype="f32", sep=1):
    print(f"[gpu] leaky layer n={len(heights)} C={P.C} H={P.H} dtype={x_dtype}", flush=True)
    dl = DeviceLayout(heights, widths, canvas_w_min, sep, "packed", DEV)
    lay = PackedLayer(dl, P.C, P.H, x_dtype)
    poison(lay)
    Pd = DeviceParams.from_host(P, DEV)
    assert Pd.cell == M.MDL_CELL_LEAKY_LP
    lay.scatter(flat_input(xs, x_dtype, DEV))
    lay.forward(Pd)
    lay.dirsum()
    dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in dys]).astype(np.float32), device=DEV)
    g = LayerGrads(*(torch.full_like(t, float("nan")) for t in (Pd.Wx, Pd.Ul, Pd.Uu, Pd.b, Pd.Vl, Pd.Vu)))
    dx = torch.full((int(sum(np.asarray(x).size for x in xs)),), float("nan"), device=DEV)
    lay.backward(Pd, g, dy_flat=dy, dx_flat=dx)
    torch.cuda.synchronize()
    return lay, g, dx


def check(lay, g, dx, o, tol=F32_TOL):
    sn = o["sens"]
    assert_close("leaky h_dirs", _np(lay.h_dirs), o["hd"], tol, sens=lambda: sn()["hd"])
    assert_close("leaky y", _np(lay.y), _cat(o["ys"]), tol, sens=lambda: _cat(sn()["ys"]))
    assert_close("leaky dx", _np(dx), _cat(o["dxs"]), tol, sens=lambda: _cat(sn()["dxs"]))
    for k, name in enumerate(NAMES):
        assert_close(f"leaky {name}", _np(getattr(g, name)), o["dW"][k], tol, sens=lambda k=k: sn()["dW"][k])


@pytest.mark.parametrize("seed", [0, 1])
def test_leaky_tiny(seed):
    wl = make_workload("tiny", seed, cell="leaky")
    P = wl.layers[0]
    dys = cotangent(seed, wl.heights, wl.widths, wl.H)
    lay, g, dx = run_leaky(wl.heights, wl.widths, wl.xs, P, 8, dys)
    check(lay, g, dx, oracle_leaky(wl.heights, wl.widths, wl.xs, P, 8, dys))


LEAKY_RAGGED = [
    # (heights, widths, C, H)
    ([1, 1, 3, 17, 2, 9], [1, 23, 1, 5, 40, 9], 4, 16),
    ([40, 12, 33, 25], [8, 200, 61, 25], 4, 16),
    ([64, 5, 2], [70, 64, 9], 4, 16),              # the widest diagonal the H = 16 kernels take (64 cells)
    ([32, 32, 20], [256, 300, 33], 4, 32),
    ([7, 3, 11, 5, 6, 2, 9], [13, 27, 4, 16, 6, 31, 2], 6, 8),
    ([6, 9, 4, 1], [12, 7, 15, 3], 3, 4),
    ([5, 3, 4], [9, 7, 3], 13, 16),                # more than 4 input channels: several projection k-steps
    ([100, 6], [104, 30], 4, 16),                  # 7 cell tiles: the 16-bit kernels at their LDS limit
    ([120, 9], [126, 14], 4, 16),                  # 8 cell tiles: past that limit, the fp32 kernels
]


@pytest.mark.parametrize("case", range(len(LEAKY_RAGGED)))
def test_leaky_ragged(case):
    h, w, C, H = LEAKY_RAGGED[case]
    P = random_leaky_layer(800 + case, C, H)
    xs = random_images(900 + case, h, w, C)
    dys = cotangent(1000 + case, h, w, H)
    cw = max(max(w), 64)
    lay, g, dx = run_leaky(h, w, xs, P, cw, dys)
    check(lay, g, dx, oracle_leaky(h, w, xs, P, cw, dys))


def test_leaky_bf16_line_subset():
    wl = make_workload("line", 0, cell="leaky")
    idx = [0, 1]
    h, w = wl.heights[idx], wl.widths[idx]
    xs = [wl.xs[i] for i in idx]
    P = wl.layers[0]
    dys = cotangent(4, h, w, wl.H)
    lay, g, dx = run_leaky(h, w, xs, P, 2048, dys, x_dtype="bf16")
    o = oracle_leaky(h, w, xs, P, 2048, dys)
    check(lay, g, dx, o, BF16_TOL)
    check(lay, g, dx, o, F32_TOL)


@pytest.mark.parametrize("name", ["word", "line"])
def test_leaky_full_size(name):
    """Every example of the word and line batches with the Leaky-LP cell; on the line batch also the memory
    state's bound, where the plain cell's grows to about 1e10."""
    wl = make_workload(name, 0, cell="leaky")
    P = wl.layers[0]
    dys = cotangent(11, wl.heights, wl.widths, wl.H)
    lay, g, dx = run_leaky(wl.heights, wl.widths, wl.xs, P, wl.canvas_w_min[0], dys, x_dtype=wl.x_dtype)
    o = oracle_leaky(wl.heights, wl.widths, wl.xs, P, wl.canvas_w_min[0], dys)
    check(lay, g, dx, o)
    assert np.max(np.abs(o["sd"])) <= 1.0
    # the stash's memory states (second of each (g, s) pair) as the GPU computed them
    T = lay.dl.info["computed_cells"]
    H = wl.H
    s2 = lay.ws.view(torch.float32)[4 * T * 4 * H:4 * T * 6 * H].view(-1, 2)[:, 1]
    assert float(s2.abs().max()) <= 1.0
