"""The overlaps with the wavefronts change no result.

The weight gradients beside the reverse wavefront:
mdl_backward lets persistent weight-gradient workgroups run beside the reverse wavefront (on the compute
units its units leave free) and computes the blocks they did not get to after it; every block goes through
the same code, so the gradients must equal, bit for bit, those of a call with the overlap switched off, and
those of a call in which every task claimed beside the wavefront is given up there (no time allowed for its
wait) and computed after it.
Checked on the line batch (32 examples, 128 units: the overlap runs) and on a small batch, with the flat and
the canvas input gradient; a second backward with the overlap on repeats the first exactly (the counters and
the claim queue start from zero on every call).

The direction sum beside the forward wavefront: mdl_forward_dirsum's output and h planes must equal those of
mdl_forward followed by mdl_dirsum_unpack, bit for bit, in the same modes.
"""

import numpy as np
import pytest
import torch

from test_gpu_parity import DEV, poison, run_layer
from workloads import cotangent, make_workload, random_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import directional_mdlstm_handwriting_amd as M
    from directional_mdlstm_handwriting_amd.layer import DeviceLayout, DeviceParams, LayerGrads, PackedLayer, flat_input


def _backward(out, P, dys, overlap):
    M.mdl_set_wgrad_overlap(overlap)
    try:
        lay, dl = out["layer"], out["dl"]
        Pd = DeviceParams.from_host(P, DEV)
        dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in dys]).astype(np.float32), device=DEV)
        g = LayerGrads(*(torch.full_like(t, float("nan")) for t in (Pd.Wx, Pd.Ul, Pd.Uu, Pd.b)))
        n_in = int(out["dx"].numel())
        dx = torch.full((n_in,), float("nan"), device=DEV)
        dxc = torch.full((dl.info["canvas_h"], dl.info["canvas_w"], P.C), float("nan"), device=DEV)
        lay.backward(Pd, g, dy_flat=dy, dx_flat=dx, dx_canvas=dxc)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (g.dWx, g.dUl, g.dUu, g.db, dx, dxc)]
    finally:
        M.mdl_set_wgrad_overlap(1)


def _check(name, heights, widths, xs, P, x_dtype="f32", sep=1, canvas_w_min=None):
    dys = cotangent(5, heights, widths, P.H)
    out = run_layer(heights, widths, xs, P, x_dtype=x_dtype, sep=sep, canvas_w_min=canvas_w_min, dys=dys)
    print(f"[gpu] overlap on / off / given up: {name}", flush=True)
    a = _backward(out, P, dys, 1)
    b = _backward(out, P, dys, 0)
    c = _backward(out, P, dys, 1)
    g = _backward(out, P, dys, 2)  # every task claimed beside the wavefront given up, done after it
    for nm, x, y, z, w in zip(("dWx", "dUl", "dUu", "db", "dx", "dx_canvas"), a, b, c, g):
        assert np.all(np.isfinite(x)), f"{name} {nm}: non-finite values"
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{name} {nm}: overlap changed the result"
        assert np.array_equal(x.view(np.uint32), z.view(np.uint32)), f"{name} {nm}: repeated call differs"
        assert np.array_equal(x.view(np.uint32), w.view(np.uint32)), f"{name} {nm}: given-up tasks differ"


def test_overlap_line_batch():
    wl = make_workload("line", 0)
    _check("line", wl.heights, wl.widths, wl.xs, wl.layers[0], x_dtype=wl.x_dtype, sep=wl.sep,
           canvas_w_min=wl.canvas_w_min[0])


@pytest.mark.parametrize("H", [16, 32])
def test_overlap_small_batch(H):
    rng = np.random.default_rng(40 + H)
    heights = rng.integers(3, 19, size=9)
    widths = rng.integers(3, 41, size=9)
    C = 4
    xs = [rng.standard_normal((int(h), int(w), C)).astype(np.float32) for h, w in zip(heights, widths)]
    P = random_layer(H, C, H)
    _check(f"9 examples, H={H}", heights, widths, xs, P)


def _check_forward(name, heights, widths, xs, P, x_dtype="f32", sep=1, canvas_w_min=None):
    """mdl_forward_dirsum (the direction sum beside the forward wavefront) against mdl_forward followed by
    mdl_dirsum_unpack: y and h_dirs bit for bit, with the overlap on, off, repeated, and with every wait beside
    the wavefront given up at once."""
    cw = canvas_w_min or max(int(max(widths)), 8)
    print(f"[gpu] forward + direction sum, overlap on / off / given up: {name}", flush=True)
    dl = DeviceLayout(heights, widths, cw, sep, "packed", DEV)
    lay = PackedLayer(dl, P.C, P.H, x_dtype)
    poison(lay)
    Pd = DeviceParams.from_host(P, DEV)
    lay.scatter(flat_input(xs, x_dtype, DEV))
    lay.forward(Pd)
    lay.dirsum()
    torch.cuda.synchronize()
    ref_y, ref_h = lay.y.cpu().numpy().copy(), lay.h_dirs.cpu().numpy().copy()
    assert np.all(np.isfinite(ref_y))
    for mode in (1, 0, 1, 2):
        M.mdl_set_wgrad_overlap(mode)
        try:
            lay.y.fill_(float("nan"))
            lay.h_dirs.fill_(float("nan"))
            lay.forward_dirsum(Pd)
            torch.cuda.synchronize()
        finally:
            M.mdl_set_wgrad_overlap(1)
        y, h = lay.y.cpu().numpy(), lay.h_dirs.cpu().numpy()
        assert np.array_equal(y.view(np.uint32), ref_y.view(np.uint32)), f"{name}: y differs (mode {mode})"
        assert np.array_equal(h.view(np.uint32), ref_h.view(np.uint32)), f"{name}: h_dirs differs (mode {mode})"


def test_forward_dirsum_line_batch():
    wl = make_workload("line", 0)
    _check_forward("line", wl.heights, wl.widths, wl.xs, wl.layers[0], x_dtype=wl.x_dtype, sep=wl.sep,
                   canvas_w_min=wl.canvas_w_min[0])


@pytest.mark.parametrize("H", [16, 32])
def test_forward_dirsum_small_batch(H):
    rng = np.random.default_rng(50 + H)
    heights = rng.integers(3, 19, size=9)
    widths = rng.integers(3, 41, size=9)
    C = 4
    xs = [rng.standard_normal((int(h), int(w), C)).astype(np.float32) for h, w in zip(heights, widths)]
    _check_forward(f"9 examples, H={H}", heights, widths, xs, random_layer(H + 1, C, H))
