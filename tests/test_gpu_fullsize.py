"""Full-size parity: the word, line and stack workloads at their real sizes, every example compared (the
word batch also on its exact-height-rows canvas).

The layer runs over the whole packed canvas with the layout, shapes and
launches the bench times; the oracle runs the same whole batch (float64, a
few seconds on the word and stack batches, about ten on the line batch) and
every element of h_dirs (the whole canvas, zeros outside the examples
included), y, dx and the weight gradients is compared under the tolerance and
conditioning criterion of test_gpu_parity. The upstream gradient is a seeded
N(0, 1) draw on every example. A second backward with the upstream gradient
cleared on every other example checks the mask of "No Padding Please" §V from
the other side: those examples' input gradients must be exactly zero.
"""

import numpy as np
import pytest
import torch

from test_gpu_parity import (BF16_TOL, DEV, F32_TOL, _cat, _np, assert_close, check_layer, oracle_layer, oracle_stack,
                             poison, run_layer)
from workloads import cotangent, make_workload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import directional_mdlstm_handwriting_amd as M
    from directional_mdlstm_handwriting_amd.layer import DeviceParams, LayerGrads, PackedStack, flat_input


def offsets(heights, widths, K):
    sizes = np.asarray(heights, np.int64) * np.asarray(widths, np.int64) * K
    return np.concatenate([[0], np.cumsum(sizes)])


@pytest.mark.parametrize("name,mode", [("word", "packed"), ("word", "exact"), ("line", "packed")])
def test_layer_full_size(name, mode):
    wl = make_workload(name, 0)
    P, H, C = wl.layers[0], wl.H, wl.C
    print(f"[gpu] full-size {name} ({mode}): {wl.n} images, every example", flush=True)
    dys = cotangent(11, wl.heights, wl.widths, H)
    g = run_layer(wl.heights, wl.widths, wl.xs, P, mode=mode, canvas_w_min=wl.canvas_w_min[0], sep=wl.sep,
                  x_dtype=wl.x_dtype, dys=dys)
    o = oracle_layer(wl.heights, wl.widths, wl.xs, P, mode=mode, canvas_w_min=wl.canvas_w_min[0], sep=wl.sep,
                     dys=dys)
    check_layer(g, o)
    if wl.x_dtype == "bf16":  # the bf16-input bound as well (the fp32 one above is stricter)
        assert_close("y (bf16 bound)", _np(g["layer"].y), _cat(o["ys"]), BF16_TOL)

    # examples with a zero upstream gradient get exactly zero input gradient
    lay = g["layer"]
    zeroed = [d if e % 2 == 0 else np.zeros_like(d) for e, d in enumerate(dys)]
    dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in zeroed]), device=DEV)
    Pd = DeviceParams.from_host(P, DEV)
    gr = LayerGrads.like(Pd)
    dx = torch.full((int(sum(x.size for x in wl.xs)),), float("nan"), device=DEV)
    lay.backward(Pd, gr, dy_flat=dy, dx_flat=dx)
    torch.cuda.synchronize()
    dx = _np(dx)
    xo = offsets(wl.heights, wl.widths, C)
    for e in range(1, wl.n, 2):
        assert np.all(dx[xo[e]:xo[e + 1]] == 0.0), f"input gradient of example {e}, whose upstream gradient is zero"
    assert np.all(np.isfinite(dx))


def test_stack_full_size():
    wl = make_workload("stack", 0)
    print(f"[gpu] full-size stack: {wl.n} images, every example", flush=True)
    Hs = [P.H for P in wl.layers]
    couts = [c.b.shape[0] for c in wl.convs]
    st = PackedStack(wl.heights, wl.widths, wl.C, Hs, couts, wl.canvas_w_min, sep=wl.sep, device=DEV)
    for lay in st.levels:
        poison(lay)
    for t in st.dx_canvas + st.dh_dirs:
        t.fill_(float("nan"))
    for wsb, _ in st.conv_ws:
        wsb.view(torch.float32).fill_(float("nan"))
    params = [DeviceParams.from_host(P, DEV) for P in wl.layers]
    cdev = [(torch.as_tensor(c.W, device=DEV), torch.as_tensor(c.b, device=DEV)) for c in wl.convs]
    y = _np(st.forward(flat_input(wl.xs, "f32", DEV), params, cdev))
    hL, wL = st.level_sizes[-1]
    HL = Hs[-1]
    rng = np.random.default_rng(29)
    dys = [rng.standard_normal((int(hL[e]), int(wL[e]), HL)).astype(np.float32) for e in range(wl.n)]
    dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in dys]), device=DEV)
    lg = [LayerGrads(*(torch.full_like(t, float("nan")) for t in (p.Wx, p.Ul, p.Uu, p.b))) for p in params]
    cg = [(torch.full_like(W, float("nan")), torch.full_like(b, float("nan"))) for W, b in cdev]
    dx = torch.full((int(sum(x.size for x in wl.xs)),), float("nan"), device=DEV)
    st.backward(params, cdev, dy, lg, cg, dx_flat=dx)
    torch.cuda.synchronize()
    o = oracle_stack(wl.heights, wl.widths, wl.xs, wl.layers, wl.convs, wl.canvas_w_min, dys)
    sn = o["sens"]
    assert_close("stack y", y, _cat(o["ys"]), F32_TOL, sens=lambda: _cat(sn()["ys"]))
    assert_close("stack dx", _np(dx), _cat(o["dxs"]), F32_TOL, sens=lambda: _cat(sn()["dxs"]))
    for lvl in range(len(Hs)):
        for k, (nm, got, ref) in enumerate(zip(("dWx", "dUl", "dUu", "db"),
                                               (lg[lvl].dWx, lg[lvl].dUl, lg[lvl].dUu, lg[lvl].db), o["lg"][lvl])):
            assert_close(f"L{lvl} {nm}", _np(got), ref, F32_TOL, sens=lambda lvl=lvl, k=k: sn()["lg"][lvl][k])
    for j in range(len(wl.convs)):
        for k, nm in enumerate(("dW", "db")):
            assert_close(f"conv{j} {nm}", _np(cg[j][k]), o["cg"][j][k], F32_TOL,
                         sens=lambda j=j, k=k: sn()["cg"][j][k])
