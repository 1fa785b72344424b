"""Full-size parity: the word, line and stack workloads at their real sizes, checked on sampled examples
(the word batch also on its exact-height-rows canvas).

The layer runs over the whole packed canvas with the layout, shapes and
launches the bench times. Examples on a packed canvas are independent (the
mask cuts every dependency at an example's edge, "No Padding Please" §V), so
the oracle computes a sample of them one by one, each alone. The upstream
gradient is nonzero only on the sampled examples. Then every other example's
input gradient is exactly zero, and the weight gradients are sums over the
sampled examples only, which the oracle fixes as well. The sample always holds
the deepest example (most dependent diagonals) and the smallest one. The
tolerance and its conditioning fallback are those of test_gpu_parity.
"""

import numpy as np
import pytest
import torch

from test_gpu_parity import BF16_TOL, DEV, F32_TOL, _np, assert_close, oracle_layer, oracle_stack, poison, run_layer
from workloads import cotangent, make_workload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import directional_mdlstm_handwriting_amd as M
    from directional_mdlstm_handwriting_amd.layer import DeviceParams, LayerGrads, PackedStack, flat_input


def sample(heights, widths, n_random, seed):
    h = np.asarray(heights, np.int64)
    w = np.asarray(widths, np.int64)
    idx = {int(np.argmax(h + w)), int(np.argmin(h * w))}
    rest = [e for e in range(len(h)) if e not in idx]
    idx.update(int(e) for e in np.random.default_rng(seed).choice(rest, n_random, replace=False))
    return sorted(idx)


def offsets(heights, widths, K):
    sizes = np.asarray(heights, np.int64) * np.asarray(widths, np.int64) * K
    return np.concatenate([[0], np.cumsum(sizes)])


@pytest.mark.parametrize("name,n_random,mode", [("word", 4, "packed"), ("word", 2, "exact"), ("line", 0, "packed")])
def test_layer_full_size_sampled(name, n_random, mode):
    wl = make_workload(name, 0)
    P, H, C = wl.layers[0], wl.H, wl.C
    idx = sample(wl.heights, wl.widths, n_random, 17)
    print(f"[gpu] full-size {name} ({mode}): {wl.n} images, sampled {idx}", flush=True)
    dys = [d if e in idx else np.zeros_like(d) for e, d in enumerate(cotangent(11, wl.heights, wl.widths, H))]
    g = run_layer(wl.heights, wl.widths, wl.xs, P, mode=mode, canvas_w_min=wl.canvas_w_min[0], sep=wl.sep,
                  x_dtype=wl.x_dtype, dys=dys)
    _, real = M.mdl_layout_rects(g["dl"].layout)
    y, dx = _np(g["layer"].y), _np(g["dx"])
    yo, xo = offsets(wl.heights, wl.widths, H), offsets(wl.heights, wl.widths, C)
    dW = [0.0] * 4
    sens = []
    for e in idx:
        h, w = int(wl.heights[e]), int(wl.widths[e])
        o = oracle_layer([h], [w], [wl.xs[e]], P, dys=[dys[e]])
        sn = o["sens"]
        sens.append(sn)
        y0, x0 = int(real[e][0]), int(real[e][1])
        assert_close(f"h_dirs[{e}]", _np(g["layer"].h_dirs[:, y0:y0 + h, x0:x0 + w, :]), o["hd"][:, :h, :w, :], F32_TOL,
                     sens=lambda sn=sn, h=h, w=w: sn()["hd"][:, :h, :w, :])
        assert_close(f"y[{e}]", y[yo[e]:yo[e + 1]], o["ys"][0], F32_TOL, sens=lambda sn=sn: sn()["ys"][0])
        if wl.x_dtype == "bf16":  # the bf16-input bound as well (the fp32 one above is stricter)
            assert_close(f"y[{e}] (bf16 bound)", y[yo[e]:yo[e + 1]], o["ys"][0], BF16_TOL)
        assert_close(f"dx[{e}]", dx[xo[e]:xo[e + 1]], o["dxs"][0], F32_TOL, sens=lambda sn=sn: sn()["dxs"][0])
        dW = [a + b for a, b in zip(dW, o["dW"])]
    others = np.ones(dx.size, bool)
    for e in idx:
        others[xo[e]:xo[e + 1]] = False
    assert np.all(dx[others] == 0.0), "input gradient of an example with zero upstream gradient"
    for k, (nm, got, ref) in enumerate(zip(("dWx", "dUl", "dUu", "db"), (g["g"].dWx, g["g"].dUl, g["g"].dUu, g["g"].db),
                                            dW)):
        assert_close(nm, _np(got), ref, F32_TOL, sens=lambda k=k: sum(sn()["dW"][k] for sn in sens))


def test_stack_full_size_sampled():
    wl = make_workload("stack", 0)
    idx = sample(wl.heights, wl.widths, 2, 23)
    print(f"[gpu] full-size stack: {wl.n} images, sampled {idx}", flush=True)
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
    # last-level sizes: each level divides by the 2 x 4 block, rounding up
    hL = [int(h) for h in wl.heights]
    wL = [int(w) for w in wl.widths]
    for _ in range(len(Hs) - 1):
        hL = [-(-h // 2) for h in hL]
        wL = [-(-w // 4) for w in wL]
    HL = Hs[-1]
    rng = np.random.default_rng(29)
    dys = [rng.standard_normal((hL[e], wL[e], HL)).astype(np.float32) if e in idx
           else np.zeros((hL[e], wL[e], HL), np.float32) for e in range(wl.n)]
    dy = torch.as_tensor(np.concatenate([d.reshape(-1) for d in dys]), device=DEV)
    lg = [LayerGrads(*(torch.full_like(t, float("nan")) for t in (p.Wx, p.Ul, p.Uu, p.b))) for p in params]
    cg = [(torch.full_like(W, float("nan")), torch.full_like(b, float("nan"))) for W, b in cdev]
    dx = torch.full((int(sum(x.size for x in wl.xs)),), float("nan"), device=DEV)
    st.backward(params, cdev, dy, lg, cg, dx_flat=dx)
    torch.cuda.synchronize()
    dx = _np(dx)
    yo, xo = offsets(hL, wL, HL), offsets(wl.heights, wl.widths, wl.C)
    lg_ref = [[0.0] * 4 for _ in Hs]
    cg_ref = [[0.0] * 2 for _ in wl.convs]
    sens = []
    for e in idx:
        h, w = int(wl.heights[e]), int(wl.widths[e])
        o = oracle_stack([h], [w], [wl.xs[e]], wl.layers, wl.convs, wl.canvas_w_min, [dys[e]])
        sn = o["sens"]
        sens.append(sn)
        assert_close(f"stack y[{e}]", y[yo[e]:yo[e + 1]], o["ys"][0], F32_TOL, sens=lambda sn=sn: sn()["ys"][0])
        assert_close(f"stack dx[{e}]", dx[xo[e]:xo[e + 1]], o["dxs"][0], F32_TOL, sens=lambda sn=sn: sn()["dxs"][0])
        lg_ref = [[a + b for a, b in zip(acc, r)] for acc, r in zip(lg_ref, o["lg"])]
        cg_ref = [[a + b for a, b in zip(acc, r)] for acc, r in zip(cg_ref, o["cg"])]
    others = np.ones(dx.size, bool)
    for e in idx:
        others[xo[e]:xo[e + 1]] = False
    assert np.all(dx[others] == 0.0), "input gradient of an example with zero upstream gradient"
    for lvl in range(len(Hs)):
        for k, (nm, got, ref) in enumerate(zip(("dWx", "dUl", "dUu", "db"),
                                               (lg[lvl].dWx, lg[lvl].dUl, lg[lvl].dUu, lg[lvl].db), lg_ref[lvl])):
            assert_close(f"L{lvl} {nm}", _np(got), ref, F32_TOL,
                         sens=lambda lvl=lvl, k=k: sum(sn()["lg"][lvl][k] for sn in sens))
    for j in range(len(wl.convs)):
        for k, nm in enumerate(("dW", "db")):
            assert_close(f"conv{j} {nm}", _np(cg[j][k]), cg_ref[j][k], F32_TOL,
                         sens=lambda j=j, k=k: sum(sn()["cg"][j][k] for sn in sens))
