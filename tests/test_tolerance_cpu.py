"""The parity criterion of the GPU tests, pinned on the CPU with the oracle (no GPU needed).

* an output rounded to fp32 passes the elementwise bound;
* a planted error of 1 % in one element, or of 1e-3 of the largest magnitude, fails it, and also fails the
  conditioning fallback, whose one-ulp perturbation response is far smaller on a well-conditioned case;
* on a long chain the one-ulp response of the weight gradients is large (the recurrence is ill-conditioned),
  and an error of K_COND times that response plus a margin still fails.
"""

import numpy as np
import pytest

from test_gpu_parity import F32_TOL, K_COND, assert_close, oracle_layer
from workloads import cotangent, make_workload, random_images, random_layer


def _tiny():
    wl = make_workload("tiny", 0)
    dys = cotangent(0, wl.heights, wl.widths, wl.H)
    return oracle_layer(wl.heights, wl.widths, wl.xs, wl.layers[0], canvas_w_min=8, dys=dys)


def test_fp32_rounding_passes():
    o = _tiny()
    for ref in (o["hd"], o["dW"][0], o["dW"][1]):
        assert_close("rounded", np.asarray(ref, np.float32), ref, F32_TOL)


@pytest.mark.parametrize("k", [0, 1, 2])
def test_planted_errors_fail(k):
    o = _tiny()
    ref = np.asarray(o["dW"][k], np.float64).reshape(-1)
    sens = lambda: o["sens"]()["dW"][k]
    i = int(np.argmax(np.abs(ref)))
    bad = ref.copy()
    bad[i] *= 1.01                                      # 1 % in the largest element
    with pytest.raises(AssertionError):
        assert_close("planted", bad, ref, F32_TOL, sens=sens)
    bad = ref.copy()
    bad[len(ref) // 2] += 1e-3 * np.max(np.abs(ref))    # 1e-3 of the scale in a middle element
    with pytest.raises(AssertionError):
        assert_close("planted", bad, ref, F32_TOL, sens=sens)


def test_long_chain_response_bounds_the_fallback():
    h, w, C, H = [2, 3], [60, 9], 4, 8
    P = random_layer(7, C, H)
    xs = random_images(8, h, w, C)
    dys = cotangent(9, h, w, H)
    o = oracle_layer(h, w, xs, P, canvas_w_min=64, dys=dys)
    ref = np.asarray(o["dW"][1], np.float64).reshape(-1)
    resp = np.abs(np.asarray(o["sens"]()["dW"][1])).max()
    assert resp > 0
    bad = ref.copy()
    bad[0] += 3 * K_COND * resp + 1e-4 * max(1.0, np.abs(ref).max())
    with pytest.raises(AssertionError):
        assert_close("planted", bad, ref, F32_TOL, sens=lambda: o["sens"]()["dW"][1])
