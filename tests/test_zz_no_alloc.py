"""The block-conv backward that allocates nothing (mdl_blockconv_backward_noalloc) against the workspace form
(mdl_blockconv_backward), through the C ABI: the same kernels in the same order, so dh, dWc and dbc must be
bit-identical. Two calls in a row share the library's fixed scratch; the second is smaller (fewer examples,
a smaller hidden size and output count), so it runs over the first call's leftover partials."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(heights, widths, H, Cout, cw_k, cw_k1, seed):
    import directional_mdlstm_handwriting_amd as M
    from directional_mdlstm_handwriting_amd.layer import DeviceLayout
    print(f"[gpu] no-alloc block conv: n={len(heights)} H={H} Cout={Cout}", flush=True)
    dk = DeviceLayout(heights, widths, cw_k, 1, "packed", DEV)
    dk1 = DeviceLayout(None, None, 0, device=DEV, layout=M.mdl_pack_level(dk.layout, 2, 4, cw_k1, 1))
    g = torch.Generator(device="cpu").manual_seed(seed)
    hk = torch.randn(4, dk.layout.Hc, dk.layout.Wc, H, generator=g).to(DEV)
    dx1 = torch.randn(dk1.layout.Hc, dk1.layout.Wc, Cout, generator=g).to(DEV)
    W = (0.1 * torch.randn(Cout, 4, H, 2, 4, generator=g)).to(DEV)
    nb = M.mdl_blockconv_workspace_size(dk1.layout, H, 2, 4, Cout)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=DEV)

    def run(noalloc):
        dh = torch.full_like(hk, float("nan"))
        dW = torch.full_like(W, float("nan"))
        db = torch.full((Cout,), float("nan"), device=DEV)
        if noalloc:
            M.mdl_blockconv_backward_noalloc(dk.layout, dk.desc, dk1.layout, dk1.desc, hk, H, 2, 4, W, Cout, dx1, dh,
                                             dW, db)
        else:
            M.mdl_blockconv_backward(dk.layout, dk.desc, dk1.layout, dk1.desc, hk, H, 2, 4, W, Cout, dx1, dh, dW, db,
                                     ws, nb)
        torch.cuda.synchronize()
        return dh, dW, db

    return run


def test_noalloc_matches_workspace_form_twice():
    big = _case([9, 14, 6, 12, 20, 33, 40], [30, 17, 40, 9, 51, 120, 77], 10, 20, 128, 64, 1)
    small = _case([5, 8], [12, 9], 2, 6, 16, 8, 2)
    for run in (big, small):
        ref = run(False)
        got = run(True)
        for name, a, b in zip(("dh", "dWc", "dbc"), got, ref):
            assert torch.isfinite(a).all(), name
            assert torch.equal(a, b), name
    # and the large case again after the small one
    ref = big(False)
    got = big(True)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
