"""The layer entry point without allocation (moe_ffn_forward_noalloc, static device scratch) against
moe_ffn_forward with a caller workspace: two calls in a row on one GPU, the second smaller than the
first (it reuses the scratch the first left behind), each bit-identical to the workspace entry point
and within the layer tolerance of the CPU oracle."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_w4a16_grouped_amd as moe  # noqa: E402


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _both(inp, layout):
    wl = inp.wl
    d = gu.DeviceInputs(inp)
    q13, s13, q2, s2 = d.w13_q, d.w13_s, d.w2_q, d.w2_s
    if layout == moe.MOE_LAYOUT_PACKED:
        q13, s13 = moe.moe_w4_prepack(q13, s13)
        q2, s2 = moe.moe_w4_prepack(q2, s2)
    y_ref = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids_ref = torch.full((wl.T, wl.k), -1, dtype=torch.int32, device="cuda")
    ws = torch.full((max(moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y_ref, topk_ids_out=ids_ref, workspace=ws,
                        weight_layout=layout)
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((wl.T, wl.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((wl.T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_ffn_forward_noalloc(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, topk_ids_out=ids, topk_w_out=w,
                                weight_layout=layout)
    torch.cuda.synchronize()
    return y_ref, ids_ref, y, ids, w


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_CANONICAL, moe.MOE_LAYOUT_PACKED])
def test_noalloc_matches_workspace_entry_point_twice(layout):
    # first call: 640 tokens over 64 experts top-6 (32-row tiles, separate routing launches);
    # second, smaller: 5 tokens over 128 experts top-8 (16-row tiles, routing in the gate_up prologue)
    for wl in (mi.custom("noalloc_big", 640, 64, 6, 512, 256, seed=41),
               mi.custom("noalloc_small", 5, 128, 8, 256, 128, seed=42)):
        print(f"noalloc layout={layout} {wl.name}: T={wl.T} E={wl.E} k={wl.k} H={wl.H} I={wl.I}", flush=True)
        assert moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k) <= moe.moe_ffn_noalloc_scratch_bytes()
        inp = mi.make_inputs(wl)
        y_ref, ids_ref, y, ids, w = _both(inp, layout)
        np.testing.assert_array_equal(_bits(y), _bits(y_ref))
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref.cpu().numpy())
        rid, rw = oracle.route(inp.logits, wl.k)
        np.testing.assert_array_equal(ids.cpu().numpy(), rid)
        assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= gu.ROUTE_W_ATOL
        tok = np.arange(0, wl.T, max(1, wl.T // 48))
        gu.assert_within_tolerance(gu.host_bf16_to_f64(y)[tok], oracle.moe_ffn(inp, tokens=tok), wl.name)


def test_noalloc_rejects_oversized_layer_without_launching():
    wl = mi.custom("noalloc_over", 4096, 8, 2, 4096, 14336, seed=43)
    assert moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k) > moe.moe_ffn_noalloc_scratch_bytes()
    x = torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((wl.T, wl.E), dtype=torch.float32, device="cuda")
    q13 = torch.zeros((wl.E, 2 * wl.I, wl.H // 2), dtype=torch.uint8, device="cuda")
    s13 = torch.zeros((wl.E, 2 * wl.I, wl.H // 32), dtype=torch.int16, device="cuda")
    q2 = torch.zeros((wl.E, wl.H, wl.I // 2), dtype=torch.uint8, device="cuda")
    s2 = torch.zeros((wl.E, wl.H, wl.I // 32), dtype=torch.int16, device="cuda")
    y = torch.full((wl.T, wl.H), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError, match="static"):
        moe.moe_ffn_forward_noalloc(x, lg, q13, s13, q2, s2, wl.k, y=y)
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))  # nothing was launched
