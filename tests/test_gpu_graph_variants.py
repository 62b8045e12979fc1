"""HIP-graph capture of the quantized layers (MXFP4, W4A8, FP8): each layer captured once and replayed
several times, with eager work (re-poisoning the workspace and the output) and synchronisation in
between; every replay must reproduce the eager output bits.  The layers record no memset and no host
synchronisation, so a replay recomputes everything from the inputs."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_w4a16_grouped_amd as moe  # noqa: E402  (loads the HIP library; fails loudly if missing)


def _layer(method, wl):
    """(callable(y, ws), workspace bytes) of one quantized layer on seeded inputs."""
    if method == "f8":
        inp = mi.make_f8_inputs(wl)
        w = (gu.dev(inp.w13_q), gu.dev(inp.w13_s), gu.dev(inp.w2_q), gu.dev(inp.w2_s))
        fwd, wsb, layout = moe.moe_ffn_forward_f8, moe.moe_ffn_f8_workspace_bytes, None
    else:
        inp = mi.make_mx_inputs(wl)
        w = moe.moe_mx_prepack(gu.dev(inp.w13_q), gu.dev(inp.w13_e)) + moe.moe_mx_prepack(gu.dev(inp.w2_q),
                                                                                          gu.dev(inp.w2_e))
        fwd = moe.moe_ffn_forward_mxfp4 if method == "mxfp4" else moe.moe_ffn_forward_w4a8
        wsb = moe.moe_ffn_mxfp4_workspace_bytes if method == "mxfp4" else moe.moe_ffn_w4a8_workspace_bytes
        layout = moe.MOE_LAYOUT_PACKED
    x, logits = gu.dev_bf16(inp.x), gu.dev(inp.logits)
    kw = {} if layout is None else {"weight_layout": layout}

    def run(y, ws):
        fwd(x, logits, *w, wl.k, y=y, workspace=ws, **kw)

    return run, wsb(wl.T, wl.H, wl.I, wl.E, wl.k)


@pytest.mark.parametrize("method", ["mxfp4", "w4a8", "f8"])
@pytest.mark.parametrize("name", ["dec8", "pre800"])
def test_quantized_layer_graph_replays_match_eager(method, name):
    wl = mi.WORKLOADS[name]
    print(f"graph replay {method} {name}", flush=True)
    run, wsb = _layer(method, wl)
    ws = torch.full((max(wsb, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    y_ref = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    run(y_ref, ws)
    torch.cuda.synchronize()
    ref = y_ref.view(torch.int16).cpu().numpy()
    assert np.all(np.isfinite(gu.host_bf16_to_f64(y_ref)))
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(y, ws)
    for rep in range(3):
        y.fill_(float("nan"))
        ws.fill_(0xFF)  # eager work between replays: poison what the replay must rewrite
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.view(torch.int16).cpu().numpy(), ref)
