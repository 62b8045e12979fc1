"""MOE_DUMP=1: the layer entry point prints one line of diagnostics per call and leaves its results
bit for bit unchanged.  Every field of the line is checked against what it reports, computed here
from the inputs, the oracle's routing and the layer's own output: rows per expert and tile counts
from the oracle's routing (bit-exact by the routing tests), the ten largest logits of token 0 from
the logits, and the norms of x and y in fp64."""
import re

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_w4a16_grouped_amd as moe  # noqa: E402  (loads the HIP library; fails loudly if missing)

LINE = re.compile(
    r"moe_dump: T=(\d+) H=(\d+) I=(\d+) E=(\d+) k=(\d+) block_m=(\d+) tiles=(\d+) rows_per_expert "
    r"min=(\d+) max=(\d+) empty=(\d+) max_tiles_per_expert=(\d+) logits0_top=\[([^\]]*)\] "
    r"x_norm=(\S+) y_norm=(\S+)$")


def _bits(t):
    return t.view(torch.int16).cpu().numpy().copy()


@pytest.mark.parametrize("name", ["tiny", "dec8", "pre800"])
def test_dump_line_and_unchanged_output(name, monkeypatch, capfd):
    wl = mi.WORKLOADS[name]
    inp = mi.make_inputs(wl)
    d = gu.DeviceInputs(inp)
    print(f"MOE_DUMP {name}", flush=True)
    monkeypatch.delenv("MOE_DUMP", raising=False)
    y0 = moe.moe_ffn_forward(d.x, d.logits, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k)
    torch.cuda.synchronize()
    capfd.readouterr()
    monkeypatch.setenv("MOE_DUMP", "1")
    y1 = moe.moe_ffn_forward(d.x, d.logits, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    monkeypatch.delenv("MOE_DUMP")
    np.testing.assert_array_equal(_bits(y1), _bits(y0))

    lines = [l for l in err.splitlines() if l.startswith("moe_dump:")]
    assert len(lines) == 1, err
    m = LINE.match(lines[0])
    assert m, lines[0]
    T, H, I, E, k, bm, tiles, cmin, cmax, empty, tmax = (int(v) for v in m.groups()[:11])
    assert (T, H, I, E, k) == (wl.T, wl.H, wl.I, wl.E, wl.k)
    assert bm == moe.moe_ffn_block_m(wl.T, wl.E, wl.k, moe.MOE_LAYOUT_CANONICAL)

    rid, _ = oracle.route(inp.logits, wl.k)
    counts = np.bincount(rid.ravel(), minlength=wl.E)
    per_expert_tiles = (counts + bm - 1) // bm
    assert (cmin, cmax, empty) == (counts.min(), counts.max(), int((counts == 0).sum()))
    assert tiles == int(per_expert_tiles.sum())
    assert tmax == int(per_expert_tiles.max())

    top = [p.split(":") for p in m.group(12).split()]
    row = inp.logits[0].astype(np.float64)
    order = sorted(range(wl.E), key=lambda e: (-row[e], e))[:min(10, wl.E)]
    assert [int(e) for e, _ in top] == order
    np.testing.assert_allclose([float(v) for _, v in top], row[order], rtol=1e-5, atol=1e-12)

    x64 = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    assert float(m.group(13)) == pytest.approx(np.linalg.norm(x64), rel=1e-7)
    assert float(m.group(14)) == pytest.approx(np.linalg.norm(gu.host_bf16_to_f64(y1)), rel=1e-7)


def test_dump_off_unless_exactly_one(monkeypatch, capfd):
    wl = mi.WORKLOADS["tiny"]
    inp = mi.make_inputs(wl)
    d = gu.DeviceInputs(inp)
    for v in ("0", "", "yes", "11"):
        monkeypatch.setenv("MOE_DUMP", v)
        moe.moe_ffn_forward(d.x, d.logits, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k)
        torch.cuda.synchronize()
        assert "moe_dump:" not in capfd.readouterr().err, v
    monkeypatch.delenv("MOE_DUMP")
