"""The exact fp16 path of the 64- and 128-row tiles: activations in fp16 with power-of-two exponents
(x per row, h per tile and 64 columns), weights dequantized to fp16 as code * scale.

Checked against the CPU oracle: the row conversion bit for bit against its rule; the grouped GEMMs
per element within the fp32 accumulation bound plus one fp16 rounding of h; the forms a step takes
when a group scale is outside fp16's exact range, when x rows are far larger than fp16's range and
when h blocks overflow it; and the layer on shapes that select these tiles."""
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


def _log(msg):
    print(msg, flush=True)


def _x_to_f16_rule(bits):
    """The conversion rule in numpy: e = floor(log2 max finite |x|) - 14 (0 for an all-zero row),
    clamped to [-110, 113]; x16 = fp16(x * 2^-e), round to nearest even."""
    x = mi.bf16_bits_to_f32(bits)
    a = np.abs(x.astype(np.float64))
    a[~np.isfinite(a)] = 0.0
    m = a.max(axis=1)
    _, ex = np.frexp(m)
    e = np.where(m > 0, ex - 1 - 14, 0).clip(-110, 113)
    x16 = (x * np.ldexp(np.float32(1.0), -e).astype(np.float32)[:, None]).astype(np.float16)
    return x16.view(np.uint16), e.astype(np.int32)


@pytest.mark.parametrize("T,H", [(37, 256), (5, 4096), (64, 168)])
def test_x_to_f16_matches_rule(T, H):
    rng = np.random.default_rng(T + H)
    x = rng.standard_normal((T, H), dtype=np.float32)
    x[1] *= 2.0 ** 40          # far above fp16's range
    x[2] *= 2.0 ** -30         # far below it
    x[3] = 0.0                 # all zero
    x[4, :5] = [np.inf, -np.inf, np.nan, 3.0e38, -7.0]  # non-finite values beside finite ones
    if T > 6:
        x[5, 7] = 2.0 ** 100   # one huge value: the rest of the row rounds toward fp16's subnormals
        x[6] *= 2.0 ** -120    # bf16 subnormal range
    bits = mi.f32_to_bf16_bits(x)
    x16, e = moe.moe_x_to_f16(gu.dev_bf16(bits))
    torch.cuda.synchronize()
    ref16, refe = _x_to_f16_rule(bits)
    np.testing.assert_array_equal(e.cpu().numpy(), refe)
    got = x16.view(torch.int16).cpu().numpy().view(np.uint16)
    nan = np.isnan(ref16.view(np.float16))
    np.testing.assert_array_equal(np.isnan(got.view(np.float16)), nan)
    np.testing.assert_array_equal(got[~nan], ref16[~nan])
    # every value at most 2^31 below its row's largest magnitude converts exactly
    xf = mi.bf16_bits_to_f32(bits).astype(np.float64)
    back = got.view(np.float16).astype(np.float64) * np.ldexp(1.0, refe)[:, None]
    fin = np.isfinite(xf)
    rowmax = np.where(fin, np.abs(xf), 0).max(axis=1, keepdims=True)
    exact = fin & (np.abs(xf) >= rowmax * 2.0 ** -31)
    np.testing.assert_array_equal(back[exact], xf[exact])


def _gate_up_case(E, T, k, H, I, seed, bm, layout, x_scale_rows=(), bad_scales=False):
    wl = mi.custom("f16gu", T, E, k, H, I, skew=True, seed=seed)
    inp = mi.make_inputs(wl)
    if x_scale_rows:
        xf = mi.bf16_bits_to_f32(inp.x)
        for r, sc in x_scale_rows:
            xf[r] *= sc
        inp.x = mi.f32_to_bf16_bits(xf)
    if bad_scales:
        s = mi.bf16_bits_to_f32(inp.w13_s)
        s[0, :, 1] = 2.0 ** -20   # below fp16's exact range: the step takes the fp32-scale form
        s[1 % E, 5, :] = 1.5 * 2.0 ** 13  # above it (6 * scale would exceed fp16's range)
        inp.w13_s = mi.f32_to_bf16_bits(s)
    return inp


@pytest.mark.parametrize("bm,layout", [(64, 0), (64, 1), (128, 1)])
@pytest.mark.parametrize("variant", ["plain", "huge_x_rows", "scales_out_of_range"])
def test_grouped_gemm_w4f16_gate_up(bm, layout, variant):
    E, T, k, H, I = 4, 260, 2, 384, 256
    inp = _gate_up_case(E, T, k, H, I, seed=bm + layout, bm=bm, layout=layout,
                        x_scale_rows=[(3, 2.0 ** 30), (11, 2.0 ** -40)] if variant == "huge_x_rows" else (),
                        bad_scales=variant == "scales_out_of_range")
    wl = inp.wl
    d = gu.DeviceInputs(inp)
    rid, _ = oracle.route(inp.logits, k)
    a = moe.moe_align(gu.dev(rid), E, bm)
    R = T * k
    q13, s13 = (d.w13_q, d.w13_s) if layout == 0 else moe.moe_w4_prepack(d.w13_q, d.w13_s)
    x16, xe = moe.moe_x_to_f16(d.x)
    h, he = moe.moe_grouped_gemm_w4f16(x16, xe, None, a["sorted_ids"], k, q13, s13, a["tiles"], a["max_tiles"],
                                       a["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, moe.MOE_OUT_H16,
                                       weight_layout=layout)
    torch.cuda.synchronize()
    ra = oracle.align(rid, E, bm)
    ref = oracle.grouped_proj(inp.x, ra["sorted_ids"], k, inp.w13_q, inp.w13_s, ra["offsets"], silu_mul=True)
    G = oracle.grouped_proj(inp.x, ra["sorted_ids"], k, inp.w13_q, inp.w13_s, ra["offsets"])
    Gabs = oracle.grouped_proj(inp.x & 0x7FFF, ra["sorted_ids"], k, inp.w13_q & 0x77, inp.w13_s, ra["offsets"])
    # decode h: row r's 32-column block j times 2^exp[r, j] where its tile's flag is set
    hv = h.float().cpu().numpy().astype(np.float64)
    flags = he[0].cpu().numpy().astype(np.int64)
    rexp = he[1].cpu().numpy().view(np.int8).astype(np.int64)  # signed exponents
    tiles = ra["tiles"]
    hexp = np.zeros((R, I // 32), np.int64)
    for i, (e_, row0, rows) in enumerate(tiles):
        hexp[row0:row0 + rows] = np.where(flags[i][None, :] != 0, rexp[row0:row0 + rows], 0)
    assert np.all((flags[:len(tiles)] != 0) == np.array([[hexp[r0:r0 + n, j].any() for j in range(I // 32)]
                                                          for (_, r0, n) in tiles]))
    hv *= np.ldexp(1.0, np.repeat(hexp, 32, axis=1))
    # fp32 sums of exact products (with the x conversion exact for these rows): (64 + H/32) * 2^-24
    # * sum|terms| for gate and up, propagated through silu(g) * u, then one fp16 rounding of h
    dG = (64 + H / 32) * 2.0 ** -24 * Gabs
    g, u, dg, du = G[:, :I], G[:, I:], dG[:, :I], dG[:, I:]
    scale = np.ldexp(1.0, np.repeat(hexp, 32, axis=1))
    bound = 2.0 ** -11 * np.abs(ref) + 1.1 * np.abs(u) * dg + np.abs(g) * du + 2.0 ** -25 * scale + 1e-6 * np.abs(ref)
    assert np.all(np.abs(hv - ref) <= bound), f"w4f16 gate_up bm={bm}: worst excess {np.max(np.abs(hv - ref) - bound)}"
    if variant == "huge_x_rows":
        assert hexp.max() > 0  # the huge rows' h overflowed fp16's range: their blocks carry exponents
        big = np.isin(ra["sorted_ids"] // k, [3, 11])  # (token 11 is 2^40 below the rest: scaled up)
        assert np.all(hexp[~big] == 0)  # ... and only theirs: the other rows of those tiles keep exponent 0
        assert hexp[np.isin(ra["sorted_ids"] // k, [11])].min() < 0
    elif variant == "plain":
        assert hexp.max() == 0


@pytest.mark.parametrize("bm,layout", [(64, 0), (128, 1)])
@pytest.mark.parametrize("out_dtype", [moe.MOE_OUT_F32, moe.MOE_OUT_F16E])
def test_grouped_gemm_w4f16_down_with_block_exponents(bm, layout, out_dtype):
    """Identity-row fp16 A whose 64-column blocks carry exponents (as h after an overflow): values
    chosen exact in bf16 and fp16 alike, so the oracle sees the same A."""
    E, T, k, N, K = 3, 200, 2, 256, 384
    rng = np.random.default_rng(bm + out_dtype)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    rid, _ = oracle.route(logits, k)
    R = T * k
    a = moe.moe_align(gu.dev(rid), E, bm)
    ra = oracle.align(rid, E, bm)
    A16 = (rng.integers(-128, 128, (R, K)) / 32.0).astype(np.float32)  # exact in bf16 and fp16 alike
    nt = a["max_tiles"]
    nb = K // 32
    rexp = np.zeros((R, nb), np.int8)
    rexp[::7, 1] = 20          # a few rows with a large block
    rexp[3::11, -1] = 3
    rexp[5::13, 4] = 9
    rexp[6::17, 3] = -12       # and a small one
    flags = np.zeros((nt, nb), np.uint8)
    for i, (e_, row0, rows) in enumerate(ra["tiles"]):
        flags[i] = rexp[row0:row0 + rows].any(axis=0)
    rexp_dev = rexp.copy()
    rexp_dev[:, 2] = 77        # unflagged block 2: its row bytes must be ignored
    Atrue = A16.astype(np.float64) * np.ldexp(1.0, np.repeat(rexp.astype(np.int64), 32, axis=1))
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    Ws = mi.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    wq, ws = gu.dev(Wq), gu.dev(Ws.view(np.int16))
    if layout:
        wq, ws = moe.moe_w4_prepack(wq, ws)
    flags[:, 2] = 0
    out = moe.moe_grouped_gemm_w4f16(gu.dev(A16.astype(np.float16)), None,
                                     (gu.dev(flags), gu.dev(rexp_dev.view(np.uint8))), None, 1,
                                     wq, ws,
                                     a["tiles"], nt, a["num_tiles"], bm, moe.MOE_EPI_NONE, R, out_dtype,
                                     weight_layout=layout)
    torch.cuda.synchronize()
    Ab = mi.f32_to_bf16_bits(Atrue.astype(np.float32))  # exact: bf16 values times powers of two
    ref = oracle.grouped_proj(Ab, None, 1, Wq, Ws, ra["offsets"])
    ref_abs = oracle.grouped_proj(Ab & 0x7FFF, None, 1, Wq & 0x77, Ws, ra["offsets"])
    acc_err = (64 + K / 32) * 2.0 ** -24 * ref_abs
    if out_dtype == moe.MOE_OUT_F32:
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= acc_err)
    else:
        from tests.test_gpu_parity import f16e_to_f64
        got, ex = f16e_to_f64(*out)
        sc = np.repeat(np.ldexp(1.0, ex), 8, axis=1)
        assert np.all(np.abs(got - ref) <= acc_err + 2.0 ** -11 * (np.abs(ref) + acc_err) + 2.0 ** -25 * sc)


def _forward(inp, layout):
    wl = inp.wl
    d = gu.DeviceInputs(inp)
    q13, s13, q2, s2 = d.w13_q, d.w13_s, d.w2_q, d.w2_s
    if layout == moe.MOE_LAYOUT_PACKED:
        q13, s13 = moe.moe_w4_prepack(q13, s13)
        q2, s2 = moe.moe_w4_prepack(q2, s2)
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((max(moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, workspace=ws, weight_layout=layout)
    torch.cuda.synchronize()
    return gu.host_bf16_to_f64(y)


@pytest.mark.parametrize("case", ["plain", "ragged", "hot", "huge_rows", "bad_scales"])
def test_layer_on_fp16_path(case):
    """Layers whose experts average more than 256 rows with packed weights (128-row tiles, the exact
    fp16 path), against the oracle at the layer tolerance."""
    layout = moe.MOE_LAYOUT_PACKED
    if case == "ragged":
        wl = mi.custom("f16_ragged", 700, 2, 1, 256, 128, seed=51)  # 350 rows per expert: partial tiles
    else:
        wl = mi.custom("f16_" + case, 600, 2, 1, 256, 256, seed=52)  # 300 rows per expert
    inp = mi.make_inputs(wl)
    if case == "hot":
        inp.logits[:, 0] += 50.0
    if case == "huge_rows":
        xf = mi.bf16_bits_to_f32(inp.x)
        xf[::17] *= 2.0 ** 30   # gate and up near 2^30: h near 2^60, far beyond fp16's range
        xf[5::23] *= 2.0 ** -40
        inp.x = mi.f32_to_bf16_bits(xf)
    if case == "bad_scales":
        s = mi.bf16_bits_to_f32(inp.w2_s)
        s[0, ::3, 0] = 2.0 ** -21
        s[1, 7, :] = 1.25 * 2.0 ** 14
        inp.w2_s = mi.f32_to_bf16_bits(s)
        s = mi.bf16_bits_to_f32(inp.w13_s)
        s[1, 3, 2] = 2.0 ** -19
        inp.w13_s = mi.f32_to_bf16_bits(s)
    _log(f"fp16-path layer {wl.name} block_m={moe.moe_ffn_block_m(wl.T, wl.E, wl.k, layout)}")
    assert moe.moe_ffn_block_m(wl.T, wl.E, wl.k, layout) == 128
    got = _forward(inp, layout)
    ref = oracle.moe_ffn(inp)
    if case == "huge_rows":
        # rows 2^70 apart: the layer bound applies to each token row against its own rms (y's bf16
        # rounding alone would exceed a bound taken over the mixed rows' rms)
        assert np.all(np.isfinite(got))
        for t in range(wl.T):
            r = gu.tolerance_report(got[t:t + 1], ref[t:t + 1])
            assert r["max_over_rms"] <= gu.MAX_ABS_OVER_RMS and r["mean_rel"] <= 4 * gu.MEAN_REL, (t, r)
        r = gu.tolerance_report(got, ref)
        assert r["mean_rel"] <= gu.MEAN_REL, r
    elif case == "bad_scales":
        # output column 7 of expert 1 is 2^14 times larger than the rest: each part against its own rms
        # (y's bf16 rounding of that column alone would exceed a bound over the mixed rms)
        rest = np.ones(wl.H, bool)
        rest[7] = False
        gu.assert_within_tolerance(got[:, rest], ref[:, rest], wl.name + " (other columns)")
        r = gu.assert_within_tolerance(got[:, 7:8], ref[:, 7:8], wl.name + " (column 7)")
    else:
        r = gu.assert_within_tolerance(got, ref, wl.name)
    _log(f"  {r}")
