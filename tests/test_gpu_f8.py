"""GPU parity of the FP8 (W8A8, per-1x128) variant against the CPU oracle.

The activation quantizer is bit-exact: both sides take every decision on the same fp32 values (the
block maximum, s = amax / 448 by fp32 division, the fp32 quotient v / s, nearest-even E4M3).

The FP8 matrix instruction does not sum its 128 products in fp32: it aligns them to the largest
product and keeps 13 bits below that product's leading bit (measured on MI355X: a product 2^-13.2
below the largest is lost; partial bits are truncated toward zero; products within a few binades of
each other sum exactly).  Hence two kinds of grouped-GEMM checks:
  * operands whose products span few binades: the instruction's sums are exact, and outputs must be
    within the fp32 bound of the scale products and the accumulation, relative to sum |terms|;
  * operands over the full E4M3 range: per K step each of the 128 products can lose less than
    2^-13 of the largest, so the step's error is below 2^-6 * max|a| * max|w| * s_a * s_w.
In the layer, h is quantized from the GPU's fp32 h and in the oracle from its fp64 h.  Where h lies
within rounding of a decision boundary the codes can differ by one E4M3 step, so layer outputs are
held to the layer tolerance (max|gpu-ref| <= 3e-2 * rms(ref), mean relative error <= 5e-3) plus,
per output, the effect of exactly those elements of the oracle's h whose quotient lies within a
relative 2^-8 of a rounding midpoint: one E4M3 step each, through |W2| and the routing weight.
"""
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


def _log(msg):
    print(msg, flush=True)


class F8Device:
    def __init__(self, inp):
        self.inp = inp
        self.x = gu.dev_bf16(inp.x)
        self.logits = gu.dev(inp.logits)
        self.w13_q, self.w13_s = gu.dev(inp.w13_q), gu.dev(inp.w13_s)
        self.w2_q, self.w2_s = gu.dev(inp.w2_q), gu.dev(inp.w2_s)


# ---------------------------------------------------------------------------------------------------
# activation quantization

def _planted_block(K):
    v = np.zeros(K, np.float32)
    # amax 448 -> s = 1: ties between adjacent codes, the subnormal range, -0.0 in a live block
    v[:10] = [448.0, 1.0625, 1.1875, -3.0, 2.0 ** -10, 3 * 2.0 ** -9, -0.0, 20.0, 300.0, -2.0 ** -9]
    return v


@pytest.mark.parametrize("rows,K", [(1, 128), (7, 384), (33, 2048), (300, 4096)])
@pytest.mark.parametrize("in_f32", [False, True])
def test_f8_quantize_bit_exact(rows, K, in_f32):
    rng = np.random.default_rng(rows + K + in_f32)
    v = rng.standard_normal((rows, K)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (rows, 1))).astype(np.float32)
    v[0, :128] = 0.0                      # all-zero block
    if K >= 256:
        v[0, 128:256] = _planted_block(128)
    if in_f32:
        xin = gu.dev(v)
        ref_in = v.astype(np.float64)
    else:
        bits = mi.f32_to_bf16_bits(v)
        xin = gu.dev_bf16(bits)
        ref_in = mi.bf16_bits_to_f32(bits).astype(np.float64)
    q, s = moe.moe_f8_quantize(xin)
    torch.cuda.synchronize()
    rq, rs = oracle.f8_quantize(ref_in)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_f8_quantize_every_code_boundary():
    # amax 448 makes s = 1, so each quotient is the value itself: every midpoint between adjacent
    # E4M3 magnitudes and its fp32 neighbours, both signs, must round as the oracle rounds
    mags = np.sort(np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float32))
    mids = (mags[1:] + mags[:-1]) / np.float32(2)
    vals = np.concatenate([mags, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    n = ((len(vals) + 126) // 127) * 127
    vals = np.resize(vals, n).reshape(-1, 127)
    v = np.concatenate([np.full((vals.shape[0], 1), 448.0, np.float32), vals], axis=1)
    q, s = moe.moe_f8_quantize(gu.dev(np.ascontiguousarray(v)))
    torch.cuda.synchronize()
    rq, rs = oracle.f8_quantize(v.astype(np.float64))
    assert np.all(rs == 1.0)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


# ---------------------------------------------------------------------------------------------------
# grouped GEMM

def _routing(T, E, k, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    return ids, oracle.align(ids, E, bm)


def _narrow_codes(rng, shape):
    # exponent fields 6..8 (magnitudes 0.5 .. 3.75): products of two such codes span under 6 binades,
    # which the instruction sums exactly
    sign = rng.integers(0, 2, shape, dtype=np.uint8) << 7
    return sign | (rng.integers(6, 9, shape, dtype=np.uint8) << 3) | rng.integers(0, 8, shape, dtype=np.uint8)


def _f8_operands(rows, N, K, E, seed, full_range=False):
    rng = np.random.default_rng(seed)
    codes = mi.e4m3_codes_uniform if full_range else _narrow_codes
    Aq = codes(rng, (rows, K))
    As = rng.uniform(0.25, 4.0, (rows, K // 128)).astype(np.float32)
    Wq = codes(rng, (E, N, K))
    Ws = rng.uniform(1e-4, 1e-3, (E, N, K // 128)).astype(np.float32)
    return Aq, As, Wq, Ws


def _f8_bound_terms(K):
    # exact instruction sums; per K step two roundings of the scale products and one of the
    # accumulation, and the final fp32 value: at most (3 K/128 + 8) * 2^-24 relative to sum |terms|
    return (3 * K / 128 + 8) * 2.0 ** -24


_E4M3 = np.array([oracle.e4m3_value(c) if (c & 0x7F) != 0x7F else 0.0 for c in range(256)])


def _truncation_bound(Aq, As, a_rows, Wq, Ws, offsets):
    """Per-output bound of the instruction's alignment loss over the full code range:
    sum over K steps of 2^-6 * max|a| * max|w| * s_a * s_w (rows in permuted order)."""
    K = Aq.shape[1]
    amax = np.abs(_E4M3[Aq]).reshape(Aq.shape[0], K // 128, 128).max(axis=2) * As
    out = np.zeros((len(a_rows), Wq.shape[1]))
    for e in range(Wq.shape[0]):
        wmax = np.abs(_E4M3[Wq[e]]).reshape(Wq.shape[1], K // 128, 128).max(axis=2) * Ws[e]
        r0, r1 = offsets[e], offsets[e + 1]
        out[r0:r1] = 2.0 ** -6 * (amax[a_rows[r0:r1]] @ wmax.T)
    return out


# (T, E, k, bm): few tiles take the K-split kernel, more tiles the N-split ones
GEMM_CASES = [(3, 8, 2, 16), (40, 16, 4, 16), (90, 12, 3, 32), (300, 8, 2, 64), (600, 4, 2, 128)]


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
@pytest.mark.parametrize("N,K", [(256, 2048), (200, 384), (48, 128)])
def test_grouped_gemm_f8_plain(T, E, k, bm, N, K):
    _log(f"f8 gemm T={T} E={E} k={k} bm={bm} N={N} K={K}")
    ids, al = _routing(T, E, k, bm, seed=T * 7 + N)
    R = T * k
    Aq, As, Wq, Ws = _f8_operands(R, N, K, E, seed=K + bm)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    C = torch.full((R, N), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_gemm_f8(gu.dev(Aq), gu.dev(As), None, 1, gu.dev(Wq), gu.dev(Ws), tiles, al["num_tiles"], nt, bm,
                            moe.MOE_EPI_NONE, R, C=C)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_f8(Aq, As, None, 1, Wq, Ws, al["offsets"])
    ref_abs = oracle.grouped_proj_f8(Aq & 0x7F, As, None, 1, Wq & 0x7F, Ws, al["offsets"])
    assert np.all(np.isfinite(got)), "rows not written"
    assert np.all(np.abs(got - ref) <= _f8_bound_terms(K) * ref_abs + 1e-30)
    # bf16 output: one more rounding
    Cb = moe.moe_grouped_gemm_f8(gu.dev(Aq), gu.dev(As), None, 1, gu.dev(Wq), gu.dev(Ws), tiles, al["num_tiles"], nt,
                                 bm, moe.MOE_EPI_NONE, R, out_dtype=moe.MOE_OUT_BF16)
    torch.cuda.synchronize()
    gotb = gu.host_bf16_to_f64(Cb)
    assert np.all(np.abs(gotb - ref) <= 2.0 ** -8 * np.abs(ref) + _f8_bound_terms(K) * ref_abs + 1e-30)


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
def test_grouped_gemm_f8_full_code_range(T, E, k, bm):
    N, K = 192, 1024
    _log(f"f8 gemm full range T={T} E={E} k={k} bm={bm}")
    ids, al = _routing(T, E, k, bm, seed=T * 5 + 1)
    R = T * k
    Aq, As, Wq, Ws = _f8_operands(R, N, K, E, seed=bm + 77, full_range=True)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    C = moe.moe_grouped_gemm_f8(gu.dev(Aq), gu.dev(As), None, 1, gu.dev(Wq), gu.dev(Ws), tiles, al["num_tiles"], nt,
                                bm, moe.MOE_EPI_NONE, R)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_f8(Aq, As, None, 1, Wq, Ws, al["offsets"])
    ref_abs = oracle.grouped_proj_f8(Aq & 0x7F, As, None, 1, Wq & 0x7F, Ws, al["offsets"])
    bound = _truncation_bound(Aq, As, np.arange(R), Wq, Ws, al["offsets"]) + _f8_bound_terms(K) * ref_abs
    assert np.all(np.abs(got - ref) <= bound), f"worst excess {np.max(np.abs(got - ref) - bound)}"
    rel = np.abs(got - ref).sum() / np.abs(ref).sum()
    _log(f"  mean relative error {rel:.2e}")
    assert rel <= 1e-3


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
@pytest.mark.parametrize("I,K", [(128, 2048), (64, 384)])
def test_grouped_gemm_f8_silu_mul(T, E, k, bm, I, K):
    _log(f"f8 gemm silu T={T} E={E} k={k} bm={bm} I={I} K={K}")
    ids, al = _routing(T, E, k, bm, seed=T + I)
    R = T * k
    Aq, As, Wq, Ws = _f8_operands(T, 2 * I, K, E, seed=I + bm)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    h = moe.moe_grouped_gemm_f8(gu.dev(Aq), gu.dev(As), srt, k, gu.dev(Wq), gu.dev(Ws), tiles, al["num_tiles"], nt,
                                bm, moe.MOE_EPI_SILU_MUL, R)
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_f8(Aq, As, al["sorted_ids"], k, Wq, Ws, al["offsets"], silu_mul=True)
    G = oracle.grouped_proj_f8(Aq, As, al["sorted_ids"], k, Wq, Ws, al["offsets"])
    Gabs = oracle.grouped_proj_f8(Aq & 0x7F, As, al["sorted_ids"], k, Wq & 0x7F, Ws, al["offsets"])
    dG = _f8_bound_terms(K) * Gabs
    g, u, dg, du = G[:, :I], G[:, I:], dG[:, :I], dG[:, I:]
    # silu(g) * u in fp32 with the fast exponential and reciprocal: a few ulps of |h|, plus the
    # propagated sum errors (|d silu/dg| <= 1.1, |silu(g)| <= |g|)
    bound = 2.0 ** -18 * np.abs(ref) + 1.1 * np.abs(u) * dg + np.abs(g) * du + 1e-30
    assert np.all(np.abs(got - ref) <= bound), f"worst excess {np.max(np.abs(got - ref) - bound)}"


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
def test_f8_h_quantization_close_to_oracle(T, E, k, bm):
    # gate_up (fp32 h) -> FP8 quantization on the GPU against the oracle's quantization of its fp64 h
    ids, al = _routing(T, E, k, bm, seed=T + 3)
    R, I, H = T * k, 256, 512
    rng = np.random.default_rng(bm + T)
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    inp = mi.make_f8_inputs(mi.custom("f8h", 1, E, 1, H, I, seed=4))
    xq, xs = moe.moe_f8_quantize(gu.dev_bf16(x))
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    h = moe.moe_grouped_gemm_f8(xq, xs, srt, k, gu.dev(inp.w13_q), gu.dev(inp.w13_s), tiles, al["num_tiles"], nt, bm,
                                moe.MOE_EPI_SILU_MUL, R)
    hq, hs = moe.moe_f8_quantize(h)
    torch.cuda.synchronize()
    rxq, rxs = oracle.f8_quantize(mi.bf16_bits_to_f32(x).astype(np.float64))
    np.testing.assert_array_equal(xq.cpu().numpy(), rxq)
    h_ref = oracle.grouped_proj_f8(rxq, rxs, al["sorted_ids"], k, inp.w13_q, inp.w13_s, al["offsets"], silu_mul=True)
    rq, rs = oracle.f8_quantize(h_ref)
    gq, gs = hq.cpu().numpy(), hs.cpu().numpy()
    code_diff = np.mean(gq != rq)
    _log(f"  h codes differing {code_diff:.2e}, scale rel diff {np.max(np.abs(gs / rs - 1)):.2e}")
    # the GPU's h is within a relative 2^-10 of the oracle's here, so its block scales are too, and a
    # code may differ only where the oracle's quotient lies near a rounding midpoint, by one step
    assert np.all(np.abs(gs / rs - 1) <= 2.0 ** -10)
    near, move = _near_midpoint(h_ref, rq, rs)
    differs = gq != rq
    assert np.all(near[differs]), "a code differs away from any rounding boundary"
    deq_g = oracle.f8_dequant(gq, gs)
    deq_r = oracle.f8_dequant(rq, rs)
    worst = np.max((np.abs(deq_g - deq_r) / move)[differs], initial=0.0)
    _log(f"  worst differing element moved {worst:.3f} of its allowance")
    assert worst <= 1.01
    assert code_diff <= 0.02


_MAGS = np.sort(np.unique(np.abs(_E4M3[:0x7F])))
_MIDS = (_MAGS[1:] + _MAGS[:-1]) / 2
NEAR_REL = 2.0 ** -8  # relative distance to a rounding midpoint within which a code may differ
# ... plus an absolute floor (in quotient units): the GPU's error in h follows the size of the terms
# summed, not h itself, so near-zero h can move by about 2^-13 of the block's largest quotient (448)
NEAR_ABS = 448.0 * 2.0 ** -13


def _near_midpoint(h, q, s):
    """For values h [rows, K] quantized by the oracle to (q, s): which elements have a quotient
    h / s within NEAR_REL (relative) plus NEAR_ABS of a rounding midpoint, and how far such an
    element's dequantized value can move: that distance plus one E4M3 step (the larger of the two
    gaps around the quotient), times s."""
    S = np.repeat(np.asarray(s, np.float64), 128, axis=1)
    a = np.abs(np.where(S > 0, h / np.where(S > 0, S, 1), 0.0))
    i = np.clip(np.searchsorted(_MIDS, a), 1, len(_MIDS) - 1)
    dist = np.minimum(np.abs(a - _MIDS[i - 1]), np.abs(a - _MIDS[i]))
    near = (dist <= NEAR_REL * a + NEAR_ABS) & (S > 0)
    j = np.clip(np.searchsorted(_MAGS, a), 1, len(_MAGS) - 1)
    gap = np.maximum(_MAGS[j] - _MAGS[j - 1], _MAGS[np.minimum(j + 1, len(_MAGS) - 1)] - _MAGS[j])
    return near, (gap + NEAR_REL * a + NEAR_ABS) * S


def _flip_allowance(inp, tok):
    """Per output of the sampled tokens: sum over slots of w * |W2_e| @ (how far each h element near a
    rounding midpoint can move), from oracle quantities only."""
    wl = inp.wl
    y, h = oracle.moe_ffn_f8(inp, tokens=tok, diagnostics=True)
    ids, w = oracle.route(inp.logits, wl.k)
    n, k, I = h.shape
    q, s = oracle.f8_quantize(h.reshape(n * k, I))
    near, move = _near_midpoint(h.reshape(n * k, I), q, s)
    dev = (near * move).reshape(n, k, I)
    allow = np.zeros((n, wl.H))
    w2 = {}
    for j, t in enumerate(tok):
        for slot in range(k):
            e = int(ids[t, slot])
            if not dev[j, slot].any():
                continue
            if e not in w2:
                w2[e] = np.abs(oracle.f8_dequant(inp.w2_q[e], inp.w2_s[e]))
            allow[j] += w[t, slot] * (w2[e] @ dev[j, slot])
    return y, allow, float(np.mean(near))


def _assert_layer(yh, inp, tok, label):
    ref, allow, near_frac = _flip_allowance(inp, tok)
    d = np.abs(yh - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    r = gu.tolerance_report(yh, ref)
    # one bf16 rounding of y on top of the allowance
    excess = d - (gu.MAX_ABS_OVER_RMS * rms + allow + 2.0 ** -8 * np.abs(ref))
    _log(f"  {label}: {r}, h near a midpoint {near_frac:.2e}, max allowance/rms {allow.max() / rms:.2e}")
    assert np.all(np.isfinite(yh)), f"{label}: non-finite output"
    assert np.all(excess <= 0), f"{label}: worst excess over tolerance + allowance {excess.max() / rms:.3e} rms"
    assert r["mean_rel"] <= gu.MEAN_REL, f"{label}: {r}"
    return r


@pytest.mark.parametrize("epi", [0, 1])
def test_grouped_gemm_f8_large_tile_matches_register_kernel_bits(epi):
    # the 128-row LDS-staged kernel and the 64-row register kernel take the same products, scale
    # arithmetic and K order per row: identical bits on the same routing
    T, E, k, N, K = 500, 6, 2, 384, 1024
    ids, al64 = _routing(T, E, k, 64, seed=41)
    al128 = oracle.align(ids, E, 128)
    R = T * k
    Aq, As, Wq, Ws = _f8_operands(T if epi else R, N, K, E, seed=42, full_range=True)
    outs = []
    for bm, al in ((64, al64), (128, al128)):
        tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
        nt = gu.dev(np.array([al["num_tiles"]], np.int32))
        aro = gu.dev(al["sorted_ids"].astype(np.int32)) if epi else None
        C = moe.moe_grouped_gemm_f8(gu.dev(Aq), gu.dev(As), aro, k if epi else 1, gu.dev(Wq), gu.dev(Ws), tiles,
                                    al["num_tiles"], nt, bm, moe.MOE_EPI_SILU_MUL if epi else moe.MOE_EPI_NONE, R)
        torch.cuda.synchronize()
        outs.append(C.view(torch.int32).cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_grouped_gemm_f8_fused_h_quantization_matches_separate_quantizer_bits():
    # SILU_MUL with out_dtype F8 (128-row kernel): the epilogue quantizes h exactly as moe_f8_quantize
    # does on the fp32 h of the same kernel
    T, E, k, I, K = 600, 5, 2, 384, 1024
    ids, al = _routing(T, E, k, 128, seed=61)
    R = T * k
    Aq, As, Wq, Ws = _f8_operands(T, 2 * I, K, E, seed=62, full_range=True)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    args = (gu.dev(Aq), gu.dev(As), srt, k, gu.dev(Wq), gu.dev(Ws), tiles, al["num_tiles"], nt, 128, moe.MOE_EPI_SILU_MUL, R)
    h = moe.moe_grouped_gemm_f8(*args)
    q0, s0 = moe.moe_f8_quantize(h)
    q1 = torch.full((R, I), 0x7F, dtype=torch.uint8, device="cuda")
    s1 = torch.full((R, I // 128), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_gemm_f8(*args, out_dtype=moe.MOE_OUT_F8, C=q1, Cs=s1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q1.cpu().numpy(), q0.cpu().numpy())
    np.testing.assert_array_equal(s1.cpu().numpy().view(np.uint32), s0.cpu().numpy().view(np.uint32))


# ---------------------------------------------------------------------------------------------------
# whole layer

def _forward(d, wl):
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((max(moe.moe_ffn_f8_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    moe.moe_ffn_forward_f8(d.x, d.logits, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k, y=y, topk_ids_out=ids, workspace=ws)
    torch.cuda.synchronize()
    return y, ids


F8_CASES = [("tiny", 16), ("dec1", 1), ("dec8", 8), ("dec32", 32), ("dec64", 64), ("pre800", 200),
            ("big4096", 512), ("skew8192", 1024)]


@pytest.mark.parametrize("name,nsample", F8_CASES)
def test_ffn_forward_f8_matches_oracle(name, nsample):
    wl = mi.WORKLOADS[name]
    _log(f"fp8 layer {name}: T={wl.T} E={wl.E} k={wl.k} H={wl.H} I={wl.I}")
    inp = mi.make_f8_inputs(wl)
    d = F8Device(inp)
    y, ids = _forward(d, wl)
    rid = oracle.route(inp.logits, wl.k)[0]
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    yh = gu.host_bf16_to_f64(y)
    assert np.all(np.isfinite(yh)), "output not fully written"
    tok = gu.sample_tokens(wl.T, nsample, rid)
    _assert_layer(yh[tok], inp, tok, name)


@pytest.mark.parametrize("wl", [
    mi.custom("f8_one_expert", 3, 1, 1, 256, 128, seed=5),
    mi.custom("f8_ragged", 37, 16, 4, 384, 128, seed=6),
    mi.custom("f8_k_eq_E", 20, 6, 6, 128, 256, seed=7),
    mi.custom("f8_many_experts", 40, 1024, 8, 128, 128, seed=8),
    mi.custom("f8_t1_big_k", 1, 64, 32, 256, 256, seed=9),
    mi.custom("f8_hot", 300, 32, 4, 256, 128, seed=12),
])
def test_ffn_forward_f8_edges(wl):
    _log(f"fp8 layer edge {wl}")
    inp = mi.make_f8_inputs(wl)
    if wl.name == "f8_hot":
        inp.logits[:, 0] += 50.0  # every token's slot 0 on expert 0
    d = F8Device(inp)
    y, ids = _forward(d, wl)
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    _assert_layer(gu.host_bf16_to_f64(y), inp, np.arange(wl.T), wl.name)


@pytest.mark.parametrize("E", [8, 32])
def test_ffn_forward_f8_fp16_o_matches_fp32_o(E):
    """With 128-row tiles and from 16384 rows the layer keeps the down projection's output as fp16
    with per-(row, 8 columns) exponents; below, as fp32.  The first 1024 of 2048 tokens (k = 8:
    16384 rows, fp16 O) are run again on their own (8192 rows, fp32 O) with the same tile height, so
    that only O's format differs (every other step is per row).  Tokens scaled by 2^40 (outputs near
    2^80) and by 2^-30 (outputs near 2^-60) take the exponent path.  Per element the two results may
    differ by what one fp16 rounding of each O value (2^-11 relative) can move y, which can flip y's
    bf16 rounding by one step (2^-7 relative), plus 2^-8 of the class's rms for sums that cancel."""
    T, k, H, I = 2048, 8, 256, 256
    wl = mi.custom(f"f8_o16_e{E}", T, E, k, H, I, seed=31 + E)
    half = mi.custom(f"f8_o32_e{E}", T // 2, E, k, H, I, seed=31 + E)
    assert moe.moe_ffn_f8_block_m(T, E, k) == 128 == moe.moe_ffn_f8_block_m(T // 2, E, k)
    inp = mi.make_f8_inputs(wl)
    x = mi.bf16_bits_to_f32(inp.x)
    x[0::3] *= np.float32(2.0 ** 40)
    x[1::3] *= np.float32(2.0 ** -30)
    inp.x = mi.f32_to_bf16_bits(x)
    assert np.array_equal(mi.bf16_bits_to_f32(inp.x), x)
    inp_half = mi.F8Inputs(half, inp.x[:T // 2].copy(), inp.logits[:T // 2].copy(), inp.w13_q, inp.w13_s,
                           inp.w2_q, inp.w2_s)
    _log(f"fp8 fp16 O against fp32 O: E={E}")
    y16, ids16 = _forward(F8Device(inp), wl)
    y32, ids32 = _forward(F8Device(inp_half), half)
    np.testing.assert_array_equal(ids16.cpu().numpy()[:T // 2], ids32.cpu().numpy())
    a = gu.host_bf16_to_f64(y16)[:T // 2]
    b = gu.host_bf16_to_f64(y32)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    for c, label in enumerate(["x 2^40", "x 2^-30", "unscaled"]):
        ac, bc = a[c::3], b[c::3]
        rms = float(np.sqrt(np.mean(bc * bc)))
        assert rms > 0
        bound = 2.0 ** -7 * np.maximum(np.abs(ac), np.abs(bc)) + 2.0 ** -8 * rms
        worst = float(np.max(np.abs(ac - bc) - bound))
        assert worst <= 0, f"{label}: worst excess {worst / rms:.3e} rms"
    assert np.abs(b[0::3]).max() > 2.0 ** 60 and 0 < np.abs(b[1::3]).max() < 2.0 ** -40


def test_ffn_forward_f8_deterministic_and_empty():
    wl = mi.custom("f8_det", 200, 32, 4, 512, 256, seed=13)
    d = F8Device(mi.make_f8_inputs(wl))
    a = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    b = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    empty = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    y = moe.moe_ffn_forward_f8(empty, torch.empty((0, 32), dtype=torch.float32, device="cuda"), d.w13_q, d.w13_s,
                               d.w2_q, d.w2_s, 4)
    assert y.shape == (0, 512)
