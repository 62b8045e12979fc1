"""GPU parity of the W4A8 variant (MXFP8 activations on MXFP4 weights) against the CPU oracle.

The activation quantizer is bit-exact (the block exponent and every rounding decision are made on
values exact in fp32 and fp64 alike; every E4M3 midpoint and its bf16 neighbours are checked).
Grouped GEMM outputs (fp32) are checked per element: with operands whose products span few binades
the instruction sums exactly and only fp32 accumulation is left; over the full code ranges each
128-K step may also lose bits below the step's largest product (the alignment window measured for
the FP8 instruction), which the bound allows.  The gate_up epilogue quantizes h = silu(g)*u computed
in fp32, the oracle its fp64 h: codes agree except near rounding midpoints, so codes are compared by
count and every element is checked to be within one E4M3 step.  Layer outputs use the layer
tolerance: max|gpu-ref| <= 3e-2 * rms(ref) and mean relative error <= 5e-3.
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


_E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _codes4(q):
    q = np.asarray(q, np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.int64)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def _scale(s):
    return np.repeat(np.exp2(np.asarray(s, np.float64) - 127.0), 32, axis=-1)


def _deq4(q, s):
    return _E2M1[_codes4(q)] * _scale(s)


def _deq8(q, s):
    return _E4M3[np.asarray(q, np.int64)] * _scale(s)


class MXDevice:
    def __init__(self, inp):
        self.inp = inp
        self.x = gu.dev_bf16(inp.x)
        self.logits = gu.dev(inp.logits)
        self.w13_q, self.w13_e = gu.dev(inp.w13_q), gu.dev(inp.w13_e)
        self.w2_q, self.w2_e = gu.dev(inp.w2_q), gu.dev(inp.w2_e)
        self._packed = None

    def packed(self):
        if self._packed is None:
            self._packed = moe.moe_mx_prepack(self.w13_q, self.w13_e) + moe.moe_mx_prepack(self.w2_q, self.w2_e)
        return self._packed


# ---------------------------------------------------------------------------------------------------
# activation quantization

def _quantize_both(v):
    bits = mi.f32_to_bf16_bits(np.asarray(v, np.float32))
    q, s = moe.moe_mx8_quantize(gu.dev_bf16(bits))
    torch.cuda.synchronize()
    rq, rs = oracle.mx8_quantize(mi.bf16_bits_to_f32(bits).astype(np.float64))
    return q.cpu().numpy(), s.cpu().numpy(), rq, rs


@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (33, 2048), (300, 4096)])
def test_mx8_quantize_bit_exact(rows, K):
    rng = np.random.default_rng(rows + K + 1)
    v = rng.standard_normal((rows, K)).astype(np.float32) * np.exp2(rng.integers(-60, 60, (rows, 1))).astype(np.float32)
    v[0, :32] = 0.0                                    # all-zero block
    if K >= 64:
        v[0, 32:64] = [300.0, 500.0, 304.0, -1.0625, 2.0 ** -10, -0.0, 3.0, 17.0] * 4  # ties, saturation at X = 1
    q, s, rq, rs = _quantize_both(v)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


def test_mx8_quantize_every_e4m3_midpoint():
    # blocks with X = 1 (an anchor of 300 sets floor(log2 amax) = 8): every midpoint between adjacent
    # finite E4M3 magnitudes, and its bf16 neighbours, both signs
    mags = np.array([_E4M3[c] for c in range(0x7F)])
    mids = (mags[:-1] + mags[1:]) / 2
    bits = mi.f32_to_bf16_bits(mids.astype(np.float32))
    assert np.all(mi.bf16_bits_to_f32(bits) == mids)   # midpoints are bf16 values
    vals = np.concatenate([mids, mi.bf16_bits_to_f32(bits - 1), mi.bf16_bits_to_f32(bits + 1)])
    vals = vals[(vals > 0) & (vals < 448)]
    vals = np.concatenate([vals, -vals, [448.0, 460.0, 464.0, 480.0, -470.0]])
    n = (len(vals) + 30) // 31
    v = np.zeros((n, 32), np.float32)
    v[:, 0] = 300.0
    v.reshape(-1)[np.arange(len(vals)) // 31 * 32 + np.arange(len(vals)) % 31 + 1] = vals
    q, s, rq, rs = _quantize_both(v.reshape(1, -1))
    assert np.all(rs == 127)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


# ---------------------------------------------------------------------------------------------------
# grouped GEMM

def _routing(T, E, k, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    return ids, oracle.align(ids, E, bm)


def _operands(rows, N, K, E, seed, narrow=False):
    rng = np.random.default_rng(seed)
    if narrow:
        # E4M3 magnitudes in [1, 2) (exponent field 7) and E2M1 magnitudes in {1, 1.5}: products within
        # one binade and a half, summed exactly by the instruction
        Aq = (rng.integers(0, 2, (rows, K)) << 7 | 7 << 3 | rng.integers(0, 8, (rows, K))).astype(np.uint8)
        nib = (rng.integers(0, 2, (E, N, K)) << 3 | rng.integers(2, 4, (E, N, K))).astype(np.uint8)
        Wq = (nib[..., 0::2] | nib[..., 1::2] << 4).astype(np.uint8)
        As = np.full((rows, K // 32), 127, np.uint8)
        We = np.full((E, N, K // 32), 124, np.uint8)
    else:
        Aq = rng.integers(0, 256, (rows, K), dtype=np.uint8)
        Aq[(Aq & 0x7F) == 0x7F] = 0x7E                 # no NaN codes
        As = rng.integers(112, 118, (rows, K // 32), dtype=np.uint8)
        Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
        We = rng.integers(118, 123, (E, N, K // 32), dtype=np.uint8)
    return Aq, As, Wq, We


def _bounds(Aq, As, a_rows, Wq, We, ids_of_row, K):
    """Per output: sum of |terms| and the sum over 128-K steps of the step's largest |term|."""
    A = _deq8(Aq, As)[a_rows]                          # [R, K]
    R = len(a_rows)
    N = Wq.shape[1]
    tsum = np.zeros((R, N))
    smax = np.zeros((R, N))
    for r in range(R):
        W = np.abs(_deq4(Wq[ids_of_row[r]], We[ids_of_row[r]]))
        P = np.abs(A[r])[None, :] * W                  # [N, K]
        tsum[r] = P.sum(axis=1)
        pad = (-K) % 128
        smax[r] = np.pad(P, ((0, 0), (0, pad))).reshape(N, -1, 128).max(axis=2).sum(axis=1)
    return tsum, smax


def _row_experts(al, R):
    e_of = np.empty(R, np.int64)
    off = al["offsets"]
    for e in range(len(off) - 1):
        e_of[off[e]:off[e + 1]] = e
    return e_of


GEMM_CASES = [(3, 8, 2, 16), (40, 16, 4, 16), (90, 12, 3, 32), (300, 8, 2, 64)]


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
@pytest.mark.parametrize("N,K", [(256, 2048), (200, 160), (48, 96)])
@pytest.mark.parametrize("narrow", [True, False])
def test_grouped_gemm_w4a8_plain(T, E, k, bm, N, K, narrow):
    ids, al = _routing(T, E, k, bm, seed=T * 5 + N)
    R = T * k
    Aq, As, Wq, We = _operands(R, N, K, E, seed=K + bm + narrow, narrow=narrow)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    C = moe.moe_grouped_gemm_w4a8(gu.dev(Aq), gu.dev(As), None, 1, gu.dev(Wq), gu.dev(We), tiles, al["num_tiles"], nt,
                                  bm, moe.MOE_EPI_NONE, R)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_w4a8(Aq, As, None, 1, Wq, We, al["offsets"])
    tsum, smax = _bounds(Aq, As, np.arange(R), Wq, We, _row_experts(al, R), K)
    bound = (64 + K / 32) * 2.0 ** -24 * tsum + 1e-30
    if not narrow:
        bound = bound + 2.0 ** -5 * smax
    err = np.abs(got - ref)
    _log(f"  max err / bound {np.max(err / bound):.3f}; max err / sum|terms| {np.max(err / (tsum + 1e-30)):.2e}")
    assert np.all(err <= bound)


# the 128-row LDS-staged kernel (K % 128 == 0)
MM_CASES = [(600, 4, 2, 128), (700, 6, 3, 128)]


@pytest.mark.parametrize("T,E,k,bm", MM_CASES)
@pytest.mark.parametrize("N,K", [(512, 2048), (200, 384)])
@pytest.mark.parametrize("narrow", [True, False])
@pytest.mark.parametrize("layout", [0, 1])
def test_grouped_gemm_w4a8_large_tile(T, E, k, bm, N, K, narrow, layout):
    ids, al = _routing(T, E, k, bm, seed=T * 3 + N)
    R = T * k
    Aq, As, Wq, We = _operands(R, N, K, E, seed=K + narrow, narrow=narrow)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    dWq, dWe = gu.dev(Wq), gu.dev(We)
    if layout == moe.MOE_LAYOUT_PACKED:
        if N % 16:
            pytest.skip("packed weights need N % 16 == 0")
        dWq, dWe = moe.moe_mx_prepack(dWq, dWe)
    C = moe.moe_grouped_gemm_w4a8(gu.dev(Aq), gu.dev(As), None, 1, dWq, dWe, tiles, al["num_tiles"], nt, bm,
                                  moe.MOE_EPI_NONE, R, weight_layout=layout)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_w4a8(Aq, As, None, 1, Wq, We, al["offsets"])
    tsum, smax = _bounds(Aq, As, np.arange(R), Wq, We, _row_experts(al, R), K)
    bound = (64 + K / 32) * 2.0 ** -24 * tsum + 1e-30
    if not narrow:
        bound = bound + 2.0 ** -5 * smax
    err = np.abs(got - ref)
    _log(f"  max err / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("epi", [0, 1])
def test_grouped_gemm_w4a8_large_tile_matches_register_kernel_bits(epi):
    # the same rows in 128-row tiles (LDS-staged kernel) and in 64-row tiles (register kernel): each
    # output is the same instruction sequence, so the bits agree
    T, E, k, N, K = 700, 6, 3, 512, 1024
    rng = np.random.default_rng(41)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    a128, a64 = oracle.align(ids, E, 128), oracle.align(ids, E, 64)
    np.testing.assert_array_equal(a128["sorted_ids"], a64["sorted_ids"])
    R = T * k
    Aq, As, Wq, We = _operands(T, N, K, E, seed=42)
    out = []
    for al, bm in ((a128, 128), (a64, 64)):
        tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
        nt = gu.dev(np.array([al["num_tiles"]], np.int32))
        srt = gu.dev(al["sorted_ids"].astype(np.int32))
        r = moe.moe_grouped_gemm_w4a8(gu.dev(Aq), gu.dev(As), srt, k, gu.dev(Wq), gu.dev(We), tiles, al["num_tiles"],
                                      nt, bm, epi, R)
        torch.cuda.synchronize()
        out.append([t.cpu().numpy() for t in r] if epi else [r.cpu().numpy()])
    for a, b in zip(*out):
        np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))


def _e4m3_step(mag):
    """Spacing of the E4M3 grid at quotient magnitude mag (subnormal spacing 2^-9 below 2^-6)."""
    mag = np.maximum(mag, 2.0 ** -6)
    return np.exp2(np.floor(np.log2(mag)) - 3)


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES + MM_CASES[:1])
@pytest.mark.parametrize("I,K", [(128, 2048), (96, 160)])
def test_grouped_gemm_w4a8_silu_quantized_h(T, E, k, bm, I, K):
    if bm == 128 and K % 128:
        pytest.skip("the 128-row kernel steps K by 128")
    ids, al = _routing(T, E, k, bm, seed=T + I + 1)
    R = T * k
    Aq, As, Wq, We = _operands(T, 2 * I, K, E, seed=I + bm + 1)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    sorted_ids = gu.dev(al["sorted_ids"].astype(np.int32))
    hq, hs = moe.moe_grouped_gemm_w4a8(gu.dev(Aq), gu.dev(As), sorted_ids, k, gu.dev(Wq), gu.dev(We), tiles,
                                       al["num_tiles"], nt, bm, moe.MOE_EPI_SILU_MUL, R)
    torch.cuda.synchronize()
    a_rows = al["sorted_ids"].astype(np.int64) // k
    G = oracle.grouped_proj_w4a8(Aq, As, al["sorted_ids"], k, Wq, We, al["offsets"])
    h_ref = oracle.grouped_proj_w4a8(Aq, As, al["sorted_ids"], k, Wq, We, al["offsets"], silu_mul=True)
    tsum, smax = _bounds(Aq, As, a_rows, Wq, We, _row_experts(al, R), K)
    dG = (64 + K / 32) * 2.0 ** -24 * tsum + 2.0 ** -5 * smax
    g, u, dg, du = G[:, :I], G[:, I:], dG[:, :I], dG[:, I:]
    # |h_gpu - h_ref|: silu(g) * u in fp32 (a few ulps) plus the propagated sum errors
    # (|d silu / dg| <= 1.1, |silu(g)| <= |g|, and the product of the two errors)
    dh = 2.0 ** -18 * np.abs(h_ref) + 1.1 * np.abs(u) * dg + (np.abs(g) + dg) * du + 1e-30
    rq, rs = oracle.mx8_quantize(h_ref)
    gq, gs = hq.cpu().numpy(), hs.cpu().numpy()
    same_scale = np.repeat(gs == rs, 32, axis=1)
    scale_diff = np.mean(gs != rs)
    code_diff = np.mean(gq != rq)
    _log(f"  h codes differing {code_diff:.2e}, scales differing {scale_diff:.2e}")
    assert scale_diff <= 1e-3
    # quantization is monotone and saturating: the GPU's code lies within the h error bound plus half
    # a grid step of the oracle's quotient (in units of the shared block scale)
    X = _scale(gs)
    t, d = h_ref / X, dh / X
    c = _E4M3[gq.astype(np.int64)]
    allow = d + 0.5 * _e4m3_step(np.minimum(np.abs(t) + d, 448.0))
    excess = (np.abs(c - np.clip(t, -448.0, 448.0)) - allow * (1 + 1e-12))[same_scale]
    _log(f"  worst code distance minus allowance {np.max(excess):.3e} (quotient units)")
    assert np.all(excess <= 0)


@pytest.mark.parametrize("bm", [16, 32, 64])
def test_grouped_gemm_w4a8_packed_matches_canonical_bits(bm):
    T, E, k, N, K = 70, 8, 3, 256, 384
    ids, al = _routing(T, E, k, bm, seed=bm)
    R = T * k
    Aq, As, Wq, We = _operands(R, N, K, E, seed=bm + 3)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    dWq, dWe = gu.dev(Wq), gu.dev(We)
    pq, pe = moe.moe_mx_prepack(dWq, dWe)
    for epi in (moe.MOE_EPI_NONE, moe.MOE_EPI_SILU_MUL):
        a = moe.moe_grouped_gemm_w4a8(gu.dev(Aq), gu.dev(As), None, 1, dWq, dWe, tiles, al["num_tiles"], nt, bm, epi, R)
        b = moe.moe_grouped_gemm_w4a8(gu.dev(Aq), gu.dev(As), None, 1, pq, pe, tiles, al["num_tiles"], nt, bm, epi, R,
                                      weight_layout=moe.MOE_LAYOUT_PACKED)
        torch.cuda.synchronize()
        if epi == moe.MOE_EPI_NONE:
            np.testing.assert_array_equal(a.cpu().numpy().view(np.int32), b.cpu().numpy().view(np.int32))
        else:
            np.testing.assert_array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
            np.testing.assert_array_equal(a[1].cpu().numpy(), b[1].cpu().numpy())


@pytest.mark.parametrize("T,E,k,bm", [(3, 8, 2, 16), (40, 16, 4, 16), (90, 12, 3, 32), (300, 8, 2, 64)])
def test_w4a8_tiled_activation_chain_matches_row_major_bits(T, E, k, bm):
    # x -> quantize -> gate_up (SiLU*mul, h quantized) -> down, once with row-major activations and
    # canonical weights, once with tile-blocked MXFP8 activations and packed weights: same O bits
    ids, al = _routing(T, E, k, bm, seed=T + 13)
    R, H, I = T * k, 256, 128
    rng = np.random.default_rng(bm + T + 1)
    x = gu.dev_bf16(mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    _, _, W13, E13 = _operands(1, 2 * I, H, E, seed=5)
    _, _, W2, E2 = _operands(1, H, I, E, seed=6)
    W13, E13, W2, E2 = gu.dev(W13), gu.dev(E13), gu.dev(W2), gu.dev(E2)
    P13, Q13 = moe.moe_mx_prepack(W13, E13)
    P2, Q2 = moe.moe_mx_prepack(W2, E2)
    mt = al["num_tiles"]
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([mt], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    xq, xs = moe.moe_mx8_quantize(x)
    hq, hs = moe.moe_grouped_gemm_w4a8(xq, xs, srt, k, W13, E13, tiles, mt, nt, bm, moe.MOE_EPI_SILU_MUL, R)
    O1 = moe.moe_grouped_gemm_w4a8(hq, hs, None, 1, W2, E2, tiles, mt, nt, bm, moe.MOE_EPI_NONE, R)
    tq, ts = moe.moe_mx8_quantize_tiles(x, srt, k, tiles, mt, nt, bm)
    gq, gs = moe.moe_grouped_gemm_w4a8(tq, ts, None, 1, P13, Q13, tiles, mt, nt, bm, moe.MOE_EPI_SILU_MUL, R,
                                       weight_layout=moe.MOE_LAYOUT_PACKED, act_layout=moe.MOE_ACT_TILED)
    O2 = moe.moe_grouped_gemm_w4a8(gq, gs, None, 1, P2, Q2, tiles, mt, nt, bm, moe.MOE_EPI_NONE, R,
                                   weight_layout=moe.MOE_LAYOUT_PACKED, act_layout=moe.MOE_ACT_TILED)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(O1.view(torch.int32).cpu().numpy(), O2.view(torch.int32).cpu().numpy())


def test_mx8_quantize_tiles_is_the_row_major_quantization_rearranged():
    T, E, k, bm, K = 37, 8, 3, 16, 384
    ids, al = _routing(T, E, k, bm, seed=7)
    rng = np.random.default_rng(8)
    bits = mi.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32) * 3)
    x = gu.dev_bf16(bits)
    mt = al["num_tiles"]
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([mt], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    tq, ts = moe.moe_mx8_quantize_tiles(x, srt, k, tiles, mt, nt, bm)
    torch.cuda.synchronize()
    rq, rs = oracle.mx8_quantize(mi.bf16_bits_to_f32(bits).astype(np.float64))
    tq, ts = tq.cpu().numpy().reshape(-1), ts.cpu().numpy().reshape(-1)
    nks = K // 128
    for t in range(mt):
        e, row0, rows = al["tiles"][t]
        for i in range(rows):
            src = al["sorted_ids"][row0 + i] // k
            for s_ in range(nks):
                blk = (t * (bm // 16) + i // 16) * nks + s_
                for qq in range(4):
                    lane = qq * 16 + (i % 16)
                    a = tq[blk * 2048 + lane * 16: blk * 2048 + lane * 16 + 16]
                    b = tq[blk * 2048 + 1024 + lane * 16: blk * 2048 + 1024 + lane * 16 + 16]
                    np.testing.assert_array_equal(a, rq[src, s_ * 128 + 16 * qq: s_ * 128 + 16 * qq + 16])
                    np.testing.assert_array_equal(b, rq[src, s_ * 128 + 64 + 16 * qq: s_ * 128 + 80 + 16 * qq])
                    assert ts[blk * 64 + lane] == rs[src, s_ * 4 + qq]


# ---------------------------------------------------------------------------------------------------
# whole layer

def _forward(d, wl, layout=moe.MOE_LAYOUT_CANONICAL):
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((max(moe.moe_ffn_w4a8_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    w = d.packed() if layout == moe.MOE_LAYOUT_PACKED else (d.w13_q, d.w13_e, d.w2_q, d.w2_e)
    moe.moe_ffn_forward_w4a8(d.x, d.logits, *w, wl.k, y=y, topk_ids_out=ids, workspace=ws, weight_layout=layout)
    torch.cuda.synchronize()
    return y, ids


W4A8_CASES = [("tiny", 16), ("dec1", 1), ("dec8", 8), ("dec32", 32), ("dec64", 64), ("pre800", 200),
            ("big4096", 512), ("skew8192", 1024)]


@pytest.mark.parametrize("name,nsample", W4A8_CASES)
def test_ffn_forward_w4a8_matches_oracle(name, nsample):
    wl = mi.WORKLOADS[name]
    _log(f"w4a8 layer {name}: T={wl.T} E={wl.E} k={wl.k} H={wl.H} I={wl.I}")
    inp = mi.make_mx_inputs(wl)
    d = MXDevice(inp)
    y, ids = _forward(d, wl, moe.MOE_LAYOUT_PACKED if wl.H % 128 == 0 and wl.I % 128 == 0 else 0)
    rid = oracle.route(inp.logits, wl.k)[0]
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    yh = gu.host_bf16_to_f64(y)
    assert np.all(np.isfinite(yh)), "output not fully written"
    tok = gu.sample_tokens(wl.T, nsample, rid)
    r = gu.assert_within_tolerance(yh[tok], oracle.moe_ffn_w4a8(inp, tokens=tok), name)
    _log(f"  {name}: {r}")


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_CANONICAL, moe.MOE_LAYOUT_PACKED])
@pytest.mark.parametrize("E,bm", [(128, 64), (8, 128)])
def test_ffn_forward_w4a8_fp16_o_matches_fp32_o(E, bm, layout):
    """From 16384 rows the layer keeps the down projection's output as fp16 with per-(row, 8 columns)
    exponents; below, as fp32.  The first 1024 of 2048 tokens (k = 8: 16384 rows, fp16 O) are run
    again on their own (8192 rows, fp32 O) with the same tile height, so that only O's format
    differs (every other step is per row).  Tokens scaled by 2^40 (outputs near 2^80) and by 2^-30
    (outputs near 2^-60) take the exponent path.  Per element the two results may differ by what one
    fp16 rounding of each O value (2^-11 relative) can move y, which can flip y's bf16 rounding by one
    step (2^-7 relative), plus 2^-8 of the class's rms for sums that cancel."""
    T, k, H, I = 2048, 8, 256, 128
    wl = mi.custom(f"w8_o16_e{E}", T, E, k, H, I, seed=23 + E)
    half = mi.custom(f"w8_o32_e{E}", T // 2, E, k, H, I, seed=23 + E)
    assert moe.moe_ffn_w4a8_block_m(T, H, I, E, k) == bm == moe.moe_ffn_w4a8_block_m(T // 2, H, I, E, k)
    inp = mi.make_mx_inputs(wl)
    x = mi.bf16_bits_to_f32(inp.x)
    x[0::3] *= np.float32(2.0 ** 40)
    x[1::3] *= np.float32(2.0 ** -30)
    inp.x = mi.f32_to_bf16_bits(x)
    assert np.array_equal(mi.bf16_bits_to_f32(inp.x), x)
    inp_half = mi.MXInputs(half, inp.x[:T // 2].copy(), inp.logits[:T // 2].copy(), inp.w13_q, inp.w13_e,
                           inp.w2_q, inp.w2_e)
    _log(f"w4a8 fp16 O against fp32 O: E={E} bm={bm} layout {layout}")
    d = MXDevice(inp)
    d_half = MXDevice(inp_half)
    d_half._packed = d.packed() if layout == moe.MOE_LAYOUT_PACKED else None
    y16, ids16 = _forward(d, wl, layout)
    y32, ids32 = _forward(d_half, half, layout)
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
    # the classes are where they were put: far above and far below fp16's range
    assert np.abs(b[0::3]).max() > 2.0 ** 60 and 0 < np.abs(b[1::3]).max() < 2.0 ** -40


@pytest.mark.parametrize("wl", [
    mi.custom("w8_one_expert", 3, 1, 1, 256, 128, seed=5),
    mi.custom("w8_ragged", 37, 16, 4, 160, 96, seed=6),
    mi.custom("w8_k_eq_E", 20, 6, 6, 128, 64, seed=7),
    mi.custom("w8_many_experts", 40, 1024, 8, 128, 64, seed=8),
    mi.custom("w8_t1_big_k", 1, 64, 32, 256, 256, seed=9),
    mi.custom("w8_hot", 300, 32, 4, 256, 128, seed=12),
])
def test_ffn_forward_w4a8_edges(wl):
    inp = mi.make_mx_inputs(wl)
    if wl.name == "w8_hot":
        inp.logits[:, 0] += 50.0  # every token's slot 0 on expert 0
    d = MXDevice(inp)
    y, ids = _forward(d, wl)
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    r = gu.assert_within_tolerance(gu.host_bf16_to_f64(y), oracle.moe_ffn_w4a8(inp), wl.name)
    _log(f"  {wl.name}: {r}")


@pytest.mark.parametrize("name", ["tiny", "dec64", "pre800"])
def test_ffn_forward_w4a8_packed_matches_canonical_bits(name):
    wl = mi.WORKLOADS[name]
    d = MXDevice(mi.make_mx_inputs(wl))
    a = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    b = _forward(d, wl, moe.MOE_LAYOUT_PACKED)[0].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(a, b)


def test_ffn_forward_w4a8_deterministic_and_empty():
    wl = mi.custom("w8_det", 200, 32, 4, 512, 256, seed=13)
    d = MXDevice(mi.make_mx_inputs(wl))
    a = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    b = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    empty = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    y = moe.moe_ffn_forward_w4a8(empty, torch.empty((0, 32), dtype=torch.float32, device="cuda"), d.w13_q, d.w13_e,
                                 d.w2_q, d.w2_e, 4)
    assert y.shape == (0, 512)


def test_ffn_forward_w4a8_closer_to_bf16_activations_than_w4a4():
    # the same weights and routing: 8-bit activations leave the layer closer to the W4A16 oracle
    # evaluated on the MX weights' values than 4-bit ones
    wl = mi.WORKLOADS["dec64"]
    inp = mi.make_mx_inputs(wl)
    d = MXDevice(inp)
    y8 = gu.host_bf16_to_f64(_forward(d, wl)[0])
    y4 = gu.host_bf16_to_f64(moe.moe_ffn_forward_mxfp4(d.x, d.logits, d.w13_q, d.w13_e, d.w2_q, d.w2_e, wl.k))
    tok = np.arange(16)
    exact = oracle.moe_ffn_w4a8(inp, tokens=tok)  # reference of the same method
    r8 = np.linalg.norm(y8[tok] - exact) / np.linalg.norm(exact)
    r4 = np.linalg.norm(y4[tok] - exact) / np.linalg.norm(exact)
    _log(f"  relative distance to the W4A8 oracle: W4A8 {r8:.2e}, W4A4 {r4:.2e}")
    assert r8 < 0.1 * r4
