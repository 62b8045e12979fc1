"""GPU parity of the MXFP4 (W4A4) variant against the CPU oracle.

The activation quantizer is bit-exact (the block exponent and every rounding decision are made on
values that are exact in fp32 and fp64 alike).  Grouped GEMM outputs (fp32) are checked per element
within the rounding bound of fp32 accumulation.  The fused gate_up epilogue quantizes h = silu(g)*u
computed in fp32, while the oracle quantizes its fp64 h: codes agree except where h lies within
fp32 rounding of a rounding boundary, so codes are compared by count and every element is checked to
be within one E2M1 step.  Layer outputs use the layer tolerance: max|gpu-ref| <= 3e-2 * rms(ref) and
mean relative error <= 5e-3.
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


def _codes(q):
    q = np.asarray(q, np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.int64)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def _deq(q, s):
    return _E2M1[_codes(q)] * np.repeat(np.exp2(np.asarray(s, np.float64) - 127.0), 32, axis=-1)


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

@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (33, 2048), (300, 4096)])
def test_mx_quantize_bit_exact(rows, K):
    rng = np.random.default_rng(rows + K)
    v = rng.standard_normal((rows, K)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (rows, 1))).astype(np.float32)
    v[0, :32] = 0.0                                    # all-zero block
    if K >= 64:
        v[0, 32:64] = [0.25, -0.75, 1.25, 3.5, 5.0, -2.5, 7.0, 0.5] * 4   # ties and saturation at X = 1
    bits = mi.f32_to_bf16_bits(v)
    q, s = moe.moe_mx_quantize(gu.dev_bf16(bits))
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(mi.bf16_bits_to_f32(bits).astype(np.float64))
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


# ---------------------------------------------------------------------------------------------------
# grouped GEMM

def _routing(T, E, k, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    return ids, oracle.align(ids, E, bm)


def _mx_operands(rows, N, K, E, seed):
    rng = np.random.default_rng(seed)
    Aq = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    As = rng.integers(122, 130, (rows, K // 32), dtype=np.uint8)
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    We = rng.integers(118, 123, (E, N, K // 32), dtype=np.uint8)
    return Aq, As, Wq, We


# (T, E, k, bm): few tiles take the K-split kernel, more tiles the N-split one
GEMM_CASES = [(3, 8, 2, 16), (40, 16, 4, 16), (90, 12, 3, 32), (300, 8, 2, 64)]
# the 128-row LDS-staged kernel needs K % 128 == 0
MM_CASES = [(600, 4, 2, 128), (700, 6, 3, 128)]


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
@pytest.mark.parametrize("N,K", [(256, 2048), (200, 160), (48, 96)])
def test_grouped_gemm_mxfp4_plain(T, E, k, bm, N, K):
    ids, al = _routing(T, E, k, bm, seed=T * 7 + N)
    R = T * k
    Aq, As, Wq, We = _mx_operands(R, N, K, E, seed=K + bm)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    C = moe.moe_grouped_gemm_mxfp4(gu.dev(Aq), gu.dev(As), None, 1, gu.dev(Wq), gu.dev(We), tiles, al["num_tiles"], nt,
                                   bm, moe.MOE_EPI_NONE, R)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_mx(Aq, As, None, 1, Wq, We, al["offsets"])
    ref_abs = oracle.grouped_proj_mx(Aq & 0x77, As, None, 1, Wq & 0x77, We, al["offsets"])
    # fp32 accumulation: at most (64 + K/32) roundings of 2^-24 relative to the sum of |terms|
    assert np.all(np.abs(got - ref) <= (64 + K / 32) * 2.0 ** -24 * ref_abs + 1e-30)


@pytest.mark.parametrize("T,E,k,bm", MM_CASES)
@pytest.mark.parametrize("N,K", [(512, 2048), (200, 384)])
@pytest.mark.parametrize("layout", [0, 1])
def test_grouped_gemm_mxfp4_large_tile(T, E, k, bm, N, K, layout):
    ids, al = _routing(T, E, k, bm, seed=T * 3 + N)
    R = T * k
    if layout == 1 and N % 16:
        N = 208
    Aq, As, Wq, We = _mx_operands(R, N, K, E, seed=K + N)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    dWq, dWe = gu.dev(Wq), gu.dev(We)
    if layout == 1:
        dWq, dWe = moe.moe_mx_prepack(dWq, dWe)
    C = moe.moe_grouped_gemm_mxfp4(gu.dev(Aq), gu.dev(As), None, 1, dWq, dWe, tiles, al["num_tiles"], nt, bm,
                                   moe.MOE_EPI_NONE, R, weight_layout=layout)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = oracle.grouped_proj_mx(Aq, As, None, 1, Wq, We, al["offsets"])
    ref_abs = oracle.grouped_proj_mx(Aq & 0x77, As, None, 1, Wq & 0x77, We, al["offsets"])
    assert np.all(np.abs(got - ref) <= (64 + K / 32) * 2.0 ** -24 * ref_abs + 1e-30)


@pytest.mark.parametrize("epi", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_grouped_gemm_mxfp4_large_tile_matches_register_kernel_bits(epi, layout):
    # the 128-row LDS-staged kernel issues the same scaled instructions per output as the 64-row
    # register kernel: identical bits (fp32 output, or h codes and scale bytes) on the same routing
    T, E, k, N, K = 500, 6, 2, 512, 1024
    rng = np.random.default_rng(51)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    R = T * k
    Aq, As, Wq, We = _mx_operands(T if epi else R, N, K, E, seed=52)
    dWq, dWe = gu.dev(Wq), gu.dev(We)
    if layout == 1:
        dWq, dWe = moe.moe_mx_prepack(dWq, dWe)
    outs = []
    for bm in (64, 128):
        al = oracle.align(ids, E, bm)
        tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
        nt = gu.dev(np.array([al["num_tiles"]], np.int32))
        aro = gu.dev(al["sorted_ids"].astype(np.int32)) if epi else None
        out = moe.moe_grouped_gemm_mxfp4(gu.dev(Aq), gu.dev(As), aro, k if epi else 1, dWq, dWe, tiles,
                                         al["num_tiles"], nt, bm, moe.MOE_EPI_SILU_MUL if epi else moe.MOE_EPI_NONE,
                                         R, weight_layout=layout)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in out] if epi else [out.view(torch.int32).cpu().numpy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES + MM_CASES[:1])
@pytest.mark.parametrize("I,K", [(128, 2048), (96, 160)])
def test_grouped_gemm_mxfp4_silu_quantized_h(T, E, k, bm, I, K):
    if bm == 128 and K % 128:
        pytest.skip("the 128-row kernel steps K by 128")
    ids, al = _routing(T, E, k, bm, seed=T + I)
    R = T * k
    Aq, _, Wq, We = _mx_operands(T, 2 * I, K, E, seed=I + bm)
    As = np.random.default_rng(1).integers(124, 128, (T, K // 32), dtype=np.uint8)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    sorted_ids = gu.dev(al["sorted_ids"].astype(np.int32))
    hq, hs = moe.moe_grouped_gemm_mxfp4(gu.dev(Aq), gu.dev(As), sorted_ids, k, gu.dev(Wq), gu.dev(We), tiles,
                                        al["num_tiles"], nt, bm, moe.MOE_EPI_SILU_MUL, R)
    torch.cuda.synchronize()
    h_ref = oracle.grouped_proj_mx(Aq, As, al["sorted_ids"], k, Wq, We, al["offsets"], silu_mul=True)
    rq, rs = oracle.mx_quantize(h_ref)
    gq, gs = hq.cpu().numpy(), hs.cpu().numpy()
    scale_diff = np.mean(gs != rs)
    code_diff = np.mean(_codes(gq) != _codes(rq))
    _log(f"  h codes differing {code_diff:.2e}, scales differing {scale_diff:.2e}")
    assert scale_diff <= 1e-3 and code_diff <= 1e-3
    # every element within one E2M1 step (of the larger block scale) of the oracle's
    step = 2.0 * np.repeat(np.exp2(np.maximum(gs, rs).astype(np.float64) - 127.0), 32, axis=-1)
    assert np.all(np.abs(_deq(gq, gs) - _deq(rq, rs)) <= step)


# ---------------------------------------------------------------------------------------------------
# whole layer

def _forward(d, wl, layout=moe.MOE_LAYOUT_CANONICAL):
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((max(moe.moe_ffn_mxfp4_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    if layout == moe.MOE_LAYOUT_PACKED:
        w = d.packed()
    else:
        w = (d.w13_q, d.w13_e, d.w2_q, d.w2_e)
    moe.moe_ffn_forward_mxfp4(d.x, d.logits, *w, wl.k, y=y, topk_ids_out=ids, workspace=ws, weight_layout=layout)
    torch.cuda.synchronize()
    return y, ids


MX_CASES = [("tiny", 16), ("dec1", 1), ("dec8", 8), ("dec32", 32), ("dec64", 64), ("pre800", 200),
            ("big4096", 512), ("skew8192", 1024)]


@pytest.mark.parametrize("name,nsample", MX_CASES)
def test_ffn_forward_mxfp4_matches_oracle(name, nsample):
    wl = mi.WORKLOADS[name]
    _log(f"mxfp4 layer {name}: T={wl.T} E={wl.E} k={wl.k} H={wl.H} I={wl.I}")
    inp = mi.make_mx_inputs(wl)
    d = MXDevice(inp)
    y, ids = _forward(d, wl)
    rid = oracle.route(inp.logits, wl.k)[0]
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    yh = gu.host_bf16_to_f64(y)
    assert np.all(np.isfinite(yh)), "output not fully written"
    tok = gu.sample_tokens(wl.T, nsample, rid)
    r = gu.assert_within_tolerance(yh[tok], oracle.moe_ffn_mx(inp, tokens=tok), name)
    _log(f"  {name}: {r}")


@pytest.mark.parametrize("wl", [
    mi.custom("mx_one_expert", 3, 1, 1, 256, 128, seed=5),
    mi.custom("mx_ragged", 37, 16, 4, 160, 96, seed=6),
    mi.custom("mx_k_eq_E", 20, 6, 6, 128, 64, seed=7),
    mi.custom("mx_many_experts", 40, 1024, 8, 128, 64, seed=8),
    mi.custom("mx_t1_big_k", 1, 64, 32, 256, 256, seed=9),
    mi.custom("mx_hot", 300, 32, 4, 256, 128, seed=12),
])
def test_ffn_forward_mxfp4_edges(wl):
    inp = mi.make_mx_inputs(wl)
    if wl.name == "mx_hot":
        inp.logits[:, 0] += 50.0  # every token's slot 0 on expert 0
    d = MXDevice(inp)
    y, ids = _forward(d, wl)
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    gu.assert_within_tolerance(gu.host_bf16_to_f64(y), oracle.moe_ffn_mx(inp), wl.name)


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_CANONICAL, moe.MOE_LAYOUT_PACKED])
@pytest.mark.parametrize("wl,bm", [
    (mi.custom("mx_o16_small_tiles", 64, 32, 8, 256, 128, seed=21), 16),
    (mi.custom("mx_o16_large_tiles", 1024, 8, 2, 256, 128, seed=22), 128),
])
def test_ffn_forward_mxfp4_fp16_o_extreme_rows(wl, bm, layout):
    """From 256 rows the layer keeps the down projection's output as fp16 with per-(row, 8 columns)
    exponents.  Tokens scaled by 2^40 (outputs near 2^80, far past fp16's range) and by 2^-30 (outputs
    near 2^-60, below its normal range) take the exponent path in both the register-tile and the
    128-row kernels; each class of rows is held to the layer's tolerance on its own, so an error in
    the small rows is not hidden by the large ones.  The scalings are powers of two, so x stays
    exact in bf16."""
    inp = mi.make_mx_inputs(wl)
    assert wl.T * wl.k >= 256
    assert moe.moe_ffn_mxfp4_block_m(wl.T, wl.H, wl.I, wl.E, wl.k) == bm
    x = mi.bf16_bits_to_f32(inp.x)
    x[0::3] *= np.float32(2.0 ** 40)
    x[1::3] *= np.float32(2.0 ** -30)
    inp.x = mi.f32_to_bf16_bits(x)
    assert np.array_equal(mi.bf16_bits_to_f32(inp.x), x)
    _log(f"mxfp4 layer {wl.name} (fp16 O, extreme rows, layout {layout})")
    d = MXDevice(inp)
    y, ids = _forward(d, wl, layout)
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    yh, ref = gu.host_bf16_to_f64(y), oracle.moe_ffn_mx(inp)
    assert np.abs(ref[0::3]).max() > 2.0 ** 60 and 0 < np.abs(ref[1::3]).max() < 2.0 ** -40
    for c, label in enumerate(["x 2^40", "x 2^-30", "unscaled"]):
        gu.assert_within_tolerance(yh[c::3], ref[c::3], f"{wl.name} {label}")


def test_ffn_forward_mxfp4_deterministic_and_empty():
    wl = mi.custom("mx_det", 200, 32, 4, 512, 256, seed=13)
    d = MXDevice(mi.make_mx_inputs(wl))
    a = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    b = _forward(d, wl)[0].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    empty = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    y = moe.moe_ffn_forward_mxfp4(empty, torch.empty((0, 32), dtype=torch.float32, device="cuda"), d.w13_q, d.w13_e,
                                  d.w2_q, d.w2_e, 4)
    assert y.shape == (0, 512)


# ---------------------------------------------------------------------------------------------------
# packed weights (and, in the layer, tile-blocked activations): same values, same bits

def test_mx_prepack_is_a_permutation_of_bytes():
    rng = np.random.default_rng(30)
    wq = rng.integers(0, 256, (3, 48, 128), dtype=np.uint8)
    we = rng.integers(100, 140, (3, 48, 8), dtype=np.uint8)
    pq, pe = moe.moe_mx_prepack(gu.dev(wq), gu.dev(we))
    torch.cuda.synchronize()
    pq, pe = pq.cpu().numpy(), pe.cpu().numpy()
    assert not np.array_equal(pq, wq)
    np.testing.assert_array_equal(np.sort(pq.ravel()), np.sort(wq.ravel()))
    np.testing.assert_array_equal(np.sort(pe.ravel()), np.sort(we.ravel()))
    # block (e, row block, K block), lane l: row 16 rb + l % 16, K elements [128 kb + 32 (l / 16), +32)
    e, rb, kb, lane = 2, 1, 1, 37
    blk = (e * 3 + rb) * 2 + kb
    row, qd = 16 * rb + lane % 16, lane // 16
    np.testing.assert_array_equal(pq.reshape(-1)[blk * 1024 + 16 * lane: blk * 1024 + 16 * lane + 16],
                                  wq[e, row, 64 * kb + 16 * qd: 64 * kb + 16 * qd + 16])
    assert pe.reshape(-1)[blk * 64 + lane] == we[e, row, 4 * kb + qd]


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
def test_grouped_gemm_mxfp4_packed_matches_canonical_bits(T, E, k, bm):
    ids, al = _routing(T, E, k, bm, seed=T + 5)
    R, I, K = T * k, 128, 256
    Aq, As, Wq, We = _mx_operands(T, 2 * I, K, E, seed=bm)
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([al["num_tiles"]], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    dWq, dWe = gu.dev(Wq), gu.dev(We)
    pWq, pWe = moe.moe_mx_prepack(dWq, dWe)
    outs = []
    for Wt, Et, lay in ((dWq, dWe, moe.MOE_LAYOUT_CANONICAL), (pWq, pWe, moe.MOE_LAYOUT_PACKED)):
        h = moe.moe_grouped_gemm_mxfp4(gu.dev(Aq), gu.dev(As), srt, k, Wt, Et, tiles, al["num_tiles"], nt, bm,
                                       moe.MOE_EPI_SILU_MUL, R, weight_layout=lay)
        o = moe.moe_grouped_gemm_mxfp4(gu.dev(Aq), gu.dev(As), srt, k, Wt, Et, tiles, al["num_tiles"], nt, bm,
                                       moe.MOE_EPI_NONE, R, weight_layout=lay)
        torch.cuda.synchronize()
        outs.append((h[0].cpu().numpy(), h[1].cpu().numpy(), o.view(torch.int32).cpu().numpy()))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["tiny", "dec1", "dec64", "pre800", "big4096", "skew8192"])
def test_ffn_forward_mxfp4_packed_matches_canonical_bits(name):
    wl = mi.WORKLOADS[name]
    d = MXDevice(mi.make_mx_inputs(wl))
    y0, i0 = _forward(d, wl)
    y1, i1 = _forward(d, wl, moe.MOE_LAYOUT_PACKED)
    np.testing.assert_array_equal(i0.cpu().numpy(), i1.cpu().numpy())
    np.testing.assert_array_equal(y0.view(torch.int16).cpu().numpy(), y1.view(torch.int16).cpu().numpy())


@pytest.mark.parametrize("wl", [mi.custom("mxp_bm16", 40, 16, 4, 256, 128, seed=21),
                                mi.custom("mxp_bm32", 90, 12, 3, 384, 256, seed=22),
                                mi.custom("mxp_bm64", 300, 8, 2, 256, 384, seed=23)])
def test_ffn_forward_mxfp4_packed_matches_oracle(wl):
    inp = mi.make_mx_inputs(wl)
    d = MXDevice(inp)
    y, ids = _forward(d, wl, moe.MOE_LAYOUT_PACKED)
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    gu.assert_within_tolerance(gu.host_bf16_to_f64(y), oracle.moe_ffn_mx(inp), wl.name)


@pytest.mark.parametrize("T,E,k,bm", GEMM_CASES)
def test_mxfp4_tiled_activation_chain_matches_row_major_bits(T, E, k, bm):
    # x -> quantize -> gate_up (SiLU*mul, h quantized) -> down, once with row-major activations and
    # canonical weights, once with tile-blocked activations and packed weights: same O bits
    ids, al = _routing(T, E, k, bm, seed=T + 11)
    R, H, I = T * k, 256, 128
    rng = np.random.default_rng(bm + T)
    x = gu.dev_bf16(mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    _, _, W13, E13 = _mx_operands(1, 2 * I, H, E, seed=3)
    _, _, W2, E2 = _mx_operands(1, H, I, E, seed=4)
    W13, E13, W2, E2 = gu.dev(W13), gu.dev(E13), gu.dev(W2), gu.dev(E2)
    P13, Q13 = moe.moe_mx_prepack(W13, E13)
    P2, Q2 = moe.moe_mx_prepack(W2, E2)
    mt = al["num_tiles"]
    tiles = gu.dev(np.ascontiguousarray(al["tiles"].astype(np.int32)))
    nt = gu.dev(np.array([mt], np.int32))
    srt = gu.dev(al["sorted_ids"].astype(np.int32))
    xq, xs = moe.moe_mx_quantize(x)
    hq, hs = moe.moe_grouped_gemm_mxfp4(xq, xs, srt, k, W13, E13, tiles, mt, nt, bm, moe.MOE_EPI_SILU_MUL, R)
    O1 = moe.moe_grouped_gemm_mxfp4(hq, hs, None, 1, W2, E2, tiles, mt, nt, bm, moe.MOE_EPI_NONE, R)
    tq, ts = moe.moe_mx_quantize_tiles(x, srt, k, tiles, mt, nt, bm)
    gq, gs = moe.moe_grouped_gemm_mxfp4(tq, ts, None, 1, P13, Q13, tiles, mt, nt, bm, moe.MOE_EPI_SILU_MUL, R,
                                        weight_layout=moe.MOE_LAYOUT_PACKED, act_layout=moe.MOE_ACT_TILED)
    O2 = moe.moe_grouped_gemm_mxfp4(gq, gs, None, 1, P2, Q2, tiles, mt, nt, bm, moe.MOE_EPI_NONE, R,
                                    weight_layout=moe.MOE_LAYOUT_PACKED, act_layout=moe.MOE_ACT_TILED)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(O1.view(torch.int32).cpu().numpy(), O2.view(torch.int32).cpu().numpy())
