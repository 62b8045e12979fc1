"""GPU parity: every entry point of libmoe_w4a16 against the CPU oracle on the same seeded inputs.

Integer results (routing ids, counts, offsets, permutation, tiles) must be bit-exact; routing weights
within 1e-6; layer outputs within max|gpu-ref| <= 3e-2 * rms(ref) and mean relative error <= 5e-3.
Full-size workloads are checked on sampled tokens (each token's output is independent) in the same
launch configuration the benchmark times, plus properties that hold at any size.
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

_CACHE = {}


def workload_inputs(name_or_wl):
    wl = mi.WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    key = (wl.name, wl.T, wl.E, wl.k, wl.H, wl.I, wl.skew, wl.seed)
    if key not in _CACHE:
        if len(_CACHE) > 3:
            _CACHE.clear()
            torch.cuda.empty_cache()
        inp = mi.make_inputs(wl)
        _CACHE[key] = (inp, gu.DeviceInputs(inp))
    return _CACHE[key]


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------------------------------
# routing

ROUTE_CASES = ["tiny", "dec64", "pre800", "big4096", "skew8192"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_topk_matches_oracle(name):
    inp, d = workload_inputs(name)
    ids, w = moe.moe_route_topk(d.logits, inp.wl.k)
    torch.cuda.synchronize()
    rid, rw = oracle.route(inp.logits, inp.wl.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= gu.ROUTE_W_ATOL


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 65, 65), (33, 1024, 16), (130, 64, 6), (5, 3, 2)])
def test_route_topk_edges_and_ties(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.integers(-3, 4, (T, E)).astype(np.float32)  # many equal logits: ties by lower id
    logits[0, ::2] = -0.0
    logits[0, 1::2] = 0.0
    ids, w = moe.moe_route_topk(gu.dev(logits), k)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= gu.ROUTE_W_ATOL


def _threshold_logits(T, E, k, seed):
    """Logits whose selection boundary sits at different depths of the radix select: token t % 3 == 0
    has its k-th and (k+1)-th largest logits one float apart (every bit decides), t % 3 == 1 has exactly
    k positive logits (the sign bit decides), t % 3 == 2 has the k-th and (k+1)-th largest equal (a tie
    at the boundary, resolved by the lower expert id).  Needs 1 <= k < E."""
    rng = np.random.default_rng(seed)
    out = np.empty((T, E), np.float32)
    for t in range(T):
        vals = np.sort(rng.standard_normal(E).astype(np.float32))[::-1].copy()
        mode = t % 3
        if mode == 0:
            vals[k] = np.nextafter(vals[k - 1], np.float32(-np.inf))
            vals[k + 1:] = np.minimum(vals[k + 1:], np.nextafter(vals[k], np.float32(-np.inf)))
        elif mode == 1:
            vals = np.abs(vals) + np.float32(0.25)
            vals[k:] = -vals[k:]
        else:
            vals[k] = vals[k - 1]
        out[t, rng.permutation(E)] = vals
    return out


@pytest.mark.parametrize("E,k", [(64, 8), (128, 8), (128, 1), (256, 8), (512, 10), (1000, 16), (33, 32)])
def test_route_topk_boundary_depths(E, k):
    """The selection stops once a key prefix separates exactly k logits; boundaries decided by the
    sign bit, by the last mantissa bit, and by a tie must all give the oracle's routing."""
    logits = _threshold_logits(9, E, k, seed=E + k)
    ids, w = moe.moe_route_topk(gu.dev(logits), k)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= gu.ROUTE_W_ATOL


@pytest.mark.parametrize("E", [128, 256])
def test_ffn_forward_prologue_boundary_depths(E):
    """At 12 tokens the gate_up launch routes in its prologue; with the boundary logits above its
    routing, permutation and output must equal, bit for bit, those of the separate entry points."""
    wl = mi.custom("boundary", 12, E, 8, 256, 128, seed=31)
    inp = mi.make_inputs(wl)
    inp.logits = _threshold_logits(wl.T, E, wl.k, seed=31 + E)
    rid, _ = oracle.route(inp.logits, wl.k)
    d = gu.DeviceInputs(inp)
    _log(f"prologue boundary logits E={E}")
    y_ref = _bits(_layer_from_entry_points(d, inp, True))
    q13, s13, q2, s2 = _packed(d)
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    wsb = moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k)
    ws = torch.full((max(wsb, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    ids = torch.full((wl.T, wl.k), -1, dtype=torch.int32, device="cuda")
    moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, workspace=ws,
                        weight_layout=moe.MOE_LAYOUT_PACKED, topk_ids_out=ids)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_array_equal(_bits(y), y_ref)


# ---------------------------------------------------------------------------------------------------
# permutation

ALIGN_CASES = [("tiny", 16), ("dec1", 16), ("dec64", 16), ("pre800", 32), ("pre800", 128), ("big4096", 128),
               ("skew8192", 128), ("skew8192", 16)]


def _check_align(got, ref):
    for key in ("counts", "offsets"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(got["sorted_ids"].cpu().numpy()[:R], ref["sorted_ids"])
    np.testing.assert_array_equal(got["inv_perm"].cpu().numpy()[:R], ref["inv_perm"])
    nt = int(got["num_tiles"].item())
    assert nt == ref["num_tiles"]
    np.testing.assert_array_equal(got["tiles"].cpu().numpy()[:nt], ref["tiles"])


@pytest.mark.parametrize("name,bm", ALIGN_CASES)
def test_align_matches_oracle(name, bm):
    inp, d = workload_inputs(name)
    rid, _ = oracle.route(inp.logits, inp.wl.k)
    got = moe.moe_align(gu.dev(rid), inp.wl.E, bm)
    torch.cuda.synchronize()
    _check_align(got, oracle.align(rid, inp.wl.E, bm))


@pytest.mark.parametrize("T,E,k,bm", [(0, 8, 2, 16), (1, 1, 1, 16), (5000, 4, 4, 64), (300, 1024, 8, 32),
                                      (16385, 2, 1, 128), (3000, 600, 6, 16)])
def test_align_edges(T, E, k, bm):
    rng = np.random.default_rng(T + 7 * E)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        if T > 10 and t < T // 2:  # a hot expert: slot 0 of half the tokens goes to expert 0
            ids[t] = [0, *rng.choice(np.arange(1, E), k - 1, replace=False)]
        else:
            ids[t] = rng.choice(E, k, replace=False)
    got = moe.moe_align(gu.dev(ids) if T else torch.empty((0, k), dtype=torch.int32, device="cuda"), E, bm)
    torch.cuda.synchronize()
    _check_align(got, oracle.align(ids, E, bm))


# ---------------------------------------------------------------------------------------------------
# grouped GEMM entry point on its own

@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("I,H", [(128, 256), (96, 160), (256, 96)])
def test_grouped_gemm_gate_up_silu_mul(bm, I, H):
    wl = mi.custom("gg", 150, 8, 3, H, I, skew=True, seed=11)
    inp, d = workload_inputs(wl)
    rid, _ = oracle.route(inp.logits, wl.k)
    a = moe.moe_align(gu.dev(rid), wl.E, bm)
    R = wl.T * wl.k
    C = moe.moe_grouped_gemm_w4a16(d.x, a["sorted_ids"], wl.k, d.w13_q, d.w13_s, a["tiles"], a["max_tiles"],
                                   a["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R)
    torch.cuda.synchronize()
    ra = oracle.align(rid, wl.E, bm)
    ref = oracle.grouped_proj(inp.x, ra["sorted_ids"], wl.k, inp.w13_q, inp.w13_s, ra["offsets"], silu_mul=True)
    # Per-element bound from the arithmetic: h is rounded once to bf16 (<= 2^-8 relative); the fp32
    # gate and up sums carry at most (64 + H/32) * 2^-24 * sum|terms| each, which silu(g)*u propagates
    # with |d silu/dg| <= 1.1 and |silu(g)| <= |g|.
    G = oracle.grouped_proj(inp.x, ra["sorted_ids"], wl.k, inp.w13_q, inp.w13_s, ra["offsets"])
    Gabs = oracle.grouped_proj(inp.x & 0x7FFF, ra["sorted_ids"], wl.k, inp.w13_q & 0x77, inp.w13_s, ra["offsets"])
    dG = (64 + H / 32) * 2.0 ** -24 * Gabs
    g, u, dg, du = G[:, :I], G[:, I:], dG[:, :I], dG[:, I:]
    bound = 2.0 ** -8 * np.abs(ref) + 1.1 * np.abs(u) * dg + np.abs(g) * du + 1e-6 * np.abs(ref)
    got = gu.host_bf16_to_f64(C)
    assert np.all(np.abs(got - ref) <= bound), f"gate_up bm={bm}: worst excess {np.max(np.abs(got - ref) - bound)}"
    assert gu.tolerance_report(got, ref)["mean_rel"] <= gu.MEAN_REL


@pytest.mark.parametrize("I,H", [(128, 256), (96, 160), (256, 384)])
def test_grouped_gemm_split_k_gate_up(I, H):
    # 40 tokens top-2 over 8 experts with 16-row tiles: a tile list short enough for the split-K
    # kernel (four waves each own a quarter of K; partial sums reduced in wave order).
    wl = mi.custom("sk", 40, 8, 2, H, I, skew=True, seed=17)
    inp, d = workload_inputs(wl)
    rid, _ = oracle.route(inp.logits, wl.k)
    a = moe.moe_align(gu.dev(rid), wl.E, 16)
    assert a["max_tiles"] <= 32
    R = wl.T * wl.k
    C = moe.moe_grouped_gemm_w4a16(d.x, a["sorted_ids"], wl.k, d.w13_q, d.w13_s, a["tiles"], a["max_tiles"],
                                   a["num_tiles"], 16, moe.MOE_EPI_SILU_MUL, R)
    torch.cuda.synchronize()
    ra = oracle.align(rid, wl.E, 16)
    ref = oracle.grouped_proj(inp.x, ra["sorted_ids"], wl.k, inp.w13_q, inp.w13_s, ra["offsets"], silu_mul=True)
    G = oracle.grouped_proj(inp.x, ra["sorted_ids"], wl.k, inp.w13_q, inp.w13_s, ra["offsets"])
    Gabs = oracle.grouped_proj(inp.x & 0x7FFF, ra["sorted_ids"], wl.k, inp.w13_q & 0x77, inp.w13_s, ra["offsets"])
    dG = (64 + H / 32) * 2.0 ** -24 * Gabs
    g, u, dg, du = G[:, :I], G[:, I:], dG[:, :I], dG[:, I:]
    bound = 2.0 ** -8 * np.abs(ref) + 1.1 * np.abs(u) * dg + np.abs(g) * du + 1e-6 * np.abs(ref)
    got = gu.host_bf16_to_f64(C)
    assert np.all(np.abs(got - ref) <= bound), f"split-K gate_up: worst excess {np.max(np.abs(got - ref) - bound)}"
    if H % 128 == 0:
        pq, ps = moe.moe_w4_prepack(d.w13_q, d.w13_s)
        Cp = moe.moe_grouped_gemm_w4a16(d.x, a["sorted_ids"], wl.k, pq, ps, a["tiles"], a["max_tiles"],
                                        a["num_tiles"], 16, moe.MOE_EPI_SILU_MUL, R,
                                        weight_layout=moe.MOE_LAYOUT_PACKED)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Cp.view(torch.int16).cpu().numpy(), C.view(torch.int16).cpu().numpy())


def f16e_decode(bits, side):
    """fp16 values (uint16 bits [rows, N]) with in-band exponents and side values [rows, N/8] ->
    (float64 values, exponent per 8-column segment).  A segment whose first element is the marker
    (fp16 quiet NaN 0x7E00 | (exp + 256)) is scaled by 2^exp and its first value is the side value."""
    bits = np.asarray(bits, np.uint16)
    rows, N = bits.shape
    v = bits.view(np.float16).astype(np.float64).reshape(rows, N // 8, 8)
    first = bits.reshape(rows, N // 8, 8)[:, :, 0]
    marked = (first & 0x7E00) == 0x7E00
    ex = np.where(marked, (first & 0x1FF).astype(np.int64) - 256, 0)
    v[:, :, 0] = np.where(marked, side, v[:, :, 0])
    return (v * np.ldexp(1.0, ex)[:, :, None]).reshape(rows, N), ex


def f16e_to_f64(C, Cs):
    return f16e_decode(C.view(torch.int16).cpu().numpy().view(np.uint16), Cs.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("bm", [16, 64, 128])
@pytest.mark.parametrize("out_dtype", [moe.MOE_OUT_F32, moe.MOE_OUT_BF16, moe.MOE_OUT_F16E])
@pytest.mark.parametrize("N,K", [(256, 128), (200, 160), (48, 1056)])
def test_grouped_gemm_plain(bm, out_dtype, N, K):
    E, T, k = 6, 90, 2
    rng = np.random.default_rng(N + K + bm)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    logits[:, 0] += 3.0  # uneven expert sizes, several tiles for expert 0
    rid, _ = oracle.route(logits, k)
    R = T * k
    A = mi.f32_to_bf16_bits(rng.standard_normal((R, K), dtype=np.float32))
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    Ws = mi.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    a = moe.moe_align(gu.dev(rid), E, bm)
    C = moe.moe_grouped_gemm_w4a16(gu.dev_bf16(A), None, 1, gu.dev(Wq), gu.dev(Ws.view(np.int16)), a["tiles"],
                                   a["max_tiles"], a["num_tiles"], bm, moe.MOE_EPI_NONE, R, out_dtype)
    torch.cuda.synchronize()
    ra = oracle.align(rid, E, bm)
    ref = oracle.grouped_proj(A, None, 1, Wq, Ws, ra["offsets"])
    if out_dtype == moe.MOE_OUT_F16E:
        C, Cs = C
        got, ex = f16e_to_f64(C, Cs)
        assert np.all(ex == 0)  # magnitudes of order 1: no segment is scaled
    else:
        got = C.cpu().numpy().astype(np.float64) if out_dtype == moe.MOE_OUT_F32 else gu.host_bf16_to_f64(C)
    # bf16 x E2M1 products are exact in fp32; the fp32 summation takes at most (32 + K/32) roundings
    # along any path, so |err| <= (64 + K/32) * 2^-24 * sum|terms|; an fp16 output adds one rounding
    # (2^-11 relative, 2^-25 absolute below fp16's normal range).
    ref_abs = oracle.grouped_proj(A & 0x7FFF, None, 1, Wq & 0x77, Ws, ra["offsets"])
    acc_err = (64 + K / 32) * 2.0 ** -24 * ref_abs
    if out_dtype == moe.MOE_OUT_F32:
        assert np.all(np.abs(got - ref) <= acc_err)
    elif out_dtype == moe.MOE_OUT_F16E:
        assert np.all(np.abs(got - ref) <= acc_err + 2.0 ** -11 * (np.abs(ref) + acc_err) + 2.0 ** -25)
    gu.assert_within_tolerance(got, ref, "plain")


@pytest.mark.parametrize("bm,layout", [(32, 0), (64, 0), (16, 0), (128, 1)])
def test_grouped_gemm_f16e_exponents(bm, layout):
    """Outputs far beyond fp16's range: each 8-column row segment holding a magnitude >= 2^15 is
    stored scaled by 2^-exp (its largest magnitude then below 2^15), marked in its first element,
    whose value goes to the side array; decoded values stay within the fp32 summation bound plus one
    fp16 rounding, and unmarked segments are plain fp16."""
    E, T, k, N, K = 4, 70, 2, 256, 256
    rng = np.random.default_rng(bm + 5)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    rid, _ = oracle.route(logits, k)
    R = T * k
    A = rng.standard_normal((R, K), dtype=np.float32)
    A[::3] *= 2.0 ** 20  # every third row: outputs around 2^22
    A[1::7, :8] *= 2.0 ** 40  # a few rows with a huge first group: far above the rest
    A[2::9] *= 2.0 ** -30  # tiny rows: scaled up, keeping their relative precision
    A = mi.f32_to_bf16_bits(A)
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    Ws = mi.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    a = moe.moe_align(gu.dev(rid), E, bm)
    d_wq, d_ws = gu.dev(Wq), gu.dev(Ws.view(np.int16))
    if layout:
        d_wq, d_ws = moe.moe_w4_prepack(d_wq, d_ws)
    C, Cs = moe.moe_grouped_gemm_w4a16(gu.dev_bf16(A), None, 1, d_wq, d_ws, a["tiles"], a["max_tiles"],
                                       a["num_tiles"], bm, moe.MOE_EPI_NONE, R, moe.MOE_OUT_F16E, weight_layout=layout)
    torch.cuda.synchronize()
    ra = oracle.align(rid, E, bm)
    ref = oracle.grouped_proj(A, None, 1, Wq, Ws, ra["offsets"])
    ref_abs = oracle.grouped_proj(A & 0x7FFF, None, 1, Wq & 0x77, Ws, ra["offsets"])
    got, ex = f16e_to_f64(C, Cs)
    acc_err = (64 + K / 32) * 2.0 ** -24 * ref_abs
    scale = np.repeat(np.ldexp(1.0, ex), 8, axis=1)
    assert np.all(np.abs(got - ref) <= acc_err + 2.0 ** -11 * (np.abs(ref) + acc_err) + 2.0 ** -25 * scale)
    # a segment is marked exactly where its largest magnitude reaches 2^15
    seg_max = np.abs(got).reshape(R, N // 8, 8).max(axis=2)  # (after one fp16 rounding)
    assert np.all(seg_max[ex > 0] >= 2.0 ** 15 * (1 - 2.0 ** -10)) and np.all(seg_max[ex == 0] <= 2.0 ** 15)
    assert np.all(seg_max[ex < 0] < 2.0 ** -6)
    assert np.all((seg_max[ex == 0] >= 2.0 ** -6 * (1 - 2.0 ** -10)) | (seg_max[ex == 0] == 0))
    assert ex.max() >= 40 and ex.min() <= -20 and (ex == 0).any()


@pytest.mark.parametrize("k", [5, 8, 10, 16])
def test_combine_f16e_matches_oracle(k):
    """fp16 O with in-band exponents (the layer's down-projection output): every fifth row has its
    segments marked with exponents -40..29 (side values in place of their first elements); each value
    decodes exactly to fp32, so the bound is that of fp32 O."""
    T, H = 29, 272
    rng = np.random.default_rng(7 + k)
    O16 = rng.standard_normal((T * k, H)).astype(np.float16)
    bits = O16.view(np.uint16).copy()
    side = rng.standard_normal((T * k, H // 8)).astype(np.float32)
    ex = rng.integers(-40, 30, (T * k, H // 8))
    marked = np.zeros((T * k, H // 8), bool)
    marked[::5] = True
    bits.reshape(T * k, H // 8, 8)[:, :, 0] = np.where(marked, 0x7E00 | (ex + 256),
                                                       bits.reshape(T * k, H // 8, 8)[:, :, 0])
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    y = moe.moe_combine(gu.dev(bits.view(np.int16)).view(torch.float16), gu.dev(inv), gu.dev(w), O_side=gu.dev(side))
    torch.cuda.synchronize()
    O, _ = f16e_decode(bits, side.astype(np.float64))
    ref = oracle.combine(O, inv, w.astype(np.float64), T, k)
    terms = oracle.combine(np.abs(O), inv, w.astype(np.float64), T, k)
    got = gu.host_bf16_to_f64(y)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + (k + 2) * 2.0 ** -23 * terms)


@pytest.mark.parametrize("k", [5, 8, 10, 16])
@pytest.mark.parametrize("with_shared", [False, True])
def test_combine_matches_oracle(k, with_shared):
    """k = 5: the slot-by-slot tail only; 8: one whole chunk of 8 slots; 10: a chunk and a tail;
    16: two chunks.  fp32 sums of at most k + 1 terms (each rounding at most 2^-24 of the running
    sum, itself at most sum|terms|), then one bf16 rounding (2^-8 relative); the bound below doubles
    the summation term to cover the rounding of the rounded sum."""
    T, H = 37, 264
    rng = np.random.default_rng(3 + k)
    O = rng.standard_normal((T * k, H)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    S = rng.standard_normal((T, H)).astype(np.float32) if with_shared else None
    y = moe.moe_combine(gu.dev(O), gu.dev(inv), gu.dev(w), shared=None if S is None else gu.dev(S))
    torch.cuda.synchronize()
    ref = oracle.combine(O.astype(np.float64), inv, w.astype(np.float64), T, k)
    terms = oracle.combine(np.abs(O.astype(np.float64)), inv, w.astype(np.float64), T, k)
    if S is not None:
        ref = ref + S
        terms = terms + np.abs(S)
    got = gu.host_bf16_to_f64(y)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + (k + 2) * 2.0 ** -23 * terms)


# ---------------------------------------------------------------------------------------------------
# whole layer

def _forward(d, inp, poison=True):
    wl = inp.wl
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((wl.T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    wsb = moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k)
    ws = torch.full((max(wsb, 256),), 0xFF if poison else 0, dtype=torch.uint8, device="cuda")
    moe.moe_ffn_forward(d.x, d.logits, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k, y=y, topk_ids_out=ids,
                        topk_w_out=w, workspace=ws)
    torch.cuda.synchronize()
    return y, ids, w


# Sampled tokens cover every touched expert (the skewed workload's rarely chosen ones included); the
# 800-token layer is checked on every token.
FULL_CASES = [("tiny", 16), ("dec1", 1), ("dec8", 8), ("dec32", 32), ("dec64", 64), ("pre800", 800),
              ("big4096", 512), ("skew8192", 1024)]


@pytest.mark.parametrize("name,nsample", FULL_CASES)
def test_ffn_forward_matches_oracle(name, nsample):
    inp, d = workload_inputs(name)
    wl = inp.wl
    _log(f"ffn_forward {name}: T={wl.T} E={wl.E} k={wl.k} H={wl.H} I={wl.I}")
    y, ids, w = _forward(d, inp)
    rid, rw = oracle.route(inp.logits, wl.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= gu.ROUTE_W_ATOL
    yh = gu.host_bf16_to_f64(y)
    assert np.all(np.isfinite(yh)), "output not fully written"
    tok = gu.sample_tokens(wl.T, nsample, rid)
    ref = oracle.moe_ffn(inp, tokens=tok)
    r = gu.assert_within_tolerance(yh[tok], ref, name)
    _log(f"  {name}: {r}")


@pytest.mark.parametrize("wl", [
    mi.custom("one_expert", 3, 1, 1, 256, 128, seed=5),
    mi.custom("ragged", 37, 16, 4, 160, 96, seed=6),
    mi.custom("k_eq_E", 20, 6, 6, 128, 64, seed=7),
    mi.custom("many_experts", 40, 1024, 8, 128, 64, seed=8),
    mi.custom("t1_big_k", 1, 64, 32, 256, 256, seed=9),
    # the fused small-batch routing + permutation at its limits (16 tokens, k = 64: 1024 slots;
    # 512 experts) and just past them (17 tokens: separate launches)
    mi.custom("fused_max", 16, 128, 64, 128, 64, seed=10),
    mi.custom("fused_e512", 16, 512, 8, 128, 64, seed=15),
    mi.custom("fused_past", 17, 128, 8, 128, 64, seed=16),
    # a few dozen tokens: k = 16 with 1024 slots, 256 experts, 65 tokens
    mi.custom("t64_k16", 64, 128, 16, 128, 64, seed=21),
    mi.custom("t40_e256", 40, 256, 8, 128, 64, seed=22),
    mi.custom("t65", 65, 64, 4, 128, 64, seed=23),
    # the gate_up launch's routing prologue (at most 16 tokens, k <= 16) at its limits: 512 experts
    # with k = 16, 129 experts (the wider selection), k = E, one token; k = 17 falls back
    mi.custom("prologue_max", 16, 512, 16, 128, 64, seed=17),
    mi.custom("prologue_e129", 5, 129, 16, 160, 96, seed=18),
    mi.custom("prologue_k_eq_E", 3, 4, 4, 128, 64, seed=19),
    mi.custom("prologue_t1", 1, 256, 8, 256, 128, seed=20),
    mi.custom("prologue_past_k", 4, 64, 17, 128, 64, seed=24),
])
def test_ffn_forward_edges(wl):
    inp, d = workload_inputs(wl)
    y, ids, _ = _forward(d, inp)
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    gu.assert_within_tolerance(gu.host_bf16_to_f64(y), oracle.moe_ffn(inp), wl.name)


def test_ffn_forward_hot_expert():
    wl = mi.custom("hot", 300, 32, 4, 256, 128, seed=12)
    inp = mi.make_inputs(wl)
    inp.logits[:, 0] += 50.0  # every token's slot 0 goes to expert 0: ceil(300/BM) tiles there
    d = gu.DeviceInputs(inp)
    y, ids, _ = _forward(d, inp)
    assert np.all(ids.cpu().numpy()[:, 0] == 0)
    gu.assert_within_tolerance(gu.host_bf16_to_f64(y), oracle.moe_ffn(inp), "hot")


# ---------------------------------------------------------------------------------------------------
# exact invariants of the GPU path (no oracle needed, hold at any size)

def _bits(y):
    return y.view(torch.int16).cpu().numpy()


def test_deterministic_and_scale_equivariant():
    wl = mi.custom("inv", 200, 32, 4, 512, 256, seed=13)
    inp = mi.make_inputs(wl)
    d = gu.DeviceInputs(inp)
    y1 = _bits(_forward(d, inp)[0])
    y2 = _bits(_forward(d, inp, poison=False)[0])
    np.testing.assert_array_equal(y1, y2)
    base = gu.host_bf16_to_f64(_forward(d, inp)[0])
    # doubling every up-projection scale (rows I..2I of gate_up) doubles y exactly
    s = inp.w13_s.copy()
    s[:, wl.I:, :] = mi.f32_to_bf16_bits(mi.bf16_bits_to_f32(s[:, wl.I:, :]) * 2)
    d.w13_s = gu.dev(s.view(np.int16))
    np.testing.assert_array_equal(gu.host_bf16_to_f64(_forward(d, inp)[0]), 2 * base)
    d.w13_s = gu.dev(inp.w13_s.view(np.int16))
    s2 = mi.f32_to_bf16_bits(mi.bf16_bits_to_f32(inp.w2_s) * 2)
    d.w2_s = gu.dev(s2.view(np.int16))
    np.testing.assert_array_equal(gu.host_bf16_to_f64(_forward(d, inp)[0]), 2 * base)


def test_token_permutation_equivariant():
    wl = mi.custom("perm", 160, 16, 4, 256, 128, seed=14)
    inp = mi.make_inputs(wl)
    d = gu.DeviceInputs(inp)
    y = _bits(_forward(d, inp)[0])
    p = np.random.default_rng(0).permutation(wl.T)
    inp2 = mi.MoEInputs(wl, inp.x[p].copy(), inp.logits[p].copy(), inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s)
    d2 = gu.DeviceInputs(inp2)
    np.testing.assert_array_equal(_bits(_forward(d2, inp2)[0]), y[p])


# ---------------------------------------------------------------------------------------------------
# decode batches (at most 16 routed rows in 16-row tiles, the split-K kernels), every token checked

DC_CASES = [
    mi.custom("dc_t1_k16", 1, 64, 16, 256, 128, seed=51),    # 16 tiles of one row: two rounds of 8 slots
    mi.custom("dc_t16_k1", 16, 32, 1, 256, 128, seed=52),    # 16 tokens, up to 16 tiles
    mi.custom("dc_t2_k8", 2, 128, 8, 512, 256, seed=53),     # K = 256: both K halves of a tile busy
    mi.custom("dc_t4_e2", 4, 2, 2, 128, 128, seed=54),       # two tiles of 4 rows each
    mi.custom("dc_t3_tail", 3, 8, 4, 160, 96, seed=55),      # I = 96: the canonical form's K tail
    mi.custom("dc_t5_k3", 5, 16, 3, 256, 128, seed=56),      # 15 rows
]


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_CANONICAL, moe.MOE_LAYOUT_PACKED])
@pytest.mark.parametrize("wl", DC_CASES, ids=lambda w: w.name)
def test_decode_batch_matches_oracle(wl, layout):
    """Every token against the oracle, the routing bit-exact, and two calls bit-identical."""
    assert wl.T * wl.k <= 16 and moe.moe_ffn_block_m(wl.T, wl.E, wl.k, layout) == 16
    if layout == moe.MOE_LAYOUT_PACKED and wl.I % 128:
        pytest.skip("packed weights need K % 128 == 0")
    inp = mi.make_inputs(wl)
    d = gu.DeviceInputs(inp)
    wts = _packed(d) if layout == moe.MOE_LAYOUT_PACKED else (d.w13_q, d.w13_s, d.w2_q, d.w2_s)
    _log(f"decode down+combine {wl.name} layout {layout}")
    outs = []
    for _ in range(2):
        y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        ids = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
        ws = torch.full((max(moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256),), 0xFF,
                        dtype=torch.uint8, device="cuda")
        moe.moe_ffn_forward(d.x, d.logits, *wts, wl.k, y=y, topk_ids_out=ids, workspace=ws, weight_layout=layout)
        torch.cuda.synchronize()
        outs.append((y, ids))
    np.testing.assert_array_equal(_bits(outs[0][0]), _bits(outs[1][0]))
    np.testing.assert_array_equal(outs[0][1].cpu().numpy(), oracle.route(inp.logits, wl.k)[0])
    gu.assert_within_tolerance(gu.host_bf16_to_f64(outs[0][0]), oracle.moe_ffn(inp), wl.name)


# ---------------------------------------------------------------------------------------------------
# packed weight layout: same values re-laid out; results must be bit-identical to the canonical path

def _packed(d):
    q13, s13 = moe.moe_w4_prepack(d.w13_q, d.w13_s)
    q2, s2 = moe.moe_w4_prepack(d.w2_q, d.w2_s)
    return q13, s13, q2, s2


def test_prepack_is_a_permutation_of_bytes():
    wl = mi.custom("pk", 4, 3, 1, 256, 128, seed=21)
    inp, d = workload_inputs(wl)
    q13, s13 = moe.moe_w4_prepack(d.w13_q, d.w13_s)
    torch.cuda.synchronize()
    a = np.sort(d.w13_q.cpu().numpy().ravel())
    b = np.sort(q13.cpu().numpy().ravel())
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(np.sort(d.w13_s.cpu().numpy().ravel()), np.sort(s13.cpu().numpy().ravel()))


@pytest.mark.parametrize("name", ["tiny", "dec1", "dec64", "pre800", "big4096", "skew8192"])
def test_ffn_forward_packed_matches_canonical_bits(name):
    """Packed weights give the canonical layout's bits wherever both run the same arithmetic; where
    the packed layout's 128-row tiles take the exact fp16 path (the canonical one stays on bf16), the
    packed layer is checked against the oracle on sampled tokens instead."""
    inp, d = workload_inputs(name)
    wl = inp.wl
    _log(f"packed forward {name}")
    y_c = _bits(_forward(d, inp)[0])
    q13, s13, q2, s2 = _packed(d)
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, weight_layout=moe.MOE_LAYOUT_PACKED)
    torch.cuda.synchronize()
    if moe.moe_ffn_block_m(wl.T, wl.E, wl.k, moe.MOE_LAYOUT_PACKED) < 128:
        np.testing.assert_array_equal(_bits(y), y_c)
        return
    yh = gu.host_bf16_to_f64(y)
    assert np.all(np.isfinite(yh)), "output not fully written"
    rid, _ = oracle.route(inp.logits, wl.k)
    tok = gu.sample_tokens(wl.T, 256, rid)
    r = gu.assert_within_tolerance(yh[tok], oracle.moe_ffn(inp, tokens=tok), name + " (packed, fp16 path)")
    _log(f"  {name}: {r}")


def _layer_from_entry_points(d, inp, packed):
    """The layer composed from the separate entry points, ending with the stand-alone combine."""
    wl = inp.wl
    layout = moe.MOE_LAYOUT_PACKED if packed else moe.MOE_LAYOUT_CANONICAL
    q13, s13, q2, s2 = _packed(d) if packed else (d.w13_q, d.w13_s, d.w2_q, d.w2_s)
    ids, w = moe.moe_route_topk(d.logits, wl.k)
    bm = moe.moe_ffn_block_m(wl.T, wl.E, wl.k, layout)
    al = moe.moe_align(ids, wl.E, bm)
    R = wl.T * wl.k
    if bm >= 128:  # the layer runs 128-row tiles on the exact fp16 path
        x16, xe = moe.moe_x_to_f16(d.x)
        h, he = moe.moe_grouped_gemm_w4f16(x16, xe, None, al["sorted_ids"], wl.k, q13, s13, al["tiles"],
                                           al["max_tiles"], al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R,
                                           moe.MOE_OUT_H16, weight_layout=layout)
        O, Os = moe.moe_grouped_gemm_w4f16(h, None, he, None, 1, q2, s2, al["tiles"], al["max_tiles"],
                                           al["num_tiles"], bm, moe.MOE_EPI_NONE, R, moe.MOE_OUT_F16E,
                                           weight_layout=layout)
    else:
        h = moe.moe_grouped_gemm_w4a16(d.x, al["sorted_ids"], wl.k, q13, s13, al["tiles"], al["max_tiles"],
                                       al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, weight_layout=layout)
        O, Os = moe.moe_grouped_gemm_w4a16(h, None, 1, q2, s2, al["tiles"], al["max_tiles"], al["num_tiles"], bm,
                                           moe.MOE_EPI_NONE, R, out_dtype=moe.MOE_OUT_F16E, weight_layout=layout)
    y = moe.moe_combine(O, al["inv_perm"], w, O_side=Os)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name,packed", [("tiny", False), ("dec1", True), ("dec8", True), ("dec8", False),
                                         # the fp16 path with K tails (H = 160, I = 96; 64-row tiles)
                                         (mi.custom("f16_tails", 300, 4, 2, 160, 96, seed=28), False),
                                         # decode batches with a K tail (I = 96): down rows reduced as
                                         # the split-K kernel (<= 32 tiles) and as the tiled kernel
                                         (mi.custom("tail_split", 2, 16, 4, 160, 96, seed=25), False),
                                         (mi.custom("tail_tiled", 12, 64, 4, 160, 96, seed=26), False),
                                         (mi.custom("k16_tiled", 9, 32, 16, 256, 128, seed=27), False),
                                         ("dec64", True),
                                         ("pre800", True), ("pre800", False), ("skew8192", True),
                                         ("big4096", True)])
def test_ffn_forward_matches_entry_point_chain_bits(name, packed):
    """The layer entry point must give, bit for bit, what the chain of the separate entry points gives
    (routing, permutation, both grouped GEMMs, combine) with the same tile heights; the workspace,
    including every routing region, starts poisoned."""
    inp, d = workload_inputs(name)
    wl = inp.wl
    _log(f"layer vs entry-point chain {wl.name} packed={packed}")
    y_ref = _bits(_layer_from_entry_points(d, inp, packed))
    if packed:
        q13, s13, q2, s2 = _packed(d)
        y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        wsb = moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k)
        ws = torch.full((max(wsb, 256),), 0xFF, dtype=torch.uint8, device="cuda")
        moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, workspace=ws,
                            weight_layout=moe.MOE_LAYOUT_PACKED)
        torch.cuda.synchronize()
    else:
        y = _forward(d, inp)[0]
    np.testing.assert_array_equal(_bits(y), y_ref)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_grouped_gemm_packed_matches_canonical_bits(bm):
    wl = mi.custom("gp", 150, 8, 3, 256, 128, skew=True, seed=23)
    inp, d = workload_inputs(wl)
    rid, _ = oracle.route(inp.logits, wl.k)
    a = moe.moe_align(gu.dev(rid), wl.E, bm)
    R = wl.T * wl.k
    q13, s13, q2, s2 = _packed(d)
    for (wq, ws, pq, ps, epi, A, aro, div, od) in [
            (d.w13_q, d.w13_s, q13, s13, moe.MOE_EPI_SILU_MUL, d.x, a["sorted_ids"], wl.k, moe.MOE_OUT_BF16),
            (d.w2_q, d.w2_s, q2, s2, moe.MOE_EPI_NONE,
             gu.dev_bf16(mi.f32_to_bf16_bits(np.random.default_rng(2).standard_normal((R, wl.I), dtype=np.float32))),
             None, 1, moe.MOE_OUT_F32),
            (d.w2_q, d.w2_s, q2, s2, moe.MOE_EPI_NONE,
             gu.dev_bf16(mi.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((R, wl.I), dtype=np.float32))),
             None, 1, moe.MOE_OUT_F16E)]:
        c1 = moe.moe_grouped_gemm_w4a16(A, aro, div, wq, ws, a["tiles"], a["max_tiles"], a["num_tiles"], bm, epi, R, od)
        c2 = moe.moe_grouped_gemm_w4a16(A, aro, div, pq, ps, a["tiles"], a["max_tiles"], a["num_tiles"], bm, epi, R, od,
                                        weight_layout=moe.MOE_LAYOUT_PACKED)
        torch.cuda.synchronize()
        if od == moe.MOE_OUT_F16E:  # no marked segment at these magnitudes: the side values are unused
            assert np.all(f16e_to_f64(*c1)[1] == 0)
            c1, c2 = c1[0], c2[0]
        view = torch.int32 if od == moe.MOE_OUT_F32 else torch.int16
        np.testing.assert_array_equal(c1.view(view).cpu().numpy(), c2.view(view).cpu().numpy())


# The 128-row large-tile kernel (packed weights, block_m 128) against the canonical 64-row kernel: per
# output element both accumulate the same group partials in K order, so the bits must agree.  Shapes
# cover 1..5 K steps (pipeline prologue and tail), a ragged last N block and ragged row tiles.
@pytest.mark.parametrize("T,E,k,H,I,seed", [
    (300, 4, 2, 640, 416, 31),   # gate_up: 5 K steps, 416 = 3.25 column blocks; down not packable (I % 128)
    (260, 3, 2, 640, 384, 32),   # down: 3 K steps, 640 = 2.5 column blocks; gate_up 5 K steps
    (200, 2, 1, 128, 256, 33),   # gate_up 1 K step; down 2 K steps
])
def test_large_tile_gemm_matches_canonical_bits(T, E, k, H, I, seed):
    wl = mi.custom("mm", T, E, k, H, I, skew=True, seed=seed)
    inp, d = workload_inputs(wl)
    rid, _ = oracle.route(inp.logits, wl.k)
    a64 = moe.moe_align(gu.dev(rid), wl.E, 64)
    a128 = moe.moe_align(gu.dev(rid), wl.E, 128)
    R = wl.T * wl.k
    h = gu.dev_bf16(mi.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((R, wl.I), dtype=np.float32)))
    projs = []
    if wl.H % 128 == 0:
        projs.append((d.w13_q, d.w13_s, moe.MOE_EPI_SILU_MUL, d.x, "sorted", wl.k, moe.MOE_OUT_BF16))
    if wl.I % 128 == 0:
        projs.append((d.w2_q, d.w2_s, moe.MOE_EPI_NONE, h, None, 1, moe.MOE_OUT_F32))
        projs.append((d.w2_q, d.w2_s, moe.MOE_EPI_NONE, h, None, 1, moe.MOE_OUT_F16E))
    assert projs
    for (wq, ws, epi, A, aro, div, od) in projs:
        _log(f"large tile T={T} E={E} k={k} H={H} I={I} epi={epi}")
        pq, ps = moe.moe_w4_prepack(wq, ws)
        ref = moe.moe_grouped_gemm_w4a16(A, a64["sorted_ids"] if aro else None, div, wq, ws, a64["tiles"],
                                         a64["max_tiles"], a64["num_tiles"], 64, epi, R, od)
        out = moe.moe_grouped_gemm_w4a16(A, a128["sorted_ids"] if aro else None, div, pq, ps, a128["tiles"],
                                         a128["max_tiles"], a128["num_tiles"], 128, epi, R, od,
                                         weight_layout=moe.MOE_LAYOUT_PACKED)
        torch.cuda.synchronize()
        if od == moe.MOE_OUT_F16E:  # no marked segment at these magnitudes: the side values are unused
            assert np.all(f16e_to_f64(*ref)[1] == 0)
            out, ref = out[0], ref[0]
        view = torch.int32 if od == moe.MOE_OUT_F32 else torch.int16
        np.testing.assert_array_equal(out.view(view).cpu().numpy(), ref.view(view).cpu().numpy())



@pytest.mark.parametrize("bm,layout", [(16, 0), (64, 1), (128, 1)])
def test_grouped_gemm_large_capacity_grid(bm, layout):
    # A tile-list capacity far above the tiles used makes the work list longer than one grid row
    # (2-D launch); unused slots must cost nothing and change no output bit.  (300 tokens: the
    # normal capacity is above the split-K limit too, so both calls use the same kernel.)
    wl = mi.custom("cap", 300, 8, 2, 256, 128, seed=41)
    inp, d = workload_inputs(wl)
    rid, _ = oracle.route(inp.logits, wl.k)
    R = wl.T * wl.k
    wq, ws = (d.w13_q, d.w13_s) if layout == 0 else moe.moe_w4_prepack(d.w13_q, d.w13_s)
    outs = []
    for cap in (None, 300000):
        a = moe.moe_align(gu.dev(rid), wl.E, bm, max_tiles=cap)
        _log(f"capacity grid bm={bm} layout={layout} max_tiles={a['max_tiles']}")
        outs.append(moe.moe_grouped_gemm_w4a16(d.x, a["sorted_ids"], wl.k, wq, ws, a["tiles"], a["max_tiles"],
                                               a["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, moe.MOE_OUT_BF16,
                                               weight_layout=layout))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outs[1].view(torch.int16).cpu().numpy(), outs[0].view(torch.int16).cpu().numpy())


@pytest.mark.parametrize("name", ["pre800", "dec1"])
def test_ffn_forward_graph_replays_match_eager(name):
    # The whole layer captured in a HIP graph (no memset or host sync is recorded) and replayed
    # several times, with eager work and synchronisation in between: every replay must reproduce
    # the eager output bits.
    inp, d = workload_inputs(name)
    wl = inp.wl
    q13, s13, q2, s2 = _packed(d)
    ws = torch.empty(moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), dtype=torch.uint8, device="cuda")
    y_ref = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y_ref, workspace=ws,
                        weight_layout=moe.MOE_LAYOUT_PACKED)
    torch.cuda.synchronize()
    ref = _bits(y_ref)
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, workspace=ws,
                            weight_layout=moe.MOE_LAYOUT_PACKED)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_ffn_forward(d.x, d.logits, q13, s13, q2, s2, wl.k, y=y, workspace=ws,
                            weight_layout=moe.MOE_LAYOUT_PACKED)
    for rep in range(3):
        y.fill_(float("nan"))
        ws.fill_(0xFF)  # eager work between replays: poison the workspace the replay must rewrite
        torch.cuda.synchronize()
        _log(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y), ref)
