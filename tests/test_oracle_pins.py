"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term, a wrong sign, a
transposed operand, a swapped nibble, an off-by-one in a scale index, an unstable sort) fails it:
  * the E2M1 table of the published OCP MX element format (golden fixture),
  * exhaustive exactness of dequantisation (fp32 product == fp64 product),
  * hand-worked routing example (golden fixture) and brute-force routing by a full sort,
  * brute-force permutation by Python's sorted(),
  * the whole layer against a dense formulation (all experts on all tokens, a dense [T, E] routing
    matrix with zeros off the top-k) written with numpy matmul in float64,
  * special cases: E = k = 1 is the textbook SwiGLU FFN; unit codes and unit scales give row sums;
    zero input gives zero output.
"""
import math
import os

import numpy as np
import pytest

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)])


TABLE = _e2m1_table()


def _np_dequant(q, s):
    """Independent numpy dequantisation from the golden table (low nibble = even K index)."""
    N, K = q.shape[0], q.shape[1] * 2
    c = np.empty((N, K))
    c[:, 0::2] = TABLE[q & 15]
    c[:, 1::2] = TABLE[q >> 4]
    sc = mi.bf16_bits_to_f32(s).astype(np.float64)
    return c * np.repeat(sc, 32, axis=1)


def test_e2m1_matches_ocp_table():
    for code in range(16):
        v = oracle.e2m1_value(code)
        assert v == TABLE[code], (code, v)
        assert math.copysign(1.0, v) == math.copysign(1.0, TABLE[code])  # code 8 is -0.0
    assert oracle.e2m1_value(2) == 1.0 and oracle.e2m1_value(7) == 6.0 and oracle.e2m1_value(15) == -6.0


def test_bf16_decode_matches_numpy_widening():
    bits = np.arange(0, 65536, 257, dtype=np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_dequant_exhaustive_exact():
    # every finite bf16 scale (one per row) times every code (each code twice per 32-element group)
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    scales = scales[(scales & 0x7F80) != 0x7F80]  # drop Inf/NaN patterns
    sf = mi.bf16_bits_to_f32(scales).astype(np.float64)
    scales = scales[np.abs(sf) * 6.0 < np.finfo(np.float32).max]  # products stay finite in fp32
    codes = np.arange(32) % 16
    q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    qm = np.tile(q, (len(scales), 1))
    got = oracle.dequant(qm, scales[:, None])
    ref = TABLE[codes][None, :] * mi.bf16_bits_to_f32(scales).astype(np.float64)[:, None]
    np.testing.assert_array_equal(got, ref)


def test_dequant_layout_nibble_and_group_index():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, (7, 96 // 2), dtype=np.uint8)
    s = mi.f32_to_bf16_bits(rng.uniform(0.5, 2.0, (7, 96 // 32)).astype(np.float32))
    np.testing.assert_array_equal(oracle.dequant(q, s), _np_dequant(q, s))


def _golden_route():
    with open(os.path.join(GOLDEN, "route_worked_example.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    logits = np.array([float(v) for v in rows[0][1:]], np.float32)[None, :]
    return logits, {int(r[0][1:]): [int(v) for v in r[1:]] for r in rows[1:]}


def test_route_worked_example():
    logits, expect = _golden_route()
    ids, w = oracle.route(logits, 2)
    assert ids[0].tolist() == expect[2]
    np.testing.assert_allclose(w[0], [0.5, 0.5], rtol=0, atol=1e-15)
    ids, w = oracle.route(logits, 3)
    assert ids[0].tolist() == expect[3]
    a = 1.0 / (2.0 + math.exp(-1.0))
    np.testing.assert_allclose(w[0], [a, a, math.exp(-1.0) * a], rtol=1e-14, atol=0)


@pytest.mark.parametrize("T,E,k,skew", [(16, 8, 2, False), (64, 128, 8, False), (200, 512, 10, True)])
def test_route_brute_force_and_invariants(T, E, k, skew):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if skew:
        logits = (logits + mi.skew_bias(E)[None, :]).astype(np.float32)
    logits[0, :4] = 1.25  # plant ties
    ids, w = oracle.route(logits, k)
    for t in range(T):
        full = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p = full / full.sum()
        order = sorted(range(E), key=lambda e: (-p[e], e))[:k]
        assert ids[t].tolist() == order
        assert len(set(ids[t].tolist())) == k
        ref_w = p[order] / p[order].sum()
        np.testing.assert_allclose(w[t], ref_w, rtol=1e-12, atol=1e-15)
        assert abs(w[t].sum() - 1.0) <= 1e-12
        assert np.all(np.diff(w[t]) <= 0)


@pytest.mark.parametrize("T,E,k,bm", [(16, 8, 2, 4), (1, 128, 8, 16), (300, 64, 6, 32), (64, 512, 10, 128)])
def test_align_brute_force(T, E, k, bm):
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    a = oracle.align(ids, E, bm)
    flat = ids.reshape(-1).tolist()
    R = T * k
    order = sorted(range(R), key=lambda f: (flat[f], f))
    assert a["sorted_ids"].tolist() == order
    inv = [0] * R
    for r, f in enumerate(order):
        inv[f] = r
    assert a["inv_perm"].tolist() == inv
    assert a["counts"].tolist() == [flat.count(e) for e in range(E)]
    assert a["offsets"][0] == 0 and a["offsets"][-1] == R
    assert np.all(np.diff(a["offsets"]) == a["counts"])
    tiles = []
    for e in range(E):
        rows = [r for r in range(R) if flat[order[r]] == e]
        for j in range(0, len(rows), bm):
            tiles.append([e, rows[j], len(rows[j:j + bm])])
    assert a["tiles"].tolist() == tiles and a["num_tiles"] == len(tiles)
    assert a["max_m_tiles"] == max(-(-flat.count(e) // bm) for e in range(E))


def _dense_layer(inp):
    """Y = sum_e diag(Rw[:, e]) FFN_e(X): every expert on every token, dense routing matrix."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    L = inp.logits.astype(np.float64)
    P = np.exp(L - L.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    Rw = np.zeros((T, E))
    for t in range(T):
        top = sorted(range(E), key=lambda e: (-inp.logits[t, e], e))[:k]
        Rw[t, top] = P[t, top] / P[t, top].sum()
    Y = np.zeros((T, H))
    for e in range(E):
        W13 = _np_dequant(inp.w13_q[e], inp.w13_s[e])
        W2 = _np_dequant(inp.w2_q[e], inp.w2_s[e])
        G = np.matmul(X, W13.T)
        Hh = G[:, :I] / (1.0 + np.exp(-G[:, :I])) * G[:, I:]
        Y += Rw[:, e:e + 1] * np.matmul(Hh, W2.T)
    return Y


@pytest.mark.parametrize("wl", [mi.WORKLOADS["tiny"], mi.custom("odd", 9, 6, 3, 128, 64, seed=3),
                                mi.custom("skewed", 24, 16, 4, 64, 96, skew=True, seed=4)])
def test_full_layer_vs_dense_brute_force(wl):
    inp = mi.make_inputs(wl)
    y = oracle.moe_ffn(inp)
    ref = _dense_layer(inp)
    scale = np.sqrt((ref ** 2).mean())
    assert np.abs(y - ref).max() <= 1e-12 * scale


def test_token_subset_matches_full():
    inp = mi.make_inputs(mi.WORKLOADS["tiny"])
    y = oracle.moe_ffn(inp)
    sub = np.array([15, 0, 7])
    np.testing.assert_array_equal(oracle.moe_ffn(inp, tokens=sub), y[sub])


def test_single_expert_is_textbook_swiglu():
    inp = mi.make_inputs(mi.custom("one", 5, 1, 1, 64, 32, seed=9))
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    W = _np_dequant(inp.w13_q[0], inp.w13_s[0])
    W1, W3 = W[:32], W[32:]
    W2 = _np_dequant(inp.w2_q[0], inp.w2_s[0])
    a = X @ W1.T
    ref = (a * (1.0 / (1.0 + np.exp(-a))) * (X @ W3.T)) @ W2.T
    y = oracle.moe_ffn(inp)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_unit_codes_give_row_sums():
    # every code 2 (= 1.0), every scale 1.0: each gate/up output is the row sum of x
    wl = mi.custom("ones", 4, 2, 1, 64, 32, seed=2)
    inp = mi.make_inputs(wl)
    inp.w13_q[:] = 0x22
    inp.w13_s[:] = mi.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    y, h, o = oracle.moe_ffn(inp, diagnostics=True)
    g = mi.bf16_bits_to_f32(inp.x).astype(np.float64).sum(1)
    expect_h = g / (1.0 + np.exp(-g)) * g
    np.testing.assert_allclose(h[:, 0, :], np.repeat(expect_h[:, None], 32, 1), rtol=1e-13)


def test_zero_input_gives_zero():
    inp = mi.make_inputs(mi.WORKLOADS["tiny"])
    inp.x[:] = 0
    assert np.all(oracle.moe_ffn(inp) == 0.0)


def test_grouped_proj_and_combine_match_per_expert_numpy():
    inp = mi.make_inputs(mi.WORKLOADS["tiny"])
    wl = inp.wl
    ids, w = oracle.route(inp.logits, wl.k)
    a = oracle.align(ids, wl.E, 8)
    G = oracle.grouped_proj(inp.x, a["sorted_ids"], wl.k, inp.w13_q, inp.w13_s, a["offsets"], silu_mul=True)
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    for r in range(wl.T * wl.k):
        f = a["sorted_ids"][r]
        e = ids.reshape(-1)[f]
        W = _np_dequant(inp.w13_q[e], inp.w13_s[e])
        g = W @ X[f // wl.k]
        np.testing.assert_allclose(G[r], g[:wl.I] / (1 + np.exp(-g[:wl.I])) * g[wl.I:], rtol=1e-12, atol=1e-13)
    # combine: a permuted O gathers back to token order with slot weights
    O = np.random.default_rng(1).standard_normal((wl.T * wl.k, wl.H))
    y = oracle.combine(O, a["inv_perm"], w, wl.T, wl.k)
    ref = np.zeros((wl.T, wl.H))
    for t in range(wl.T):
        for s in range(wl.k):
            ref[t] += w[t, s] * O[a["inv_perm"][t * wl.k + s]]
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)
    # row scale multiplies each permuted row
    rs = np.linspace(0.5, 1.5, wl.T * wl.k)
    G2 = oracle.grouped_proj(inp.x, a["sorted_ids"], wl.k, inp.w13_q, inp.w13_s, a["offsets"], silu_mul=True,
                             row_scale=rs)
    np.testing.assert_allclose(G2, G * rs[:, None], rtol=1e-15, atol=0)


def _golden_combine():
    rows = {}
    with open(os.path.join(GOLDEN, "combine_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


def test_combine_worked_example():
    """Hand-worked scatter-reduce (golden fixture): y[t] = sum_s w[t,s] O[inv_perm[t*k+s]]."""
    g = _golden_combine()
    T, k, H = 2, 2, 3
    ids = np.array(g["ids"], np.int32).reshape(T, k)
    a = oracle.align(ids, 2, 4)
    np.testing.assert_array_equal(a["sorted_ids"], np.array(g["sorted_ids"], np.int32))
    np.testing.assert_array_equal(a["inv_perm"], np.array(g["inv_perm"], np.int32))
    O = np.array(g["O"], np.float64).reshape(T * k, H)
    w = np.array(g["w"], np.float64).reshape(T, k)
    y = oracle.combine(O, a["inv_perm"], w, T, k)
    np.testing.assert_array_equal(y, np.array(g["y"], np.float64).reshape(T, H))


@pytest.mark.parametrize("K,N,bm", [(64, 48, 4), (160, 96, 8), (256, 32, 16)])
def test_grouped_proj_plain_matches_rowwise_numpy(K, N, bm):
    """The plain (no SiLU) projection: identity rows (a_row_of = None) and gathered rows with a
    divisor, each row against its expert's dequantized matrix times the row (numpy, float64)."""
    rng = np.random.default_rng(K + N)
    T, E, k = 23, 5, 2
    logits = rng.standard_normal((T, E), dtype=np.float32)
    logits[:, 1] += 2.0  # uneven expert sizes, one expert with several tiles
    ids, _ = oracle.route(logits, k)
    a = oracle.align(ids, E, bm)
    R = T * k
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    Ws = mi.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    W = [_np_dequant(Wq[e], Ws[e]) for e in range(E)]
    expert_of_row = np.repeat(np.arange(E), a["counts"])
    # identity rows: permuted row r reads A[r]
    A = mi.f32_to_bf16_bits(rng.standard_normal((R, K), dtype=np.float32))
    Af = mi.bf16_bits_to_f32(A).astype(np.float64)
    C = oracle.grouped_proj(A, None, 1, Wq, Ws, a["offsets"])
    assert C.shape == (R, N)
    for r in range(R):
        np.testing.assert_allclose(C[r], W[expert_of_row[r]] @ Af[r], rtol=1e-12, atol=1e-13)
    # gathered rows: permuted row r reads token sorted_ids[r] // k of X [T, K]
    X = mi.f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    Xf = mi.bf16_bits_to_f32(X).astype(np.float64)
    Cg = oracle.grouped_proj(X, a["sorted_ids"], k, Wq, Ws, a["offsets"])
    for r in range(R):
        t = a["sorted_ids"][r] // k
        assert ids[t].tolist()[a["sorted_ids"][r] % k] == expert_of_row[r]
        np.testing.assert_allclose(Cg[r], W[expert_of_row[r]] @ Xf[t], rtol=1e-12, atol=1e-13)


def _bf16_round_f64(v):
    return mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(v.astype(np.float32))).astype(np.float64)


@pytest.mark.parametrize("wl", [mi.WORKLOADS["tiny"], mi.custom("odd", 9, 6, 3, 128, 64, seed=3),
                                mi.custom("skewed", 24, 16, 4, 64, 96, skew=True, seed=4)])
@pytest.mark.parametrize("bm", [4, 16])
def test_chain_of_steps_matches_layer_and_dense(wl, bm):
    """The layer as the GPU runs it, step by step through the oracle: route -> align -> gathered
    gate_up with SiLU*mul -> plain down on identity rows -> combine.  Pinned two ways:
      * gate_up's permuted rows equal the per-token layer's h (its diagnostics) and the dense
        formulation's h (every expert on every token, numpy float64), within 1e-12;
      * with h rounded to bf16 between the projections (the boundary's h is bf16), y equals the
        dense formulation fed the same bf16 h, within 1e-12 * rms, and differs from the fp64-h layer
        by no more than that rounding can move it (2^-8 relative per h element, through |W2| and w)."""
    inp = mi.make_inputs(wl)
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    ids, w = oracle.route(inp.logits, k)
    a = oracle.align(ids, E, bm)
    R = T * k
    Hp = oracle.grouped_proj(inp.x, a["sorted_ids"], k, inp.w13_q, inp.w13_s, a["offsets"], silu_mul=True)
    y_layer, h_diag, _ = oracle.moe_ffn(inp, diagnostics=True)
    f = a["sorted_ids"]
    h_tok = h_diag.reshape(R, I)[f]  # the layer's h of slot f, in permuted order
    hs = np.sqrt((h_tok ** 2).mean())
    assert np.abs(Hp - h_tok).max() <= 1e-12 * hs
    # dense h: every expert on every token
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    flat = ids.reshape(-1)
    for e in range(E):
        G = X @ _np_dequant(inp.w13_q[e], inp.w13_s[e]).T
        Hd = G[:, :I] / (1.0 + np.exp(-G[:, :I])) * G[:, I:]
        rows = np.nonzero(flat[f] == e)[0]
        assert np.abs(Hp[rows] - Hd[f[rows] // k]).max(initial=0.0) <= 1e-12 * hs
    # down on identity rows, then combine
    hb = mi.f32_to_bf16_bits(Hp.astype(np.float32))
    O = oracle.grouped_proj(hb, None, 1, inp.w2_q, inp.w2_s, a["offsets"])
    y = oracle.combine(O, a["inv_perm"], w, T, k)
    # dense down + combine fed the same bf16 h: Y = sum_e diag(Rw[:, e]) (Hb_e W2_e^T)
    Hbf = mi.bf16_bits_to_f32(hb).astype(np.float64)
    L = inp.logits.astype(np.float64)
    P = np.exp(L - L.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    Y = np.zeros((T, H))
    W2abs = []
    for e in range(E):
        Hb_e = np.zeros((T, I))
        rows = np.nonzero(flat[f] == e)[0]
        Hb_e[f[rows] // k] = Hbf[rows]
        W2 = _np_dequant(inp.w2_q[e], inp.w2_s[e])
        W2abs.append(np.abs(W2))
        Rw = np.zeros(T)
        for t in range(T):
            top = sorted(range(E), key=lambda j: (-inp.logits[t, j], j))[:k]
            if e in top:
                Rw[t] = P[t, e] / P[t, top].sum()
        Y += Rw[:, None] * (Hb_e @ W2.T)
    rms = np.sqrt((Y ** 2).mean())
    assert np.abs(y - Y).max() <= 1e-12 * rms
    # against the per-token fp64-h layer: only h's bf16 rounding separates them
    bound = np.zeros((T, H))
    for r in range(R):
        t, s = divmod(int(f[r]), k)
        bound[t] += w[t, s] * (W2abs[flat[f[r]]] @ (2.0 ** -8 * np.abs(Hp[r])))
    assert np.all(np.abs(y - y_layer) <= bound + 1e-12 * rms)
    assert np.abs(y - y_layer).max() > 0  # the rounding is visible, so the bound is not vacuous


def test_page_byte_figures():
    # Atlas page, section "编译时内核选择和W4A16 Grouped GEMM": 1611 MB for BF16 expert weights and
    # 302 MB for W4A16 at the 256-expert shape (hidden 2048, intermediate 512).
    E, H, I = 256, 2048, 512
    assert E * 3 * H * I * 2 == 1_610_612_736
    gate_up_4bit = E * (2 * I * H // 2 + 2 * I * (H // 32) * 2)
    assert gate_up_4bit == 301_989_888
    assert E * mi.weight_bytes_per_expert(H, I) == 452_984_832


# ---------------------------------------------------------------------------------------------------
# router gate and shared expert (the Atlas debug section names gate logits and a shared expert output)

def test_router_logits_one_hot_gate_selects_inputs():
    # a gate whose row e is the unit vector at column 3e reads x[t, 3e] exactly
    T, H, E = 4, 64, 6
    inp = mi.make_inputs(mi.custom("rl", T, E, 2, H, 32, seed=21))
    wr = np.zeros((E, H), np.uint16)
    for e in range(E):
        wr[e, 3 * e] = 0x3F80  # bf16 1.0
    lg = oracle.router_logits(inp.x, wr)
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    np.testing.assert_array_equal(lg, X[:, 0:3 * E:3])


def test_router_logits_match_dense_matmul_and_scale():
    wl = mi.custom("rl2", 7, 33, 4, 96, 32, seed=22)
    inp, blk = mi.make_inputs(wl), mi.make_block_inputs(wl, 32)
    lg = oracle.router_logits(inp.x, blk.w_router)
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    Wr = mi.bf16_bits_to_f32(blk.w_router).astype(np.float64)
    np.testing.assert_allclose(lg, X @ Wr.T, rtol=1e-12, atol=1e-12)
    # doubling every gate weight (exact in bf16) doubles every logit exactly
    w2 = mi.f32_to_bf16_bits(mi.bf16_bits_to_f32(blk.w_router) * 2)
    np.testing.assert_array_equal(oracle.router_logits(inp.x, w2), 2 * lg)
    # the generator's gate gives logits of about unit variance, as the workloads' logits
    big = mi.custom("rl3", 256, 64, 8, 2048, 32, seed=23)
    s = oracle.router_logits(mi.make_inputs(big).x, mi.make_block_inputs(big, 32).w_router).std()
    assert 0.9 < s < 1.1


def test_shared_expert_is_textbook_swiglu_and_a_one_expert_layer():
    wl = mi.custom("sh", 6, 3, 2, 64, 32, seed=24)
    inp, blk = mi.make_inputs(wl), mi.make_block_inputs(wl, 64)
    sh = oracle.shared_ffn(inp.x, blk.w13s_q, blk.w13s_s, blk.w2s_q, blk.w2s_s)
    X = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    W = _np_dequant(blk.w13s_q, blk.w13s_s)
    W1, W3 = W[:64], W[64:]
    W2 = _np_dequant(blk.w2s_q, blk.w2s_s)
    a = X @ W1.T
    ref = (a * (1.0 / (1.0 + np.exp(-a))) * (X @ W3.T)) @ W2.T
    np.testing.assert_allclose(sh, ref, rtol=1e-12, atol=1e-14)
    # the same weights as the only expert of a top-1 routed layer (weight 1) give the same output
    one = mi.MoEInputs(mi.custom("sh1", 6, 1, 1, 64, 64, seed=24), inp.x, np.zeros((6, 1), np.float32),
                       blk.w13s_q[None], blk.w13s_s[None], blk.w2s_q[None], blk.w2s_s[None])
    np.testing.assert_array_equal(oracle.moe_ffn(one), sh)
    np.testing.assert_array_equal(oracle.shared_ffn(inp.x, blk.w13s_q, blk.w13s_s, blk.w2s_q, blk.w2s_s,
                                                    tokens=np.array([4, 1])), sh[[4, 1]])


# ---------------------------------------------------------------------------------------------------
# MXFP4 (W4A4): E8M0 scales, MX quantization, the W4A4 layer

def _golden_mx():
    blocks = []
    with open(os.path.join(GOLDEN, "mx_quant_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals, scale, codes = (part.split() for part in line.split("|"))
            v = np.zeros(32)
            v[:len(vals)] = [float(t) for t in vals]
            c = np.zeros(32, np.int64)
            c[:len(codes)] = [int(t) for t in codes]
            blocks.append((v, int(scale[0]), c))
    return blocks


def _codes_of(q):
    q = np.asarray(q, np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.int64)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def _np_mx_dequant(q, s):
    """Independent numpy dequantisation: golden E2M1 table times 2^(byte - 127)."""
    table = _e2m1_table()
    codes = _codes_of(q)
    scale = np.exp2(np.asarray(s, np.float64) - 127.0)
    return table[codes] * np.repeat(scale, 32, axis=-1)


def test_e8m0_scale_decode():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(119) == 2.0 ** -8
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def test_mx_quantize_golden_blocks():
    for v, scale, codes in _golden_mx():
        q, s = oracle.mx_quantize(v[None])
        assert int(s[0, 0]) == scale, (v[:8], s)
        np.testing.assert_array_equal(_codes_of(q)[0], codes)


def test_e2m1_nearest_matches_grid_search():
    # brute force over the eight codes of v's sign: the smallest distance, ties to an even code,
    # magnitudes at or above 6 saturate
    table = _e2m1_table()
    rng = np.random.default_rng(5)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    vals = np.concatenate([rng.uniform(-8, 8, 4000), mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 9),
                           [0.0, -0.0, 6.0, -6.0, 7.99, 100.0, 1e-300]])
    for v in vals:
        sign = 8 if np.signbit(v) else 0
        cand = [sign | c for c in range(8)]
        if abs(v) >= 6:
            want = sign | 7
        else:
            d = [abs(v - table[c]) for c in cand]
            dmin = min(d)
            ties = [c for c, dc in zip(cand, d) if dc == dmin]
            even = [c for c in ties if c % 2 == 0]
            want = (even or ties)[0]
        assert oracle.e2m1_nearest(float(v)) == want, v


def test_mx_quantize_invariants():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    v[3, 32:64] = 0.0
    q, s = oracle.mx_quantize(v)
    codes = _codes_of(q)
    # powers of two move only the scale byte
    for m in (-3, 1, 7):
        q2, s2 = oracle.mx_quantize(v * 2.0 ** m)
        np.testing.assert_array_equal(q2, q)
        nz = s != 0
        np.testing.assert_array_equal(s2[nz].astype(int), s[nz].astype(int) + m)
    # negation flips every sign bit
    qn, sn = oracle.mx_quantize(-v)
    np.testing.assert_array_equal(_codes_of(qn), codes ^ 8)
    np.testing.assert_array_equal(sn, s)
    # the scaled block maximum lands in [4, 8): its code magnitude is 4 or 6
    X = np.exp2(s.astype(np.float64) - 127)
    blocks = np.abs(v).reshape(64, 4, 32).max(axis=2)
    live = blocks > 0
    assert np.all((blocks[live] / X[live] >= 4) & (blocks[live] / X[live] < 8))
    # every element is within half the local E2M1 spacing of its value (below saturation)
    deq = _np_mx_dequant(q, s)
    scaled = np.abs(v) / np.repeat(X, 32, axis=1)
    spacing = np.where(scaled < 2, 0.5, np.where(scaled < 4, 1.0, 2.0))
    ok = (np.abs(deq - v) <= 0.5 * spacing * np.repeat(X, 32, axis=1) * (1 + 1e-12)) | (scaled >= 6)
    assert np.all(ok)
    # the all-zero block
    assert s[3, 1] == 0 and np.all(codes[3, 32:64] == 0)


def _mx_layer_dense(inp):
    """The W4A4 layer written densely in numpy: every expert on every token, a [T, E] routing matrix
    with the renormalised top-k weights and zeros elsewhere; activations quantized by the oracle's MX
    quantizer, every MX tensor dequantized by the numpy table above."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    ids, w = oracle.route(inp.logits, k)
    route = np.zeros((T, E))
    for t in range(T):
        route[t, ids[t]] = w[t]
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    xq, xs = oracle.mx_quantize(x)
    xd = _np_mx_dequant(xq, xs)
    y = np.zeros((T, H))
    for e in range(E):
        W13 = _np_mx_dequant(inp.w13_q[e], inp.w13_e[e])
        W2 = _np_mx_dequant(inp.w2_q[e], inp.w2_e[e])
        g = xd @ W13.T
        h = g[:, :I] / (1.0 + np.exp(-g[:, :I])) * g[:, I:]
        hq, hs = oracle.mx_quantize(h)
        y += route[:, e:e + 1] * (_np_mx_dequant(hq, hs) @ W2.T)
    return y


@pytest.mark.parametrize("T,E,k,H,I,skew", [(9, 6, 2, 64, 96, False), (5, 4, 4, 128, 64, False),
                                             (12, 8, 3, 96, 64, True)])
def test_mx_layer_matches_dense_formulation(T, E, k, H, I, skew):
    inp = mi.make_mx_inputs(mi.custom("mxdense", T, E, k, H, I, skew=skew, seed=T + E))
    ref = _mx_layer_dense(inp)
    y = oracle.moe_ffn_mx(inp)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_mx_single_expert_is_quantized_swiglu():
    inp = mi.make_mx_inputs(mi.custom("mx1", 7, 1, 1, 64, 64, seed=3))
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    xd = _np_mx_dequant(*oracle.mx_quantize(x))
    W1 = _np_mx_dequant(inp.w13_q[0, :64], inp.w13_e[0, :64])
    W3 = _np_mx_dequant(inp.w13_q[0, 64:], inp.w13_e[0, 64:])
    W2 = _np_mx_dequant(inp.w2_q[0], inp.w2_e[0])
    a, b = xd @ W1.T, xd @ W3.T
    h = a * (1 / (1 + np.exp(-a))) * b
    ref = _np_mx_dequant(*oracle.mx_quantize(h)) @ W2.T
    np.testing.assert_allclose(oracle.moe_ffn_mx(inp), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_grouped_proj_mx_matches_rowwise_products():
    rng = np.random.default_rng(8)
    E, N, K, R = 3, 48, 96, 20
    Aq = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    As = rng.integers(120, 130, (R, K // 32), dtype=np.uint8)
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    We = rng.integers(118, 124, (E, N, K // 32), dtype=np.uint8)
    offsets = np.array([0, 7, 7, R], np.int32)
    a_row_of = rng.permutation(R).astype(np.int32)
    C = oracle.grouped_proj_mx(Aq, As, a_row_of, 1, Wq, We, offsets)
    A = _np_mx_dequant(Aq, As)
    for e in range(E):
        W = _np_mx_dequant(Wq[e], We[e])
        for r in range(offsets[e], offsets[e + 1]):
            np.testing.assert_allclose(C[r], W @ A[a_row_of[r]], rtol=1e-13, atol=1e-300)
    Cs = oracle.grouped_proj_mx(Aq, As, None, 1, Wq, We, offsets, silu_mul=True)
    for e in range(E):
        W = _np_mx_dequant(Wq[e], We[e])
        for r in range(offsets[e], offsets[e + 1]):
            g = W @ A[r]
            np.testing.assert_allclose(Cs[r], g[:N // 2] / (1 + np.exp(-g[:N // 2])) * g[N // 2:], rtol=1e-12,
                                       atol=1e-300)


# ---------------------------------------------------------------------------------------------------
# FP8 (E4M3 codes, per-1x128 fp32 scales)

def _golden_e4m3():
    out = {}
    with open(os.path.join(GOLDEN, "e4m3_ocp_fp8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            out[int(c, 16)] = float(v)
    return out


def _torch_e4m3_table():
    """The 256 E4M3 values decoded by torch's float8_e4m3fn (an independent implementation)."""
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _np_f8_dequant(q, s):
    return _torch_e4m3_table()[np.asarray(q, np.int64)] * np.repeat(np.asarray(s, np.float64), 128, axis=-1)


def test_e4m3_decode_golden_and_library():
    for c, v in _golden_e4m3().items():
        got = oracle.e4m3_value(c)
        if math.isnan(v):
            assert math.isnan(got), c
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), (hex(c), got, v)
    table = _torch_e4m3_table()
    for c in range(256):
        got = oracle.e4m3_value(c)
        assert (math.isnan(got) and math.isnan(table[c])) or got == table[c], hex(c)


def test_e4m3_nearest_matches_library_rounding():
    # torch's float8_e4m3fn cast rounds to nearest, ties to even, for |v| <= 464 (beyond, it gives NaN
    # where the quantizer saturates): every midpoint between adjacent codes, its neighbours and
    # random values across the exponent range
    import torch
    table = _torch_e4m3_table()
    # (values are float32, the precision the quantizer's quotients have; torch narrows wider values
    # to float32 before the cast)
    mags = np.sort(table[:0x7F]).astype(np.float32)
    mids = (mags[1:] + mags[:-1]) / np.float32(2)
    rng = np.random.default_rng(11)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), mags,
                           (rng.uniform(-1, 1, 3000) * np.exp2(rng.integers(-12, 9, 3000))).astype(np.float32),
                           np.array([464.0, 2.0 ** -10], np.float32)])
    vals = np.concatenate([vals, -vals])
    vals = vals[np.abs(vals) <= 464]
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_nearest(float(v)) for v in vals])
    np.testing.assert_array_equal(got, want)
    # saturation (closed form): anything beyond 448 maps to +-448
    for v in (465.0, 1e6, 1e300):
        assert oracle.e4m3_nearest(v) == 0x7E and oracle.e4m3_nearest(-v) == 0xFE


def _golden_f8():
    out = []
    with open(os.path.join(GOLDEN, "f8_quant_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            vals, sbits, codes = line.split("|")
            v = np.zeros(128)
            vv = [float(t) for t in vals.split()]
            v[:len(vv)] = vv
            c = np.zeros(128, np.uint8)
            cc = [int(t, 16) for t in codes.split()]
            c[:len(cc)] = cc
            out.append((v, int(sbits.strip(), 16), c))
    return out


def test_f8_quantize_golden_blocks():
    for v, sbits, codes in _golden_f8():
        q, s = oracle.f8_quantize(v[None])
        assert int(s.view(np.uint32)[0, 0]) == sbits, (v[:4], hex(int(s.view(np.uint32)[0, 0])))
        np.testing.assert_array_equal(q[0], codes)


def test_f8_quantize_invariants():
    rng = np.random.default_rng(12)
    v = (rng.standard_normal((48, 512)) * np.exp2(rng.integers(-20, 20, (48, 1)))).astype(np.float32).astype(np.float64)
    v[5, 128:256] = 0.0
    q, s = oracle.f8_quantize(v)
    # a power of two moves only the scale
    for m in (-4, 3):
        q2, s2 = oracle.f8_quantize(v * 2.0 ** m)
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, (s * np.float32(2.0 ** m)).astype(np.float32))
    # negation flips every sign bit of a non-zero block
    qn, sn = oracle.f8_quantize(-v)
    live = np.repeat(s > 0, 128, axis=1)
    np.testing.assert_array_equal(qn[live], q[live] ^ 0x80)
    np.testing.assert_array_equal(sn, s)
    # the block maximum maps to +-448; every element within half the local E4M3 spacing (relative
    # 2^-4 of a normal value, 2^-10 absolute below 2^-6) times s, up to the two fp32 roundings
    blk = np.abs(v).reshape(48, 4, 128)
    arg = blk.argmax(axis=2)
    qb = q.reshape(48, 4, 128)
    for r in range(48):
        for b in range(4):
            if s[r, b] > 0:
                assert qb[r, b, arg[r, b]] & 0x7F == 0x7E
    deq = _np_f8_dequant(q, s)
    S = np.repeat(s.astype(np.float64), 128, axis=1)
    scaled = np.abs(v) / np.where(S > 0, S, 1)
    half = np.where(scaled >= 2.0 ** -6, scaled * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(deq - v) <= (half * (1 + 1e-6) + scaled * 2e-7) * S)
    assert s[5, 1] == 0 and np.all(q[5, 128:256] == 0)


def _f8_layer_dense(inp):
    """The W8A8 layer written densely in numpy: every expert on every token, a [T, E] routing matrix
    with the renormalised top-k weights and zeros elsewhere; activations quantized by the oracle's FP8
    quantizer, every FP8 tensor dequantized through torch's E4M3 decode."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    ids, w = oracle.route(inp.logits, k)
    route = np.zeros((T, E))
    for t in range(T):
        route[t, ids[t]] = w[t]
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    xd = _np_f8_dequant(*oracle.f8_quantize(x))
    y = np.zeros((T, H))
    for e in range(E):
        W13 = _np_f8_dequant(inp.w13_q[e], inp.w13_s[e])
        W2 = _np_f8_dequant(inp.w2_q[e], inp.w2_s[e])
        g = xd @ W13.T
        h = g[:, :I] / (1.0 + np.exp(-g[:, :I])) * g[:, I:]
        y += route[:, e:e + 1] * (_np_f8_dequant(*oracle.f8_quantize(h)) @ W2.T)
    return y


@pytest.mark.parametrize("T,E,k,H,I,skew", [(9, 6, 2, 128, 256, False), (5, 4, 4, 256, 128, False),
                                             (12, 8, 3, 128, 128, True)])
def test_f8_layer_matches_dense_formulation(T, E, k, H, I, skew):
    inp = mi.make_f8_inputs(mi.custom("f8dense", T, E, k, H, I, skew=skew, seed=T + E))
    ref = _f8_layer_dense(inp)
    y = oracle.moe_ffn_f8(inp)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_f8_single_expert_is_quantized_swiglu():
    inp = mi.make_f8_inputs(mi.custom("f81", 7, 1, 1, 128, 128, seed=3))
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    xd = _np_f8_dequant(*oracle.f8_quantize(x))
    W1 = _np_f8_dequant(inp.w13_q[0, :128], inp.w13_s[0, :128])
    W3 = _np_f8_dequant(inp.w13_q[0, 128:], inp.w13_s[0, 128:])
    W2 = _np_f8_dequant(inp.w2_q[0], inp.w2_s[0])
    a, b = xd @ W1.T, xd @ W3.T
    h = a * (1 / (1 + np.exp(-a))) * b
    ref = _np_f8_dequant(*oracle.f8_quantize(h)) @ W2.T
    np.testing.assert_allclose(oracle.moe_ffn_f8(inp), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_grouped_proj_f8_matches_rowwise_products():
    rng = np.random.default_rng(9)
    E, N, K, R = 3, 48, 256, 20
    Aq = mi.e4m3_codes(rng, (R, K))
    As = rng.uniform(0.5, 2.0, (R, K // 128)).astype(np.float32)
    Wq = mi.e4m3_codes(rng, (E, N, K))
    Ws = rng.uniform(1e-6, 1e-5, (E, N, K // 128)).astype(np.float32)
    offsets = np.array([0, 7, 7, R], np.int32)
    a_row_of = rng.permutation(R).astype(np.int32)
    C = oracle.grouped_proj_f8(Aq, As, a_row_of, 1, Wq, Ws, offsets)
    A = _np_f8_dequant(Aq, As)
    # fp64 sums in another order: within K * 2^-53 of the sum of |terms|
    for e in range(E):
        W = _np_f8_dequant(Wq[e], Ws[e])
        for r in range(offsets[e], offsets[e + 1]):
            a = A[a_row_of[r]]
            assert np.all(np.abs(C[r] - W @ a) <= 1e-13 * (np.abs(W) @ np.abs(a)))
    Cs = oracle.grouped_proj_f8(Aq, As, None, 1, Wq, Ws, offsets, silu_mul=True)
    for e in range(E):
        W = _np_f8_dequant(Wq[e], Ws[e])
        for r in range(offsets[e], offsets[e + 1]):
            g = W @ A[r]
            ga = np.abs(W) @ np.abs(A[r])
            want = g[:N // 2] / (1 + np.exp(-g[:N // 2])) * g[N // 2:]
            slack = 1e-12 * (np.abs(want) + ga[:N // 2] * np.abs(g[N // 2:]) + np.abs(g[:N // 2]) * ga[N // 2:])
            assert np.all(np.abs(Cs[r] - want) <= slack)


# ---------------------------------------------------------------------------------------------------
# W4A8: MXFP8 activation quantization (E4M3 elements, E8M0 per 32) and the W4A8 layer

def _golden_mx8():
    blocks = []
    with open(os.path.join(GOLDEN, "mx8_quant_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals, scale, codes = (part.split() for part in line.split("|"))
            v = np.zeros(32)
            v[:len(vals)] = [float(t) for t in vals]
            c = np.zeros(32, np.int64)
            c[:len(codes)] = [int(t) for t in codes]
            blocks.append((v, int(scale[0]), c))
    return blocks


def _np_mx8_dequant(q, s):
    """Independent dequantisation: torch's E4M3 decode times 2^(byte - 127)."""
    table = _torch_e4m3_table()
    scale = np.exp2(np.asarray(s, np.float64) - 127.0)
    return table[np.asarray(q, np.int64)] * np.repeat(scale, 32, axis=-1)


def test_mx8_quantize_golden_blocks():
    for v, scale, codes in _golden_mx8():
        q, s = oracle.mx8_quantize(v[None])
        assert int(s[0, 0]) == scale, (v[:8], s)
        np.testing.assert_array_equal(q[0].astype(np.int64), codes)


def test_mx8_quantize_invariants():
    rng = np.random.default_rng(31)
    v = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    v[5, 64:96] = 0.0
    q, s = oracle.mx8_quantize(v)
    # powers of two move only the scale byte
    for m in (-4, 1, 9):
        q2, s2 = oracle.mx8_quantize(v * 2.0 ** m)
        np.testing.assert_array_equal(q2, q)
        nz = s != 0
        np.testing.assert_array_equal(s2[nz].astype(int), s[nz].astype(int) + m)
    # negation flips every sign bit
    qn, sn = oracle.mx8_quantize(-v)
    np.testing.assert_array_equal(qn, q ^ 0x80)
    np.testing.assert_array_equal(sn, s)
    # the scaled block maximum lies in [256, 512): its code is one of 256 .. 448 (codes 120 .. 126)
    X = np.exp2(s.astype(np.float64) - 127)
    blocks = np.abs(v).reshape(64, 4, 32)
    bmax = blocks.max(axis=2)
    live = bmax > 0
    assert np.all((bmax[live] / X[live] >= 256) & (bmax[live] / X[live] < 512))
    arg = blocks.argmax(axis=2)
    qmax = np.take_along_axis(q.reshape(64, 4, 32), arg[..., None], axis=2)[..., 0] & 0x7F
    assert np.all((qmax[live] >= 120) & (qmax[live] <= 126))
    # every element is within half the local E4M3 spacing of its value, or saturated at 448
    deq = _np_mx8_dequant(q, s)
    Xr = np.repeat(X, 32, axis=1)
    scaled = np.abs(v) / Xr
    spacing = np.where(scaled < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(scaled, 2.0 ** -6))) - 3))
    ok = (np.abs(deq - v) <= 0.5 * spacing * Xr * (1 + 1e-12)) | ((scaled > 448) & (np.abs(deq) == 448 * Xr))
    assert np.all(ok)
    # the all-zero block
    assert s[5, 2] == 0 and np.all(q[5, 64:96] == 0)


def _w4a8_layer_dense(inp):
    """The W4A8 layer written densely in numpy: every expert on every token, a [T, E] routing matrix
    with the renormalised top-k weights and zeros elsewhere; activations quantized by the oracle's MXFP8
    quantizer and decoded with torch's E4M3 table, weights decoded with the numpy E2M1 table."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    ids, w = oracle.route(inp.logits, k)
    route = np.zeros((T, E))
    for t in range(T):
        route[t, ids[t]] = w[t]
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    xd = _np_mx8_dequant(*oracle.mx8_quantize(x))
    y = np.zeros((T, H))
    for e in range(E):
        W13 = _np_mx_dequant(inp.w13_q[e], inp.w13_e[e])
        W2 = _np_mx_dequant(inp.w2_q[e], inp.w2_e[e])
        g = xd @ W13.T
        h = g[:, :I] / (1.0 + np.exp(-g[:, :I])) * g[:, I:]
        y += route[:, e:e + 1] * (_np_mx8_dequant(*oracle.mx8_quantize(h)) @ W2.T)
    return y


@pytest.mark.parametrize("T,E,k,H,I,skew", [(9, 6, 2, 64, 96, False), (5, 4, 4, 128, 64, False),
                                             (12, 8, 3, 96, 64, True)])
def test_w4a8_layer_matches_dense_formulation(T, E, k, H, I, skew):
    inp = mi.make_mx_inputs(mi.custom("w4a8dense", T, E, k, H, I, skew=skew, seed=T + E + 1))
    ref = _w4a8_layer_dense(inp)
    y = oracle.moe_ffn_w4a8(inp)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_w4a8_single_expert_is_quantized_swiglu():
    inp = mi.make_mx_inputs(mi.custom("w4a8one", 7, 1, 1, 64, 64, seed=33))
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    xd = _np_mx8_dequant(*oracle.mx8_quantize(x))
    W1 = _np_mx_dequant(inp.w13_q[0, :64], inp.w13_e[0, :64])
    W3 = _np_mx_dequant(inp.w13_q[0, 64:], inp.w13_e[0, 64:])
    W2 = _np_mx_dequant(inp.w2_q[0], inp.w2_e[0])
    a, b = xd @ W1.T, xd @ W3.T
    h = a * (1 / (1 + np.exp(-a))) * b
    ref = _np_mx8_dequant(*oracle.mx8_quantize(h)) @ W2.T
    np.testing.assert_allclose(oracle.moe_ffn_w4a8(inp), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_w4a8_activations_differ_from_w4a4_only_by_the_element_format():
    # same weights and routing: the W4A8 layer is closer to the unquantized-activation layer than
    # the W4A4 one (E4M3 keeps 3 mantissa bits, E2M1 one)
    inp = mi.make_mx_inputs(mi.custom("w4a8cmp", 12, 8, 2, 128, 64, seed=34))
    x = mi.bf16_bits_to_f32(inp.x).astype(np.float64)
    ids, w = oracle.route(inp.logits, 2)
    exact = np.zeros((12, 128))
    for t in range(12):
        for s_ in range(2):
            e = ids[t, s_]
            g = _np_mx_dequant(inp.w13_q[e], inp.w13_e[e]) @ x[t]
            h = g[:64] / (1 + np.exp(-g[:64])) * g[64:]
            exact[t] += w[t, s_] * (_np_mx_dequant(inp.w2_q[e], inp.w2_e[e]) @ h)
    err8 = np.linalg.norm(oracle.moe_ffn_w4a8(inp) - exact)
    err4 = np.linalg.norm(oracle.moe_ffn_mx(inp) - exact)
    assert err8 < 0.25 * err4


def test_grouped_proj_w4a8_matches_rowwise_products():
    rng = np.random.default_rng(35)
    E, N, K, R = 3, 48, 96, 20
    Aq = rng.integers(0, 256, (R, K), dtype=np.uint8)
    Aq[(Aq & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    As = rng.integers(108, 114, (R, K // 32), dtype=np.uint8)  # E4M3 magnitudes up to 448: keep silu finite
    Wq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    We = rng.integers(118, 124, (E, N, K // 32), dtype=np.uint8)
    offsets = np.array([0, 7, 7, R], np.int32)
    a_row_of = rng.permutation(R).astype(np.int32)
    C = oracle.grouped_proj_w4a8(Aq, As, a_row_of, 1, Wq, We, offsets)
    A = _np_mx8_dequant(Aq, As)
    for e in range(E):
        W = _np_mx_dequant(Wq[e], We[e])
        for r in range(offsets[e], offsets[e + 1]):
            terms = np.abs(W) @ np.abs(A[a_row_of[r]])
            assert np.all(np.abs(C[r] - W @ A[a_row_of[r]]) <= 1e-13 * terms + 1e-300)
    Cs = oracle.grouped_proj_w4a8(Aq, As, None, 1, Wq, We, offsets, silu_mul=True)
    for e in range(E):
        W = _np_mx_dequant(Wq[e], We[e])
        for r in range(offsets[e], offsets[e + 1]):
            g = W @ A[r]
            np.testing.assert_allclose(Cs[r], g[:N // 2] / (1 + np.exp(-g[:N // 2])) * g[N // 2:], rtol=1e-10,
                                       atol=1e-9 * np.abs(g).max())
