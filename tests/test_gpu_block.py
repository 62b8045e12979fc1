"""GPU parity of the steps either side of the routed layer: the router gate GEMM, the shared expert
(a dense W4A16 SwiGLU on the same grouped-GEMM kernels) and the whole MoE block built from them.

Gate logits are fp32 MFMA sums of exact bf16 products; they are checked against the fp64 oracle
within the rounding bound of that summation.  Routing is then checked bit-exact against the oracle's
routing of the GPU's own logits (a near-tie may order differently between fp32 and fp64 sums, and
the routing contract is defined on the fp32 logits).  Layer outputs use the layer tolerance:
max|gpu-ref| <= 3e-2 * rms(ref) and mean relative error <= 5e-3.
"""
import dataclasses

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


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _logit_bound(x_bits, wr_bits):
    # fp32 MFMA accumulation of H exact products: at most (64 + H/32) roundings of 2^-24 relative to
    # the running sum of |terms| along any summation order.
    H = x_bits.shape[1]
    ref_abs = oracle.router_logits(x_bits & 0x7FFF, wr_bits & 0x7FFF)
    return (64 + H / 32) * 2.0 ** -24 * ref_abs + 1e-30


def _sample(T, n, seed=99):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(8, T - 1), n - 9, replace=False)
    return np.sort(np.concatenate([np.arange(8), rest, [T - 1]]))


class BlockDevice:
    def __init__(self, wl, Is):
        self.inp = mi.make_inputs(wl)
        self.blk = mi.make_block_inputs(wl, Is) if Is else mi.make_block_inputs(wl, 32)
        self.Is = Is
        d = gu.DeviceInputs(self.inp)
        self.d = d
        self.w_router = gu.dev_bf16(self.blk.w_router)
        if Is:
            self.shared = (gu.dev(self.blk.w13s_q), gu.dev(self.blk.w13s_s.view(np.int16)),
                           gu.dev(self.blk.w2s_q), gu.dev(self.blk.w2s_s.view(np.int16)))
        else:
            self.shared = None

    def packed(self):
        q13, s13 = moe.moe_w4_prepack(self.d.w13_q, self.d.w13_s)
        q2, s2 = moe.moe_w4_prepack(self.d.w2_q, self.d.w2_s)
        sh = None
        if self.shared:
            a, b, c, e = self.shared
            pa, pb = moe.moe_w4_prepack(a[None], b[None])
            pc, pe = moe.moe_w4_prepack(c[None], e[None])
            sh = (pa[0], pb[0], pc[0], pe[0])
        return (q13, s13, q2, s2), sh

    def run(self, layout=moe.MOE_LAYOUT_CANONICAL):
        wl = self.inp.wl
        if layout == moe.MOE_LAYOUT_PACKED:
            (q13, s13, q2, s2), sh = self.packed()
        else:
            q13, s13, q2, s2, sh = self.d.w13_q, self.d.w13_s, self.d.w2_q, self.d.w2_s, self.shared
        y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        lg = torch.full((wl.T, wl.E), float("nan"), dtype=torch.float32, device="cuda")
        ids = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
        Is = self.Is
        ws = torch.full((max(moe.moe_ffn_block_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k, Is), 256),), 0xFF,
                        dtype=torch.uint8, device="cuda")
        moe.moe_ffn_block_forward(self.d.x, self.w_router, q13, s13, q2, s2, wl.k, shared=sh, y=y, logits_out=lg,
                                  topk_ids_out=ids, workspace=ws, weight_layout=layout)
        torch.cuda.synchronize()
        return y, lg, ids


# ---------------------------------------------------------------------------------------------------
# router gate

@pytest.mark.parametrize("name,nsample", [("tiny", 16), ("dec1", 1), ("dec64", 64), ("pre800", 64),
                                          ("skew8192", 40)])
def test_router_logits_matches_oracle(name, nsample):
    wl = mi.WORKLOADS[name]
    inp = mi.make_inputs(wl)
    blk = mi.make_block_inputs(wl, 32)
    lg = moe.moe_router_logits(gu.dev_bf16(inp.x), gu.dev_bf16(blk.w_router))
    torch.cuda.synchronize()
    tok = _sample(wl.T, nsample)
    got = lg.cpu().numpy().astype(np.float64)[tok]
    ref = oracle.router_logits(inp.x[tok], blk.w_router)
    assert np.all(np.abs(got - ref) <= _logit_bound(inp.x[tok], blk.w_router)), name


# decode sizes and H % 64 != 0 take the direct-fragment kernel; larger ones the LDS-staged kernel
# with 32 x 32 tiles and K split 4 ways (H = 192: one group gets no K stage), 64 x 64 tiles (H = 128:
# fewer K stages than the ring) or 128 x 64 tiles
@pytest.mark.parametrize("T,E,H", [(1, 1, 32), (37, 65, 96), (33, 1024, 64), (100, 200, 160), (31, 63, 2048),
                                   (1000, 300, 96), (1000, 300, 192), (2051, 129, 256), (4100, 520, 128),
                                   (4100, 1000, 128)])
def test_router_logits_ragged_shapes(T, E, H):
    rng = np.random.default_rng(T + E + H)
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    wr = mi.f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32))
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(gu.dev_bf16(x), gu.dev_bf16(wr), logits=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.router_logits(x, wr)
    assert np.all(np.abs(got - ref) <= _logit_bound(x, wr))


# ---------------------------------------------------------------------------------------------------
# shared expert (dense FFN)

DENSE_CASES = [(1, 256, 128, 0), (5, 256, 128, 1), (16, 160, 96, 0), (37, 160, 96, 0), (40, 256, 128, 1),
               (300, 256, 256, 0), (300, 256, 256, 1), (800, 2048, 512, 1)]


@pytest.mark.parametrize("T,H,Is,layout", DENSE_CASES)
def test_dense_ffn_matches_oracle(T, H, Is, layout):
    wl = mi.custom("dense", T, 4, 1, H, 64, seed=T + Is)
    inp = mi.make_inputs(wl)
    blk = mi.make_block_inputs(wl, Is)
    x = gu.dev_bf16(inp.x)
    w = [gu.dev(blk.w13s_q), gu.dev(blk.w13s_s.view(np.int16)), gu.dev(blk.w2s_q), gu.dev(blk.w2s_s.view(np.int16))]
    if layout == moe.MOE_LAYOUT_PACKED:
        a, b = moe.moe_w4_prepack(w[0][None], w[1][None])
        c, e = moe.moe_w4_prepack(w[2][None], w[3][None])
        w = [a[0], b[0], c[0], e[0]]
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((max(moe.moe_dense_ffn_workspace_bytes(T, H, Is), 256),), 0xFF, dtype=torch.uint8, device="cuda")
    moe.moe_dense_ffn_w4a16(x, *w, out=out, workspace=ws, weight_layout=layout)
    torch.cuda.synchronize()
    tok = _sample(T, 48)
    got = out.cpu().numpy().astype(np.float64)[tok]
    ref = oracle.shared_ffn(inp.x, blk.w13s_q, blk.w13s_s, blk.w2s_q, blk.w2s_s, tokens=tok)
    gu.assert_within_tolerance(got, ref, f"dense T={T} H={H} Is={Is} layout={layout}")


@pytest.mark.parametrize("T", [7, 300])
def test_dense_ffn_packed_matches_canonical_bits(T):
    H, Is = 256, 256
    wl = mi.custom("dense", T, 4, 1, H, 64, seed=21)
    inp = mi.make_inputs(wl)
    blk = mi.make_block_inputs(wl, Is)
    x = gu.dev_bf16(inp.x)
    w = [gu.dev(blk.w13s_q), gu.dev(blk.w13s_s.view(np.int16)), gu.dev(blk.w2s_q), gu.dev(blk.w2s_s.view(np.int16))]
    a, b = moe.moe_w4_prepack(w[0][None], w[1][None])
    c, e = moe.moe_w4_prepack(w[2][None], w[3][None])
    y0 = moe.moe_dense_ffn_w4a16(x, *w)
    y1 = moe.moe_dense_ffn_w4a16(x, a[0], b[0], c[0], e[0], weight_layout=moe.MOE_LAYOUT_PACKED)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y0.view(torch.int32).cpu().numpy(), y1.view(torch.int32).cpu().numpy())


def test_combine_adds_shared_term():
    T, k, H = 29, 3, 136
    rng = np.random.default_rng(4)
    O = rng.standard_normal((T * k, H)).astype(np.float32)
    S = rng.standard_normal((T, H)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    y = moe.moe_combine(gu.dev(O), gu.dev(inv), gu.dev(w), shared=gu.dev(S))
    torch.cuda.synchronize()
    ref = oracle.combine(O.astype(np.float64), inv, w.astype(np.float64), T, k) + S.astype(np.float64)
    got = gu.host_bf16_to_f64(y)
    # fp32 sums of at most k + 1 terms, then one bf16 rounding
    terms = oracle.combine(np.abs(O).astype(np.float64), inv, w.astype(np.float64), T, k) + np.abs(S)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + (k + 2) * 2.0 ** -23 * terms)


# ---------------------------------------------------------------------------------------------------
# the whole block

# Is == I: the shared expert runs inside the routed grouped GEMMs (its tiles after the routed ones);
# other sizes run it as a dense FFN before the routed layer; Is == 0: no shared expert.
BLOCK_CASES = [("tiny", 128, 16), ("dec1", 768, 1), ("dec8", 768, 8), ("dec64", 768, 24), ("pre800", 512, 40),
               ("skew8192", 512, 24), ("tiny", 256, 16), ("dec8", 256, 8), ("pre800", 1024, 24), ("tiny", 0, 16),
               ("pre800", 0, 24)]


@pytest.mark.parametrize("name,Is,nsample", BLOCK_CASES)
def test_block_forward_matches_oracle(name, Is, nsample):
    wl = mi.WORKLOADS[name]
    _log(f"block {name}: T={wl.T} E={wl.E} k={wl.k} H={wl.H} I={wl.I} Is={Is}")
    b = BlockDevice(wl, Is)
    y, lg, ids = b.run()
    tok = _sample(wl.T, nsample)
    glog = lg.cpu().numpy()
    assert np.all(np.abs(glog[tok].astype(np.float64) - oracle.router_logits(b.inp.x[tok], b.blk.w_router))
                  <= _logit_bound(b.inp.x[tok], b.blk.w_router))
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.route(glog, wl.k)[0])
    ref = oracle.moe_ffn(dataclasses.replace(b.inp, logits=glog), tokens=tok)
    if Is:
        ref = ref + oracle.shared_ffn(b.inp.x, b.blk.w13s_q, b.blk.w13s_s, b.blk.w2s_q, b.blk.w2s_s, tokens=tok)
    yh = gu.host_bf16_to_f64(y)
    assert np.all(np.isfinite(yh)), "output not fully written"
    r = gu.assert_within_tolerance(yh[tok], ref, name)
    _log(f"  {name} Is={Is}: {r}")
    if not Is:
        # without a shared expert the block is the routed layer on the gate logits, bit for bit
        y2 = moe.moe_ffn_forward(b.d.x, lg, b.d.w13_q, b.d.w13_s, b.d.w2_q, b.d.w2_s, wl.k)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y2), _bits(y))


@pytest.mark.parametrize("name,Is", [("dec8", 768), ("pre800", 512), ("pre800", 256)])
def test_block_forward_packed_matches_canonical_bits(name, Is):
    b = BlockDevice(mi.WORKLOADS[name], Is)
    y0, lg0, _ = b.run()
    y1, lg1, _ = b.run(moe.MOE_LAYOUT_PACKED)
    np.testing.assert_array_equal(_bits(lg0), _bits(lg1))
    np.testing.assert_array_equal(_bits(y0), _bits(y1))


def test_block_forward_graph_replays_match_eager():
    wl = mi.WORKLOADS["pre800"]
    b = BlockDevice(wl, 512)
    ref = _bits(b.run()[0])
    ws = torch.empty(moe.moe_ffn_block_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k, 512), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    d = b.d
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_ffn_block_forward(d.x, b.w_router, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k, shared=b.shared, y=y,
                                  workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_ffn_block_forward(d.x, b.w_router, d.w13_q, d.w13_s, d.w2_q, d.w2_s, wl.k, shared=b.shared, y=y,
                                  workspace=ws)
    for rep in range(3):
        y.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        _log(f"block graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y), ref)
