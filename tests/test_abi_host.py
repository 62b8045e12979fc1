"""Host-side tests of the C-ABI library: it loads, exports every function the public header declares,
and rejects invalid arguments before anything is launched (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import moe_w4a16_grouped_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z0-9_]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return moe.load()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("moe_align", "moe_grouped_gemm_w4a16", "moe_ffn_forward", "moe_route_topk", "moe_combine"):
        assert required in names
    assert set(names) == set(moe.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 2
    assert lib.moe_status_string(0) == b"MOE_OK"
    for code, name in [(-1, b"MOE_ERR_INVALID_ARG"), (-2, b"MOE_ERR_UNSUPPORTED_SHAPE"), (-3, b"MOE_ERR_MISALIGNED"),
                       (-4, b"MOE_ERR_WORKSPACE"), (-5, b"MOE_ERR_HIP")]:
        assert lib.moe_status_string(code) == name


def test_pure_size_queries(lib):
    # floor(R / block_m) + min(E, R)
    assert moe.moe_max_tiles(800, 8, 256, 32) == 6400 // 32 + 256
    assert moe.moe_max_tiles(1, 8, 128, 16) == 0 + 8
    assert moe.moe_max_tiles(0, 8, 128, 16) == 0
    assert moe.moe_max_tiles(-1, 8, 128, 16) == -1
    assert moe.moe_align_workspace_bytes(64, 8, 128) == 0          # one workgroup
    assert moe.moe_align_workspace_bytes(8192, 10, 512) == 20 * 4 * 512 * 4
    ws = moe.moe_ffn_workspace_bytes(800, 2048, 512, 256, 8)
    R = 800 * 8
    assert ws >= R * 512 * 2 + R * 2048 * 2 + R * 2048 // 8 * 4  # h (bf16), the down output (fp16), its side values
    assert moe.moe_ffn_workspace_bytes(4, 2048, 512, 8, 9) == 0    # k > E


def test_block_m_choice():
    P, C = moe.MOE_LAYOUT_PACKED, moe.MOE_LAYOUT_CANONICAL
    assert moe.moe_ffn_block_m(1, 128, 8, P) == 16        # decode: 8 rows over 128 experts
    assert moe.moe_ffn_block_m(800, 256, 8, P) == 32      # 25 rows per expert
    assert moe.moe_ffn_block_m(8192, 512, 10, P) == 64    # 160 rows per expert
    assert moe.moe_ffn_block_m(4096, 8, 2, P) == 128      # 1024 rows per expert: large-tile kernel
    assert moe.moe_ffn_block_m(4096, 8, 2, C) == 64       # ... which needs packed weights
    assert moe.moe_ffn_block_m(4096, 8, 2, 7) == -1
    assert moe.moe_ffn_block_m(4, 8, 9, P) == -1
    # one workspace size serves both layouts: the tile list is sized for the smaller tile height
    R, E = 4096 * 2, 8
    ws = moe.moe_ffn_workspace_bytes(4096, 4096, 14336, E, 2)
    assert ws >= R * 14336 * 2 + R * 4096 * 2 + R * 4096 // 8 * 4 + moe.moe_max_tiles(4096, 2, E, 64) * 12


FAKE = 1 << 20  # an aligned, never-dereferenced pointer value: validation fails before any launch


def _ptr(v):
    return ctypes.c_void_p(v)


@pytest.mark.parametrize("T,E,k,expect", [(4, 8, 9, -1), (-1, 8, 2, -1), (4, 0, 1, -1), (4, 2000, 2, -2),
                                          (1 << 24, 8, 8, -2)])
def test_route_rejects_bad_shapes(lib, T, E, k, expect):
    st = lib.moe_route_topk(_ptr(FAKE), T, E, k, _ptr(FAKE), _ptr(FAKE), None)
    assert st == expect
    assert lib.moe_last_error()


def test_route_zero_tokens_is_a_noop(lib):
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == 0


def test_route_null_and_misaligned(lib):
    assert lib.moe_route_topk(None, 4, 8, 2, _ptr(FAKE), _ptr(FAKE), None) == -1
    assert lib.moe_route_topk(_ptr(FAKE + 2), 4, 8, 2, _ptr(FAKE), _ptr(FAKE), None) == -3


def test_align_rejects(lib):
    f = _ptr(FAKE)
    # too few tiles
    mt = moe.moe_max_tiles(16, 2, 8, 16)
    st = lib.moe_align(f, 16, 2, 8, 16, f, f, f, f, f, mt - 1, f, None, 0, None)
    assert st == -4 and b"max_tiles" in lib.moe_last_error()
    # multi-workgroup sizes need a workspace
    mt = moe.moe_max_tiles(8192, 10, 512, 128)
    st = lib.moe_align(f, 8192, 10, 512, 128, f, f, f, f, f, mt, f, None, 0, None)
    assert st == -4
    assert lib.moe_align(f, 16, 2, 8, 0, f, f, f, f, f, 100, f, None, 0, None) == -1
    assert lib.moe_align(f, 16, 2, 8, 16, f, f, f, f, None, 100, f, None, 0, None) == -1
    assert lib.moe_align(_ptr(FAKE + 1), 16, 2, 8, 16, f, f, f, f, f, 100, f, None, 0, None) == -3


def test_grouped_gemm_rejects(lib):
    f = _ptr(FAKE)
    args = dict(A=f, aro=None, div=1, Wq=f, Ws=f, lay=0, E=8, N=256, K=256, tiles=f, mt=10, nt=f, bm=16, epi=0, C=f,
                out=0)

    def call(**kw):
        a = dict(args, **kw)
        return lib.moe_grouped_gemm_w4a16(a["A"], a["aro"], a["div"], a["Wq"], a["Ws"], a["lay"], a["E"], a["N"],
                                          a["K"], a["tiles"], a["mt"], a["nt"], a["bm"], a["epi"], a["C"], a["out"],
                                          a.get("cexp"), None)

    assert call(K=48) == -2            # K not a multiple of 32
    assert call(bm=24) == -2           # unsupported tile height
    assert call(epi=7) == -1
    assert call(epi=1, out=1) == -1    # SiLU*mul writes bf16 only
    assert call(epi=1, N=255) == -1    # odd N cannot pair gate and up
    assert call(A=_ptr(FAKE + 8)) == -3
    assert call(C=None) == -1
    assert call(E=0) == -1
    assert call(mt=0) == 0             # nothing to do: no launch
    assert call(lay=2) == -1           # unknown layout
    assert call(lay=1, K=96) == -2     # packed needs K % 128 == 0
    assert call(lay=1, N=200) == -2    # packed needs N % 16 == 0
    assert call(lay=1, N=80, epi=1) == -2  # packed SiLU*mul needs N % 32 == 0 (up rows start a block)
    assert call(lay=1, Ws=_ptr(FAKE + 2)) == -3  # packed scales need 8-byte alignment
    assert call(out=3) == -1                     # fp16 with in-band exponents needs its side array
    assert call(out=3, epi=1, cexp=f) == -1      # ... and the plain epilogue
    assert call(out=4) == -1                     # unknown output kind


def test_prepack_rejects(lib):
    f = _ptr(FAKE)
    assert lib.moe_w4_prepack(f, f, 8, 200, 256, f, f, None) == -2
    assert lib.moe_w4_prepack(f, f, 8, 256, 96, f, f, None) == -1   # K < 128
    assert lib.moe_w4_prepack(f, f, 8, 256, 160, f, f, None) == -2
    assert lib.moe_w4_prepack(f, f, 0, 256, 256, f, f, None) == -1
    assert lib.moe_w4_prepack(f, None, 8, 256, 256, f, f, None) == -1
    assert lib.moe_w4_prepack(_ptr(FAKE + 4), f, 8, 256, 256, f, f, None) == -3


def test_combine_and_forward_reject(lib):
    f = _ptr(FAKE)
    F32, F16E = moe.MOE_OUT_F32, moe.MOE_OUT_F16E
    assert lib.moe_combine(f, F32, None, f, f, None, 4, 2, 12, f, None) == -2   # H % 8
    assert lib.moe_combine(f, F16E, f, f, f, None, 4, 2, 12, f, None) == -2     # fp16 O: H % 8 too
    assert lib.moe_combine(f, F32, None, f, f, None, 0, 2, 16, f, None) == 0    # T == 0
    assert lib.moe_combine(_ptr(FAKE + 4), F32, None, f, f, None, 4, 2, 16, f, None) == -3
    assert lib.moe_combine(f, F16E, None, f, f, None, 4, 2, 16, f, None) == -1  # fp16 O needs its side values
    assert lib.moe_combine(f, 0, None, f, f, None, 4, 2, 16, f, None) == -1     # bf16 O is not accepted
    ws = moe.moe_ffn_workspace_bytes(16, 256, 128, 8, 2)
    fw = lambda **kw: lib.moe_ffn_forward(kw.get("x", f), f, kw.get("T", 16), kw.get("H", 256), kw.get("I", 128),
                                          kw.get("E", 8), kw.get("k", 2), f, f, f, f, kw.get("lay", 0), f, None,
                                          None, f, kw.get("ws", ws), None)
    assert fw(H=250) == -2
    assert fw(I=48) == -2
    assert fw(k=9) == -1
    assert fw(ws=ws - 1) == -4
    assert fw(x=_ptr(FAKE + 2)) == -3
    assert fw(T=0) == 0
    assert fw(lay=5) == -1
    assert fw(lay=1, I=96) == -2       # packed needs I % 128 == 0


def test_router_logits_rejects(lib):
    f = _ptr(FAKE)
    rl = lambda **kw: lib.moe_router_logits(kw.get("x", f), f, kw.get("T", 8), kw.get("H", 256), kw.get("E", 64),
                                            kw.get("lg", f), None)
    assert rl(H=250) == -1            # H % 32
    assert rl(H=0) == -1
    assert rl(E=0) == -1
    assert rl(E=1025) == -2           # above MOE_MAX_EXPERTS
    assert rl(T=-1) == -1
    assert rl(T=0) == 0
    assert rl(x=None) == -1
    assert rl(x=_ptr(FAKE + 8)) == -3
    assert rl(lg=_ptr(FAKE + 2)) == -3


def test_dense_ffn_rejects(lib):
    f = _ptr(FAKE)
    ws = moe.moe_dense_ffn_workspace_bytes(16, 256, 128)
    assert ws == 16 * 128 * 2
    df = lambda **kw: lib.moe_dense_ffn_w4a16(kw.get("x", f), kw.get("T", 16), kw.get("H", 256), kw.get("I", 128),
                                              f, f, kw.get("w2q", f), f, kw.get("lay", 0), f, f, kw.get("ws", ws),
                                              None)
    assert df(H=250) == -2
    assert df(I=40) == -2
    assert df(lay=1, I=96) == -2
    assert df(lay=3) == -1
    assert df(ws=ws - 1) == -4
    assert df(w2q=None) == -1
    assert df(x=_ptr(FAKE + 2)) == -3
    assert df(T=0) == 0


def test_block_forward_rejects(lib):
    f = _ptr(FAKE)
    T, H, I, E, k = 16, 256, 128, 8, 2
    base = moe.moe_ffn_workspace_bytes(T, H, I, E, k)
    ws0 = moe.moe_ffn_block_workspace_bytes(T, H, I, E, k, 0)
    ws1 = moe.moe_ffn_block_workspace_bytes(T, H, I, E, k, 256)
    assert ws0 == base + T * E * 4
    assert ws1 == ws0 + T * 256 * 2 + T * H * 4
    bf = lambda **kw: lib.moe_ffn_block_forward(
        f, kw.get("wr", f), kw.get("T", T), H, I, E, k, f, f, f, f, kw.get("Is", 256), kw.get("s1", f), f, f, f,
        kw.get("lay", 0), f, kw.get("lg", None), None, None, f, kw.get("ws", ws1), None)
    assert bf(Is=-32) == -1
    assert bf(Is=48) == -2            # shared expert size follows the rules for I
    assert bf(Is=96, lay=1) == -2
    assert bf(s1=None) == -1          # NULL shared weight with Is > 0
    assert bf(wr=None) == -1
    assert bf(wr=_ptr(FAKE + 4)) == -3
    assert bf(lg=_ptr(FAKE + 2)) == -3
    assert bf(ws=ws1 - 1) == -4
    assert bf(T=0) == 0
    assert moe.moe_ffn_block_workspace_bytes(T, H, I, E, k, -1) == 0



def test_mxfp4_entry_points_reject(lib):
    f = _ptr(FAKE)
    # quantizer
    assert lib.moe_mx_quantize(f, 4, 48, f, f, None) == -1         # K % 32
    assert lib.moe_mx_quantize(f, 0, 64, f, f, None) == 0
    assert lib.moe_mx_quantize(_ptr(FAKE + 4), 4, 64, f, f, None) == -3
    # prepack
    assert lib.moe_mx_prepack(f, f, 2, 40, 256, f, f, None) == -2   # N % 16
    assert lib.moe_mx_prepack(f, f, 2, 48, 160, f, f, None) == -2   # K % 128
    assert lib.moe_mx_prepack(f, None, 2, 48, 256, f, f, None) == -1
    # grouped GEMM
    g = lambda **kw: lib.moe_grouped_gemm_mxfp4(f, f, None, 1, f, f, kw.get("lay", 0), kw.get("act", 0), 4, kw.get("N", 256),
                                                kw.get("K", 256), f, 8, f, kw.get("bm", 16), kw.get("epi", 0), f,
                                                kw.get("cs", f), 1, None)
    assert g(K=100) == -2
    assert g(bm=256) == -2                                         # MXFP4 tiles are 16, 32, 64 or 128 rows
    assert g(bm=128, K=160) == -2                                  # the 128-row kernel steps K by 128
    assert g(bm=128, act=1, lay=1) == -2                           # ... and reads row-major activations
    assert g(epi=1, N=96) == -2                                    # h blocks of 32 need N % 64 == 0
    assert g(epi=1, cs=None) == -1
    assert g(lay=1, K=160) == -2
    assert g(lay=7) == -1
    assert g(act=1) == -1                                          # tile-blocked activations need packed weights
    assert g(act=1, lay=1, epi=1, N=192) == -2                     # tile-blocked h needs N/2 % 128 == 0
    assert g(act=2, lay=1) == -1
    qt = lambda **kw: lib.moe_mx_quantize_tiles(f, 16, kw.get("K", 256), None, 1, f, 8, f, kw.get("bm", 16), f, f, None)
    assert qt(K=96) == -1
    assert qt(bm=128) == -2
    # layer
    assert moe.moe_ffn_mxfp4_block_m(800, 2048, 512, 256, 8) == 32
    assert moe.moe_ffn_mxfp4_block_m(4096, 4096, 14336, 8, 2) == 128  # large experts: the LDS-staged kernel
    assert moe.moe_ffn_mxfp4_block_m(4096, 4096, 14336 + 32, 8, 2) == 64  # ... which needs K % 128 == 0
    assert moe.moe_ffn_mxfp4_workspace_bytes(16, 256, 96, 8, 2) > 0
    assert moe.moe_ffn_mxfp4_workspace_bytes(16, 250, 96, 8, 2) == 0
    ws = moe.moe_ffn_mxfp4_workspace_bytes(16, 256, 128, 8, 2)
    fw = lambda **kw: lib.moe_ffn_forward_mxfp4(kw.get("x", f), f, kw.get("T", 16), kw.get("H", 256), kw.get("I", 128),
                                                8, kw.get("k", 2), f, f, f, f, kw.get("lay", 0), f, None, None, f,
                                                kw.get("ws", ws), None)
    assert fw(H=250) == -2
    assert fw(k=9) == -1
    assert fw(ws=ws - 1) == -4
    assert fw(x=_ptr(FAKE + 2)) == -3
    assert fw(lay=1, I=96) == -2                                   # packed needs I % 128 == 0
    assert fw(lay=3) == -1
    assert fw(T=0) == 0


def test_f8_entry_points_reject(lib):
    f = _ptr(FAKE)
    # quantizer
    assert lib.moe_f8_quantize(f, 0, 4, 96, f, f, None) == -1      # K % 128
    assert lib.moe_f8_quantize(f, 2, 4, 128, f, f, None) == -1     # unknown input dtype
    assert lib.moe_f8_quantize(f, 0, 0, 128, f, f, None) == 0
    assert lib.moe_f8_quantize(_ptr(FAKE + 4), 1, 4, 128, f, f, None) == -3
    assert lib.moe_f8_quantize(f, 0, 4, 128, f, None, None) == -1
    # grouped GEMM
    g = lambda **kw: lib.moe_grouped_gemm_f8(f, f, None, 1, f, f, 4, kw.get("N", 256), kw.get("K", 256), f,
                                             kw.get("mt", 8), f, kw.get("bm", 16), kw.get("epi", 0), kw.get("C", f),
                                             kw.get("cs", None), kw.get("od", 1), None)
    assert g(K=160) == -2
    assert g(K=32768 + 128) == -2                                  # activation scales of a tile staged in LDS
    assert g(bm=256) == -2
    assert g(epi=1, N=255) == -1                                   # SiLU*mul pairs gate and up rows
    assert g(epi=1, od=0) == -1                                    # h is written in fp32
    assert g(epi=5) == -1
    assert g(C=None) == -1
    assert g(C=_ptr(FAKE + 8)) == -3
    assert g(mt=0, C=None) == 0                                    # no tiles: nothing to launch
    assert g(epi=1, od=2, bm=64, cs=f) == -2                       # fused h quantization: 128-row tiles
    assert g(epi=1, od=2, bm=128, N=384, cs=f) == -2               # ... and whole 1x128 blocks of h
    assert g(epi=0, od=2, bm=128, cs=f) == -2                      # ... of the SiLU*mul output
    assert g(epi=1, od=2, bm=128, N=512) == -1                     # ... into a scale array
    assert g(epi=1, od=2, bm=128, N=512, cs=_ptr(FAKE + 2)) == -3
    # layer
    assert moe.moe_ffn_f8_block_m(800, 256, 8) == 32
    assert moe.moe_ffn_f8_block_m(4096, 8, 2) == 128               # large experts: the LDS-staged kernel
    assert moe.moe_ffn_f8_workspace_bytes(16, 256, 128, 8, 2) > 0
    assert moe.moe_ffn_f8_workspace_bytes(16, 256, 96, 8, 2) == 0  # I % 128
    T, H, I, E, k = 16, 256, 128, 8, 2
    ws = moe.moe_ffn_f8_workspace_bytes(T, H, I, E, k)
    R = T * k
    assert ws >= T * H + R * I * 4 + R * I + R * H * 4            # x codes, h fp32, h codes, down output
    fw = lambda **kw: lib.moe_ffn_forward_f8(kw.get("x", f), f, kw.get("T", T), kw.get("H", H), kw.get("I", I), E,
                                             kw.get("k", k), f, kw.get("ws13", f), f, f, f, None, None, f,
                                             kw.get("ws", ws), None)
    assert fw(H=192) == -2
    assert fw(k=9) == -1
    assert fw(ws=ws - 1) == -4
    assert fw(x=_ptr(FAKE + 2)) == -3
    assert fw(ws13=_ptr(FAKE + 2)) == -3                           # fp32 scales need 4-byte alignment
    assert fw(ws13=None) == -1
    assert fw(T=0) == 0


def test_w4a8_entry_points_reject(lib):
    f = _ptr(FAKE)
    # quantizer
    assert lib.moe_mx8_quantize(f, 4, 48, f, f, None) == -1          # K % 32
    assert lib.moe_mx8_quantize(f, 0, 64, f, f, None) == 0
    assert lib.moe_mx8_quantize(_ptr(FAKE + 8), 4, 64, f, f, None) == -3
    assert lib.moe_mx8_quantize(f, 4, 64, f, None, None) == -1
    # grouped GEMM (MXFP8 activations, row-major)
    g = lambda **kw: lib.moe_grouped_gemm_w4a8(f, f, None, 1, f, f, kw.get("wl", 0), kw.get("al", 0), 4,
                                               kw.get("N", 256), kw.get("K", 256), f, kw.get("mt", 8), f,
                                               kw.get("bm", 16), kw.get("epi", 0), kw.get("C", f), kw.get("cs", f),
                                               kw.get("od", 1), None)
    assert g(K=48) == -2
    assert g(bm=256) == -2
    assert g(bm=128, K=160) == -2                                   # the 128-row kernel steps K by 128
    assert lib.moe_grouped_gemm_w4a8(f, _ptr(FAKE + 1), None, 1, f, f, 0, 0, 4, 256, 256, f, 8, f, 128, 0, f, None,
                                     1, None) == -3                 # the 128-row kernel loads scales 4 bytes wide
    assert g(al=1) == -1                                            # tile-blocked activations: packed weights
    assert g(al=1, wl=1, bm=128) == -1                              # ... and tiles of at most 64 rows
    assert g(al=1, wl=1, epi=1, N=320) == -2                        # a tile-blocked h needs N/2 % 128 == 0
    assert g(al=3) == -1
    q8 = lambda **kw: lib.moe_mx8_quantize_tiles(f, 4, kw.get("K", 256), None, 1, f, 8, f, kw.get("bm", 16), f, f,
                                                 None)
    assert q8(K=96) == -1
    assert q8(bm=128) == -2
    assert g(epi=1, N=96) == -2                                     # h blocks of 32 columns
    assert g(epi=5) == -1
    assert g(od=7) == -1
    assert g(wl=1, K=96) == -2                                      # packed weights: K % 128
    assert g(epi=1, cs=None) == -1                                  # h scale bytes
    assert g(C=_ptr(FAKE + 4)) == -3
    assert g(mt=0, C=None) == 0                                     # no tiles: nothing to launch
    # layer
    assert moe.moe_ffn_w4a8_block_m(800, 2048, 512, 256, 8) == 32
    assert moe.moe_ffn_w4a8_block_m(4096, 4096, 14336, 8, 2) == 128  # large experts: the LDS-staged kernel
    assert moe.moe_ffn_w4a8_block_m(4096, 4096, 14336 - 32, 8, 2) == 64  # ... which steps K by 128
    assert moe.moe_ffn_w4a8_block_m(4, 256, 128, 8, 9) == -1
    T, H, I, E, k = 16, 256, 128, 8, 2
    ws = moe.moe_ffn_w4a8_workspace_bytes(T, H, I, E, k)
    R = T * k
    assert ws >= T * H + R * I + R * H * 4                          # x codes, h codes, down output
    assert moe.moe_ffn_w4a8_workspace_bytes(T, H, 96, E, 10) == 0   # k > E
    fw = lambda **kw: lib.moe_ffn_forward_w4a8(kw.get("x", f), f, kw.get("T", T), kw.get("H", H), kw.get("I", I), E,
                                               kw.get("k", k), f, f, f, f, kw.get("wl", 0), f, None, None, f,
                                               kw.get("ws", ws), None)
    assert fw(H=200) == -2
    assert fw(wl=1, I=96) == -2                                     # packed weights: I % 128
    assert fw(k=9) == -1
    assert fw(ws=ws - 1) == -4
    assert fw(x=_ptr(FAKE + 2)) == -3
    assert fw(T=0) == 0


@pytest.mark.parametrize("variant,T,E,k,H,I", [
    ("mxfp4", 32, 8, 8, 256, 128),     # 256 rows
    ("w4a8", 2048, 8, 8, 256, 128),    # 16384 rows
    ("f8", 2048, 8, 8, 256, 256),      # 16384 rows, 128-row tiles
])
def test_variant_layers_switch_to_fp16_o_at_their_row_threshold(variant, T, E, k, H, I):
    """From a row threshold a variant layer keeps the down projection's output as fp16 with in-band
    exponents (R*H*2 bytes plus R*H/8 fp32 side values) instead of fp32 (R*H*4): the workspace
    shrinks by about R*H*1.5 bytes between T - 1 and T tokens although everything else grows."""
    ws = {"mxfp4": moe.moe_ffn_mxfp4_workspace_bytes, "w4a8": moe.moe_ffn_w4a8_workspace_bytes,
          "f8": moe.moe_ffn_f8_workspace_bytes}[variant]
    below, at = ws(T - 1, H, I, E, k), ws(T, H, I, E, k)
    R = T * k
    assert 0 < at and below - at > R * H  # the O saving (R*H*1.5) outweighs one token's other growth
    assert ws(T + 1, H, I, E, k) > at      # and it keeps growing above


def test_noalloc_entry_point_rejects_sizes_beyond_its_scratch(lib):
    """The entry point without allocation checks its fixed scratch size on the host, before any
    device call, so an oversized layer fails the same way with or without a GPU."""
    assert moe.moe_ffn_noalloc_scratch_bytes() == 64 << 20
    # the 800-token, 256-expert layer fits; the 4096-token, 8-expert one (about 305 MB) does not
    assert moe.moe_ffn_workspace_bytes(800, 2048, 512, 256, 8) <= moe.moe_ffn_noalloc_scratch_bytes()
    assert moe.moe_ffn_workspace_bytes(4096, 4096, 14336, 8, 2) > moe.moe_ffn_noalloc_scratch_bytes()
    P = _ptr(FAKE)
    st = lib.moe_ffn_forward_noalloc(P, P, 4096, 4096, 14336, 8, 2, P, P, P, P, moe.MOE_LAYOUT_PACKED, P, None,
                                     None, None)
    assert st == -4 and b"static" in lib.moe_last_error()
    # shape errors come first, as in moe_ffn_forward
    st = lib.moe_ffn_forward_noalloc(P, P, 4, 2048, 512, 8, 9, P, P, P, P, 0, P, None, None, None)
    assert st == -1
    # an empty batch is a valid no-op that needs no device
    assert lib.moe_ffn_forward_noalloc(P, P, 0, 2048, 512, 8, 2, P, P, P, P, 0, P, None, None, None) == 0
