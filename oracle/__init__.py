"""CPU oracle of the MoE W4A16 layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product (``moe_w4a16_grouped_amd``) never imports it, and it never imports the product.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, loops in definition order); this module only
builds that file with gcc and marshals numpy arrays into it.  See the C file's header for the pages
and sections each function follows and for the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
            lib.oracle_e2m1_value.restype = ctypes.c_double
            lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_value.restype = ctypes.c_double
            lib.oracle_dequant.argtypes = [P, P, I64, I64, P]
            lib.oracle_dequant.restype = None
            lib.oracle_route.argtypes = [P, I64, I64, I64, P, P]
            lib.oracle_route.restype = None
            lib.oracle_align.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P]
            lib.oracle_align.restype = I64
            lib.oracle_moe_ffn.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, P, P, P, I64, P, P, P]
            lib.oracle_moe_ffn.restype = None
            lib.oracle_grouped_proj.argtypes = [P, P, I64, P, P, I64, I64, I64, P, ctypes.c_int, P, P]
            lib.oracle_grouped_proj.restype = None
            lib.oracle_combine.argtypes = [P, P, P, I64, I64, I64, P]
            lib.oracle_router_logits.argtypes = [P, P, I64, I64, I64, P]
            lib.oracle_shared_ffn.argtypes = [P, I64, I64, P, P, P, P, P, I64, P]
            lib.oracle_combine.restype = None
            lib.oracle_e8m0_value.argtypes = [ctypes.c_int]
            lib.oracle_e8m0_value.restype = ctypes.c_double
            lib.oracle_e2m1_nearest.argtypes = [ctypes.c_double]
            lib.oracle_e2m1_nearest.restype = ctypes.c_int
            lib.oracle_mx_quantize.argtypes = [P, I64, I64, P, P]
            lib.oracle_mx_dequant.argtypes = [P, P, I64, I64, P]
            lib.oracle_moe_ffn_mx.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, P, P, P, I64, P, P]
            lib.oracle_grouped_proj_mx.argtypes = [P, P, P, I64, P, P, I64, I64, I64, P, ctypes.c_int, P]
            lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
            lib.oracle_e4m3_value.restype = ctypes.c_double
            lib.oracle_e4m3_nearest.argtypes = [ctypes.c_double]
            lib.oracle_e4m3_nearest.restype = ctypes.c_int
            lib.oracle_f8_quantize.argtypes = [P, I64, I64, P, P]
            lib.oracle_f8_dequant.argtypes = [P, P, I64, I64, P]
            lib.oracle_moe_ffn_f8.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, P, P, P, I64, P, P]
            lib.oracle_grouped_proj_f8.argtypes = [P, P, P, I64, P, P, I64, I64, I64, P, ctypes.c_int, P]
            lib.oracle_mx8_quantize.argtypes = [P, I64, I64, P, P]
            lib.oracle_mx8_dequant.argtypes = [P, P, I64, I64, P]
            lib.oracle_moe_ffn_w4a8.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, P, P, P, I64, P, P]
            lib.oracle_grouped_proj_w4a8.argtypes = [P, P, P, I64, P, P, I64, I64, I64, P, ctypes.c_int, P]
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def dequant(q, s) -> np.ndarray:
    """[N, K/2] codes + [N, K/32] bf16 scales -> fp64 [N, K]."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    N, K = q.shape[0], q.shape[1] * 2
    out = np.empty((N, K), np.float64)
    _load().oracle_dequant(_ptr(q), _ptr(s), N, K, _ptr(out))
    return out


def route(logits, k: int):
    """fp32 [T, E] logits -> (ids int32 [T, k], weights fp64 [T, k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().oracle_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w))
    return ids, w


def align(ids, E: int, block_m: int):
    """Stable permutation of flat slots by expert; returns a dict of int32 arrays and counts."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    R = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ids = np.empty(R, np.int32)
    inv_perm = np.empty(R, np.int32)
    mmt = np.zeros(1, np.int32)
    lib = _load()
    nt = lib.oracle_align(_ptr(ids), T, k, E, block_m, _ptr(counts), _ptr(offsets), _ptr(sorted_ids),
                          _ptr(inv_perm), None, _ptr(mmt))
    tiles = np.empty((max(nt, 1), 3), np.int32)
    lib.oracle_align(_ptr(ids), T, k, E, block_m, _ptr(counts), _ptr(offsets), _ptr(sorted_ids),
                     _ptr(inv_perm), _ptr(tiles), _ptr(mmt))
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids, inv_perm=inv_perm,
                tiles=tiles[:nt], num_tiles=int(nt), max_m_tiles=int(mmt[0]))


def moe_ffn(inp, tokens=None, diagnostics: bool = False):
    """Full layer on ``moe_inputs.MoEInputs``; returns y fp64 [n_tok, H] (and h, o if asked).

    ``tokens``: optional 1-D array of token indices to evaluate (each token is independent)."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    y = np.empty((n, H), np.float64)
    h = np.empty((n, k, I), np.float64) if diagnostics else None
    o = np.empty((n, k, H), np.float64) if diagnostics else None
    x = _c(inp.x, np.uint16)
    lg = _c(inp.logits, np.float32)
    a13q, a13s = _c(inp.w13_q, np.uint8), _c(inp.w13_s, np.uint16)
    a2q, a2s = _c(inp.w2_q, np.uint8), _c(inp.w2_s, np.uint16)
    _load().oracle_moe_ffn(_ptr(x), _ptr(lg), T, H, I, E, k, _ptr(a13q), _ptr(a13s), _ptr(a2q), _ptr(a2s),
                           _ptr(tok), n, _ptr(y), _ptr(h), _ptr(o))
    return (y, h, o) if diagnostics else y


def grouped_proj(A, a_row_of, a_row_div: int, Wq, Ws, offsets, silu_mul: bool = False, row_scale=None):
    """Grouped per-expert projection over permuted rows (see the C function); returns fp64."""
    A = _c(A, np.uint16)
    Wq = _c(Wq, np.uint8)
    Ws = _c(Ws, np.uint16)
    offsets = _c(offsets, np.int32)
    E, N, K = Wq.shape[0], Wq.shape[1], Wq.shape[2] * 2
    R = int(offsets[-1])
    nout = N // 2 if silu_mul else N
    C = np.empty((R, nout), np.float64)
    aro = None if a_row_of is None else _c(a_row_of, np.int32)
    rs = None if row_scale is None else _c(row_scale, np.float64)
    _load().oracle_grouped_proj(_ptr(A), _ptr(aro), a_row_div, _ptr(Wq), _ptr(Ws), E, N, K, _ptr(offsets),
                                int(bool(silu_mul)), _ptr(rs), _ptr(C))
    return C


def combine(O, inv_perm, w, T: int, k: int):
    """y[t] = sum_s w[t,s] * O[inv_perm[t*k+s]]; O fp64 [R, H]; returns fp64 [T, H]."""
    O = _c(O, np.float64)
    inv_perm = _c(inv_perm, np.int32)
    w = _c(w, np.float64)
    H = O.shape[1]
    y = np.empty((T, H), np.float64)
    _load().oracle_combine(_ptr(O), _ptr(inv_perm), _ptr(w), T, k, H, _ptr(y))
    return y


def router_logits(x, w_router):
    """Gate logits x [T, H] @ w_router [E, H]^T from bf16 bits, fp64 [T, E]."""
    x = _c(x, np.uint16)
    wr = _c(w_router, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(_ptr(x), _ptr(wr), T, H, E, _ptr(out))
    return out


def shared_ffn(x, w13s_q, w13s_s, w2s_q, w2s_s, tokens=None):
    """Shared expert (dense SwiGLU in the W4 format) on every token (or a subset); fp64 [n, H]."""
    x = _c(x, np.uint16)
    T, H = x.shape
    Is = w2s_q.shape[1] * 2
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    out = np.empty((n, H), np.float64)
    a13q, a13s = _c(w13s_q, np.uint8), _c(w13s_s, np.uint16)
    a2q, a2s = _c(w2s_q, np.uint8), _c(w2s_s, np.uint16)
    _load().oracle_shared_ffn(_ptr(x), H, Is, _ptr(a13q), _ptr(a13s), _ptr(a2q), _ptr(a2s), _ptr(tok), n, _ptr(out))
    return out


# ---- MXFP4 (E2M1 codes, E8M0 block scales on both operands) -------------------------------------

def e8m0_value(byte: int) -> float:
    return float(_load().oracle_e8m0_value(int(byte)))


def e2m1_nearest(v: float) -> int:
    return int(_load().oracle_e2m1_nearest(float(v)))


def mx_quantize(v):
    """MX quantization of fp64 values [rows, K] -> (codes uint8 [rows, K/2], scale bytes uint8 [rows, K/32])."""
    v = _c(v, np.float64)
    if v.ndim == 1:
        v = v[None]
    rows, K = v.shape
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // 32), np.uint8)
    _load().oracle_mx_quantize(_ptr(v), rows, K, _ptr(q), _ptr(s))
    return q, s


def mx_dequant(q, s) -> np.ndarray:
    """MX codes [rows, K/2] + scale bytes [rows, K/32] -> fp64 [rows, K]."""
    q, s = _c(q, np.uint8), _c(s, np.uint8)
    rows, K = q.shape[0], q.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    _load().oracle_mx_dequant(_ptr(q), _ptr(s), rows, K, _ptr(out))
    return out


def moe_ffn_mx(inp, tokens=None, diagnostics: bool = False):
    """MXFP4 (W4A4) layer on ``moe_inputs.MXInputs``; returns y fp64 [n_tok, H] (and h before its
    quantization, [n_tok, k, I], if asked)."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    y = np.empty((n, H), np.float64)
    h = np.empty((n, k, I), np.float64) if diagnostics else None
    _load().oracle_moe_ffn_mx(_ptr(_c(inp.x, np.uint16)), _ptr(_c(inp.logits, np.float32)), T, H, I, E, k,
                              _ptr(_c(inp.w13_q, np.uint8)), _ptr(_c(inp.w13_e, np.uint8)),
                              _ptr(_c(inp.w2_q, np.uint8)), _ptr(_c(inp.w2_e, np.uint8)), _ptr(tok), n, _ptr(y),
                              _ptr(h))
    return (y, h) if diagnostics else y


def grouped_proj_mx(Aq, As, a_row_of, a_row_div: int, Wq, We, offsets, silu_mul: bool = False):
    """Grouped MX projection over permuted rows (see the C function); fp64, before any quantization."""
    Aq, As = _c(Aq, np.uint8), _c(As, np.uint8)
    Wq, We = _c(Wq, np.uint8), _c(We, np.uint8)
    offsets = _c(offsets, np.int32)
    E, N, K = Wq.shape[0], Wq.shape[1], Wq.shape[2] * 2
    R = int(offsets[-1])
    nout = N // 2 if silu_mul else N
    C = np.empty((R, nout), np.float64)
    aro = None if a_row_of is None else _c(a_row_of, np.int32)
    _load().oracle_grouped_proj_mx(_ptr(Aq), _ptr(As), _ptr(aro), a_row_div, _ptr(Wq), _ptr(We), E, N, K,
                                   _ptr(offsets), int(bool(silu_mul)), _ptr(C))
    return C


# ---- FP8 (E4M3 codes, per-1x128 fp32 scales on both operands) -------------------------------------

def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_nearest(v: float) -> int:
    return int(_load().oracle_e4m3_nearest(float(v)))


def f8_quantize(v):
    """Per-1x128 FP8 quantization of values [rows, K] (fp64 in; decisions in fp32) ->
    (codes uint8 [rows, K], scales float32 [rows, K/128])."""
    v = _c(v, np.float64)
    if v.ndim == 1:
        v = v[None]
    rows, K = v.shape
    q = np.empty((rows, K), np.uint8)
    s = np.empty((rows, K // 128), np.float32)
    _load().oracle_f8_quantize(_ptr(v), rows, K, _ptr(q), _ptr(s))
    return q, s


def f8_dequant(q, s) -> np.ndarray:
    """FP8 codes [rows, K] + fp32 scales [rows, K/128] -> fp64 [rows, K]."""
    q, s = _c(q, np.uint8), _c(s, np.float32)
    rows, K = q.shape
    out = np.empty((rows, K), np.float64)
    _load().oracle_f8_dequant(_ptr(q), _ptr(s), rows, K, _ptr(out))
    return out


def moe_ffn_f8(inp, tokens=None, diagnostics: bool = False):
    """FP8 (W8A8, per-1x128) layer on ``moe_inputs.F8Inputs``; returns y fp64 [n_tok, H] (and h
    before its quantization, [n_tok, k, I], if asked)."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    y = np.empty((n, H), np.float64)
    h = np.empty((n, k, I), np.float64) if diagnostics else None
    _load().oracle_moe_ffn_f8(_ptr(_c(inp.x, np.uint16)), _ptr(_c(inp.logits, np.float32)), T, H, I, E, k,
                              _ptr(_c(inp.w13_q, np.uint8)), _ptr(_c(inp.w13_s, np.float32)),
                              _ptr(_c(inp.w2_q, np.uint8)), _ptr(_c(inp.w2_s, np.float32)), _ptr(tok), n, _ptr(y),
                              _ptr(h))
    return (y, h) if diagnostics else y


def grouped_proj_f8(Aq, As, a_row_of, a_row_div: int, Wq, Ws, offsets, silu_mul: bool = False):
    """Grouped FP8 projection over permuted rows (see the C function); fp64, before any quantization."""
    Aq, As = _c(Aq, np.uint8), _c(As, np.float32)
    Wq, Ws = _c(Wq, np.uint8), _c(Ws, np.float32)
    offsets = _c(offsets, np.int32)
    E, N, K = Wq.shape
    R = int(offsets[-1])
    nout = N // 2 if silu_mul else N
    C = np.empty((R, nout), np.float64)
    aro = None if a_row_of is None else _c(a_row_of, np.int32)
    _load().oracle_grouped_proj_f8(_ptr(Aq), _ptr(As), _ptr(aro), a_row_div, _ptr(Wq), _ptr(Ws), E, N, K,
                                   _ptr(offsets), int(bool(silu_mul)), _ptr(C))
    return C


# ---- W4A8 (MXFP8 activations: E4M3 codes + E8M0 per 32; MXFP4 weights) --------------------------------

def mx8_quantize(v):
    """MXFP8 quantization of fp64 values [rows, K] -> (codes uint8 [rows, K], scale bytes uint8 [rows, K/32])."""
    v = _c(v, np.float64)
    if v.ndim == 1:
        v = v[None]
    rows, K = v.shape
    q = np.empty((rows, K), np.uint8)
    s = np.empty((rows, K // 32), np.uint8)
    _load().oracle_mx8_quantize(_ptr(v), rows, K, _ptr(q), _ptr(s))
    return q, s


def mx8_dequant(q, s) -> np.ndarray:
    """MXFP8 codes [rows, K] + scale bytes [rows, K/32] -> fp64 [rows, K]."""
    q, s = _c(q, np.uint8), _c(s, np.uint8)
    rows, K = q.shape
    out = np.empty((rows, K), np.float64)
    _load().oracle_mx8_dequant(_ptr(q), _ptr(s), rows, K, _ptr(out))
    return out


def moe_ffn_w4a8(inp, tokens=None, diagnostics: bool = False):
    """W4A8 layer on ``moe_inputs.MXInputs`` (the MXFP4 weights); returns y fp64 [n_tok, H] (and h
    before its quantization, [n_tok, k, I], if asked)."""
    wl = inp.wl
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    y = np.empty((n, H), np.float64)
    h = np.empty((n, k, I), np.float64) if diagnostics else None
    _load().oracle_moe_ffn_w4a8(_ptr(_c(inp.x, np.uint16)), _ptr(_c(inp.logits, np.float32)), T, H, I, E, k,
                                _ptr(_c(inp.w13_q, np.uint8)), _ptr(_c(inp.w13_e, np.uint8)),
                                _ptr(_c(inp.w2_q, np.uint8)), _ptr(_c(inp.w2_e, np.uint8)), _ptr(tok), n, _ptr(y),
                                _ptr(h))
    return (y, h) if diagnostics else y


def grouped_proj_w4a8(Aq, As, a_row_of, a_row_div: int, Wq, We, offsets, silu_mul: bool = False):
    """Grouped W4A8 projection over permuted rows (see the C function); fp64, before any quantization."""
    Aq, As = _c(Aq, np.uint8), _c(As, np.uint8)
    Wq, We = _c(Wq, np.uint8), _c(We, np.uint8)
    offsets = _c(offsets, np.int32)
    E, N, K = Wq.shape[0], Wq.shape[1], Wq.shape[2] * 2
    R = int(offsets[-1])
    nout = N // 2 if silu_mul else N
    C = np.empty((R, nout), np.float64)
    aro = None if a_row_of is None else _c(a_row_of, np.int32)
    _load().oracle_grouped_proj_w4a8(_ptr(Aq), _ptr(As), _ptr(aro), a_row_div, _ptr(Wq), _ptr(We), E, N, K,
                                     _ptr(offsets), int(bool(silu_mul)), _ptr(C))
    return C
