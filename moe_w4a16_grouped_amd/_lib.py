"""ctypes binding of libmoe_w4a16.so: argument marshalling only.

Each function has the name of the C entry point it calls, takes torch tensors on the GPU, passes
their data pointers and the current HIP stream, and raises ``MoEError`` on a negative status.  Every
step of the layer runs in the HIP kernels of the library; there is no fallback of any kind: if the
library is not built, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmoe_w4a16.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED_SHAPE = -2
MOE_ERR_MISALIGNED = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_EPI_NONE = 0
MOE_EPI_SILU_MUL = 1
MOE_OUT_BF16 = 0
MOE_OUT_F32 = 1
MOE_LAYOUT_CANONICAL = 0
MOE_LAYOUT_PACKED = 1
MOE_ACT_ROWS = 0
MOE_ACT_TILED = 1
MOE_IN_BF16 = 0
MOE_IN_F32 = 1
MOE_OUT_F8 = 2
MOE_OUT_F16E = 3
MOE_OUT_H16 = 4

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_w4a16_grouped_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_abi_version": ([], I32),
        "moe_status_string": ([I32], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_route_topk": ([P, I32, I32, I32, P, P, P], I32),
        "moe_max_tiles": ([I32, I32, I32, I32], I32),
        "moe_align_workspace_bytes": ([I32, I32, I32], SZ),
        "moe_align": ([P, I32, I32, I32, I32, P, P, P, P, P, I32, P, P, SZ, P], I32),
        "moe_w4_prepack": ([P, P, I32, I32, I32, P, P, P], I32),
        "moe_grouped_gemm_w4a16": ([P, P, I32, P, P, I32, I32, I32, I32, P, I32, P, I32, I32, P, I32, P, P], I32),
        "moe_combine": ([P, I32, P, P, P, P, I32, I32, I32, P, P], I32),
        "moe_x_to_f16": ([P, I32, I32, P, P, P], I32),
        "moe_grouped_gemm_w4f16": ([P, P, P, P, P, I32, P, P, I32, I32, I32, I32, P, I32, P, I32, I32, P, I32, P, P, P],
                                   I32),
        "moe_router_logits": ([P, P, I32, I32, I32, P, P], I32),
        "moe_dense_ffn_workspace_bytes": ([I32, I32, I32], SZ),
        "moe_dense_ffn_w4a16": ([P, I32, I32, I32, P, P, P, P, I32, P, P, SZ, P], I32),
        "moe_ffn_block_workspace_bytes": ([I32, I32, I32, I32, I32, I32], SZ),
        "moe_mx_quantize": ([P, I32, I32, P, P, P], I32),
        "moe_mx_prepack": ([P, P, I32, I32, I32, P, P, P], I32),
        "moe_mx_quantize_tiles": ([P, I32, I32, P, I32, P, I32, P, I32, P, P, P], I32),
        "moe_grouped_gemm_mxfp4": ([P, P, P, I32, P, P, I32, I32, I32, I32, I32, P, I32, P, I32, I32, P, P, I32, P],
                                   I32),
        "moe_ffn_mxfp4_block_m": ([I32, I32, I32, I32, I32], I32),
        "moe_ffn_mxfp4_workspace_bytes": ([I32, I32, I32, I32, I32], SZ),
        "moe_ffn_forward_mxfp4": ([P, P, I32, I32, I32, I32, I32, P, P, P, P, I32, P, P, P, P, SZ, P], I32),
        "moe_mx8_quantize": ([P, I32, I32, P, P, P], I32),
        "moe_mx8_quantize_tiles": ([P, I32, I32, P, I32, P, I32, P, I32, P, P, P], I32),
        "moe_grouped_gemm_w4a8": ([P, P, P, I32, P, P, I32, I32, I32, I32, I32, P, I32, P, I32, I32, P, P, I32, P],
                                  I32),
        "moe_ffn_w4a8_block_m": ([I32, I32, I32, I32, I32], I32),
        "moe_ffn_w4a8_workspace_bytes": ([I32, I32, I32, I32, I32], SZ),
        "moe_ffn_forward_w4a8": ([P, P, I32, I32, I32, I32, I32, P, P, P, P, I32, P, P, P, P, SZ, P], I32),
        "moe_ffn_block_forward": ([P, P, I32, I32, I32, I32, I32, P, P, P, P, I32, P, P, P, P, I32, P, P, P, P, P,
                                   SZ, P], I32),
        "moe_f8_quantize": ([P, I32, I32, I32, P, P, P], I32),
        "moe_grouped_gemm_f8": ([P, P, P, I32, P, P, I32, I32, I32, P, I32, P, I32, I32, P, P, I32, P], I32),
        "moe_ffn_f8_block_m": ([I32, I32, I32], I32),
        "moe_ffn_f8_workspace_bytes": ([I32, I32, I32, I32, I32], SZ),
        "moe_ffn_forward_f8": ([P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, SZ, P], I32),
        "moe_ffn_block_m": ([I32, I32, I32, I32], I32),
        "moe_ffn_workspace_bytes": ([I32, I32, I32, I32, I32], SZ),
        "moe_ffn_forward": ([P, P, I32, I32, I32, I32, I32, P, P, P, P, I32, P, P, P, P, SZ, P], I32),
        "moe_ffn_noalloc_scratch_bytes": ([], SZ),
        "moe_ffn_forward_noalloc": ([P, P, I32, I32, I32, I32, I32, P, P, P, P, I32, P, P, P, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


EXPORTED = ("moe_abi_version", "moe_status_string", "moe_last_error", "moe_route_topk", "moe_max_tiles",
            "moe_align_workspace_bytes", "moe_align", "moe_w4_prepack", "moe_grouped_gemm_w4a16", "moe_combine",
            "moe_router_logits", "moe_dense_ffn_workspace_bytes", "moe_dense_ffn_w4a16",
            "moe_ffn_block_m", "moe_ffn_workspace_bytes", "moe_ffn_forward", "moe_ffn_block_workspace_bytes",
            "moe_ffn_block_forward", "moe_mx_quantize", "moe_mx_quantize_tiles", "moe_mx_prepack", "moe_grouped_gemm_mxfp4", "moe_ffn_mxfp4_block_m",
            "moe_ffn_mxfp4_workspace_bytes", "moe_ffn_forward_mxfp4", "moe_f8_quantize", "moe_grouped_gemm_f8",
            "moe_ffn_f8_block_m", "moe_ffn_f8_workspace_bytes", "moe_ffn_forward_f8", "moe_mx8_quantize",
            "moe_mx8_quantize_tiles", "moe_grouped_gemm_w4a8", "moe_ffn_w4a8_block_m", "moe_ffn_w4a8_workspace_bytes",
            "moe_ffn_forward_w4a8", "moe_ffn_noalloc_scratch_bytes", "moe_ffn_forward_noalloc", "moe_x_to_f16",
            "moe_grouped_gemm_w4f16")


def _check(status: int):
    if status != MOE_OK:
        lib = load()
        raise MoEError(status, f"{lib.moe_status_string(status).decode()}: {lib.moe_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _req(t, dtype, name):
    ok = t.element_size() == 2 if dtype == "16bit" else t.dtype == dtype
    if not ok or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor (got {t.dtype}, {t.device})")
    return t


# ---- entry points ----------------------------------------------------------------------------------

def moe_max_tiles(T: int, k: int, E: int, block_m: int) -> int:
    return int(load().moe_max_tiles(T, k, E, block_m))


def moe_align_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(load().moe_align_workspace_bytes(T, k, E))


def moe_ffn_block_m(T: int, E: int, k: int, weight_layout: int = 0) -> int:
    return int(load().moe_ffn_block_m(T, E, k, weight_layout))


def moe_ffn_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load().moe_ffn_workspace_bytes(T, H, I, E, k))


def moe_route_topk(logits: torch.Tensor, k: int, topk_ids=None, topk_w=None, stream=None):
    """logits fp32 [T, E] -> (topk_ids int32 [T, k], topk_w fp32 [T, k])."""
    _req(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(load().moe_route_topk(_p(logits), T, E, k, _p(topk_ids), _p(topk_w), _stream(stream)))
    return topk_ids, topk_w


def moe_align(topk_ids: torch.Tensor, E: int, block_m: int, stream=None, max_tiles: int = None) -> dict:
    """topk_ids int32 [T, k] -> dict of device tensors (counts, offsets, sorted_ids, inv_perm, tiles,
    num_tiles) and the tile capacity ``max_tiles`` (default: moe_max_tiles; a larger capacity may be
    given)."""
    _req(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    R = T * k
    if max_tiles is None:
        max_tiles = moe_max_tiles(T, k, E, block_m)
    out = dict(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        sorted_ids=torch.empty(max(R, 1), dtype=torch.int32, device=dev),
        inv_perm=torch.empty(max(R, 1), dtype=torch.int32, device=dev),
        tiles=torch.empty((max(max_tiles, 1), 3), dtype=torch.int32, device=dev),
        num_tiles=torch.empty(1, dtype=torch.int32, device=dev),
    )
    wsb = moe_align_workspace_bytes(T, k, E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev) if wsb else None
    _check(load().moe_align(_p(topk_ids), T, k, E, block_m, _p(out["counts"]), _p(out["offsets"]),
                            _p(out["sorted_ids"]), _p(out["inv_perm"]), _p(out["tiles"]), max_tiles,
                            _p(out["num_tiles"]), _p(ws), wsb, _stream(stream)))
    out["max_tiles"] = max_tiles
    out["_workspace"] = ws
    return out


def moe_w4_prepack(w_q, w_s, packed_q=None, packed_s=None, stream=None):
    """Canonical [E, N, K/2] codes + [E, N, K/32] scales -> the same tensors in the packed layout
    (returned with the canonical shapes, which describe their sizes, not their element order)."""
    _req(w_q, torch.uint8, "w_q")
    _req(w_s, "16bit", "w_s")
    E, N, K2 = w_q.shape
    if packed_q is None:
        packed_q = torch.empty_like(w_q)
    if packed_s is None:
        packed_s = torch.empty_like(w_s)
    _check(load().moe_w4_prepack(_p(w_q), _p(w_s), E, N, 2 * K2, _p(packed_q), _p(packed_s), _stream(stream)))
    return packed_q, packed_s


def moe_grouped_gemm_w4a16(A, a_row_of, a_row_div: int, Wq, Ws, tiles, max_tiles: int, num_tiles,
                           block_m: int, epilogue: int, out_rows: int, out_dtype: int = MOE_OUT_BF16,
                           C=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL, C_side=None):
    """Grouped W4A16 GEMM over the tile list; returns C ([out_rows, N] or [out_rows, N/2]), or
    (C fp16, C_side fp32 [out_rows, ceil(N/8)]) for MOE_OUT_F16E."""
    _req(A, "16bit", "A")
    _req(Wq, torch.uint8, "Wq")
    E, N, K2 = Wq.shape
    K = 2 * K2
    ncols = N // 2 if epilogue == MOE_EPI_SILU_MUL else N
    if C is None:
        dt = {MOE_OUT_F32: torch.float32, MOE_OUT_F16E: torch.float16}.get(out_dtype, torch.bfloat16)
        C = torch.empty((out_rows, ncols), dtype=dt, device=A.device)
    if out_dtype == MOE_OUT_F16E and C_side is None:
        C_side = torch.empty((out_rows, (ncols + 7) // 8), dtype=torch.float32, device=A.device)
    _check(load().moe_grouped_gemm_w4a16(_p(A), _p(a_row_of), a_row_div, _p(Wq), _p(Ws), weight_layout, E, N, K,
                                         _p(tiles),
                                         max_tiles, _p(num_tiles), block_m, epilogue, _p(C), out_dtype, _p(C_side),
                                         _stream(stream)))
    return (C, C_side) if out_dtype == MOE_OUT_F16E else C


def moe_x_to_f16(x, x16=None, x_exp=None, stream=None):
    """bf16 x [T, H] -> (fp16 x16 [T, H], int32 row exponents [T]): x16 = fp16(x * 2^-x_exp)."""
    _req(x, "16bit", "x")
    T, H = x.shape
    if x16 is None:
        x16 = torch.empty((T, H), dtype=torch.float16, device=x.device)
    if x_exp is None:
        x_exp = torch.empty((T,), dtype=torch.int32, device=x.device)
    _check(load().moe_x_to_f16(_p(x), T, H, _p(x16), _p(x_exp), _stream(stream)))
    return x16, x_exp


def moe_grouped_gemm_w4f16(A, a_row_exp, a_exps, a_row_of, a_row_div: int, Wq, Ws, tiles, max_tiles: int,
                           num_tiles, block_m: int, epilogue: int, out_rows: int, out_dtype: int, C=None, C_aux=None,
                           C_aux2=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL):
    """Grouped GEMM of the exact fp16 path (fp16 activations with exponents).  a_exps: None or the
    (flags, row exponents) pair a SILU_MUL call returned for h.  Returns (h fp16, (flags, row
    exponents)) for SILU_MUL, (C fp16, side fp32) for MOE_OUT_F16E, or C fp32 for MOE_OUT_F32."""
    _req(A, "16bit", "A")
    _req(Wq, torch.uint8, "Wq")
    E, N, K2 = Wq.shape
    K = 2 * K2
    ncols = N // 2 if epilogue == MOE_EPI_SILU_MUL else N
    if C is None:
        C = torch.empty((out_rows, ncols), dtype=torch.float32 if out_dtype == MOE_OUT_F32 else torch.float16,
                        device=A.device)
    if out_dtype == MOE_OUT_H16:
        if C_aux is None:
            C_aux = torch.empty((max(max_tiles, 1), (ncols + 31) // 32), dtype=torch.uint8, device=A.device)
        if C_aux2 is None:
            C_aux2 = torch.empty((out_rows, (ncols + 31) // 32), dtype=torch.uint8, device=A.device)
    elif C_aux is None and out_dtype == MOE_OUT_F16E:
        C_aux = torch.empty((out_rows, (ncols + 7) // 8), dtype=torch.float32, device=A.device)
    bf, be = (None, None) if a_exps is None else a_exps
    _check(load().moe_grouped_gemm_w4f16(_p(A), _p(a_row_exp), _p(bf), _p(be), _p(a_row_of), a_row_div, _p(Wq), _p(Ws),
                                         weight_layout, E, N, K, _p(tiles), max_tiles, _p(num_tiles), block_m, epilogue,
                                         _p(C), out_dtype, _p(C_aux), _p(C_aux2), _stream(stream)))
    if out_dtype == MOE_OUT_F32:
        return C
    return (C, (C_aux, C_aux2)) if out_dtype == MOE_OUT_H16 else (C, C_aux)


def moe_combine(O, inv_perm, topk_w, y=None, stream=None, shared=None, O_side=None):
    """O fp32 [T*k, H], or fp16 [T*k, H] with side values O_side fp32 [T*k, H/8] (MOE_OUT_F16E),
    inv_perm int32 [T*k], topk_w fp32 [T, k] (+ shared fp32 [T, H]) -> y bf16 [T, H]."""
    if O.dtype == torch.float16:
        if O_side is None:
            raise ValueError("fp16 O needs its side values O_side")
        _req(O_side, torch.float32, "O_side")
        o_dtype = MOE_OUT_F16E
    else:
        _req(O, torch.float32, "O")
        o_dtype = MOE_OUT_F32
    if shared is not None:
        _req(shared, torch.float32, "shared")
    T, k = topk_w.shape
    H = O.shape[1]
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=O.device)
    _check(load().moe_combine(_p(O), o_dtype, _p(O_side) if o_dtype == MOE_OUT_F16E else None, _p(inv_perm),
                              _p(topk_w), _p(shared), T, k, H, _p(y), _stream(stream)))
    return y


def moe_router_logits(x, w_router, logits=None, stream=None):
    """x bf16 [T, H], w_router bf16 [E, H] -> logits fp32 [T, E]."""
    _req(x, "16bit", "x")
    _req(w_router, "16bit", "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(load().moe_router_logits(_p(x), _p(w_router), T, H, E, _p(logits), _stream(stream)))
    return logits


def moe_dense_ffn_workspace_bytes(T: int, H: int, I: int) -> int:
    return int(load().moe_dense_ffn_workspace_bytes(T, H, I))


def moe_dense_ffn_w4a16(x, w13_q, w13_s, w2_q, w2_s, out=None, workspace=None, stream=None,
                        weight_layout: int = MOE_LAYOUT_CANONICAL):
    """One dense SwiGLU expert on every token: x bf16 [T, H], w13_q [2I, H/2], w2_q [H, I/2] -> fp32 [T, H]."""
    _req(x, "16bit", "x")
    T, H = x.shape
    I = w13_q.shape[-2] // 2
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    wsb = moe_dense_ffn_workspace_bytes(T, H, I)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    _check(load().moe_dense_ffn_w4a16(_p(x), T, H, I, _p(w13_q), _p(w13_s), _p(w2_q), _p(w2_s), weight_layout,
                                      _p(out), _p(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))
    return out


def moe_ffn_block_workspace_bytes(T: int, H: int, I: int, E: int, k: int, Is: int = 0) -> int:
    return int(load().moe_ffn_block_workspace_bytes(T, H, I, E, k, Is))


def moe_ffn_block_forward(x, w_router, w13_q, w13_s, w2_q, w2_s, k: int, shared=None, y=None, logits_out=None,
                          topk_ids_out=None, topk_w_out=None, workspace=None, stream=None,
                          weight_layout: int = MOE_LAYOUT_CANONICAL):
    """Whole MoE block: router gate, optional shared expert ``shared = (w13s_q, w13s_s, w2s_q, w2s_s)``,
    routed experts and combine.  x bf16 [T, H], w_router bf16 [E, H] -> y bf16 [T, H]."""
    _req(x, "16bit", "x")
    T, H = x.shape
    E, N13, _ = w13_q.shape
    I = N13 // 2
    if shared is None:
        Is, sh = 0, (None, None, None, None)
    else:
        Is, sh = shared[0].shape[-2] // 2, shared
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    wsb = moe_ffn_block_workspace_bytes(T, H, I, E, k, Is)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    _check(load().moe_ffn_block_forward(_p(x), _p(w_router), T, H, I, E, k, _p(w13_q), _p(w13_s), _p(w2_q),
                                        _p(w2_s), Is, *(_p(t) for t in sh), weight_layout, _p(y), _p(logits_out),
                                        _p(topk_ids_out), _p(topk_w_out), _p(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def moe_ffn_forward(x, router_logits, w13_q, w13_s, w2_q, w2_s, k: int, y=None, topk_ids_out=None,
                    topk_w_out=None, workspace=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL):
    """Whole layer: x bf16 [T, H], logits fp32 [T, E], weights in the W4 group-32 format -> y bf16."""
    T, H = x.shape
    E, N13, _ = w13_q.shape
    I = N13 // 2
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    wsb = moe_ffn_workspace_bytes(T, H, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    _check(load().moe_ffn_forward(_p(x), _p(router_logits), T, H, I, E, k, _p(w13_q), _p(w13_s), _p(w2_q),
                                  _p(w2_s), weight_layout, _p(y), _p(topk_ids_out), _p(topk_w_out), _p(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def moe_ffn_noalloc_scratch_bytes() -> int:
    return int(load().moe_ffn_noalloc_scratch_bytes())


def moe_ffn_forward_noalloc(x, router_logits, w13_q, w13_s, w2_q, w2_s, k: int, y=None, topk_ids_out=None,
                            topk_w_out=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL):
    """moe_ffn_forward working in the library's static device scratch (the C call allocates nothing;
    y is allocated here only when the caller passes none)."""
    T, H = x.shape
    E, N13, _ = w13_q.shape
    I = N13 // 2
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(load().moe_ffn_forward_noalloc(_p(x), _p(router_logits), T, H, I, E, k, _p(w13_q), _p(w13_s), _p(w2_q),
                                          _p(w2_s), weight_layout, _p(y), _p(topk_ids_out), _p(topk_w_out),
                                          _stream(stream)))
    return y


# ---- MXFP4 (W4A4) ----------------------------------------------------------------------------------

def moe_mx_quantize(x, q=None, s=None, stream=None):
    """x bf16 [rows, K] -> (codes uint8 [rows, K/2], scale bytes uint8 [rows, K/32])."""
    _req(x, "16bit", "x")
    rows, K = x.shape
    if q is None:
        q = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(load().moe_mx_quantize(_p(x), rows, K, _p(q), _p(s), _stream(stream)))
    return q, s


def moe_mx_prepack(w_q, w_e, packed_q=None, packed_e=None, stream=None):
    """Canonical MXFP4 weights (codes [E, N, K/2], scale bytes [E, N, K/32]) -> the packed layout
    (returned with the canonical shapes, which describe sizes, not element order)."""
    _req(w_q, torch.uint8, "w_q")
    _req(w_e, torch.uint8, "w_e")
    E, N, K2 = w_q.shape
    if packed_q is None:
        packed_q = torch.empty_like(w_q)
    if packed_e is None:
        packed_e = torch.empty_like(w_e)
    _check(load().moe_mx_prepack(_p(w_q), _p(w_e), E, N, 2 * K2, _p(packed_q), _p(packed_e), _stream(stream)))
    return packed_q, packed_e


def moe_mx_quantize_tiles(x, a_row_of, a_row_div: int, tiles, max_tiles: int, num_tiles, block_m: int, q=None, s=None,
                          stream=None):
    """x bf16 [T, K] -> tile-blocked codes (uint8 [max_tiles * block_m, K/2]) and scale bytes
    (uint8 [max_tiles * block_m, K/32]) of the tile list (shapes give sizes, not element order)."""
    _req(x, "16bit", "x")
    T, K = x.shape
    rows = max(max_tiles, 1) * block_m
    if q is None:
        q = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    if q.numel() < rows * (K // 2) or s.numel() < rows * (K // 32):
        raise ValueError(f"tile-blocked activations need {rows} rows (max_tiles * block_m)")
    _check(load().moe_mx_quantize_tiles(_p(x), T, K, _p(a_row_of), a_row_div, _p(tiles), max_tiles, _p(num_tiles),
                                        block_m, _p(q), _p(s), _stream(stream)))
    return q, s


def moe_grouped_gemm_mxfp4(Aq, As, a_row_of, a_row_div: int, Wq, We, tiles, max_tiles: int, num_tiles,
                           block_m: int, epilogue: int, out_rows: int, out_dtype: int = MOE_OUT_F32, C=None,
                           Cs=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL,
                           act_layout: int = MOE_ACT_ROWS):
    """Grouped MXFP4 GEMM over the tile list.  NONE: returns C [out_rows, N]; SILU_MUL: returns the
    quantized h as (codes [out_rows, N/4], scale bytes [out_rows, N/64]); with act_layout TILED the
    h buffers must hold max_tiles * block_m rows (tile-blocked)."""
    _req(Aq, torch.uint8, "Aq")
    _req(Wq, torch.uint8, "Wq")
    E, N, K2 = Wq.shape
    K = 2 * K2
    dev = Aq.device
    if act_layout == MOE_ACT_TILED and epilogue == MOE_EPI_SILU_MUL:
        out_rows = max(out_rows, max(max_tiles, 1) * block_m)  # h is written tile-blocked
    if epilogue == MOE_EPI_SILU_MUL:
        if C is None:
            C = torch.empty((out_rows, N // 4), dtype=torch.uint8, device=dev)
        if Cs is None:
            Cs = torch.empty((out_rows, N // 64), dtype=torch.uint8, device=dev)
    elif C is None:
        C = torch.empty((out_rows, N), dtype=torch.float32 if out_dtype == MOE_OUT_F32 else torch.bfloat16, device=dev)
    if act_layout == MOE_ACT_TILED and epilogue == MOE_EPI_SILU_MUL:
        need = max(max_tiles, 1) * block_m
        if C.shape[0] < need or Cs.shape[0] < need:
            raise ValueError(f"tile-blocked h needs {need} rows (max_tiles * block_m), got {C.shape[0]}")
    _check(load().moe_grouped_gemm_mxfp4(_p(Aq), _p(As), _p(a_row_of), a_row_div, _p(Wq), _p(We), weight_layout,
                                         act_layout, E, N, K, _p(tiles),
                                         max_tiles, _p(num_tiles), block_m, epilogue, _p(C), _p(Cs), out_dtype,
                                         _stream(stream)))
    return (C, Cs) if epilogue == MOE_EPI_SILU_MUL else C


def moe_ffn_mxfp4_block_m(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load().moe_ffn_mxfp4_block_m(T, H, I, E, k))


def moe_ffn_mxfp4_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load().moe_ffn_mxfp4_workspace_bytes(T, H, I, E, k))


def moe_ffn_forward_mxfp4(x, router_logits, w13_q, w13_e, w2_q, w2_e, k: int, y=None, topk_ids_out=None,
                          topk_w_out=None, workspace=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL):
    """Whole MXFP4 (W4A4) layer: x bf16 [T, H], logits fp32 [T, E], MXFP4 weights -> y bf16 [T, H]."""
    _req(x, "16bit", "x")
    T, H = x.shape
    E, N13, _ = w13_q.shape
    I = N13 // 2
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    wsb = moe_ffn_mxfp4_workspace_bytes(T, H, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    _check(load().moe_ffn_forward_mxfp4(_p(x), _p(router_logits), T, H, I, E, k, _p(w13_q), _p(w13_e), _p(w2_q),
                                        _p(w2_e), weight_layout, _p(y), _p(topk_ids_out), _p(topk_w_out), _p(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


# ---- W4A8 (MXFP8 activations on MXFP4 weights) ------------------------------------------------------

def moe_mx8_quantize(x, q=None, s=None, stream=None):
    """x bf16 [rows, K] -> MXFP8 (codes uint8 [rows, K], scale bytes uint8 [rows, K/32])."""
    _req(x, "16bit", "x")
    rows, K = x.shape
    if q is None:
        q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(load().moe_mx8_quantize(_p(x), rows, K, _p(q), _p(s), _stream(stream)))
    return q, s


def moe_mx8_quantize_tiles(x, a_row_of, a_row_div: int, tiles, max_tiles: int, num_tiles, block_m: int, q=None,
                           s=None, stream=None):
    """x bf16 [T, K] -> tile-blocked MXFP8 codes [max_tiles * block_m, K] and scale bytes [.., K/32]."""
    _req(x, "16bit", "x")
    T, K = x.shape
    rows = max(max_tiles, 1) * block_m
    if q is None:
        q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(load().moe_mx8_quantize_tiles(_p(x), T, K, _p(a_row_of), a_row_div, _p(tiles), max_tiles, _p(num_tiles),
                                         block_m, _p(q), _p(s), _stream(stream)))
    return q, s


def moe_grouped_gemm_w4a8(Aq, As, a_row_of, a_row_div: int, Wq, We, tiles, max_tiles: int, num_tiles,
                          block_m: int, epilogue: int, out_rows: int, out_dtype: int = MOE_OUT_F32, C=None,
                          Cs=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL,
                          act_layout: int = MOE_ACT_ROWS):
    """Grouped W4A8 GEMM over the tile list (MXFP8 activations).  NONE: returns C [out_rows, N];
    SILU_MUL: returns the MXFP8 h as (codes [out_rows, N/2], scale bytes [out_rows, N/64]); with
    act_layout TILED the h buffers hold max_tiles * block_m rows (tile-blocked)."""
    _req(Aq, torch.uint8, "Aq")
    _req(Wq, torch.uint8, "Wq")
    E, N, K2 = Wq.shape
    K = 2 * K2
    dev = Aq.device
    if act_layout == MOE_ACT_TILED and epilogue == MOE_EPI_SILU_MUL:
        out_rows = max(out_rows, max(max_tiles, 1) * block_m)  # h is written tile-blocked
    if epilogue == MOE_EPI_SILU_MUL:
        if C is None:
            C = torch.empty((out_rows, N // 2), dtype=torch.uint8, device=dev)
        if Cs is None:
            Cs = torch.empty((out_rows, N // 64), dtype=torch.uint8, device=dev)
    elif C is None:
        C = torch.empty((out_rows, N), dtype=torch.float32 if out_dtype == MOE_OUT_F32 else torch.bfloat16, device=dev)
    _check(load().moe_grouped_gemm_w4a8(_p(Aq), _p(As), _p(a_row_of), a_row_div, _p(Wq), _p(We), weight_layout,
                                        act_layout, E, N, K, _p(tiles), max_tiles, _p(num_tiles), block_m, epilogue,
                                        _p(C), _p(Cs), out_dtype, _stream(stream)))
    return (C, Cs) if epilogue == MOE_EPI_SILU_MUL else C


def moe_ffn_w4a8_block_m(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load().moe_ffn_w4a8_block_m(T, H, I, E, k))


def moe_ffn_w4a8_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load().moe_ffn_w4a8_workspace_bytes(T, H, I, E, k))


def moe_ffn_forward_w4a8(x, router_logits, w13_q, w13_e, w2_q, w2_e, k: int, y=None, topk_ids_out=None,
                         topk_w_out=None, workspace=None, stream=None, weight_layout: int = MOE_LAYOUT_CANONICAL):
    """Whole W4A8 layer: x bf16 [T, H], logits fp32 [T, E], MXFP4 weights -> y bf16 [T, H]."""
    _req(x, "16bit", "x")
    T, H = x.shape
    E, N13, _ = w13_q.shape
    I = N13 // 2
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    wsb = moe_ffn_w4a8_workspace_bytes(T, H, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    _check(load().moe_ffn_forward_w4a8(_p(x), _p(router_logits), T, H, I, E, k, _p(w13_q), _p(w13_e), _p(w2_q),
                                       _p(w2_e), weight_layout, _p(y), _p(topk_ids_out), _p(topk_w_out), _p(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


# ---- FP8 (W8A8, per-1x128) -------------------------------------------------------------------------

def moe_f8_quantize(x, q=None, s=None, stream=None):
    """x bf16 or fp32 [rows, K] -> (E4M3 codes uint8 [rows, K], fp32 scales [rows, K/128])."""
    if x.dtype == torch.float32:
        in_dtype = MOE_IN_F32
    else:
        _req(x, "16bit", "x")
        in_dtype = MOE_IN_BF16
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous CUDA tensor")
    rows, K = x.shape
    if q is None:
        q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, K // 128), dtype=torch.float32, device=x.device)
    _check(load().moe_f8_quantize(_p(x), in_dtype, rows, K, _p(q), _p(s), _stream(stream)))
    return q, s


def moe_grouped_gemm_f8(Aq, As, a_row_of, a_row_div: int, Wq, Ws, tiles, max_tiles: int, num_tiles, block_m: int,
                        epilogue: int, out_rows: int, out_dtype: int = MOE_OUT_F32, C=None, Cs=None, stream=None):
    """Grouped FP8 GEMM over the tile list.  NONE: returns C [out_rows, N] (fp32 or bf16); SILU_MUL:
    returns h fp32 [out_rows, N/2], or with out_dtype MOE_OUT_F8 the quantized h as (codes uint8
    [out_rows, N/2], scales fp32 [out_rows, N/256])."""
    _req(Aq, torch.uint8, "Aq")
    _req(Wq, torch.uint8, "Wq")
    E, N, K = Wq.shape
    if out_dtype == MOE_OUT_F8:
        if C is None:
            C = torch.empty((out_rows, N // 2), dtype=torch.uint8, device=Aq.device)
        if Cs is None:
            Cs = torch.empty((out_rows, max(N // 256, 1)), dtype=torch.float32, device=Aq.device)
    elif C is None:
        cols = N // 2 if epilogue == MOE_EPI_SILU_MUL else N
        dt = torch.float32 if out_dtype == MOE_OUT_F32 else torch.bfloat16
        C = torch.empty((out_rows, cols), dtype=dt, device=Aq.device)
    _check(load().moe_grouped_gemm_f8(_p(Aq), _p(As), _p(a_row_of), a_row_div, _p(Wq), _p(Ws), E, N, K, _p(tiles),
                                      max_tiles, _p(num_tiles), block_m, epilogue, _p(C), _p(Cs), out_dtype,
                                      _stream(stream)))
    return (C, Cs) if out_dtype == MOE_OUT_F8 else C


def moe_ffn_f8_block_m(T: int, E: int, k: int) -> int:
    return int(load().moe_ffn_f8_block_m(T, E, k))


def moe_ffn_f8_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load().moe_ffn_f8_workspace_bytes(T, H, I, E, k))


def moe_ffn_forward_f8(x, router_logits, w13_q, w13_s, w2_q, w2_s, k: int, y=None, topk_ids_out=None,
                       topk_w_out=None, workspace=None, stream=None):
    """Whole FP8 (W8A8, per-1x128) layer: x bf16 [T, H], logits fp32 [T, E], E4M3 weights with fp32
    scales -> y bf16 [T, H]."""
    _req(x, "16bit", "x")
    T, H = x.shape
    E, N13, _ = w13_q.shape
    I = N13 // 2
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    wsb = moe_ffn_f8_workspace_bytes(T, H, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=x.device)
    _check(load().moe_ffn_forward_f8(_p(x), _p(router_logits), T, H, I, E, k, _p(w13_q), _p(w13_s), _p(w2_q),
                                     _p(w2_s), _p(y), _p(topk_ids_out), _p(topk_w_out), _p(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return y

