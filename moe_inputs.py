"""Seeded synthetic inputs for the MoE W4A16 layer (shared by the product, the tests and the oracle).

This module holds input generation only: it draws random numbers and packs them into the storage
formats the layer consumes. It contains none of the layer's arithmetic (no decoding, no routing, no
matmul), so the CPU oracle and the HIP path can both use it without sharing any computation.

Workloads stand in for the shapes the pages name: the Qwen3-Next shape of 800 tokens over 256 experts
(page "告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM", section "编译时内核选择和W4A16
Grouped GEMM"), a Qwen3-MoE-like 128-expert top-8 decode shape and a Mixtral-like 8-expert top-2
shape (page "AMD ATOM推理引擎…", model table). No model weights are used.

Draw order with ``numpy.random.default_rng(seed)``:
  1. x       = standard_normal((T, H), float32), rounded to bf16 (round-to-nearest-even)
  2. logits  = standard_normal((T, E), float32)   (+ a per-expert Zipf-like bias for the skewed workload)
  3. w13_q   = integers(0, 256, (E, 2I, H/2), uint8)   two E2M1 codes per byte, even K index in the low nibble
  4. w13_s   = uniform(0.005, 0.02, (E, 2I, H/32)) -> float32 -> bf16 (RNE)
  5. w2_q    = integers(0, 256, (E, H, I/2), uint8)
  6. w2_s    = uniform(0.005, 0.02, (E, H, I/32)) -> float32 -> bf16 (RNE)
bf16 values are carried as uint16 bit patterns.

The router gate and the shared expert (``make_block_inputs``) come from a second generator,
``default_rng(seed + 1000)``, so the draws above are unchanged; in order:
  1. w_router = standard_normal((E, H), float32) / sqrt(H), rounded to bf16 (x @ w_router^T is then
     about N(0, 1), the router-logit distribution of the workloads)
  2. w13s_q, 3. w13s_s, 4. w2s_q, 5. w2s_s: one expert of intermediate size Is in the same W4 format
     and distributions as the routed experts.

The MXFP4 variant (``make_mx_inputs``) draws with ``default_rng(seed)`` in the order above, so x,
logits and the codes are those of the W4A16 inputs at the same seed; its scales are E8M0 bytes: each
uniform(0.005, 0.02) draw u becomes 127 + rint(log2(u)) (the nearest power of two in log scale,
2^-8 .. 2^-6).

The FP8 variant (``make_f8_inputs``) draws with ``default_rng(seed)`` in the same order (x and logits
are those of the W4A16 inputs at the same seed), with one byte per weight element and one fp32 scale
per 128 K elements:
  3. w13_q [E, 2I, H]: E4M3 codes drawn field by field, in this order: sign bits integers(0, 2),
     exponent field 15 - min(geometric(0.5) - 1, 15) (half the codes in the top binade, a quarter in
     the next, ..., the shape of amax-scaled near-Gaussian weights rather than a log-uniform spread),
     mantissa integers(0, 8); the NaN pattern (exponent 15, mantissa 7) becomes mantissa 6 (448)
  4. w13_s = uniform(0.005, 0.02, (E, 2I, H/128)) / 128 as float32 (the 2^-7 keeps weights near the
     W4 layer's rms, about 0.03, while the codes reach 448)
  5. w2_q, 6. w2_s likewise for (E, H, I) and (E, H, I/128).
"""
from __future__ import annotations

import dataclasses

import numpy as np

GROUP = 32  # K elements per bf16 scale


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    skew: bool = False
    seed: int = 0


# The workloads: tiny parity case, decode batches, the 800-token/256-expert prefill shape,
# the large-expert prefill shape and the skewed-routing shape.
WORKLOADS = {
    "tiny": Workload("tiny", 16, 8, 2, 256, 128),
    "dec1": Workload("dec1", 1, 128, 8, 2048, 768),
    "dec8": Workload("dec8", 8, 128, 8, 2048, 768),
    "dec32": Workload("dec32", 32, 128, 8, 2048, 768),
    "dec64": Workload("dec64", 64, 128, 8, 2048, 768),
    "pre800": Workload("pre800", 800, 256, 8, 2048, 512),
    "big4096": Workload("big4096", 4096, 8, 2, 4096, 14336),
    "skew8192": Workload("skew8192", 8192, 512, 10, 2048, 512, skew=True),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def skew_bias(E: int) -> np.ndarray:
    """Per-expert Zipf-like logit bias b_e = 2*ln(1/rank_e^1.2), rank_e = e+1, float64 then float32."""
    rank = np.arange(1, E + 1, dtype=np.float64)
    return (2.0 * np.log(1.0 / rank ** 1.2)).astype(np.float32)


@dataclasses.dataclass
class MoEInputs:
    wl: Workload
    x: np.ndarray        # uint16 [T, H]      bf16 bits
    logits: np.ndarray   # float32 [T, E]
    w13_q: np.ndarray    # uint8  [E, 2I, H/2]
    w13_s: np.ndarray    # uint16 [E, 2I, H/32] bf16 bits
    w2_q: np.ndarray     # uint8  [E, H, I/2]
    w2_s: np.ndarray     # uint16 [E, H, I/32]  bf16 bits


def make_inputs(wl: Workload, seed: int | None = None) -> MoEInputs:
    """Draw one workload's inputs in the documented order."""
    T, E, H, I = wl.T, wl.E, wl.H, wl.I
    if H % GROUP or I % GROUP:
        raise ValueError("H and I must be multiples of 32")
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if wl.skew:
        logits = (logits + skew_bias(E)[None, :]).astype(np.float32)
    w13_q = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13_s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, 2 * I, H // GROUP)).astype(np.float32))
    w2_q = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2_s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, H, I // GROUP)).astype(np.float32))
    return MoEInputs(wl, x, logits, w13_q, w13_s, w2_q, w2_s)


def custom(name: str, T: int, E: int, k: int, H: int, I: int, skew: bool = False, seed: int = 0) -> Workload:
    return Workload(name, T, E, k, H, I, skew, seed)


def weight_bytes_per_expert(H: int, I: int) -> int:
    """Packed 4-bit codes plus bf16 group scales of one expert's gate_up and down weights."""
    return 2 * I * H // 2 + 2 * I * (H // GROUP) * 2 + H * I // 2 + H * (I // GROUP) * 2


@dataclasses.dataclass(frozen=True)
class BlockInputs:
    """Router gate weight and shared expert for the whole MoE block (routed experts in MoEInputs)."""
    w_router: np.ndarray  # uint16 [E, H] bf16 bits
    w13s_q: np.ndarray    # uint8  [2Is, H/2]
    w13s_s: np.ndarray    # uint16 [2Is, H/32] bf16 bits
    w2s_q: np.ndarray     # uint8  [H, Is/2]
    w2s_s: np.ndarray     # uint16 [H, Is/32] bf16 bits


def make_block_inputs(wl: Workload, Is: int, seed: int | None = None) -> BlockInputs:
    """Draw the router gate weight and a shared expert of intermediate size Is (documented order)."""
    E, H = wl.E, wl.H
    if Is % GROUP:
        raise ValueError("Is must be a multiple of 32")
    rng = np.random.default_rng((wl.seed if seed is None else seed) + 1000)
    w_router = f32_to_bf16_bits((rng.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H))))
    w13s_q = rng.integers(0, 256, (2 * Is, H // 2), dtype=np.uint8)
    w13s_s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, (2 * Is, H // GROUP)).astype(np.float32))
    w2s_q = rng.integers(0, 256, (H, Is // 2), dtype=np.uint8)
    w2s_s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, (H, Is // GROUP)).astype(np.float32))
    return BlockInputs(w_router, w13s_q, w13s_s, w2s_q, w2s_s)


@dataclasses.dataclass
class MXInputs:
    """Inputs of the MXFP4 (W4A4) variant: same x, logits and codes, E8M0 scale bytes."""
    wl: Workload
    x: np.ndarray        # uint16 [T, H] bf16 bits
    logits: np.ndarray   # float32 [T, E]
    w13_q: np.ndarray    # uint8  [E, 2I, H/2]
    w13_e: np.ndarray    # uint8  [E, 2I, H/32] E8M0
    w2_q: np.ndarray     # uint8  [E, H, I/2]
    w2_e: np.ndarray     # uint8  [E, H, I/32]  E8M0


def e8m0_from_uniform(u: np.ndarray) -> np.ndarray:
    """Scale draws -> E8M0 bytes of the nearest power of two in log scale."""
    return (127 + np.rint(np.log2(u))).astype(np.uint8)


def make_mx_inputs(wl: Workload, seed: int | None = None) -> MXInputs:
    """Draw one workload's MXFP4 inputs (the W4A16 draw order, scales as E8M0 bytes)."""
    T, E, H, I = wl.T, wl.E, wl.H, wl.I
    if H % GROUP or I % GROUP:
        raise ValueError("H and I must be multiples of 32")
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if wl.skew:
        logits = (logits + skew_bias(E)[None, :]).astype(np.float32)
    w13_q = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13_e = e8m0_from_uniform(rng.uniform(0.005, 0.02, (E, 2 * I, H // GROUP)))
    w2_q = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2_e = e8m0_from_uniform(rng.uniform(0.005, 0.02, (E, H, I // GROUP)))
    return MXInputs(wl, x, logits, w13_q, w13_e, w2_q, w2_e)


def mx_weight_bytes_per_expert(H: int, I: int) -> int:
    """E2M1 codes plus E8M0 scales of one expert's gate_up and down weights."""
    return 2 * I * H // 2 + 2 * I * (H // GROUP) + H * I // 2 + H * (I // GROUP)


F8_BLOCK = 128  # K elements per FP8 scale


@dataclasses.dataclass
class F8Inputs:
    """Inputs of the FP8 (W8A8, per-1x128) variant: same x and logits, E4M3 codes, fp32 scales."""
    wl: Workload
    x: np.ndarray        # uint16  [T, H] bf16 bits
    logits: np.ndarray   # float32 [T, E]
    w13_q: np.ndarray    # uint8   [E, 2I, H]     E4M3 codes
    w13_s: np.ndarray    # float32 [E, 2I, H/128]
    w2_q: np.ndarray     # uint8   [E, H, I]      E4M3 codes
    w2_s: np.ndarray     # float32 [E, H, I/128]


def e4m3_codes(rng, shape) -> np.ndarray:
    """E4M3 codes: uniform sign, exponent field 15 - min(geometric(1/2) - 1, 15), uniform mantissa;
    the NaN pattern (exponent 15, mantissa 7) moved to the largest finite magnitude."""
    sign = rng.integers(0, 2, shape, dtype=np.uint8)
    expo = (15 - np.minimum(rng.geometric(0.5, shape) - 1, 15)).astype(np.uint8)
    mant = rng.integers(0, 8, shape, dtype=np.uint8)
    q = (sign << 7) | (expo << 3) | mant
    q[(q & 0x7F) == 0x7F] -= 1
    return q


def e4m3_codes_uniform(rng, shape) -> np.ndarray:
    """Every finite E4M3 code equally likely (log-uniform magnitudes 2^-9 .. 448): uniform bytes with
    the two NaN codes moved to the largest finite magnitude.  For tests of the full code range."""
    q = rng.integers(0, 256, shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] -= 1
    return q


def make_f8_inputs(wl: Workload, seed: int | None = None) -> F8Inputs:
    """Draw one workload's FP8 inputs (documented order)."""
    T, E, H, I = wl.T, wl.E, wl.H, wl.I
    if H % F8_BLOCK or I % F8_BLOCK:
        raise ValueError("H and I must be multiples of 128 for the FP8 variant")
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if wl.skew:
        logits = (logits + skew_bias(E)[None, :]).astype(np.float32)
    w13_q = e4m3_codes(rng, (E, 2 * I, H))
    w13_s = (rng.uniform(0.005, 0.02, (E, 2 * I, H // F8_BLOCK)) / 128.0).astype(np.float32)
    w2_q = e4m3_codes(rng, (E, H, I))
    w2_s = (rng.uniform(0.005, 0.02, (E, H, I // F8_BLOCK)) / 128.0).astype(np.float32)
    return F8Inputs(wl, x, logits, w13_q, w13_s, w2_q, w2_s)


def f8_weight_bytes_per_expert(H: int, I: int) -> int:
    """E4M3 codes plus fp32 per-1x128 scales of one expert's gate_up and down weights."""
    return 2 * I * H + 2 * I * (H // F8_BLOCK) * 4 + H * I + H * (I // F8_BLOCK) * 4
