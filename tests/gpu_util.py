"""Helpers for the GPU tests: move seeded inputs to the device and results back, and the tolerance
check of the layer output against the fp64 oracle."""
import numpy as np
import torch

import moe_inputs as mi

# Layer-output tolerance: max|gpu - ref| <= 3e-2 * rms(ref) and sum|gpu - ref| / sum|ref| <= 5e-3.
MAX_ABS_OVER_RMS = 3e-2
MEAN_REL = 5e-3
# Routing weights are fp32 on the GPU and fp64 in the oracle; both lie in [0, 1].
ROUTE_W_ATOL = 1e-6


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return mi.bf16_bits_to_f32(bits).astype(np.float64)


class DeviceInputs:
    def __init__(self, inp: "mi.MoEInputs"):
        self.inp = inp
        self.x = dev_bf16(inp.x)
        self.logits = dev(inp.logits)
        self.w13_q = dev(inp.w13_q)
        self.w13_s = dev(inp.w13_s.view(np.int16))
        self.w2_q = dev(inp.w2_q)
        self.w2_s = dev(inp.w2_s.view(np.int16))


def tolerance_report(y: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(y - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return dict(max_over_rms=float(d.max() / rms), mean_rel=float(d.sum() / np.abs(ref).sum()),
                norm_ratio=float(np.linalg.norm(y) / np.linalg.norm(ref)), rms=rms)


def assert_within_tolerance(y: np.ndarray, ref: np.ndarray, label: str = ""):
    assert np.all(np.isfinite(y)), f"{label}: non-finite output"
    r = tolerance_report(y, ref)
    assert r["max_over_rms"] <= MAX_ABS_OVER_RMS and r["mean_rel"] <= MEAN_REL, f"{label}: {r}"
    return r


def sample_tokens(T: int, n: int, ids=None, per_expert: int = 2, seed: int = 99) -> np.ndarray:
    """Token indices to check against the oracle at full size (each token's output is independent):
    the first 8 and the last token, up to `per_expert` tokens routed to each touched expert (when the
    routing ids [T, k] are given, so that every touched expert's rows appear, the rarely chosen ones
    included), then random tokens up to n in all.  All tokens when T <= n."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    chosen = set(range(min(8, T))) | {T - 1}
    if ids is not None:
        flat_t = np.repeat(np.arange(T), ids.shape[1])
        flat_e = ids.reshape(-1)
        for e in np.unique(flat_e):
            toks = np.unique(flat_t[flat_e == e])
            chosen.update(rng.choice(toks, min(per_expert, len(toks)), replace=False).tolist())
    rest = np.setdiff1d(np.arange(T), np.fromiter(chosen, np.int64))
    extra = max(0, n - len(chosen))
    if extra:
        chosen.update(rng.choice(rest, min(extra, len(rest)), replace=False).tolist())
    return np.array(sorted(chosen), np.int64)
