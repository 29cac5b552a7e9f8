"""Shared test helpers: tensor conversion and the parity metric."""
import numpy as np
import torch

import synth


def bf16_dev(bits, device="cuda"):
    """uint16 bf16 bit array -> torch.bfloat16 device tensor (bit-identical)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def f32_dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to64(t):
    """Device tensor (bf16 / f32) -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def upcast(d):
    return synth.floats(d)


def rel_err(got, ref):
    """max |got - ref| / max |ref| (0 when both are identically zero)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


BF16_TOL = 2e-2
F32_TOL = 1e-4
