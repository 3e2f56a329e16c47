"""Shared helpers for the GPU parity tests: tensor marshalling, the layer
runner, and the acceptance rule.

Acceptance for bf16 outputs (floating point): elementwise
    |y - y_ref| <= half a bf16 ulp of y_ref + 2e-3 * max|y_ref|.
The 2e-3 relative bound is the stated output tolerance for bf16 I/O with fp32
accumulation; the half-ulp term is the unavoidable final rounding of a bf16
output (a correctly rounded bf16 result of the exact value alone reaches
2e-3 .. 3.4e-3 of max|y| on these layers, so the bare ratio cannot be met by
any bf16-output implementation).  Integer and byte results are compared
bit-exactly.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 2e-3


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def half_ulp_bf16(a):
    a = np.abs(np.asarray(a, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (np.maximum(e, -126) - 8).astype(np.int64)), 0.0)


def check_bf16_output(y_bits, y_ref, rel_tol=REL_TOL):
    """Returns (ok, stats) for a bf16 output against a float64 reference."""
    y = bf16_bits_to_f64(y_bits)
    y_ref = np.asarray(y_ref, np.float64)
    m = float(np.abs(y_ref).max()) if y_ref.size else 0.0
    err = np.abs(y - y_ref)
    bound = half_ulp_bf16(y_ref) + rel_tol * m
    ok = bool(np.all(err <= bound)) and bool(np.all(np.isfinite(y)))
    stats = {
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "literal_ratio": float(err.max() / m) if m > 0 else 0.0,
        "excess": float((err - bound).max()) if err.size else 0.0,
    }
    return ok, stats


# ------------------------------------------------------------ torch plumbing
def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(device).view(
        torch.bfloat16)


def to_dev_f32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def to_dev_u32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).to(device)


def to_dev_u16(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(device)


def from_dev_u16(t):
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def from_dev_u32(t):
    return t.cpu().numpy().view(np.uint32)
