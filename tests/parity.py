"""Shared helpers of the GPU parity tests: host<->device transfer and the
acceptance bounds.

Bounds (f64 oracle values y_ref, a_ref = sum_k |x_k w_k|):
  * f32 output : |y - y_ref| <= 1e-3 * a_ref + 1e-5
  * f16 output : |y - y_ref| <= 2e-3 * |y_ref| + 1e-3 * a_ref + 1e-5
                 (relative 2e-3 for the f16 rounding, which alone is at most
                 2^-11 relative, plus the f32 accumulation allowance; a purely
                 relative bound cannot hold near y_ref = 0)
  * FFN h (f16): |h - h_ref| <= 2e-3 |h_ref| + 1.1 |u_ref| tol_g
                 + |silu(g_ref)| tol_u + 1.1 tol_g tol_u + 1e-5,
                 tol_x = 1e-3 a_x + 1e-5 and 1.1 >= max |silu'| (~1.0998)
  * integer / byte / index results: exact.
"""
from __future__ import annotations

import numpy as np
import torch


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.float16)).cuda()


def dev_u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f16_as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float64)


def tol_f32(a_ref):
    return 1e-3 * np.asarray(a_ref) + 1e-5


def tol_f16(y_ref, a_ref):
    return 2e-3 * np.abs(y_ref) + 1e-3 * np.asarray(a_ref) + 1e-5


def tol_ffn(ref: dict):
    tg, tu = tol_f32(ref["ag"]), tol_f32(ref["au"])
    silu_g = ref["g"] / (1.0 + np.exp(-ref["g"]))
    return (2e-3 * np.abs(ref["h"]) + 1.1 * np.abs(ref["u"]) * tg + np.abs(silu_g) * tu
            + 1.1 * tg * tu + 1e-5)


def assert_within(got, ref, tol, what: str):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (
        f"{what}: {bad.size} of {got.size} outside tolerance; first {bad[:5].tolist()}: "
        f"got {got[bad[:5]].tolist()} ref {np.asarray(ref)[bad[:5]].tolist()} "
        f"tol {np.asarray(tol)[bad[:5]].tolist()}")
    return float(np.max(err / tol)) if got.size else 0.0


def argmax_ok(idx: int, y_ref, a_ref, idx_ref: int) -> bool:
    """The index is right, or the oracle's gap between the two is within
    their combined tolerance (several answers are then correct)."""
    if idx == idx_ref:
        return True
    if not (0 <= idx < len(y_ref)):
        return False
    t = tol_f32(a_ref)
    return y_ref[idx_ref] - y_ref[idx] <= t[idx_ref] + t[idx]
