"""Shared helpers for the GPU parity tests: tolerance, conversions, canary buffers.

Tolerance (reading of the stated budgets, which are given for bf16 outputs): for every
element, |gpu - ref| / max(1, |ref|) where ref is the oracle's unrounded float64 value and gpu
is the kernel's output widened exactly. Forward and decode y: 5e-3. dx, dw, dbias: 8e-3.
Rounding a value to bf16 alone costs up to 2^-8 = 3.9e-3 of it, so the bound leaves room for
fp32 arithmetic and the sigmoid's error, and nothing more.
"""

from __future__ import annotations

import numpy as np
import torch

TOL_FWD = 5e-3
TOL_BWD = 8e-3
CANARY = 0x7FA5  # a NaN pattern no kernel writes (outputs of finite inputs are finite)


def as_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def rel_err(gpu, ref) -> float:
    g, r = as_f64(gpu), as_f64(ref)
    assert g.shape == r.shape, f"{g.shape} vs {r.shape}"
    if g.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r))))


def assert_close(gpu, ref, tol, what):
    e = rel_err(gpu, ref)
    assert e <= tol, f"{what}: max |gpu-ref|/max(1,|ref|) = {e:.3e} > {tol:.1e}"
    return e


def bits(t: torch.Tensor) -> torch.Tensor:
    """The raw bit patterns of a tensor (for bitwise comparisons)."""
    t = t.detach().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.view(torch.int16).cpu()
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32).cpu()
    return t.cpu()


def guarded(shape, dtype, device, margin=64):
    """A tensor of `shape` placed in the middle of a canary-filled buffer; returns (view, buffer, lo, hi)."""
    n = int(np.prod(shape)) if len(shape) else 1
    esz = torch.tensor([], dtype=dtype).element_size()
    m = margin * 16 // esz  # keep 16-byte alignment of the view
    buf = torch.empty(n + 2 * m, dtype=dtype, device=device)
    if dtype == torch.bfloat16:
        buf.view(torch.int16).fill_(CANARY)
    else:
        buf.view(torch.int32).fill_(0x7FA5A5A5)
    view = buf[m : m + n].view(shape)
    return view, buf, m, m + n


def canaries_intact(buf, lo, hi) -> bool:
    b = bits(buf)
    return _all_canary(b[:lo], buf.dtype) and _all_canary(b[hi:], buf.dtype)


def _all_canary(b, dtype) -> bool:
    if b.numel() == 0:
        return True
    want = CANARY if dtype == torch.bfloat16 else 0x7FA5A5A5
    return bool((b == want).all())
