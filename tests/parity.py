"""Shared helpers for the GPU parity tests: tolerance, conversions, canary buffers.

Tolerance (reading of the stated budgets, which are given for bf16 outputs): for every
element, |gpu - ref| / max(1, |ref|) where ref is the oracle's unrounded float64 value and gpu
is the kernel's output widened exactly. Forward and decode y: 5e-3. dx, dw, dbias: 8e-3.
Rounding a value to bf16 alone costs up to 2^-8 = 3.9e-3 of it, so the bound leaves room for
fp32 arithmetic and the sigmoid's error, and nothing more.

Because that bound is mostly the rounding step, every comparison also checks what fp32
arithmetic followed by one round-to-nearest-even can give, element by element:
  * bf16 outputs: at most 1 bf16 ulp from the oracle's value rounded to bf16 (RTNE from
    float64, the oracle's own rounding). Elements that are not within 1 ulp must be within an
    absolute floor instead: 2^-18 for element-wise outputs (y, dx, decode y, history
    gradients), where a z or a dx that cancels to near zero has an fp32 error of a few 2^-24
    times its terms, larger than the ulp of so small a value; 1e-5 times the largest |ref|
    for the long sums dw and dbias;
  * fp32 dw and dbias (long sums), compared as tensors of at least 64 sums: max |gpu - ref|
    <= 1e-5 * max |ref| and the normalized RMS ||gpu - ref||_2 / ||ref||_2 <= 1e-5. The error of
    an fp32 sum scales with the size of its terms, which the largest |ref| of many sums
    reflects; a lone sum whose terms cancel can lose more of its own digits (1.1e-5 of itself
    measured for one channel), so a handful of sums is held to the relative budget only.
A dropped term, a wrong tap or an error of the sigmoid beyond a few fp32 ulps fails these even
where it stays inside the relative budget.
"""

from __future__ import annotations

import re

import numpy as np
import torch

TOL_FWD = 5e-3
TOL_BWD = 8e-3
ULP_FLOOR = 2.0**-18  # element-wise bf16 outputs: absolute error allowed where 1 ulp is smaller
SUM_REL = 1e-5  # dw, dbias: error relative to the largest |ref|, and normalized RMS
CANARY = 0x7FA5  # a NaN pattern no kernel writes (outputs of finite inputs are finite)
_REDUCTION = re.compile(r"\b(dw|dbias)\b")


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


def _ordered(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers in value order (ulp distance = difference)."""
    b = b.astype(np.int32) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_stats(gpu: torch.Tensor, ref, floor: float):
    """(max ulp distance, number of elements further than 1 ulp) between a bf16 tensor and the
    float64 reference rounded to bf16 by the oracle; elements within `floor` of ref count as
    0 ulps."""
    import oracle

    g = bits(gpu).numpy().view(np.uint16).reshape(-1)
    r = np.ascontiguousarray(as_f64(ref)).reshape(-1)
    rb = oracle.round_bf16(r)
    d = np.abs(_ordered(g) - _ordered(rb))
    near = np.abs(as_f64(gpu).reshape(-1) - r) <= floor
    d = np.where(near, 0, d)
    return (int(d.max()) if d.size else 0), int(np.count_nonzero(d > 1))


def sum_errors(gpu, ref):
    """(max |gpu - ref| / max |ref|, ||gpu - ref||_2 / ||ref||_2) for fp32 sums."""
    g, r = as_f64(gpu).reshape(-1), as_f64(ref).reshape(-1)
    if g.size == 0:
        return 0.0, 0.0
    scale = max(float(np.max(np.abs(r))), 1e-30)
    norm = max(float(np.linalg.norm(r)), 1e-30)
    return float(np.max(np.abs(g - r))) / scale, float(np.linalg.norm(g - r)) / norm


def assert_close(gpu, ref, tol, what):
    """The relative budget, plus the element-wise checks of the module docstring. `what` names
    the output; names containing dw or dbias are the long sums."""
    e = rel_err(gpu, ref)
    assert e <= tol, f"{what}: max |gpu-ref|/max(1,|ref|) = {e:.3e} > {tol:.1e}"
    if as_f64(ref).size == 0:
        return e
    reduction = bool(_REDUCTION.search(what))
    if isinstance(gpu, torch.Tensor) and gpu.dtype == torch.bfloat16:
        floor = SUM_REL * float(np.max(np.abs(as_f64(ref)))) if reduction else ULP_FLOOR
        mu, nbad = bf16_ulp_stats(gpu, ref, floor)
        assert nbad == 0, f"{what}: {nbad} elements more than 1 bf16 ulp from RTNE(oracle) (max {mu} ulps)"
    elif isinstance(gpu, torch.Tensor) and gpu.dtype == torch.float32 and reduction and gpu.numel() >= 64:
        mx, nr = sum_errors(gpu, ref)
        assert mx <= SUM_REL and nr <= SUM_REL, f"{what}: fp32 sum error {mx:.2e} of max |ref|, normalized RMS {nr:.2e}"
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
