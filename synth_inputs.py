"""Seeded synthetic inputs for the depthwise causal short convolution + SiLU.

This module draws random tensors and nothing else: it holds none of the operation's
arithmetic, so both the CPU oracle (under ``oracle/``) and the HIP path may take their
inputs from it without sharing any of the computation.

Recipe (the same for every workload):
  * a CPU ``torch.Generator`` seeded per workload;
  * tensors drawn in a fixed order (training: x, w, bias, dy; decode: x, state, slot
    permutation, w, bias); a training history (state before t = 0) from a second generator;
  * every draw is fp32 ``N(0, var)`` scaled by ``sqrt(var)`` and, where the tensor is bf16,
    rounded to bf16 by torch's round-to-nearest-even cast. The bf16 bits that result are
    what both sides receive.

The variances follow the workloads the kernel-fun wheel page describes for this op
(``cconv/__init__.py`` docstring: B=16, T=8192, D=2048, W=4 production call; D a multiple
of n_heads*128): x and dy ~ N(0, 1), taps ~ N(0, 1/W) so that Var z is about 1, bias ~
N(0, 0.1). The decode workload follows the cudnn-frontend PR #797 "Add experimental causal
conv1d decode update" description (state ``[S, D, W-1]``, ``state_indices`` drawn without
repeats).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class TrainShape:
    """A fwd+bwd workload: x, dy are bf16 [B, T, D]; w is [D, W]; bias fp32 [D] or absent."""

    name: str
    B: int
    T: int
    D: int
    W: int
    bias: bool
    seed: int


@dataclass(frozen=True)
class DecodeShape:
    """A one-token decode workload: x bf16 [N, D], state bf16 [S, D, W-1], indices [N]."""

    name: str
    N: int
    S: int
    D: int
    W: int
    bias: bool
    seed: int


# The five workloads this implementation is checked and measured on.
TINY = TrainShape("B1_T256_D512_W4_bias", 1, 256, 512, 4, True, 0)
MEDIUM = TrainShape("B8_T1024_D4096_W4_nobias", 8, 1024, 4096, 4, False, 1)
HEADLINE = TrainShape("B8_T8192_D4096_W4_bias", 8, 8192, 4096, 4, True, 2)
RAGGED = TrainShape("B3_T1000_D2000_W2_bias", 3, 1000, 2000, 2, True, 3)
DECODE = DecodeShape("decode_N256_S512_D4096_W4_bias", 256, 512, 4096, 4, True, 4)
# the production call the kernel-fun wheel's cconv/__init__.py docstring measures (the
# headline's element count): a parity case, not a bench line
PRODUCTION = TrainShape("B16_T8192_D2048_W4_bias", 16, 8192, 2048, 4, True, 5)

TRAIN_SHAPES = (TINY, MEDIUM, HEADLINE, RAGGED)


def _normal(g: torch.Generator, shape, var: float) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32) * math.sqrt(var)


def train_inputs(
    B: int,
    T: int,
    D: int,
    W: int,
    *,
    bias: bool,
    seed: int,
    w_dtype: torch.dtype = torch.bfloat16,
    x_var: float = 1.0,
) -> dict:
    """Host tensors for one fwd+bwd call: x, w, bias (or None), dy.

    x, dy: bf16 [B, T, D] contiguous. w: [D, W] in ``w_dtype`` (bf16 or fp32), variance 1/W.
    bias: fp32 [D], variance 0.1, or None.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = _normal(g, (B, T, D), x_var).to(torch.bfloat16)
    w = _normal(g, (D, W), 1.0 / W).to(w_dtype)
    b = _normal(g, (D,), 0.1) if bias else None
    dy = _normal(g, (B, T, D), 1.0).to(torch.bfloat16)
    return {"x": x, "w": w, "bias": b, "dy": dy}


def train_inputs_for(shape: TrainShape, **kw) -> dict:
    return train_inputs(shape.B, shape.T, shape.D, shape.W, bias=shape.bias, seed=shape.seed, **kw)


def history_input(B: int, D: int, W: int, *, seed: int) -> torch.Tensor:
    """A history before t = 0 for each sequence: bf16 [B, D, W-1] ~ N(0, 1), oldest first (the
    decode state layout). Drawn from its own generator (seed + 1000) so that the training draws
    of the same seed are unchanged."""
    g = torch.Generator(device="cpu").manual_seed(seed + 1000)
    return _normal(g, (B, D, W - 1), 1.0).to(torch.bfloat16)


def decode_inputs(
    N: int,
    S: int,
    D: int,
    W: int,
    *,
    bias: bool,
    seed: int,
    w_dtype: torch.dtype = torch.bfloat16,
    identity: bool = False,
) -> dict:
    """Host tensors for one decode update: x, state, state_indices, w, bias.

    x: bf16 [N, D]; state: bf16 [S, D, W-1]; state_indices: int32 [N], the first N entries of
    a random permutation of range(S) (distinct, all valid), or None when ``identity``.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = _normal(g, (N, D), 1.0).to(torch.bfloat16)
    state = _normal(g, (S, D, W - 1), 1.0).to(torch.bfloat16)
    perm = torch.randperm(S, generator=g)[:N].to(torch.int32)
    w = _normal(g, (D, W), 1.0 / W).to(w_dtype)
    b = _normal(g, (D,), 0.1) if bias else None
    return {"x": x, "state": state, "state_indices": None if identity else perm, "w": w, "bias": b}


def decode_inputs_for(shape: DecodeShape, **kw) -> dict:
    return decode_inputs(shape.N, shape.S, shape.D, shape.W, bias=shape.bias, seed=shape.seed, **kw)


def train_inputs_device(
    B: int, T: int, D: int, W: int, *, bias: bool, seed: int, device: str = "cuda"
) -> dict:
    """The same recipe as train_inputs, drawn by a seeded generator on the device (for sizes
    whose host copies would be impractical). Values differ from train_inputs' for the same
    seed; both sides still see identical bits, since host windows are copied from these."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = (torch.randn(B, T, D, generator=g, device=device, dtype=torch.float32)).to(torch.bfloat16)
    w = (torch.randn(D, W, generator=g, device=device, dtype=torch.float32) * math.sqrt(1.0 / W)).to(torch.bfloat16)
    b = torch.randn(D, generator=g, device=device, dtype=torch.float32) * math.sqrt(0.1) if bias else None
    dy = torch.randn(B, T, D, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return {"x": x, "w": w, "bias": b, "dy": dy}


def packed_lengths(total: int, *, seed: int, max_len: int = 16384) -> list:
    """Sequence lengths for a packed batch of ``total`` rows: log-uniform on [1, max_len]
    (many short sequences, a few long ones), drawn until the rows are used up, the last one
    cut to fit. The pages' packed batches give no length distribution; this mix covers
    single-token sequences and ones longer than a wave's segment."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    lens, used = [], 0
    while used < total:
        u = float(torch.rand(1, generator=g))
        n = max(1, min(max_len, int(round(math.exp(u * math.log(max_len))))))
        n = min(n, total - used)
        lens.append(n)
        used += n
    return lens
