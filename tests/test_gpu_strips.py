"""GPU parity of the channel strips, through the C ABI.

The D/vec lane groups of a row are dealt to ceil(D / (64 vec)) strips in near-equal runs (strip
s takes groups floor(s L / n) .. floor((s+1) L / n) - 1), so that no strip holds only a handful
of lanes. Each channel is written by exactly one wave per row: a guard band around y and dx
stays untouched, and every output matches the oracle. Widths: 17 strips of 60-61 groups (D =
4100 on 8-byte rows, 4104, and 4098 on 4-byte rows, whose last 4-channel group overlaps the one
before), 3 strips of 43-44 groups (520), 33 strips of 62-63 groups (8200), and widths below one
strip (12; 6 with two overlapping groups).
"""

from __future__ import annotations

import pytest
import torch

import causal_depthwise_short_amd as cc
import oracle
import synth_inputs as si
from parity import TOL_BWD, TOL_FWD, assert_close, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 64  # guard elements on each side (128 bytes: the outputs keep their alignment)


@pytest.mark.parametrize("D", [4100, 4104, 4098, 520, 8200, 1032, 12, 6])
def test_balanced_strips_write_each_channel_once(D):
    B, T, W = 2, 300, 4
    inp = si.train_inputs(B, T, D, W, bias=True, seed=360 + D)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    n = B * T * D
    yb = torch.full((n + 2 * PAD,), 1536.0, dtype=torch.bfloat16, device=DEV)
    dxb = torch.full((n + 2 * PAD,), -768.0, dtype=torch.bfloat16, device=DEV)
    y = yb[PAD : PAD + n].view(B, T, D)
    dx = dxb[PAD : PAD + n].view(B, T, D)
    cc.cconv_fwd(g["x"], g["w"], g["bias"], y=y)
    _, dw, db = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], dx=dx)
    torch.cuda.synchronize()
    for buf, v in ((yb, 1536.0), (dxb, -768.0)):
        assert bool((buf[:PAD].float() == v).all()) and bool((buf[PAD + n :].float() == v).all()), "guard band written"
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
    ey = assert_close(y.cpu(), yr, TOL_FWD, f"D{D} y")
    edx = assert_close(dx.cpu(), dxr, TOL_BWD, f"D{D} dx")
    edw = assert_close(dw.cpu(), dwr, TOL_BWD, f"D{D} dw")
    edb = assert_close(db.cpu(), dbr, TOL_BWD, f"D{D} dbias")
    print(f"D{D}: err y {ey:.2e} dx {edx:.2e} dw {edw:.2e} dbias {edb:.2e}", flush=True)


@pytest.mark.parametrize("D", [4100, 4104])
def test_strip_blocks_over_balanced_strips(D):
    """Blocks holding several strips (the general kernel, 2 and 4 strips per block, the last
    block partly past the 17th strip) give y and dx bit for bit equal to one-strip blocks."""
    B, T, W = 3, 257, 3
    inp = si.train_inputs(B, T, D, W, bias=True, seed=370 + D)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    y0 = cc.cconv_fwd(g["x"], g["w"], g["bias"])
    dx0, _, _ = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"])
    for ws in (2, 4):
        c = cc.Config(vec=4, rows_per_group=8, waves_per_block=2 * ws, strips_per_block=ws, options=3, seg_rows=64)
        y = cc.cconv_fwd(g["x"], g["w"], g["bias"], config=c)
        dx, dw, db = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], config=c)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y0)) and torch.equal(bits(dx), bits(dx0)), ws
        dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
        assert_close(dw.cpu(), dwr, TOL_BWD, f"D{D} ws{ws} dw")
        assert_close(db.cpu(), dbr, TOL_BWD, f"D{D} ws{ws} dbias")
