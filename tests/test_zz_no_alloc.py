"""GPU test of cconv_bwd_noalloc, the backward that keeps its dw/dbias partials in the
library's static scratch array instead of a caller workspace (for callers that cannot
allocate), through the C ABI.

Two calls in a row, the second with a smaller input (so it runs on what the first left in the
shared array): dx, dw and dbias must equal cconv_bwd's bit for bit, and the smaller call must
also match the oracle within the backward tolerance.
"""

from __future__ import annotations

import pytest
import torch

import causal_depthwise_short_amd as cc
import oracle
import synth_inputs as si
from parity import TOL_BWD, assert_close, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _compare(B, T, D, W, seed, dw_dtype):
    inp = si.train_inputs(B, T, D, W, bias=True, seed=seed)
    x, w, b, dy = (inp[k].to(DEV) for k in ("x", "w", "bias", "dy"))
    dx0, dw0, db0 = cc.cconv_bwd(x, dy, w, b, dw_dtype=dw_dtype)
    dx1 = torch.full_like(dx0, 7.0)
    dw1 = torch.full_like(dw0, 7.0)
    db1 = torch.full_like(db0, 7.0)
    cc.cconv_bwd_noalloc(x, dy, w, b, dx=dx1, dw=dw1, dbias=db1)
    torch.cuda.synchronize()
    what = f"B{B} T{T} D{D} W{W}"
    assert torch.equal(bits(dx1), bits(dx0)), f"{what}: dx differs from cconv_bwd"
    assert torch.equal(bits(dw1), bits(dw0)), f"{what}: dw differs from cconv_bwd"
    assert torch.equal(bits(db1), bits(db0)), f"{what}: dbias differs from cconv_bwd"
    return inp, dx1, dw1, db1


def test_noalloc_equals_cconv_bwd_two_calls():
    need_big = cc.cconv_bwd_workspace_bytes(8, 8192, 4096, 4)
    assert 0 < need_big <= cc.cconv_bwd_noalloc_max_workspace()
    # the headline shape (10.5 MB of partials), then a smaller ragged one with fp32 dw
    _compare(8, 8192, 4096, 4, seed=900, dw_dtype=torch.bfloat16)
    inp, dx, dw, db = _compare(3, 1000, 2000, 2, seed=901, dw_dtype=torch.float32)
    dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
    assert_close(dx, dxr, TOL_BWD, "dx")
    assert_close(dw, dwr, TOL_BWD, "dw")
    assert_close(db, dbr, TOL_BWD, "dbias")


def test_noalloc_rejects_an_oversized_problem():
    """A problem whose partials exceed the static array fails before anything is enqueued."""
    D, W = 1 << 20, 4
    assert cc.cconv_bwd_workspace_bytes(1, 64, D, W) > cc.cconv_bwd_noalloc_max_workspace()
    x = torch.zeros(1, 64, D, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(D, W, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    with pytest.raises(cc.CconvError, match="WORKSPACE"):
        cc.cconv_bwd_noalloc(x, x, w, None, dx=dx, dw=dw)
