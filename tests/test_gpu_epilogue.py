"""GPU parity of the epilogue variants (no activation; a residual added after the activation)
through cconv_fwd_ex / cconv_bwd_ex, alone and combined with a history and with packed
batches, against the oracle's oracle_fwd_epi / oracle_bwd_epi.

Tolerances in parity.py. The default options must reproduce the plain entry points bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import causal_depthwise_short_amd as cc
import oracle
import synth_inputs as si
from parity import TOL_BWD, TOL_FWD, assert_close, bits, canaries_intact, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _g(t):
    return None if t is None else t.to(DEV)


def _case(B, T, D, W, *, seed, history, residual):
    inp = si.train_inputs(B, T, D, W, bias=True, seed=seed)
    h0 = si.history_input(B, D, W, seed=seed) if history else None
    r = si.train_inputs(B, T, D, W, bias=False, seed=seed + 77)["x"] if residual else None
    return inp["x"], inp["dy"], inp["w"], inp["bias"], h0, r


@pytest.mark.parametrize("history", [False, True], ids=["zero_history", "history"])
@pytest.mark.parametrize("residual", [False, True], ids=["no_residual", "residual"])
@pytest.mark.parametrize("act", ["silu", None], ids=["silu", "linear"])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_epilogue_parity(W, act, residual, history):
    B, T, D = 2, 777, 1032
    x, dy, w, b, h0, r = _case(B, T, D, W, seed=700 + W, history=history, residual=residual)
    y, hT, _ = cc.cconv_fwd_ex(_g(x), _g(w), _g(b), activation=act, residual=_g(r), init_state=_g(h0),
                               want_final_state=True)
    dx, dw, db, dh0, _ = cc.cconv_bwd_ex(_g(x), _g(dy), _g(w), _g(b), activation=act, init_state=_g(h0),
                                         want_d_init_state=True)
    torch.cuda.synchronize()
    what = f"W{W} act={act} residual={residual} history={history}"
    yr = oracle.fwd_epi(x, w, b, h0=h0, residual=r, act=act is not None)
    dxr, dwr, dbr, dh0r = oracle.bwd_epi(x, dy, w, b, h0=h0, act=act is not None)
    assert_close(y.cpu(), yr, TOL_FWD, f"{what} y")
    assert_close(dx.cpu(), dxr, TOL_BWD, f"{what} dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, f"{what} dw")
    assert_close(db.cpu(), dbr, TOL_BWD, f"{what} dbias")
    if W > 1:
        assert_close(dh0.cpu(), dh0r, TOL_BWD, f"{what} d_init_state")
        _, hTr = oracle.fwd_state(x, h0, w, b)
        assert np.array_equal(hT.cpu().float().numpy(), hTr), f"{what}: final state"


def test_default_options_match_plain_entry_points():
    x, dy, w, b, _, _ = _case(3, 500, 2048, 4, seed=710, history=False, residual=False)
    y, _, _ = cc.cconv_fwd_ex(_g(x), _g(w), _g(b))
    dx, dw, db, _, _ = cc.cconv_bwd_ex(_g(x), _g(dy), _g(w), _g(b))
    y2 = cc.cconv_fwd(_g(x), _g(w), _g(b))
    dx2, dw2, db2 = cc.cconv_bwd(_g(x), _g(dy), _g(w), _g(b))
    torch.cuda.synchronize()
    for a, c, n in ((y, y2, "y"), (dx, dx2, "dx"), (dw, dw2, "dw"), (db, db2, "dbias")):
        assert torch.equal(bits(a), bits(c)), n


def test_linear_medium_and_strided_residual():
    """8 x 1024 x 4096 without an activation, the residual a column slice of a wider tensor."""
    B, T, D, W = 8, 1024, 4096, 4
    x, dy, w, b, _, _ = _case(B, T, D, W, seed=720, history=False, residual=False)
    wide = si.train_inputs(B, T, D + 512, W, bias=False, seed=721)["x"]
    r = wide[:, :, 256:256 + D]
    y, _, _ = cc.cconv_fwd_ex(_g(x), _g(w), _g(b), activation=None, residual=_g(wide)[:, :, 256:256 + D])
    dx, dw, db, _, _ = cc.cconv_bwd_ex(_g(x), _g(dy), _g(w), _g(b), activation=None)
    torch.cuda.synchronize()
    assert_close(y.cpu(), oracle.fwd_epi(x, w, b, residual=r.contiguous(), act=False), TOL_FWD, "linear y")
    dxr, dwr, dbr, _ = oracle.bwd_epi(x, dy, w, b, act=False)
    assert_close(dx.cpu(), dxr, TOL_BWD, "linear dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, "linear dw")
    assert_close(db.cpu(), dbr, TOL_BWD, "linear dbias")


@pytest.mark.parametrize("act", ["silu", None], ids=["silu", "linear"])
def test_packed_with_epilogue(act):
    """A packed batch with a residual (and no activation): each sequence as its own oracle
    forward/backward with its own history, dw and dbias summed."""
    lens = [300, 0, 1, 2, 650, 5, 1]
    D, W = 520, 4
    total = sum(lens)
    inp = si.train_inputs(1, total, D, W, bias=True, seed=730)
    x, dy, w, b = inp["x"][0], inp["dy"][0], inp["w"], inp["bias"]
    r = si.train_inputs(1, total, D, W, bias=False, seed=731)["x"][0]
    h0 = si.history_input(len(lens), D, W, seed=732)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    y, hT, st = cc.cconv_fwd_ex(_g(x), _g(w), _g(b), activation=act, residual=_g(r), init_state=_g(h0),
                                want_final_state=True, cu_seqlens=_g(cu))
    dx, dw, db, dh0, st2 = cc.cconv_bwd_ex(_g(x), _g(dy), _g(w), _g(b), activation=act, init_state=_g(h0),
                                           want_d_init_state=True, cu_seqlens=_g(cu), dw_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    lin = act is not None
    yr = np.zeros((total, D))
    dxr = np.zeros((total, D))
    dwr = np.zeros((D, W))
    dbr = np.zeros(D)
    for i, L in enumerate(lens):
        a = int(cu[i])
        if L == 0:
            continue
        xs, dys, rs = x[a:a + L][None], dy[a:a + L][None], r[a:a + L][None]
        yr[a:a + L] = oracle.fwd_epi(xs, w, b, h0=h0[i:i + 1], residual=rs, act=lin)[0]
        dxi, dwi, dbi, _ = oracle.bwd_epi(xs, dys, w, b, h0=h0[i:i + 1], act=lin)
        dxr[a:a + L] = dxi[0]
        dwr += dwi
        dbr += dbi
    assert_close(y.cpu(), yr, TOL_FWD, f"packed {act} y")
    assert_close(dx.cpu(), dxr, TOL_BWD, f"packed {act} dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, f"packed {act} dw")
    assert_close(db.cpu(), dbr, TOL_BWD, f"packed {act} dbias")
    ok, _, hTr = oracle.fwd_varlen(x, cu.numpy(), w, b, h0)
    assert ok and np.array_equal(hT.cpu().float().numpy(), hTr)


def test_residual_guard_bands():
    B, T, D, W = 2, 130, 1032, 4
    x, _, w, b, _, r = _case(B, T, D, W, seed=740, history=False, residual=True)
    y, buf, lo, hi = guarded((B, T, D), torch.bfloat16, DEV)
    cc.cconv_fwd_ex(_g(x), _g(w), _g(b), activation=None, residual=_g(r), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf, lo, hi)
    assert_close(y.cpu(), oracle.fwd_epi(x, w, b, residual=r, act=False), TOL_FWD, "guarded y")


@pytest.mark.parametrize("act", ["silu", None], ids=["silu", "linear"])
@pytest.mark.parametrize("D,pitch,extra_rows", [(96, 128, 0), (1032, 2048, 5), (100, 131, 3)],
                         ids=["vector", "vector_padded_batch", "element_granular"])
def test_strided_outputs_equal_contiguous(D, pitch, extra_rows, act):
    """y and dx written into wider rows (row pitch `pitch`, batch stride (T + extra_rows) * pitch)
    equal the contiguous outputs bit for bit, dw and dbias too, and the padding around the D
    channels of each row is never written."""
    B, T, W = 2, 300, 4
    x, dy, w, b, h0, _ = _case(B, T, D, W, seed=730 + D, history=True, residual=False)
    gx, gdy, gw, gb, gh0 = _g(x), _g(dy), _g(w), _g(b), _g(h0)
    y0, hT0, _ = cc.cconv_fwd_ex(gx, gw, gb, activation=act, init_state=gh0, want_final_state=True)
    dx0, dw0, db0, dh0, _ = cc.cconv_bwd_ex(gx, gdy, gw, gb, activation=act, init_state=gh0, want_d_init_state=True)
    canary = -12345
    ybuf = torch.full((B, T + extra_rows, pitch), canary, dtype=torch.int16, device=DEV)
    dxbuf = torch.full((B, T + extra_rows, pitch), canary, dtype=torch.int16, device=DEV)
    y = ybuf.view(torch.bfloat16)[:, :T, :D]
    dx = dxbuf.view(torch.bfloat16)[:, :T, :D]
    assert not y.is_contiguous() and y.stride() == ((T + extra_rows) * pitch, pitch, 1)
    _, hT, _ = cc.cconv_fwd_ex(gx, gw, gb, activation=act, init_state=gh0, want_final_state=True, y=y)
    _, dw, db, dh, _ = cc.cconv_bwd_ex(gx, gdy, gw, gb, activation=act, init_state=gh0, want_d_init_state=True, dx=dx)
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(y0)) and torch.equal(bits(hT), bits(hT0))
    assert torch.equal(bits(dx), bits(dx0)) and torch.equal(bits(dh), bits(dh0))
    assert torch.equal(bits(dw), bits(dw0)) and torch.equal(db, db0)
    for buf in (ybuf, dxbuf):
        assert bool((buf[:, :, D:] == canary).all()) and bool((buf[:, T:, :] == canary).all()), "padding written"


def test_strided_outputs_packed():
    """A packed batch's y and dx written into wider rows equal the contiguous outputs."""
    D, pitch, W = 264, 512, 4
    lens = [5, 0, 300, 1, 77]
    total = sum(lens)
    inp = si.train_inputs(1, total, D, W, bias=True, seed=740)
    x, dy = inp["x"][0].to(DEV), inp["dy"][0].to(DEV)
    w, b = _g(inp["w"]), _g(inp["bias"])
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    y0, _, st0 = cc.cconv_fwd_ex(x, w, b, cu_seqlens=cu)
    dx0, dw0, db0, _, _ = cc.cconv_bwd_ex(x, dy, w, b, cu_seqlens=cu)
    canary = -4321
    ybuf = torch.full((total, pitch), canary, dtype=torch.int16, device=DEV)
    dxbuf = torch.full((total, pitch), canary, dtype=torch.int16, device=DEV)
    y, dx = ybuf.view(torch.bfloat16)[:, :D], dxbuf.view(torch.bfloat16)[:, :D]
    _, _, st = cc.cconv_fwd_ex(x, w, b, cu_seqlens=cu, y=y)
    _, dw, db, _, st2 = cc.cconv_bwd_ex(x, dy, w, b, cu_seqlens=cu, dx=dx)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0 and int(st0.item()) == 0
    assert torch.equal(bits(y), bits(y0)) and torch.equal(bits(dx), bits(dx0))
    assert torch.equal(bits(dw), bits(dw0)) and torch.equal(db, db0)
    assert bool((ybuf[:, D:] == canary).all()) and bool((dxbuf[:, D:] == canary).all()), "padding written"
