"""GPU parity for channel counts that are not multiples of 8, for every entry point, against
the oracle, through the C ABI: the element-granular paths (one channel per lane for odd D, two
for D = 2) and, for the training calls, the 4-channel lanes that D = 4 (mod 8) takes (D = 100
and 4100 below) and that D = 2 (mod 4) takes with its last lane group overlapping the one
before (D = 6, 46, 78, 130, 1002, 4098). Tolerances in parity.py; states bit for bit.
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


def _check_train(x, dy, w, b, h0, what, *, config_f=None, config_b=None):
    y, hT, _ = cc.cconv_fwd_ex(_g(x), _g(w), _g(b), init_state=_g(h0), want_final_state=True)
    dx, dw, db, dh0, _ = cc.cconv_bwd_ex(_g(x), _g(dy), _g(w), _g(b), init_state=_g(h0), want_d_init_state=True)
    torch.cuda.synchronize()
    yr, hTr = oracle.fwd_state(x, h0, w, b)
    dxr, dwr, dbr, dh0r = oracle.bwd_state(x, h0, dy, w, b)
    assert_close(y.cpu(), yr, TOL_FWD, f"{what} y")
    assert_close(dx.cpu(), dxr, TOL_BWD, f"{what} dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, f"{what} dw")
    assert_close(db.cpu(), dbr, TOL_BWD, f"{what} dbias")
    if w.shape[1] > 1:
        assert np.array_equal(hT.cpu().float().numpy(), hTr), f"{what}: final state"
        assert_close(dh0.cpu(), dh0r, TOL_BWD, f"{what} d_init_state")


@pytest.mark.parametrize("D", [1, 2, 7, 100, 130, 1003])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_narrow_train_parity(D, W):
    inp = si.train_inputs(2, 300, D, W, bias=True, seed=800 + D + W)
    h0 = si.history_input(2, D, W, seed=801 + D)
    _check_train(inp["x"], inp["dy"], inp["w"], inp["bias"], h0, f"D{D} W{W}")


def test_narrow_plain_entry_points_and_fp32_taps():
    inp = si.train_inputs(3, 1000, 333, 4, bias=True, seed=810, w_dtype=torch.float32)
    x, w, b, dy = (_g(inp[k]) for k in ("x", "w", "bias", "dy"))
    y = cc.cconv_fwd(x, w, b)
    dx, dw, db = cc.cconv_bwd(x, dy, w, b)
    torch.cuda.synchronize()
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
    assert dw.dtype == torch.float32
    assert_close(y.cpu(), yr, TOL_FWD, "D333 y")
    assert_close(dx.cpu(), dxr, TOL_BWD, "D333 dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, "D333 dw")
    assert_close(db.cpu(), dbr, TOL_BWD, "D333 dbias")


def test_narrow_decode_pr_width():
    """D = 4100 (not a multiple of 8), 2 x 2048 rows: the whole path against the oracle."""
    inp = si.train_inputs(2, 2048, 4100, 4, bias=True, seed=820)
    _check_train(inp["x"], inp["dy"], inp["w"], inp["bias"], None, "D4100")


def test_narrow_unaligned_strides_and_guards():
    """x and dy as column slices at odd offsets of wider tensors (any stride, 2-byte alignment);
    nothing written outside y and dx."""
    B, T, D, W = 2, 257, 131, 4
    big = si.train_inputs(B, T, D + 9, W, bias=True, seed=830)
    x = big["x"][:, :, 3:3 + D]
    dy = big["dy"][:, :, 5:5 + D]
    w, b = big["w"][:D].contiguous(), big["bias"][:D].contiguous()
    xd, dyd = _g(big["x"])[:, :, 3:3 + D], _g(big["dy"])[:, :, 5:5 + D]
    y, ybuf, ylo, yhi = guarded((B, T, D), torch.bfloat16, DEV)
    dx, xbuf, xlo, xhi = guarded((B, T, D), torch.bfloat16, DEV)
    cc.cconv_fwd(xd, _g(w), _g(b), y=y)
    cc.cconv_bwd(xd, dyd, _g(w), _g(b), dx=dx)
    torch.cuda.synchronize()
    assert canaries_intact(ybuf, ylo, yhi) and canaries_intact(xbuf, xlo, xhi)
    _, yr = oracle.fwd(x.contiguous(), w, b)
    dxr, _, _ = oracle.bwd(x.contiguous(), dy.contiguous(), w, b)
    assert_close(y.cpu(), yr, TOL_FWD, "strided y")
    assert_close(dx.cpu(), dxr, TOL_BWD, "strided dx")


@pytest.mark.parametrize("i", range(4))
def test_narrow_launch_invariance(i):
    cfgs = [
        dict(vec=1, rows_per_group=16, waves_per_block=1, options=0, seg_rows=16),
        dict(vec=1, rows_per_group=16, waves_per_block=8, options=0, seg_rows=32),
        dict(vec=1, rows_per_group=16, waves_per_block=2, strips_per_block=2, options=0, seg_rows=48),
        dict(vec=1, rows_per_group=16, waves_per_block=4, options=0, seg_rows=4096),
    ]
    inp = si.train_inputs(2, 700, 199, 4, bias=True, seed=840)
    x, w, b, dy = (_g(inp[k]) for k in ("x", "w", "bias", "dy"))
    ref_y = cc.cconv_fwd(x, w, b)
    ref_dx, ref_dw, _ = cc.cconv_bwd(x, dy, w, b, dw_dtype=torch.float32)
    cf = cc.Config(**cfgs[i])
    cb = cc.Config(**dict(cfgs[i], options=0))
    y = cc.cconv_fwd(x, w, b, config=cf)
    dx, dw, _ = cc.cconv_bwd(x, dy, w, b, config=cb, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(ref_y)) and torch.equal(bits(dx), bits(ref_dx))
    # fp32 partial sums grouped per launch: rounding-order differences only (~1e-5 here)
    assert_close(dw.cpu(), ref_dw.cpu(), 1e-4, "narrow dw across launches")


@pytest.mark.parametrize("D", [77, 78, 100])
def test_narrow_packed_and_epilogue(D):
    """Packed batches and the epilogue variants at D = 77 (one channel per lane), D = 78 (four,
    the last lane group overlapping) and D = 100 (four)."""
    lens = [100, 0, 1, 3, 250]
    W = 4
    total = sum(lens)
    inp = si.train_inputs(1, total, D, W, bias=True, seed=850)
    x, dy, w, b = inp["x"][0], inp["dy"][0], inp["w"], inp["bias"]
    h0 = si.history_input(len(lens), D, W, seed=851)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    y, hT, st = cc.cconv_fwd_varlen(_g(x), _g(cu), _g(w), _g(b), _g(h0), want_final_state=True)
    dx, dw, db, dh0, st2 = cc.cconv_bwd_varlen(_g(x), _g(dy), _g(cu), _g(w), _g(b), _g(h0), want_d_init_state=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    ok, yr, hTr = oracle.fwd_varlen(x, cu.numpy(), w, b, h0)
    _, dxr, dwr, dbr, dh0r = oracle.bwd_varlen(x, dy, cu.numpy(), w, b, h0)
    assert_close(y.cpu(), yr, TOL_FWD, "packed y")
    assert np.array_equal(hT.cpu().float().numpy(), hTr)
    assert_close(dx.cpu(), dxr, TOL_BWD, "packed dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, "packed dw")
    assert_close(dh0.cpu(), dh0r, TOL_BWD, "packed dh0")
    # epilogue, fixed length
    e = si.train_inputs(2, 150, D, W, bias=True, seed=852)
    r = si.train_inputs(2, 150, D, W, bias=False, seed=853)["x"]
    ye, _, _ = cc.cconv_fwd_ex(_g(e["x"]), _g(e["w"]), _g(e["bias"]), activation=None, residual=_g(r))
    dxe, _, _, _, _ = cc.cconv_bwd_ex(_g(e["x"]), _g(e["dy"]), _g(e["w"]), _g(e["bias"]), activation=None)
    torch.cuda.synchronize()
    assert_close(ye.cpu(), oracle.fwd_epi(e["x"], e["w"], e["bias"], residual=r, act=False), TOL_FWD, "epilogue y")
    assert_close(dxe.cpu(), oracle.bwd_epi(e["x"], e["dy"], e["w"], e["bias"], act=False)[0], TOL_BWD, "epilogue dx")


@pytest.mark.parametrize("ld_pad", [0, 3], ids=["compact", "padded"])
@pytest.mark.parametrize("D", [5, 4100])
def test_narrow_decode(D, ld_pad):
    """Decode with any D: compact rows, or rows padded to a stride that is a multiple of 8."""
    N, S, W = 40, 64, 4
    inp = si.decode_inputs(N, S, D, W, bias=True, seed=860 + D)
    ld = D if ld_pad == 0 else ((D + 7) // 8) * 8 + 8
    xw = torch.zeros(N, ld, dtype=torch.bfloat16)
    xw[:, :D] = inp["x"]
    st = inp["state"].to(DEV)
    y, status = cc.cconv_update(_g(xw)[:, :D], st, _g(inp["state_indices"]), _g(inp["w"]), _g(inp["bias"]))
    torch.cuda.synchronize()
    ok, yr, sr = oracle.update(inp["x"], inp["state"], inp["state_indices"], inp["w"], inp["bias"])
    assert ok and int(status.item()) == 0
    assert torch.equal(bits(st.cpu()), bits(torch.from_numpy(sr).to(torch.bfloat16)))
    assert_close(y.cpu(), yr, TOL_FWD, f"decode D{D} ld{ld}")
    # circular variant, L = W
    state4 = torch.randn(S, D, W, generator=torch.Generator().manual_seed(861)).to(torch.bfloat16)
    cs = torch.randint(0, 50, (N,), generator=torch.Generator().manual_seed(862), dtype=torch.int32)
    st4 = state4.to(DEV)
    y4, status = cc.cconv_update_ex(_g(xw)[:, :D], st4, _g(inp["state_indices"]), _g(inp["w"]), _g(inp["bias"]),
                                    cache_seqlens=_g(cs))
    torch.cuda.synchronize()
    ok, yr4, sr4 = oracle.update_ex(inp["x"], state4, inp["state_indices"].numpy(), cs.numpy(), inp["w"], inp["bias"])
    assert ok and int(status.item()) == 0
    assert torch.equal(bits(st4.cpu()), bits(torch.from_numpy(sr4).to(torch.bfloat16)))
    assert_close(y4.cpu(), yr4, TOL_FWD, f"circular decode D{D}")


@pytest.mark.parametrize("D", [45, 46, 60])
def test_narrow_pool(D):
    """The prefill into a decode pool at D = 45 (one channel per lane), D = 46 (four, the last
    lane group overlapping) and D = 60 (four)."""
    B, T, W, S = 3, 90, 4, 7
    inp = si.train_inputs(B, T, D, W, bias=True, seed=870)
    state = torch.randn(S, D, W - 1, generator=torch.Generator().manual_seed(871)).to(torch.bfloat16)
    idx = torch.tensor([5, -1, 2], dtype=torch.int32)
    has = torch.tensor([1, 0, 0], dtype=torch.uint8)
    st = state.to(DEV)
    y, status = cc.cconv_fwd_pool(_g(inp["x"]), _g(inp["w"]), _g(inp["bias"]), st, _g(idx), _g(has))
    torch.cuda.synchronize()
    ok, yr, sr = oracle.fwd_pool(inp["x"], state, idx.numpy(), has.numpy(), inp["w"], inp["bias"])
    assert ok and int(status.item()) == 0
    assert np.array_equal(st.cpu().float().numpy(), sr)
    assert_close(y.cpu(), yr, TOL_FWD, "pool y")


@pytest.mark.parametrize("D", [4, 1028])
@pytest.mark.parametrize("W", [1, 4])
def test_four_channel_lanes_d_4_mod_8(D, W):
    """D = 4 (mod 8) runs 4 channels per lane: x and dy as 8-byte aligned column slices of wider
    tensors (row stride D + 8), y and dx into guarded buffers, a ragged last strip and segment;
    against the oracle, and y and dx equal to the one-channel plan's bit for bit."""
    B, T = 2, 1000
    assert cc.cconv_default_config("fwd", B, T, D, W).vec == 4
    assert cc.cconv_default_config("bwd", B, T, D, W).vec == 4
    big = si.train_inputs(B, T, D + 8, W, bias=True, seed=860 + D + W)
    x = big["x"][:, :, 4:4 + D]
    dy = big["dy"][:, :, 4:4 + D]
    w, b = big["w"][:D].contiguous(), big["bias"][:D].contiguous()
    xd, dyd = _g(big["x"])[:, :, 4:4 + D], _g(big["dy"])[:, :, 4:4 + D]
    wd, bd = _g(w), _g(b)
    y, ybuf, ylo, yhi = guarded((B, T, D), torch.bfloat16, DEV)
    dx, xbuf, xlo, xhi = guarded((B, T, D), torch.bfloat16, DEV)
    cc.cconv_fwd(xd, wd, bd, y=y)
    _, dw, db = cc.cconv_bwd(xd, dyd, wd, bd, dx=dx, dw_dtype=torch.float32)
    one = cc.Config(vec=1, rows_per_group=16, waves_per_block=1, options=0, seg_rows=64)
    y1 = cc.cconv_fwd(xd, wd, bd, config=one)
    dx1, dw1, _ = cc.cconv_bwd(xd, dyd, wd, bd, config=one, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    assert canaries_intact(ybuf, ylo, yhi) and canaries_intact(xbuf, xlo, xhi)
    _, yr = oracle.fwd(x.contiguous(), w, b)
    dxr, dwr, dbr = oracle.bwd(x.contiguous(), dy.contiguous(), w, b)
    assert_close(y.cpu(), yr, TOL_FWD, f"D{D} W{W} y")
    assert_close(dx.cpu(), dxr, TOL_BWD, f"D{D} W{W} dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, f"D{D} W{W} dw")
    assert_close(db.cpu(), dbr, TOL_BWD, f"D{D} W{W} dbias")
    assert torch.equal(bits(y), bits(y1)) and torch.equal(bits(dx), bits(dx1))
    # fp32 partial sums grouped per launch: rounding-order differences only
    assert_close(dw.cpu(), dw1.cpu(), 1e-4, f"D{D} W{W} dw across lane widths")


@pytest.mark.parametrize("D", [2, 6, 10, 1002, 4098])
@pytest.mark.parametrize("W", [1, 4])
def test_lanes_d_2_mod_4(D, W):
    """D = 2 (mod 4) runs 4 channels per lane from D = 6 on (the last lane group starts at
    D - 4 and overlaps the one before by two channels) and 2 at D = 2: x and dy as 4-byte
    aligned column slices of wider tensors (row stride D + 2), y and dx into guarded buffers, a
    ragged last strip and segment; against the oracle, and y and dx equal bit for bit to the
    two- and one-channel plans' and to four-channel plans with other hints and block shapes."""
    B, T = 2, 1000
    v = 2 if D == 2 else 4
    assert cc.cconv_default_config("fwd", B, T, D, W).vec == v
    assert cc.cconv_default_config("bwd", B, T, D, W).vec == v
    big = si.train_inputs(B, T, D + 2, W, bias=True, seed=880 + D + W)
    x = big["x"][:, :, 2:2 + D]
    dy = big["dy"][:, :, 2:2 + D]
    w, b = big["w"][:D].contiguous(), big["bias"][:D].contiguous()
    xd, dyd = _g(big["x"])[:, :, 2:2 + D], _g(big["dy"])[:, :, 2:2 + D]
    wd, bd = _g(w), _g(b)
    y, ybuf, ylo, yhi = guarded((B, T, D), torch.bfloat16, DEV)
    dx, xbuf, xlo, xhi = guarded((B, T, D), torch.bfloat16, DEV)
    cc.cconv_fwd(xd, wd, bd, y=y)
    _, dw, db = cc.cconv_bwd(xd, dyd, wd, bd, dx=dx, dw_dtype=torch.float32)
    others = [dict(vec=1, rows_per_group=16, waves_per_block=1, options=0, seg_rows=64),
              dict(vec=2, rows_per_group=16, waves_per_block=1, options=0, seg_rows=128)]
    if D > 4:
        others += [dict(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=96),
                   dict(vec=4, rows_per_group=8, waves_per_block=4, strips_per_block=2, options=3, seg_rows=48),
                   dict(vec=4, rows_per_group=4, waves_per_block=8, options=0, seg_rows=32)]
    outs = []
    for cf in others:
        c = cc.Config(**cf)
        yo = cc.cconv_fwd(xd, wd, bd, config=c)
        dxo, dwo, _ = cc.cconv_bwd(xd, dyd, wd, bd, config=c, dw_dtype=torch.float32)
        outs.append((cf, yo, dxo, dwo))
    # off the 4-byte rule (x and dy at odd element offsets): the default plan takes one channel
    # per lane, the same values
    xo, dyo = _g(big["x"])[:, :, 1:1 + D], _g(big["dy"])[:, :, 1:1 + D]
    yo = cc.cconv_fwd(xo, wd, bd)
    dxo, _, _ = cc.cconv_bwd(xo, dyo, wd, bd)
    torch.cuda.synchronize()
    assert canaries_intact(ybuf, ylo, yhi) and canaries_intact(xbuf, xlo, xhi)
    _, yr = oracle.fwd(x.contiguous(), w, b)
    dxr, dwr, dbr = oracle.bwd(x.contiguous(), dy.contiguous(), w, b)
    assert_close(y.cpu(), yr, TOL_FWD, f"D{D} W{W} y")
    assert_close(dx.cpu(), dxr, TOL_BWD, f"D{D} W{W} dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, f"D{D} W{W} dw")
    assert_close(db.cpu(), dbr, TOL_BWD, f"D{D} W{W} dbias")
    for cf, y2, dx2, dw2 in outs:
        assert torch.equal(bits(y), bits(y2)) and torch.equal(bits(dx), bits(dx2)), cf
        # fp32 partial sums grouped per launch: rounding-order differences only
        assert_close(dw.cpu(), dw2.cpu(), 1e-4, f"D{D} W{W} dw across launches {cf}")
    _, yro = oracle.fwd(big["x"][:, :, 1:1 + D].contiguous(), w, b)
    dxro, _, _ = oracle.bwd(big["x"][:, :, 1:1 + D].contiguous(), big["dy"][:, :, 1:1 + D].contiguous(), w, b)
    assert_close(yo.cpu(), yro, TOL_FWD, f"D{D} W{W} y off the 4-byte rule")
    assert_close(dxo.cpu(), dxro, TOL_BWD, f"D{D} W{W} dx off the 4-byte rule")


@pytest.mark.parametrize("D", [6, 1002])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_overlapping_lane_group_with_states(D, W):
    """The overlapping last lane group of D = 2 (mod 4) through the state paths: a history in,
    the final state and the history's gradient out, and the packed batches with their states,
    at D = 6 (two lane groups, one wave) and 1002 (the overlap in the last of four strips)."""
    inp = si.train_inputs(3, 333, D, W, bias=True, seed=890 + D + W)
    h0 = si.history_input(3, D, W, seed=891 + D)
    _check_train(inp["x"], inp["dy"], inp["w"], inp["bias"], h0, f"D{D} W{W} states")
    lens = [5, 0, 2, 300, 26]
    total = sum(lens)
    x, dy = inp["x"][0, :total], inp["dy"][0, :total]
    hp = si.history_input(len(lens), D, W, seed=892 + D)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    y, hT, st = cc.cconv_fwd_varlen(_g(x), _g(cu), _g(inp["w"]), _g(inp["bias"]), _g(hp), want_final_state=True)
    dx, dw, db, dh0, st2 = cc.cconv_bwd_varlen(_g(x), _g(dy), _g(cu), _g(inp["w"]), _g(inp["bias"]), _g(hp),
                                               want_d_init_state=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    ok, yr, hTr = oracle.fwd_varlen(x, cu.numpy(), inp["w"], inp["bias"], hp)
    _, dxr, dwr, dbr, dh0r = oracle.bwd_varlen(x, dy, cu.numpy(), inp["w"], inp["bias"], hp)
    assert_close(y.cpu(), yr, TOL_FWD, "packed y")
    assert np.array_equal(hT.cpu().float().numpy(), hTr)
    assert_close(dx.cpu(), dxr, TOL_BWD, "packed dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, "packed dw")
    assert_close(db.cpu(), dbr, TOL_BWD, "packed dbias")
    assert_close(dh0.cpu(), dh0r, TOL_BWD, "packed dh0")


def test_backward_beyond_the_group_offset_strides():
    """Rows of x and dy 2^26 + 8 elements apart (134 MB): past the row strides the 4-channel
    backward addresses as 32-bit offsets, so the default plan runs one channel per lane; the
    result still matches the oracle, and the forward (no such limit) too."""
    B, T, D, W = 1, 5, 512, 4
    st = (1 << 26) + 8
    inp = si.train_inputs(B, T, D, W, bias=True, seed=895)
    xb = torch.zeros(T, st, dtype=torch.bfloat16, device=DEV)
    dyb = torch.zeros(T, st, dtype=torch.bfloat16, device=DEV)
    xb[:, :D] = inp["x"][0].to(DEV)
    dyb[:, :D] = inp["dy"][0].to(DEV)
    x, dy = xb[:, :D].unsqueeze(0), dyb[:, :D].unsqueeze(0)
    assert x.stride() == (T * st, st, 1)
    w, b = _g(inp["w"]), _g(inp["bias"])
    y = cc.cconv_fwd(x, w, b)
    dx, dw, db = cc.cconv_bwd(x, dy, w, b, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
    assert_close(y.cpu(), yr, TOL_FWD, "huge-stride y")
    assert_close(dx.cpu(), dxr, TOL_BWD, "huge-stride dx")
    assert_close(dw.cpu(), dwr, TOL_BWD, "huge-stride dw")
    assert_close(db.cpu(), dbr, TOL_BWD, "huge-stride dbias")
