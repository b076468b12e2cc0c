"""GPU parity of the one-token decode update against the CPU oracle, through the C ABI.

y is compared within the forward tolerance; the state shift and the index gather are
compared bit for bit (every slot, touched or not). Invalid indices must leave the state
bitwise unchanged, report CCONV_ERR_INDEX in the device status word, and leave the process
usable (no device trap).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import causal_depthwise_short_amd as cc
import oracle
import synth_inputs as si
from parity import TOL_FWD, assert_close, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
CCONV_OK, CCONV_ERR_INDEX = 0, 8


_FROM_INPUTS = object()


def run_update(inp, *, x=None, idx=_FROM_INPUTS):
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    if idx is not _FROM_INPUTS:
        g["state_indices"] = None if idx is None else torch.as_tensor(idx, dtype=torch.int32, device=DEV)
    xs = g["x"] if x is None else x
    y, status = cc.cconv_update(xs, g["state"], g["state_indices"], g["w"], g["bias"])
    torch.cuda.synchronize()
    return y.cpu(), g["state"].cpu(), int(status.item())


def check_update(inp, y, new_state, status, idx, what):
    ok, yr, sr = oracle.update(inp["x"], inp["state"], idx, inp["w"], inp["bias"])
    assert ok and status == CCONV_OK, f"{what}: status {status}"
    ref_state = torch.from_numpy(sr).to(torch.bfloat16)  # exact: the values are bf16
    assert torch.equal(bits(new_state), bits(ref_state)), f"{what}: state differs from the oracle"
    e = assert_close(y, yr, TOL_FWD, f"{what} y")
    print(f"{what}: err y {e:.2e}, state bit-exact", flush=True)


def test_decode_workload_parity():
    s = si.DECODE
    inp = si.decode_inputs_for(s)
    y, st, status = run_update(inp)
    check_update(inp, y, st, status, inp["state_indices"], s.name)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("w_dtype", [torch.bfloat16, torch.float32], ids=["wbf16", "wf32"])
def test_decode_widths(W, w_dtype):
    inp = si.decode_inputs(37, 50, 264, W, bias=(W % 2 == 0), seed=40 + W, w_dtype=w_dtype)
    y, st, status = run_update(inp)
    check_update(inp, y, st, status, inp["state_indices"], f"W={W}")


def test_decode_identity_and_padding_rows():
    inp = si.decode_inputs(64, 80, 1032, 4, bias=True, seed=50, identity=True)
    y, st, status = run_update(inp, idx=None)
    check_update(inp, y, st, status, None, "identity")
    idx = np.arange(64, dtype=np.int32)[::-1].copy()
    idx[::3] = -1
    y, st, status = run_update(inp, idx=idx)
    check_update(inp, y, st, status, idx, "padding rows")
    assert not y[::3].float().any(), "padding rows must output 0"


def test_decode_strided_x():
    N, S, D, W = 48, 64, 512, 4
    inp = si.decode_inputs(N, S, D, W, bias=True, seed=60)
    wide = torch.zeros(N, 3 * D, dtype=torch.bfloat16, device=DEV)
    wide[:, D : 2 * D] = inp["x"].to(DEV)
    xs = wide[:, D : 2 * D]
    assert xs.stride() == (3 * D, 1)
    y, st, status = run_update(inp, x=xs)
    check_update(inp, y, st, status, inp["state_indices"], "strided x")


@pytest.mark.parametrize("case", ["negative", "out_of_range", "duplicate"])
def test_decode_invalid_indices_fail_closed(case):
    N, S, D, W = 32, 40, 512, 4
    inp = si.decode_inputs(N, S, D, W, bias=True, seed=70)
    idx = inp["state_indices"].numpy().copy()
    if case == "negative":
        idx[5] = -2
    elif case == "out_of_range":
        idx[N - 1] = S
    else:
        idx[7] = idx[20]
    before = bits(inp["state"])
    _, st, status = run_update(inp, idx=idx)
    assert status == CCONV_ERR_INDEX, f"{case}: status {status}"
    assert torch.equal(bits(st), before), f"{case}: state modified by an invalid call"
    ok, _, _ = oracle.update(inp["x"], inp["state"], idx, inp["w"], inp["bias"])
    assert not ok, "oracle must reject it too"
    # the process is still usable: a valid call right after succeeds
    y, st, status = run_update(inp)
    check_update(inp, y, st, status, inp["state_indices"], f"after {case}")


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_decode_equals_forward(W):
    """Token-by-token updates from a zero state reproduce the GPU forward bitwise, and the
    final state holds the last W-1 inputs."""
    B, T, D = 5, 11, 520
    inp = si.train_inputs(B, T, D, W, bias=True, seed=80 + W)
    x = inp["x"].to(DEV)
    w = inp["w"].to(DEV)
    b = inp["bias"].to(DEV)
    y_fwd = cc.cconv_fwd(x, w, b)
    S = 9
    idx = torch.tensor([4, 0, 8, 2, 6], dtype=torch.int32, device=DEV)
    state = torch.zeros(S, D, W - 1, dtype=torch.bfloat16, device=DEV)
    for t in range(T):
        y_t, status = cc.cconv_update(x[:, t, :], state, idx, w, b)
        assert int(status.item()) == CCONV_OK
        assert torch.equal(bits(y_t), bits(y_fwd[:, t, :])), f"decode != forward at t={t}"
    for r in range(B):
        want = x[r, T - (W - 1) :, :].transpose(0, 1) if W > 1 else state[0, :, :0]
        assert torch.equal(bits(state[int(idx[r])]), bits(want.contiguous())), f"final state row {r}"


def test_decode_empty():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    state = torch.randn(4, 64, 3).to(torch.bfloat16).to(DEV)
    w = torch.randn(64, 4).to(torch.bfloat16).to(DEV)
    status = torch.full((1,), 123, dtype=torch.int32, device=DEV)
    before = bits(state)
    y, status = cc.cconv_update(x, state, torch.empty(0, dtype=torch.int32, device=DEV), w, None, status=status)
    torch.cuda.synchronize()
    assert y.numel() == 0 and int(status.item()) == CCONV_OK and torch.equal(bits(state), before)


def test_decode_graph_replay():
    inp = si.decode_inputs_for(si.DECODE)
    g = {k: v.to(DEV) for k, v in inp.items() if v is not None}
    s0 = g["state"].clone()
    y_e, _ = cc.cconv_update(g["x"], g["state"], g["state_indices"], g["w"], g["bias"])
    torch.cuda.synchronize()
    st_e = g["state"].clone()
    g["state"].copy_(s0)
    y = torch.empty_like(y_e)
    status = torch.empty(1, dtype=torch.int32, device=DEV)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        cc.cconv_update(g["x"], g["state"], g["state_indices"], g["w"], g["bias"], y=y, status=status)
    for rep in range(3):
        g["state"].copy_(s0)
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_e)) and torch.equal(bits(g["state"]), bits(st_e)), f"replay {rep}"
        assert int(status.item()) == CCONV_OK


def test_fused_qkv_decode_one_launch_equals_three():
    """One decode update over a fused q|k|v projection row ([N, Dq + Dk + Dv], one state of
    Dq + Dk + Dv channels, the three taps and biases concatenated) equals three updates on the
    channel slices (x row stride Dq + Dk + Dv, three states): y and the new states bit for
    bit, with the same slots for all three."""
    split, W = (256, 256, 512), 4
    Dt = sum(split)
    inp = si.decode_inputs(64, 96, Dt, W, bias=True, seed=91)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    st_all = g["state"].clone()
    y_all, s_all = cc.cconv_update(g["x"], st_all, g["state_indices"], g["w"], g["bias"])
    ys, states, lo = [], [], 0
    for Dj in split:
        sl = slice(lo, lo + Dj)
        lo += Dj
        st = g["state"][:, sl, :].contiguous()
        yj, sj = cc.cconv_update(g["x"][:, sl], st, g["state_indices"], g["w"][sl].contiguous(), g["bias"][sl].contiguous())
        torch.cuda.synchronize()
        assert int(sj.item()) == CCONV_OK
        ys.append(yj)
        states.append(st)
    torch.cuda.synchronize()
    assert int(s_all.item()) == CCONV_OK
    assert torch.equal(bits(y_all), bits(torch.cat(ys, dim=1)))
    assert torch.equal(bits(st_all), bits(torch.cat(states, dim=1)))
    check_update(inp, y_all.cpu(), st_all.cpu(), int(s_all.item()), inp["state_indices"].numpy(), "fused q|k|v decode")
