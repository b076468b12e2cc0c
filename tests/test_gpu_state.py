"""GPU parity of the forward and backward with a history before t = 0, through the C ABI.

The history (init_state) is what a sequence saw before its first token; the forward also
returns the final state (the last W-1 values of history-then-x, in the decode state layout)
and the backward the gradient of every history value. Checked against the oracle's
oracle_fwd_state / oracle_bwd_state element by element; the final state is a copy of input
values, so it must match bit for bit. Continuation properties (two chunks equal one call,
prefill then decode equals a longer forward) tie the three entry points together.
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


def _inputs(B, T, D, W, *, bias=True, seed=11, history=True):
    inp = si.train_inputs(B, T, D, W, bias=bias, seed=seed)
    inp["h0"] = si.history_input(B, D, W, seed=seed) if history else None
    return inp


def _gpu(t):
    return None if t is None else t.to(DEV)


def _run(inp):
    x, w, b, dy, h0 = (_gpu(inp[k]) for k in ("x", "w", "bias", "dy", "h0"))
    y, hT = cc.cconv_fwd_state(x, w, b, h0)
    dx, dw, db, dh0 = cc.cconv_bwd_state(x, dy, w, b, h0)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.cpu() for t in (y, hT, dx, dw, db, dh0))


def _check(inp, outs, what):
    y, hT, dx, dw, db, dh0 = outs
    yr, hTr = oracle.fwd_state(inp["x"], inp["h0"], inp["w"], inp["bias"])
    dxr, dwr, dbr, dh0r = oracle.bwd_state(inp["x"], inp["h0"], inp["dy"], inp["w"], inp["bias"])
    ey = assert_close(y, yr, TOL_FWD, f"{what} y")
    # the final state holds input values: exact
    assert np.array_equal(hT.float().numpy(), hTr), f"{what}: final state differs"
    edx = assert_close(dx, dxr, TOL_BWD, f"{what} dx")
    edw = assert_close(dw, dwr, TOL_BWD, f"{what} dw")
    edb = assert_close(db, dbr, TOL_BWD, f"{what} dbias") if db is not None else 0.0
    edh = assert_close(dh0, dh0r, TOL_BWD, f"{what} d_init_state")
    print(f"{what}: err y {ey:.2e} dx {edx:.2e} dw {edw:.2e} dbias {edb:.2e} dh0 {edh:.2e}", flush=True)


@pytest.mark.parametrize(
    "B,T,D,W,bias",
    [
        (1, 256, 512, 4, True),
        (3, 1000, 2000, 2, True),
        (2, 777, 1032, 3, False),
        (8, 1024, 4096, 4, True),  # several segments per sequence and strips per row
        (2, 4099, 520, 4, True),  # ragged tail after many segments
    ],
)
def test_state_parity(B, T, D, W, bias):
    inp = _inputs(B, T, D, W, bias=bias)
    _check(inp, _run(inp), f"B{B}_T{T}_D{D}_W{W}")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 9])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_state_short_sequences(T, W):
    """T < W-1 keeps part of the history in the final state; T = 1 has one output row."""
    inp = _inputs(2, T, 264, W, seed=20 + T)
    _check(inp, _run(inp), f"T{T}_W{W}")


def test_no_history_matches_plain_entry_points():
    """init_state None is the zero history: y, dx, dw, dbias bit-identical to cconv_fwd/bwd."""
    inp = _inputs(2, 300, 1024, 4, history=False)
    y, hT, dx, dw, db, dh0 = _run(inp)
    g = {k: _gpu(v) for k, v in inp.items()}
    y2 = cc.cconv_fwd(g["x"], g["w"], g["bias"])
    dx2, dw2, db2 = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"])
    torch.cuda.synchronize()
    for a, b2, n in ((y, y2, "y"), (dx, dx2, "dx"), (dw, dw2, "dw"), (db, db2, "dbias")):
        assert torch.equal(bits(a), bits(b2)), n
    _check(inp, (y, hT, dx, dw, db, dh0), "no history")


def test_in_place_state_advance():
    """final_state may be init_state's own buffer: the cache advances in place."""
    for T in (1, 2, 100):
        inp = _inputs(2, T, 512, 4, seed=30 + T)
        x, w, b = (_gpu(inp[k]) for k in ("x", "w", "bias"))
        st = inp["h0"].clone().to(DEV)
        y, out = cc.cconv_fwd_state(x, w, b, st, final_state=st)
        torch.cuda.synchronize()
        assert out.data_ptr() == st.data_ptr()
        yr, hTr = oracle.fwd_state(inp["x"], inp["h0"], inp["w"], inp["bias"])
        assert np.array_equal(st.cpu().float().numpy(), hTr), T
        assert_close(y.cpu(), yr, TOL_FWD, f"in place T{T} y")


def test_chunked_continuation_equals_one_call():
    """Running a sequence in two chunks, the second starting from the first's final state,
    gives the same y (bit for bit: every row is computed from the same values in the same
    order) and the same final state as one call over the whole sequence."""
    B, T, D, W = 3, 1500, 1024, 4
    inp = _inputs(B, T, D, W, seed=40)
    x, w, b, h0 = (_gpu(inp[k]) for k in ("x", "w", "bias", "h0"))
    y_all, h_all = cc.cconv_fwd_state(x, w, b, h0)
    for cut in (1, 2, 3, 517, 1499):
        y1, h1 = cc.cconv_fwd_state(x[:, :cut].contiguous(), w, b, h0)
        y2, h2 = cc.cconv_fwd_state(x[:, cut:].contiguous(), w, b, h1)
        torch.cuda.synchronize()
        assert torch.equal(bits(torch.cat([y1, y2], 1)), bits(y_all)), cut
        assert torch.equal(bits(h2), bits(h_all)), cut


def test_chunked_backward_gradients_chain():
    """The backward of the second chunk hands its history gradient to the first chunk's dy-side:
    dx of the whole sequence equals [dx1 + the second chunk's d_init_state at the first chunk's
    last W-1 rows, dx2] and dw adds up (checked to the backward's tolerance against the oracle
    of the whole sequence)."""
    B, T, D, W = 2, 600, 512, 4
    R = W - 1
    inp = _inputs(B, T, D, W, seed=41)
    x, w, b, dy, h0 = (_gpu(inp[k]) for k in ("x", "w", "bias", "dy", "h0"))
    cut = 250
    _, h1 = cc.cconv_fwd_state(x[:, :cut].contiguous(), w, b, h0)
    dxa, dwa, dba, dh0a = cc.cconv_bwd_state(x[:, :cut].contiguous(), dy[:, :cut].contiguous(), w, b, h0,
                                             dw_dtype=torch.float32)
    dxb, dwb, dbb, dh1 = cc.cconv_bwd_state(x[:, cut:].contiguous(), dy[:, cut:].contiguous(), w, b, h1,
                                            dw_dtype=torch.float32)
    torch.cuda.synchronize()
    dx = torch.cat([dxa.float(), dxb.float()], 1)
    dx[:, cut - R:cut] += dh1.float().permute(0, 2, 1)
    dxr, dwr, dbr, dh0r = oracle.bwd_state(inp["x"], inp["h0"], inp["dy"], inp["w"], inp["bias"])
    # two bf16 roundings meet at the seam: twice the per-output budget there
    assert_close(dx.cpu(), dxr, 2 * TOL_BWD, "chunked dx")
    assert_close((dwa + dwb).cpu(), dwr, TOL_BWD, "chunked dw")
    assert_close((dba + dbb).cpu(), dbr, TOL_BWD, "chunked dbias")
    assert_close(dh0a.cpu(), dh0r, TOL_BWD, "chunked d_init_state")


@pytest.mark.parametrize("W", [2, 3, 4])
def test_prefill_then_decode(W):
    """A prefill's final state is the state cconv_update continues from: decoding token T after
    prefilling tokens 0..T-1 gives the forward's row T, and the advanced state equals the final
    state of a prefill over T+1 tokens (bit for bit)."""
    B, T, D = 4, 333, 1024
    inp = _inputs(B, T + 1, D, W, seed=50 + W)
    x, w, b, h0 = (_gpu(inp[k]) for k in ("x", "w", "bias", "h0"))
    _, st = cc.cconv_fwd_state(x[:, :T].contiguous(), w, b, h0)
    y_dec, status = cc.cconv_update(x[:, T].contiguous(), st, None, w, b)
    _, st_full = cc.cconv_fwd_state(x, w, b, h0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(bits(st), bits(st_full))
    yr, _ = oracle.fwd_state(inp["x"], inp["h0"], inp["w"], inp["bias"])
    assert_close(y_dec.cpu(), yr[:, T], TOL_FWD, f"decode after prefill W{W}")


def test_width_one_ignores_state():
    inp = _inputs(2, 100, 512, 1, seed=60, history=False)
    x, w, b, dy = (_gpu(inp[k]) for k in ("x", "w", "bias", "dy"))
    y, hT = cc.cconv_fwd_state(x, w, b, None)
    dx, dw, db, dh0 = cc.cconv_bwd_state(x, dy, w, b, None)
    torch.cuda.synchronize()
    assert hT.shape == (2, 512, 0) and dh0.shape == (2, 512, 0)
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    assert_close(y.cpu(), yr, TOL_FWD, "W1 y")


def test_state_guard_bands():
    """Nothing is written outside y, the final state, dx and the history gradient."""
    B, T, D, W = 2, 130, 1032, 4
    inp = _inputs(B, T, D, W, seed=70)
    x, w, b, dy, h0 = (_gpu(inp[k]) for k in ("x", "w", "bias", "dy", "h0"))
    hT, hbuf, hlo, hhi = guarded((B, D, W - 1), torch.bfloat16, DEV)
    dh, dbuf, dlo, dhi = guarded((B, D, W - 1), torch.bfloat16, DEV)
    y, ybuf, ylo, yhi = guarded((B, T, D), torch.bfloat16, DEV)
    cc.cconv_fwd_state(x, w, b, h0, final_state=hT, y=y)
    cc.cconv_bwd_state(x, dy, w, b, h0, d_init_state=dh)
    torch.cuda.synchronize()
    assert canaries_intact(hbuf, hlo, hhi) and canaries_intact(dbuf, dlo, dhi) and canaries_intact(ybuf, ylo, yhi)
    _check(inp, _run(inp), "guarded")


def test_empty_sequence_with_state_is_rejected():
    x = torch.empty((2, 0, 512), dtype=torch.bfloat16, device=DEV)
    w = torch.randn(512, 4, device=DEV).to(torch.bfloat16)
    h0 = torch.zeros((2, 512, 3), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(cc.CconvError):
        cc.cconv_fwd_state(x, w, None, h0)
    y, hT = cc.cconv_fwd_state(x, w, None, h0, want_final_state=False)
    assert y.shape == (2, 0, 512) and hT is None


# ---- prefill straight into the decode pool (cconv_fwd_pool) ----


def _pool_case(B, T, D, W, S, *, seed, pad=True):
    inp = si.train_inputs(B, T, D, W, bias=True, seed=seed)
    g = torch.Generator().manual_seed(seed + 7)
    state = (torch.randn(S, D, W - 1, generator=g)).to(torch.bfloat16)
    idx = torch.randperm(S, generator=g)[:B].to(torch.int32)
    if pad and B > 1:
        idx[1] = -1
    has = (torch.arange(B) % 3 != 2).to(torch.uint8)
    return inp, state, idx, has


@pytest.mark.parametrize("T", [1, 2, 300, 1500])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_pool_parity(T, W):
    B, D, S = 5, 1032, 11
    inp, state, idx, has = _pool_case(B, T, D, W, S, seed=80 + T + W)
    st = state.to(DEV)
    y, status = cc.cconv_fwd_pool(_gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"]), st, idx.to(DEV), has.to(DEV))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ok, yr, sr = oracle.fwd_pool(inp["x"], state, idx.numpy(), has.numpy(), inp["w"], inp["bias"])
    assert ok
    assert_close(y.cpu(), yr, TOL_FWD, f"pool T{T} W{W} y")
    assert np.array_equal(st.cpu().float().numpy(), sr), f"pool T{T} W{W}: state differs"


def test_pool_without_flags_starts_from_zeros():
    B, T, D, W, S = 4, 77, 512, 4, 9
    inp, state, idx, _ = _pool_case(B, T, D, W, S, seed=90)
    st = state.to(DEV)
    y, status = cc.cconv_fwd_pool(_gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"]), st, idx.to(DEV), None)
    y_plain = cc.cconv_fwd(_gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"]))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(bits(y), bits(y_plain))
    ok, _, sr = oracle.fwd_pool(inp["x"], state, idx.numpy(), None, inp["w"], inp["bias"])
    assert ok and np.array_equal(st.cpu().float().numpy(), sr)


@pytest.mark.parametrize(
    "bad",
    [[0, 1, 9, 3], [0, -2, 1, 2], [4, 2, 4, 1], [2**31 - 1, 0, 1, 2], [0, 1, -(2**31), 2], [-1, -1, 3, 3]],
    ids=["past_end", "below_minus_one", "repeat", "int32_max", "int32_min", "repeat_after_padding"],
)
def test_pool_invalid_indices_write_nothing(bad):
    B, T, D, W, S = 4, 200, 520, 4, 9
    inp, state, _, has = _pool_case(B, T, D, W, S, seed=100)
    st = state.to(DEV)
    y, ybuf, ylo, yhi = guarded((B, T, D), torch.bfloat16, DEV)
    y.view(torch.int16).fill_(0x7FA5)
    _, status = cc.cconv_fwd_pool(_gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"]), st,
                                  torch.tensor(bad, dtype=torch.int32, device=DEV), has.to(DEV), y=y)
    torch.cuda.synchronize()
    assert int(status.item()) == 8
    assert torch.equal(bits(st), bits(state)), "a rejected call changed the pool"
    assert canaries_intact(ybuf, ylo, yhi) and bool((bits(y) == 0x7FA5).all()), "a rejected call wrote y"
    ok, _, _ = oracle.fwd_pool(inp["x"], state, np.array(bad, np.int32), has.numpy(), inp["w"], inp["bias"])
    assert not ok
    # the status word is rewritten by the next good call
    _, status = cc.cconv_fwd_pool(_gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"]), st,
                                  torch.tensor([0, 1, 2, 3], dtype=torch.int32, device=DEV), None, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_pool_equals_gathered_history():
    """The pool forward is cconv_fwd_state on the gathered histories, bit for bit, with the
    final states scattered to the slots."""
    B, T, D, W, S = 6, 640, 2048, 4, 16
    inp, state, idx, has = _pool_case(B, T, D, W, S, seed=110)
    h0 = torch.zeros(B, D, W - 1, dtype=torch.bfloat16)
    for b in range(B):
        if idx[b] >= 0 and has[b]:
            h0[b] = state[idx[b]]
    st = state.to(DEV)
    x, w, bias = _gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"])
    y, status = cc.cconv_fwd_pool(x, w, bias, st, idx.to(DEV), has.to(DEV))
    y2, hT = cc.cconv_fwd_state(x, w, bias, h0.to(DEV))
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(bits(y), bits(y2))
    stc, hTc = st.cpu(), hT.cpu()
    named = set()
    for b in range(B):
        if idx[b] >= 0:
            named.add(int(idx[b]))
            assert torch.equal(bits(stc[idx[b]]), bits(hTc[b])), b
    for s_ in range(S):
        if s_ not in named:
            assert torch.equal(bits(stc[s_]), bits(state[s_])), s_


@pytest.mark.parametrize("W", [2, 4])
def test_pool_chunked_prefill_then_decode(W):
    """Two prefill chunks into the pool (the first ignoring stale slot contents, the second
    continuing from them), then decode steps from the same slots: every output matches the
    oracle's forward of the whole sequence, and the final slots match it bit for bit."""
    B, D, S = 4, 1024, 10
    T1, T2, T3 = 129, 200, 5
    T = T1 + T2 + T3
    inp, state, idx, _ = _pool_case(B, T, D, W, S, seed=120 + W, pad=False)
    x, w, bias = _gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"])
    st, di = state.to(DEV), idx.to(DEV)
    y1, s1 = cc.cconv_fwd_pool(x[:, :T1].contiguous(), w, bias, st, di, torch.zeros(B, dtype=torch.bool, device=DEV))
    y2, s2 = cc.cconv_fwd_pool(x[:, T1:T1 + T2].contiguous(), w, bias, st, di,
                               torch.ones(B, dtype=torch.bool, device=DEV))
    ys = [y1, y2]
    for t in range(T1 + T2, T):
        yt, sd = cc.cconv_update(x[:, t].contiguous(), st, di, w, bias)
        ys.append(yt[:, None])
        assert int(sd.item()) == 0
    torch.cuda.synchronize()
    assert int(s1.item()) == 0 and int(s2.item()) == 0
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    assert_close(torch.cat([t.cpu() for t in ys], 1), yr, TOL_FWD, f"chunked pool W{W}")
    stc = st.cpu()
    for b in range(B):
        want = inp["x"][b, T - (W - 1):].transpose(0, 1)
        assert torch.equal(bits(stc[idx[b]]), bits(want.contiguous())), b


def test_pool_headline_size():
    """8 x 8192 x 4096 into a 64-slot pool in the benchmark's forward launch: y bit-identical
    to the plain forward (zero histories) and each slot holds its sequence's last 3 rows."""
    s = si.HEADLINE
    g = si.train_inputs_device(s.B, s.T, s.D, s.W, bias=True, seed=s.seed)
    S = 64
    st = torch.zeros(S, s.D, s.W - 1, dtype=torch.bfloat16, device=DEV)
    idx = torch.arange(S - 1, S - 1 - 2 * s.B, -2, dtype=torch.int32, device=DEV)
    y, status = cc.cconv_fwd_pool(g["x"], g["w"], g["bias"], st, idx)
    y2 = cc.cconv_fwd(g["x"], g["w"], g["bias"])
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(y.view(torch.int16), y2.view(torch.int16))
    for b in range(s.B):
        want = g["x"][b, s.T - 3:].transpose(0, 1).contiguous()
        assert torch.equal(st[idx[b]].view(torch.int16), want.view(torch.int16)), b
    assert not st[0].any()


def test_pool_width_one_and_empty_batch():
    inp = si.train_inputs(3, 50, 256, 1, bias=True, seed=130)
    x, w, bias = _gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"])
    st = torch.empty(5, 256, 0, dtype=torch.bfloat16, device=DEV)
    y, status = cc.cconv_fwd_pool(x, w, bias, st, torch.tensor([4, -1, 0], dtype=torch.int32, device=DEV))
    y2 = cc.cconv_fwd(x, w, bias)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(bits(y), bits(y2))
    _, status = cc.cconv_fwd_pool(x, w, bias, st, torch.tensor([4, 4, 0], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert int(status.item()) == 8
    w4 = torch.randn(256, 4, device=DEV).to(torch.bfloat16)
    st4 = torch.zeros(5, 256, 3, dtype=torch.bfloat16, device=DEV)
    status = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    y, status = cc.cconv_fwd_pool(x[:0], w4, None, st4, torch.empty(0, dtype=torch.int32, device=DEV), status=status)
    torch.cuda.synchronize()
    assert y.shape == (0, 50, 256) and int(status.item()) == 0


def test_pool_graph_replay():
    """The pool forward (slot check + forward) captured in a HIP graph: each replay advances the
    pool exactly as the same eager calls do."""
    B, T, D, W, S = 3, 96, 1024, 4, 6
    inp, state, idx, _ = _pool_case(B, T, D, W, S, seed=140, pad=False)
    x, w, bias = _gpu(inp["x"]), _gpu(inp["w"]), _gpu(inp["bias"])
    di = idx.to(DEV)
    has = torch.ones(B, dtype=torch.uint8, device=DEV)
    # eager reference: three calls in a row
    ref = state.to(DEV)
    ys_ref = []
    for _ in range(3):
        y, stt = cc.cconv_fwd_pool(x, w, bias, ref, di, has)
        ys_ref.append(y.clone())
    torch.cuda.synchronize()
    st = state.to(DEV)
    y_out = torch.empty(B, T, D, dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cc.cconv_fwd_pool(x, w, bias, st, di, has, y=y_out, status=status, stream=s)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    st.copy_(state.to(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cc.cconv_fwd_pool(x, w, bias, st, di, has, y=y_out, status=status, stream=s)
    torch.cuda.synchronize()
    st.copy_(state.to(DEV))
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(bits(y_out), bits(ys_ref[r])), f"replay {r}"
    assert torch.equal(bits(st), bits(ref))
