"""GPU parity of the decode variants (state of L = W-1 or W entries; shift or circular
cache_seqlens addressing) against the oracle's oracle_update_ex, through the C ABI.

y within the forward tolerance, the state bit for bit (every slot, touched or not). Token by
token, each variant must reproduce the forward of the whole sequence, and a negative
cache_seqlens entry must fail the call closed.
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


def _inputs(N, S, D, W, L, *, seed, circular, pad=True):
    inp = si.decode_inputs(N, S, D, W, bias=True, seed=seed)
    g = torch.Generator().manual_seed(seed + 5)
    state = torch.randn(S, D, L, generator=g).to(torch.bfloat16)
    idx = inp["state_indices"].clone()
    if pad:
        idx[::7] = -1
    cs = torch.randint(0, 1000, (N,), generator=g, dtype=torch.int32) if circular else None
    return inp["x"], state, idx, cs, inp["w"], inp["bias"]


def _run(x, state, idx, cs, w, b):
    st = state.to(DEV)
    y, status = cc.cconv_update_ex(x.to(DEV), st, None if idx is None else idx.to(DEV), w.to(DEV),
                                   None if b is None else b.to(DEV), cache_seqlens=None if cs is None else cs.to(DEV))
    torch.cuda.synchronize()
    return y.cpu(), st.cpu(), int(status.item())


@pytest.mark.parametrize("circular", [False, True], ids=["shift", "circular"])
@pytest.mark.parametrize("WL", [(1, 1), (2, 1), (2, 2), (3, 2), (3, 3), (4, 3), (4, 4)], ids=lambda p: f"W{p[0]}L{p[1]}")
def test_variant_parity(WL, circular):
    W, L = WL
    for N, S, D in ((256, 512, 4096), (37, 50, 1032)):
        x, state, idx, cs, w, b = _inputs(N, S, D, W, L, seed=300 + 10 * W + L, circular=circular)
        y, st, status = _run(x, state, idx, cs, w, b)
        ok, yr, sr = oracle.update_ex(x, state, idx.numpy(), None if cs is None else cs.numpy(), w, b)
        assert ok and status == 0
        assert torch.equal(bits(st), bits(torch.from_numpy(sr).to(torch.bfloat16))), f"W{W} L{L} N{N}: state"
        assert_close(y, yr, TOL_FWD, f"W{W} L{L} {'circular' if circular else 'shift'} N{N}")


def test_shift_with_w_minus_one_entries_is_plain_update():
    x, state, idx, _, w, b = _inputs(256, 512, 4096, 4, 3, seed=320, circular=False)
    y, st, status = _run(x, state, idx, None, w, b)
    st2 = state.to(DEV)
    y2, status2 = cc.cconv_update(x.to(DEV), st2, idx.to(DEV), w.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    assert status == 0 and int(status2.item()) == 0
    assert torch.equal(bits(y), bits(y2.cpu())) and torch.equal(bits(st), bits(st2.cpu()))


@pytest.mark.parametrize("L", [3, 4])
@pytest.mark.parametrize("c0", [0, 1, 6])
def test_circular_decode_reproduces_forward(L, c0):
    """A prefill's final state is a circular state with c = 0 (mod L): placed at ring start c0
    and decoded token by token with cache_seqlens = c0, c0+1, ..., every output matches the
    forward of the whole sequence."""
    B, T0, T, D, W = 4, 100, 112, 1024, 4
    inp = si.train_inputs(B, T, D, W, bias=True, seed=330 + L + c0)
    x, w, bias = (inp[k].to(DEV) for k in ("x", "w", "bias"))
    _, hT = cc.cconv_fwd_state(x[:, :T0].contiguous(), w, bias, None)
    ring = torch.zeros(B, D, L, dtype=torch.bfloat16, device=DEV)
    for k in range(1, W):  # the token k steps back from T0 sits in entry (c0 - k) mod L
        ring[:, :, (c0 - k) % L] = hT[:, :, W - 1 - k]
    ys = []
    cs = torch.full((B,), c0, dtype=torch.int32, device=DEV)
    for t in range(T0, T):
        yt, st = cc.cconv_update_ex(x[:, t].contiguous(), ring, None, w, bias, cache_seqlens=cs)
        cs += 1
        ys.append(yt)
        assert int(st.item()) == 0
    torch.cuda.synchronize()
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    assert_close(torch.stack([t.cpu() for t in ys], 1), yr[:, T0:T], TOL_FWD, f"circular L{L} c0={c0}")
    # the ring now holds the last tokens in circular order
    c = c0 + (T - T0)
    for k in range(1, W):
        assert torch.equal(bits(ring[:, :, (c - k) % L].cpu()), bits(inp["x"][:, T - k].contiguous())), k


def test_negative_seqlen_fails_closed():
    x, state, idx, cs, w, b = _inputs(64, 80, 512, 4, 4, seed=340, circular=True)
    cs[17] = -3
    y, st, status = _run(x, state, idx, cs, w, b)
    assert status == 8 and torch.equal(bits(st), bits(state))
    ok, _, _ = oracle.update_ex(x, state, idx.numpy(), cs.numpy(), w, b)
    assert not ok


def test_circular_graph_replay():
    """Circular updates captured in a HIP graph with the cache_seqlens advance: each replay
    matches the same eager step."""
    N, S, D, W, L = 32, 40, 2048, 4, 4
    x, state, idx, cs, w, b = _inputs(N, S, D, W, L, seed=350, circular=True, pad=False)
    xd, wd, bd, idd = x.to(DEV), w.to(DEV), b.to(DEV), idx.to(DEV)
    ref, csr = state.to(DEV), cs.to(DEV)
    ys = []
    for _ in range(3):
        y, _ = cc.cconv_update_ex(xd, ref, idd, wd, bd, cache_seqlens=csr)
        csr += 1
        ys.append(y.clone())
    torch.cuda.synchronize()
    st, csd = state.to(DEV), cs.to(DEV)
    y_out = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cc.cconv_update_ex(xd, st, idd, wd, bd, cache_seqlens=csd, y=y_out, status=status, stream=s)
        csd.add_(1)
    st.copy_(state.to(DEV))
    csd.copy_(cs.to(DEV))
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and torch.equal(bits(y_out), bits(ys[r])), r
    assert torch.equal(bits(st), bits(ref))


# (vec, block_threads, options, rows_per_block, rows_per_thread): 8, 4 and 1 channels per
# thread, block shapes from one wave to sixteen, both cache hints, threads that carry one or
# two rows at once, and blocks that walk several groups of rows (the next group's loads
# issued before the current group's arithmetic), with ragged last groups
UPDATE_CONFIGS = [(8, 64, 0, 1, 1), (8, 128, 1, 3, 1), (8, 256, 0, 7, 2), (8, 512, 1, 2, 2), (8, 1024, 0, 5, 1),
                  (8, 256, 1, 64, 2), (8, 256, 3, 1, 2), (8, 128, 2, 4, 1), (8, 256, 5, 2, 2), (8, 64, 4, 3, 1),
                  (8, 512, 5, 1, 2), (8, 512, 4, 2, 1), (4, 64, 1, 9, 2), (4, 256, 0, 1, 1),
                  (4, 512, 1, 5, 2), (4, 1024, 1, 3, 1), (4, 256, 3, 2, 2), (4, 64, 2, 1, 1),
                  (1, 64, 0, 1, 1), (1, 256, 0, 6, 1), (1, 1024, 0, 2, 1)]


@pytest.mark.parametrize("D", [4096, 1032, 1004, 1003])
@pytest.mark.parametrize("circular", [False, True], ids=["shift", "circular"])
@pytest.mark.parametrize("WL", [(1, 1), (2, 1), (3, 3), (4, 3), (4, 4)], ids=lambda p: f"W{p[0]}L{p[1]}")
def test_update_launch_config_invariance(WL, circular, D):
    """y and the new state do not depend on the launch configuration, bit for bit; the default
    launch matches the oracle (state bit-exact, y within tolerance)."""
    W, L = WL
    N, S = 37, 50
    x, state, idx, cs, w, b = _inputs(N, S, D, W, L, seed=500 + 10 * W + L + D % 7, circular=circular)
    y0, st0, status = _run(x, state, idx, cs, w, b)
    ok, yr, sr = oracle.update_ex(x, state, idx.numpy(), None if cs is None else cs.numpy(), w, b)
    assert ok and status == 0
    assert torch.equal(bits(st0), bits(torch.from_numpy(sr).to(torch.bfloat16)))
    assert_close(y0, yr, TOL_FWD, f"W{W} L{L} D{D} default launch")
    ran = 0
    for vec, bt, opt, rpb, rpt in UPDATE_CONFIGS:
        if D % vec != 0:
            continue
        cfg = cc.UpdateConfig(vec=vec, block_threads=bt, options=opt if vec > 1 else 0, rows_per_block=rpb,
                              rows_per_thread=rpt if vec > 1 else 1)
        st = state.to(DEV)
        y, s = cc.cconv_update_config(x.to(DEV), st, idx.to(DEV), w.to(DEV), b.to(DEV), config=cfg,
                                      cache_seqlens=None if cs is None else cs.to(DEV))
        torch.cuda.synchronize()
        assert int(s.item()) == 0, cfg
        assert torch.equal(bits(y.cpu()), bits(y0)), f"y differs under {cfg}"
        assert torch.equal(bits(st.cpu()), bits(st0)), f"state differs under {cfg}"
        ran += 1
    assert ran >= 3


@pytest.mark.parametrize("circular", [False, True], ids=["shift", "circular"])
def test_update_many_rows_per_block(circular):
    """N = 3000 rows: the default launch walks several rows per block (about 1024 blocks)."""
    N, S, D, W, L = 3000, 3500, 4096, 4, 3
    cfg = cc.cconv_default_update_config(N, D)
    assert cfg.rows_per_block > 1
    x, state, idx, cs, w, b = _inputs(N, S, D, W, L, seed=540, circular=circular)
    y, st, status = _run(x, state, idx, cs, w, b)
    ok, yr, sr = oracle.update_ex(x, state, idx.numpy(), None if cs is None else cs.numpy(), w, b)
    assert ok and status == 0
    assert torch.equal(bits(st), bits(torch.from_numpy(sr).to(torch.bfloat16)))
    assert_close(y, yr, TOL_FWD, f"N{N} {'circular' if circular else 'shift'}")


@pytest.mark.parametrize("case", ["duplicate_late", "out_of_range_late", "negative_seqlen_late"])
def test_update_invalid_entry_past_the_first_block_of_rows(case):
    """An invalid entry beyond the first blockDim rows (the slot check's later rounds) still
    fails the whole call closed: nothing written, CCONV_ERR_INDEX."""
    N, S, D, W, L = 1500, 1600, 512, 4, 3
    x, state, idx, cs, w, b = _inputs(N, S, D, W, L, seed=550, circular=(case == "negative_seqlen_late"), pad=False)
    idx = idx.clone()
    if case == "duplicate_late":
        idx[1400] = idx[3]
    elif case == "out_of_range_late":
        idx[1499] = S
    else:
        cs = cs.clone()
        cs[1333] = -1
    y, st, status = _run(x, state, idx, cs, w, b)
    assert status == 8, case
    assert torch.equal(bits(st), bits(state)), f"{case}: state modified"


@pytest.mark.parametrize("circular", [False, True], ids=["shift", "circular"])
def test_update_staging_dropped_for_a_large_pool(circular):
    """With S near the largest indexed pool the slot check's bit set leaves no LDS room for the
    staged state runs: the default launch drops the staging and stays correct (an explicit
    staged configuration is refused)."""
    N, S, D, W, L = 64, (1 << 19) - 64, 8, 4, 3
    x, state, idx, cs, w, b = _inputs(N, S, D, W, L, seed=560, circular=circular)
    y, st, status = _run(x, state, idx, cs, w, b)
    ok, yr, sr = oracle.update_ex(x, state, idx.numpy(), None if cs is None else cs.numpy(), w, b)
    assert ok and status == 0
    assert torch.equal(bits(st), bits(torch.from_numpy(sr).to(torch.bfloat16)))
    assert_close(y, yr, TOL_FWD, f"S{S} {'circular' if circular else 'shift'}")
    cfg = cc.cconv_default_update_config(N, D)
    assert cfg.options & 4
    with pytest.raises(cc.CconvError):
        cc.cconv_update_config(x.to(DEV), state.to(DEV), idx.to(DEV), w.to(DEV), b.to(DEV), config=cfg,
                               cache_seqlens=None if cs is None else cs.to(DEV))
