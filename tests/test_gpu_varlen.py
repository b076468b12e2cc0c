"""GPU parity of packed variable-length batches (cu_seqlens) through the C ABI.

Sequences of different lengths are packed into one [total, D] tensor; each is convolved on its
own with its own history. Compared with the oracle's oracle_fwd_varlen / oracle_bwd_varlen
element by element (tolerances in parity.py; final states bit for bit). Equal lengths must
reproduce the fixed-length entry points (y and dx bit for bit: the same arithmetic per row),
invalid offsets must leave every output untouched, and the result must not depend on the
launch configuration.
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


def _case(lens, D, W, *, seed, bias=True, history=True):
    total = int(sum(lens))
    inp = si.train_inputs(1, total, D, W, bias=bias, seed=seed)
    x, dy = inp["x"][0], inp["dy"][0]
    h0 = si.history_input(len(lens), D, W, seed=seed) if history else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return x, dy, inp["w"], inp["bias"], h0, cu


def _g(t):
    return None if t is None else t.to(DEV)


def _run(x, dy, w, b, h0, cu, *, cfg_f=None, cfg_b=None, dw_dtype=None):
    y, hT, st = cc.cconv_fwd_varlen(_g(x), _g(cu), _g(w), _g(b), _g(h0), want_final_state=True, config=cfg_f)
    dx, dw, db, dh0, st2 = cc.cconv_bwd_varlen(_g(x), _g(dy), _g(cu), _g(w), _g(b), _g(h0), want_d_init_state=True,
                                               config=cfg_b, dw_dtype=dw_dtype)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    return tuple(None if t is None else t.cpu() for t in (y, hT, dx, dw, db, dh0))


def _check(x, dy, w, b, h0, cu, outs, what):
    y, hT, dx, dw, db, dh0 = outs
    ok, yr, hTr = oracle.fwd_varlen(x, cu.numpy(), w, b, h0)
    ok2, dxr, dwr, dbr, dh0r = oracle.bwd_varlen(x, dy, cu.numpy(), w, b, h0)
    assert ok and ok2
    ey = assert_close(y, yr, TOL_FWD, f"{what} y")
    assert np.array_equal(hT.float().numpy(), hTr), f"{what}: final states differ"
    edx = assert_close(dx, dxr, TOL_BWD, f"{what} dx")
    edw = assert_close(dw, dwr, TOL_BWD, f"{what} dw")
    edb = assert_close(db, dbr, TOL_BWD, f"{what} dbias") if db is not None else 0.0
    edh = assert_close(dh0, dh0r, TOL_BWD, f"{what} d_init_state")
    print(f"{what}: err y {ey:.2e} dx {edx:.2e} dw {edw:.2e} dbias {edb:.2e} dh0 {edh:.2e}", flush=True)


LENS = {
    "mixed": [700, 0, 1, 2, 3, 64, 65, 1000, 5, 0, 1234, 7, 900],
    "short_first": [1, 1, 2, 3000, 2],
    "one": [2500],
    "tails": [63, 64, 65, 127, 128, 129, 31, 33, 17, 900],
}


@pytest.mark.parametrize("name", list(LENS))
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_varlen_parity(name, W):
    x, dy, w, b, h0, cu = _case(LENS[name], 1032, W, seed=200 + W)
    _check(x, dy, w, b, h0, cu, _run(x, dy, w, b, h0, cu), f"{name} W{W}")


def test_varlen_without_history_or_bias():
    x, dy, w, b, h0, cu = _case(LENS["mixed"], 520, 4, seed=210, bias=False, history=False)
    outs = _run(x, dy, w, b, h0, cu)
    assert outs[4] is not None  # dbias is produced even when the forward has no bias
    _check(x, dy, w, b, h0, cu, outs, "no history, no bias")


def test_varlen_equal_lengths_match_batch():
    """B sequences of length T packed: y, dx bit for bit as the [B, T, D] entry points, final
    states and history gradients bit for bit as the history entry points, dw and dbias to
    the tolerance (the partial sums are grouped differently)."""
    B, T, D, W = 4, 1500, 2048, 4
    x, dy, w, b, h0, cu = _case([T] * B, D, W, seed=220)
    y, hT, dx, dw, db, dh0 = _run(x, dy, w, b, h0, cu)
    yb, hTb = cc.cconv_fwd_state(_g(x.view(B, T, D)), _g(w), _g(b), _g(h0))
    dxb, dwb, dbb, dh0b = cc.cconv_bwd_state(_g(x.view(B, T, D)), _g(dy.view(B, T, D)), _g(w), _g(b), _g(h0))
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(yb.view(B * T, D))) and torch.equal(bits(hT), bits(hTb))
    assert torch.equal(bits(dx), bits(dxb.view(B * T, D))) and torch.equal(bits(dh0), bits(dh0b))
    assert_close(dw, dwb.cpu().float(), TOL_BWD, "dw vs batch")
    assert_close(db, dbb.cpu(), TOL_BWD, "dbias vs batch")


@pytest.mark.parametrize(
    "cu",
    [[1, 5, 9], [0, 5, 4, 9], [0, 4, 8], [0, 4, 10], [0, 10, 9], [-1, 4, 9], [0, 2**31 - 1, 9]],
    ids=["start_not_zero", "decreasing", "short_end", "long_end", "decreasing_last", "negative", "huge"],
)
def test_varlen_invalid_offsets_write_nothing(cu):
    total, D, W = 9, 264, 4
    n = len(cu) - 1
    g = torch.Generator().manual_seed(230)
    x = torch.randn(total, D, generator=g).to(torch.bfloat16).to(DEV)
    dy = torch.randn(total, D, generator=g).to(torch.bfloat16).to(DEV)
    w = torch.randn(D, W, generator=g).to(torch.bfloat16).to(DEV)
    h0 = torch.randn(n, D, W - 1, generator=g).to(torch.bfloat16).to(DEV)
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)
    y, ybuf, ylo, yhi = guarded((total, D), torch.bfloat16, DEV)
    hT, hbuf, hlo, hhi = guarded((n, D, W - 1), torch.bfloat16, DEV)
    dx, xbuf, xlo, xhi = guarded((total, D), torch.bfloat16, DEV)
    dw, wbuf, wlo, whi = guarded((D, W), torch.bfloat16, DEV)
    db, bbuf, blo, bhi = guarded((D,), torch.float32, DEV)
    dh, dbuf, dlo, dhi = guarded((n, D, W - 1), torch.bfloat16, DEV)
    _, _, st = cc.cconv_fwd_varlen(x, cud, w, None, h0, final_state=hT, y=y)
    *_, st2 = cc.cconv_bwd_varlen(x, dy, cud, w, None, h0, dx=dx, dw=dw, dbias=db, d_init_state=dh)
    torch.cuda.synchronize()
    assert int(st.item()) == 8 and int(st2.item()) == 8
    for buf in (ybuf, hbuf, xbuf, wbuf, bbuf, dbuf):
        assert canaries_intact(buf, 0, 0), "a rejected call wrote an output"
    assert not oracle.fwd_varlen(x.cpu(), cu, w.cpu(), None, h0.cpu())[0]


CONFIGS_F = [
    dict(vec=8, rows_per_group=8, waves_per_block=1, options=11, seg_rows=64),
    dict(vec=4, rows_per_group=4, waves_per_block=4, options=3, seg_rows=8),
    dict(vec=8, rows_per_group=4, waves_per_block=2, strips_per_block=2, options=3, seg_rows=100),
    dict(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=4096),
]
CONFIGS_B = [
    dict(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=64),
    dict(vec=8, rows_per_group=4, waves_per_block=4, options=3, seg_rows=8),
    dict(vec=4, rows_per_group=8, waves_per_block=8, strips_per_block=2, options=3, seg_rows=24),
    dict(vec=8, rows_per_group=8, waves_per_block=1, options=11, seg_rows=4096),
]


@pytest.mark.parametrize("i", range(4))
def test_varlen_launch_invariance(i):
    """y and dx bit for bit whatever the launch (segments cut sequences anywhere), dw to the
    tolerance."""
    x, dy, w, b, h0, cu = _case(LENS["mixed"], 1032, 4, seed=240)
    ref = _run(x, dy, w, b, h0, cu)
    got = _run(x, dy, w, b, h0, cu, cfg_f=cc.Config(**CONFIGS_F[i]), cfg_b=cc.Config(**CONFIGS_B[i]))
    for k, n in ((0, "y"), (1, "final state"), (2, "dx"), (5, "d_init_state")):
        assert torch.equal(bits(got[k]), bits(ref[k])), f"config {i}: {n} differs"
    assert_close(got[3], ref[3].float(), TOL_BWD, f"config {i} dw")


def test_varlen_many_tiny_sequences():
    """3000 sequences of 0 to 4 rows: every wave crosses many boundaries and histories."""
    rng = np.random.default_rng(250)
    lens = rng.integers(0, 5, 3000).tolist()
    x, dy, w, b, h0, cu = _case(lens, 256, 4, seed=251)
    _check(x, dy, w, b, h0, cu, _run(x, dy, w, b, h0, cu), "tiny sequences")


@pytest.mark.parametrize("D", [65, 264], ids=["narrow_1_lane", "vector_2_lanes"])
def test_varlen_sequence_search_with_few_active_lanes(D):
    """The last channel strip has one active lane (D = 65, one channel per lane) or two (D = 264,
    four channels per lane): the waves of that strip find their first sequence with one or two
    probes per round, over many rounds (300 sequences, empty ones among them)."""
    rng = np.random.default_rng(260 + D)
    lens = rng.integers(0, 40, 300).tolist()
    x, dy, w, b, h0, cu = _case(lens, D, 4, seed=261 + D)
    _check(x, dy, w, b, h0, cu, _run(x, dy, w, b, h0, cu), f"D{D} few active lanes")


def test_varlen_empty_batches():
    D, W = 512, 4
    w = torch.randn(D, W).to(torch.bfloat16).to(DEV)
    x = torch.empty(0, D, dtype=torch.bfloat16, device=DEV)
    # no sequences at all
    y, hT, st = cc.cconv_fwd_varlen(x, torch.zeros(1, dtype=torch.int32, device=DEV), w, None, None,
                                    want_final_state=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and y.shape == (0, D) and hT.shape == (0, D, W - 1)
    # three empty sequences: final state = history, history gradient 0, dw = dbias = 0
    h0 = torch.randn(3, D, W - 1).to(torch.bfloat16).to(DEV)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    _, hT, st = cc.cconv_fwd_varlen(x, cu, w, None, h0, want_final_state=True)
    dx, dw, db, dh0, st2 = cc.cconv_bwd_varlen(x, x, cu, w, None, h0, want_d_init_state=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    assert torch.equal(bits(hT), bits(h0)) and not dh0.any() and not dw.any() and not db.any()


def test_varlen_headline_packed():
    """8 sequences of 8192 rows packed (65536 x 4096): y and dx bit for bit as the fixed-length
    forward and backward of the same rows, dw and dbias to the tolerance."""
    s = si.HEADLINE
    g = si.train_inputs_device(s.B, s.T, s.D, s.W, bias=True, seed=s.seed)
    cu = torch.arange(0, (s.B + 1) * s.T, s.T, dtype=torch.int32, device=DEV)
    xp, dyp = g["x"].view(s.B * s.T, s.D), g["dy"].view(s.B * s.T, s.D)
    y, _, st = cc.cconv_fwd_varlen(xp, cu, g["w"], g["bias"])
    dx, dw, db, _, st2 = cc.cconv_bwd_varlen(xp, dyp, cu, g["w"], g["bias"], dw_dtype=torch.float32)
    yb = cc.cconv_fwd(g["x"], g["w"], g["bias"])
    dxb, dwb, dbb = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], dw_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    assert torch.equal(y.view(torch.int16), yb.view(s.B * s.T, s.D).view(torch.int16))
    assert torch.equal(dx.view(torch.int16), dxb.view(s.B * s.T, s.D).view(torch.int16))
    rel = ((dw - dwb).abs() / dwb.abs().clamp(min=1.0)).max().item()
    relb = ((db - dbb).abs() / dbb.abs().clamp(min=1.0)).max().item()
    assert rel < 1e-4 and relb < 1e-4, (rel, relb)


@pytest.mark.timeout(900)
def test_varlen_headline_mixed_lengths_full_parity():
    """The benchmark's packed workload: 65536 rows of 4096 channels cut into sequences of 1 to
    ~15k rows with histories, against the float64 oracle in full (every y and dx element, all
    final states, dw, dbias and the history gradients)."""
    lens = si.packed_lengths(8 * 8192, seed=si.HEADLINE.seed + 3)
    x, dy, w, b, h0, cu = _case(lens, 4096, 4, seed=270)
    _check(x, dy, w, b, h0, cu, _run(x, dy, w, b, h0, cu), f"packed {len(lens)} sequences, 65536 x 4096")


def test_varlen_graph_replay():
    """The packed forward and backward (offset check, empty-sequence states, streaming kernels,
    reduction) captured in a HIP graph replay bit for bit."""
    x, dy, w, b, h0, cu = _case(LENS["mixed"], 520, 4, seed=260)
    xd, dyd, wd, bd, hd, cud = (_g(t) for t in (x, dy, w, b, h0, cu))
    ref = _run(x, dy, w, b, h0, cu)
    n, (total, D) = cu.numel() - 1, x.shape
    y = torch.empty(total, D, dtype=torch.bfloat16, device=DEV)
    hT = torch.empty(n, D, 3, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(y)
    dw = torch.empty(D, 4, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(D, dtype=torch.float32, device=DEV)
    dh = torch.empty_like(hT)
    ws = torch.empty((cc.cconv_bwd_workspace_bytes(1, total, D, 4) + 3) // 4, dtype=torch.float32, device=DEV)
    st = torch.empty(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cc.cconv_fwd_varlen(xd, cud, wd, bd, hd, final_state=hT, y=y, status=st, stream=s)
        cc.cconv_bwd_varlen(xd, dyd, cud, wd, bd, hd, dx=dx, dw=dw, dbias=db, d_init_state=dh, workspace=ws,
                            status=st, stream=s)
    for r in range(3):
        for t in (y, hT, dx, dw, dh):
            t.view(torch.int16).fill_(0x7FA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for got, want, nm in ((y, ref[0], "y"), (hT, ref[1], "hT"), (dx, ref[2], "dx"), (dw, ref[3], "dw"),
                              (db, ref[4], "dbias"), (dh, ref[5], "dh0")):
            assert torch.equal(bits(got), bits(want)), f"replay {r}: {nm}"


def test_varlen_beyond_2_31_elements():
    """A packed batch of 600,000 rows x 4096 channels (2.5e9 elements, 4.9 GB per tensor) in three
    sequences: y and dx bit for bit as the fixed-length path on the same sequences (zero
    histories), the final states the last rows of each sequence."""
    D, W = 4096, 4
    lens = [300_000, 1, 299_999]
    total = sum(lens)
    assert total * D > 2**31
    g = si.train_inputs_device(1, total, D, W, bias=True, seed=270)
    x, dy = g["x"][0], g["dy"][0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    y, hT, st = cc.cconv_fwd_varlen(x, cu, g["w"], g["bias"], want_final_state=True)
    dx, _, _, _, st2 = cc.cconv_bwd_varlen(x, dy, cu, g["w"], g["bias"])
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    a = 0
    for i, L in enumerate(lens):
        xs, dys = x[a:a + L][None], dy[a:a + L][None]
        yb = cc.cconv_fwd(xs, g["w"], g["bias"])
        dxb, _, _ = cc.cconv_bwd(xs, dys, g["w"], g["bias"])
        torch.cuda.synchronize()
        assert torch.equal(y[a:a + L].view(torch.int16), yb[0].view(torch.int16)), i
        assert torch.equal(dx[a:a + L].view(torch.int16), dxb[0].view(torch.int16)), i
        tail = torch.zeros(W - 1, D, dtype=torch.bfloat16, device=DEV)
        k = min(L, W - 1)
        tail[W - 1 - k:] = x[a + L - k:a + L]
        assert torch.equal(hT[i].view(torch.int16), tail.transpose(0, 1).contiguous().view(torch.int16)), i
        del yb, dxb
        a += L
