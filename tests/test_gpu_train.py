"""GPU parity of the forward and backward against the CPU oracle, through the C ABI.

Sizes the oracle finishes in seconds are compared element by element (every y, dx, dw,
dbias). The 8x8192x4096 workload (and the 16x8192x2048 production call), in the launch
configuration the benchmark times, is compared in full too (every element of y and dx, every
channel of dw and dbias: the multithreaded oracle takes seconds), and also on sampled outputs
the oracle computes one by one (random points plus the sequence start, segment boundaries,
the sequence end and strip edges). Tolerances and the element-wise ulp checks are in
parity.py.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import causal_depthwise_short_amd as cc
import oracle
import synth_inputs as si
from parity import TOL_BWD, TOL_FWD, as_f64, assert_close, bits, canaries_intact, guarded

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def run_train(inp, *, config_fwd=None, config_bwd=None, dw_dtype=None, want_dbias=True):
    g = _gpu(inp)
    y = cc.cconv_fwd(g["x"], g["w"], g["bias"], config=config_fwd)
    dx, dw, db = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], config=config_bwd, dw_dtype=dw_dtype,
                              want_dbias=want_dbias)
    torch.cuda.synchronize()
    return y.cpu(), dx.cpu(), dw.cpu(), (None if db is None else db.cpu())


def check_against_oracle(inp, outs, what):
    y, dx, dw, db = outs
    _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
    dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
    ey = assert_close(y, yr, TOL_FWD, f"{what} y")
    edx = assert_close(dx, dxr, TOL_BWD, f"{what} dx")
    edw = assert_close(dw, dwr, TOL_BWD, f"{what} dw")
    edb = assert_close(db, dbr, TOL_BWD, f"{what} dbias") if db is not None else 0.0
    print(f"{what}: err y {ey:.2e} dx {edx:.2e} dw {edw:.2e} dbias {edb:.2e}", flush=True)


@pytest.mark.parametrize("shape", [si.TINY, si.RAGGED, si.MEDIUM], ids=lambda s: s.name)
def test_parity_full(shape):
    inp = si.train_inputs_for(shape)
    check_against_oracle(inp, run_train(inp), shape.name)


@pytest.fixture(scope="module", params=[si.HEADLINE, si.PRODUCTION], ids=lambda s: s.name)
def headline(request):
    s = request.param
    inp = si.train_inputs_for(s)
    outs = run_train(inp)
    xf = inp["x"].float().numpy()
    dyf = inp["dy"].float().numpy()
    return s, inp, outs, xf, dyf


def _sample_points(s, cfg, rng, n_random=6000):
    B, T, D = s.B, s.T, s.D
    pts = [np.stack([rng.integers(0, B, n_random), rng.integers(0, T, n_random), rng.integers(0, D, n_random)], 1)]
    # sequence start, end, segment boundaries and strip edges
    ts = {0, 1, 2, 3, 4, T - 1, T - 2, T - 3, T - 4}
    for k in range(1, min(64, (T + cfg.seg_rows - 1) // cfg.seg_rows)):
        for off in (-4, -3, -2, -1, 0, 1, 2, 3):
            t = k * cfg.seg_rows + off
            if 0 <= t < T:
                ts.add(t)
    strip = 64 * cfg.vec
    ds = sorted({0, 1, 7, 8, strip - 1, strip, D - 1, D - 8} | set(int(v) for v in rng.integers(0, D, 6)))
    ds = [d for d in ds if 0 <= d < D]
    for b in range(B):
        for t in sorted(ts):
            pts.append(np.array([[b, t, d] for d in ds]))
    p = np.concatenate(pts, 0)
    return p[:, 0], p[:, 1], p[:, 2]


def test_headline_sampled_parity(headline):
    s, inp, (y, dx, dw, db), xf, dyf = headline
    rng = np.random.default_rng(1234)
    cfg_f = cc.cconv_default_config("fwd", s.B, s.T, s.D, s.W)
    pb, pt, pd = _sample_points(s, cfg_f, rng)
    yr = oracle.fwd_points(xf, inp["w"], inp["bias"], pb, pt, pd)
    e1 = assert_close(y[pb, pt, pd], yr, TOL_FWD, f"{s.name} y (sampled)")
    cfg_b = cc.cconv_default_config("bwd", s.B, s.T, s.D, s.W)
    pb, pt, pd = _sample_points(s, cfg_b, rng)
    dxr = oracle.dx_points(xf, dyf, inp["w"], inp["bias"], pb, pt, pd)
    e2 = assert_close(dx[pb, pt, pd], dxr, TOL_BWD, f"{s.name} dx (sampled)")
    ch = np.unique(np.concatenate([rng.integers(0, s.D, 40), [0, 1, 511, 512, s.D - 1]]))
    dwr, dbr = oracle.dw_channels(xf, dyf, inp["w"], inp["bias"], ch)
    e3 = assert_close(dw[ch], dwr, TOL_BWD, f"{s.name} dw (sampled channels)")
    e4 = assert_close(db[ch], dbr, TOL_BWD, f"{s.name} dbias (sampled channels)")
    print(f"{s.name} sampled: err y {e1:.2e} dx {e2:.2e} dw {e3:.2e} dbias {e4:.2e} ({pb.size} points, {ch.size} channels)")


@pytest.mark.timeout(900)
def test_headline_full_parity(headline):
    """Every element of the full-size workload against the float64 oracle, in the launch the
    benchmark times: all of y and dx (the last W-1 rows of every batch row included, where the
    halo reads past T), all channels of dw and dbias, and dw again accumulated to fp32 (the
    tight check of the long sums)."""
    s, inp, (y, dx, dw, db), xf, dyf = headline
    _, yr = oracle.fwd(xf, inp["w"], inp["bias"])
    dxr, dwr, dbr = oracle.bwd(xf, dyf, inp["w"], inp["bias"])
    ey = max(assert_close(y[b], yr[b], TOL_FWD, f"{s.name} y[{b}]") for b in range(s.B))
    del yr
    edx = max(assert_close(dx[b], dxr[b], TOL_BWD, f"{s.name} dx[{b}]") for b in range(s.B))
    del dxr
    edw = assert_close(dw, dwr, TOL_BWD, f"{s.name} dw")
    edb = assert_close(db, dbr, TOL_BWD, f"{s.name} dbias")
    _, _, dw32, _ = run_train(inp, dw_dtype=torch.float32)
    edw32 = assert_close(dw32, dwr, TOL_BWD, f"{s.name} fp32 dw")
    print(f"{s.name} full: err y {ey:.2e} dx {edx:.2e} dw {edw:.2e} dbias {edb:.2e} fp32 dw {edw32:.2e}", flush=True)


def test_headline_outputs_finite_and_deterministic(headline):
    s, inp, (y, dx, dw, db), _, _ = headline
    assert torch.isfinite(y.float()).all() and torch.isfinite(dx.float()).all()
    _, dx2, dw2, db2 = run_train(inp)
    assert torch.equal(bits(dx2), bits(dx)), "dx differs run to run"
    assert torch.equal(bits(dw2), bits(dw)) and torch.equal(bits(db2), bits(db)), "dw/dbias not bitwise reproducible"


@pytest.mark.parametrize("T", [1, 2, 3, 5, 9])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_short_sequences(T, W):
    inp = si.train_inputs(2, T, 64, W, bias=True, seed=100 + T * 4 + W)
    check_against_oracle(inp, run_train(inp), f"T={T} W={W}")


@pytest.mark.parametrize("D", [8, 16, 24, 520, 1032, 2056])
def test_channel_tails(D):
    inp = si.train_inputs(2, 77, D, 4, bias=True, seed=200 + D)
    check_against_oracle(inp, run_train(inp), f"D={D}")


@pytest.mark.parametrize("D", [4104, 4160], ids=["rows_off_lines", "rows_on_lines"])
def test_seventeen_strip_plans(D):
    """D = 4104 and 4160 give 17 channel strips, so the default plan cuts the batch rows into
    segments that fit the wave slots. This call streams less than 256 MB, so it keeps the
    non-temporal hints at both widths; at 4104, whose rows do not start on 128-byte lines, the
    plain-hint plan that large calls take runs too. Against the oracle, every output."""
    B, T = 4, 700
    cf = cc.cconv_default_config("fwd", B, T, D, 4)
    cb = cc.cconv_default_config("bwd", B, T, D, 4)
    assert cf.vec == 4 and cf.options == 11 and cb.options == cf.options
    inp = si.train_inputs(B, T, D, 4, bias=True, seed=130 + D)
    check_against_oracle(inp, run_train(inp), f"D{D}")
    if D == 4104:
        pf = cc.Config(**{**cf.as_dict(), "options": 8})
        pb = cc.Config(**{**cb.as_dict(), "options": 8})
        check_against_oracle(inp, run_train(inp, config_fwd=pf, config_bwd=pb), f"D{D} plain hints")


@pytest.mark.parametrize("split", [(512, 512, 512), (256, 256, 512)])
def test_fused_qkv_one_launch_equals_three(split):
    """A fused q|k|v projection [B, T, Dq + Dk + Dv] convolved in one call (the three taps and
    biases concatenated) equals three calls on its channel slices (row stride Dq + Dk + Dv, no
    copy): y and dx bit for bit (the same arithmetic per channel and row), dw and dbias to the
    tolerance (their fixed-order sums are grouped by a different plan). Splits: equal thirds,
    and a KDA layer's (v twice as wide as q and k) [kernel-fun wheel, cconv/__init__.py
    docstring]."""
    B, T, W = 2, 600, 4
    Dt = sum(split)
    inp = si.train_inputs(B, T, Dt, W, bias=True, seed=150)
    g = _gpu(inp)
    y, (dx, dw, db) = cc.cconv_fwd(g["x"], g["w"], g["bias"]), cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"])
    parts, lo = [], 0
    for Dj in split:
        sl = slice(lo, lo + Dj)
        lo += Dj
        xs, dys = g["x"][:, :, sl], g["dy"][:, :, sl]
        wj, bj = g["w"][sl].contiguous(), g["bias"][sl].contiguous()
        parts.append((cc.cconv_fwd(xs, wj, bj),) + tuple(cc.cconv_bwd(xs, dys, wj, bj)))
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(torch.cat([p[0] for p in parts], dim=2)))
    assert torch.equal(bits(dx), bits(torch.cat([p[1] for p in parts], dim=2)))
    assert_close(dw.cpu(), torch.cat([p[2] for p in parts]).cpu().float(), TOL_BWD, "fused dw")
    assert_close(db.cpu(), torch.cat([p[3] for p in parts]).cpu(), TOL_BWD, "fused dbias")
    check_against_oracle(inp, (y.cpu(), dx.cpu(), dw.cpu(), db.cpu()), "fused q|k|v")


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("w_dtype", [torch.bfloat16, torch.float32], ids=["wbf16", "wf32"])
def test_widths_bias_dtypes(W, bias, w_dtype):
    inp = si.train_inputs(2, 301, 264, W, bias=bias, seed=300 + W, w_dtype=w_dtype)
    for dw_dtype in (torch.bfloat16, torch.float32):
        outs = run_train(inp, dw_dtype=dw_dtype)
        assert outs[2].dtype == dw_dtype
        check_against_oracle(inp, outs, f"W={W} bias={bias} w={w_dtype} dw={dw_dtype}")


def test_binding_rejects_mismatched_outputs():
    """The library sees only addresses: an output of the wrong shape, dtype or layout, or one in
    host memory, is refused by the binding before any launch, and nothing is written."""
    B, T, D, W = 2, 64, 256, 4
    g = _gpu(si.train_inputs(B, T, D, W, bias=True, seed=160))
    x, dy, w, b = g["x"], g["dy"], g["w"], g["bias"]
    small = torch.zeros((B, T - 1, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        cc.cconv_fwd(x, w, b, y=small)
    with pytest.raises(ValueError):
        cc.cconv_bwd(x, dy, w, b, dx=small)
    with pytest.raises(ValueError):
        cc.cconv_bwd(x, dy, w, b, dw=torch.zeros((D, W + 1), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        cc.cconv_bwd(x, dy, w, b, dbias=torch.zeros((D,), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        cc.cconv_bwd(x, dy, w, b, dx=torch.zeros((B, T, D), dtype=torch.bfloat16))  # host memory
    with pytest.raises(ValueError):
        cc.cconv_bwd(x, dy, w, b, dx=torch.zeros((B, T, 2 * D), dtype=torch.bfloat16, device=DEV)[:, :, :D])
    torch.cuda.synchronize()
    assert not small.any()


def test_binding_launches_on_the_current_stream():
    """Without a stream argument the binding launches on torch's current stream (read through
    its raw handle), also inside a side-stream context."""
    assert cc._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert cc._stream(None) == s.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert cc._stream(s) == s.cuda_stream


def test_empty_problems():
    for B, T in [(0, 16), (3, 0)]:
        inp = si.train_inputs(B, T, 64, 4, bias=True, seed=1)
        g = _gpu(inp)
        y = cc.cconv_fwd(g["x"], g["w"], g["bias"])
        dw = torch.full((64, 4), 7.0, dtype=torch.float32, device=DEV)
        db = torch.full((64,), 7.0, dtype=torch.float32, device=DEV)
        dx, dw, db = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], dw=dw, dbias=db)
        torch.cuda.synchronize()
        assert y.numel() == 0 and dx.numel() == 0
        assert not dw.any() and not db.any(), "empty batch/sequence must give zero dw/dbias"


def test_strided_inputs_match_contiguous():
    B, T, D, W = 2, 257, 512, 4
    inp = si.train_inputs(B, T, D, W, bias=True, seed=7)
    g = _gpu(inp)
    wide_x = torch.zeros(B, T, 3 * D, dtype=torch.bfloat16, device=DEV)
    wide_x[:, :, D : 2 * D] = g["x"]
    wide_dy = torch.zeros(B, T + 5, 2 * D, dtype=torch.bfloat16, device=DEV)
    wide_dy[:, :T, :D] = g["dy"]
    xs = wide_x[:, :, D : 2 * D]
    dys = wide_dy[:, :T, :D]
    assert xs.stride() == (T * 3 * D, 3 * D, 1) and dys.stride() == ((T + 5) * 2 * D, 2 * D, 1)
    y = cc.cconv_fwd(xs, g["w"], g["bias"])
    dx, dw, db = cc.cconv_bwd(xs, dys, g["w"], g["bias"])
    y0 = cc.cconv_fwd(g["x"], g["w"], g["bias"])
    dx0, dw0, db0 = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"])
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(y0)) and torch.equal(bits(dx), bits(dx0))
    assert torch.equal(bits(dw), bits(dw0)) and torch.equal(bits(db), bits(db0))


CONFIGS_FWD = [
    dict(vec=8, rows_per_group=8, waves_per_block=4, seg_rows=64),
    dict(vec=8, rows_per_group=4, waves_per_block=1, seg_rows=8),
    dict(vec=8, rows_per_group=8, waves_per_block=8, options=4, seg_rows=96),
    dict(vec=4, rows_per_group=8, waves_per_block=2, seg_rows=40),
    dict(vec=4, rows_per_group=4, waves_per_block=4, seg_rows=1000),
    dict(vec=8, rows_per_group=8, waves_per_block=8, strips_per_block=8, options=7, seg_rows=128),
    dict(vec=4, rows_per_group=4, waves_per_block=4, strips_per_block=2, options=3, seg_rows=200),
    dict(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=128),
]
CONFIGS_BWD = [
    dict(vec=8, rows_per_group=4, waves_per_block=4, seg_rows=64),
    dict(vec=8, rows_per_group=4, waves_per_block=1, options=5, seg_rows=8),
    dict(vec=8, rows_per_group=8, waves_per_block=8, seg_rows=96),
    dict(vec=4, rows_per_group=4, waves_per_block=2, seg_rows=40),
    dict(vec=4, rows_per_group=8, waves_per_block=4, seg_rows=1000),
    dict(vec=8, rows_per_group=4, waves_per_block=8, strips_per_block=2, options=7, seg_rows=64),
    dict(vec=4, rows_per_group=8, waves_per_block=8, strips_per_block=8, options=3, seg_rows=128),
    dict(vec=8, rows_per_group=8, waves_per_block=1, options=15, seg_rows=96),
]


def test_launch_config_invariance():
    """y and dx are bitwise independent of the launch shape; dw/dbias stay within tolerance."""
    inp = si.train_inputs(3, 1000, 2000, 4, bias=True, seed=9)
    base = run_train(inp)
    dwr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])
    for cf, cb in zip(CONFIGS_FWD, CONFIGS_BWD):
        y, dx, dw, db = run_train(inp, config_fwd=cc.Config(**cf), config_bwd=cc.Config(**cb))
        assert torch.equal(bits(y), bits(base[0])), f"y depends on launch config {cf}"
        assert torch.equal(bits(dx), bits(base[1])), f"dx depends on launch config {cb}"
        assert_close(dw, dwr[1], TOL_BWD, f"dw under {cb}")
        assert_close(db, dwr[2], TOL_BWD, f"dbias under {cb}")
        _, _, dw2, db2 = run_train(inp, config_bwd=cc.Config(**cb))
        assert torch.equal(bits(dw2), bits(dw)) and torch.equal(bits(db2), bits(db)), f"dw not reproducible {cb}"


def test_w2_equals_zero_padded_w4():
    """W=2 equals W=4 with zero taps on the oldest side (the pages' w2 check)."""
    inp2 = si.train_inputs(2, 500, 512, 2, bias=True, seed=11)
    inp4 = dict(inp2)
    w4 = torch.zeros(512, 4, dtype=torch.bfloat16)
    w4[:, 2:] = inp2["w"]
    inp4["w"] = w4
    y2, dx2, dw2, db2 = run_train(inp2)
    y4, dx4, dw4, db4 = run_train(inp4)
    assert torch.equal(y2.float(), y4.float()) and torch.equal(dx2.float(), dx4.float())
    assert torch.equal(bits(dw2), bits(dw4[:, 2:].contiguous())) and torch.equal(bits(db2), bits(db4))
    assert not dw4[:, :2].isnan().any()


def test_guard_bands_and_inputs_untouched():
    B, T, D, W = 3, 1000, 2000, 2
    inp = si.train_inputs(B, T, D, W, bias=True, seed=13)
    g = _gpu(inp)
    keep = {k: bits(v) for k, v in g.items() if v is not None}
    y, ybuf, ylo, yhi = guarded((B, T, D), torch.bfloat16, DEV)
    dx, dxbuf, dxlo, dxhi = guarded((B, T, D), torch.bfloat16, DEV)
    dw, dwbuf, dwlo, dwhi = guarded((D, W), torch.bfloat16, DEV)
    db, dbbuf, dblo, dbhi = guarded((D,), torch.float32, DEV)
    cc.cconv_fwd(g["x"], g["w"], g["bias"], y=y)
    cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], dx=dx, dw=dw, dbias=db)
    torch.cuda.synchronize()
    for name, (buf, lo, hi) in {"y": (ybuf, ylo, yhi), "dx": (dxbuf, dxlo, dxhi), "dw": (dwbuf, dwlo, dwhi),
                                "dbias": (dbbuf, dblo, dbhi)}.items():
        assert canaries_intact(buf, lo, hi), f"{name} written outside its extent"
    for k, v in g.items():
        if v is not None:
            assert torch.equal(bits(v), keep[k]), f"input {k} modified"
    check_against_oracle(inp, (y.cpu(), dx.cpu(), dw.cpu(), db.cpu()), "guarded")


def test_graph_capture_replay_bitwise():
    """fwd + bwd captured into a HIP graph on their first call replay bit-identically."""
    B, T, D, W = 2, 600, 1024, 4
    inp = si.train_inputs(B, T, D, W, bias=True, seed=17)
    g = _gpu(inp)
    eager = run_train(inp)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    y = torch.empty(B, T, D, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(y)
    dw = torch.empty(D, W, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(D, dtype=torch.float32, device=DEV)
    ws = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, D, W) // 4, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        cc.cconv_fwd(g["x"], g["w"], g["bias"], y=y)
        cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], dx=dx, dw=dw, dbias=db, workspace=ws)
    for rep in range(3):
        for t in (y, dx, dw, db):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = (y.cpu(), dx.cpu(), dw.cpu(), db.cpu())
        for a, b_, name in zip(got, eager, ("y", "dx", "dw", "dbias")):
            assert torch.equal(bits(a), bits(b_)), f"graph replay {rep}: {name} differs from eager"
        _ = run_train(inp)  # eager work between replays


def test_two_stage_backward_equals_fused():
    B, T, D, W = 3, 1000, 2000, 2
    inp = si.train_inputs(B, T, D, W, bias=True, seed=19)
    g = _gpu(inp)
    dx0, dw0, db0 = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"])
    ws = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, D, W) // 4, dtype=torch.float32, device=DEV)
    dx = torch.empty_like(dx0)
    dw = torch.empty_like(dw0)
    db = torch.empty_like(db0)
    cc.cconv_bwd_main(g["x"], g["dy"], g["w"], g["bias"], dx, ws)
    cc.cconv_bwd_finish(ws, dw, db, B, T, D, W)
    torch.cuda.synchronize()
    assert torch.equal(bits(dx), bits(dx0)) and torch.equal(bits(dw), bits(dw0)) and torch.equal(bits(db), bits(db0))


def test_launch_options_do_not_change_results():
    inp = si.train_inputs(2, 700, 1024, 4, bias=True, seed=23)
    base = run_train(inp)
    for h in range(1, 16):
        wpb = 1 if h & 8 else 2
        cf = cc.Config(vec=8, rows_per_group=8, waves_per_block=wpb, options=h, seg_rows=128)
        cb = cc.Config(vec=4, rows_per_group=8, waves_per_block=wpb, options=h, seg_rows=128)
        y, dx, _, _ = run_train(inp, config_fwd=cf, config_bwd=cb)
        assert torch.equal(bits(y), bits(base[0])) and torch.equal(bits(dx), bits(base[1])), f"options {h}"


def test_offsets_beyond_2_31_elements():
    """B*T*D > 2^31 (4.3 GB per tensor, ragged last segment): every offset is 64-bit. Checked
    against the oracle on windows of the full tensors around sampled points and on full
    per-channel sums for sampled channels."""
    B, T, D, W = 2, 262151, 4096, 4
    assert B * T * D > 2**31
    g = si.train_inputs_device(B, T, D, W, bias=True, seed=31)
    y = cc.cconv_fwd(g["x"], g["w"], g["bias"])
    dx, dw, db = cc.cconv_bwd(g["x"], g["dy"], g["w"], g["bias"], dw_dtype=torch.float32)
    torch.cuda.synchronize()
    w_h, b_h = g["w"].cpu(), g["bias"].cpu()
    rng = np.random.default_rng(5)
    pts = [(b_, t, d) for b_, t, d in zip(rng.integers(0, B, 40), rng.integers(0, T, 40), rng.integers(0, D, 40))]
    pts += [(1, T - 1, D - 1), (1, T - 4, 4095), (0, 0, 0), (1, 3, 777)]
    for b_, t, d in pts:
        b_, t, d = int(b_), int(t), int(d)
        lo, hi = max(0, t - (W - 1)), min(T, t + W)
        xw = g["x"][b_ : b_ + 1, max(0, lo - (W - 1)) : hi].cpu()
        dyw = g["dy"][b_ : b_ + 1, max(0, lo - (W - 1)) : hi].cpu()
        off = t - max(0, lo - (W - 1))
        # windows start at the sequence start or at least W-1 rows before every row they
        # answer for, and end at the sequence end or W-1 rows after it
        _, yr = oracle.fwd(xw, w_h, b_h)
        assert abs(float(y[b_, t, d]) - yr[0, off, d]) <= TOL_FWD * max(1.0, abs(yr[0, off, d])), (b_, t, d)
        if hi == T or hi - t >= W:
            dxr, _, _ = oracle.bwd(xw, dyw, w_h, b_h)
            assert abs(float(dx[b_, t, d]) - dxr[0, off, d]) <= TOL_BWD * max(1.0, abs(dxr[0, off, d])), (b_, t, d)
    for d in (0, 1, 2047, 4095):
        xc = g["x"][:, :, d : d + 1].cpu()
        dyc = g["dy"][:, :, d : d + 1].cpu()
        dwr, dbr = oracle.dw_channels(xc, dyc, w_h[d : d + 1], b_h[d : d + 1], [0])
        assert_close(dw[d : d + 1].cpu(), dwr, TOL_BWD, f"dw channel {d}")
        assert_close(db[d : d + 1].cpu(), dbr, TOL_BWD, f"dbias channel {d}")


def test_very_wide_channels():
    inp = si.train_inputs(1, 33, 131072, 3, bias=True, seed=37)
    check_against_oracle(inp, run_train(inp), "D=131072")
