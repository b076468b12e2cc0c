"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each check takes an ``oracle.Oracle`` and raises AssertionError when it disagrees. The test
suite runs every check on the real oracle (tests/test_oracle_pins.py) and on copies of the
oracle with a planted mistake (tests/test_oracle_mutants.py), where at least one check must
fail. Nothing here retypes the oracle's formulas: the pins are a library convolution with
autograd (float64 torch), finite differences, hand-worked fixtures, impulses, closed forms,
exact invariants and torch's own bf16 cast.
"""

from __future__ import annotations

import math
from pathlib import Path

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = Path(__file__).resolve().parent / "golden"


# ----------------------------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------------------------


def _bf16_values(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """Random values that are exactly bf16 (so that fp32 holds them and small shifts are exact)."""
    a = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return a.to(torch.bfloat16).float().numpy()


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _dsilu(z):
    s = _sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _problem(seed, B, T, D, W, bias=True, wscale=None):
    rng = np.random.default_rng(seed)
    x = _bf16_values(rng, (B, T, D))
    w = _bf16_values(rng, (D, W), wscale if wscale is not None else 1.0 / math.sqrt(W))
    b = _bf16_values(rng, (D,), 0.3) if bias else None
    dy = _bf16_values(rng, (B, T, D))
    return x, w, b, dy


def _torch_reference(x, w, b, dy):
    """float64 torch: grouped conv1d (cross-correlation) with W-1 left zeros, SiLU, autograd."""
    B, T, D = x.shape
    W = w.shape[1]
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True) if b is not None else None
    z = F.conv1d(xt.transpose(1, 2), wt[:, None, :], bt, padding=W - 1, groups=D)[..., :T]
    y = F.silu(z).transpose(1, 2)
    loss = (y * torch.tensor(dy, dtype=torch.float64)).sum()
    loss.backward()
    return (
        y.detach().numpy(),
        xt.grad.numpy(),
        wt.grad.numpy(),
        None if bt is None else bt.grad.numpy(),
    )


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    worst = np.max(err - bound) if err.size else 0.0
    assert worst <= 0.0, f"{what}: max err {np.max(err) if err.size else 0:.3e} exceeds rtol={rtol}, atol={atol}"


def _read_fixture(name):
    rows = []
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        rows.append((key, [float(v) for v in vals]))
    return rows


# ----------------------------------------------------------------------------------------------
# checks
# ----------------------------------------------------------------------------------------------


def check_rounding_matches_torch(orc):
    """RTNE to bf16 equals torch's fp32 -> bf16 cast on random values, exact ties, specials."""
    rng = np.random.default_rng(11)
    n = 200_000
    rand = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    pat = rng.integers(0, 0x7F80, 50_000).astype(np.uint32)
    ties = ((pat << 16) | 0x8000).view(np.float32)
    near = np.concatenate([((pat << 16) | 0x7FFF).view(np.float32), ((pat << 16) | 0x8001).view(np.float32)])
    specials = np.array(
        [0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1.1754942e-38, 3.4028235e38, -3.4028235e38, 1.0, -1.0],
        dtype=np.float32,
    )
    a = np.concatenate([rand, ties, -ties, near, specials])
    want = torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for prec in ("f64", "f32"):
        got = orc.round_bf16(a.astype(np.float64) if prec == "f64" else a, precision=prec)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{prec} rounding differs from torch at {a[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"
    nan = orc.round_bf16(np.array([np.nan]), precision="f64")
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x007F) != 0, "NaN must stay NaN"


def check_rounding_from_double_is_direct(orc):
    """A double just above a bf16 tie rounds up: rounding must not pass through fp32 first."""
    lo = 1.0  # bf16 neighbours 1.0 and 1.0078125; tie at 1.00390625
    v = np.array([1.00390625 + 2.0**-40, 1.00390625 - 2.0**-40, 1.00390625, 1.01171875])
    got = orc.round_bf16(v, precision="f64")
    want = np.array([0x3F81, 0x3F80, 0x3F80, 0x3F82], dtype=np.uint16)  # last: tie 1.0117 -> even 1.015625
    assert lo == 1.0 and np.array_equal(got, want), f"{got} vs {want}"


def check_worked_example(orc):
    """Hand-worked W=3 example (tests/golden/worked_example_w3.txt): z exact, y, dx, dw, dbias."""
    rows = _read_fixture("worked_example_w3.txt")
    kv = {}
    cases = []
    for key, vals in rows:
        if key == "case":
            cases.append({"t": int(vals[0])})
        elif cases:
            cases[-1][key] = vals
        else:
            kv[key] = vals
    W = int(kv["W"][0])
    x = np.array(kv["x"], np.float32).reshape(1, -1, 1)
    T = x.shape[1]
    w = np.array(kv["w"], np.float32).reshape(1, W)
    b = np.array(kv["bias"], np.float32)
    zwant = np.array(kv["z"])
    z, y = orc.fwd(x, w, b)
    assert np.array_equal(z[0, :, 0], zwant), f"z {z[0, :, 0]} vs {zwant}"
    _close(y[0, :, 0], zwant * _sigmoid(zwant), 1e-14, what="worked y")
    for c in cases:
        dy = np.zeros_like(x)
        dy[0, c["t"], 0] = 1.0
        g = _dsilu(zwant[c["t"]])
        dx, dw, db = orc.bwd(x, dy, w, b)
        _close(dx[0, :, 0], np.array(c["dx_over_g"]) * g, 1e-14, 1e-300, what=f"worked dx t={c['t']}")
        _close(dw[0], np.array(c["dw_over_g"]) * g, 1e-14, 1e-300, what=f"worked dw t={c['t']}")
        _close(db, [g], 1e-14, what=f"worked dbias t={c['t']}")
    assert T == 5


def check_impulse(orc):
    """x = 1 at one (b, t0, d), bias 0: z[t0+k] = w[d, W-1-k] for k < W, exactly, else 0."""
    for W in (1, 2, 3, 4):
        rng = np.random.default_rng(20 + W)
        B, T, D = 2, 12, 3
        w = _bf16_values(rng, (D, W))
        x = np.zeros((B, T, D), np.float32)
        b0, t0, d0 = 1, 5, 2
        x[b0, t0, d0] = 1.0
        z, _ = orc.fwd(x, w, None)
        want = np.zeros((B, T, D))
        for k in range(W):
            want[b0, t0 + k, d0] = w[d0, W - 1 - k]
        assert np.array_equal(z, want), f"impulse W={W}"


def check_w1_closed_form(orc):
    """W = 1 is pointwise: y = silu(w[d,0] * x + bias[d])."""
    x, w, b, _ = _problem(3, 2, 17, 6, 1)
    z, y = orc.fwd(x, w, b)
    zz = b.astype(np.float64) + w[:, 0].astype(np.float64) * x.astype(np.float64)
    assert np.array_equal(z, zz), "W=1 z"
    _close(y, zz * _sigmoid(zz), 1e-14, 1e-300, what="W=1 y")


def check_constant_input(orc):
    """x = c everywhere: z[t] = bias + c * (sum of the taps that see rows >= 0)."""
    for W in (2, 3, 4):
        rng = np.random.default_rng(30 + W)
        B, T, D = 1, 9, 4
        c = 0.75
        x = np.full((B, T, D), c, np.float32)
        w = _bf16_values(rng, (D, W))
        b = _bf16_values(rng, (D,), 0.3)
        z, _ = orc.fwd(x, w, b)
        for t in range(T):
            first = max(0, W - 1 - t)  # taps j with t-(W-1)+j >= 0
            want = b.astype(np.float64) + c * w[:, first:].astype(np.float64).sum(axis=1)
            _close(z[0, t], want, 1e-14, 1e-15, what=f"constant W={W} t={t}")


def check_torch_conv1d(orc):
    """float64 torch conv1d(groups=D, left pad W-1) + SiLU + autograd: y, dx, dw, dbias."""
    for W in (1, 2, 3, 4):
        for bias in (True, False):
            x, w, b, dy = _problem(40 + W, 2, 37, 5, W, bias)
            y_t, dx_t, dw_t, db_t = _torch_reference(x, w, b, dy)
            _, y = orc.fwd(x, w, b)
            dx, dw, db = orc.bwd(x, dy, w, b)
            _close(y, y_t, 1e-12, 1e-14, what=f"torch y W={W}")
            _close(dx, dx_t, 1e-12, 1e-13, what=f"torch dx W={W}")
            _close(dw, dw_t, 1e-12, 1e-12, what=f"torch dw W={W}")
            if bias:
                _close(db, db_t, 1e-12, 1e-12, what=f"torch dbias W={W}")
            else:
                # with no bias the returned dbias is still sum(g): compare against torch's
                # gradient of a zero bias
                _, _, _, db0 = _torch_reference(x, w, np.zeros(x.shape[2], np.float32), dy)
                _close(db, db0, 1e-12, 1e-12, what=f"torch dbias (no bias) W={W}")


def check_finite_differences(orc):
    """Central differences of L = sum(dy * y) in fp64, Richardson-extrapolated (h = 2^-10 and
    2^-11: exact shifts of bf16 values), against the analytic dx, dw, dbias."""
    h = 2.0**-10

    def fd(loss, arr, i):
        def central(hh):
            p, m = arr.copy(), arr.copy()
            p[i] += hh
            m[i] -= hh
            return (loss(p) - loss(m)) / (2 * hh)

        return (4 * central(h / 2) - central(h)) / 3

    for W in (1, 2, 3, 4):
        for bias in (True, False):
            x, w, b, dy = _problem(50 + W, 2, 7, 3, W, bias)
            dx, dw, db = orc.bwd(x, dy, w, b)

            def loss(xx, ww, bb):
                _, y = orc.fwd(xx, ww, bb)
                return float(np.sum(dy.astype(np.float64) * y))

            fdx = np.array([fd(lambda a: loss(a, w, b), x, i) for i in np.ndindex(x.shape)]).reshape(x.shape)
            _close(dx, fdx, 1e-6, 1e-8, what=f"FD dx W={W}")
            fdw = np.array([fd(lambda a: loss(x, a, b), w, i) for i in np.ndindex(w.shape)]).reshape(w.shape)
            _close(dw, fdw, 1e-6, 1e-8, what=f"FD dw W={W}")
            if bias:
                fdb = np.array([fd(lambda a: loss(x, w, a), b, (i,)) for i in range(b.shape[0])])
                _close(db, fdb, 1e-6, 1e-8, what=f"FD dbias W={W}")


def check_w_padding(orc):
    """W = 2 equals W = 4 with zero taps on the oldest side, exactly (y, dx; dw[:, 2:])."""
    x, w2, b, dy = _problem(60, 2, 19, 5, 2, True)
    w4 = np.zeros((5, 4), np.float32)
    w4[:, 2:] = w2
    _, y2 = orc.fwd(x, w2, b)
    _, y4 = orc.fwd(x, w4, b)
    assert np.array_equal(y2, y4), "padded y"
    dx2, dw2, db2 = orc.bwd(x, dy, w2, b)
    dx4, dw4, db4 = orc.bwd(x, dy, w4, b)
    assert np.array_equal(dx2, dx4), "padded dx"
    assert np.array_equal(dw2, dw4[:, 2:]), "padded dw"
    assert np.array_equal(db2, db4), "padded dbias"


def check_dbias_is_dw_of_unit_input(orc):
    """With W = 1 and x = 1 everywhere, dw[:, 0] = sum g * 1 = dbias, exactly."""
    rng = np.random.default_rng(70)
    B, T, D = 2, 11, 4
    x = np.ones((B, T, D), np.float32)
    w = _bf16_values(rng, (D, 1))
    b = _bf16_values(rng, (D,), 0.3)
    dy = _bf16_values(rng, (B, T, D))
    _, dw, db = orc.bwd(x, dy, w, b)
    assert np.array_equal(dw[:, 0], db), "dbias vs dw with unit input"


def check_channel_and_batch_independence(orc):
    """Permuting channels permutes every output exactly; each batch row stands alone."""
    x, w, b, dy = _problem(80, 3, 13, 6, 4, True)
    perm = np.array([3, 0, 5, 1, 4, 2])
    _, y = orc.fwd(x, w, b)
    dx, dw, db = orc.bwd(x, dy, w, b)
    _, yp = orc.fwd(x[:, :, perm], w[perm], b[perm])
    dxp, dwp, dbp = orc.bwd(x[:, :, perm], dy[:, :, perm], w[perm], b[perm])
    assert np.array_equal(yp, y[:, :, perm]) and np.array_equal(dxp, dx[:, :, perm])
    assert np.array_equal(dwp, dw[perm]) and np.array_equal(dbp, db[perm])
    dw_sum = np.zeros_like(dw)
    for bi in range(3):
        _, y1 = orc.fwd(x[bi : bi + 1], w, b)
        dx1, dw1, _ = orc.bwd(x[bi : bi + 1], dy[bi : bi + 1], w, b)
        assert np.array_equal(y1[0], y[bi]) and np.array_equal(dx1[0], dx[bi]), f"batch row {bi}"
        dw_sum += dw1
    _close(dw, dw_sum, 1e-12, 1e-12, what="dw = sum over batch rows")


def check_decode_equals_forward(orc):
    """Token-by-token decode from a zero state reproduces the forward bitwise; the final state
    holds the last W-1 inputs (zero-filled when T < W-1); untouched slots stay as they were."""
    for W in (1, 2, 3, 4):
        for T in (7, 2):
            x, w, b, _ = _problem(90 + W + T, 3, T, 5, W, True)
            _, yf = orc.fwd(x, w, b)
            S = 5
            idx = np.array([3, 0, 4], np.int32)
            rng = np.random.default_rng(7)
            state = np.zeros((S, 5, W - 1), np.float32)
            other = _bf16_values(rng, (5, W - 1))
            state[1] = other  # a slot no row touches
            for t in range(T):
                ok, y, state = orc.update(x[:, t, :], state, idx, w, b)
                assert ok, "valid indices rejected"
                assert np.array_equal(y, yf[:, t, :]), f"decode != forward at W={W} t={t}"
            for r, s in enumerate(idx):
                hist = np.zeros((W - 1, 5), np.float32)
                for j in range(W - 1):
                    tt = T - (W - 1) + j
                    if tt >= 0:
                        hist[j] = x[r, tt]
                assert np.array_equal(state[s], hist.T), f"final state W={W} T={T} row {r}"
            assert np.array_equal(state[1], other) and not np.any(state[2]), "untouched slots changed"


def check_decode_worked_example(orc):
    """Hand-worked decode (tests/golden/worked_example_decode_w4.txt)."""
    kv = dict(_read_fixture("worked_example_decode_w4.txt"))
    W = int(kv["W"][0])
    state = np.array(kv["state"], np.float32).reshape(1, 1, W - 1)
    x = np.array(kv["x"], np.float32).reshape(1, 1)
    w = np.array(kv["w"], np.float32).reshape(1, W)
    ok, y, st = orc.update(x, state, None, w, None)
    z = kv["z"][0]
    assert ok
    _close(y[0, 0], z * _sigmoid(z), 1e-14, what="decode worked y")
    assert np.array_equal(st[0, 0], np.array(kv["new_state"], np.float32)), f"state {st[0, 0]}"


def check_decode_index_validation(orc):
    """Indices outside [-1, S) or repeated make the call fail and change nothing; -1 rows give
    zero output and touch no slot; NULL indices are the identity and need N <= S."""
    N, S, D, W = 4, 6, 3, 4
    rng = np.random.default_rng(100)
    x = _bf16_values(rng, (N, D))
    w = _bf16_values(rng, (D, W))
    b = _bf16_values(rng, (D,), 0.3)
    state = _bf16_values(rng, (S, D, W - 1))
    for bad in ([0, 1, -2, 3], [0, 1, 6, 3], [0, 5, 2, 5], [7, 0, 1, 2], [-1, -3, 0, 1]):
        ok, y, st = orc.update(x, state, np.array(bad, np.int32), w, b)
        assert not ok and y is None and np.array_equal(st, state), f"invalid {bad} accepted"
    ok, y, st = orc.update(x, state, np.array([2, -1, 5, -1], np.int32), w, b)
    assert ok
    assert not np.any(y[1]) and not np.any(y[3]), "padding rows must output 0"
    for s in (0, 1, 3, 4):
        assert np.array_equal(st[s], state[s]), f"slot {s} touched"
    assert not np.array_equal(st[2], state[2]) and not np.array_equal(st[5], state[5])
    ok, y, st = orc.update(x, state, None, w, b)
    assert ok and np.array_equal(st[4:], state[4:]) and not np.array_equal(st[0], state[0])
    ok, _, _ = orc.update(_bf16_values(rng, (S + 1, D)), state, None, w, b)
    assert not ok, "identity mapping with N > S accepted"


def check_points_match_full(orc):
    """The sampled entry points agree exactly with the full ones."""
    x, w, b, dy = _problem(110, 2, 23, 7, 3, True)
    _, y = orc.fwd(x, w, b)
    dx, dw, db = orc.bwd(x, dy, w, b)
    pb, pt, pd = np.meshgrid(np.arange(2), np.arange(23), np.arange(7), indexing="ij")
    pb, pt, pd = pb.ravel(), pt.ravel(), pd.ravel()
    assert np.array_equal(orc.fwd_points(x, w, b, pb, pt, pd), y[pb, pt, pd])
    assert np.array_equal(orc.dx_points(x, dy, w, b, pb, pt, pd), dx[pb, pt, pd])
    dwc, dbc = orc.dw_channels(x, dy, w, b, np.arange(7)[::-1])
    assert np.array_equal(dwc, dw[::-1]) and np.array_equal(dbc, db[::-1])


def check_f32_close_to_f64(orc):
    """The fp32 build agrees with the fp64 build far inside the parity tolerances."""
    x, w, b, dy = _problem(120, 2, 64, 16, 4, True)
    _, y64 = orc.fwd(x, w, b, precision="f64")
    _, y32 = orc.fwd(x, w, b, precision="f32")
    dx64, dw64, db64 = orc.bwd(x, dy, w, b, precision="f64")
    dx32, dw32, db32 = orc.bwd(x, dy, w, b, precision="f32")
    _close(y32, y64, 1e-5, 1e-6, what="f32 y")
    _close(dx32, dx64, 1e-5, 1e-6, what="f32 dx")
    _close(dw32, dw64, 1e-5, 1e-5, what="f32 dw")
    _close(db32, db64, 1e-5, 1e-5, what="f32 dbias")


def _problem_h0(seed, B, T, D, W, bias=True):
    x, w, b, dy = _problem(seed, B, T, D, W, bias)
    rng = np.random.default_rng(seed + 1000)
    h0 = _bf16_values(rng, (B, D, W - 1))
    return x, h0, w, b, dy


def check_history_torch(orc):
    """float64 torch conv1d (no padding) over the history followed by x, SiLU, autograd: y, the
    final state (the last W-1 inputs), dx, dw, dbias and the history's gradient."""
    for W in (1, 2, 3, 4):
        for T in (1, 2, 13):
            x, h0, w, b, dy = _problem_h0(140 + W + T, 2, T, 5, W)
            B, _, D = x.shape
            xe = torch.cat([torch.tensor(h0, dtype=torch.float64).permute(0, 2, 1), torch.tensor(x, dtype=torch.float64)], 1)
            xe.requires_grad_(True)
            wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
            bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
            z = F.conv1d(xe.transpose(1, 2), wt[:, None, :], bt, padding=0, groups=D)
            y_t = F.silu(z).transpose(1, 2)
            (y_t * torch.tensor(dy, dtype=torch.float64)).sum().backward()
            y, hT = orc.fwd_state(x, h0, w, b)
            _close(y, y_t.detach().numpy(), 1e-12, 1e-14, what=f"history y W={W} T={T}")
            want_hT = xe.detach()[:, T:, :].permute(0, 2, 1).numpy()  # the last W-1 rows of [h0; x]
            assert np.array_equal(hT.astype(np.float64), want_hT), f"final state W={W} T={T}"
            dx, dw, db, dh0 = orc.bwd_state(x, h0, dy, w, b)
            ge = xe.grad.numpy()
            _close(dx, ge[:, W - 1 :, :], 1e-12, 1e-13, what=f"history dx W={W} T={T}")
            _close(dh0, ge[:, : W - 1, :].transpose(0, 2, 1), 1e-12, 1e-13, what=f"history dh0 W={W} T={T}")
            _close(dw, wt.grad.numpy(), 1e-12, 1e-12, what=f"history dw W={W} T={T}")
            _close(db, bt.grad.numpy(), 1e-12, 1e-12, what=f"history dbias W={W} T={T}")


def check_history_chunking(orc):
    """Processing a sequence in two chunks, the second starting from the first's final state,
    equals processing it whole: y and the final state exactly; dx exactly on the second chunk
    and, on the first, after adding the second chunk's history gradient; dw as a sum."""
    for W in (2, 3, 4):
        x, h0, w, b, dy = _problem_h0(160 + W, 2, 17, 4, W)
        T1 = 9
        y, hT = orc.fwd_state(x, h0, w, b)
        y1, h1 = orc.fwd_state(x[:, :T1], h0, w, b)
        y2, h2 = orc.fwd_state(x[:, T1:], h1, w, b)
        assert np.array_equal(y, np.concatenate([y1, y2], 1)) and np.array_equal(hT, h2), f"chunked forward W={W}"
        dx, dw, db, dh0 = orc.bwd_state(x, h0, dy, w, b)
        dx1, dw1, db1, dh01 = orc.bwd_state(x[:, :T1], h0, dy[:, :T1], w, b)
        dx2, dw2, db2, dh02 = orc.bwd_state(x[:, T1:], h1, dy[:, T1:], w, b)
        assert np.array_equal(dx[:, T1:], dx2), f"chunked dx (second chunk) W={W}"
        joined = dx1.copy()
        joined[:, T1 - (W - 1) :, :] += dh02.transpose(0, 2, 1)
        _close(dx[:, :T1], joined, 1e-12, 1e-13, what=f"chunked dx (first chunk) W={W}")
        assert np.array_equal(dh0, dh01), f"chunked history gradient W={W}"
        _close(dw, dw1 + dw2, 1e-12, 1e-12, what=f"chunked dw W={W}")
        _close(db, db1 + db2, 1e-12, 1e-12, what=f"chunked dbias W={W}")


def check_history_zero_is_plain(orc):
    """A zero history is the plain op, exactly; the history gradient is dx at the W-1 rows
    before t = 0 (equal to the plain op's gradient of a zero-padded input)."""
    x, _, w, b, dy = _problem_h0(180, 2, 11, 5, 4)
    z0 = np.zeros((2, 5, 3), np.float32)
    _, y = orc.fwd(x, w, b)
    ys, _ = orc.fwd_state(x, z0, w, b)
    ysn, _ = orc.fwd_state(x, None, w, b)
    assert np.array_equal(y, ys) and np.array_equal(y, ysn)
    dx, dw, db = orc.bwd(x, dy, w, b)
    dxs, dws, dbs, dh0 = orc.bwd_state(x, z0, dy, w, b)
    assert np.array_equal(dx, dxs) and np.array_equal(dw, dws) and np.array_equal(db, dbs)
    xp = np.concatenate([np.zeros((2, 3, 5), np.float32), x], 1)
    dyp = np.concatenate([np.zeros((2, 3, 5), np.float32), dy], 1)
    dxp, _, _ = orc.bwd(xp, dyp, w, b)
    assert np.array_equal(dh0, dxp[:, :3].transpose(0, 2, 1)), "history gradient vs zero-padded input"


def check_prefill_then_decode(orc):
    """A prefill from a history, then token-by-token decode from its final state, reproduces
    the forward of the whole extended sequence bitwise (in the oracle)."""
    for W in (2, 4):
        x, h0, w, b, _ = _problem_h0(190 + W, 3, 12, 6, W)
        T1 = 7
        y, hT = orc.fwd_state(x, h0, w, b)
        _, state = orc.fwd_state(x[:, :T1], h0, w, b)
        for t in range(T1, 12):
            ok, yt, state = orc.update(x[:, t], state, None, w, b)
            assert ok and np.array_equal(yt, y[:, t]), f"decode after prefill W={W} t={t}"
        assert np.array_equal(state, hT), f"final state after decode W={W}"


def check_pool_matches_gathered_history(orc):
    """Prefill into a decode pool is the forward with history gathered from the slots (zeros
    for -1 or has_initial_state = 0), with each final state scattered back to its slot; slots
    no sequence names are untouched."""
    for W in (2, 3, 4):
        B, T, D, S = 4, 9, 5, 7
        x, w, b, _ = _problem(300 + W, B, T, D, W)
        rng = np.random.default_rng(310 + W)
        state = _bf16_values(rng, (S, D, W - 1))
        idx = np.array([5, -1, 0, 3], np.int32)
        for has in (np.array([1, 1, 0, 1], np.uint8), None):
            ok, y, st = orc.fwd_pool(x, state, idx, has, w, b)
            assert ok
            h0 = np.zeros((B, D, W - 1), np.float32)
            for i in range(B):
                if idx[i] >= 0 and has is not None and has[i]:
                    h0[i] = state[idx[i]]
            yr, hT = orc.fwd_state(x, h0, w, b)
            assert np.array_equal(y, yr), f"pool y W={W}"
            for i in range(B):
                if idx[i] >= 0:
                    assert np.array_equal(st[idx[i]], hT[i]), f"slot {idx[i]} W={W}"
            for sl in (1, 2, 4, 6):
                assert np.array_equal(st[sl], state[sl]), f"slot {sl} touched W={W}"
            # by hand: a sequence's final state is its last W-1 inputs (T >= W-1 here)
            assert np.array_equal(st[5], x[0, T - (W - 1):].T), f"slot 5 by hand W={W}"


def check_pool_prefill_then_decode(orc):
    """Chunked prefill through the pool (second chunk with has_initial_state) and then decode
    from the pool reproduce the plain forward of the whole sequence bitwise (in the oracle)."""
    for W in (2, 4):
        B, T, D, S = 3, 14, 6, 5
        x, w, b, _ = _problem(320 + W, B, T, D, W)
        rng = np.random.default_rng(330 + W)
        state = _bf16_values(rng, (S, D, W - 1))  # stale contents: must be ignored at first
        idx = np.array([4, 0, 2], np.int32)
        _, y = orc.fwd(x, w, b)
        ok, y1, st = orc.fwd_pool(x[:, :5], state, idx, np.zeros(B, np.uint8), w, b)
        assert ok and np.array_equal(y1, y[:, :5]), f"first chunk W={W}"
        ok, y2, st = orc.fwd_pool(x[:, 5:11], st, idx, np.ones(B, np.uint8), w, b)
        assert ok and np.array_equal(y2, y[:, 5:11]), f"second chunk W={W}"
        xs = np.zeros((S, D), np.float32)
        for t in range(11, T):
            xs = x[:, t]
            ok, yt, st = orc.update(xs, st, idx, w, b)
            assert ok and np.array_equal(yt, y[:, t]), f"decode t={t} W={W}"
        assert np.array_equal(st[1], state[1]) and np.array_equal(st[3], state[3])


def check_pool_index_validation(orc):
    """The pool follows the decode slot rule: the same verdict as the decode update for the
    same index arrays, and a rejected call changes nothing."""
    B, T, D, S, W = 4, 3, 2, 6, 3
    x, w, b, _ = _problem(340, B, T, D, W)
    rng = np.random.default_rng(341)
    state = _bf16_values(rng, (S, D, W - 1))
    xd = _bf16_values(rng, (B, D))
    cases = ([0, 1, -2, 3], [0, 1, 6, 3], [0, 5, 2, 5], [7, 0, 1, 2], [-1, -3, 0, 1],
             [-1, -1, 5, 0], [5, 4, 3, 2], [0, 1, 2, -1])
    expect = (False, False, False, False, False, True, True, True)
    for case, want in zip(cases, expect):
        idx = np.array(case, np.int32)
        ok, y, st = orc.fwd_pool(x, state, idx, np.ones(B, np.uint8), w, b)
        okd, _, _ = orc.update(xd, state, idx, w, b)
        assert ok == want == okd, f"{case}: pool {ok}, decode {okd}, expected {want}"
        if not ok:
            assert y is None and np.array_equal(st, state), f"rejected {case} changed the state"


def _varlen_problem(seed, lens, D, W, bias=True):
    rng = np.random.default_rng(seed)
    total = int(sum(lens))
    x = _bf16_values(rng, (total, D))
    dy = _bf16_values(rng, (total, D))
    w = _bf16_values(rng, (D, W), 1.0 / math.sqrt(W))
    b = _bf16_values(rng, (D,), 0.3) if bias else None
    h0 = _bf16_values(rng, (len(lens), D, W - 1))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, dy, w, b, h0, cu


def check_varlen_torch(orc):
    """Each packed sequence against float64 torch conv1d over [its history; its rows], SiLU and
    autograd: y, final state, dx, history gradient; dw and dbias summed over the sequences.
    Lengths include 0, 1, 2 and lengths around W."""
    for W in (1, 2, 4):
        lens = [5, 0, 1, 2, 3, 9, 4, 0]
        x, dy, w, b, h0, cu = _varlen_problem(400 + W, lens, 6, W)
        D = x.shape[1]
        ok, y, hT = orc.fwd_varlen(x, cu, w, b, h0)
        ok2, dx, dw, db, dh0 = orc.bwd_varlen(x, dy, cu, w, b, h0)
        assert ok and ok2
        wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
        bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
        for i, L in enumerate(lens):
            a = int(cu[i])
            if L == 0:  # nothing to convolve: the state passes through, no gradient reaches it
                assert np.array_equal(hT[i], h0[i]) and not np.any(dh0[i]), f"empty seq {i} W={W}"
                continue
            xe = torch.cat([torch.tensor(h0[i], dtype=torch.float64).T, torch.tensor(x[a:a + L], dtype=torch.float64)], 0)
            xe.requires_grad_(True)
            z = F.conv1d(xe.T[None], wt[:, None, :], bt, padding=0, groups=D)[0].T
            yi = F.silu(z)
            (yi * torch.tensor(dy[a:a + L], dtype=torch.float64)).sum().backward()
            _close(y[a:a + L], yi.detach().numpy(), 1e-12, 1e-14, what=f"varlen y W={W} seq {i}")
            assert np.array_equal(hT[i].astype(np.float64), xe.detach()[L:].T.numpy()), f"varlen hT W={W} seq {i}"
            g = xe.grad.numpy()
            _close(dx[a:a + L], g[W - 1:], 1e-12, 1e-13, what=f"varlen dx W={W} seq {i}")
            _close(dh0[i], g[:W - 1].T, 1e-12, 1e-13, what=f"varlen dh0 W={W} seq {i}")
        _close(dw, wt.grad.numpy(), 1e-12, 1e-12, what=f"varlen dw W={W}")
        _close(db, bt.grad.numpy(), 1e-12, 1e-12, what=f"varlen dbias W={W}")


def check_varlen_equal_lengths_is_batch(orc):
    """Packing B sequences of equal length T is the [B, T, D] batch: y, dx and the states bit for
    bit, dw and dbias up to the order of the sums."""
    B, T, D, W = 3, 7, 5, 4
    x, dy, w, b, h0, cu = _varlen_problem(420, [T] * B, D, W)
    ok, y, hT = orc.fwd_varlen(x, cu, w, b, h0)
    _, dx, dw, db, dh0 = orc.bwd_varlen(x, dy, cu, w, b, h0)
    yb, hTb = orc.fwd_state(x.reshape(B, T, D), h0, w, b)
    dxb, dwb, dbb, dh0b = orc.bwd_state(x.reshape(B, T, D), h0, dy.reshape(B, T, D), w, b)
    assert ok and np.array_equal(y, yb.reshape(B * T, D)) and np.array_equal(hT, hTb)
    assert np.array_equal(dx, dxb.reshape(B * T, D)) and np.array_equal(dh0, dh0b)
    _close(dw, dwb, 1e-13, 1e-14, what="varlen vs batch dw")
    _close(db, dbb, 1e-13, 1e-14, what="varlen vs batch dbias")


def check_varlen_offsets_validation(orc):
    """Offsets must start at 0, never decrease and end at the row count; otherwise nothing is
    computed."""
    x, dy, w, b, h0, _ = _varlen_problem(430, [4, 4], 3, 3)
    for bad in ([1, 4, 8], [0, 5, 4, 8], [0, 4, 7], [0, 4, 9], [0, 9, 8]):
        n = len(bad) - 1
        hh = np.zeros((n, 3, 2), np.float32)
        ok, y, hT = orc.fwd_varlen(x, np.array(bad, np.int32), w, b, hh)
        ok2 = orc.bwd_varlen(x, dy, np.array(bad, np.int32), w, b, hh)[0]
        assert not ok and not ok2 and y is None, f"offsets {bad} accepted"
    for good in ([0, 8], [0, 0, 8], [0, 8, 8], [0, 3, 3, 8]):
        n = len(good) - 1
        assert orc.fwd_varlen(x, np.array(good, np.int32), w, b, np.zeros((n, 3, 2), np.float32))[0], good


def check_varlen_sequences_independent(orc):
    """A sequence's outputs do not depend on its neighbours' rows or histories; an empty
    sequence's final state is its history and its history gradient is zero."""
    lens = [6, 0, 5, 3]
    x, dy, w, b, h0, cu = _varlen_problem(440, lens, 4, 4)
    _, y, hT = orc.fwd_varlen(x, cu, w, b, h0)
    _, dx, _, _, dh0 = orc.bwd_varlen(x, dy, cu, w, b, h0)
    assert np.array_equal(hT[1], h0[1]) and not np.any(dh0[1]), "empty sequence"
    x2, dy2, h02 = x.copy(), dy.copy(), h0.copy()
    x2[:6] += 1.0
    x2[11:] -= 0.5
    dy2[:6] *= -1
    h02[0] += 2.0
    h02[3] -= 1.0
    _, y2, hT2 = orc.fwd_varlen(x2, cu, w, b, h02)
    _, dx2, _, _, dh02 = orc.bwd_varlen(x2, dy2, cu, w, b, h02)
    assert np.array_equal(y2[6:11], y[6:11]) and np.array_equal(dx2[6:11], dx[6:11]), "sequence 2 moved"
    assert np.array_equal(hT2[2], hT[2]) and np.array_equal(dh02[2], dh0[2])
    assert not np.array_equal(y2[:6], y[:6]) and not np.array_equal(y2[11:], y[11:])


def check_update_ex_by_hand(orc):
    """Small decode steps worked by hand (values exact in float): which entries feed z and
    which entry takes the token, for shift and circular states of both lengths."""
    w = np.array([[0.5, 2.0]], np.float32)  # W = 2: w0 pairs with the previous token, w1 with x
    x = np.array([[4.0]], np.float32)
    st = np.array([[[1.0, 3.0]]], np.float32)  # L = 2 = W: entries [a, b]
    # shift: previous token = last entry b = 3 -> z = 0.5*3 + 2*4 = 9.5; state -> [3, 4]
    ok, y, ns = orc.update_ex(x, st, None, None, w)
    assert ok and np.array_equal(ns[0, 0], [3.0, 4.0])
    _close(y[0, 0], 9.5 * _sigmoid(9.5), 1e-14, what="shift L=W")
    # circular, c = 3: previous token in entry (3-1) mod 2 = 0 -> a = 1 -> z = 0.5 + 8 = 8.5;
    # the token goes to entry 3 mod 2 = 1 -> [1, 4]
    ok, y, ns = orc.update_ex(x, st, None, np.array([3], np.int32), w)
    assert ok and np.array_equal(ns[0, 0], [1.0, 4.0])
    _close(y[0, 0], 8.5 * _sigmoid(8.5), 1e-14, what="circular L=W c=3")
    # W = 4, L = 4, circular, c = 5: tokens 1, 2, 3 steps back in entries 0, 3, 2; entry 1 takes x
    w4 = np.array([[0.25, 0.5, 1.0, 2.0]], np.float32)
    st4 = np.array([[[10.0, 20.0, 30.0, 40.0]]], np.float32)
    ok, y, ns = orc.update_ex(x, st4, None, np.array([5], np.int32), w4)
    z = 0.25 * 30.0 + 0.5 * 40.0 + 1.0 * 10.0 + 2.0 * 4.0  # x[t-3]=e2, x[t-2]=e3, x[t-1]=e0
    assert ok and np.array_equal(ns[0, 0], [10.0, 4.0, 30.0, 40.0])
    _close(y[0, 0], z * _sigmoid(z), 1e-14, what="circular W=4 L=4 c=5")
    # W = 4, L = 3, circular, c = 7: entries (7-1)%3=0, (7-2)%3=2, (7-3)%3=1; x -> entry 7%3=1
    st3 = np.array([[[10.0, 20.0, 30.0]]], np.float32)
    ok, y, ns = orc.update_ex(x, st3, None, np.array([7], np.int32), w4)
    z = 0.25 * 20.0 + 0.5 * 30.0 + 1.0 * 10.0 + 2.0 * 4.0
    assert ok and np.array_equal(ns[0, 0], [10.0, 4.0, 30.0])
    _close(y[0, 0], z * _sigmoid(z), 1e-14, what="circular W=4 L=3 c=7")


def check_update_ex_matches_update(orc):
    """L = W-1 with a shift is the plain decode update, bit for bit (y and state), padding
    rows and all."""
    N, S, D, W = 5, 9, 6, 4
    rng = np.random.default_rng(500)
    x = _bf16_values(rng, (N, D))
    w = _bf16_values(rng, (D, W))
    b = _bf16_values(rng, (D,), 0.3)
    state = _bf16_values(rng, (S, D, W - 1))
    idx = np.array([3, -1, 0, 8, 5], np.int32)
    ok, y, st = orc.update(x, state, idx, w, b)
    ok2, y2, st2 = orc.update_ex(x, state, idx, None, w, b)
    assert ok and ok2 and np.array_equal(y, y2) and np.array_equal(st, st2)


def check_update_ex_decode_equals_forward(orc):
    """Token by token, every variant (L = W-1 or W; shift, or circular from ring start c0)
    reproduces the forward over the sequence from its history, bit for bit in the oracle."""
    B, T, D = 3, 11, 5
    for W in (2, 3, 4):
        x, h0, w, b, _ = _problem_h0(510 + W, B, T, D, W)
        y_ref, _ = orc.fwd_state(x, h0, w, b)
        for L in (W - 1, W):
            for c0 in (None, 0, 1, 5):
                st = np.zeros((B, D, L), np.float32)
                for k in range(1, W):  # the history, k steps back from the first token
                    e = (L - k) if c0 is None else (c0 - k) % L
                    st[:, :, e] = h0[:, :, W - 1 - k]
                for t in range(T):
                    cs = None if c0 is None else np.full(B, c0 + t, np.int32)
                    ok, yt, st = orc.update_ex(x[:, t], st, None, cs, w, b)
                    assert ok and np.array_equal(yt, y_ref[:, t]), f"W={W} L={L} c0={c0} t={t}"


def check_update_ex_oldest_entry_unused(orc):
    """With L = W the oldest entry is carried but never used; a shift drops it."""
    N, D, W = 3, 4, 4
    rng = np.random.default_rng(520)
    x = _bf16_values(rng, (N, D))
    w = _bf16_values(rng, (D, W))
    st = _bf16_values(rng, (N, D, W))
    _, y, ns = orc.update_ex(x, st, None, None, w)
    st2 = st.copy()
    st2[:, :, 0] += 5.0
    _, y2, ns2 = orc.update_ex(x, st2, None, None, w)
    assert np.array_equal(y, y2) and np.array_equal(ns, ns2)
    assert np.array_equal(ns[:, :, :W - 1], st[:, :, 1:]) and np.array_equal(ns[:, :, W - 1], x)


def check_update_ex_validation(orc):
    """A negative cache_seqlens entry, a bad state length or a circular state without entries
    fail the whole call, which then changes nothing."""
    N, D, W = 3, 2, 4
    rng = np.random.default_rng(530)
    x = _bf16_values(rng, (N, D))
    w = _bf16_values(rng, (D, W))
    for L, cs in ((3, [0, -1, 2]), (4, [-5, 0, 0]), (2, None), (5, None)):
        st = _bf16_values(rng, (N, D, L))
        ok, y, ns = orc.update_ex(x, st, None, None if cs is None else np.array(cs, np.int32), w)
        assert not ok and y is None and np.array_equal(ns, st), (L, cs)
    w1 = _bf16_values(rng, (D, 1))
    ok, _, _ = orc.update_ex(x, np.zeros((N, D, 0), np.float32), None, np.zeros(N, np.int32), w1)
    assert not ok, "circular state without entries accepted"
    ok, _, _ = orc.update_ex(x, np.zeros((N, D, 0), np.float32), None, None, w1)
    assert ok


def check_epilogue_torch(orc):
    """float64 torch conv1d over [history; x], then no activation or SiLU, plus a residual after
    it, with autograd: y, dx, history gradient, dw, dbias; the residual's gradient is dy."""
    for W in (1, 2, 4):
        for act in (False, True):
            for with_res in (False, True):
                x, h0, w, b, dy = _problem_h0(600 + W + 2 * act + with_res, 2, 9, 5, W)
                rng = np.random.default_rng(610 + W)
                r = _bf16_values(rng, x.shape) if with_res else None
                B, T, D = x.shape
                xe = torch.cat([torch.tensor(h0, dtype=torch.float64).permute(0, 2, 1),
                                torch.tensor(x, dtype=torch.float64)], 1).requires_grad_(True)
                wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
                bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
                rt = torch.tensor(r, dtype=torch.float64, requires_grad=True) if with_res else None
                z = F.conv1d(xe.transpose(1, 2), wt[:, None, :], bt, padding=0, groups=D).transpose(1, 2)
                yt = F.silu(z) if act else z
                if with_res:
                    yt = yt + rt
                (yt * torch.tensor(dy, dtype=torch.float64)).sum().backward()
                what = f"W={W} act={act} residual={with_res}"
                y = orc.fwd_epi(x, w, b, h0=h0, residual=r, act=act)
                _close(y, yt.detach().numpy(), 1e-12, 1e-14, what=f"epilogue y {what}")
                dx, dw, db, dh0 = orc.bwd_epi(x, dy, w, b, h0=h0, act=act)
                g = xe.grad.numpy()
                _close(dx, g[:, W - 1:], 1e-12, 1e-13, what=f"epilogue dx {what}")
                _close(dh0, g[:, :W - 1].transpose(0, 2, 1), 1e-12, 1e-13, what=f"epilogue dh0 {what}")
                _close(dw, wt.grad.numpy(), 1e-12, 1e-12, what=f"epilogue dw {what}")
                _close(db, bt.grad.numpy(), 1e-12, 1e-12, what=f"epilogue dbias {what}")
                if with_res:
                    assert np.array_equal(rt.grad.numpy(), dy.astype(np.float64)), "residual gradient"


def check_epilogue_default_is_plain(orc):
    """SiLU without a residual is the history forward and backward, bit for bit."""
    x, h0, w, b, dy = _problem_h0(620, 2, 13, 6, 4)
    y, _ = orc.fwd_state(x, h0, w, b)
    assert np.array_equal(orc.fwd_epi(x, w, b, h0=h0), y)
    for a, c in zip(orc.bwd_epi(x, dy, w, b, h0=h0), orc.bwd_state(x, h0, dy, w, b)):
        assert np.array_equal(a, c)


ALL_CHECKS = [
    check_rounding_matches_torch,
    check_rounding_from_double_is_direct,
    check_worked_example,
    check_impulse,
    check_w1_closed_form,
    check_constant_input,
    check_torch_conv1d,
    check_finite_differences,
    check_w_padding,
    check_dbias_is_dw_of_unit_input,
    check_channel_and_batch_independence,
    check_decode_equals_forward,
    check_decode_worked_example,
    check_decode_index_validation,
    check_points_match_full,
    check_f32_close_to_f64,
    check_history_torch,
    check_history_chunking,
    check_history_zero_is_plain,
    check_prefill_then_decode,
    check_pool_matches_gathered_history,
    check_pool_prefill_then_decode,
    check_pool_index_validation,
    check_varlen_torch,
    check_varlen_equal_lengths_is_batch,
    check_varlen_offsets_validation,
    check_varlen_sequences_independent,
    check_update_ex_by_hand,
    check_update_ex_matches_update,
    check_update_ex_decode_equals_forward,
    check_update_ex_oldest_entry_unused,
    check_update_ex_validation,
    check_epilogue_torch,
    check_epilogue_default_is_plain,
]
