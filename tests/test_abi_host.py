"""Host-side contract of libcconv.so (CPU only: no kernel is ever launched here).

The library must load and export every function include/*.h declares, and every problem the
host can see must come back as its status code before any HIP call is made. Device pointers
are fake integers: validation never dereferences them, and no case here passes validation
with a non-empty problem.
"""

import ctypes
import re
from pathlib import Path

import pytest

import causal_depthwise_short_amd as cc

ROOT = Path(__file__).resolve().parent.parent
OK, NULLP, SHAPE, STRIDE, DTYPE, MISAL, ALIAS, WS, INDEX, LAUNCH, CONFIG = range(11)
BF16, F32 = 0, 1

# fake, 16-byte aligned, widely separated device addresses
X, DY, WT, BIAS, Y, DX, DW, DB, WSP, ST, IDX, STATUS = (0x10_0000_0000 + i * 0x1_0000_0000 for i in range(12))


def _declared(header: Path):
    text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(cconv_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    for header, path in ((ROOT / "include" / "cconv.h", cc.LIB_PATH), (ROOT / "include" / "cconv_roofline.h", cc.ROOFLINE_LIB_PATH)):
        names = _declared(header)
        assert names, header
        lib = ctypes.CDLL(str(path))
        missing = [n for n in names if not hasattr(lib, n)]
        assert not missing, f"{path.name} lacks {missing}"


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """With no built library and no way to build one, every entry point raises: there is no
    fallback path that computes anything without the HIP library."""
    import causal_depthwise_short_amd._build as build

    monkeypatch.setattr(cc, "_lib", None)
    monkeypatch.setattr(cc, "LIB_PATH", tmp_path / "libcconv.so")
    monkeypatch.setattr(build, "build", lambda *a, **k: None)
    with pytest.raises(cc.CconvError):
        cc.lib()
    with pytest.raises(cc.CconvError):
        cc.cconv_default_config("fwd", 1, 16, 64, 4)


def test_host_tensors_are_refused_before_any_call():
    """The binding hands the library bare addresses, so it refuses tensors that are not on the
    GPU (inputs and caller-provided outputs alike) before calling it."""
    import torch

    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    w = torch.zeros(64, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        cc.cconv_fwd(x, w)
    with pytest.raises(ValueError, match="GPU"):
        cc.cconv_bwd(x, x, w)
    with pytest.raises(ValueError, match="GPU"):
        cc.cconv_update(x[0], torch.zeros(4, 64, 3, dtype=torch.bfloat16), None, w)


def test_version_and_status_strings():
    assert "gfx950" in cc.cconv_version()
    for code in range(11):
        s = cc.cconv_status_string(code)
        assert s and s != "unknown status"
    assert cc.cconv_status_string(99) == "unknown status"


def fwd(x=X, x_sb=None, x_st=None, w=WT, w_dt=BF16, bias=BIAS, y=Y, B=2, T=64, D=512, W=4):
    x_st = D if x_st is None else x_st
    x_sb = T * x_st if x_sb is None else x_sb
    return cc.lib().cconv_fwd(x, x_sb, x_st, w, w_dt, bias, y, B, T, D, W, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(x=None), NULLP),
        (dict(w=None), NULLP),
        (dict(y=None), NULLP),
        (dict(B=-1), SHAPE),
        (dict(T=-5), SHAPE),
        (dict(W=0), SHAPE),
        (dict(W=5), SHAPE),
        (dict(D=500, y=Y + 1), MISAL),  # any D is accepted: element alignment on that path
        (dict(D=500, x=X + 1), MISAL),
        (dict(D=500, x_st=499), STRIDE),
        (dict(x_st=504, D=512), STRIDE),
        (dict(x_st=516), STRIDE),
        (dict(x_sb=-8), STRIDE),
        (dict(w_dt=7), DTYPE),
        (dict(x=X + 2), MISAL),
        (dict(y=Y + 8), MISAL),
        (dict(w=WT + 4), MISAL),
        (dict(bias=BIAS + 4), MISAL),
        (dict(y=X), ALIAS),
        (dict(y=X + 64 * 512), ALIAS),
        (dict(y=WT - 16), ALIAS),
        (dict(bias=Y + 1024), ALIAS),
    ],
)
def test_fwd_host_errors(kw, code):
    assert fwd(**kw) == code


def test_fwd_empty_is_ok_without_launch():
    assert fwd(B=0) == OK
    assert fwd(T=0) == OK
    assert fwd(D=0) == OK


def bwd(x=X, dy=DY, w=WT, w_dt=BF16, bias=BIAS, dx=DX, dw=DW, dw_dt=BF16, db=DB, ws=WSP, ws_bytes=1 << 40,
        B=2, T=64, D=512, W=4, x_st=None, dy_st=None):
    x_st = D if x_st is None else x_st
    dy_st = D if dy_st is None else dy_st
    return cc.lib().cconv_bwd(x, T * x_st, x_st, dy, T * dy_st, dy_st, w, w_dt, bias, dx, dw, dw_dt, db, ws, ws_bytes,
                              B, T, D, W, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(x=None), NULLP),
        (dict(dy=None), NULLP),
        (dict(dx=None), NULLP),
        (dict(dw=None), NULLP),
        (dict(ws=None), NULLP),
        (dict(W=7), SHAPE),
        (dict(D=12, dx=DX + 1), MISAL),
        (dict(dy_st=100), STRIDE),
        (dict(dw_dt=3), DTYPE),
        (dict(w_dt=2), DTYPE),
        (dict(dx=DX + 2), MISAL),
        (dict(dw=DW + 8), MISAL),
        (dict(db=DB + 4), MISAL),
        (dict(ws=WSP + 8), MISAL),
        (dict(dx=DY), ALIAS),
        (dict(dw=DX + 16), ALIAS),
        (dict(db=DW), ALIAS),
        (dict(ws=X), ALIAS),
        (dict(ws_bytes=16), WS),
    ],
)
def test_bwd_host_errors(kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_matches_plan():
    for B, T, D, W in [(1, 256, 512, 4), (8, 8192, 4096, 4), (3, 1000, 2000, 2), (2, 5, 8, 1)]:
        cfg = cc.cconv_default_config("bwd", B, T, D, W)
        assert cfg.seg_rows % cfg.rows_per_group == 0 and cfg.seg_rows >= 8
        segs = -(-T // cfg.seg_rows)
        groups = -(-segs // cfg.waves_per_block)
        assert cc.cconv_bwd_workspace_bytes(B, T, D, W) == B * groups * (W + 1) * D * 4
        # and the config entry point agrees
        assert cc.cconv_bwd_workspace_bytes(B, T, D, W, cfg) == B * groups * (W + 1) * D * 4
    assert cc.cconv_bwd_workspace_bytes(0, 10, 8, 4) == 0
    bad = cc.Config(vec=8, rows_per_group=3, waves_per_block=4, seg_rows=64)
    assert cc.cconv_bwd_workspace_bytes(2, 64, 512, 4, bad) == 0


@pytest.mark.parametrize(
    "cfg",
    [
        dict(vec=6, rows_per_group=8, waves_per_block=4, seg_rows=64),
        dict(vec=8, rows_per_group=5, waves_per_block=4, seg_rows=64),
        dict(vec=8, rows_per_group=8, waves_per_block=3, seg_rows=64),
        dict(vec=8, rows_per_group=8, waves_per_block=4, seg_rows=60),
        dict(vec=8, rows_per_group=8, waves_per_block=4, seg_rows=0),
        dict(vec=8, rows_per_group=8, waves_per_block=2, options=8, seg_rows=64),
        dict(vec=8, rows_per_group=8, waves_per_block=1, options=16, seg_rows=64),
    ],
)
def test_bad_config_rejected(cfg):
    c = cc.Config(**cfg)
    st = cc.lib().cconv_fwd_config(X, 64 * 512, 512, WT, BF16, BIAS, Y, 2, 64, 512, 4, ctypes.byref(c), None)
    assert st == CONFIG


def upd(x=X, x_ld=None, state=ST, S=512, idx=IDX, w=WT, w_dt=BF16, bias=BIAS, y=Y, N=256, D=4096, W=4, status=STATUS):
    x_ld = D if x_ld is None else x_ld
    return cc.lib().cconv_update(x, x_ld, state, S, idx, w, w_dt, bias, y, N, D, W, status, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(x=None), NULLP),
        (dict(state=None), NULLP),
        (dict(y=None), NULLP),
        (dict(W=5), SHAPE),
        (dict(D=4100, x_ld=4101), STRIDE),  # neither compact rows nor a stride that is a multiple of 8
        (dict(D=4100, x=X + 1), MISAL),
        (dict(N=-1), SHAPE),
        (dict(N=(1 << 24) + 1), SHAPE),
        (dict(S=(1 << 19) - 31), SHAPE),
        (dict(idx=None, N=600, S=512), SHAPE),
        (dict(x_ld=4000), STRIDE),
        (dict(x_ld=4100), STRIDE),
        (dict(w_dt=9), DTYPE),
        (dict(state=ST + 2), MISAL),
        (dict(idx=IDX + 2), MISAL),
        (dict(status=STATUS + 1), MISAL),
        (dict(y=X), ALIAS),
        (dict(state=WT), ALIAS),
        (dict(status=ST + 64), ALIAS),
        (dict(status=Y + 4), ALIAS),
        (dict(status=None), NULLP),  # indices given: only the device sees their verdict
        (dict(D=(1 << 26) + 8, x_ld=(1 << 26) + 8), SHAPE),
    ],
)
def test_update_host_errors(kw, code):
    assert upd(**kw) == code


def test_update_empty_without_status_is_ok():
    assert upd(N=0, status=None) == OK


def test_bwd_noalloc_host_errors():
    """The static-scratch backward checks like cconv_bwd and refuses problems whose partials do
    not fit its array, before any device call."""
    L = cc.lib()
    cap = L.cconv_bwd_noalloc_max_workspace()
    assert cap == 16 << 20
    call = lambda B, T, D, W, **k: L.cconv_bwd_noalloc(k.get("x", X), T * D, D, DY, T * D, D, WT, BF16, BIAS,
                                                       k.get("dx", DX), DW, BF16, DB, B, T, D, W, None)
    assert L.cconv_bwd_workspace_bytes(1, 64, 1 << 20, 4) > cap
    assert call(1, 64, 1 << 20, 4) == WS
    assert call(2, 64, 512, 5) == SHAPE
    assert call(2, 64, 512, 4, x=None) == NULLP


def test_bwd_stages_host_errors():
    L = cc.lib()
    D, T, B, W = 512, 64, 2, 4
    main = lambda **k: L.cconv_bwd_main(k.get("x", X), T * D, D, k.get("dy", DY), T * D, D, k.get("w", WT), BF16,
                                        BIAS, k.get("dx", DX), k.get("ws", WSP), k.get("ws_bytes", 1 << 40), B, T, D, W,
                                        None)
    fin = lambda **k: L.cconv_bwd_finish(k.get("ws", WSP), k.get("ws_bytes", 1 << 40), k.get("dw", DW),
                                         k.get("dw_dt", BF16), k.get("db", DB), B, T, D, W, None)
    assert main(x=None) == NULLP and main(dx=None) == NULLP and main(ws=None) == NULLP
    assert main(dx=X) == ALIAS and main(ws=DY) == ALIAS and main(ws_bytes=8) == WS
    assert fin(dw=None) == NULLP and fin(ws=None) == NULLP and fin(dw_dt=5) == DTYPE
    assert fin(dw=WSP) == ALIAS and fin(db=DW) == ALIAS and fin(ws_bytes=8) == WS and fin(db=DB + 4) == MISAL


@pytest.mark.parametrize("which", ["fwd", "bwd"])
def test_default_plan_fits_the_wave_slots(which):
    """Default plans cut each batch row into as many segments as the wave slots allow (1024
    one-wave-per-SIMD waves with four channels per lane, also at D = 2 (mod 4); 2048 with two
    (D = 2); 3072 (forward) and 2048 (backward) with one (odd D)) and no more, down to one
    16-row group, and take streaming cache hints when output rows start on 128-byte lines or the
    call streams at most 256 MB."""
    for B, T, D in [(8, 8192, 4096), (8, 8192, 4160), (8, 8192, 4104), (16, 8192, 2048), (3, 1000, 2000),
                    (8, 8192, 4100), (1, 65536, 4096), (2, 100003, 520), (64, 4096, 4096), (1, 256, 512),
                    (8, 8192, 4098), (8, 8192, 4097), (4, 4096, 1002), (2, 5000, 333), (4, 100, 2), (4, 100, 6)]:
        c = cc.cconv_default_config(which, B, T, D, 4)
        narrow = D % 2 != 0 or D == 2
        fwd = which in ("fwd", 0)
        small = B * T * D * (4 if fwd else 6) <= 256 << 20
        off_lines = (2 * D) % 128 != 0 and not small
        slots = (2048 if D == 2 else 3072 if fwd else 2048) if narrow else 1024
        strips = -(-(-(-D // c.vec)) // 64)
        waves = B * strips * -(-T // c.seg_rows)
        if B * strips <= slots:
            assert waves <= slots, (B, T, D, c, waves)
        if c.seg_rows > 16:  # not held up by the one-group minimum: one more segment would not fit
            assert B * strips * (-(-T // c.seg_rows) + 1) > slots or -(-T // c.seg_rows) * c.seg_rows - T < c.seg_rows
        if narrow:
            assert c.vec == (2 if D == 2 else 1) and c.options == 0
        else:
            assert c.vec == 4 and c.options == (8 if off_lines else 11), (D, c.options)
    assert cc.cconv_default_config(which, 8, 8192, 4096, 4).seg_rows == 1024
    assert cc.cconv_default_config(which, 8, 8192, 4160, 4).seg_rows == 1184
    assert cc.cconv_default_config(which, 8, 8192, 4098, 4).seg_rows == 1184  # 17 strips, as D = 4100
    # the small workloads: one-group segments at B1 T256 D512, 32-row ones at B3 T1000 D2000
    assert cc.cconv_default_config(which, 1, 256, 512, 4).seg_rows == 16
    assert cc.cconv_default_config(which, 3, 1000, 2000, 2).seg_rows == 32


@pytest.mark.parametrize("which", ["fwd", "bwd"])
def test_default_configs_are_valid(which):
    """Every default plan over a grid of shapes is one the library accepts."""
    for B in (1, 3, 8):
        for T in (1, 2, 7, 8, 15, 16, 17, 100, 1000, 8192, 100003):
            for D in (8, 520, 4096, 1, 7, 1003):
                for W in (1, 4):
                    c = cc.cconv_default_config(which, B, T, D, W)
                    assert c.seg_rows % c.rows_per_group == 0 and c.seg_rows >= 8, (which, B, T, D, W, c)
                    assert c.waves_per_block % c.strips_per_block == 0
                    assert cc.cconv_bwd_workspace_bytes(B, T, D, W, c if which == "bwd" else None) > 0
                    if which == "fwd":
                        # y aliases x on purpose: the aliasing check comes after the config check,
                        # so ALIAS (not BAD_CONFIG) means the plan was accepted, with nothing launched
                        st = cc.lib().cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, B, T, D, W, ctypes.byref(c), None)
                        assert st == ALIAS, (B, T, D, W, c, st)


H0, HT, DH = (0x30_0000_0000 + i * 0x1_0000_0000 for i in range(3))


def fwd_state(x=X, w=WT, bias=BIAS, h0=H0, hT=HT, y=Y, B=2, T=64, D=512, W=4):
    return cc.lib().cconv_fwd_state(x, T * D, D, w, BF16, bias, h0, hT, y, B, T, D, W, None)


def bwd_state(x=X, dy=DY, h0=H0, dx=DX, dw=DW, db=DB, dh=DH, ws=WSP, ws_bytes=1 << 40, B=2, T=64, D=512, W=4):
    return cc.lib().cconv_bwd_state(x, T * D, D, dy, T * D, D, WT, BF16, BIAS, h0, dx, dw, BF16, db, dh, ws, ws_bytes,
                                    B, T, D, W, None)


STATE_BYTES = 2 * 512 * 3 * 2  # B * D * (W-1) bf16


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(x=None), NULLP),
        (dict(h0=H0 + 2), MISAL),
        (dict(hT=HT + 8), MISAL),
        (dict(hT=X + 16), ALIAS),
        (dict(hT=WT), ALIAS),
        (dict(hT=BIAS), ALIAS),
        (dict(hT=Y + 32), ALIAS),
        (dict(h0=Y), ALIAS),
        (dict(hT=H0 + 16), ALIAS),  # overlaps the history without being the same buffer
        (dict(hT=H0 - STATE_BYTES + 16), ALIAS),
        (dict(T=0), SHAPE),  # a final state needs at least one token
        (dict(T=0, hT=H0), SHAPE),  # in place passes the aliasing check (fails later on T)
        (dict(W=5), SHAPE),
    ],
)
def test_fwd_state_host_errors(kw, code):
    assert fwd_state(**kw) == code


def test_fwd_state_empty_and_unused():
    assert fwd_state(B=0) == OK and fwd_state(D=0) == OK
    assert fwd_state(T=0, hT=None) == OK  # nothing to produce
    # W = 1 holds no state: the state pointers are ignored, even misaligned ones
    assert fwd_state(W=1, h0=H0 + 2, hT=HT + 2, T=0) == OK


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(dh=DH + 2), MISAL),
        (dict(h0=H0 + 8), MISAL),
        (dict(dh=X), ALIAS),
        (dict(dh=H0 + 16), ALIAS),
        (dict(dh=DX + 64), ALIAS),
        (dict(dh=WSP), ALIAS),
        (dict(dx=H0), ALIAS),
        (dict(ws=H0), ALIAS),
        (dict(T=0), SHAPE),
        (dict(dh=None, ws_bytes=8), WS),
    ],
)
def test_bwd_state_host_errors(kw, code):
    assert bwd_state(**kw) == code


POOL, PIDX, PFLAG, PST = (0x40_0000_0000 + i * 0x1_0000_0000 for i in range(4))


def fwd_pool(x=X, state=POOL, S=64, idx=PIDX, flags=PFLAG, status=PST, y=Y, B=2, T=64, D=512, W=4):
    return cc.lib().cconv_fwd_pool(x, T * D, D, WT, BF16, BIAS, state, S, idx, flags, status, y, B, T, D, W, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(status=None), NULLP),
        (dict(idx=None), NULLP),
        (dict(state=None), NULLP),
        (dict(S=-1), SHAPE),
        (dict(S=(1 << 19) - 31), SHAPE),
        (dict(B=(1 << 24) + 1, T=1), SHAPE),
        (dict(T=0), SHAPE),
        (dict(status=PST + 2), MISAL),
        (dict(idx=PIDX + 2), MISAL),
        (dict(state=POOL + 8), MISAL),
        (dict(state=X), ALIAS),
        (dict(state=Y + 64), ALIAS),
        (dict(status=X + 16), ALIAS),
        (dict(status=POOL + 64), ALIAS),
        (dict(status=PIDX), ALIAS),
        (dict(status=PFLAG + 1 - 1), ALIAS),
        (dict(idx=Y), ALIAS),
        (dict(flags=POOL + 32), ALIAS),
        (dict(y=PIDX - 64), ALIAS),
    ],
)
def test_fwd_pool_host_errors(kw, code):
    assert fwd_pool(**kw) == code


def test_fwd_pool_null_state_allowed_when_empty():
    """The pool may be NULL when it holds nothing (S = 0 or W = 1): validation goes on past the
    NULL check (here to the misaligned y, so nothing is launched)."""
    assert fwd_pool(state=None) == NULLP
    assert fwd_pool(state=None, S=0, y=Y + 8) == MISAL
    assert fwd_pool(state=None, W=1, y=Y + 8) == MISAL


CU = 0x50_0000_0000


def fwd_varlen(x=X, x_st=512, cu=CU, nseq=4, total=1000, h0=H0, hT=HT, status=PST, y=Y, D=512, W=4, cfg=None):
    L = cc.lib()
    args = (x, x_st, cu, nseq, total, WT, BF16, BIAS, h0, hT, status, y, D, W)
    if cfg is None:
        return L.cconv_fwd_varlen(*args, None)
    return L.cconv_fwd_varlen_config(*args, ctypes.byref(cfg), None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(status=None), NULLP),
        (dict(cu=None), NULLP),
        (dict(x=None), NULLP),
        (dict(nseq=-1), SHAPE),
        (dict(nseq=(1 << 24) + 1), SHAPE),
        (dict(total=1 << 31), SHAPE),
        (dict(total=-1), SHAPE),
        (dict(D=100, y=Y + 1), MISAL),
        (dict(x_st=500), STRIDE),
        (dict(cu=CU + 2), MISAL),
        (dict(status=PST + 1), MISAL),
        (dict(hT=HT + 8), MISAL),
        (dict(hT=H0), ALIAS),  # packed batches do not advance a state in place
        (dict(hT=H0 + 4 * 512 * 3 * 2 - 16), ALIAS),  # the last 16 bytes of the history
        (dict(status=CU + 4), ALIAS),
        (dict(status=X), ALIAS),
        (dict(status=HT + 32), ALIAS),
        (dict(y=CU - 64), ALIAS),
        (dict(hT=CU), ALIAS),
        (dict(cfg=cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=15, seg_rows=64)), CONFIG),
        (dict(cfg=cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=8, seg_rows=64)), CONFIG),
        (dict(cfg=cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=64), y=Y + 8), MISAL),
    ],
)
def test_fwd_varlen_host_errors(kw, code):
    assert fwd_varlen(**kw) == code


def bwd_varlen(x=X, dy=DY, cu=CU, nseq=4, total=1000, h0=H0, dx=DX, dw=DW, db=DB, dh=DH, ws=WSP, ws_bytes=1 << 40,
               status=PST, D=512, W=4, cfg=None):
    L = cc.lib()
    args = (x, D, dy, D, cu, nseq, total, WT, BF16, BIAS, h0, dx, dw, BF16, db, dh, ws, ws_bytes, status, D, W)
    if cfg is None:
        return L.cconv_bwd_varlen(*args, None)
    return L.cconv_bwd_varlen_config(*args, ctypes.byref(cfg), None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(status=None), NULLP),
        (dict(cu=None), NULLP),
        (dict(dx=None), NULLP),
        (dict(total=1 << 31), SHAPE),
        (dict(dh=H0), ALIAS),
        (dict(dh=DX + 16), ALIAS),
        (dict(dx=H0), ALIAS),
        (dict(dh=CU), ALIAS),
        (dict(status=DW), ALIAS),
        (dict(ws=CU), ALIAS),
        (dict(dh=DH + 2), MISAL),
        (dict(ws_bytes=16), WS),
        (dict(cfg=cc.Config(vec=8, rows_per_group=8, waves_per_block=1, options=15, seg_rows=64)), CONFIG),
        (dict(cfg=cc.Config(vec=8, rows_per_group=8, waves_per_block=1, options=11, seg_rows=64), ws_bytes=16), WS),
    ],
)
def test_bwd_varlen_host_errors(kw, code):
    assert bwd_varlen(**kw) == code


CSL = 0x60_0000_0000


def upd_ex(x=X, state=ST, S=512, L=3, idx=IDX, cs=CSL, y=Y, N=256, D=4096, W=4, status=STATUS):
    return cc.lib().cconv_update_ex(x, D, state, S, L, idx, cs, WT, BF16, BIAS, y, N, D, W, status, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(L=2), SHAPE),
        (dict(L=5), SHAPE),
        (dict(W=1, L=0), SHAPE),  # a circular state needs entries
        (dict(state=None), NULLP),
        (dict(cs=CSL + 2), MISAL),
        (dict(state=ST + 16 * 0 + 8), MISAL),
        (dict(cs=Y + 64), ALIAS),
        (dict(cs=ST + 4096), ALIAS),
        (dict(status=CSL), ALIAS),
        (dict(y=CSL - 512), ALIAS),
        (dict(L=4, state=Y - 512 * 4096 * 4 * 2 + 16), ALIAS),  # an L = 4 pool reaches further than L = 3
        (dict(idx=None, status=None), NULLP),  # cache_seqlens given: a negative entry fails on the device
    ],
)
def test_update_ex_host_errors(kw, code):
    assert upd_ex(**kw) == code


def test_update_ex_width_one_shift_needs_no_state():
    # W = 1, L = 0, shift: no state at all; nothing to launch for N = 0
    assert upd_ex(W=1, L=0, cs=None, state=None, N=0, status=None) == OK


def upd_cfg(cfg, **kw):
    a = dict(x=X, state=ST, S=512, L=3, idx=IDX, cs=None, y=Y, N=256, D=4096, W=4, status=STATUS, x_ld=None)
    a.update(kw)
    x_ld = a["D"] if a["x_ld"] is None else a["x_ld"]
    return cc.lib().cconv_update_config(a["x"], x_ld, a["state"], a["S"], a["L"], a["idx"], a["cs"], WT, BF16, BIAS,
                                        a["y"], a["N"], a["D"], a["W"], a["status"],
                                        None if cfg is None else ctypes.byref(cfg), None)


@pytest.mark.parametrize(
    "cfg,kw,code",
    [
        (None, {}, NULLP),
        (dict(block_threads=32, options=0, rows_per_block=1), {}, CONFIG),
        (dict(block_threads=96, options=0, rows_per_block=1), {}, CONFIG),
        (dict(block_threads=2048, options=0, rows_per_block=1), {}, CONFIG),
        (dict(block_threads=256, options=6, rows_per_block=1), {}, CONFIG),  # staged with non-temporal loads
        (dict(block_threads=256, options=8, rows_per_block=1), {}, CONFIG),
        (dict(vec=4, block_threads=256, options=4, rows_per_block=1), dict(D=4100), CONFIG),  # staged: vec 8 only
        (dict(block_threads=1024, options=4, rows_per_block=1), dict(S=(1 << 19) - 64, D=8), CONFIG),  # LDS over 64 KiB
        (dict(block_threads=256, options=0, rows_per_block=0), {}, CONFIG),
        (dict(block_threads=256, options=0, rows_per_block=4, rows_per_thread=4), {}, CONFIG),
        (dict(block_threads=1024, options=0, rows_per_block=4, rows_per_thread=2), {}, CONFIG),  # registers
        (dict(vec=2, block_threads=256, options=0, rows_per_block=1), {}, CONFIG),
        (dict(vec=8, block_threads=256, options=0, rows_per_block=1), dict(D=4100), CONFIG),  # 8 does not divide D
        (dict(vec=4, block_threads=256, options=0, rows_per_block=1), dict(D=4098), CONFIG),
        (dict(vec=4, block_threads=256, options=0, rows_per_block=1), dict(D=4100, x_ld=4102), STRIDE),
        (dict(vec=4, block_threads=256, options=0, rows_per_block=1), dict(D=4100, x=X + 2), MISAL),
        (dict(vec=1, block_threads=256, options=1, rows_per_block=1), dict(D=4100), CONFIG),  # one channel: no hints
        (dict(vec=1, block_threads=256, options=0, rows_per_block=2, rows_per_thread=2), {}, CONFIG),
        (dict(block_threads=64, options=0, rows_per_block=1), dict(N=65536 * 2, S=65536 * 2), CONFIG),  # grid rows
    ],
)
def test_update_config_host_errors(cfg, kw, code):
    c = None if cfg is None else cc.UpdateConfig(**cfg)
    assert upd_cfg(c, **kw) == code


def test_default_update_config():
    c = cc.UpdateConfig()
    assert cc.lib().cconv_default_update_config(256, 4096, ctypes.byref(c)) == OK
    assert c.vec == 8 and c.rows_per_block >= 1
    assert c.options == 5  # non-temporal stores, state runs staged through LDS
    assert cc.lib().cconv_default_update_config(256, 4100, ctypes.byref(c)) == OK
    assert c.vec == 4 and c.options == 1
    assert cc.lib().cconv_default_update_config(256, 4098, ctypes.byref(c)) == OK
    assert (c.vec, c.options, c.rows_per_thread) == (1, 0, 1)
    assert cc.lib().cconv_default_update_config(1 << 20, 4096, ctypes.byref(c)) == OK
    blocks_x = -(-(4096 // c.vec) // c.block_threads)
    assert -(-(1 << 20) // c.rows_per_block) * blocks_x <= 1024 + blocks_x
    assert cc.lib().cconv_default_update_config(-1, 4096, ctypes.byref(c)) == SHAPE
    assert cc.lib().cconv_default_update_config(4, 4096, None) == NULLP


def test_option_structs_match_the_header(tmp_path):
    """The binding's ctypes structures have the C layout of cconv_fwd_opts_t / cconv_bwd_opts_t."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"cconv.h\"\n"
        "#define O(T, f) printf(\"%zu \", offsetof(T, f))\n"
        "int main(void) {\n"
        "  printf(\"%zu %zu \", sizeof(cconv_fwd_opts_t), sizeof(cconv_bwd_opts_t));\n"
        "  O(cconv_fwd_opts_t, activation); O(cconv_fwd_opts_t, residual); O(cconv_fwd_opts_t, residual_sb);\n"
        "  O(cconv_fwd_opts_t, residual_st); O(cconv_fwd_opts_t, init_state); O(cconv_fwd_opts_t, final_state);\n"
        "  O(cconv_fwd_opts_t, cu_seqlens); O(cconv_fwd_opts_t, nseq); O(cconv_fwd_opts_t, status);\n"
        "  O(cconv_fwd_opts_t, y_sb); O(cconv_fwd_opts_t, y_st);\n"
        "  O(cconv_bwd_opts_t, activation); O(cconv_bwd_opts_t, init_state); O(cconv_bwd_opts_t, d_init_state);\n"
        "  O(cconv_bwd_opts_t, cu_seqlens); O(cconv_bwd_opts_t, nseq); O(cconv_bwd_opts_t, status);\n"
        "  O(cconv_bwd_opts_t, dx_sb); O(cconv_bwd_opts_t, dx_st);\n"
        "  return 0;\n}\n"
    )
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", str(ROOT / "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", str(src),
                    "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(cc.FwdOpts), ctypes.sizeof(cc.BwdOpts)]
    want += [getattr(cc.FwdOpts, f).offset for f, _ in cc.FwdOpts._fields_]
    want += [getattr(cc.BwdOpts, f).offset for f, _ in cc.BwdOpts._fields_]
    assert got == want


RES = 0x70_0000_0000


def fwd_ex(x=X, y=Y, B=2, T=64, D=512, W=4, act=1, res=RES, r_st=None, r_sb=None, h0=H0, hT=HT, cu=None, nseq=0,
           status=None, y_sb=0, y_st=0):
    r_st = D if r_st is None else r_st
    r_sb = T * r_st if r_sb is None else r_sb
    o = cc.FwdOpts(act, res, r_sb, r_st, h0, hT, cu, nseq, status, y_sb, y_st)
    return cc.lib().cconv_fwd_ex(x, T * D, D, WT, BF16, BIAS, y, B, T, D, W, ctypes.byref(o), None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(act=2), CONFIG),
        (dict(act=-1), CONFIG),
        (dict(cu=CU, nseq=2), SHAPE),  # packed batches have B = 1
        (dict(cu=CU, nseq=2, B=1, status=None), NULLP),
        (dict(res=RES + 2), MISAL),
        (dict(r_st=500), STRIDE),
        (dict(r_st=516), STRIDE),
        (dict(y=RES + 32), ALIAS),
        (dict(hT=RES), ALIAS),
        (dict(res=Y), ALIAS),
        (dict(W=5), SHAPE),
        (dict(y_st=500, y_sb=64 * 512), STRIDE),  # row stride below D
        (dict(y_st=516, y_sb=64 * 516), STRIDE),  # not a multiple of 8 on the vector path
        (dict(y_st=1024, y_sb=1024 * 63), STRIDE),  # batch rows would overlap
        (dict(y_st=1024, y_sb=1024 * 64 + 4), STRIDE),
        (dict(y=Y + 8, y_st=1024, y_sb=1024 * 64), MISAL),
        (dict(y_st=1024, y_sb=1024 * 64, res=RES + 2), MISAL),  # valid strides: the next check speaks
    ],
)
def test_fwd_ex_host_errors(kw, code):
    assert fwd_ex(**kw) == code


def bwd_ex(act=1, dx=DX, h0=H0, dh=DH, cu=None, nseq=0, status=None, B=2, T=64, D=512, W=4, ws_bytes=1 << 40,
           dx_sb=0, dx_st=0):
    o = cc.BwdOpts(act, h0, dh, cu, nseq, status, dx_sb, dx_st)
    return cc.lib().cconv_bwd_ex(X, T * D, D, DY, T * D, D, WT, BF16, BIAS, dx, DW, BF16, DB, WSP, ws_bytes, B, T, D, W,
                                 ctypes.byref(o), None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(act=3), CONFIG),
        (dict(cu=CU, nseq=2), SHAPE),
        (dict(cu=CU, nseq=2, B=1), NULLP),
        (dict(dh=H0), ALIAS),
        (dict(dx=H0 + 16), ALIAS),
        (dict(ws_bytes=16), WS),
        (dict(act=0, ws_bytes=16), WS),  # the variant without an activation exists for the default launch
        (dict(dx_st=504, dx_sb=64 * 504), STRIDE),
        (dict(dx_st=1020, dx_sb=64 * 1020), STRIDE),
        (dict(dx_st=1024, dx_sb=1024 * 63), STRIDE),
        (dict(dx_st=1024, dx_sb=1024 * 64, ws_bytes=16), WS),  # valid strides: the next check speaks
    ],
)
def test_bwd_ex_host_errors(kw, code):
    assert bwd_ex(**kw) == code


def test_odd_channel_counts_need_the_narrow_launch():
    """With D odd only the one-channel-per-lane plan is accepted, with plain hints and the
    general kernel; two or four channels per lane need an even D."""
    L = cc.lib()
    T, D = 64, 501
    vec4 = cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=64)
    assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, 2, T, D, 4, ctypes.byref(vec4), None) == CONFIG
    narrow = cc.cconv_default_config("fwd", 2, T, D, 4)
    assert narrow.vec == 1 and narrow.rows_per_group == 16 and narrow.options == 0
    # accepted: with y aliasing x it gets as far as the aliasing check
    assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, 2, T, D, 4, ctypes.byref(narrow), None) == ALIAS
    for vv in (1, 2):
        solo = cc.Config(vec=vv, rows_per_group=16, waves_per_block=1, options=11, seg_rows=64)
        assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, 2, T, D, 4, ctypes.byref(solo), None) == CONFIG
        g8 = cc.Config(vec=vv, rows_per_group=8, waves_per_block=1, options=0, seg_rows=64)
        assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, 2, T, D, 4, ctypes.byref(g8), None) == CONFIG
    nb = cc.cconv_default_config("bwd", 2, T, D, 4)
    assert nb.vec == 1 and nb.options == 0 and nb.waves_per_block == 1
    pair = cc.Config(vec=2, rows_per_group=16, waves_per_block=1, options=0, seg_rows=64)
    assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, 2, T, D, 4, ctypes.byref(pair), None) == CONFIG


def test_four_channel_plans_for_d_2_mod_4():
    """D = 2 (mod 4), D >= 6: the default plan runs 4 channels per lane (the last lane group
    overlapping its neighbour) on the solo kernels; its activations need 4-byte alignment and
    even strides, everything else element alignment; activations off that rule take one
    channel per lane with the same segments (so the same workspace). Explicit two- and
    four-channel plans are checked against the same rule; eight channels per lane and four at
    D = 2 are refused. A call that passes every check stops at the aliasing check (y on x), so
    nothing is launched."""
    L = cc.lib()
    D, T, B = 502, 64, 2
    assert fwd(D=D, y=X) == ALIAS
    assert fwd(D=D, x=X + 4, y=X + 4) == ALIAS
    assert fwd(D=D, w=WT + 2, bias=BIAS + 4, y=X) == ALIAS
    # off the rule: 2-byte aligned rows, odd strides -> one channel per lane, accepted
    assert fwd(D=D, x=X + 2, y=X + 2) == ALIAS
    assert fwd(D=D, x_st=503, y=X) == ALIAS
    assert fwd(D=D, x_sb=T * D + 1, y=X) == ALIAS
    assert fwd(D=D, y=Y + 1) == MISAL
    assert bwd(D=D, dx=X) == ALIAS
    assert bwd(D=D, dx=X + 2) == ALIAS
    assert bwd(D=D, dy_st=503, dx=X) == ALIAS
    need = L.cconv_bwd_workspace_bytes(B, T, D, 4)
    assert need > 0
    assert bwd(D=D, dx=DX + 2, dy=DY + 2, x=X + 2, ws_bytes=need - 1) == WS
    for vec, opts in ((2, 0), (4, 8), (4, 11)):
        c = cc.Config(vec=vec, rows_per_group=16, waves_per_block=1, options=opts, seg_rows=64)
        assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, B, T, D, 4, ctypes.byref(c), None) == ALIAS
        assert L.cconv_fwd_config(X + 4, T * D, D, WT, BF16, BIAS, X + 4, B, T, D, 4, ctypes.byref(c), None) == ALIAS
        assert L.cconv_fwd_config(X + 2, T * D, D, WT, BF16, BIAS, Y, B, T, D, 4, ctypes.byref(c), None) == MISAL
        assert L.cconv_fwd_config(X, T * 503, 503, WT, BF16, BIAS, Y, B, T, D, 4, ctypes.byref(c), None) == STRIDE
    v8 = cc.Config(vec=8, rows_per_group=8, waves_per_block=1, options=11, seg_rows=64)
    assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, B, T, D, 4, ctypes.byref(v8), None) == CONFIG
    v4 = cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=8, seg_rows=64)
    assert L.cconv_fwd_config(X, T * 2, 2, WT, BF16, BIAS, X, B, T, 2, 4, ctypes.byref(v4), None) == CONFIG
    assert cc.cconv_default_config("fwd", B, T, 2, 4).vec == 2
    assert cc.cconv_default_config("fwd", B, T, 6, 4).vec == 4
    # the default plan's partials (and the workspace) follow the shape, not the layout
    c4 = cc.cconv_default_config("bwd", 8, 8192, 4098, 4)
    assert (c4.vec, c4.options) == (4, 8)
    one = cc.Config(**{**c4.as_dict(), "vec": 1, "options": 0})
    assert cc.cconv_bwd_workspace_bytes(8, 8192, 4098, 4, one) == cc.cconv_bwd_workspace_bytes(8, 8192, 4098, 4)


def test_four_channel_plans_for_d_4_mod_8():
    """D = 4 (mod 8): the default plan runs 4 channels per lane, its activations need 8-byte
    alignment and strides that are multiples of 4, its taps, bias, dw and states only element
    alignment; 8 channels per lane is refused, and an explicit one-channel plan still takes any
    layout. A call that passes every check stops at the aliasing check (y on x), so nothing is
    launched."""
    L = cc.lib()
    D, T, B = 500, 64, 2
    for which in ("fwd", "bwd"):
        # a small call keeps the streaming hints; a large one, whose rows miss the 128-byte
        # lines, takes plain ones
        c = cc.cconv_default_config(which, B, T, D, 4)
        assert c.vec == 4 and c.options == 11 and c.rows_per_group == 16
        c = cc.cconv_default_config(which, 8, 8192, 4100, 4)
        assert c.vec == 4 and c.options == 8
    # accepted: 8-byte aligned activations, strides a multiple of 4, taps and bias off 16 bytes
    assert fwd(D=D, y=X) == ALIAS
    assert fwd(D=D, x=X + 8, y=X + 8) == ALIAS
    assert fwd(D=D, x_st=504, y=X) == ALIAS
    assert fwd(D=D, w=WT + 2, bias=BIAS + 4, y=X) == ALIAS
    assert fwd(D=D, w=WT + 4, w_dt=F32, y=X) == ALIAS
    # activations off the rule (4-byte aligned rows, strides off the 4-element granule): the
    # default plan runs one channel per lane instead, so these are accepted too
    assert fwd(D=D, x=X + 4, y=X + 4) == ALIAS
    assert fwd(D=D, x_st=502, y=X) == ALIAS
    assert fwd(D=D, x_sb=T * D + 2, y=X) == ALIAS
    assert fwd(D=D, y=Y + 1) == MISAL
    assert fwd(D=D, w=WT + 1) == MISAL
    # the backward: dw and dbias per element; dx, x, dy on the 8-byte rule or the fallback
    assert bwd(D=D, dx=X) == ALIAS
    assert bwd(D=D, dw=DW + 2, db=DB + 4, dx=X) == ALIAS
    assert bwd(D=D, dx=X + 4) == ALIAS
    assert bwd(D=D, dy_st=502, dx=X) == ALIAS
    assert bwd(D=D, dx=DX + 1) == MISAL
    # the fallback keeps the shape's partials: the workspace is the 4-channel plan's
    need = L.cconv_bwd_workspace_bytes(B, T, D, 4)
    assert need > 0
    assert bwd(D=D, dx=DX + 4, dy=DY + 4, x=X + 4, ws_bytes=need - 1) == WS
    # D a multiple of 8 keeps the 16-byte rule
    assert fwd(D=512, x=X + 8) == MISAL
    assert fwd(D=512, x_st=516) == STRIDE
    # explicit plans: 8 channels per lane needs D % 8 == 0; one channel per lane takes any layout
    vec8 = cc.Config(vec=8, rows_per_group=16, waves_per_block=1, options=8, seg_rows=64)
    vec4 = cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=8, seg_rows=64)
    one = cc.Config(vec=1, rows_per_group=16, waves_per_block=1, options=0, seg_rows=64)
    assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, B, T, D, 4, ctypes.byref(vec8), None) == CONFIG
    assert L.cconv_fwd_config(X, T * D, D, WT, BF16, BIAS, X, B, T, D, 4, ctypes.byref(vec4), None) == ALIAS
    assert L.cconv_fwd_config(X + 4, T * D, D, WT, BF16, BIAS, Y, B, T, D, 4, ctypes.byref(vec4), None) == MISAL
    assert L.cconv_fwd_config(X + 2, T * 502, 502, WT, BF16, BIAS, X + 2, B, T, D, 4, ctypes.byref(one), None) == ALIAS


def test_backward_row_strides_beyond_the_group_offsets():
    """The 4- and 8-channel backward addresses a row group as 32-bit offsets from its first row,
    so its row strides are at most 2^26 elements: beyond that the default plan runs one channel
    per lane (same segments, so the same workspace) and an explicit 4-channel plan is
    CCONV_ERR_BAD_STRIDE. The forward has no such limit. A call that passes every check stops at
    the aliasing check (dx or y on x), so nothing is launched."""
    L = cc.lib()
    B, T, D, W = 1, 16, 512, 4
    big, edge = (1 << 26) + 8, 1 << 26
    assert bwd(B=B, T=T, D=D, x_st=big, dx=X) == ALIAS
    assert bwd(B=B, T=T, D=D, dy_st=big, dx=X) == ALIAS
    assert bwd(B=B, T=T, D=D, x_st=edge, dx=X) == ALIAS
    assert fwd(B=B, T=T, D=D, x_st=big, y=X) == ALIAS

    def bwd_cfg(cfg, x_st):
        return L.cconv_bwd_config(X, T * x_st, x_st, DY, T * D, D, WT, BF16, BIAS, X, DW, BF16, DB, WSP, 1 << 40,
                                  B, T, D, W, ctypes.byref(cfg), None)

    v4 = cc.Config(vec=4, rows_per_group=16, waves_per_block=1, options=11, seg_rows=16)
    v1 = cc.Config(vec=1, rows_per_group=16, waves_per_block=1, options=0, seg_rows=16)
    assert bwd_cfg(v4, big) == STRIDE
    assert bwd_cfg(v4, edge) == ALIAS
    assert bwd_cfg(v1, big) == ALIAS
