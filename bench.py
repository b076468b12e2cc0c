#!/usr/bin/env python
"""Benchmark of the causal depthwise short convolution + SiLU hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
    forward  y = silu(conv(x))            x bf16 [8, 8192, 4096], w bf16 [4096, 4], bias fp32
    backward dx, dw, dbias (main kernel + fixed-order dw/dbias reduction)
    decode   one-token update of a rolling state: x [256, 4096], state [512, 4096, 3]
The printed value is the algorithmic bytes of every timed step (what the method must move:
x + y + taps + bias forward; x + dy + dx + taps + dw + bias + dbias backward; x + state read
and write + y + taps + bias + indices decode) divided by the wall time of the timed region,
inputs already resident in HBM. HIP events on the launch stream around the backward's main
kernel, the dominant one, give its duration inside the timed region (the only events there);
it is reported against MI355X's 8 TB/s HBM peak ("roofline"). A second pass of as many steps,
with events around every phase, gives the per-phase breakdown, each phase set against a flat
copy with the same read:write mix measured in the same run. The CPU oracle is timed beside it on a bounded
sample of the same workload ("cpu_baseline"); that leg also serves as the parity gate.

After the headline (outside the printed value): the decode update timed as a graph of 24
back-to-back calls (from HBM and cache-resident), the other training workloads (B1/T256/D512,
B8/T1024/D4096 without bias, B3/T1000/D2000/W2) each as graphs of back-to-back calls over
rotated buffer sets with a same-size flat copy beside them and the oracle timed and checked on
each, and every widened row of the path timed alone
at its own workload ("variants": a history in and the final state or its gradient out, prefill
into a decode pool, a packed batch of mixed lengths, no activation and a residual, a D that is
not a multiple of 8, D = 6144 contiguous and in rows of 8192, the pages' production call, a
fused q|k|v projection in one call and in three, and the decode state of W entries, shifted or
circular), each checked
against the oracle on a sample and the oracle timed on that sample.

Usage: python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--profile]
(--gpus N with N > 1 is refused: the library runs on one GPU; how the path would shard is a
design note, not code.)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "effective HBM GB/s (fwd, bwd) B8/T8192/D4096/W4 bf16; % of flat-copy roofline"
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
TRAFFIC_FILE = ROOT / "profiles" / "bwd_main_B8_T8192_D4096_W4_traffic.txt"
KERNEL_SOURCES = [
    "causal_depthwise_short_amd/csrc/cconv_bwd.hip",
    "causal_depthwise_short_amd/csrc/cconv_bwd_body.hpp",
    "causal_depthwise_short_amd/csrc/cconv_device.hpp",
    "causal_depthwise_short_amd/csrc/cconv_internal.hpp",
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (and with it the parity gate)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--profile", action="store_true",
                    help="profiling run: steps, decode graph replays and calibration copies only (no sweep, no oracle)")
    ap.add_argument("--profile-shapes", action="store_true",
                    help="profiling run of the widths off the 8-channel path: forward and backward at [8,8192,D] for "
                         "D = 4098, 4100, 4104 and 6144, then calibration copies")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per backward-main launch from the committed rocprofv3 counter summary, or
    None if it is absent or was taken on a different kernel source."""
    if not TRAFFIC_FILE.exists():
        return None
    vals = {}
    for line in TRAFFIC_FILE.read_text().splitlines():
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_variants(cc, si, torch, dev, host, dhost, s, dshape, x, dy, w, b, y, dxo, dwo, dbo, ws, quant, copy1, copy2,
                 peak, rounds=7, reps=5):
    """Times each widened row of the path alone at its own workload and keeps, for the parity
    check in the oracle leg, host copies of the GPU outputs of a sample (batch row 0, the first
    packed sequences, or the whole decode call) together with the inputs the oracle needs.
    Algorithmic bytes as for the headline phases, plus each row's own state traffic.

    All inputs are set up first; then a sustained warm-up; then `rounds` round-robin passes
    over the variants, `reps` back-to-back calls each (event-timed), so that no variant is
    timed right after an idle gap; the parity samples are copied out only after all timing."""
    B, T, D, W = s.B, s.T, s.D, s.W
    R = W - 1
    n = B * T * D
    wb = w.numel() * w.element_size()
    fwd_b = 4 * n + wb + D * 4
    bwd_b = 6 * n + wb + 2 * D * 4 + dwo.numel() * dwo.element_size()
    hist_b = B * D * R * 2
    st = torch.empty(1, dtype=torch.int32, device=dev)
    S = {"_host": {
        "x1": host["x"][:1], "dy1": host["dy"][:1], "w": host["w"], "b": host["bias"],
        "xp": host["x"].view(B * T, D), "dyp": host["dy"].view(B * T, D),
        "xd": dhost["x"], "idxd": dhost["state_indices"], "wd": dhost["w"], "bd": dhost["bias"],
        "state": dhost["state"],
    }}
    todo = []  # (name, what, workload, bytes, fn, copy GB/s, extra, capture)

    def sync_ok():
        torch.cuda.synchronize()
        return int(st.item()) == 0

    shape = f"[{B},{T},{D}] W={W}"
    # state handoff: a history before t = 0 in, the final state (forward) or the history's
    # gradient (backward) out, [B, D, W-1] each
    h0 = si.history_input(B, D, W, seed=s.seed)
    h0d = h0.to(dev)
    hT, dh0 = torch.empty_like(h0d), torch.empty_like(h0d)

    def cap_fwd_state():
        torch.cuda.synchronize()
        S["fwd_state"] = {"h0": h0[:1], "y": y[0].cpu(), "hT": hT[0].cpu()}

    def cap_bwd_state():
        torch.cuda.synchronize()
        S["bwd_state"] = {"h0": h0[:1], "dx": dxo[0].cpu(), "dh0": dh0[0].cpu()}

    todo.append(("fwd_state", "forward from a history, final state out", shape, fwd_b + 2 * hist_b,
                 lambda: cc.cconv_fwd_state(x, w, b, h0d, final_state=hT, y=y), copy1, {}, cap_fwd_state))
    todo.append(("bwd_state", "backward with a history, its gradient out", shape, bwd_b + 2 * hist_b,
                 lambda: cc.cconv_bwd_state(x, dy, w, b, h0d, dx=dxo, dw=dwo, dbias=dbo, d_init_state=dh0,
                                            workspace=ws), copy2, {}, cap_bwd_state))

    # prefill into a decode pool of 64 slots: rows 0, 1, 3, 4, 6, 7 continue from their slot,
    # rows 2 and 5 start fresh; every row's final state goes back to its slot
    Sp = 64
    g = torch.Generator().manual_seed(s.seed + 2000)
    pool = si.history_input(Sp, D, W, seed=s.seed + 7)
    idx = torch.randperm(Sp, generator=g)[:B].to(torch.int32)
    has = (torch.arange(B) % 3 != 2).to(torch.uint8)
    poold, idxd, hasd = pool.to(dev), idx.to(dev), has.to(dev)
    fn_pool = lambda: cc.cconv_fwd_pool(x, w, b, poold, idxd, hasd, y=y, status=st)  # noqa: E731

    def cap_pool():
        poold.copy_(pool.to(dev))
        fn_pool()
        ok = sync_ok()
        S["fwd_pool"] = {"pool": pool, "idx": idx[:1], "has": has[:1], "y": y[0].cpu(),
                         "slot": poold[int(idx[0])].cpu(), "status_ok": ok}

    todo.append(("fwd_pool", "prefill into a decode pool (slot indices, has_initial_state)",
                 f"{shape}, pool [{Sp},{D},{R}]", fwd_b + int(has.sum()) * D * R * 2 + hist_b + B * 5, fn_pool, copy1,
                 {}, cap_pool))

    # packed batch: the same B*T rows as one [total, D] batch of a log-uniform length mix,
    # each sequence with its own history, final state and history gradient
    lens = si.packed_lengths(B * T, seed=s.seed + 3)
    nseq = len(lens)
    cu = torch.zeros(nseq + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    cud = cu.to(dev)
    h0v = si.history_input(nseq, D, W, seed=s.seed + 11)
    h0vd = h0v.to(dev)
    hTv, dh0v = torch.empty_like(h0vd), torch.empty_like(h0vd)
    xp, dyp, yp, dxp = (t.view(B * T, D) for t in (x, dy, y, dxo))
    wsv = torch.empty(cc.cconv_bwd_workspace_bytes(1, B * T, D, W) // 4 + 1, dtype=torch.float32, device=dev)
    vb = 2 * nseq * D * R * 2 + (nseq + 1) * 4
    work = f"[{B * T},{D}] W={W}, {nseq} sequences of 1..{max(lens)} rows"
    fnf = lambda: cc.cconv_fwd_varlen(xp, cud, w, b, h0vd, final_state=hTv, want_final_state=True,  # noqa: E731
                                      y=yp, status=st)
    fnb = lambda: cc.cconv_bwd_varlen(xp, dyp, cud, w, b, h0vd, dx=dxp, dw=dwo, dbias=dbo,  # noqa: E731
                                      d_init_state=dh0v, want_d_init_state=True, workspace=wsv, status=st)

    def cap_varlen():
        k = max(1, int((cu[1:] <= 12288).sum()))
        rows = int(cu[k])
        fnf()
        okf = sync_ok()
        fnb()
        okb = sync_ok()
        S["varlen"] = {"rows": rows, "cu": cu[: k + 1], "h0": h0v[:k], "y": yp[:rows].cpu(), "hT": hTv[:k].cpu(),
                       "dx": dxp[:rows].cpu(), "dh0": dh0v[:k].cpu(), "status_ok": okf and okb}

    todo.append(("fwd_varlen", "packed batch forward (histories in, final states out)", work, fwd_b + vb, fnf,
                 copy1, {}, None))
    todo.append(("bwd_varlen", "packed batch backward (histories in, their gradients out)", work, bwd_b + vb, fnb,
                 copy2, {}, cap_varlen))

    # epilogues: no activation with a residual added (forward), no activation (backward)
    def cap_lin_f():
        torch.cuda.synchronize()
        S["fwd_linear_residual"] = {"y": y[0].cpu()}

    def cap_lin_b():
        torch.cuda.synchronize()
        S["bwd_linear"] = {"dx": dxo[0].cpu()}

    todo.append(("fwd_linear_residual", "forward without activation, residual added (dy as the residual)", shape,
                 6 * n + wb + D * 4, lambda: cc.cconv_fwd_ex(x, w, b, activation=None, residual=dy, y=y), copy2, {},
                 cap_lin_f))
    todo.append(("bwd_linear", "backward without activation", shape, bwd_b,
                 lambda: cc.cconv_bwd_ex(x, dy, w, b, activation=None, dx=dxo, dw=dwo, dbias=dbo, workspace=ws),
                 copy2, {}, cap_lin_b))

    # D other than the headline's: 4098 = 2 (mod 4) 4-channel lanes on 4-byte aligned rows (the
    # last group overlapping the one before), 4100 = 4 (mod 8) 4-channel lanes on 8-byte aligned
    # rows, 4104 the vector path with 17 channel strips whose rows do not start on cache lines
    big = []
    for Bn, Dn, tag, what in ((B, 4098, "any_d", "D = 4098 (4 channels per lane, 4-byte aligned rows)"),
                              (B, 4100, "d4100", "D = 4100 (4 channels per lane, 8-byte aligned rows)"),
                              (B, 4104, "d4104", "D = 4104 (vector path, rows not on 128-byte lines)"),
                              (2 * B, D // 2, "b16_d2048", "the pages' production call shape (B = 16, D = 2048)")):
        nin = si.train_inputs_device(Bn, T, Dn, W, bias=True, seed=s.seed + 5, device=dev)
        xn, wn, bn, dyn = nin["x"], nin["w"], nin["bias"], nin["dy"]
        yn, dxn = torch.empty_like(xn), torch.empty_like(xn)
        dwn, dbn = torch.empty_like(wn), torch.empty(Dn, dtype=torch.float32, device=dev)
        wsn = torch.empty(cc.cconv_bwd_workspace_bytes(Bn, T, Dn, W) // 4 + 1, dtype=torch.float32, device=dev)
        big.append((nin, yn, dxn, wsn))
        nn_ = Bn * T * Dn
        wnb = wn.numel() * wn.element_size()
        work = f"[{Bn},{T},{Dn}] W={W}"

        def cap(tag=tag, xn=xn, dyn=dyn, wn=wn, bn=bn, yn=yn, dxn=dxn):
            torch.cuda.synchronize()
            S[tag] = {"x": xn[:1].cpu(), "dy": dyn[:1].cpu(), "w": wn.cpu(), "b": bn.cpu(), "y": yn[0].cpu(),
                      "dx": dxn[0].cpu()}

        todo.append((f"fwd_{tag}", f"forward, {what}", work, 4 * nn_ + wnb + Dn * 4,
                     lambda xn=xn, wn=wn, bn=bn, yn=yn: cc.cconv_fwd(xn, wn, bn, y=yn), copy1, {}, None))
        todo.append((f"bwd_{tag}", f"backward, {what}", work, 6 * nn_ + 2 * wnb + 2 * Dn * 4,
                     lambda xn=xn, dyn=dyn, wn=wn, bn=bn, dxn=dxn, dwn=dwn, dbn=dbn, wsn=wsn:
                     cc.cconv_bwd(xn, dyn, wn, bn, dx=dxn, dw=dwn, dbias=dbn, workspace=wsn), copy2, {}, cap))

    # a width that is not a power of two (6144, v of a 24-head KDA layer), once contiguous and
    # once with every row of x, dy, y and dx at a power-of-two pitch (8192) through the general
    # entry points' strides
    Dp, Pp = 6144, 8192
    pin = si.train_inputs_device(B, T, Dp, W, bias=True, seed=s.seed + 7, device=dev)
    xc, dyc, wp, bp = pin["x"], pin["dy"], pin["w"], pin["bias"]

    def pitched(t=None):
        v = torch.empty(B, T, Pp, dtype=torch.bfloat16, device=dev)[:, :, :Dp]
        if t is not None:
            v.copy_(t)
        return v

    xpd, dypd, ypd, dxpd = pitched(xc), pitched(dyc), pitched(), pitched()
    yc, dxc = torch.empty_like(xc), torch.empty_like(xc)
    dwp, dbp = torch.empty_like(wp), torch.empty(Dp, dtype=torch.float32, device=dev)
    wsp = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, Dp, W) // 4 + 1, dtype=torch.float32, device=dev)
    npd = B * T * Dp
    wpb = wp.numel() * wp.element_size()
    fb_p, bb_p = 4 * npd + wpb + Dp * 4, 6 * npd + 2 * wpb + 2 * Dp * 4

    def cap_pitch():
        cc.cconv_fwd(xc, wp, bp, y=yc)
        cc.cconv_fwd_ex(xpd, wp, bp, y=ypd)
        cc.cconv_bwd(xc, dyc, wp, bp, dx=dxc, dw=dwp, dbias=dbp, workspace=wsp)
        cc.cconv_bwd_ex(xpd, dypd, wp, bp, dx=dxpd, workspace=wsp)
        torch.cuda.synchronize()
        S["pitch"] = {"x": xc[:1].cpu(), "dy": dyc[:1].cpu(), "w": wp.cpu(), "b": bp.cpu(), "y": yc[0].cpu(),
                      "dx": dxc[0].cpu(), "y_p": ypd[0].contiguous().cpu(), "dx_p": dxpd[0].contiguous().cpu()}

    work_c, work_p = f"[{B},{T},{Dp}] W={W}", f"[{B},{T},{Dp}] W={W}, rows at pitch {Pp}"
    todo.append(("fwd_d6144", "forward, D = 6144 contiguous", work_c, fb_p,
                 lambda: cc.cconv_fwd(xc, wp, bp, y=yc), copy1, {}, None))
    todo.append(("fwd_d6144_pitch8192", "forward, D = 6144 in rows of 8192", work_p, fb_p,
                 lambda: cc.cconv_fwd_ex(xpd, wp, bp, y=ypd), copy1, {}, None))
    todo.append(("bwd_d6144", "backward, D = 6144 contiguous", work_c, bb_p,
                 lambda: cc.cconv_bwd(xc, dyc, wp, bp, dx=dxc, dw=dwp, dbias=dbp, workspace=wsp), copy2, {}, None))
    todo.append(("bwd_d6144_pitch8192", "backward, D = 6144 in rows of 8192", work_p, bb_p,
                 lambda: cc.cconv_bwd_ex(xpd, dypd, wp, bp, dx=dxpd, dw=dwp, dbias=dbp, workspace=wsp), copy2, {},
                 cap_pitch))
    big.append((pin, xpd, dypd, ypd, dxpd, yc, dxc, wsp))

    # a fused q|k|v projection of a KDA layer: q and k at 1024 channels, v at twice that, so
    # [B, T, 4096] in all; one call over the 4096 channels (the three taps and biases
    # concatenated) against three calls on its channel slices (row stride 4096)
    parts = (1024, 1024, 2048)
    Dq = sum(parts)
    qin = si.train_inputs_device(B, T, Dq, W, bias=True, seed=s.seed + 6, device=dev)
    xq, wq, bq, dyq = qin["x"], qin["w"], qin["bias"], qin["dy"]
    yq, dxq = torch.empty_like(xq), torch.empty_like(xq)
    dwq, dbq = torch.empty_like(wq), torch.empty(Dq, dtype=torch.float32, device=dev)
    wsq = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, Dq, W) // 4 + 1, dtype=torch.float32, device=dev)
    edges = [0, parts[0], parts[0] + parts[1], Dq]
    sl = [slice(edges[j], edges[j + 1]) for j in range(3)]
    x3 = [xq[:, :, q] for q in sl]
    dy3 = [dyq[:, :, q] for q in sl]
    w3 = [wq[q].contiguous() for q in sl]
    b3 = [bq[q].contiguous() for q in sl]
    y3 = [torch.empty(B, T, p_, dtype=torch.bfloat16, device=dev) for p_ in parts]
    dx3 = [torch.empty(B, T, p_, dtype=torch.bfloat16, device=dev) for p_ in parts]
    dw3 = [torch.empty_like(t) for t in w3]
    db3 = [torch.empty(p_, dtype=torch.float32, device=dev) for p_ in parts]
    ws3 = [torch.empty(cc.cconv_bwd_workspace_bytes(B, T, p_, W) // 4 + 1, dtype=torch.float32, device=dev)
           for p_ in parts]
    nq = B * T * Dq
    wqb = wq.numel() * wq.element_size()
    work = f"[{B},{T},{parts[0]}+{parts[1]}+{parts[2]}] W={W}"

    def fwd3():
        for j in range(3):
            cc.cconv_fwd(x3[j], w3[j], b3[j], y=y3[j])

    def bwd3():
        for j in range(3):
            cc.cconv_bwd(x3[j], dy3[j], w3[j], b3[j], dx=dx3[j], dw=dw3[j], dbias=db3[j], workspace=ws3[j])

    def cap_qkv():
        cc.cconv_fwd(xq, wq, bq, y=yq)
        cc.cconv_bwd(xq, dyq, wq, bq, dx=dxq, dw=dwq, dbias=dbq, workspace=wsq)
        fwd3()
        bwd3()
        torch.cuda.synchronize()
        S["qkv"] = {"x": xq[:1].cpu(), "dy": dyq[:1].cpu(), "w": wq.cpu(), "b": bq.cpu(), "y": yq[0].cpu(),
                    "dx": dxq[0].cpu(), "y3": torch.cat([t[0] for t in y3], dim=1).cpu(),
                    "dx3": torch.cat([t[0] for t in dx3], dim=1).cpu()}

    todo.append(("fwd_qkv_one", "forward, fused q|k|v in one call", work, 4 * nq + wqb + Dq * 4,
                 lambda: cc.cconv_fwd(xq, wq, bq, y=yq), copy1, {}, None))
    todo.append(("fwd_qkv_three", "forward, fused q|k|v as three strided calls", work, 4 * nq + wqb + Dq * 4,
                 fwd3, copy1, {}, None))
    todo.append(("bwd_qkv_one", "backward, fused q|k|v in one call", work, 6 * nq + 2 * wqb + 2 * Dq * 4,
                 lambda: cc.cconv_bwd(xq, dyq, wq, bq, dx=dxq, dw=dwq, dbias=dbq, workspace=wsq), copy2, {}, None))
    todo.append(("bwd_qkv_three", "backward, fused q|k|v as three strided calls", work,
                 6 * nq + 2 * wqb + 2 * Dq * 4, bwd3, copy2, {}, cap_qkv))
    big.append((qin, yq, dxq, wsq, y3, dx3, ws3))

    # decode variants at the decode workload: a state of L = W entries, rewritten (shift) or
    # addressed as a circular buffer by cache_seqlens (one entry written per channel)
    Nd, Sd, Dd = dshape.N, dshape.S, dshape.D
    g = torch.Generator().manual_seed(dshape.seed + 9)
    st4 = torch.randn(Sd, Dd, W, generator=g).to(torch.bfloat16)
    cs = torch.randint(0, 1 << 20, (Nd,), generator=g, dtype=torch.int32)
    xdd, idd = dhost["x"].to(dev), dhost["state_indices"].to(dev)
    wdd, bdd = dhost["w"].to(dev), dhost["bias"].to(dev)
    st4d, csd = st4.to(dev), cs.to(dev)
    yd4 = torch.empty(Nd, Dd, dtype=torch.bfloat16, device=dev)
    fixed = 4 * Nd * Dd + dhost["w"].numel() * dhost["w"].element_size() + Dd * 4 + Nd * 4
    work = f"x [{Nd},{Dd}], state [{Sd},{Dd},{W}], W={W}"
    for name, what, nb, kw in (
        ("update_shift_l4", "decode, state of L = W entries, shifted", fixed + 2 * Nd * Dd * (R + W), {}),
        ("update_circular_l4", "decode, circular state (cache_seqlens)", fixed + 2 * Nd * Dd * (R + 1) + Nd * 4,
         {"cache_seqlens": csd}),
    ):
        fn = lambda kw=kw: cc.cconv_update_ex(xdd, st4d, idd, wdd, bdd, y=yd4, status=st, **kw)  # noqa: E731

        def cap(name=name, fn=fn, kw=kw):
            st4d.copy_(st4.to(dev))
            fn()
            ok = sync_ok()
            S[name] = {"state": st4, "cs": cs if kw else None, "y": yd4.cpu(), "new_state": st4d.cpu(),
                       "status_ok": ok}

        todo.append((name, what, work, nb, fn, copy1, {"cache_resident": True}, cap))

    # the headline decode with its buffers rotated over 24 sets (x, state, y: 302 MB, more than
    # the 256 MB Infinity Cache), so that each call finds its data in HBM
    nsets = 24
    L = W - 1
    xs_r = [dhost["x"].to(dev) for _ in range(nsets)]
    st_r = [dhost["state"].to(dev) for _ in range(nsets)]
    y_r = [torch.empty(Nd, Dd, dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    rot = {"i": 0}

    def fn_rot():
        i = rot["i"]
        rot["i"] = (i + 1) % nsets
        cc.cconv_update(xs_r[i], st_r[i], idd, wdd, bdd, y=y_r[i], status=st)

    def cap_rot():
        st_r[0].copy_(dhost["state"].to(dev))
        cc.cconv_update(xs_r[0], st_r[0], idd, wdd, bdd, y=y_r[0], status=st)
        ok = sync_ok()
        S["update_hbm"] = {"y": y_r[0].cpu(), "new_state": st_r[0].cpu(), "status_ok": ok}

    todo.append(("update_hbm", "decode (the headline's), buffers rotated over 24 sets so data comes from HBM",
                 f"x [{Nd},{Dd}], state [{Sd},{Dd},{L}], W={W}, 24 sets", fixed + 2 * Nd * Dd * 2 * L, fn_rot, copy1,
                 {"cache_resident": False}, cap_rot))

    # sustained warm-up (every variant, then the plain path for ~30 ms), then the rounds
    for item in todo:
        item[4]()
    torch.cuda.synchronize()
    for _ in range(60):
        cc.cconv_fwd(x, w, b, y=y)
    times = {item[0]: [] for item in todo}
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for _ in range(rounds):
        evs = []
        for item in todo:
            for _ in range(reps):
                e0, e1 = mk(), mk()
                e0.record()
                item[4]()
                e1.record()
                evs.append((item[0], e0, e1))
        torch.cuda.synchronize()
        for name, e0, e1 in evs:
            times[name].append(e0.elapsed_time(e1) * 1e-3)
    V = {}
    for name, what, workload, nb, _, copy_gbps, extra, _ in todo:
        q = quant(times[name])
        gbps = nb / q[1] / 1e9
        V[name] = {
            "what": what, "workload": workload, "us": round(q[1] * 1e6, 2),
            "us_p10_p90": [round(q[0] * 1e6, 2), round(q[2] * 1e6, 2)], "bytes": nb, "GBps": round(gbps, 1),
            "pct_flat_copy": round(100 * gbps / copy_gbps, 1), "pct_hbm_peak": round(100 * gbps / peak, 1),
            "parity": None, **extra,
        }
    # parity samples, after all timing: each variant runs again first (the variants share the
    # output buffers)
    for item in todo:
        if item[7] is not None:
            item[4]()
            item[7]()
    del big, xs_r, st_r, y_r
    return V, S


def oracle_variants(oracle, np, torch, S, err):
    """The oracle on each variant's sample: its throughput (algorithmic bytes of the sample over
    the oracle's time) and the parity of the GPU outputs against it (max |gpu - oracle| /
    max(1, |oracle|); 5e-3 for forward outputs, 8e-3 for gradients; states bit for bit)."""
    import time as _t

    H = S["_host"]
    cpu, gate = {}, {}
    bits = lambda t: t.contiguous().view(torch.int16)  # noqa: E731

    def same(g, r):
        return bool(torch.equal(bits(g), bits(torch.from_numpy(np.asarray(r, np.float32)).to(torch.bfloat16))))

    def put(name, t, nbytes, sample, checks):
        cpu[name] = {"GBps": round(nbytes / t / 1e9, 4), "s": round(t, 2), "sample": sample}
        gate[name] = dict(checks, **{"pass": all(v is True or (isinstance(v, float) and v <= lim)
                                                 for (v, lim) in checks.values())})

    x1, dy1, w, b = H["x1"], H["dy1"], H["w"], H["b"]
    T, D, W = x1.shape[1], x1.shape[2], w.shape[1]
    one = f"batch row 0 ({T} x {D})"
    t0 = _t.perf_counter()
    yr, hTr = oracle.fwd_state(x1, S["fwd_state"]["h0"], w, b, precision="f32")
    t = _t.perf_counter() - t0
    v = S["fwd_state"]
    put("fwd_state", t, 4 * T * D, one, {"y": (err(v["y"].float(), yr[0]), 5e-3),
                                           "final_state_bit_exact": (same(v["hT"], hTr[0]), None)})
    t0 = _t.perf_counter()
    dxr, _, _, dh0r = oracle.bwd_state(x1, S["bwd_state"]["h0"], dy1, w, b, precision="f32")
    t = _t.perf_counter() - t0
    v = S["bwd_state"]
    put("bwd_state", t, 6 * T * D, one, {"dx": (err(v["dx"].float(), dxr[0]), 8e-3),
                                           "d_init_state": (err(v["dh0"].float(), dh0r[0]), 8e-3)})
    v = S["fwd_pool"]
    t0 = _t.perf_counter()
    ok, yr, sr = oracle.fwd_pool(x1, v["pool"], v["idx"].numpy(), v["has"].numpy(), w, b, precision="f32")
    t = _t.perf_counter() - t0
    put("fwd_pool", t, 4 * T * D, one, {"y": (err(v["y"].float(), yr[0]), 5e-3),
                                          "slot_bit_exact": (bool(ok and v["status_ok"]) and same(v["slot"], sr[int(v["idx"][0])]), None)})
    v = S["varlen"]
    rows = v["rows"]
    xs, dys = H["xp"][:rows], H["dyp"][:rows]
    t0 = _t.perf_counter()
    okf, yr, hTr = oracle.fwd_varlen(xs, v["cu"].numpy(), w, b, v["h0"], precision="f32")
    t1 = _t.perf_counter()
    okb, dxr, _, _, dh0r = oracle.bwd_varlen(xs, dys, v["cu"].numpy(), w, b, v["h0"], precision="f32")
    t2 = _t.perf_counter()
    samp = f"the first {len(v['cu']) - 1} sequences ({rows} rows)"
    put("fwd_varlen", t1 - t0, 4 * rows * D, samp,
        {"y": (err(v["y"].float(), yr), 5e-3),
         "final_state_bit_exact": (bool(okf and v["status_ok"]) and same(v["hT"], hTr), None)})
    put("bwd_varlen", t2 - t1, 6 * rows * D, samp,
        {"dx": (err(v["dx"].float(), dxr) if okb else 1.0, 8e-3),
         "d_init_state": (err(v["dh0"].float(), dh0r) if okb else 1.0, 8e-3)})
    t0 = _t.perf_counter()
    yr = oracle.fwd_epi(x1, w, b, residual=dy1, act=False, precision="f32")
    t = _t.perf_counter() - t0
    put("fwd_linear_residual", t, 6 * T * D, one, {"y": (err(S["fwd_linear_residual"]["y"].float(), yr[0]), 5e-3)})
    t0 = _t.perf_counter()
    dxr = oracle.bwd_epi(x1, dy1, w, b, act=False, precision="f32")[0]
    t = _t.perf_counter() - t0
    put("bwd_linear", t, 6 * T * D, one, {"dx": (err(S["bwd_linear"]["dx"].float(), dxr[0]), 8e-3)})
    for tag in ("any_d", "d4100", "d4104", "b16_d2048"):
        v = S[tag]
        Dn = v["x"].shape[2]
        t0 = _t.perf_counter()
        _, yr = oracle.fwd(v["x"], v["w"], v["b"], precision="f32")
        t1 = _t.perf_counter()
        dxr, _, _ = oracle.bwd(v["x"], v["dy"], v["w"], v["b"], precision="f32")
        t2 = _t.perf_counter()
        oned = f"batch row 0 ({T} x {Dn})"
        put(f"fwd_{tag}", t1 - t0, 4 * T * Dn, oned, {"y": (err(v["y"].float(), yr[0]), 5e-3)})
        put(f"bwd_{tag}", t2 - t1, 6 * T * Dn, oned, {"dx": (err(v["dx"].float(), dxr[0]), 8e-3)})
    for name in ("update_shift_l4", "update_circular_l4"):
        v = S[name]
        N, Dd = v["y"].shape
        Wd = v["state"].shape[2]
        t0 = _t.perf_counter()
        ok, yr, sr = oracle.update_ex(H["xd"], v["state"], H["idxd"].numpy(), None if v["cs"] is None else v["cs"].numpy(),
                                      H["wd"], H["bd"], precision="f32")
        t = _t.perf_counter() - t0
        nb = 2 * N * Dd * (1 + (Wd - 1) + (Wd if v["cs"] is None else 1) + 1)
        put(name, t, nb, f"the whole call (N={N})",
            {"y": (err(v["y"].float(), yr) if ok else 1.0, 5e-3),
             "state_bit_exact": (bool(ok and v["status_ok"]) and same(v["new_state"], sr), None)})
    v = S["pitch"]
    Dp = v["x"].shape[2]
    t0 = _t.perf_counter()
    _, yr = oracle.fwd(v["x"], v["w"], v["b"], precision="f32")
    t1 = _t.perf_counter()
    dxr, _, _ = oracle.bwd(v["x"], v["dy"], v["w"], v["b"], precision="f32")
    t2 = _t.perf_counter()
    onep = f"batch row 0 ({T} x {Dp})"
    put("fwd_d6144", t1 - t0, 4 * T * Dp, onep, {"y": (err(v["y"].float(), yr[0]), 5e-3)})
    put("bwd_d6144", t2 - t1, 6 * T * Dp, onep, {"dx": (err(v["dx"].float(), dxr[0]), 8e-3)})
    put("fwd_d6144_pitch8192", t1 - t0, 4 * T * Dp, onep,
        {"y": (err(v["y_p"].float(), yr[0]), 5e-3), "same_bits_as_contiguous": (bool(torch.equal(bits(v["y_p"]), bits(v["y"]))), None)})
    put("bwd_d6144_pitch8192", t2 - t1, 6 * T * Dp, onep,
        {"dx": (err(v["dx_p"].float(), dxr[0]), 8e-3), "same_bits_as_contiguous": (bool(torch.equal(bits(v["dx_p"]), bits(v["dx"]))), None)})
    v = S["qkv"]
    Dq3 = v["x"].shape[2]
    t0 = _t.perf_counter()
    _, yr = oracle.fwd(v["x"], v["w"], v["b"], precision="f32")
    t1 = _t.perf_counter()
    dxr, _, _ = oracle.bwd(v["x"], v["dy"], v["w"], v["b"], precision="f32")
    t2 = _t.perf_counter()
    oneq = f"batch row 0 ({T} x {Dq3})"
    put("fwd_qkv_one", t1 - t0, 4 * T * Dq3, oneq, {"y": (err(v["y"].float(), yr[0]), 5e-3)})
    put("bwd_qkv_one", t2 - t1, 6 * T * Dq3, oneq, {"dx": (err(v["dx"].float(), dxr[0]), 8e-3)})
    # the three strided calls must give the one call's y and dx bit for bit
    put("fwd_qkv_three", t1 - t0, 4 * T * Dq3, oneq,
        {"y": (err(v["y3"].float(), yr[0]), 5e-3), "same_bits_as_one_call": (bool(torch.equal(bits(v["y3"]), bits(v["y"]))), None)})
    put("bwd_qkv_three", t2 - t1, 6 * T * Dq3, oneq,
        {"dx": (err(v["dx3"].float(), dxr[0]), 8e-3), "same_bits_as_one_call": (bool(torch.equal(bits(v["dx3"]), bits(v["dx"]))), None)})
    v = S["update_hbm"]
    N, Dd = v["y"].shape
    t0 = _t.perf_counter()
    ok, yr, sr = oracle.update(H["xd"], H["state"], H["idxd"], H["wd"], H["bd"], precision="f32")
    t = _t.perf_counter() - t0
    put("update_hbm", t, 2 * N * Dd * (2 + 2 * H["state"].shape[2]), f"the whole call (N={N})",
        {"y": (err(v["y"].float(), yr) if ok else 1.0, 5e-3),
         "state_bit_exact": (bool(ok and v["status_ok"]) and same(v["new_state"], sr), None)})
    for g in gate.values():
        for k_, val in list(g.items()):
            if isinstance(val, tuple):
                g[k_] = val[0]
    return cpu, gate


def graph_time(torch, calls, reps=20, warm=3):
    """Per-call device time of `calls` (a list of zero-argument launches) captured back to back
    into one HIP graph: the median over `reps` replays of (replay time / number of calls), and
    the 10th and 90th percentiles. Host launch overhead and the gaps between eager launches are
    not in it. The calls run once eagerly first (outputs and lazily loaded code in place)."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for c in calls:
            c()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3 / len(calls))
    ts.sort()
    del g
    return ts[len(ts) // 10], ts[len(ts) // 2], ts[min(len(ts) - 1, (9 * len(ts)) // 10)]


def ulp_and_rms(oracle, np, gpu_bf16, ref, sum_of_terms=False):
    """(max bf16 ulps between a bf16 tensor and the oracle's value rounded to bf16 by the
    oracle, among elements further than a floor from it; normalized RMS ||gpu - ref|| /
    ||ref||). The floor is 2^-18 for element-wise outputs (an output that cancels to near zero
    carries an fp32 error of a few 2^-24 times its terms) and 1e-5 of the largest |ref| for
    the long sums dw (whose fp32 error scales with the size of their terms)."""
    import torch

    g16 = gpu_bf16.contiguous().view(torch.int16).reshape(-1).numpy().view(np.uint16)
    r = np.ascontiguousarray(np.asarray(ref, np.float64)).reshape(-1)
    rb = oracle.round_bf16(r)

    def ordered(b):
        b = b.astype(np.int32) & 0xFFFF
        m = b & 0x7FFF
        return np.where(b & 0x8000, -m, m)

    gf = gpu_bf16.float().contiguous().view(-1).numpy().astype(np.float64)
    d = np.abs(ordered(g16) - ordered(rb))
    floor = 1e-5 * float(np.max(np.abs(r))) if (sum_of_terms and r.size) else 2.0**-18
    d = np.where(np.abs(gf - r) <= floor, 0, d)
    nr = float(np.linalg.norm(gf - r) / max(np.linalg.norm(r), 1e-30))
    return (int(d.max()) if d.size else 0), nr


def time_configs(cc, si, torch, np, dev, copy_rates, peak, with_oracle, min_bytes=600e6):
    """The other training workloads (B1/T256/D512 with bias, B8/T1024/D4096 without, and the
    ragged B3/T1000/D2000/W2 with bias): forward and backward each timed as back-to-back calls
    in one graph, rotating over enough buffer sets (x, dy, y, dx) that a call finds its rows
    in HBM rather than in the 256 MB Infinity Cache; set against a flat copy of the same
    per-call size timed the same way. With `with_oracle`, the outputs of set 0 are checked
    against the float64 oracle in full and the fp32 oracle is timed on the whole workload."""
    R = cc.roofline_lib()
    cur = torch.cuda.current_stream
    out, cpu = {}, {}
    for shp in (si.TINY, si.MEDIUM, si.RAGGED):
        B, T, D, W = shp.B, shp.T, shp.D, shp.W
        inp = si.train_inputs_for(shp)
        ne = B * T * D
        nsets = int(min(512, max(2, -(-min_bytes // (8 * ne)))))
        xa = inp["x"].to(dev).unsqueeze(0).repeat(nsets, 1, 1, 1)
        dya = inp["dy"].to(dev).unsqueeze(0).repeat(nsets, 1, 1, 1)
        ya, dxa = torch.empty_like(xa), torch.empty_like(xa)
        w = inp["w"].to(dev)
        b = None if inp["bias"] is None else inp["bias"].to(dev)
        dwo, dbo = torch.empty_like(w), torch.empty(D, dtype=torch.float32, device=dev)
        ws = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, D, W) // 4 + 1, dtype=torch.float32, device=dev)
        wb = w.numel() * w.element_size()
        bb = 0 if b is None else 4 * D
        fwd_b = 4 * ne + wb + bb
        bwd_b = 6 * ne + 2 * wb + 2 * bb
        fwd_calls = [lambda i=i: cc.cconv_fwd(xa[i], w, b, y=ya[i]) for i in range(nsets)]
        bwd_calls = [lambda i=i: cc.cconv_bwd(xa[i], dya[i], w, b, dx=dxa[i], dw=dwo, dbias=dbo, workspace=ws)
                     for i in range(nsets)]

        def cp(kind, i, a, bsrc, dst):
            rc = R.cconv_roofline_copy(kind, a[i].data_ptr(), bsrc[i].data_ptr(), dst[i].data_ptr(), 2 * ne, 1, 256, 1,
                                       cur().cuda_stream)
            assert rc == 0

        c1_calls = [lambda i=i: cp(1, i, xa, xa, ya) for i in range(nsets)]
        c2_calls = [lambda i=i: cp(2, i, xa, dya, dxa) for i in range(nsets)]
        tf = graph_time(torch, fwd_calls)
        tb = graph_time(torch, bwd_calls)
        t1 = graph_time(torch, c1_calls)
        t2 = graph_time(torch, c2_calls)
        g1, g2 = 4 * ne / t1[1] / 1e9, 6 * ne / t2[1] / 1e9

        def row(nb, q, copy_same, copy_big):
            gb = nb / q[1] / 1e9
            return {"us": round(q[1] * 1e6, 2), "us_p10_p90": [round(q[0] * 1e6, 2), round(q[2] * 1e6, 2)], "bytes": nb,
                    "GBps": round(gb, 1), "pct_flat_copy_same_size": round(100 * gb / copy_same, 1),
                    "pct_flat_copy_large": round(100 * gb / copy_big, 1), "pct_hbm_peak": round(100 * gb / peak, 1)}

        rec = {"workload": f"x bf16 [{B},{T},{D}], w bf16 [{D},{W}], " + ("bias fp32" if b is not None else "no bias"),
               "sets_rotated": nsets, "bytes_rotated": nsets * 8 * ne, "cache_resident": False,
               "timing": "graph of back-to-back calls over the rotated sets",
               "flat_copy_same_size_GBps": {"1r1w": round(g1, 1), "2r1w": round(g2, 1)},
               "fwd": row(fwd_b, tf, g1, copy_rates[0]), "bwd": row(bwd_b, tb, g2, copy_rates[1])}
        if with_oracle:
            import oracle

            cc.cconv_fwd(xa[0], w, b, y=ya[0])
            cc.cconv_bwd(xa[0], dya[0], w, b, dx=dxa[0], dw=dwo, dbias=dbo, workspace=ws)
            torch.cuda.synchronize()
            y0, dx0, dw0, db0 = ya[0].cpu(), dxa[0].cpu(), dwo.cpu(), dbo.cpu()
            _, yr = oracle.fwd(inp["x"], inp["w"], inp["bias"])
            dxr, dwr, dbr = oracle.bwd(inp["x"], inp["dy"], inp["w"], inp["bias"])

            def err(g, r):
                g = g.double().numpy()
                return float(np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r)))) if g.size else 0.0

            uy, ny = ulp_and_rms(oracle, np, y0, yr)
            udx, ndx = ulp_and_rms(oracle, np, dx0, dxr)
            udw, ndw = ulp_and_rms(oracle, np, dw0, dwr, sum_of_terms=True)
            par = {"y": err(y0.float(), yr), "dx": err(dx0.float(), dxr), "dw": err(dw0.float(), dwr),
                   "dbias": err(db0, dbr), "max_ulps": {"y": uy, "dx": udx, "dw": udw},
                   "nrms": {"y": ny, "dx": ndx, "dw": ndw,
                            "dbias": float(np.linalg.norm(db0.double().numpy() - dbr) / max(np.linalg.norm(dbr), 1e-30))}}
            par["pass"] = (par["y"] <= 5e-3 and par["dx"] <= 8e-3 and par["dw"] <= 8e-3 and par["dbias"] <= 8e-3
                           and uy <= 1 and udx <= 1)
            rec["parity"] = par
            threads = oracle.threads("f32")
            xf, dyf = inp["x"].float().numpy(), inp["dy"].float().numpy()
            ta = time.perf_counter()
            reps = 0
            while True:  # repeat small workloads until about a second of CPU time
                oracle.fwd(xf, inp["w"], inp["bias"], precision="f32")
                oracle.bwd(xf, dyf, inp["w"], inp["bias"], precision="f32")
                reps += 1
                if time.perf_counter() - ta > 1.0:
                    break
            tc = (time.perf_counter() - ta) / reps
            cpu[shp.name] = {"value": round((fwd_b + bwd_b) / tc / 1e9, 4), "unit": "GB/s", "cores": threads,
                             "kind": "oracle", "sample": f"fwd+bwd on the whole workload (fp32 oracle build), {reps} runs"}
        out[shp.name] = rec
        del xa, dya, ya, dxa, ws
        torch.cuda.empty_cache()
    return out, cpu


def profile_shapes(cc, si, torch, dev, steps):
    """Forward and backward at [8, 8192, D] for the widths that leave the 8-channel path
    (4-channel lanes on rows that miss the 128-byte lines at 4098, 4100 and 4104; contiguous
    6144), `steps` calls each, then one 1R:1W and one 2R:1W flat copy of the
    D = 4096 activation size for counter calibration."""
    R = cc.roofline_lib()
    out = {}
    for D in (4098, 4100, 4104, 6144):
        inp = si.train_inputs(8, 8192, D, 4, bias=True, seed=30 + D % 97)
        x, w, b, dy = (inp[k].to(dev) for k in ("x", "w", "bias", "dy"))
        y, dx = torch.empty_like(x), torch.empty_like(x)
        dw, db = torch.empty_like(w), torch.empty(D, dtype=torch.float32, device=dev)
        ws = torch.empty(cc.cconv_bwd_workspace_bytes(8, 8192, D, 4) // 4 + 1, dtype=torch.float32, device=dev)
        for _ in range(steps):
            cc.cconv_fwd(x, w, b, y=y)
            cc.cconv_bwd(x, dy, w, b, dx=dx, dw=dw, dbias=db, workspace=ws)
        torch.cuda.synchronize()
        out[D] = {"fwd": cc.cconv_default_config("fwd", 8, 8192, D, 4).as_dict(),
                  "bwd": cc.cconv_default_config("bwd", 8, 8192, D, 4).as_dict()}
        del x, dy, y, dx, ws
        torch.cuda.empty_cache()
    nbytes = 8 * 8192 * 4096 * 2
    a, bb, c = (torch.empty(nbytes // 2, dtype=torch.int16, device=dev) for _ in range(3))
    st = torch.cuda.current_stream().cuda_stream
    assert R.cconv_roofline_copy(1, a.data_ptr(), a.data_ptr(), c.data_ptr(), nbytes, 1, 256, 1, st) == 0
    assert R.cconv_roofline_copy(2, a.data_ptr(), bb.data_ptr(), c.data_ptr(), nbytes, 1, 256, 1, st) == 0
    torch.cuda.synchronize()
    return {"profile_shapes": True, "steps": steps, "copy_bytes_per_operand": nbytes, "launch": out}


def decode_graph(cc, torch, dev, dhost, nbytes, peak, nsets=24, reps=30):
    """The decode update timed as 24 back-to-back calls in one graph: each call on its own
    buffer set (x, state, y; 400 MB in all, more than the Infinity Cache holds, so each finds
    its rows in HBM), and again with every call on set 0 (cache-resident)."""
    N, D = dhost["x"].shape
    xs = [dhost["x"].to(dev) for _ in range(nsets)]
    sts = [dhost["state"].to(dev) for _ in range(nsets)]
    ys = [torch.empty(N, D, dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    idx, w, b = dhost["state_indices"].to(dev), dhost["w"].to(dev), dhost["bias"].to(dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    out = {"calls_per_graph": nsets, "launch": cc.cconv_default_update_config(N, D).as_dict()}
    for label, sets in (("hbm", list(range(nsets))), ("cache_resident", [0] * nsets)):
        q = graph_time(torch, [lambda i=i: cc.cconv_update(xs[i], sts[i], idx, w, b, y=ys[i], status=st) for i in sets],
                       reps=reps)
        gb = nbytes / q[1] / 1e9
        out[label] = {"us": round(q[1] * 1e6, 2), "us_p10_p90": [round(q[0] * 1e6, 2), round(q[2] * 1e6, 2)],
                      "GBps": round(gb, 1), "pct_hbm_peak": round(100 * gb / peak, 1)}
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    del xs, sts, ys
    return out


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
            "the library has no multi-GPU path to time.",
            file=sys.stderr,
        )
        sys.exit(2)

    import numpy as np
    import torch

    import causal_depthwise_short_amd as cc
    import synth_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cur = torch.cuda.current_stream
    if args.profile_shapes:
        print(json.dumps(profile_shapes(cc, si, torch, dev, args.steps)))
        return

    s = si.HEADLINE
    dshape = si.DECODE
    B, T, D, W = s.B, s.T, s.D, s.W
    n = B * T * D
    log(f"inputs: {s.name} + {dshape.name}")
    host = si.train_inputs_for(s)
    x, w, b, dy = (host[k].to(dev) for k in ("x", "w", "bias", "dy"))
    dhost = si.decode_inputs_for(dshape)
    dx_in = dhost["x"].to(dev)
    state = dhost["state"].to(dev)
    sidx = dhost["state_indices"].to(dev)
    dw_ = dhost["w"].to(dev)
    db_ = dhost["bias"].to(dev)
    y = torch.empty_like(x)
    dxo = torch.empty_like(x)
    dwo = torch.empty_like(w)
    dbo = torch.empty(D, dtype=torch.float32, device=dev)
    ws = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, D, W) // 4 + 1, dtype=torch.float32, device=dev)
    yd = torch.empty(dshape.N, dshape.D, dtype=torch.bfloat16, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)

    bytes_fwd = 4 * n + w.numel() * w.element_size() + D * 4
    bytes_bwd_main = 6 * n + w.numel() * w.element_size() + D * 4
    bytes_bwd_finish = dwo.numel() * dwo.element_size() + D * 4
    bytes_bwd = bytes_bwd_main + bytes_bwd_finish
    L = dshape.W - 1
    bytes_upd = (
        2 * dshape.N * dshape.D  # x
        + 2 * 2 * dshape.N * dshape.D * L  # state rows read and written
        + 2 * dshape.N * dshape.D  # y
        + dw_.numel() * dw_.element_size() + dshape.D * 4 + dshape.N * 4
    )
    bytes_step = bytes_fwd + bytes_bwd + bytes_upd

    # launches of the backward main kernel at this shape, counted so that a kernel trace of this
    # run can be cut at the first variant (variants launch the same kernel at other shapes)
    n_main = [0]

    def bwd_main():
        n_main[0] += 1
        cc.cconv_bwd_main(x, dy, w, b, dxo, ws)

    def step(ev=None):
        """One step. ev: None, two events (around the backward main kernel only: the timed
        region's instrumentation) or five (every phase: the breakdown pass)."""
        full = ev is not None and len(ev) == 5
        if full:
            ev[0].record()
        cc.cconv_fwd(x, w, b, y=y)
        if ev is not None:
            ev[1 if full else 0].record()
        bwd_main()
        if ev is not None:
            ev[2 if full else 1].record()
        cc.cconv_bwd_finish(ws, dwo, dbo, B, T, D, W)
        if full:
            ev[3].record()
        cc.cconv_update(dx_in, state, sidx, dw_, db_, y=yd, status=status)
        if full:
            ev[4].record()

    # ---- outputs for the parity gate (before any timing) --------------------------------
    state0 = state.clone()
    step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "decode update rejected valid indices"
    gate_inputs = None
    if not args.no_cpu_baseline and not args.profile:
        gate_inputs = {
            "y": y.cpu(), "dx": dxo.cpu(), "dw": dwo.float().cpu(), "dw_bf16": dwo.cpu(), "db": dbo.cpu(),
            "yd": yd.cpu(), "state": state.cpu(), "state0": state0.cpu(),
        }
    state.copy_(state0)

    # ---- flat-copy roofline: same byte volume, same read:write mixes --------------------
    R = cc.roofline_lib()
    nbytes = x.numel() * x.element_size()

    def copy(kind, unroll, threads, nt):
        rc = R.cconv_roofline_copy(kind, x.data_ptr(), dy.data_ptr(), y.data_ptr(), nbytes, unroll, threads, nt,
                                   cur().cuda_stream)
        assert rc == 0

    def quant(v):
        v = sorted(v)
        return v[len(v) // 10], v[len(v) // 2], v[min(len(v) - 1, (9 * len(v)) // 10)]

    def time_fn(fn, reps=20, warm=3):
        for _ in range(warm):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)
        return ts[len(ts) // 2]

    def copy_p(kind, blocks, unroll, threads, nt):
        rc = R.cconv_roofline_copy_persistent(kind, x.data_ptr(), dy.data_ptr(), y.data_ptr(), nbytes, blocks, unroll,
                                              threads, nt, cur().cuda_stream)
        assert rc == 0

    def dtod():
        # a contiguous same-dtype device copy is one hipMemcpyAsync(..., device-to-device)
        y.view(-1).copy_(x.view(-1))

    # one-shot grids (one block per chunk of threads x unroll vectors) and persistent
    # grid-stride grids (a fixed number of blocks, unroll loads in flight per thread)
    copy_cfgs = [("oneshot", (u, th, nt)) for u in (1, 2, 4) for th in (256, 512) for nt in (0, 1)]
    copy_cfgs += [("persistent", (blk, u, 256, nt)) for blk in (1024, 2048, 4096) for u in (4, 8) for nt in (0, 1)]
    if args.profile:
        copy_cfgs = [("oneshot", (1, 256, 1))]

    def copy_any(kind, fam, cfg):
        if fam == "oneshot":
            copy(kind, *cfg)
        else:
            copy_p(kind, *cfg)

    def copy_label(fam, cfg):
        if fam == "oneshot":
            return f"one-shot u={cfg[0]} threads={cfg[1]} nt={cfg[2]}"
        return f"persistent blocks={cfg[0]} u={cfg[1]} threads={cfg[2]} nt={cfg[3]}"

    def copy_roofline():
        best, table = {}, {}
        for kind in (1, 2):
            res = []
            for fam, cfg in copy_cfgs:
                t = time_fn(lambda: copy_any(kind, fam, cfg), reps=10 if not args.profile else 3, warm=2)
                res.append(((kind + 1) * nbytes / t / 1e9, copy_label(fam, cfg), (fam, cfg)))
            best[kind] = max(res)
            table[kind] = {r[1]: round(r[0], 1) for r in res}
        t = time_fn(dtod, reps=10 if not args.profile else 3, warm=2)
        best["dtod"] = 2 * nbytes / t / 1e9
        return best, table

    log("flat copy roofline (before)")
    cp_a, cp_table_a = copy_roofline()

    # ---- timed region ----------------------------------------------------------------------
    K, Wm = args.steps, args.warmup
    log(f"timing {K} steps after {Wm} warm-up steps")
    for _ in range(Wm):
        step()
    # the timed region carries only the two events the roofline needs (around the backward main
    # kernel); the per-phase breakdown comes from a second pass of K steps with five events each
    main_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(main_ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    q_main = quant([e[0].elapsed_time(e[1]) * 1e-3 for e in main_ev])

    log(f"per-phase breakdown: {K} more steps with events around every phase")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(events[i])
    torch.cuda.synchronize()

    def med(i, j):
        return quant([events[k][i].elapsed_time(events[k][j]) * 1e-3 for k in range(K)])

    q_fwd, q_fin, q_upd, q_bwd = med(0, 1), med(2, 3), med(3, 4), med(1, 3)
    t_fwd, t_main, t_fin, t_upd, t_bwd = q_fwd[1], q_main[1], q_fin[1], q_upd[1], q_bwd[1]

    log("flat copy roofline (after)")
    cp_b, cp_table_b = copy_roofline()
    copy1 = max(cp_a[1], cp_b[1])
    copy2 = max(cp_a[2], cp_b[2])
    dtod_gbps = max(cp_a["dtod"], cp_b["dtod"])
    # the 1R:1W denominator is the best of the copy kernels and hipMemcpyAsync device-to-device
    if dtod_gbps > copy1[0]:
        copy1 = (dtod_gbps, "hipMemcpyAsync device-to-device", ("dtod", None))

    if args.profile:
        # the decode update from HBM and cache-resident (graph replays), then calibration
        # dispatches of known size for the HBM counters: one 1R:1W copy and one 2R:1W copy of
        # `nbytes` per source
        dgraph = decode_graph(cc, torch, dev, dhost, bytes_upd, HBM_PEAK_GBPS, reps=5)
        copy(1, 1, 256, 1)
        copy(2, 1, 256, 1)
        torch.cuda.synchronize()
        log(f"profile run done: {K} steps; calibration copies of {nbytes} bytes per operand")
        print(json.dumps({"profile_run": True, "steps": K, "copy_bytes_per_operand": nbytes, "decode_graph": dgraph,
                          "kernel_source_sha256_16": kernel_source_hash(),
                          "launch_bwd": cc.cconv_default_config("bwd", B, T, D, W).as_dict()}))
        return

    def phase(nb, q, copy_gbps):
        t = q[1]
        gbps = nb / t / 1e9
        return {
            "us": round(t * 1e6, 2),
            "us_p10_p90": [round(q[0] * 1e6, 2), round(q[2] * 1e6, 2)],
            "bytes": nb,
            "GBps": round(gbps, 1),
            "pct_flat_copy": round(100 * gbps / copy_gbps, 1) if copy_gbps else None,
            "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        }

    breakdown = {
        "fwd": phase(bytes_fwd, q_fwd, copy1[0]),
        "bwd": phase(bytes_bwd, q_bwd, copy2[0]),
        "bwd_main": phase(bytes_bwd_main, q_main, copy2[0]),
        "bwd_finish": {"us": round(t_fin * 1e6, 2), "bytes": bytes_bwd_finish},
        "update": dict(phase(bytes_upd, q_upd, copy1[0]), cache_resident=True),
    }

    # ---- AB/BA interleaving with the flat copy: kernels and copies alternate in order, so
    # the percentages also hold under the same clocks and memory state (outside `value`) ----
    def interleaved(pairs=21):
        mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        kt, ct = [], []
        for i in range(pairs):
            for part in ((0, 1) if i % 2 == 0 else (1, 0)):
                ev = [mk(), mk(), mk()]
                if part == 0:
                    ev[0].record()
                    cc.cconv_fwd(x, w, b, y=y)
                    ev[1].record()
                    bwd_main()
                    ev[2].record()
                    cc.cconv_bwd_finish(ws, dwo, dbo, B, T, D, W)
                    kt.append(ev)
                else:
                    ev[0].record()
                    if copy1[2][0] == "dtod":
                        dtod()
                    else:
                        copy_any(1, *copy1[2])
                    ev[1].record()
                    copy_any(2, *copy2[2])
                    ev[2].record()
                    ct.append(ev)
        torch.cuda.synchronize()
        f = quant([e[0].elapsed_time(e[1]) * 1e-3 for e in kt])[1]
        m = quant([e[1].elapsed_time(e[2]) * 1e-3 for e in kt])[1]
        c1 = 2 * nbytes / quant([e[0].elapsed_time(e[1]) * 1e-3 for e in ct])[1] / 1e9
        c2 = 3 * nbytes / quant([e[1].elapsed_time(e[2]) * 1e-3 for e in ct])[1] / 1e9
        return {
            "pairs": pairs,
            "fwd_us": round(f * 1e6, 2),
            "bwd_main_us": round(m * 1e6, 2),
            "copy_1r1w_GBps": round(c1, 1),
            "copy_2r1w_GBps": round(c2, 1),
            "pct_flat_copy": {"fwd": round(100 * bytes_fwd / f / 1e9 / c1, 1),
                              "bwd_main": round(100 * bytes_bwd_main / m / 1e9 / c2, 1)},
        }

    log("AB/BA interleaved kernels and flat copies")
    inter = interleaved()

    # ---- the widened rows, each timed alone at its own workload (outside `value`) ---------
    log("variants: state handoff, pool prefill, packed batch, epilogues, any D, decode variants")
    main_launches = n_main[0]
    variants, vsample = run_variants(cc, si, torch, dev, host, dhost, s, dshape, x, dy, w, b, y, dxo, dwo, dbo, ws,
                                     quant, copy1[0], copy2[0], HBM_PEAK_GBPS)

    # ---- the decode update by graph replay (launch gaps out of the number), from HBM and
    # cache-resident ---------------------------------------------------------------------------
    log("decode update: graph replays of 24 back-to-back calls")
    dgraph = decode_graph(cc, torch, dev, dhost, bytes_upd, HBM_PEAK_GBPS)

    # ---- the other training workloads, each with its oracle timed and checked ---------------
    log("other workloads: B1/T256/D512, B8/T1024/D4096 (no bias), B3/T1000/D2000/W2")
    configs, cfg_cpu = time_configs(cc, si, torch, np, dev, (copy1[0], copy2[0]), HBM_PEAK_GBPS,
                                    with_oracle=not args.no_cpu_baseline)

    # ---- host enqueue cost of one eager decode update through the Python binding: wall time
    # per call over back-to-back calls (each runs ~6 us on the GPU, so the host sets the pace)
    def host_enqueue(fn, n=400):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            ts.append((time.perf_counter() - t0) / n)
            torch.cuda.synchronize()
        return sorted(ts)[len(ts) // 2]

    enqueue_us = round(1e6 * host_enqueue(
        lambda: cc.cconv_update(dx_in, state, sidx, dw_, db_, y=yd, status=status)), 2)

    # ---- CPU baseline: the oracle, timed on a bounded sample of the same workload ---------
    cpu = None
    gate = None
    if not args.no_cpu_baseline:
        import oracle  # test infrastructure, used only in this leg

        xf = host["x"].float().numpy()
        dyf = host["dy"].float().numpy()
        threads = oracle.threads("f32")

        def oracle_rows(nb):
            ta = time.perf_counter()
            _, yr = oracle.fwd(xf[:nb], host["w"], host["bias"], precision="f32")
            dxr, dwr, dbr = oracle.bwd(xf[:nb], dyf[:nb], host["w"], host["bias"], precision="f32")
            return time.perf_counter() - ta, yr, dxr, dwr, dbr

        log("cpu baseline: calibrating the oracle on one batch row")
        t_one, *_ = oracle_rows(1)
        rows = int(max(1, min(B, args.cpu_seconds // max(t_one, 1e-3))))
        log(f"cpu baseline: oracle on {rows} of {B} batch rows ({threads} threads)")
        t_cpu, yr, dxr, dwr, dbr = oracle_rows(rows)
        # one-thread figure on a smaller sample: the first rows of batch row 0
        rows1 = 2048
        oracle.set_threads(1, "f32")
        t1a = time.perf_counter()
        oracle.fwd(xf[:1, :rows1], host["w"], host["bias"], precision="f32")
        oracle.bwd(xf[:1, :rows1], dyf[:1, :rows1], host["w"], host["bias"], precision="f32")
        t_cpu1 = time.perf_counter() - t1a
        oracle.set_threads(threads, "f32")
        tu = time.perf_counter()
        ok, ydr, sr = oracle.update(dhost["x"], dhost["state"], dhost["state_indices"], dhost["w"], dhost["bias"],
                                    precision="f32")
        t_cpu_upd = time.perf_counter() - tu
        sample_bytes = rows * T * D * 10 + 2 * (w.numel() * w.element_size() + D * 4) + bytes_bwd_finish + bytes_upd
        cpu = {
            "value": round(sample_bytes / (t_cpu + t_cpu_upd) / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": (
                f"fwd+bwd on batch rows 0..{rows - 1} of the {B}x{T}x{D} W={W} workload (fp32 oracle build) "
                f"+ one decode update N={dshape.N} S={dshape.S}; {t_cpu + t_cpu_upd:.1f} s"
            ),
            "host": platform.processor() or platform.machine(),
            "value_1thread": round((rows1 * D * 10 + 2 * (w.numel() * w.element_size() + D * 4)) / t_cpu1 / 1e9, 4),
            "sample_1thread": f"fwd+bwd on rows 0..{rows1 - 1} of batch row 0, one thread; {t_cpu1:.1f} s",
        }

        # parity gate: the GPU outputs of the timed configuration against the oracle
        def err(g, r):
            g = g.double().numpy() if hasattr(g, "numpy") else np.asarray(g, np.float64)
            return float(np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r))))

        gi = gate_inputs
        e_y = err(gi["y"][:rows].float(), yr)
        e_dx = err(gi["dx"][:rows].float(), dxr)  # every row, the last W-1 (the halo past T) included
        e_dw = err(gi["dw"], dwr) if rows == B else None
        e_db = err(gi["db"], dbr) if rows == B else None
        e_yd = err(gi["yd"].float(), ydr)
        u_y, n_y = ulp_and_rms(oracle, np, gi["y"][:rows], yr)
        u_dx, n_dx = ulp_and_rms(oracle, np, gi["dx"][:rows], dxr)
        u_yd, n_yd = ulp_and_rms(oracle, np, gi["yd"], ydr)
        u_dw, n_dw = ulp_and_rms(oracle, np, gi["dw_bf16"], dwr, sum_of_terms=True) if rows == B else (None, None)
        n_db = float(np.linalg.norm(gi["db"].double().numpy() - dbr) / max(np.linalg.norm(dbr), 1e-30)) if rows == B else None
        state_exact = bool(
            ok and torch.equal(gi["state"].view(torch.int16), torch.from_numpy(sr).to(torch.bfloat16).view(torch.int16))
        )
        passed = (
            e_y <= 5e-3 and e_dx <= 8e-3 and e_yd <= 5e-3 and state_exact
            and (e_dw is None or e_dw <= 8e-3) and (e_db is None or e_db <= 8e-3)
            and u_y <= 1 and u_dx <= 1 and u_yd <= 1 and (u_dw is None or u_dw <= 1)
        )
        gate = {
            "pass": passed, "rows": rows, "y": e_y, "dx": e_dx, "dw": e_dw, "dbias": e_db, "decode_y": e_yd,
            "decode_state_bit_exact": state_exact,
            "max_ulps": {"y": u_y, "dx": u_dx, "decode_y": u_yd, "dw": u_dw},
            "nrms": {"y": n_y, "dx": n_dx, "decode_y": n_yd, "dw": n_dw, "dbias": n_db},
            "metric": ("max |gpu-oracle|/max(1,|oracle|); bounds 5e-3 (y), 8e-3 (dx, dw, dbias); max_ulps: bf16 ulps "
                       "from the oracle's value rounded to bf16 (elements within 2^-18 of it, 1e-5 of max |dw| for dw, count 0), "
                       "bound 1; "
                       "nrms: ||gpu-oracle||/||oracle|| (reported); oracle: the fp32 build on the timed rows"),
        }
        log("cpu baseline: the variants' samples")
        vcpu, vgate = oracle_variants(oracle, np, torch, vsample, err)
        cpu["variants"] = vcpu
        cpu["configs"] = cfg_cpu
        gate["variants"] = vgate
        gate["configs"] = {k: v["parity"] for k, v in configs.items()}
        for k, v in vgate.items():
            variants[k]["parity"] = v["pass"]
        passed = passed and all(v["pass"] for v in vgate.values()) and all(v["pass"] for v in gate["configs"].values())
        gate["pass"] = passed
        if not passed:
            print(json.dumps({"parity_gate": gate}), file=sys.stderr)
            raise SystemExit("parity gate failed: no throughput is reported")

    value = K * bytes_step / elapsed / 1e9
    traffic = read_traffic()
    achieved = bytes_bwd_main / t_main / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (
                f"fwd+bwd x bf16 [{B},{T},{D}], w bf16 [{D},{W}], bias fp32 [{D}], dy bf16; "
                f"then one decode update x [{dshape.N},{dshape.D}], state bf16 [{dshape.S},{dshape.D},{L}], "
                f"{dshape.N} distinct slots"
            ),
            "B": B, "T": T, "D": D, "W": W, "io_dtype": "bf16",
            "launch_fwd": cc.cconv_default_config("fwd", B, T, D, W).as_dict(),
            "launch_bwd": cc.cconv_default_config("bwd", B, T, D, W).as_dict(),
            "bytes_per_step": bytes_step,
        },
        # the metric's two figures, each on its own: forward and backward (main + finish) GB/s,
        # % of the flat copy with the same read:write mix, % of the 8 TB/s peak
        "fwd": {k: breakdown["fwd"][k] for k in ("GBps", "pct_flat_copy", "pct_hbm_peak", "us")},
        "bwd": {k: breakdown["bwd"][k] for k in ("GBps", "pct_flat_copy", "pct_hbm_peak", "us")},
        "pct_flat_copy": {"fwd": breakdown["fwd"]["pct_flat_copy"], "bwd": breakdown["bwd"]["pct_flat_copy"]},
        "breakdown": breakdown,
        "flat_copy": {
            "1r1w_GBps": round(copy1[0], 1), "1r1w_kernel": copy1[1],
            "2r1w_GBps": round(copy2[0], 1), "2r1w_kernel": copy2[1],
            "dtod_GBps": round(dtod_gbps, 1),
            "bytes_per_operand": nbytes,
            "sweep_1r1w_GBps": {k: max(v, cp_table_b[1][k]) for k, v in cp_table_a[1].items()},
            "sweep_2r1w_GBps": {k: max(v, cp_table_b[2][k]) for k, v in cp_table_a[2].items()},
        },
        "interleaved": inter,
        "decode_graph": dgraph,
        "configs": configs,
        "update_host_enqueue_us": enqueue_us,
        "variants": variants,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "cconv_bwd_kernel (backward main: dx and dw/dbias partials)",
            "bytes_per_launch": bytes_bwd_main,
            "us_per_launch": round(t_main * 1e6, 2),
            # the first this many launches of the kernel in a trace of this run are at this
            # shape (the variants that follow launch it at others)
            "launches_at_shape": main_launches,
        },
        "cpu_baseline": cpu,
        "parity_gate": gate,
        "env": {
            "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None),
            "device": torch.cuda.get_device_name(0),
            "library": cc.cconv_version(),
            "kernel_source_sha256_16": kernel_source_hash(),
        },
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
