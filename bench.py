#!/usr/bin/env python
"""Benchmark of the causal depthwise short convolution + SiLU hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
    forward  y = silu(conv(x))            x bf16 [8, 8192, 4096], w bf16 [4096, 4], bias fp32
    backward dx, dw, dbias (main kernel + fixed-order dw/dbias reduction)
    decode   one-token update of a rolling state: x [256, 4096], state [512, 4096, 3]
The printed value is the algorithmic bytes of every timed step (what the method must move:
x + y + taps + bias forward; x + dy + dx + taps + dw + bias + dbias backward; x + state read
and write + y + taps + bias + indices decode) divided by the wall time of the timed region,
inputs already resident in HBM. HIP events on the launch stream give each kernel's duration
inside the same timed region; the backward's main kernel is the dominant one and is reported
against MI355X's 8 TB/s HBM peak ("roofline"), and every phase against a flat copy with the
same read:write mix measured in the same run. The CPU oracle is timed beside it on a bounded
sample of the same workload ("cpu_baseline"); that leg also serves as the parity gate.

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
                    help="profiling run: steps plus calibration copies only (no sweep, no oracle)")
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

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        cc.cconv_fwd(x, w, b, y=y)
        if ev is not None:
            ev[1].record()
        cc.cconv_bwd_main(x, dy, w, b, dxo, ws)
        if ev is not None:
            ev[2].record()
        cc.cconv_bwd_finish(ws, dwo, dbo, B, T, D, W)
        if ev is not None:
            ev[3].record()
        cc.cconv_update(dx_in, state, sidx, dw_, db_, y=yd, status=status)
        if ev is not None:
            ev[4].record()

    # ---- outputs for the parity gate (before any timing) --------------------------------
    state0 = state.clone()
    step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "decode update rejected valid indices"
    gate_inputs = None
    if not args.no_cpu_baseline and not args.profile:
        gate_inputs = {
            "y": y.cpu(), "dx": dxo.cpu(), "dw": dwo.float().cpu(), "db": dbo.cpu(),
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

    copy_cfgs = [(u, th, nt) for u in (1, 2, 4) for th in (256, 512) for nt in (0, 1)]
    if args.profile:
        copy_cfgs = [(1, 256, 1)]

    def copy_roofline():
        best = {}
        for kind in (1, 2):
            res = []
            for u, th, nt in copy_cfgs:
                t = time_fn(lambda: copy(kind, u, th, nt), reps=10 if not args.profile else 3, warm=2)
                res.append(((kind + 1) * nbytes / t / 1e9, f"u={u} threads={th} nt={nt}", (u, th, nt)))
            best[kind] = max(res)
        return best

    log("flat copy roofline (before)")
    cp_a = copy_roofline()

    # ---- timed region ----------------------------------------------------------------------
    K, Wm = args.steps, args.warmup
    log(f"timing {K} steps after {Wm} warm-up steps")
    for _ in range(Wm):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    def quant(v):
        v = sorted(v)
        return v[len(v) // 10], v[len(v) // 2], v[min(len(v) - 1, (9 * len(v)) // 10)]

    def med(i, j):
        return quant([events[k][i].elapsed_time(events[k][j]) * 1e-3 for k in range(K)])

    q_fwd, q_main, q_fin, q_upd, q_bwd = med(0, 1), med(1, 2), med(2, 3), med(3, 4), med(1, 3)
    t_fwd, t_main, t_fin, t_upd, t_bwd = q_fwd[1], q_main[1], q_fin[1], q_upd[1], q_bwd[1]

    log("flat copy roofline (after)")
    cp_b = copy_roofline()
    copy1 = max(cp_a[1], cp_b[1])
    copy2 = max(cp_a[2], cp_b[2])

    if args.profile:
        # calibration dispatches of known size for the HBM counters: one 1R:1W copy and one
        # 2R:1W copy of `nbytes` per source
        copy(1, 1, 256, 1)
        copy(2, 1, 256, 1)
        torch.cuda.synchronize()
        log(f"profile run done: {K} steps; calibration copies of {nbytes} bytes per operand")
        print(json.dumps({"profile_run": True, "steps": K, "copy_bytes_per_operand": nbytes,
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
                    cc.cconv_bwd_main(x, dy, w, b, dxo, ws)
                    ev[2].record()
                    cc.cconv_bwd_finish(ws, dwo, dbo, B, T, D, W)
                    kt.append(ev)
                else:
                    ev[0].record()
                    copy(1, *copy1[2])
                    ev[1].record()
                    copy(2, *copy2[2])
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
        e_dx = err(gi["dx"][:rows, : T - (W - 1)].float(), dxr[:, : T - (W - 1)])
        e_dw = err(gi["dw"], dwr) if rows == B else None
        e_db = err(gi["db"], dbr) if rows == B else None
        e_yd = err(gi["yd"].float(), ydr)
        state_exact = bool(
            ok and torch.equal(gi["state"].view(torch.int16), torch.from_numpy(sr).to(torch.bfloat16).view(torch.int16))
        )
        passed = (
            e_y <= 5e-3 and e_dx <= 8e-3 and e_yd <= 5e-3 and state_exact
            and (e_dw is None or e_dw <= 8e-3) and (e_db is None or e_db <= 8e-3)
        )
        gate = {
            "pass": passed, "rows": rows, "y": e_y, "dx": e_dx, "dw": e_dw, "dbias": e_db, "decode_y": e_yd,
            "decode_state_bit_exact": state_exact,
            "metric": "max |gpu-oracle|/max(1,|oracle|); bounds 5e-3 (y), 8e-3 (dx, dw, dbias)",
        }
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
        "dtype": "f32",
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
        "pct_flat_copy": {"fwd": breakdown["fwd"]["pct_flat_copy"], "bwd": breakdown["bwd"]["pct_flat_copy"]},
        "breakdown": breakdown,
        "flat_copy": {
            "1r1w_GBps": round(copy1[0], 1), "1r1w_kernel": copy1[1],
            "2r1w_GBps": round(copy2[0], 1), "2r1w_kernel": copy2[1],
            "bytes_per_operand": nbytes,
        },
        "interleaved": inter,
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
