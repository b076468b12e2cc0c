"""Graph capture from the first call: in a fresh process, before any eager call of the library
(so before any of its kernels has ever been launched there), the forward, the backward and the
decode update are captured into one HIP graph at shapes run nowhere else in the suite. Every
replay must equal the first bit for bit, and the eager calls made afterwards must equal the
replays bit for bit. The child process reports each check; the parent asserts on them.
"""

from __future__ import annotations

import subprocess
import sys
import textwrap
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu
ROOT = Path(__file__).resolve().parent.parent

_CHILD = textwrap.dedent(
    r"""
    import sys
    sys.path.insert(0, sys.argv[1])
    import torch
    import causal_depthwise_short_amd as cc
    import synth_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, D, W = 3, 1777, 1544, 3
    N, S = 77, 131
    tr = si.train_inputs(B, T, D, W, bias=True, seed=990)
    dc = si.decode_inputs(N, S, D, W, bias=True, seed=991)
    x, w, b, dy = (tr[k].to(dev) for k in ("x", "w", "bias", "dy"))
    xd, st0, idx, wd, bd = (dc[k].to(dev) for k in ("x", "state", "state_indices", "w", "bias"))
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dw, db = torch.empty_like(w), torch.empty(D, dtype=torch.float32, device=dev)
    ws = torch.empty(cc.cconv_bwd_workspace_bytes(B, T, D, W) // 4 + 1, dtype=torch.float32, device=dev)
    state = st0.clone()
    yd = torch.empty(N, D, dtype=torch.bfloat16, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):  # the library's first calls in this process
        cc.cconv_fwd(x, w, b, y=y, stream=s)
        cc.cconv_bwd(x, dy, w, b, dx=dx, dw=dw, dbias=db, workspace=ws, stream=s)
        cc.cconv_update(xd, state, idx, wd, bd, y=yd, status=status, stream=s)
    print("captured", flush=True)

    outs = (y, dx, dw, db, yd, state)
    first = None
    for rep in range(3):
        state.copy_(st0)
        for t in outs[:5]:
            t.view(torch.int16).fill_(0x7FA5) if t.dtype == torch.bfloat16 else t.fill_(float("nan"))
        status.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"replay {rep}: status {int(status.item())}"
        snap = [t.clone() for t in outs]
        if first is None:
            first = snap
        else:
            for a, c in zip(first, snap):
                assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                                   c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32)), f"replay {rep}"
        print(f"replay {rep} ok", flush=True)

    # eager calls after the replays, into fresh outputs
    state2 = st0.clone()
    y2 = cc.cconv_fwd(x, w, b)
    dx2, dw2, db2 = cc.cconv_bwd(x, dy, w, b)
    yd2, st2 = cc.cconv_update(xd, state2, idx, wd, bd)
    torch.cuda.synchronize()
    assert int(st2.item()) == 0
    for name, a, c in zip(("y", "dx", "dw", "dbias", "decode y", "state"), first, (y2, dx2, dw2, db2, yd2, state2)):
        av = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
        cv = c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32)
        assert torch.equal(av, cv), f"eager {name} differs from the replay"
    print("first-call capture ok", flush=True)
    """
)


def test_capture_on_first_call_in_a_fresh_process():
    r = subprocess.run([sys.executable, "-c", _CHILD, str(ROOT)], cwd=str(ROOT), capture_output=True, text=True,
                       timeout=600)
    print(r.stdout)
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "first-call capture ok" in r.stdout
