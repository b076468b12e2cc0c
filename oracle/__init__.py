"""CPU oracle for the depthwise causal short convolution + SiLU (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import this
package. It wraps ``cconv_oracle.c`` (plain C loops, built with gcc twice: fp64 and fp32)
through ctypes. It shares no code with the HIP library and never imports it.

Every function takes host tensors (torch or numpy) whose values are exactly representable
in fp32 (bf16 activations/state, bf16 or fp32 taps, fp32 bias), widens them to fp32 arrays
without rounding, and returns unrounded results as numpy arrays of the oracle's precision
(float64 for ``precision="f64"``, float32 for ``"f32"``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "cconv_oracle.c"
_LIBS = {"f64": _DIR / "liboracle_f64.so", "f32": _DIR / "liboracle_f32.so"}
_REAL = {"f64": "double", "f32": "float"}
_NP = {"f64": np.float64, "f32": np.float32}
_handles: dict = {}


def _compile(src: Path, prec: str, out: Path) -> None:
    tmp = out.with_suffix(".so.tmp")
    cmd = [
        "gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
        f"-DORACLE_REAL={_REAL[prec]}", str(src), "-o", str(tmp), "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = False) -> None:
    """Compile both precisions with gcc (-O2, OpenMP, no FMA contraction, no fast-math)."""
    for prec, lib in _LIBS.items():
        if lib.exists() and not force and lib.stat().st_mtime >= _SRC.stat().st_mtime:
            continue
        _compile(_SRC, prec, lib)


def _load(path: Path, prec: str):
    lib = ctypes.CDLL(str(path))
    f = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_fwd.argtypes = [f, i64, i64, i64, f, ctypes.c_int, f, f, f]
    lib.oracle_bwd.argtypes = [f, f, i64, i64, i64, f, ctypes.c_int, f, f, f, f]
    lib.oracle_fwd_points.argtypes = [f, i64, i64, i64, f, ctypes.c_int, f, i64, f, f, f, f]
    lib.oracle_dx_points.argtypes = [f, f, i64, i64, i64, f, ctypes.c_int, f, i64, f, f, f, f]
    lib.oracle_dw_channels.argtypes = [f, f, i64, i64, i64, f, ctypes.c_int, f, i64, f, f, f]
    lib.oracle_fwd_state.argtypes = [f, f, i64, i64, i64, f, ctypes.c_int, f, f, f]
    lib.oracle_bwd_state.argtypes = [f, f, f, i64, i64, i64, f, ctypes.c_int, f, f, f, f, f]
    lib.oracle_fwd_epi.argtypes = [f, f, f, ctypes.c_int, i64, i64, i64, f, ctypes.c_int, f, f]
    lib.oracle_bwd_epi.argtypes = [f, f, f, ctypes.c_int, i64, i64, i64, f, ctypes.c_int, f, f, f, f, f]
    lib.oracle_fwd_varlen.argtypes = [f, f, i64, i64, i64, f, ctypes.c_int, f, f, f, f]
    lib.oracle_fwd_varlen.restype = ctypes.c_int
    lib.oracle_bwd_varlen.argtypes = [f, f, f, i64, i64, i64, f, ctypes.c_int, f, f, f, f, f, f]
    lib.oracle_bwd_varlen.restype = ctypes.c_int
    lib.oracle_fwd_pool.argtypes = [f, i64, i64, i64, f, ctypes.c_int, f, f, i64, f, f, f]
    lib.oracle_fwd_pool.restype = ctypes.c_int
    lib.oracle_update_ex.argtypes = [f, i64, i64, f, i64, ctypes.c_int, f, f, f, ctypes.c_int, f, f]
    lib.oracle_update_ex.restype = ctypes.c_int
    lib.oracle_update.argtypes = [f, i64, i64, f, i64, f, f, ctypes.c_int, f, f]
    lib.oracle_update.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [f, f, i64]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_real_bytes.restype = ctypes.c_int
    assert lib.oracle_real_bytes() == (8 if prec == "f64" else 4)
    return lib


def _f32(a) -> np.ndarray:
    """Host tensor -> contiguous float32 numpy array (exact for bf16 / fp32 values)."""
    if a is None:
        return None
    try:
        import torch

        if isinstance(a, torch.Tensor):
            a = a.detach().cpu()
            if a.dtype not in (torch.float32, torch.bfloat16, torch.float16):
                raise TypeError(f"oracle inputs must be bf16/fp16/fp32, got {a.dtype}")
            return np.ascontiguousarray(a.float().numpy())
    except ImportError:  # pragma: no cover
        pass
    arr = np.asarray(a)
    if arr.dtype != np.float32:
        f = arr.astype(np.float32)
        if not np.array_equal(f.astype(arr.dtype), arr):
            raise ValueError("oracle input not exactly representable in fp32")
        arr = f
    return np.ascontiguousarray(arr)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _idx(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


class Oracle:
    """The oracle's entry points over a pair of compiled libraries (fp64 and fp32).

    The module-level functions use the libraries built from ``cconv_oracle.c``; the tests
    also build deliberately broken copies of the source into an ``Oracle`` to check that the
    pins catch each planted mistake.
    """

    def __init__(self, paths: dict):
        self._paths = dict(paths)
        self._handles: dict = {}

    def lib(self, prec: str):
        if prec not in self._handles:
            if not self._paths[prec].exists():
                build()
            self._handles[prec] = _load(self._paths[prec], prec)
        return self._handles[prec]

    def threads(self, precision: str = "f32") -> int:
        """OpenMP threads the oracle runs on (OMP_NUM_THREADS, else all host cores)."""
        return self.lib(precision).oracle_threads()

    def set_threads(self, n: int, precision: str = "f32") -> None:
        """Thread count for later calls of the library of this precision (results do not depend on it)."""
        self.lib(precision).oracle_set_threads(int(n))

    def fwd(self, x, w, bias=None, *, precision: str = "f64"):
        """z and y = silu(z) for x [B, T, D], w [D, W], bias [D] or None. Unrounded."""
        xf, wf, bf = _f32(x), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        assert wf.shape == (D, W)
        z = np.empty((B, T, D), _NP[precision])
        y = np.empty((B, T, D), _NP[precision])
        self.lib(precision).oracle_fwd(_p(xf), B, T, D, _p(wf), W, _p(bf), _p(z), _p(y))
        return z, y

    def bwd(self, x, dy, w, bias=None, *, precision: str = "f64"):
        """dx [B, T, D], dw [D, W], dbias [D] for y = silu(conv(x)). Unrounded."""
        xf, dyf, wf, bf = _f32(x), _f32(dy), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        assert dyf.shape == xf.shape and wf.shape == (D, W)
        dx = np.empty((B, T, D), _NP[precision])
        dw = np.empty((D, W), _NP[precision])
        db = np.empty((D,), _NP[precision])
        self.lib(precision).oracle_bwd(
            _p(xf), _p(dyf), B, T, D, _p(wf), W, _p(bf), _p(dx), _p(dw), _p(db)
        )
        return dx, dw, db

    def fwd_points(self, x, w, bias, pb, pt, pd, *, precision: str = "f64"):
        """y at the listed (b, t, d) points of a full-size problem."""
        xf, wf, bf = _f32(x), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        pb, pt, pd = _idx(pb), _idx(pt), _idx(pd)
        out = np.empty(pb.shape[0], _NP[precision])
        self.lib(precision).oracle_fwd_points(
            _p(xf), B, T, D, _p(wf), W, _p(bf), pb.shape[0], _p(pb), _p(pt), _p(pd), _p(out)
        )
        return out

    def dx_points(self, x, dy, w, bias, pb, pu, pd, *, precision: str = "f64"):
        """dx at the listed (b, u, d) points of a full-size problem."""
        xf, dyf, wf, bf = _f32(x), _f32(dy), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        pb, pu, pd = _idx(pb), _idx(pu), _idx(pd)
        out = np.empty(pb.shape[0], _NP[precision])
        self.lib(precision).oracle_dx_points(
            _p(xf), _p(dyf), B, T, D, _p(wf), W, _p(bf), pb.shape[0], _p(pb), _p(pu), _p(pd), _p(out)
        )
        return out

    def dw_channels(self, x, dy, w, bias, pd, *, precision: str = "f64"):
        """dw[d, :] and dbias[d] (full sums over batch and time) for the listed channels."""
        xf, dyf, wf, bf = _f32(x), _f32(dy), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        pd = _idx(pd)
        dw = np.empty((pd.shape[0], W), _NP[precision])
        db = np.empty((pd.shape[0],), _NP[precision])
        self.lib(precision).oracle_dw_channels(
            _p(xf), _p(dyf), B, T, D, _p(wf), W, _p(bf), pd.shape[0], _p(pd), _p(dw), _p(db)
        )
        return dw, db

    def fwd_state(self, x, h0, w, bias=None, *, precision: str = "f64"):
        """y and the final state for x [B, T, D] after the history h0 [B, D, W-1] (None =
        zeros). Returns (y unrounded, hT float32 [B, D, W-1])."""
        xf, hf, wf, bf = _f32(x), _f32(h0), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        assert wf.shape == (D, W) and (hf is None or hf.shape == (B, D, W - 1))
        y = np.empty((B, T, D), _NP[precision])
        hT = np.empty((B, D, W - 1), np.float32)
        self.lib(precision).oracle_fwd_state(_p(xf), _p(hf), B, T, D, _p(wf), W, _p(bf), _p(y), _p(hT))
        return y, hT

    def bwd_state(self, x, h0, dy, w, bias=None, *, precision: str = "f64"):
        """(dx, dw, dbias, dh0) for the forward with history h0 (None = zeros)."""
        xf, hf, dyf, wf, bf = _f32(x), _f32(h0), _f32(dy), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        assert dyf.shape == xf.shape and wf.shape == (D, W) and (hf is None or hf.shape == (B, D, W - 1))
        dx = np.empty((B, T, D), _NP[precision])
        dw = np.empty((D, W), _NP[precision])
        db = np.empty((D,), _NP[precision])
        dh0 = np.empty((B, D, W - 1), _NP[precision])
        self.lib(precision).oracle_bwd_state(
            _p(xf), _p(hf), _p(dyf), B, T, D, _p(wf), W, _p(bf), _p(dx), _p(dw), _p(db), _p(dh0)
        )
        return dx, dw, db, dh0

    def fwd_epi(self, x, w, bias=None, *, h0=None, residual=None, act: bool = True, precision: str = "f64"):
        """y = act(z) + residual (act: SiLU or none), unrounded; x [B, T, D], h0 [B, D, W-1] or None,
        residual [B, T, D] or None."""
        xf, hf, rf, wf, bf = _f32(x), _f32(h0), _f32(residual), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        assert rf is None or rf.shape == xf.shape
        y = np.empty((B, T, D), _NP[precision])
        self.lib(precision).oracle_fwd_epi(_p(xf), _p(hf), _p(rf), int(act), B, T, D, _p(wf), W, _p(bf), _p(y))
        return y

    def bwd_epi(self, x, dy, w, bias=None, *, h0=None, act: bool = True, precision: str = "f64"):
        """(dx, dw, dbias, dh0) of y = act(z) (+ residual, whose gradient is dy itself)."""
        xf, hf, dyf, wf, bf = _f32(x), _f32(h0), _f32(dy), _f32(w), _f32(bias)
        B, T, D = xf.shape
        W = wf.shape[1]
        dx = np.empty((B, T, D), _NP[precision])
        dw = np.empty((D, W), _NP[precision])
        db = np.empty((D,), _NP[precision])
        dh0 = np.empty((B, D, W - 1), _NP[precision])
        self.lib(precision).oracle_bwd_epi(_p(xf), _p(hf), _p(dyf), int(act), B, T, D, _p(wf), W, _p(bf), _p(dx),
                                           _p(dw), _p(db), _p(dh0))
        return dx, dw, db, dh0

    def fwd_varlen(self, x, cu_seqlens, w, bias=None, h0=None, *, precision: str = "f64"):
        """Packed batch: x [total, D], cu_seqlens [n+1]; h0 [n, D, W-1] or None. Returns
        (ok, y unrounded [total, D] or None, hT float32 [n, D, W-1] or None)."""
        xf, wf, bf, hf = _f32(x), _f32(w), _f32(bias), _f32(h0)
        total, D = xf.shape
        W = wf.shape[1]
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        n = cu.shape[0] - 1
        assert n >= 0 and (hf is None or hf.shape == (n, D, W - 1))
        y = np.empty((total, D), _NP[precision])
        hT = np.empty((n, D, W - 1), np.float32)
        rc = self.lib(precision).oracle_fwd_varlen(_p(xf), _p(cu), n, total, D, _p(wf), W, _p(bf), _p(hf), _p(y), _p(hT))
        if rc != 0:
            assert rc == 1, rc
            return False, None, None
        return True, y, hT

    def bwd_varlen(self, x, dy, cu_seqlens, w, bias=None, h0=None, *, precision: str = "f64"):
        """Backward of the packed batch. Returns (ok, dx, dw, dbias, dh0) (None values when the
        offsets are rejected)."""
        xf, dyf, wf, bf, hf = _f32(x), _f32(dy), _f32(w), _f32(bias), _f32(h0)
        total, D = xf.shape
        W = wf.shape[1]
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        n = cu.shape[0] - 1
        assert dyf.shape == xf.shape and (hf is None or hf.shape == (n, D, W - 1))
        dx = np.empty((total, D), _NP[precision])
        dw = np.empty((D, W), _NP[precision])
        db = np.empty((D,), _NP[precision])
        dh0 = np.empty((n, D, W - 1), _NP[precision])
        rc = self.lib(precision).oracle_bwd_varlen(
            _p(xf), _p(dyf), _p(cu), n, total, D, _p(wf), W, _p(bf), _p(hf), _p(dx), _p(dw), _p(db), _p(dh0)
        )
        if rc != 0:
            assert rc == 1, rc
            return False, None, None, None, None
        return True, dx, dw, db, dh0

    def fwd_pool(self, x, state, state_indices, has_initial_state, w, bias=None, *, precision: str = "f64"):
        """Prefill x [B, T, D] into the decode pool state [S, D, W-1] (slot state_indices[b],
        -1 = none; history read only where has_initial_state[b], None = nowhere).

        Returns (ok, y unrounded or None, new_state float32). The input state is not modified.
        """
        xf, wf, bf = _f32(x), _f32(w), _f32(bias)
        st = _f32(state).copy()
        B, T, D = xf.shape
        W = wf.shape[1]
        S = st.shape[0]
        assert st.shape == (S, D, W - 1)
        idx = np.ascontiguousarray(np.asarray(state_indices, dtype=np.int32))
        assert idx.shape == (B,)
        hi = None
        if has_initial_state is not None:
            hi = np.ascontiguousarray(np.asarray(has_initial_state, dtype=np.uint8))
            assert hi.shape == (B,)
        y = np.empty((B, T, D), _NP[precision])
        rc = self.lib(precision).oracle_fwd_pool(
            _p(xf), B, T, D, _p(wf), W, _p(bf), _p(st), S, _p(idx), _p(hi), _p(y)
        )
        if rc != 0:
            assert rc == 1, rc
            return False, None, st
        return True, y, st

    def update(self, x, state, state_indices, w, bias=None, *, precision: str = "f64"):
        """One decode step. Returns (ok, y [N, D], new_state float32 [S, D, W-1]).

        On invalid indices ok is False, y is None and the returned state equals the input
        state. The input ``state`` is not modified (a copy is advanced).
        """
        xf, wf, bf = _f32(x), _f32(w), _f32(bias)
        st = _f32(state).copy()
        N, D = xf.shape
        W = wf.shape[1]
        S = st.shape[0]
        assert st.shape == (S, D, W - 1)
        idx = None
        if state_indices is not None:
            idx = np.ascontiguousarray(np.asarray(state_indices, dtype=np.int32))
            assert idx.shape == (N,)
        y = np.empty((N, D), _NP[precision])
        rc = self.lib(precision).oracle_update(
            _p(xf), N, D, _p(st), S, _p(idx), _p(wf), W, _p(bf), _p(y)
        )
        if rc != 0:
            return False, None, st
        return True, y, st

    def update_ex(self, x, state, state_indices, cache_seqlens, w, bias=None, *, precision: str = "f64"):
        """Decode step with a state of L entries (state [S, D, L], L = W-1 or W) and, when
        cache_seqlens is given, circular-buffer addressing. Returns (ok, y, new_state float32)."""
        xf, wf, bf = _f32(x), _f32(w), _f32(bias)
        st = _f32(state).copy()
        N, D = xf.shape
        W = wf.shape[1]
        S, L = st.shape[0], st.shape[2]
        assert st.shape == (S, D, L)
        idx = None if state_indices is None else np.ascontiguousarray(np.asarray(state_indices, dtype=np.int32))
        cs = None if cache_seqlens is None else np.ascontiguousarray(np.asarray(cache_seqlens, dtype=np.int32))
        y = np.empty((N, D), _NP[precision])
        rc = self.lib(precision).oracle_update_ex(
            _p(xf), N, D, _p(st), S, L, _p(idx), _p(cs), _p(wf), W, _p(bf), _p(y)
        )
        if rc != 0:
            return False, None, st
        return True, y, st

    def round_bf16(self, a, *, precision: str = "f64") -> np.ndarray:
        """Round-to-nearest-even to bf16; returns the uint16 bit patterns."""
        arr = np.ascontiguousarray(np.asarray(a, dtype=_NP[precision]))
        out = np.empty(arr.shape, np.uint16)
        self.lib(precision).oracle_round_bf16(_p(arr), _p(out), arr.size)
        return out


def build_variant(src_text: str, workdir: Path) -> Oracle:
    """Compile an edited copy of the oracle source (used to plant mistakes in tests)."""
    workdir = Path(workdir)
    workdir.mkdir(parents=True, exist_ok=True)
    src = workdir / "cconv_oracle_variant.c"
    src.write_text(src_text)
    paths = {}
    for prec in ("f64", "f32"):
        out = workdir / f"liboracle_variant_{prec}.so"
        _compile(src, prec, out)
        paths[prec] = out
    return Oracle(paths)


def source_text() -> str:
    return _SRC.read_text()


_default = Oracle(_LIBS)
threads = _default.threads
fwd = _default.fwd
bwd = _default.bwd
fwd_points = _default.fwd_points
dx_points = _default.dx_points
dw_channels = _default.dw_channels
update = _default.update
fwd_pool = _default.fwd_pool
update_ex = _default.update_ex
fwd_epi = _default.fwd_epi
set_threads = _default.set_threads
bwd_epi = _default.bwd_epi
fwd_varlen = _default.fwd_varlen
bwd_varlen = _default.bwd_varlen
fwd_state = _default.fwd_state
bwd_state = _default.bwd_state
round_bf16 = _default.round_bf16
