"""Python binding of libcconv.so: the depthwise causal short convolution + SiLU on MI355X.

Argument marshalling only. Every function here checks that its torch tensors are device
tensors of the dtype and layout the C ABI expects, allocates outputs with ``torch.empty``
where the caller passed none, and calls the function of the same name in ``include/cconv.h``
on the current torch stream. All arithmetic runs in the HIP kernels. There is no fallback:
if the library is missing and cannot be built, or a call returns an error status, a
``CconvError`` is raised.
"""

from __future__ import annotations

import ctypes
import threading
from pathlib import Path
from typing import Optional

import torch

__all__ = [
    "CconvError",
    "Config",
    "lib",
    "cconv_fwd",
    "cconv_bwd",
    "cconv_fwd_state",
    "cconv_bwd_state",
    "cconv_fwd_pool",
    "cconv_fwd_ex",
    "cconv_bwd_ex",
    "FwdOpts",
    "BwdOpts",
    "cconv_fwd_varlen",
    "cconv_bwd_varlen",
    "cconv_bwd_workspace_bytes",
    "cconv_bwd_noalloc",
    "cconv_bwd_noalloc_max_workspace",
    "cconv_bwd_main",
    "cconv_bwd_finish",
    "cconv_update",
    "cconv_update_ex",
    "cconv_update_config",
    "UpdateConfig",
    "cconv_default_update_config",
    "cconv_default_config",
    "cconv_status_string",
    "cconv_version",
    "STATUS",
]

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libcconv.so"
ROOFLINE_LIB_PATH = _PKG / "libcconv_roofline.so"

STATUS = {
    0: "CCONV_OK",
    1: "CCONV_ERR_NULL_POINTER",
    2: "CCONV_ERR_BAD_SHAPE",
    3: "CCONV_ERR_BAD_STRIDE",
    4: "CCONV_ERR_UNSUPPORTED_DTYPE",
    5: "CCONV_ERR_MISALIGNED",
    6: "CCONV_ERR_ALIASING",
    7: "CCONV_ERR_WORKSPACE",
    8: "CCONV_ERR_INDEX",
    9: "CCONV_ERR_LAUNCH",
    10: "CCONV_ERR_BAD_CONFIG",
}
BF16, F32 = 0, 1


class Config(ctypes.Structure):
    """cconv_config_t: vec, rows_per_group, waves_per_block, strips_per_block, options, seg_rows."""

    _fields_ = [
        ("vec", ctypes.c_int),
        ("rows_per_group", ctypes.c_int),
        ("waves_per_block", ctypes.c_int),
        ("strips_per_block", ctypes.c_int),
        ("options", ctypes.c_int),
        ("seg_rows", ctypes.c_int64),
    ]

    def __init__(self, *args, **kw):
        kw.setdefault("strips_per_block", 1)
        super().__init__(*args, **kw)

    def __repr__(self):
        return "Config(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class UpdateConfig(ctypes.Structure):
    """cconv_update_config_t: vec, block_threads, rows_per_thread, options, rows_per_block."""

    _fields_ = [
        ("vec", ctypes.c_int),
        ("block_threads", ctypes.c_int),
        ("rows_per_thread", ctypes.c_int),
        ("options", ctypes.c_int),
        ("rows_per_block", ctypes.c_int64),
    ]

    def __init__(self, *args, **kw):
        kw.setdefault("rows_per_thread", 1)
        kw.setdefault("vec", 8)
        super().__init__(*args, **kw)

    def __repr__(self):
        return "UpdateConfig(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class CconvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        # the library's own text only when it is loaded (it may be what failed to load)
        if _lib is not None:
            msg += f" ({cconv_status_string(status)})"
        super().__init__(msg)


_lock = threading.Lock()
_lib = None
_roof = None


class FwdOpts(ctypes.Structure):
    """cconv_fwd_opts_t."""

    _fields_ = [
        ("activation", ctypes.c_int),
        ("residual", ctypes.c_void_p),
        ("residual_sb", ctypes.c_int64),
        ("residual_st", ctypes.c_int64),
        ("init_state", ctypes.c_void_p),
        ("final_state", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("nseq", ctypes.c_int64),
        ("status", ctypes.c_void_p),
        ("y_sb", ctypes.c_int64),
        ("y_st", ctypes.c_int64),
    ]


class BwdOpts(ctypes.Structure):
    """cconv_bwd_opts_t."""

    _fields_ = [
        ("activation", ctypes.c_int),
        ("init_state", ctypes.c_void_p),
        ("d_init_state", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("nseq", ctypes.c_int64),
        ("status", ctypes.c_void_p),
        ("dx_sb", ctypes.c_int64),
        ("dx_st", ctypes.c_int64),
    ]


ACTIVATIONS = {"silu": 1, "swish": 1, None: 0, "none": 0}


def _declare(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.cconv_fwd.argtypes = [p, i64, i64, p, i32, p, p, i64, i64, i64, i32, p]
    L.cconv_fwd.restype = i32
    L.cconv_fwd_config.argtypes = [p, i64, i64, p, i32, p, p, i64, i64, i64, i32, ctypes.POINTER(Config), p]
    L.cconv_fwd_config.restype = i32
    L.cconv_bwd_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.cconv_bwd_workspace_bytes.restype = sz
    L.cconv_bwd_workspace_bytes_config.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Config)]
    L.cconv_bwd_workspace_bytes_config.restype = sz
    bwd = [p, i64, i64, p, i64, i64, p, i32, p, p, p, i32, p, p, sz, i64, i64, i64, i32]
    L.cconv_bwd.argtypes = bwd + [p]
    L.cconv_bwd.restype = i32
    L.cconv_bwd_config.argtypes = bwd + [ctypes.POINTER(Config), p]
    L.cconv_bwd_config.restype = i32
    L.cconv_fwd_state.argtypes = [p, i64, i64, p, i32, p, p, p, p, i64, i64, i64, i32, p]
    L.cconv_fwd_state.restype = i32
    L.cconv_fwd_ex.argtypes = [p, i64, i64, p, i32, p, p, i64, i64, i64, i32, ctypes.POINTER(FwdOpts), p]
    L.cconv_fwd_ex.restype = i32
    L.cconv_bwd_ex.argtypes = [p, i64, i64, p, i64, i64, p, i32, p, p, p, i32, p, p, sz, i64, i64, i64, i32,
                               ctypes.POINTER(BwdOpts), p]
    L.cconv_bwd_ex.restype = i32
    L.cconv_fwd_pool.argtypes = [p, i64, i64, p, i32, p, p, i64, p, p, p, p, i64, i64, i64, i32, p]
    L.cconv_fwd_pool.restype = i32
    L.cconv_fwd_varlen.argtypes = [p, i64, p, i64, i64, p, i32, p, p, p, p, p, i64, i32, p]
    L.cconv_fwd_varlen.restype = i32
    L.cconv_fwd_varlen_config.argtypes = [p, i64, p, i64, i64, p, i32, p, p, p, p, p, i64, i32,
                                          ctypes.POINTER(Config), p]
    L.cconv_fwd_varlen_config.restype = i32
    bv = [p, i64, p, i64, p, i64, i64, p, i32, p, p, p, p, i32, p, p, p, sz, p, i64, i32]
    L.cconv_bwd_varlen.argtypes = bv + [p]
    L.cconv_bwd_varlen.restype = i32
    L.cconv_bwd_varlen_config.argtypes = bv + [ctypes.POINTER(Config), p]
    L.cconv_bwd_varlen_config.restype = i32
    L.cconv_bwd_state.argtypes = [p, i64, i64, p, i64, i64, p, i32, p, p, p, p, i32, p, p, p, sz, i64, i64, i64,
                                  i32, p]
    L.cconv_bwd_state.restype = i32
    L.cconv_bwd_noalloc.argtypes = [p, i64, i64, p, i64, i64, p, i32, p, p, p, i32, p, i64, i64, i64, i32, p]
    L.cconv_bwd_noalloc.restype = i32
    L.cconv_bwd_noalloc_max_workspace.argtypes = []
    L.cconv_bwd_noalloc_max_workspace.restype = sz
    L.cconv_bwd_main.argtypes = [p, i64, i64, p, i64, i64, p, i32, p, p, p, sz, i64, i64, i64, i32, p]
    L.cconv_bwd_main.restype = i32
    L.cconv_bwd_finish.argtypes = [p, sz, p, i32, p, i64, i64, i64, i32, p]
    L.cconv_bwd_finish.restype = i32
    L.cconv_update_ex.argtypes = [p, i64, p, i64, i32, p, p, p, i32, p, p, i64, i64, i32, p, p]
    L.cconv_update_ex.restype = i32
    L.cconv_update.argtypes = [p, i64, p, i64, p, p, i32, p, p, i64, i64, i32, p, p]
    L.cconv_update.restype = i32
    L.cconv_update_config.argtypes = [p, i64, p, i64, i32, p, p, p, i32, p, p, i64, i64, i32, p,
                                      ctypes.POINTER(UpdateConfig), p]
    L.cconv_update_config.restype = i32
    L.cconv_default_update_config.argtypes = [i64, i64, ctypes.POINTER(UpdateConfig)]
    L.cconv_default_update_config.restype = i32
    L.cconv_default_config.argtypes = [i32, i64, i64, i64, i32, ctypes.POINTER(Config)]
    L.cconv_default_config.restype = i32
    L.cconv_status_string.argtypes = [i32]
    L.cconv_status_string.restype = ctypes.c_char_p
    L.cconv_version.argtypes = []
    L.cconv_version.restype = ctypes.c_char_p
    return L


def _ensure_built(path: Path):
    if not path.exists():
        from . import _build

        _build.build()
    if not path.exists():
        raise CconvError(9, f"{path.name} is not built and could not be built")


def lib() -> ctypes.CDLL:
    """The loaded libcconv.so (built in-tree on first use if absent)."""
    global _lib
    L = _lib
    if L is not None:  # loaded: no lock on the per-call path
        return L
    with _lock:
        if _lib is None:
            _ensure_built(LIB_PATH)
            _lib = _declare(ctypes.CDLL(str(LIB_PATH)))
        return _lib


def roofline_lib() -> ctypes.CDLL:
    """The loaded libcconv_roofline.so (flat-copy kernels for the bandwidth roofline)."""
    global _roof
    with _lock:
        if _roof is None:
            _ensure_built(ROOFLINE_LIB_PATH)
            L = ctypes.CDLL(str(ROOFLINE_LIB_PATH))
            p = ctypes.c_void_p
            L.cconv_roofline_copy.argtypes = [ctypes.c_int, p, p, p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, p]
            L.cconv_roofline_copy.restype = ctypes.c_int
            L.cconv_roofline_copy_persistent.argtypes = [ctypes.c_int, p, p, p, ctypes.c_int64, ctypes.c_int,
                                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, p]
            L.cconv_roofline_copy_persistent.restype = ctypes.c_int
            _roof = L
        return _roof


def cconv_status_string(status: int) -> str:
    return lib().cconv_status_string(int(status)).decode()


def cconv_version() -> str:
    return lib().cconv_version().decode()


def _stream(stream) -> Optional[int]:
    if stream is None:
        if _raw_stream is not None:  # the current stream's handle without building a Stream object
            return _raw_stream(_current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    _dev(t, "every tensor handed to the library")
    return t.data_ptr()


# the current device, read without torch.cuda.current_device()'s per-call initialisation check
# (a GPU tensor exists by the time it is asked, so the runtime is initialised)
_current_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    # the library launches on the current device: an operand elsewhere would be read through a
    # foreign address
    if t.get_device() != _current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device cuda:{_current_device()}")


def _out(t: Optional[torch.Tensor], name: str, shape, dtypes):
    """A caller-provided output or buffer: the library learns only its address, so its device,
    dtype, shape and layout are checked here (an undersized tensor would be written past)."""
    if t is None:
        return
    _dev(t, name)
    if t.dtype not in dtypes or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        kinds = "/".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be a contiguous {kinds} tensor of shape {list(shape)}")


def _ws(t: Optional[torch.Tensor]) -> int:
    """Bytes of a caller-provided workspace (contiguous, on the current device)."""
    if t is None:
        return 0
    _dev(t, "workspace")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return t.numel() * t.element_size()


_BF = (torch.bfloat16,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_WT = (torch.bfloat16, torch.float32)


def _wdt(t: torch.Tensor, name: str) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"{name} must be bf16 or fp32 (got {t.dtype})")


def _act(t: torch.Tensor, name: str):
    _dev(t, name)
    if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be bf16 [B, T, D] with unit channel stride")
    return t.stride(0), t.stride(1)


def _check(status: int, where: str):
    if status != 0:
        raise CconvError(status, where)


def cconv_default_config(which: str, B: int, T: int, D: int, W: int) -> Config:
    cfg = Config()
    _check(lib().cconv_default_config(0 if which == "fwd" else 1, B, T, D, W, ctypes.byref(cfg)), "cconv_default_config")
    return cfg


def cconv_fwd(x, w, bias=None, *, y=None, config: Optional[Config] = None, stream=None):
    """y = silu(causal depthwise conv(x, w) + bias). x bf16 [B, T, D]; w [D, W]; bias fp32 [D]."""
    sb, st = _act(x, "x")
    B, T, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    if y is None:
        y = torch.empty((B, T, D), dtype=torch.bfloat16, device=x.device)
    elif y.dtype != torch.bfloat16 or tuple(y.shape) != (B, T, D) or not y.is_contiguous():
        raise ValueError("y must be a contiguous bf16 [B, T, D] tensor")
    L = lib()
    args = (_ptr(x), sb, st, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(y), B, T, D, W)
    if config is None:
        _check(L.cconv_fwd(*args, _stream(stream)), "cconv_fwd")
    else:
        _check(L.cconv_fwd_config(*args, ctypes.byref(config), _stream(stream)), "cconv_fwd_config")
    return y


def cconv_bwd_workspace_bytes(B: int, T: int, D: int, W: int, config: Optional[Config] = None) -> int:
    if config is None:
        return int(lib().cconv_bwd_workspace_bytes(B, T, D, W))
    return int(lib().cconv_bwd_workspace_bytes_config(B, T, D, W, ctypes.byref(config)))


def cconv_bwd(
    x,
    dy,
    w,
    bias=None,
    *,
    dx=None,
    dw=None,
    dbias=None,
    want_dbias: bool = True,
    dw_dtype: Optional[torch.dtype] = None,
    workspace=None,
    config: Optional[Config] = None,
    stream=None,
):
    """(dx, dw, dbias) of y = silu(conv(x, w) + bias) for upstream gradient dy.

    dw is returned in ``dw_dtype`` (default: w's dtype); dbias is fp32 (None if not wanted).
    """
    sb, st = _act(x, "x")
    dsb, dst = _act(dy, "dy")
    B, T, D = x.shape
    if tuple(dy.shape) != (B, T, D):
        raise ValueError("dy must have x's shape")
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    dev = x.device
    if dx is None:
        dx = torch.empty((B, T, D), dtype=torch.bfloat16, device=dev)
    if dw is None:
        dw = torch.empty((D, W), dtype=dw_dtype or w.dtype, device=dev)
    if want_dbias and dbias is None:
        dbias = torch.empty((D,), dtype=torch.float32, device=dev)
    _out(dx, "dx", x.shape, _BF)
    _out(dw, "dw", (D, W), _WT)
    _out(dbias, "dbias", (D,), _F32)
    need = cconv_bwd_workspace_bytes(B, T, D, W, config)
    if workspace is None and need > 0:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    ws_bytes = _ws(workspace)
    L = lib()
    args = (
        _ptr(x), sb, st, _ptr(dy), dsb, dst, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(dx), _ptr(dw),
        _wdt(dw, "dw"), _ptr(dbias), _ptr(workspace), ws_bytes, B, T, D, W,
    )
    if config is None:
        _check(L.cconv_bwd(*args, _stream(stream)), "cconv_bwd")
    else:
        _check(L.cconv_bwd_config(*args, ctypes.byref(config), _stream(stream)), "cconv_bwd_config")
    return dx, dw, dbias


def _state(t: Optional[torch.Tensor], name: str, B: int, D: int, W: int):
    if t is None:
        return
    _dev(t, name)
    if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, D, W - 1) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 [B, D, W-1] tensor")


def cconv_fwd_state(x, w, bias=None, init_state=None, *, final_state=None, want_final_state=True, y=None,
                    stream=None):
    """Forward with a history before t = 0; returns (y, final_state).

    init_state, final_state: bf16 [B, D, W-1], oldest value first (the decode state layout).
    init_state None means zeros. final_state (allocated when None and wanted) receives the last
    W-1 values of history-then-x; passing init_state itself advances it in place.
    """
    sb, st = _act(x, "x")
    B, T, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    _state(init_state, "init_state", B, D, W)
    if want_final_state and final_state is None:
        final_state = torch.empty((B, D, W - 1), dtype=torch.bfloat16, device=x.device)
    _state(final_state, "final_state", B, D, W)
    if y is None:
        y = torch.empty((B, T, D), dtype=torch.bfloat16, device=x.device)
    elif y.dtype != torch.bfloat16 or tuple(y.shape) != (B, T, D) or not y.is_contiguous():
        raise ValueError("y must be a contiguous bf16 [B, T, D] tensor")
    _check(
        lib().cconv_fwd_state(
            _ptr(x), sb, st, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(init_state), _ptr(final_state), _ptr(y),
            B, T, D, W, _stream(stream),
        ),
        "cconv_fwd_state",
    )
    return y, final_state


def cconv_fwd_pool(x, w, bias, state, state_indices, has_initial_state=None, *, y=None, status=None, stream=None):
    """Prefill x [B, T, D] into the decode pool ``state`` [S, D, W-1] (updated in place);
    returns (y, status).

    state_indices: int32 [B] (slot of sequence b, -1 = padding); has_initial_state: bool or
    uint8 [B] or None (start every sequence from zeros). status (allocated if None) receives
    0 on the device, or 8 (CCONV_ERR_INDEX) when the indices break the decode slot rule, in
    which case neither y nor state was written.
    """
    sb, st = _act(x, "x")
    B, T, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    _dev(state, "state")
    if state.dtype != torch.bfloat16 or state.dim() != 3 or state.shape[1:] != (D, W - 1) or not state.is_contiguous():
        raise ValueError("state must be a contiguous bf16 [S, D, W-1] tensor")
    S = state.shape[0]
    _dev(state_indices, "state_indices")
    if state_indices.dtype != torch.int32 or state_indices.shape != (B,) or not state_indices.is_contiguous():
        raise ValueError("state_indices must be a contiguous int32 [B] tensor")
    if has_initial_state is not None:
        _dev(has_initial_state, "has_initial_state")
        if has_initial_state.dtype not in (torch.bool, torch.uint8) or has_initial_state.shape != (B,) \
                or not has_initial_state.is_contiguous():
            raise ValueError("has_initial_state must be a contiguous bool or uint8 [B] tensor")
    if y is None:
        y = torch.empty((B, T, D), dtype=torch.bfloat16, device=x.device)
    elif y.dtype != torch.bfloat16 or tuple(y.shape) != (B, T, D) or not y.is_contiguous():
        raise ValueError("y must be a contiguous bf16 [B, T, D] tensor")
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=x.device)
    _out(status, "status", (1,), _I32)
    _check(
        lib().cconv_fwd_pool(
            _ptr(x), sb, st, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(state), S, _ptr(state_indices),
            _ptr(has_initial_state), _ptr(status), _ptr(y), B, T, D, W, _stream(stream),
        ),
        "cconv_fwd_pool",
    )
    return y, status


def cconv_bwd_state(x, dy, w, bias=None, init_state=None, *, dx=None, dw=None, dbias=None, d_init_state=None,
                    want_dbias: bool = True, want_d_init_state: bool = True, dw_dtype=None, workspace=None,
                    stream=None):
    """Backward with a history before t = 0; returns (dx, dw, dbias, d_init_state).

    dw includes the products with the history; d_init_state (bf16 [B, D, W-1]) is the gradient
    of each history value.
    """
    sb, st = _act(x, "x")
    dsb, dst = _act(dy, "dy")
    B, T, D = x.shape
    if tuple(dy.shape) != (B, T, D):
        raise ValueError("dy must have x's shape")
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    _state(init_state, "init_state", B, D, W)
    dev = x.device
    if dx is None:
        dx = torch.empty((B, T, D), dtype=torch.bfloat16, device=dev)
    if dw is None:
        dw = torch.empty((D, W), dtype=dw_dtype or w.dtype, device=dev)
    if want_dbias and dbias is None:
        dbias = torch.empty((D,), dtype=torch.float32, device=dev)
    _out(dx, "dx", x.shape, _BF)
    _out(dw, "dw", (D, W), _WT)
    _out(dbias, "dbias", (D,), _F32)
    if want_d_init_state and d_init_state is None:
        d_init_state = torch.empty((B, D, W - 1), dtype=torch.bfloat16, device=dev)
    _state(d_init_state, "d_init_state", B, D, W)
    need = cconv_bwd_workspace_bytes(B, T, D, W)
    if workspace is None and need > 0:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    ws_bytes = _ws(workspace)
    _check(
        lib().cconv_bwd_state(
            _ptr(x), sb, st, _ptr(dy), dsb, dst, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(init_state), _ptr(dx),
            _ptr(dw), _wdt(dw, "dw"), _ptr(dbias), _ptr(d_init_state), _ptr(workspace), ws_bytes, B, T, D, W,
            _stream(stream),
        ),
        "cconv_bwd_state",
    )
    return dx, dw, dbias, d_init_state


def _packed(t, name: str):
    _dev(t, name)
    if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be bf16 [total, D] with unit channel stride")
    return t.stride(0)


def _offsets(cu_seqlens, W: int, D: int, init_state, dev):
    _dev(cu_seqlens, "cu_seqlens")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 [nseq + 1] tensor")
    n = cu_seqlens.numel() - 1
    _state(init_state, "init_state", n, D, W)
    return n


def cconv_fwd_varlen(x, cu_seqlens, w, bias=None, init_state=None, *, final_state=None, want_final_state=False,
                     y=None, status=None, config: Optional[Config] = None, stream=None):
    """Packed batch forward: x bf16 [total, D]; cu_seqlens int32 [nseq+1] (device). Returns
    (y, final_state or None, status): status receives 0, or 8 when the offsets are not a valid
    partition of the rows (then nothing else was written)."""
    xst = _packed(x, "x")
    total, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    n = _offsets(cu_seqlens, W, D, init_state, x.device)
    if want_final_state and final_state is None:
        final_state = torch.empty((n, D, W - 1), dtype=torch.bfloat16, device=x.device)
    _state(final_state, "final_state", n, D, W)
    if y is None:
        y = torch.empty((total, D), dtype=torch.bfloat16, device=x.device)
    elif y.dtype != torch.bfloat16 or tuple(y.shape) != (total, D) or not y.is_contiguous():
        raise ValueError("y must be a contiguous bf16 [total, D] tensor")
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=x.device)
    _out(status, "status", (1,), _I32)
    args = (_ptr(x), xst, _ptr(cu_seqlens), n, total, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(init_state),
            _ptr(final_state), _ptr(status), _ptr(y), D, W)
    L = lib()
    if config is None:
        _check(L.cconv_fwd_varlen(*args, _stream(stream)), "cconv_fwd_varlen")
    else:
        _check(L.cconv_fwd_varlen_config(*args, ctypes.byref(config), _stream(stream)), "cconv_fwd_varlen_config")
    return y, final_state, status


def cconv_bwd_varlen(x, dy, cu_seqlens, w, bias=None, init_state=None, *, dx=None, dw=None, dbias=None,
                     d_init_state=None, want_dbias: bool = True, want_d_init_state: bool = False, dw_dtype=None,
                     workspace=None, status=None, config: Optional[Config] = None, stream=None):
    """Packed batch backward. Returns (dx, dw, dbias, d_init_state, status)."""
    xst = _packed(x, "x")
    dyst = _packed(dy, "dy")
    total, D = x.shape
    if tuple(dy.shape) != (total, D):
        raise ValueError("dy must have x's shape")
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    n = _offsets(cu_seqlens, W, D, init_state, x.device)
    dev = x.device
    if dx is None:
        dx = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    if dw is None:
        dw = torch.empty((D, W), dtype=dw_dtype or w.dtype, device=dev)
    if want_dbias and dbias is None:
        dbias = torch.empty((D,), dtype=torch.float32, device=dev)
    _out(dx, "dx", x.shape, _BF)
    _out(dw, "dw", (D, W), _WT)
    _out(dbias, "dbias", (D,), _F32)
    if want_d_init_state and d_init_state is None:
        d_init_state = torch.empty((n, D, W - 1), dtype=torch.bfloat16, device=dev)
    _state(d_init_state, "d_init_state", n, D, W)
    need = cconv_bwd_workspace_bytes(1, total, D, W, config)
    if workspace is None and need > 0:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    ws_bytes = _ws(workspace)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _out(status, "status", (1,), _I32)
    args = (_ptr(x), xst, _ptr(dy), dyst, _ptr(cu_seqlens), n, total, _ptr(w), _wdt(w, "w"), _ptr(bias),
            _ptr(init_state), _ptr(dx), _ptr(dw), _wdt(dw, "dw"), _ptr(dbias), _ptr(d_init_state), _ptr(workspace),
            ws_bytes, _ptr(status), D, W)
    L = lib()
    if config is None:
        _check(L.cconv_bwd_varlen(*args, _stream(stream)), "cconv_bwd_varlen")
    else:
        _check(L.cconv_bwd_varlen_config(*args, ctypes.byref(config), _stream(stream)), "cconv_bwd_varlen_config")
    return dx, dw, dbias, d_init_state, status


def cconv_bwd_noalloc(x, dy, w, bias=None, *, dx, dw, dbias=None, stream=None):
    """cconv_bwd with the library's static scratch instead of a workspace: nothing is
    allocated, so the outputs dx (bf16, x's shape), dw ([D, W], bf16 or fp32) and dbias
    (fp32 [D] or None) must be given. Returns (dx, dw, dbias)."""
    sb, st = _act(x, "x")
    dsb, dst = _act(dy, "dy")
    B, T, D = x.shape
    if tuple(dy.shape) != (B, T, D):
        raise ValueError("dy must have x's shape")
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    _out(dx, "dx", x.shape, _BF)
    _out(dw, "dw", (D, W), _WT)
    _out(dbias, "dbias", (D,), _F32)
    _check(
        lib().cconv_bwd_noalloc(
            _ptr(x), sb, st, _ptr(dy), dsb, dst, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(dx), _ptr(dw),
            _wdt(dw, "dw"), _ptr(dbias), B, T, D, W, _stream(stream),
        ),
        "cconv_bwd_noalloc",
    )
    return dx, dw, dbias


def cconv_bwd_noalloc_max_workspace() -> int:
    """Bytes of the static scratch cconv_bwd_noalloc uses (its largest workspace)."""
    return int(lib().cconv_bwd_noalloc_max_workspace())


def cconv_bwd_main(x, dy, w, bias, dx, workspace, *, stream=None):
    """First backward stage: dx and the fp32 dw/dbias partials (into `workspace`)."""
    sb, st = _act(x, "x")
    dsb, dst = _act(dy, "dy")
    B, T, D = x.shape
    if tuple(dy.shape) != (B, T, D):
        raise ValueError("dy must have x's shape")
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    _out(bias, "bias", (D,), _F32)
    _out(dx, "dx", (B, T, D), _BF)
    ws_bytes = _ws(workspace)
    _check(
        lib().cconv_bwd_main(
            _ptr(x), sb, st, _ptr(dy), dsb, dst, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(dx), _ptr(workspace),
            ws_bytes, B, T, D, W, _stream(stream),
        ),
        "cconv_bwd_main",
    )
    return dx


def cconv_bwd_finish(workspace, dw, dbias, B: int, T: int, D: int, W: int, *, stream=None):
    """Second backward stage: dw (in dw's dtype) and dbias from the partials."""
    _out(dw, "dw", (D, W), _WT)
    _out(dbias, "dbias", (D,), _F32)
    ws_bytes = _ws(workspace)
    _check(
        lib().cconv_bwd_finish(
            _ptr(workspace), ws_bytes, _ptr(dw), _wdt(dw, "dw"), _ptr(dbias), B, T, D, W, _stream(stream)
        ),
        "cconv_bwd_finish",
    )
    return dw, dbias


def cconv_update(x, state, state_indices, w, bias=None, *, y=None, status=None, stream=None):
    """One decode step: returns (y, status). state is updated in place.

    x bf16 [N, D] (row stride >= D); state bf16 [S, D, W-1]; state_indices int32 [N] or None;
    status: an int32 device tensor of one element (allocated if None); it receives
    CCONV_OK (0) or CCONV_ERR_INDEX (8) on the device.
    """
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be bf16 [N, D] with unit channel stride")
    N, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    _dev(state, "state")
    if state.dtype != torch.bfloat16 or state.dim() != 3 or state.shape[1:] != (D, W - 1) or not state.is_contiguous():
        raise ValueError("state must be a contiguous bf16 [S, D, W-1] tensor")
    S = state.shape[0]
    if state_indices is not None:
        _dev(state_indices, "state_indices")
        if state_indices.dtype != torch.int32 or state_indices.shape != (N,) or not state_indices.is_contiguous():
            raise ValueError("state_indices must be a contiguous int32 [N] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    if y is None:
        y = torch.empty((N, D), dtype=torch.bfloat16, device=x.device)
    _out(y, "y", (N, D), _BF)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=x.device)
    _out(status, "status", (1,), _I32)
    _check(
        lib().cconv_update(
            _ptr(x), x.stride(0) if N > 0 else D, _ptr(state), S, _ptr(state_indices), _ptr(w), _wdt(w, "w"),
            _ptr(bias), _ptr(y), N, D, W, _ptr(status), _stream(stream),
        ),
        "cconv_update",
    )
    return y, status


def cconv_update_ex(x, state, state_indices, w, bias=None, *, cache_seqlens=None, y=None, status=None, stream=None):
    """A decode step with a state of L entries (state bf16 [S, D, L], L = W-1 or W; L is read
    from the state's shape) and, with cache_seqlens (int32 [N]), circular-buffer addressing:
    the token k steps back is entry (c - k) mod L, the new token goes to entry c mod L. Returns
    (y, status); state is updated in place."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be bf16 [N, D] with unit channel stride")
    N, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    _dev(state, "state")
    if state.dtype != torch.bfloat16 or state.dim() != 3 or state.shape[1] != D or not state.is_contiguous():
        raise ValueError("state must be a contiguous bf16 [S, D, L] tensor")
    S, L = state.shape[0], state.shape[2]
    for t, name in ((state_indices, "state_indices"), (cache_seqlens, "cache_seqlens")):
        if t is not None:
            _dev(t, name)
            if t.dtype != torch.int32 or t.shape != (N,) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 [N] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    if y is None:
        y = torch.empty((N, D), dtype=torch.bfloat16, device=x.device)
    _out(y, "y", (N, D), _BF)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=x.device)
    _out(status, "status", (1,), _I32)
    _check(
        lib().cconv_update_ex(
            _ptr(x), x.stride(0) if N > 0 else D, _ptr(state), S, L, _ptr(state_indices), _ptr(cache_seqlens),
            _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(y), N, D, W, _ptr(status), _stream(stream),
        ),
        "cconv_update_ex",
    )
    return y, status


def cconv_update_config(x, state, state_indices, w, bias=None, *, config, cache_seqlens=None, y=None, status=None,
                        stream=None):
    """cconv_update_ex with an explicit launch configuration (an UpdateConfig). Returns (y, status);
    state (bf16 [S, D, L]) is updated in place."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be bf16 [N, D] with unit channel stride")
    N, D = x.shape
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    _dev(state, "state")
    if state.dtype != torch.bfloat16 or state.dim() != 3 or state.shape[1] != D or not state.is_contiguous():
        raise ValueError("state must be a contiguous bf16 [S, D, L] tensor")
    S, L = state.shape[0], state.shape[2]
    for t, name in ((state_indices, "state_indices"), (cache_seqlens, "cache_seqlens")):
        if t is not None:
            _dev(t, name)
            if t.dtype != torch.int32 or t.shape != (N,) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 [N] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    if not isinstance(config, UpdateConfig):
        raise TypeError("config must be an UpdateConfig")
    if y is None:
        y = torch.empty((N, D), dtype=torch.bfloat16, device=x.device)
    _out(y, "y", (N, D), _BF)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=x.device)
    _out(status, "status", (1,), _I32)
    _check(
        lib().cconv_update_config(
            _ptr(x), x.stride(0) if N > 0 else D, _ptr(state), S, L, _ptr(state_indices), _ptr(cache_seqlens),
            _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(y), N, D, W, _ptr(status), ctypes.byref(config), _stream(stream),
        ),
        "cconv_update_config",
    )
    return y, status


def cconv_default_update_config(N: int, D: int) -> UpdateConfig:
    """The launch configuration cconv_update / cconv_update_ex use for N rows of D channels."""
    c = UpdateConfig()
    _check(lib().cconv_default_update_config(N, D, ctypes.byref(c)), "cconv_default_update_config")
    return c


def _out_rows(t, name: str, like: torch.Tensor, packed: bool):
    """(batch stride, row stride) of a caller-provided output of the general entry points: x's
    shape, bf16, unit channel stride; (0, 0) when contiguous (the library's default layout)."""
    _dev(t, name)
    if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(like.shape) or t.stride(-1) != 1:
        raise ValueError(f"{name} must be bf16 of x's shape with unit channel stride")
    if t.is_contiguous():
        return 0, 0
    return (0, t.stride(0)) if packed else (t.stride(0), t.stride(1))


def _rows(t, name: str, packed: bool):
    """(batch stride, row stride) of a bf16 activation: [B, T, D], or [total, D] when packed."""
    if packed:
        return 0, _packed(t, name)
    return _act(t, name)


def cconv_fwd_ex(x, w, bias=None, *, activation="silu", residual=None, init_state=None, final_state=None,
                 want_final_state=False, cu_seqlens=None, y=None, status=None, stream=None):
    """The general forward: y = act(conv(x) + bias) + residual, optionally from a history, with
    a final state, over a [B, T, D] batch or (cu_seqlens) a packed [total, D] batch. Returns
    (y, final_state, status); status is None for fixed-length batches. A caller-provided y may
    be a view with wider rows (unit channel stride; e.g. D = 6144 channels of rows of 8192):
    its strides are passed to the library."""
    packed = cu_seqlens is not None
    sb, st = _rows(x, "x", packed)
    if packed:
        B, (T, D) = 1, x.shape
        n = _offsets(cu_seqlens, w.shape[1], D, init_state, x.device)
        state_rows = n
    else:
        B, T, D = x.shape
        state_rows = B
        _state(init_state, "init_state", B, D, w.shape[1])
    _dev(w, "w")
    W = w.shape[1]
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(k for k in ACTIVATIONS if k)} or None")
    rsb = rst = 0
    if residual is not None:
        if tuple(residual.shape) != tuple(x.shape):
            raise ValueError("residual must have x's shape")
        rsb, rst = _rows(residual, "residual", packed)
    if want_final_state and final_state is None:
        final_state = torch.empty((state_rows, D, W - 1), dtype=torch.bfloat16, device=x.device)
    _state(final_state, "final_state", state_rows, D, W)
    if y is None:
        y = torch.empty(tuple(x.shape), dtype=torch.bfloat16, device=x.device)
    ysb, yst = _out_rows(y, "y", x, packed)
    if packed and status is None:
        status = torch.empty(1, dtype=torch.int32, device=x.device)
    _out(status, "status", (1,), _I32)
    o = FwdOpts(ACTIVATIONS[activation], _ptr(residual), rsb, rst, _ptr(init_state), _ptr(final_state),
                _ptr(cu_seqlens), state_rows if packed else 0, _ptr(status) if packed else None, ysb, yst)
    _check(lib().cconv_fwd_ex(_ptr(x), sb, st, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(y), B, T, D, W,
                              ctypes.byref(o), _stream(stream)), "cconv_fwd_ex")
    return y, final_state, status


def cconv_bwd_ex(x, dy, w, bias=None, *, activation="silu", init_state=None, d_init_state=None,
                 want_d_init_state=False, cu_seqlens=None, dx=None, dw=None, dbias=None, want_dbias=True,
                 dw_dtype=None, workspace=None, status=None, stream=None):
    """The general backward (see cconv_fwd_ex; a residual's gradient is dy itself). Returns
    (dx, dw, dbias, d_init_state, status). A caller-provided dx may be a view with wider rows,
    as cconv_fwd_ex's y."""
    packed = cu_seqlens is not None
    sb, st = _rows(x, "x", packed)
    dsb, dst = _rows(dy, "dy", packed)
    if tuple(dy.shape) != tuple(x.shape):
        raise ValueError("dy must have x's shape")
    _dev(w, "w")
    W = w.shape[1]
    if packed:
        B, (T, D) = 1, x.shape
        state_rows = _offsets(cu_seqlens, W, D, init_state, x.device)
    else:
        B, T, D = x.shape
        state_rows = B
        _state(init_state, "init_state", B, D, W)
    if w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous [D, W] tensor")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or bias.shape != (D,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 [D] tensor")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(k for k in ACTIVATIONS if k)} or None")
    dev = x.device
    if dx is None:
        dx = torch.empty(tuple(x.shape), dtype=torch.bfloat16, device=dev)
    if dw is None:
        dw = torch.empty((D, W), dtype=dw_dtype or w.dtype, device=dev)
    if want_dbias and dbias is None:
        dbias = torch.empty((D,), dtype=torch.float32, device=dev)
    dxsb, dxst = _out_rows(dx, "dx", x, packed)
    _out(dw, "dw", (D, W), _WT)
    _out(dbias, "dbias", (D,), _F32)
    if want_d_init_state and d_init_state is None:
        d_init_state = torch.empty((state_rows, D, W - 1), dtype=torch.bfloat16, device=dev)
    _state(d_init_state, "d_init_state", state_rows, D, W)
    need = cconv_bwd_workspace_bytes(B, T, D, W)
    if workspace is None and need > 0:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    ws_bytes = _ws(workspace)
    if packed and status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _out(status, "status", (1,), _I32)
    o = BwdOpts(ACTIVATIONS[activation], _ptr(init_state), _ptr(d_init_state), _ptr(cu_seqlens),
                state_rows if packed else 0, _ptr(status) if packed else None, dxsb, dxst)
    _check(lib().cconv_bwd_ex(_ptr(x), sb, st, _ptr(dy), dsb, dst, _ptr(w), _wdt(w, "w"), _ptr(bias), _ptr(dx),
                              _ptr(dw), _wdt(dw, "dw"), _ptr(dbias), _ptr(workspace), ws_bytes, B, T, D, W,
                              ctypes.byref(o), _stream(stream)), "cconv_bwd_ex")
    return dx, dw, dbias, d_init_state, status
