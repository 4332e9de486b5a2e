"""MI355X (gfx950) selective state-space scan: thin Python binding over the C ABI in include/ssm.h.

Every step of the computation runs in the HIP kernels of ``libssm61.so``.  This module only
checks shapes and dtypes, allocates outputs with ``torch.empty`` (PyTorch is used for device
memory and streams), passes ``data_ptr()`` values and the current HIP stream through ctypes, and
turns a non-OK status into an exception.  If the library has not been built, importing works but
every call raises: there is no fallback implementation.

    y, last_state = ssm_scan_fwd(x, delta, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=True)
    y_t = ssm_state_update(state, x_t, delta_t, A, B_t, C_t, D=D, z=z_t, delta_bias=bias,
                           delta_softplus=True)

Shapes: x, delta, z (batch, seqlen, dim); A (dim, dstate) fp32; B, C (batch, seqlen, dstate);
D, delta_bias (dim,) fp32; y like x; last_state / state (batch, dim, dstate) fp32.  x, delta, B, C,
z and y share one dtype: torch.float32 or torch.bfloat16.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libssm61.so")

SSM_F32, SSM_BF16 = 0, 1
STATUS_NAMES = {0: "SSM_OK", 1: "SSM_ERR_INVALID_ARG", 2: "SSM_ERR_UNSUPPORTED", 3: "SSM_ERR_MISALIGNED",
                4: "SSM_ERR_HIP"}
EXPORTED = ("ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_fwd_noalloc", "ssm_scan_fwd_ckpt", "ssm_scan_bwd",
            "ssm_scan_bwd_ex", "ssm_scan_bwd_ckpt", "ssm_state_update", "ssm_state_update_ex",
            "ssm_causal_conv1d_fwd",
            "ssm_causal_conv1d_update", "ssm_ssd_fwd", "ssm_ssd_state_update", "ssm_status_string", "ssm_last_error", "ssm_abi_version")


class SsmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class ScanOpts(ctypes.Structure):
    _fields_ = [("chains_per_lane", ctypes.c_int32), ("segments", ctypes.c_int32),
                ("chunk_steps", ctypes.c_int32), ("bbar_mode", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("channel_groups", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


class UpdateOpts(ctypes.Structure):
    _fields_ = [("bbar_mode", ctypes.c_int32), ("reserved", ctypes.c_int32 * 7)]


class BwdOpts(ctypes.Structure):
    _fields_ = [("bbar_mode", ctypes.c_int32), ("layout", ctypes.c_int32), ("reserved", ctypes.c_int32 * 6)]


class SsdOpts(ctypes.Structure):
    _fields_ = [("head_slice", ctypes.c_int32), ("segments", ctypes.c_int32), ("gram", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 5)]


SSM_BBAR_DELTA_B, SSM_BBAR_ZOH = 0, 1
SSM_LAYOUT_AUTO, SSM_LAYOUT_CHANNEL_LANES, SSM_LAYOUT_STATE_ROWS, SSM_LAYOUT_TIME_SCAN = 0, 1, 2, 3
LAYOUTS = {"auto": SSM_LAYOUT_AUTO, "channel_lanes": SSM_LAYOUT_CHANNEL_LANES, "state_rows": SSM_LAYOUT_STATE_ROWS,
           "time_scan": SSM_LAYOUT_TIME_SCAN}


_lib_handle = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libssm61.so (raises if it is missing: build it with ``__graft_entry__.build()``)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: the HIP library must be built (there is no fallback)")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.ssm_scan_fwd.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.ssm_scan_fwd.restype = i32
    lib.ssm_scan_fwd_ex.argtypes = lib.ssm_scan_fwd.argtypes + [ctypes.POINTER(ScanOpts)]
    lib.ssm_scan_fwd_ex.restype = i32
    lib.ssm_scan_fwd_noalloc.argtypes = lib.ssm_scan_fwd_ex.argtypes
    lib.ssm_scan_fwd_noalloc.restype = i32
    lib.ssm_state_update.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.ssm_state_update.restype = i32
    lib.ssm_state_update_ex.argtypes = lib.ssm_state_update.argtypes + [ctypes.POINTER(UpdateOpts)]
    lib.ssm_state_update_ex.restype = i32
    lib.ssm_scan_bwd.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                 vp, vp, vp, vp]
    lib.ssm_scan_bwd.restype = i32
    lib.ssm_scan_bwd_ex.argtypes = lib.ssm_scan_bwd.argtypes + [ctypes.POINTER(BwdOpts)]
    lib.ssm_scan_bwd_ex.restype = i32
    # the checkpoint pair: the checkpoints pointer comes right before the stream
    lib.ssm_scan_fwd_ckpt.argtypes = lib.ssm_scan_fwd.argtypes[:-1] + [vp, vp]
    lib.ssm_scan_fwd_ckpt.restype = i32
    lib.ssm_scan_bwd_ckpt.argtypes = lib.ssm_scan_bwd.argtypes[:-1] + [vp, vp]
    lib.ssm_scan_bwd_ckpt.restype = i32
    lib.ssm_causal_conv1d_fwd.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.ssm_causal_conv1d_fwd.restype = i32
    lib.ssm_causal_conv1d_update.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, i32, vp, vp]
    lib.ssm_causal_conv1d_update.restype = i32
    lib.ssm_ssd_fwd.argtypes = [i64, i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                ctypes.POINTER(SsdOpts)]
    lib.ssm_ssd_fwd.restype = i32
    lib.ssm_ssd_state_update.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.ssm_ssd_state_update.restype = i32
    lib.ssm_status_string.argtypes = [i32]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_last_error.argtypes = []
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_abi_version.argtypes = []
    lib.ssm_abi_version.restype = i32
    _lib_handle = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise SsmError(status, lib.ssm_last_error().decode(errors="replace"))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"x, delta, B, C, z must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, device, optional: bool = False) -> None:
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def ssm_scan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                 D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False, *,
                 y: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
                 return_last_state: bool = True, chains_per_lane: int = 0, segments: int = 0,
                 chunk_steps: int = 0, zoh: bool = False, layout: str = "auto", channel_groups: int = 0,
                 stream=None, _noalloc: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selective scan forward (include/ssm.h: ssm_scan_fwd).  Returns (y, last_state); last_state
    is None when return_last_state is False and none was passed in.  chains_per_lane, segments,
    chunk_steps, layout ("auto", "channel_lanes", "state_rows", "time_scan") and channel_groups override the
    launch shape (0 / "auto" = automatic); zoh selects the exact
    zero-order-hold input term (SSM_BBAR_ZOH) instead of Delta B."""
    lib = load_library()
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, seqlen, dim) and A (dim, dstate)")
    batch, seqlen, dim = x.shape
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _need(x, "x", (batch, seqlen, dim), dt, dev)
    _need(delta, "delta", (batch, seqlen, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, seqlen, dstate), dt, dev)
    _need(C, "C", (batch, seqlen, dstate), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev, optional=True)
    _need(z, "z", (batch, seqlen, dim), dt, dev, optional=True)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", (batch, seqlen, dim), dt, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    _need(last_state, "last_state", (batch, dim, dstate), torch.float32, dev, optional=True)
    opts = ScanOpts(int(chains_per_lane), int(segments), int(chunk_steps),
                    SSM_BBAR_ZOH if zoh else SSM_BBAR_DELTA_B, LAYOUTS[layout], int(channel_groups))
    entry = lib.ssm_scan_fwd_noalloc if _noalloc else lib.ssm_scan_fwd_ex
    status = entry(batch, seqlen, dim, dstate, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                   _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), _ptr(last_state),
                   _stream(dev, stream), ctypes.byref(opts))
    _check(status)
    return y, last_state


def ssm_scan_fwd_noalloc(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                         C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                         delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False, *,
                         y: torch.Tensor, last_state: Optional[torch.Tensor] = None, chains_per_lane: int = 0,
                         segments: int = 0, chunk_steps: int = 0, zoh: bool = False, layout: str = "auto",
                         channel_groups: int = 0, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The allocation-free scan (include/ssm.h: ssm_scan_fwd_noalloc): the caller passes y (and
    last_state, or None) and nothing is allocated, by this binding or by the library."""
    if y is None:
        raise ValueError("y is required: the allocation-free scan allocates no output")
    return ssm_scan_fwd(x, delta, A, B, C, D=D, z=z, delta_bias=delta_bias, delta_softplus=delta_softplus, y=y,
                        last_state=last_state, return_last_state=False, chains_per_lane=chains_per_lane,
                        segments=segments, chunk_steps=chunk_steps, zoh=zoh, layout=layout,
                        channel_groups=channel_groups, stream=stream, _noalloc=True)


def ssm_state_update(state: torch.Tensor, x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                     z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                     delta_softplus: bool = False, *, y: Optional[torch.Tensor] = None, zoh: bool = False,
                     stream=None) -> torch.Tensor:
    """One decode step (include/ssm.h: ssm_state_update_ex); `state` is updated in place.
    Returns y (batch, dim).  zoh selects the exact zero-order-hold input term."""
    lib = load_library()
    if x.dim() != 2 or A.dim() != 2:
        raise ValueError("x must be (batch, dim) and A (dim, dstate)")
    batch, dim = x.shape
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _need(state, "state", (batch, dim, dstate), torch.float32, dev)
    _need(delta, "delta", (batch, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, dstate), dt, dev)
    _need(C, "C", (batch, dstate), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev, optional=True)
    _need(z, "z", (batch, dim), dt, dev, optional=True)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", (batch, dim), dt, dev)
    opts = UpdateOpts(SSM_BBAR_ZOH if zoh else SSM_BBAR_DELTA_B)
    status = lib.ssm_state_update_ex(batch, dim, dstate, code, _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                                     _ptr(y), _stream(dev, stream), ctypes.byref(opts))
    _check(status)
    return y


def _bwd_prepare(x, delta, A, B, C, dy, D, z, delta_bias) -> dict:
    """Shape checks and the gradient buffers of a backward call."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, seqlen, dim) and A (dim, dstate)")
    batch, seqlen, dim = x.shape
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    _need(x, "x", (batch, seqlen, dim), dt, dev)
    _need(delta, "delta", (batch, seqlen, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, seqlen, dstate), dt, dev)
    _need(C, "C", (batch, seqlen, dstate), dt, dev)
    _need(dy, "dy", (batch, seqlen, dim), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev, optional=True)
    _need(z, "z", (batch, seqlen, dim), dt, dev, optional=True)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    return {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x), "dB": torch.empty_like(B),
            "dC": torch.empty_like(C), "dA": torch.empty((dim, dstate), dtype=torch.float32, device=dev),
            "dz": torch.empty_like(x) if z is not None else None,
            "dD": torch.empty((dim,), dtype=torch.float32, device=dev) if D is not None else None,
            "ddelta_bias": torch.empty((dim,), dtype=torch.float32, device=dev) if delta_bias is not None else None}


def _bwd_args(x, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, out) -> list:
    batch, seqlen, dim = x.shape
    return [batch, seqlen, dim, A.shape[1], _dtype_code(x), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(dy), _ptr(out["dx"]),
            _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
            _ptr(out["dz"]), _ptr(out["ddelta_bias"])]


def ssm_scan_bwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                 dy: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False, zoh: bool = False,
                 layout: str = "auto", stream=None) -> dict:
    """Backward of ssm_scan_fwd (include/ssm.h: ssm_scan_bwd_ex): gradients of sum(dy * y); zoh
    differentiates the exact zero-order-hold forward; layout is "auto", "channel_lanes" or
    "state_rows" (ssm_bwd_opts_t).  Returns a dict with dx, ddelta, dB, dC (x's dtype), dA
    (fp32), and dz / dD / ddelta_bias (None unless z / D / delta_bias were given)."""
    lib = load_library()
    out = _bwd_prepare(x, delta, A, B, C, dy, D, z, delta_bias)
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    opts = BwdOpts(SSM_BBAR_ZOH if zoh else SSM_BBAR_DELTA_B, LAYOUTS[layout])
    status = lib.ssm_scan_bwd_ex(*_bwd_args(x, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, out),
                                 _stream(x.device, stream), ctypes.byref(opts))
    _check(status)
    return out


def checkpoint_shape(batch: int, seqlen: int, dim: int, dstate: int) -> Tuple[int, int, int, int]:
    """Shape of the checkpoints of ssm_scan_fwd_ckpt: the state before every 32nd step."""
    return (batch, (seqlen + 31) // 32, dim, dstate)


def ssm_scan_fwd_ckpt(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                      D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                      delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False, *,
                      y: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
                      return_last_state: bool = True, checkpoints: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """Forward that also stores the state before every 32nd step (include/ssm.h:
    ssm_scan_fwd_ckpt), for ssm_scan_bwd_ckpt.  Returns (y, last_state, checkpoints)."""
    lib = load_library()
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, seqlen, dim) and A (dim, dstate)")
    batch, seqlen, dim = x.shape
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    for t, name, shape, tdt, opt in ((x, "x", (batch, seqlen, dim), dt, False),
                                     (delta, "delta", (batch, seqlen, dim), dt, False),
                                     (A, "A", (dim, dstate), torch.float32, False),
                                     (B, "B", (batch, seqlen, dstate), dt, False),
                                     (C, "C", (batch, seqlen, dstate), dt, False),
                                     (D, "D", (dim,), torch.float32, True), (z, "z", (batch, seqlen, dim), dt, True),
                                     (delta_bias, "delta_bias", (dim,), torch.float32, True)):
        _need(t, name, shape, tdt, dev, optional=opt)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", (batch, seqlen, dim), dt, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    _need(last_state, "last_state", (batch, dim, dstate), torch.float32, dev, optional=True)
    if checkpoints is None:
        checkpoints = torch.empty(checkpoint_shape(batch, seqlen, dim, dstate), dtype=torch.float32, device=dev)
    _need(checkpoints, "checkpoints", checkpoint_shape(batch, seqlen, dim, dstate), torch.float32, dev)
    status = lib.ssm_scan_fwd_ckpt(batch, seqlen, dim, dstate, _dtype_code(x), _ptr(x), _ptr(delta), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                                   _ptr(y), _ptr(last_state), _ptr(checkpoints), _stream(dev, stream))
    _check(status)
    return y, last_state, checkpoints


def ssm_scan_bwd_ckpt(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                      dy: torch.Tensor, checkpoints: torch.Tensor, D: Optional[torch.Tensor] = None,
                      z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                      delta_softplus: bool = False, stream=None) -> dict:
    """Backward from the checkpoints of ssm_scan_fwd_ckpt on the same inputs (include/ssm.h:
    ssm_scan_bwd_ckpt); returns the same dict as ssm_scan_bwd."""
    lib = load_library()
    out = _bwd_prepare(x, delta, A, B, C, dy, D, z, delta_bias)
    batch, seqlen, dim = x.shape
    _need(checkpoints, "checkpoints", checkpoint_shape(batch, seqlen, dim, A.shape[1]), torch.float32, x.device)
    status = lib.ssm_scan_bwd_ckpt(*_bwd_args(x, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, out),
                                   _ptr(checkpoints), _stream(x.device, stream))
    _check(status)
    return out


def ssm_causal_conv1d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                          initial_state: Optional[torch.Tensor] = None, silu: bool = True, *,
                          y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                          return_final_state: bool = False,
                          stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Depthwise causal convolution before the scan (include/ssm.h: ssm_causal_conv1d_fwd).
    x: (batch, seqlen, dim); weight: (dim, width) fp32; bias: (dim,) fp32; initial_state /
    final_state: (batch, dim, width-1) in x's dtype.  Returns (y, final_state); final_state is
    None unless one was passed in or return_final_state is True."""
    lib = load_library()
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be (batch, seqlen, dim) and weight (dim, width)")
    batch, seqlen, dim = x.shape
    width = weight.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _need(weight, "weight", (dim, width), torch.float32, dev)
    _need(bias, "bias", (dim,), torch.float32, dev, optional=True)
    _need(initial_state, "initial_state", (batch, dim, width - 1), dt, dev, optional=True)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", (batch, seqlen, dim), dt, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, dim, width - 1), dtype=dt, device=dev)
    _need(final_state, "final_state", (batch, dim, width - 1), dt, dev, optional=True)
    status = lib.ssm_causal_conv1d_fwd(batch, seqlen, dim, width, code, _ptr(x), _ptr(weight), _ptr(bias),
                                       _ptr(initial_state), int(bool(silu)), _ptr(y), _ptr(final_state),
                                       _stream(dev, stream))
    _check(status)
    return y, final_state


def ssm_causal_conv1d_update(conv_state: Optional[torch.Tensor], x: torch.Tensor, weight: torch.Tensor,
                             bias: Optional[torch.Tensor] = None, silu: bool = True, *,
                             y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One token of the convolution (include/ssm.h: ssm_causal_conv1d_update); conv_state
    (batch, dim, width-1) in x's dtype is updated in place.  Returns y (batch, dim)."""
    lib = load_library()
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError("x must be (batch, dim) and weight (dim, width)")
    batch, dim = x.shape
    width = weight.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _need(weight, "weight", (dim, width), torch.float32, dev)
    _need(bias, "bias", (dim,), torch.float32, dev, optional=True)
    _need(conv_state, "conv_state", (batch, dim, width - 1), dt, dev, optional=width == 1)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", (batch, dim), dt, dev)
    status = lib.ssm_causal_conv1d_update(batch, dim, width, code, _ptr(conv_state), _ptr(x), _ptr(weight),
                                          _ptr(bias), int(bool(silu)), _ptr(y), _stream(dev, stream))
    _check(status)
    return y


def ssm_ssd_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False, *,
                initial_state: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                return_final_state: bool = True, head_slice: int = 0, segments: int = 0, gram: int = 0,
                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Mamba-2 SSD layer forward (include/ssm.h: ssm_ssd_fwd).  x, z: (batch, seqlen, nheads,
    headdim) bf16; dt: (batch, seqlen, nheads) bf16; B, C: (batch, seqlen, ngroups, dstate) bf16;
    A, D, dt_bias: (nheads,) fp32.  gram: 1 computes each chunk's C B^T once per (batch row, group)
    in a separate pass, -1 inside every head's workgroup, 0 lets the library choose.  Returns (y,
    final_state (batch, nheads, headdim, dstate) fp32 or None)."""
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim) and B (batch, seqlen, ngroups, dstate)")
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    dev, ty = x.device, x.dtype
    code = _dtype_code(x)
    _need(dt, "dt", (batch, seqlen, nheads), ty, dev)
    _need(A, "A", (nheads,), torch.float32, dev)
    _need(B, "B", (batch, seqlen, ngroups, dstate), ty, dev)
    _need(C, "C", (batch, seqlen, ngroups, dstate), ty, dev)
    _need(D, "D", (nheads,), torch.float32, dev, optional=True)
    _need(z, "z", tuple(x.shape), ty, dev, optional=True)
    _need(dt_bias, "dt_bias", (nheads,), torch.float32, dev, optional=True)
    _need(initial_state, "initial_state", (batch, nheads, headdim, dstate), torch.float32, dev, optional=True)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", tuple(x.shape), ty, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, nheads, headdim, dstate), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", (batch, nheads, headdim, dstate), torch.float32, dev, optional=True)
    opts = SsdOpts(head_slice=int(head_slice), segments=int(segments), gram=int(gram))
    status = lib.ssm_ssd_fwd(batch, seqlen, nheads, headdim, dstate, ngroups, code, _ptr(x), _ptr(dt), _ptr(A),
                             _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)),
                             _ptr(initial_state), _ptr(y), _ptr(final_state), _stream(dev, stream), ctypes.byref(opts))
    _check(status)
    return y, final_state


def ssm_ssd_state_update(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                         C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                         dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False, *,
                         y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One token of the Mamba-2 SSD layer (include/ssm.h: ssm_ssd_state_update).  state: (batch,
    nheads, headdim, dstate) fp32, updated in place; x, z: (batch, nheads, headdim) bf16; dt:
    (batch, nheads) bf16; B, C: (batch, ngroups, dstate) bf16.  Returns y (batch, nheads, headdim)."""
    lib = load_library()
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be (batch, nheads, headdim) and B (batch, ngroups, dstate)")
    batch, nheads, headdim = x.shape
    ngroups, dstate = B.shape[1], B.shape[2]
    dev, ty = x.device, x.dtype
    code = _dtype_code(x)
    _need(state, "state", (batch, nheads, headdim, dstate), torch.float32, dev)
    _need(dt, "dt", (batch, nheads), ty, dev)
    _need(A, "A", (nheads,), torch.float32, dev)
    _need(B, "B", (batch, ngroups, dstate), ty, dev)
    _need(C, "C", (batch, ngroups, dstate), ty, dev)
    _need(D, "D", (nheads,), torch.float32, dev, optional=True)
    _need(z, "z", tuple(x.shape), ty, dev, optional=True)
    _need(dt_bias, "dt_bias", (nheads,), torch.float32, dev, optional=True)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", tuple(x.shape), ty, dev)
    status = lib.ssm_ssd_state_update(batch, nheads, headdim, dstate, ngroups, code, _ptr(state), _ptr(x), _ptr(dt),
                                      _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                                      int(bool(dt_softplus)), _ptr(y), _stream(dev, stream))
    _check(status)
    return y


def abi_version() -> int:
    return load_library().ssm_abi_version()


__all__ = ["ssm_scan_fwd", "ssm_scan_bwd", "ssm_state_update", "ssm_causal_conv1d_fwd", "ssm_causal_conv1d_update",
           "ssm_ssd_fwd", "ssm_ssd_state_update", "SsdOpts", "BwdOpts", "abi_version", "load_library", "SsmError", "ScanOpts", "UpdateOpts",
           "ssm_scan_fwd_ckpt", "ssm_scan_bwd_ckpt", "checkpoint_shape",
           "LIBRARY", "EXPORTED"]
