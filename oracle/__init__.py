"""fp64 CPU oracle for the selective-scan forward and the decode state update.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports it, and the two share no code.

The arithmetic lives in ``ssm_oracle.c`` (plain sequential C in double
precision); this module only compiles it with gcc and marshals numpy arrays
through ctypes.  Tensors are passed in their storage type: ``float32``,
``float64``, or ``uint16`` holding bf16 bit patterns; the C code widens each
element to double exactly.

Every function of the oracle is pinned by ``tests/test_oracle_pins.py``
(closed forms, brute force on tiny inputs, invariants, special values).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssm_oracle.c")
LIBRARY = os.path.join(_HERE, "libssm_oracle.so")

F32, BF16, F64 = 0, 1, 2


def build(out_path: str = LIBRARY, src: str = SOURCE, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics: no -ffast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           *extra_flags, "-o", out_path + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs must be float32, float64 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a: Optional[np.ndarray], dtype=None) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


class Oracle:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        lib.oracle_scan.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32]
        lib.oracle_scan.restype = i32
        lib.oracle_scan_ex.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp,
                                       i32]
        lib.oracle_scan_ex.restype = i32
        lib.oracle_state_update_ex.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
        lib.oracle_state_update_ex.restype = i32
        lib.oracle_scan_channels.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64,
                                             vp, vp, vp, vp, i32]
        lib.oracle_scan_channels.restype = i32
        lib.oracle_state_update.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        lib.oracle_state_update.restype = i32
        lib.oracle_softplus.argtypes = [dp]
        lib.oracle_softplus.restype = dp
        lib.oracle_silu.argtypes = [dp]
        lib.oracle_silu.restype = dp
        lib.oracle_widen.argtypes = [vp, i32, i64]
        lib.oracle_widen.restype = dp
        lib.oracle_max_threads.restype = i32
        lib.oracle_scan_bwd.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                        vp, vp, vp, vp, vp, vp]
        lib.oracle_scan_bwd.restype = i32
        lib.oracle_scan_bwd_ex.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_scan_bwd_ex.restype = i32
        lib.oracle_ssd.argtypes = [i64, i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                   i32]
        lib.oracle_ssd.restype = i32
        lib.oracle_causal_conv1d.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, i32, vp, vp]
        lib.oracle_causal_conv1d.restype = i32
        lib.oracle_conv1d_update.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, i32, vp]
        lib.oracle_conv1d_update.restype = i32
        self._lib = lib

    # -- scalar helpers -------------------------------------------------------------------------
    def softplus(self, v: float) -> float:
        return self._lib.oracle_softplus(float(v))

    def silu(self, z: float) -> float:
        return self._lib.oracle_silu(float(z))

    def widen(self, a: np.ndarray) -> np.ndarray:
        a = _c(a)
        code = _dtype_code(a)
        return np.array([self._lib.oracle_widen(_ptr(a), code, i) for i in range(a.size)]).reshape(a.shape)

    def max_threads(self) -> int:
        return self._lib.oracle_max_threads()

    # -- the scan -------------------------------------------------------------------------------
    def scan(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
             h0=None, nthreads: int = 1, zoh: bool = False) -> Tuple[np.ndarray, np.ndarray]:
        """Full scan.  x, delta, z: (batch, L, dim); B, C: (batch, L, N); A: (dim, N) fp32;
        D, delta_bias: (dim,) fp32.  Returns y (batch, L, dim) and last_state (batch, dim, N),
        both float64."""
        x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
        code = _dtype_code(x)
        for t in (delta, B, C) + ((z,) if z is not None else ()):
            if _dtype_code(t) != code:
                raise TypeError("x, delta, B, C and z must share one storage type")
        A = _c(A, np.float32)
        D = _c(D, np.float32)
        delta_bias = _c(delta_bias, np.float32)
        h0 = _c(h0, np.float64)
        batch, L, dim = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and A.shape == (dim, N)
        assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (batch, dim, N)
        y = np.empty((batch, L, dim), np.float64)
        st = np.empty((batch, dim, N), np.float64)
        if zoh:
            rc = self._lib.oracle_scan_ex(batch, L, dim, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                          _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), 1,
                                          _ptr(h0), _ptr(y), _ptr(st), int(nthreads))
        else:
            rc = self._lib.oracle_scan(batch, L, dim, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                       _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0),
                                       _ptr(y), _ptr(st), int(nthreads))
        if rc != 0:
            raise ValueError("oracle_scan rejected its arguments")
        return y, st

    def scan_channels(self, x, delta, A, B, C, sel_b, sel_d, D=None, z=None, delta_bias=None,
                      delta_softplus=False, nthreads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
        """The scan for selected channels only (from zero state).  Returns y (nsel, L) and
        state (nsel, N) as float64."""
        x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
        code = _dtype_code(x)
        A = _c(A, np.float32)
        D = _c(D, np.float32)
        delta_bias = _c(delta_bias, np.float32)
        sel_b = np.ascontiguousarray(sel_b, np.int64)
        sel_d = np.ascontiguousarray(sel_d, np.int64)
        batch, L, dim = x.shape
        N = A.shape[1]
        y = np.empty((sel_b.size, L), np.float64)
        st = np.empty((sel_b.size, N), np.float64)
        rc = self._lib.oracle_scan_channels(batch, L, dim, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                            _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                            int(bool(delta_softplus)), sel_b.size, _ptr(sel_b), _ptr(sel_d),
                                            _ptr(y), _ptr(st), int(nthreads))
        if rc != 0:
            raise ValueError("oracle_scan_channels rejected its arguments")
        return y, st

    def state_update(self, state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=False, zoh: bool = False) -> Tuple[np.ndarray, np.ndarray]:
        """One decode step.  state: (batch, dim, N) (not modified; a float64 copy is updated
        and returned); x, delta, z: (batch, dim); B, C: (batch, N).  Returns (y, new_state)."""
        x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
        code = _dtype_code(x)
        A = _c(A, np.float32)
        D = _c(D, np.float32)
        delta_bias = _c(delta_bias, np.float32)
        st = np.array(state, np.float64, copy=True, order="C")
        batch, dim = x.shape
        N = A.shape[1]
        assert st.shape == (batch, dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
        y = np.empty((batch, dim), np.float64)
        rc = self._lib.oracle_state_update_ex(batch, dim, N, code, _ptr(st), _ptr(x), _ptr(delta), _ptr(A),
                                              _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                              int(bool(delta_softplus)), int(bool(zoh)), _ptr(y))
        if rc != 0:
            raise ValueError("oracle_state_update rejected its arguments")
        return y, st


    def scan_bwd(self, x, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False,
                 zoh: bool = False):
        """Gradients of sum(dy * y) for the scan from a zero state (zoh: the exact zero-order-hold
        input term of the forward).  Returns a dict of float64
        arrays: dx, ddelta (batch, L, dim); dA (dim, N); dB, dC (batch, L, N); dD, ddelta_bias
        (dim,) when D / delta_bias are given; dz (batch, L, dim) when z is given."""
        x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
        code = _dtype_code(x)
        A = _c(A, np.float32)
        D = _c(D, np.float32)
        delta_bias = _c(delta_bias, np.float32)
        dy = _c(dy, np.float64)
        batch, L, dim = x.shape
        N = A.shape[1]
        assert dy.shape == x.shape
        out = {"dx": np.empty((batch, L, dim)), "ddelta": np.empty((batch, L, dim)), "dA": np.empty((dim, N)),
               "dB": np.empty((batch, L, N)), "dC": np.empty((batch, L, N))}
        out["dD"] = np.empty(dim) if D is not None else None
        out["ddelta_bias"] = np.empty(dim) if delta_bias is not None else None
        out["dz"] = np.empty((batch, L, dim)) if z is not None else None
        rc = self._lib.oracle_scan_bwd_ex(batch, L, dim, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                       _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                                       int(bool(zoh)), _ptr(dy),
                                       _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
                                       _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                                       _ptr(out["ddelta_bias"]))
        if rc != 0:
            raise ValueError("oracle_scan_bwd rejected its arguments")
        return out

    def ssd(self, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, h0=None,
            nthreads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
        """Mamba-2 SSD layer.  x, z: (batch, L, nheads, headdim); dt: (batch, L, nheads); B, C:
        (batch, L, ngroups, dstate); A, D, dt_bias: (nheads,) fp32; h0: the entering state
        (batch, nheads, headdim, dstate) or None (zero).  Returns y (like x) and final_state
        (batch, nheads, headdim, dstate), float64."""
        x, dt, B, C, z = _c(x), _c(dt), _c(B), _c(C), _c(z)
        h0 = _c(h0, np.float64)
        code = _dtype_code(x)
        A, D, dt_bias = _c(A, np.float32), _c(D, np.float32), _c(dt_bias, np.float32)
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (batch, L, H) and B.shape == C.shape == (batch, L, G, N) and A.shape == (H,)
        y = np.empty((batch, L, H, P))
        fin = np.empty((batch, H, P, N))
        if h0 is not None:
            assert h0.shape == (batch, H, P, N)
        rc = self._lib.oracle_ssd(batch, L, H, P, N, G, code, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(h0), _ptr(y), _ptr(fin),
                                  int(nthreads))
        if rc != 0:
            raise ValueError("oracle_ssd rejected its arguments")
        return y, fin

    # -- the causal convolution before the scan ------------------------------------------------
    def causal_conv1d(self, x, weight, bias=None, init_state=None, silu=True) -> Tuple[np.ndarray, np.ndarray]:
        """Depthwise causal convolution.  x: (batch, L, dim) (float32 / float64 / bf16 bits);
        weight: (dim, K) fp32; bias: (dim,) fp32; init_state: (batch, dim, K-1) in x's storage
        type.  Returns y (batch, L, dim) and final_state (batch, dim, K-1), both float64."""
        x, init_state = _c(x), _c(init_state)
        code = _dtype_code(x)
        if init_state is not None and _dtype_code(init_state) != code:
            raise TypeError("init_state must share x's storage type")
        weight = _c(weight, np.float32)
        bias = _c(bias, np.float32)
        batch, L, dim = x.shape
        K = weight.shape[1]
        assert weight.shape == (dim, K)
        assert bias is None or bias.shape == (dim,)
        assert init_state is None or init_state.shape == (batch, dim, K - 1)
        y = np.empty((batch, L, dim), np.float64)
        fin = np.empty((batch, dim, K - 1), np.float64)
        rc = self._lib.oracle_causal_conv1d(batch, L, dim, K, code, _ptr(x), _ptr(weight), _ptr(bias),
                                            _ptr(init_state), int(bool(silu)), _ptr(y), _ptr(fin))
        if rc != 0:
            raise ValueError("oracle_causal_conv1d rejected its arguments")
        return y, fin

    def conv1d_update(self, state, x, weight, bias=None, silu=True) -> Tuple[np.ndarray, np.ndarray]:
        """One decode step of the convolution.  state: (batch, dim, K-1) (not modified; a float64
        copy is updated and returned); x: (batch, dim).  Returns (y, new_state)."""
        x = _c(x)
        code = _dtype_code(x)
        weight = _c(weight, np.float32)
        bias = _c(bias, np.float32)
        st = np.array(state, np.float64, copy=True, order="C")
        batch, dim = x.shape
        K = weight.shape[1]
        assert st.shape == (batch, dim, K - 1) and weight.shape == (dim, K)
        y = np.empty((batch, dim), np.float64)
        rc = self._lib.oracle_conv1d_update(batch, dim, K, code, _ptr(st), _ptr(x), _ptr(weight), _ptr(bias),
                                            int(bool(silu)), _ptr(y))
        if rc != 0:
            raise ValueError("oracle_conv1d_update rejected its arguments")
        return y, st


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built from ``ssm_oracle.c`` (compiled on first use if absent or stale)."""
    global _default
    if _default is None:
        if (not os.path.exists(LIBRARY)) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default
