"""Seeded synthetic inputs for the selective-scan workloads.

This module only draws random tensors.  It holds none of the scan's
arithmetic, and it is the one piece that both sides of a parity check share:
the HIP path receives these arrays on the device, the fp64 oracle receives the
same bytes on the host.

Randomness is numpy's Philox4x64 counter-based generator (Salmon et al., SC'11),
with one stream per (seed, tensor) pair, so every tensor is reproducible on its
own regardless of the order in which tensors are drawn.  Values are drawn in
fp32 and, for bf16 workloads, rounded to bf16 with round-to-nearest-even; the
bf16 tensors are returned as uint16 bit patterns.

Workload recipes (sizes and value distributions of the pages' workloads; the
pages' own datasets (the Pile, HG38, YouTubeMix, SC09) are not available and
these tensors stand in for them):

* ``default`` -- x, B, C, z ~ N(0, 1); raw delta = 0.5 * N(0, 1); A[d, n] =
  -(n + 1) (the S4D-real style initialisation of A, with A = -exp(A_log));
  D = 1; the delta bias is chosen per channel so that softplus(bias) is
  log-uniform in [1e-3, 1e-1], i.e. bias = log(expm1(v)), log10 v ~ U(-3, -1).
* ``conv`` (the depthwise convolution before the scan) -- x ~ N(0, 1) as above; weight and bias
  ~ U(-1/sqrt(K), 1/sqrt(K)), the default initialisation range of a depthwise Conv1d whose
  fan-in is the kernel width K; an initial state, when asked for, ~ N(0, 1).
* ``ssd`` (the Mamba-2 SSD layer: heads of headdim channels, one scalar A per head, B and C per
  group of heads) -- x, B, C, z ~ N(0, 1); raw dt = 0.5 * N(0, 1) per (step, head); dt bias as
  in ``default``, per head; A_h = -U(1, 16) per head; D = 1 per head.  The pages give the layer's
  shapes (headdim 64, d_state 128, expand 2) but no initialisation, so these ranges are a choice:
  decays exp(dt A) between about 0.2 and 1 per step.
* ``genomics`` -- a one-hot 4-symbol alphabet (s_t ~ U{0..3}) projected by a
  seeded (4, dim) matrix W ~ N(0, 0.5^2), so x[b, t, :] = W[s_t, :]; delta is
  passed directly (no softplus, no bias) and is log-uniform in [1e-4, 1e-1];
  B, C, z ~ N(0, 1); D = 1; A[d, n] = -(n + 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# Stream ids: one Philox key per (seed, tensor).
_TENSOR_IDS = {"x": 1, "delta": 2, "B": 3, "C": 4, "z": 5, "bias": 6, "symbols": 7, "W": 8, "conv_w": 9,
               "conv_b": 10, "conv_state": 11, "A": 12, "state": 13}

_CHUNK = 1 << 24  # elements per draw; bounds temporary memory for the 1M-step workload


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "scan" or "decode"
    batch: int
    dim: int
    dstate: int
    dtype: str                # "f32" or "bf16": storage type of x, delta, B, C, z, y
    seed: int
    seqlen: int = 0           # scan length, or number of decode steps
    recipe: str = "default"
    delta_softplus: bool = True
    has_bias: bool = True
    has_z: bool = True
    has_D: bool = True
    note: str = field(default="", compare=False)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "scan", batch=1, seqlen=64, dim=16, dstate=4, dtype="f32", seed=61000,
                     note="tiny fp32 scan; the oracle finishes in milliseconds"),
    "mamba130m": Workload("mamba130m", "scan", batch=8, seqlen=2048, dim=1536, dstate=16, dtype="bf16",
                          seed=61001, note="Mamba-130M-shaped layer scan: d_inner = 2 x 768"),
    "mamba2p8b": Workload("mamba2p8b", "scan", batch=4, seqlen=2048, dim=5120, dstate=16, dtype="bf16",
                          seed=61002, note="Mamba-2.8B-shaped layer scan: d_inner = 2 x 2560"),
    "genomics": Workload("genomics", "scan", batch=1, seqlen=1 << 20, dim=256, dstate=16, dtype="f32",
                         seed=61003, recipe="genomics", delta_softplus=False, has_bias=False,
                         note="1M-step DNA-shaped fp32 scan"),
    "decode": Workload("decode", "decode", batch=64, seqlen=256, dim=5120, dstate=16, dtype="bf16",
                       seed=61004, note="256 single-token decode steps, state (64, 5120, 16) fp32"),
}


def _rng(seed: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=(int(seed) << 8) | _TENSOR_IDS[tensor]))


def _normal(seed: int, tensor: str, shape, scale: float = 1.0) -> np.ndarray:
    g = _rng(seed, tensor)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            out[s:e] *= np.float32(scale)
    return out.reshape(shape)


def _log_uniform(seed: int, tensor: str, shape, lo_exp: float, hi_exp: float) -> np.ndarray:
    """10**U(lo_exp, hi_exp), element-wise, fp32."""
    g = _rng(seed, tensor)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        u = g.uniform(lo_exp, hi_exp, e - s)
        out[s:e] = np.power(10.0, u)
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, round-to-nearest-even; NaN stays a (quiet) NaN.  Returns uint16 bits."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def params(dim: int, dstate: int, seed: int, has_bias: bool = True, has_D: bool = True):
    """A (dim, N) fp32, D (dim,) fp32 or None, delta_bias (dim,) fp32 or None."""
    A = -np.tile(np.arange(1, dstate + 1, dtype=np.float32), (dim, 1))
    D = np.ones(dim, np.float32) if has_D else None
    bias = None
    if has_bias:
        v = _log_uniform(seed, "bias", (dim,), -3.0, -1.0).astype(np.float64)
        bias = np.log(np.expm1(v)).astype(np.float32)
    return A, D, bias


def scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str = "f32", seed: int = 0,
                recipe: str = "default", has_bias: bool = True, has_z: bool = True,
                has_D: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of one scan call: x, delta, z (batch, seqlen, dim); B, C (batch, seqlen, dstate)
    in the storage type; A (dim, dstate), D (dim,), delta_bias (dim,) in fp32."""
    shp, shn = (batch, seqlen, dim), (batch, seqlen, dstate)
    if recipe == "default":
        x = _normal(seed, "x", shp)
        delta = _normal(seed, "delta", shp, 0.5)
    elif recipe == "genomics":
        g = _rng(seed, "symbols")
        sym = g.integers(0, 4, size=(batch, seqlen), dtype=np.int8)
        W = _normal(seed, "W", (4, dim), 0.5)
        x = W[sym]
        delta = _log_uniform(seed, "delta", shp, -4.0, -1.0)
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    B = _normal(seed, "B", shn)
    C = _normal(seed, "C", shn)
    z = _normal(seed, "z", shp) if has_z else None
    A, D, bias = params(dim, dstate, seed, has_bias and recipe == "default", has_D)
    return {"x": _store(x, dtype), "delta": _store(delta, dtype), "B": _store(B, dtype), "C": _store(C, dtype),
            "z": None if z is None else _store(z, dtype), "A": A, "D": D, "delta_bias": bias}


def _uniform(seed: int, tensor: str, shape, lo: float, hi: float) -> np.ndarray:
    return _rng(seed, tensor).uniform(lo, hi, int(np.prod(shape))).astype(np.float32).reshape(shape)


def conv_inputs(batch: int, seqlen: int, dim: int, width: int, dtype: str = "f32", seed: int = 0,
                has_bias: bool = True, has_init: bool = False) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of one depthwise causal convolution: x (batch, seqlen, dim) in the storage type;
    weight (dim, width) and bias (dim,) in fp32; init (batch, dim, width-1) in the storage type
    or None."""
    bound = 1.0 / np.sqrt(width)
    x = _normal(seed, "x", (batch, seqlen, dim))
    w = _uniform(seed, "conv_w", (dim, width), -bound, bound)
    b = _uniform(seed, "conv_b", (dim,), -bound, bound) if has_bias else None
    init = _normal(seed, "conv_state", (batch, dim, width - 1)) if has_init else None
    return {"x": _store(x, dtype), "weight": w, "bias": b, "init": None if init is None else _store(init, dtype)}


@dataclass(frozen=True)
class SsdWorkload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    seed: int
    note: str = field(default="", compare=False)


SSD_WORKLOADS: Dict[str, SsdWorkload] = {
    "mamba2_layer": SsdWorkload("mamba2_layer", batch=1, seqlen=1024, nheads=64, headdim=64, dstate=128, ngroups=1,
                                seed=61010, note="the Mamba2 layer example: d_model 2048, expand 2, headdim 64, "
                                "d_state 128, input (1, 1024, 2048)"),
    "mamba2_layer_b8": SsdWorkload("mamba2_layer_b8", batch=8, seqlen=2048, nheads=64, headdim=64, dstate=128,
                                   ngroups=1, seed=61011, note="the same layer on 8 sequences of 2048 steps"),
}


def ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int = 1, seed: int = 0,
               has_z: bool = True, has_D: bool = True, has_bias: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of one SSD layer call (bf16 storage): x, z (batch, seqlen, nheads, headdim); dt
    (batch, seqlen, nheads); B, C (batch, seqlen, ngroups, dstate) as uint16 bf16 bits; A, D,
    dt_bias (nheads,) fp32."""
    shx = (batch, seqlen, nheads, headdim)
    x = _normal(seed, "x", shx)
    dt = _normal(seed, "delta", (batch, seqlen, nheads), 0.5)
    B = _normal(seed, "B", (batch, seqlen, ngroups, dstate))
    C = _normal(seed, "C", (batch, seqlen, ngroups, dstate))
    z = _normal(seed, "z", shx) if has_z else None
    A = -_uniform(seed, "A", (nheads,), 1.0, 16.0)
    D = np.ones(nheads, np.float32) if has_D else None
    bias = None
    if has_bias:
        v = _log_uniform(seed, "bias", (nheads,), -3.0, -1.0).astype(np.float64)
        bias = np.log(np.expm1(v)).astype(np.float32)
    return {"x": _store(x, "bf16"), "dt": _store(dt, "bf16"), "B": _store(B, "bf16"), "C": _store(C, "bf16"),
            "z": None if z is None else _store(z, "bf16"), "A": A, "D": D, "dt_bias": bias}


def long_scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, period: int, dtype: str = "bf16",
                     seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """A scan too long to draw element by element on the host: x, delta and z are one
    (batch, period, dim) block that the sequence repeats along time (see repeat_in_time); B and C
    are drawn for every one of the seqlen steps; A, D and the bias as scan_inputs draws them."""
    t = scan_inputs(batch, period, dim, dstate, dtype, seed)
    t["B"] = _store(_normal(seed, "B", (batch, seqlen, dstate)), dtype)
    t["C"] = _store(_normal(seed, "C", (batch, seqlen, dstate)), dtype)
    return t


def long_ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, period: int,
                    seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """An SSD layer call too long to draw element by element on the host: x and z are one
    (batch, period, nheads, headdim) block repeated along time; dt, B and C (one group) are drawn
    for every step; A, D and dt_bias as ssd_inputs draws them."""
    t = ssd_inputs(batch, period, nheads, headdim, dstate, 1, seed)
    t["dt"] = _store(_normal(seed, "delta", (batch, seqlen, nheads), 0.5), "bf16")
    t["B"] = _store(_normal(seed, "B", (batch, seqlen, 1, dstate)), "bf16")
    t["C"] = _store(_normal(seed, "C", (batch, seqlen, 1, dstate)), "bf16")
    return t


def long_decode_inputs(batch: int, dim: int, dstate: int, period: int,
                       seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """One decode step over a state too large to draw element by element on the host: the state
    is one (period, dim, dstate) fp32 block repeated along the batch (state_block); x, delta, z
    (batch, dim) and B, C (batch, dstate) are drawn in full, bf16; A, D and the bias as
    scan_inputs draws them."""
    t = scan_inputs(batch, 1, dim, dstate, "bf16", seed)
    out = {k: (v[:, 0] if k in ("x", "delta", "z", "B", "C") else v) for k, v in t.items()}
    out["state_block"] = _normal(seed, "state", (period, dim, dstate), 0.5)
    return out


def long_ssd_decode_inputs(batch: int, nheads: int, headdim: int, dstate: int, period: int,
                           seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """One SSD decode step over a state too large to draw element by element on the host: the
    state is one (period, nheads, headdim, dstate) fp32 block repeated along the batch
    (state_block); x, z (batch, nheads, headdim), dt (batch, nheads) and B, C (batch, 1, dstate)
    are drawn in full, bf16; A, D and dt_bias as ssd_inputs draws them."""
    t = ssd_inputs(batch, 1, nheads, headdim, dstate, 1, seed)
    out = {k: (v[:, 0] if k in ("x", "z", "dt", "B", "C") else v) for k, v in t.items()}
    out["state_block"] = _normal(seed, "state", (period, nheads, headdim, dstate), 0.5)
    return out


def repeat_in_time(block: np.ndarray, seqlen: int) -> np.ndarray:
    """block (batch, period, ...) repeated along axis 1 and cut to seqlen steps."""
    reps = -(-seqlen // block.shape[1])
    return np.ascontiguousarray(np.concatenate([block] * reps, axis=1)[:, :seqlen])


def ssd_workload_inputs(w: SsdWorkload) -> Dict[str, Optional[np.ndarray]]:
    return ssd_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.seed)


def workload_inputs(w: Workload) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a named workload.  For a decode workload the per-step tensors are drawn like a
    scan of ``seqlen`` steps and stored step-major: x, delta, z (steps, batch, dim); B, C
    (steps, batch, dstate); each step is then one contiguous slab."""
    if w.kind == "scan":
        return scan_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.dtype, w.seed, w.recipe,
                           w.has_bias, w.has_z, w.has_D)
    t = scan_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.dtype, w.seed, w.recipe, w.has_bias, w.has_z, w.has_D)
    for k in ("x", "delta", "z", "B", "C"):
        if t[k] is not None:
            t[k] = np.ascontiguousarray(np.swapaxes(t[k], 0, 1))
    return t
