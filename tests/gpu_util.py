"""Helpers for the GPU parity tests: move seeded numpy inputs to the device, call the HIP path,
and compare with the fp64 oracle under the tolerance rule

    max |y - y_ref| <= tol * max |y_ref|,  tol = 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs),

applied separately to y and to the final state."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, device="cuda"):
    """numpy float32 -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor; None -> None."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t):
    """float32 result as float64 numpy; bf16 result widened exactly."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err, err, scale


def assert_close(got, ref, tol, what):
    r, err, scale = rel_err(got, ref)
    say(f"  {what}: max err {err:.3e}, max |ref| {scale:.3e}, ratio {r:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert r <= tol, f"{what}: max|err|/max|ref| = {r:.3e} > {tol:.0e}"


def scan_on_gpu(t, softplus, device="cuda", **kw):
    import selective_state_space_61_amd as ssm
    d = {k: to_dev(v, device) for k, v in t.items()}
    y, st = ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                             delta_bias=d["delta_bias"], delta_softplus=softplus, **kw)
    torch.cuda.synchronize()
    return y, st, d


class Worst:
    """max |got - ref| and max |ref| gathered over the pieces of one tensor, so that the tolerance
    rule applies to the whole tensor even when the oracle computes it piece by piece."""

    def __init__(self, what):
        self.what, self.err, self.scale, self.finite, self.count = what, 0.0, 0.0, True, 0

    def add(self, got, ref):
        if ref.size == 0:
            return
        assert got.shape == ref.shape, f"{self.what}: shape {got.shape} != {ref.shape}"
        self.err = max(self.err, float(np.max(np.abs(got - ref))))
        self.scale = max(self.scale, float(np.max(np.abs(ref))))
        self.finite = self.finite and bool(np.all(np.isfinite(got)))
        self.count += ref.size

    def check(self, tol):
        r = self.err / self.scale if self.scale > 0 else self.err
        say(f"  {self.what}: {self.count} elements, max err {self.err:.3e}, max |ref| {self.scale:.3e}, "
            f"ratio {r:.3e} (tol {tol:.0e})")
        assert self.finite, f"{self.what}: non-finite values"
        assert r <= tol, f"{self.what}: max|err|/max|ref| = {r:.3e} > {tol:.0e}"


def host_f32(t):
    """A device tensor as a float32 numpy array (bf16 widened exactly)."""
    return t.float().cpu().numpy()


def scan_whole(o, t, y, st, softplus, tol, what, block=256, threads=16):
    """Every element of y (batch, L, dim) and of last_state (batch, dim, N) against the oracle,
    which runs on blocks of channels of one batch row at a time (to bound host memory); the
    tolerance applies to the maximum over the whole tensor."""
    yh, sh = host_f32(y), host_f32(st)
    batch, L, dim = yh.shape
    wy, ws = Worst(f"{what} y (whole tensor)"), Worst(f"{what} last_state (whole tensor)")
    for b in range(batch):
        for d0 in range(0, dim, block):
            d1 = min(dim, d0 + block)
            sd = np.arange(d0, d1, dtype=np.int64)
            sb = np.full(sd.size, b, np.int64)
            y_ref, st_ref = o.scan_channels(t["x"], t["delta"], t["A"], t["B"], t["C"], sb, sd, D=t["D"], z=t["z"],
                                            delta_bias=t["delta_bias"], delta_softplus=softplus, nthreads=threads)
            wy.add(yh[b, :, d0:d1].T.astype(np.float64), y_ref)
            ws.add(sh[b, d0:d1].astype(np.float64), st_ref)
    wy.check(tol)
    ws.check(tol)
