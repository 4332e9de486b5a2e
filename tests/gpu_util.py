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


def sample_channels(batch, dim, n, seed=0):
    """Channels to compare at full size: block edges, the ragged end, and random ones."""
    g = np.random.default_rng(seed)
    picks = set()
    for b in {0, batch - 1}:
        for d in {0, 1, 63, 64, dim - 1, dim // 2, min(dim - 1, 127)}:
            picks.add((b, d))
    while len(picks) < n:
        picks.add((int(g.integers(batch)), int(g.integers(dim))))
    sb, sd = zip(*sorted(picks))
    return np.array(sb), np.array(sd)
