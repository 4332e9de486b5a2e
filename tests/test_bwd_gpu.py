"""Parity of the HIP backward scan (through the C ABI) with the fp64 adjoint oracle.

Every gradient is compared element by element under the scan's tolerance rule (max |g - g_ref|
<= tol * max |g_ref| per tensor; tol 1e-4 for fp32 storage, 2e-2 for bf16 storage, where dx,
ddelta, dz, dB and dC are stored in bf16).  At the 130M-shaped size the per-channel gradients
(dx, ddelta, dz, dA, dD, ddelta_bias) of sampled channels are compared with the oracle run on
those channels alone, which is exact for them because channels do not interact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, assert_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_61_amd as ssm
    ssm.load_library()
    say(f"\n[gpu] {torch.cuda.get_device_name(0)}; library {ssm.LIBRARY}")


def dy_for(shape, dtype, seed):
    g = np.random.default_rng(seed)
    dy = g.standard_normal(shape).astype(np.float32)
    return W.f32_to_bf16_bits(dy) if dtype == "bf16" else dy


def bwd_gpu(t, dy, softplus):
    import selective_state_space_61_amd as ssm
    d = {k: to_dev(v) for k, v in t.items()}
    g = ssm.ssm_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], to_dev(dy), D=d["D"], z=d["z"],
                         delta_bias=d["delta_bias"], delta_softplus=softplus)
    torch.cuda.synchronize()
    return g


def compare(o, t, dy, dtype, softplus, what):
    say(f"[case] {what}")
    g = bwd_gpu(t, dy, softplus)
    dy64 = W.bf16_bits_to_f32(dy).astype(np.float64) if dy.dtype == np.uint16 else dy.astype(np.float64)
    ref = o.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dy64, D=t["D"], z=t["z"],
                     delta_bias=t["delta_bias"], delta_softplus=softplus)
    for k, r in ref.items():
        if r is None:
            assert g[k] is None
            continue
        tol = TOL[dtype] if k in ("dx", "ddelta", "dz", "dB", "dC") else TOL["f32"] if dtype == "f32" else 1e-3
        assert_close(to_host(g[k]), r, tol, f"{what} {k}")
    return g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
def test_dstates(o, dtype, N):
    t = W.scan_inputs(2, 70, 96, N, dtype, seed=N + 300)
    compare(o, t, dy_for((2, 70, 96), dtype, N), dtype, True, f"bwd N={N} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 100, 200, 16), (1, 17, 13, 16), (2, 1, 64, 16), (1, 33, 130, 4),
                                   (2, 48, 7, 8)])
def test_ragged_shapes(o, dtype, shape):
    batch, L, dim, N = shape
    t = W.scan_inputs(batch, L, dim, N, dtype, seed=L * 3 + dim)
    compare(o, t, dy_for((batch, L, dim), dtype, L + dim), dtype, True, f"bwd ragged {shape} {dtype}")


@pytest.mark.parametrize("variant", ["no_z", "no_D", "no_bias", "softplus_off", "bare"])
def test_variants(o, variant):
    softplus = variant not in ("softplus_off", "bare")
    t = W.scan_inputs(2, 50, 72, 16, "f32", seed=77, has_z=variant not in ("no_z", "bare"),
                      has_D=variant not in ("no_D", "bare"), has_bias=softplus and variant != "no_bias")
    if not softplus:
        t["delta"] = np.abs(t["delta"])
    compare(o, t, dy_for((2, 50, 72), "f32", 78), "f32", softplus, f"bwd variant {variant}")


def test_deterministic_and_empty(o):
    import selective_state_space_61_amd as ssm
    t = W.scan_inputs(2, 64, 128, 16, "bf16", seed=5)
    dy = dy_for((2, 64, 128), "bf16", 6)
    g1, g2 = bwd_gpu(t, dy, True), bwd_gpu(t, dy, True)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), f"{k} differs between runs"
    # seqlen 0: nothing flows back and the parameter gradients are zero
    t0 = W.scan_inputs(2, 0, 32, 16, "f32", seed=1)
    g0 = bwd_gpu(t0, np.zeros((2, 0, 32), np.float32), True)
    assert torch.count_nonzero(g0["dA"]).item() == 0 and torch.count_nonzero(g0["dD"]).item() == 0
    assert torch.count_nonzero(g0["ddelta_bias"]).item() == 0


def test_mid_size_every_gradient(o):
    """Several channel blocks, several 16-step chunks and a ragged tail, bf16."""
    t = W.scan_inputs(2, 301, 200, 16, "bf16", seed=61001)
    compare(o, t, dy_for((2, 301, 200), "bf16", 9), "bf16", True, "bwd mid-size (2, 301, 200, 16) bf16")


def test_full_mamba130m_sampled_channels(o):
    """The 130M-shaped layer (8 x 2048 x 1536, N 16, bf16): per-channel gradients of sampled
    channels against the oracle run on those channels alone."""
    w = W.WORKLOADS["mamba130m"]
    t = W.workload_inputs(w)
    dy = dy_for((w.batch, w.seqlen, w.dim), "bf16", 61)
    g = bwd_gpu(t, dy, True)
    chans = np.array([0, 1, 63, 64, 767, 1000, 1535])
    sub = {k: (v[..., chans] if k in ("x", "delta", "z") else v[chans] if k in ("A", "D", "delta_bias") else v)
           for k, v in t.items()}
    dy_sub = W.bf16_bits_to_f32(dy[..., chans]).astype(np.float64)
    ref = o.scan_bwd(np.ascontiguousarray(sub["x"]), np.ascontiguousarray(sub["delta"]), sub["A"], sub["B"],
                     sub["C"], dy_sub, D=sub["D"], z=np.ascontiguousarray(sub["z"]), delta_bias=sub["delta_bias"],
                     delta_softplus=True)
    for k in ("dx", "ddelta", "dz"):
        assert_close(to_host(g[k])[..., chans], ref[k], TOL["bf16"], f"mamba130m {k} sampled")
    for k in ("dA", "dD", "ddelta_bias"):
        assert_close(to_host(g[k])[chans], ref[k], 1e-3, f"mamba130m {k} sampled")
