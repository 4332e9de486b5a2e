"""Parity of the HIP backward scan (through the C ABI) with the fp64 adjoint oracle.

Every gradient is compared element by element under the scan's tolerance rule (max |g - g_ref|
<= tol * max |g_ref| per tensor; tol 1e-4 for fp32 storage, 2e-2 for bf16 storage, where dx,
ddelta, dz, dB and dC are stored in bf16).  At the 130M-shaped size every gradient is compared
over the whole tensor; the oracle runs there on blocks of channels, whose per-channel gradients
are exact on their own because channels do not interact, and whose dB and dC add up to the sums
over all channels."""
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


def bwd_gpu(t, dy, softplus, zoh=False, layout="auto"):
    import selective_state_space_61_amd as ssm
    d = {k: to_dev(v) for k, v in t.items()}
    g = ssm.ssm_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], to_dev(dy), D=d["D"], z=d["z"],
                         delta_bias=d["delta_bias"], delta_softplus=softplus, zoh=zoh, layout=layout)
    torch.cuda.synchronize()
    return g


def compare(o, t, dy, dtype, softplus, what, zoh=False, layout="auto"):
    say(f"[case] {what} ({layout})")
    g = bwd_gpu(t, dy, softplus, zoh, layout)
    dy64 = W.bf16_bits_to_f32(dy).astype(np.float64) if dy.dtype == np.uint16 else dy.astype(np.float64)
    ref = o.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dy64, D=t["D"], z=t["z"],
                     delta_bias=t["delta_bias"], delta_softplus=softplus, zoh=zoh)
    for k, r in ref.items():
        if r is None:
            assert g[k] is None
            continue
        tol = TOL[dtype] if k in ("dx", "ddelta", "dz", "dB", "dC") else TOL["f32"] if dtype == "f32" else 1e-3
        assert_close(to_host(g[k]), r, tol, f"{what} {k}")
    return g


@pytest.mark.parametrize("zoh", [False, True], ids=["delta_b", "zoh"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64])
def test_dstates(o, dtype, N, zoh):
    t = W.scan_inputs(2, 70, 96, N, dtype, seed=N + 300)
    compare(o, t, dy_for((2, 70, 96), dtype, N), dtype, True, f"bwd N={N} {dtype} zoh={zoh}", zoh=zoh)


@pytest.mark.parametrize("N", [16, 32, 64])
@pytest.mark.parametrize("shape", [(1, 17, 13), (2, 45, 130), (1, 3, 64)])
def test_zoh_ragged(o, N, shape):
    """Exact-ZOH backward on ragged shapes (L not a multiple of the chunk, dim not of 64)."""
    batch, L, dim = shape
    t = W.scan_inputs(batch, L, dim, N, "f32", seed=L * 7 + dim + N)
    compare(o, t, dy_for((batch, L, dim), "f32", L + N), "f32", True, f"bwd zoh ragged {shape} N={N}", zoh=True)


@pytest.mark.parametrize("variant", ["genomics_steps", "softplus_off_no_bias", "bare"])
def test_zoh_variants(o, variant):
    """Exact-ZOH backward: small steps (dt A down to ~1e-4, where phi's derivative in A takes the
    series), softplus off without a bias, and no z / D / bias."""
    if variant == "genomics_steps":
        t = W.scan_inputs(1, 200, 64, 16, "f32", seed=91, recipe="genomics", has_bias=False)
        softplus = False
    else:
        softplus = False
        t = W.scan_inputs(2, 60, 72, 16, "f32", seed=92, has_bias=False, has_z=variant != "bare",
                          has_D=variant != "bare")
        t["delta"] = np.abs(t["delta"])
    compare(o, t, dy_for(t["x"].shape, "f32", 93), "f32", softplus, f"bwd zoh {variant}", zoh=True)


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


@pytest.mark.parametrize("layout", ["channel_lanes", "state_rows"])
def test_deterministic_and_empty(o, layout):
    """Channel lanes: every gradient is bit-identical between runs.  State rows: all but dB and dC
    (whose channel sums are added with atomics in a run-dependent order)."""
    import selective_state_space_61_amd as ssm
    t = W.scan_inputs(2, 64, 128, 16, "bf16", seed=5)
    dy = dy_for((2, 64, 128), "bf16", 6)
    g1, g2 = bwd_gpu(t, dy, True, layout=layout), bwd_gpu(t, dy, True, layout=layout)
    for k in g1:
        if g1[k] is not None and not (layout == "state_rows" and k in ("dB", "dC")):
            assert torch.equal(g1[k], g2[k]), f"{k} differs between runs"
    # seqlen 0: nothing flows back and the parameter gradients are zero
    t0 = W.scan_inputs(2, 0, 32, 16, "f32", seed=1)
    g0 = bwd_gpu(t0, np.zeros((2, 0, 32), np.float32), True)
    assert torch.count_nonzero(g0["dA"]).item() == 0 and torch.count_nonzero(g0["dD"]).item() == 0
    assert torch.count_nonzero(g0["ddelta_bias"]).item() == 0


@pytest.mark.parametrize("shape", [(1, 1, 8), (1, 31, 40), (2, 33, 56), (3, 100, 200), (2, 64, 144), (1, 96, 48),
                                   (2, 65, 16)])
def test_state_rows_shapes(o, shape):
    """The state-row backward (bf16, dstate 16): sequences that are not whole 32-step chunks, channel
    counts that are not whole 48-channel workgroups (1, 2 or 3 scan waves), several batch rows."""
    batch, L, dim = shape
    t = W.scan_inputs(batch, L, dim, 16, "bf16", seed=L * 5 + dim)
    compare(o, t, dy_for((batch, L, dim), "bf16", L + 2 * dim), "bf16", True, f"bwd state rows {shape}",
            layout="state_rows")


@pytest.mark.parametrize("variant", ["no_z", "no_D", "no_bias", "softplus_off", "bare"])
def test_state_rows_variants(o, variant):
    softplus = variant not in ("softplus_off", "bare")
    t = W.scan_inputs(2, 70, 96, 16, "bf16", seed=79, has_z=variant not in ("no_z", "bare"),
                      has_D=variant not in ("no_D", "bare"), has_bias=softplus and variant != "no_bias")
    if not softplus:
        t["delta"] = t["delta"] & np.uint16(0x7FFF)
    compare(o, t, dy_for((2, 70, 96), "bf16", 80), "bf16", softplus, f"bwd state rows {variant}",
            layout="state_rows")


def test_state_rows_refusals():
    """Where the state rows do not apply, asking for them is an error before any launch (auto
    takes the channel lanes there, which the other tests cover)."""
    import selective_state_space_61_amd as ssm
    cases = [("f32", 2, 40, 48, 16, False), ("bf16", 2, 40, 44, 16, False), ("bf16", 2, 40, 48, 8, False),
             ("bf16", 2, 40, 48, 16, True)]
    for dtype, batch, L, dim, N, zoh in cases:
        t = W.scan_inputs(batch, L, dim, N, dtype, seed=3)
        with pytest.raises(ssm.SsmError, match="STATE_ROWS"):
            bwd_gpu(t, dy_for((batch, L, dim), dtype, 4), True, zoh=zoh, layout="state_rows")


def test_mid_size_every_gradient(o):
    """Several channel blocks, several 16-step chunks and a ragged tail, bf16."""
    t = W.scan_inputs(2, 301, 200, 16, "bf16", seed=61001)
    compare(o, t, dy_for((2, 301, 200), "bf16", 9), "bf16", True, "bwd mid-size (2, 301, 200, 16) bf16")


def bwd_oracle_blocks(o, t, dy64, softplus, block=128, threads=16):
    """The adjoint oracle at a large size, run on blocks of channels in parallel threads (each
    call is independent; ctypes releases the GIL).  Per-channel gradients are concatenated; dB and
    dC, which sum over channels, are the sums of the blocks' sums."""
    from concurrent.futures import ThreadPoolExecutor
    dim = t["x"].shape[2]
    blocks = [(d0, min(dim, d0 + block)) for d0 in range(0, dim, block)]

    def one(r):
        d0, d1 = r
        sl = lambda a: None if a is None else np.ascontiguousarray(a[..., d0:d1])
        pv = lambda a: None if a is None else np.ascontiguousarray(a[d0:d1])
        return o.scan_bwd(sl(t["x"]), sl(t["delta"]), pv(t["A"]), t["B"], t["C"], sl(dy64), D=pv(t["D"]),
                          z=sl(t["z"]), delta_bias=pv(t["delta_bias"]), delta_softplus=softplus)

    with ThreadPoolExecutor(max(1, min(threads, len(blocks)))) as ex:
        parts = list(ex.map(one, blocks))
    out = {}
    for k in ("dx", "ddelta", "dz"):
        out[k] = None if parts[0][k] is None else np.concatenate([p[k] for p in parts], axis=2)
    for k in ("dA", "dD", "ddelta_bias"):
        out[k] = None if parts[0][k] is None else np.concatenate([p[k] for p in parts], axis=0)
    for k in ("dB", "dC"):
        acc = np.zeros_like(parts[0][k])
        for p in parts:
            acc += p[k]
        out[k] = acc
    return out


def test_full_mamba130m_every_gradient(o):
    """The 130M-shaped layer (8 x 2048 x 1536, N 16, bf16): all eight gradients, every element,
    against the adjoint oracle (dB and dC are the sums over all 1536 channels that the
    channel-block partials and the reduce kernel produce)."""
    w = W.WORKLOADS["mamba130m"]
    say(f"[case] backward at the 130M shape, every gradient, every element")
    t = W.workload_inputs(w)
    dy = dy_for((w.batch, w.seqlen, w.dim), "bf16", 61)
    g = bwd_gpu(t, dy, True)
    dy64 = W.bf16_bits_to_f32(dy).astype(np.float64)
    ref = bwd_oracle_blocks(o, t, dy64, True)
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        assert_close(to_host(g[k]), ref[k], TOL["bf16"], f"mamba130m {k} (whole tensor)")
    for k in ("dA", "dD", "ddelta_bias"):
        assert_close(to_host(g[k]), ref[k], 1e-3, f"mamba130m {k} (whole tensor)")
