"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by element.

Every test compares every output element.  The full-size workloads run in the launch
configuration that bench.py times (automatic launch shape); the oracle computes them in blocks of
channels, and the tolerance rule max|y - y_ref| <= tol * max|y_ref| applies to the maximum over
the whole tensor, separately for y and for the final state."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, assert_close, say, scan_on_gpu, scan_whole, to_dev, to_host

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))


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


def run_and_compare(o, t, dtype, softplus, what, **kw):
    say(f"[case] {what}")
    y, st, _ = scan_on_gpu(t, softplus, **kw)
    y_ref, st_ref = o.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           delta_bias=t["delta_bias"], delta_softplus=softplus, nthreads=THREADS)
    assert_close(to_host(y), y_ref, TOL[dtype], f"{what} y")
    assert_close(to_host(st), st_ref, TOL[dtype], f"{what} last_state")
    return y, st


def test_tiny_workload(o):
    w = W.WORKLOADS["tiny"]
    run_and_compare(o, W.workload_inputs(w), w.dtype, w.delta_softplus, "tiny fp32 (1, 64, 16, N=4)")


@pytest.mark.parametrize("variant", ["no_z", "no_D", "no_bias", "softplus_off", "bf16", "bare"])
def test_tiny_variants(o, variant):
    dtype = "bf16" if variant == "bf16" else "f32"
    softplus = variant not in ("softplus_off", "bare")
    t = W.scan_inputs(1, 64, 16, 4, dtype, seed=61000, has_z=variant not in ("no_z", "bare"),
                      has_D=variant not in ("no_D", "bare"), has_bias=softplus and variant != "no_bias")
    if not softplus:
        # the step is used as given: keep it positive (|raw|), as softplus would
        t["delta"] = np.abs(t["delta"]) if dtype == "f32" else t["delta"] & np.uint16(0x7FFF)
    run_and_compare(o, t, dtype, softplus, f"tiny variant {variant}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 100, 200, 16), (2, 97, 136, 16), (1, 33, 64, 16), (2, 65, 1, 16),
                                   (4, 160, 130, 4), (1, 1, 70, 16)])
def test_tiles_and_ragged_tails(o, dtype, shape):
    batch, L, dim, N = shape
    t = W.scan_inputs(batch, L, dim, N, dtype, seed=hash(shape) % 1000)
    run_and_compare(o, t, dtype, True, f"ragged {shape} {dtype}")


CHAIN_CASES = [(n, c) for n in (1, 2, 4, 8, 16, 32, 64) for c in (1, 2, 4, 8, 16) if c <= n and n % c == 0
               and n // c <= 8]


@pytest.mark.parametrize("N,chains", CHAIN_CASES)
def test_dstate_and_chains_per_lane(o, N, chains):
    dtype = "bf16" if (N + chains) % 2 else "f32"
    t = W.scan_inputs(2, 70, 96, N, dtype, seed=N * 31 + chains)
    for chunk in ((16, 32) if N // chains <= 4 else (16,)):
        run_and_compare(o, t, dtype, True, f"N={N} chains={chains} chunk={chunk} {dtype}", chains_per_lane=chains,
                        chunk_steps=chunk)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,segments", [((3, 100, 200, 16), 1), ((2, 47, 136, 16), 1), ((1, 1000, 72, 16), 5),
                                            ((2, 333, 64, 8), 3)])
def test_chunk_lengths(o, chunk, dtype, shape, segments):
    batch, L, dim, N = shape
    t = W.scan_inputs(batch, L, dim, N, dtype, seed=L + chunk)
    run_and_compare(o, t, dtype, True, f"chunk={chunk} {shape} segments={segments} {dtype}", chunk_steps=chunk,
                    segments=segments)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("L", [16, 17, 32, 33, 48, 96, 97])
def test_whole_and_odd_chunk_counts(o, chunk, L):
    # the IO waves keep the tiles of the next two chunks in two register slots and run their loop
    # two iterations at a time: whole chunk counts of both parities, with and without a tail
    t = W.scan_inputs(2, L, 64, 16, "bf16", seed=L * 7 + chunk)
    run_and_compare(o, t, "bf16", True, f"L={L} chunk={chunk}", chunk_steps=chunk, segments=1)


@pytest.mark.parametrize("segments", [1, 3])
def test_channel_independence_bitwise(o, segments):
    # changing the inputs of one channel changes that channel's outputs and nothing else, bit for
    # bit: no lane, tile or segment mixes channels (B and C are shared, x / delta / z are not)
    t = W.scan_inputs(2, 150, 136, 16, "bf16", seed=17)
    y0, s0, _ = scan_on_gpu(t, True, segments=segments)
    t2 = dict(t)
    d0 = 70
    for k in ("x", "delta", "z"):
        if t[k] is None:
            continue
        v = t[k].copy()
        v[:, :, d0] = v[:, :, d0] ^ np.uint16(0x0040)
        t2[k] = v
    y1, s1, _ = scan_on_gpu(t2, True, segments=segments)
    say(f"[case] channel independence, segments={segments}")
    keep = [d for d in range(136) if d != d0]
    assert torch.equal(y0[:, :, keep], y1[:, :, keep]), "another channel's y changed"
    assert torch.equal(s0[:, keep], s1[:, keep]), "another channel's state changed"
    assert not torch.equal(y0[:, :, d0], y1[:, :, d0]), "the perturbed channel did not change"


@pytest.mark.parametrize("t0", [0, 31, 77, 149])
def test_causality_bitwise(o, t0):
    # changing every input at step t0 leaves all outputs before t0 unchanged, bit for bit (tiles
    # are loaded chunks ahead; none of that may reach an earlier step)
    t = W.scan_inputs(2, 150, 72, 16, "bf16", seed=23)
    y0, _, _ = scan_on_gpu(t, True)
    t2 = dict(t)
    for k in ("x", "delta", "z", "B", "C"):
        v = t[k].copy()
        v[:, t0] = v[:, t0] ^ np.uint16(0x0040)
        t2[k] = v
    y1, _, _ = scan_on_gpu(t2, True)
    say(f"[case] causality, t0={t0}")
    assert torch.equal(y0[:, :t0], y1[:, :t0]), "an output before the perturbed step changed"
    assert not torch.equal(y0[:, t0], y1[:, t0]), "the perturbed step did not change"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [2, 3, 7, 16])
def test_split_sequence(o, dtype, segments):
    t = W.scan_inputs(1, 1000, 128, 16, dtype, seed=segments)
    y, st = run_and_compare(o, t, dtype, True, f"segments={segments} {dtype}", segments=segments)
    y1, st1, _ = scan_on_gpu(t, True, segments=1)
    say(f"  max |y(seg={segments}) - y(seg=1)| = {float((y.float() - y1.float()).abs().max()):.3e}")


def test_split_sequence_genomics_recipe(o):
    t = W.scan_inputs(1, 8192, 256, 16, "f32", seed=5, recipe="genomics", has_bias=False)
    run_and_compare(o, t, "f32", False, "genomics recipe L=8192, automatic segments")


def test_empty_and_degenerate(o):
    import selective_state_space_61_amd as ssm
    dev = "cuda"
    for dt in (torch.float32, torch.bfloat16):
        x = torch.empty(2, 0, 8, dtype=dt, device=dev)
        A = -torch.ones(8, 4, device=dev)
        BC = torch.empty(2, 0, 4, dtype=dt, device=dev)
        st = torch.full((2, 8, 4), 7.0, device=dev)
        y, st = ssm.ssm_scan_fwd(x, x, A, BC, BC, last_state=st)
        torch.cuda.synchronize()
        assert y.numel() == 0 and torch.all(st == 0), "seqlen 0 must give a zero last_state"
        x0 = torch.empty(0, 5, 8, dtype=dt, device=dev)
        y0, s0 = ssm.ssm_scan_fwd(x0, x0, A, torch.empty(0, 5, 4, dtype=dt, device=dev),
                                  torch.empty(0, 5, 4, dtype=dt, device=dev))
        assert y0.shape == (0, 5, 8) and s0.shape == (0, 8, 4)
    t = W.scan_inputs(3, 1, 5, 4, "f32", seed=3)
    run_and_compare(o, t, "f32", True, "seqlen 1")


def test_zero_step_keeps_state(o):
    """delta = 0 (softplus off, no bias): the state stays zero and y = D x SiLU(z)."""
    t = W.scan_inputs(2, 77, 96, 16, "f32", seed=8, has_bias=False)
    t["delta"] = np.zeros_like(t["delta"])
    y, st, _ = scan_on_gpu(t, False)
    assert torch.all(st == 0)
    x, z = t["x"].astype(np.float64), t["z"].astype(np.float64)
    ref = x * z / (1 + np.exp(-z))
    assert_close(to_host(y), ref, 1e-5, "delta=0 output")


def test_unaligned_views(o):
    """x / delta / z / y not 16-byte aligned: the element-by-element access path."""
    import selective_state_space_61_amd as ssm
    t = W.scan_inputs(2, 50, 72, 16, "f32", seed=9)
    d = {k: to_dev(v) for k, v in t.items()}

    def shifted(a):
        buf = torch.empty(a.numel() + 1, dtype=a.dtype, device=a.device)
        v = buf[1:].view(a.shape)
        v.copy_(a)
        return v
    y = shifted(torch.zeros_like(d["x"]))
    yy, st = ssm.ssm_scan_fwd(shifted(d["x"]), shifted(d["delta"]), d["A"], d["B"], d["C"], D=d["D"],
                              z=shifted(d["z"]), delta_bias=d["delta_bias"], delta_softplus=True, y=y)
    torch.cuda.synchronize()
    assert yy.data_ptr() % 16 != 0
    y_ref, st_ref = o.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           delta_bias=t["delta_bias"], delta_softplus=True)
    assert_close(to_host(yy), y_ref, TOL["f32"], "unaligned y")
    assert_close(to_host(st), st_ref, TOL["f32"], "unaligned state")


def test_bitwise_deterministic():
    t = W.scan_inputs(2, 300, 192, 16, "bf16", seed=12)
    y1, s1, _ = scan_on_gpu(t, True)
    y2, s2, _ = scan_on_gpu(t, True)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    y3, s3, _ = scan_on_gpu(t, True, segments=4)
    y4, s4, _ = scan_on_gpu(t, True, segments=4)
    assert torch.equal(y3, y4) and torch.equal(s3, s4)


# ---------------------------------------------------------------------------------------------------
# full-size workloads, every element
# ---------------------------------------------------------------------------------------------------
def full_size(o, name):
    w = W.WORKLOADS[name]
    say(f"[case] full size {name}: batch={w.batch} L={w.seqlen} dim={w.dim} N={w.dstate} {w.dtype}")
    t = W.workload_inputs(w)
    y, st, _ = scan_on_gpu(t, w.delta_softplus)
    block = 32 if w.seqlen > 100_000 else 512
    scan_whole(o, t, y, st, w.delta_softplus, TOL[w.dtype], name, block=block, threads=THREADS)
    return t, y, st


def test_full_mamba130m(o):
    full_size(o, "mamba130m")


def test_full_mamba2p8b(o):
    full_size(o, "mamba2p8b")


def test_full_genomics(o):
    full_size(o, "genomics")


def test_full_genomics_impulse_carry(o):
    """Impulse at t = 0 with delta_0 = 1, then delta = 0 for 2^20 - 1 steps: the state is held
    exactly, so y_t = (C_t . B_0 + D x_t) SiLU(z_t) for every t; catches any carry error across
    chunks and segments.  Every element of y and of the final state."""
    w = W.WORKLOADS["genomics"]
    say(f"[case] genomics impulse carry, every element (1, 2^20, 256, N=16)")
    t = W.workload_inputs(w)
    t["delta"] = np.zeros_like(t["delta"])
    t["delta"][:, 0, :] = 1.0
    y, st, _ = scan_on_gpu(t, False)
    scan_whole(o, t, y, st, False, TOL["f32"], "impulse carry", block=32, threads=THREADS)


# ---------------------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------------------
def decode_steps(t, batch, dim, N, steps, softplus, device="cuda"):
    import selective_state_space_61_amd as ssm
    d = {k: to_dev(v, device) for k, v in t.items()}
    state = torch.zeros(batch, dim, N, device=device)
    ys = []
    for s in range(steps):
        ys.append(ssm.ssm_state_update(state, d["x"][s], d["delta"][s], d["A"], d["B"][s], d["C"][s], D=d["D"],
                                       z=None if d["z"] is None else d["z"][s], delta_bias=d["delta_bias"],
                                       delta_softplus=softplus))
    torch.cuda.synchronize()
    return torch.stack(ys), state


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64])
def test_decode_matches_scan_oracle(o, dtype, N):
    batch, dim, steps = 3, 70, 12
    w = W.Workload("dec", "decode", batch=batch, seqlen=steps, dim=dim, dstate=N, dtype=dtype, seed=N)
    t = W.workload_inputs(w)
    say(f"[case] decode N={N} {dtype}")
    ys, state = decode_steps(t, batch, dim, N, steps, True)
    sc = {k: (np.ascontiguousarray(np.swapaxes(v, 0, 1)) if k in ("x", "delta", "z", "B", "C") else v)
          for k, v in t.items()}
    y_ref, st_ref = o.scan(sc["x"], sc["delta"], sc["A"], sc["B"], sc["C"], D=sc["D"], z=sc["z"],
                           delta_bias=sc["delta_bias"], delta_softplus=True)
    assert_close(to_host(ys), np.swapaxes(y_ref, 0, 1), TOL[dtype], "decode y")
    assert_close(to_host(state), st_ref, TOL[dtype], "decode state")


def test_decode_full_workload(o):
    """The batched decode workload (64 x 5120, N 16, bf16): 256 steps from a zero state; every
    step's y and the final state, every element, against the oracle's scan of the same 256
    tokens."""
    w = W.WORKLOADS["decode"]
    say(f"[case] full decode: batch={w.batch} dim={w.dim} N={w.dstate} steps={w.seqlen}, every element")
    t = W.workload_inputs(w)
    ys, state = decode_steps(t, w.batch, w.dim, w.dstate, w.seqlen, w.delta_softplus)
    sc = {k: (np.ascontiguousarray(np.swapaxes(v, 0, 1)) if k in ("x", "delta", "z", "B", "C") else v)
          for k, v in t.items()}
    # (steps, batch, dim) -> (batch, steps, dim), the scan layout the oracle compares against
    scan_whole(o, sc, ys.transpose(0, 1), state, True, TOL[w.dtype], "decode over 256 steps", block=1024,
               threads=THREADS)


# ---------------------------------------------------------------------------------------------------
# the state-row layout (SSM_LAYOUT_STATE_ROWS): the same arithmetic in the same order as the
# channel-lane layout, so the same bits; and the oracle
# ---------------------------------------------------------------------------------------------------
ROW_SHAPES = [(2, 96, 48, 16), (1, 33, 16, 16), (3, 70, 200, 16), (2, 257, 97, 16), (1, 1, 5, 16), (2, 64, 384, 16)]


# (channel groups, chunk steps) the library instantiates: 32-step tiles fit LDS up to 3 groups
# (more is rejected with SSM_ERR_UNSUPPORTED before any launch; tests/test_abi.py)
ROW_CASES = [(g, c) for c in (16, 32) for g in range(1, 7) if c == 16 or g <= 3]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("groups,chunk", ROW_CASES)
def test_state_rows_equal_channel_lanes(o, dtype, groups, chunk):
    for k, (batch, L, dim, N) in enumerate(ROW_SHAPES):
        say(f"[case] state rows {dtype} groups={groups} chunk={chunk} shape={(batch, L, dim, N)}")
        t = W.scan_inputs(batch, L, dim, N, dtype, seed=500 + 13 * groups + k)
        yr, sr, _ = scan_on_gpu(t, True, layout="state_rows", channel_groups=groups, chunk_steps=chunk)
        yl, sl, _ = scan_on_gpu(t, True, layout="channel_lanes", chains_per_lane=4, chunk_steps=chunk, segments=1)
        assert torch.equal(yr, yl), "y differs between the layouts"
        assert torch.equal(sr, sl), "last_state differs between the layouts"
        if k < 3:
            y_ref, st_ref = o.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                   delta_bias=t["delta_bias"], delta_softplus=True, nthreads=THREADS)
            assert_close(to_host(yr), y_ref, TOL[dtype], "state rows y")
            assert_close(to_host(sr), st_ref, TOL[dtype], "state rows last_state")


@pytest.mark.parametrize("variant", ["no_z", "no_D", "no_bias", "softplus_off", "bare"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_rows_variants(o, variant, dtype):
    softplus = variant not in ("softplus_off", "bare")
    t = W.scan_inputs(2, 90, 120, 16, dtype, seed=61 + len(variant), has_z=variant not in ("no_z", "bare"),
                      has_D=variant not in ("no_D", "bare"), has_bias=softplus and variant != "no_bias")
    if not softplus:
        t["delta"] = np.abs(t["delta"]) if dtype == "f32" else t["delta"] & np.uint16(0x7FFF)
    say(f"[case] state rows variant {variant} {dtype}")
    yr, sr, _ = scan_on_gpu(t, softplus, layout="state_rows", channel_groups=3)
    yl, sl, _ = scan_on_gpu(t, softplus, layout="channel_lanes", chains_per_lane=4, segments=1)
    assert torch.equal(yr, yl) and torch.equal(sr, sl), "the layouts differ"
    y_ref, st_ref = o.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                           delta_softplus=softplus, nthreads=THREADS)
    assert_close(to_host(yr), y_ref, TOL[dtype], f"state rows {variant} y")
    assert_close(to_host(sr), st_ref, TOL[dtype], f"state rows {variant} last_state")


def test_state_rows_unaligned_views_and_empty(o):
    """Views whose rows are not 16-byte aligned take the element-wise path; L = 0 gives a zero
    state; dim not a multiple of the 16-byte vector."""
    import selective_state_space_61_amd as ssm
    t = W.scan_inputs(2, 77, 51, 16, "bf16", seed=8)
    yr, sr, _ = scan_on_gpu(t, True, layout="state_rows", channel_groups=2)
    yl, sl, _ = scan_on_gpu(t, True, layout="channel_lanes", chains_per_lane=4, segments=1)
    assert torch.equal(yr, yl) and torch.equal(sr, sl)
    d = {k: to_dev(v) for k, v in t.items()}
    y = torch.empty(2 * 77 * 51 + 1, dtype=torch.bfloat16, device="cuda")[1:].view(2, 77, 51)
    ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], delta_bias=d["delta_bias"],
                     delta_softplus=True, y=y, layout="state_rows", channel_groups=2)
    torch.cuda.synchronize()
    assert torch.equal(y, yl), "unaligned y differs"
    t0 = W.scan_inputs(2, 0, 64, 16, "f32", seed=9)
    _, s0, _ = scan_on_gpu(t0, True, layout="state_rows", channel_groups=4)
    assert torch.count_nonzero(s0).item() == 0


# ---------------------------------------------------------------------------------------------------
# the time-parallel layout (SSM_LAYOUT_TIME_SCAN): wave64 associative scan of (abar, state) pairs
# ---------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [256, 512])
def test_time_scan_layout(o, dtype, chunk):
    for k, (batch, L, dim) in enumerate([(1, 1000, 8), (2, 513, 3), (1, 1, 5), (1, 4096, 16), (3, 37, 2)]):
        say(f"[case] time scan {dtype} chunk={chunk} shape={(batch, L, dim)}")
        t = W.scan_inputs(batch, L, dim, 16, dtype, seed=700 + k + chunk)
        y, st, _ = scan_on_gpu(t, True, layout="time_scan", chunk_steps=chunk)
        y_ref, st_ref = o.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               delta_bias=t["delta_bias"], delta_softplus=True, nthreads=THREADS)
        assert_close(to_host(y), y_ref, TOL[dtype], "time scan y")
        assert_close(to_host(st), st_ref, TOL[dtype], "time scan last_state")


@pytest.mark.parametrize("variant", ["genomics", "impulse", "no_z_no_D"])
def test_time_scan_long(o, variant):
    """The genomics recipe over 2^17 steps (256 chunks of 512 carried), its impulse-carry form, and
    a bare variant."""
    L, dim = 1 << 17, 24
    if variant == "no_z_no_D":
        t = W.scan_inputs(1, L, dim, 16, "f32", seed=81, recipe="genomics", has_bias=False, has_z=False, has_D=False)
    else:
        t = W.scan_inputs(1, L, dim, 16, "f32", seed=80, recipe="genomics", has_bias=False)
    if variant == "impulse":
        t["delta"] = np.zeros_like(t["delta"])
        t["delta"][:, 0, :] = 1.0
    say(f"[case] time scan long {variant} (1, {L}, {dim})")
    y, st, _ = scan_on_gpu(t, False, layout="time_scan")
    scan_whole(o, t, y, st, False, TOL["f32"], f"time scan {variant}", block=dim, threads=THREADS)
