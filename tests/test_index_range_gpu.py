"""Tensors of more than 2^31 elements: a selective scan, a causal convolution and an SSD layer
whose x and y hold more than 2^31 elements, and the two decode steps over states of more than
2^31 elements, so that element offsets pass 2^31 and byte offsets pass 2^32 inside the kernels.
Each is compared with the oracle on sampled channels over the whole sequence (the last batch
row's late steps lie past 2^31), or on whole batch rows of the decode states (the last rows lie
past 2^31).

x, delta and z repeat a block of a few thousand steps along time (period 4099 or 1031, prime to
the tile sizes and to the row length); B, C and the SSD's dt are drawn for every step.  An
offset that wrapped at 2^31 or 2^32 would land on another channel or step, not on an equal
value; the decode states repeat a block of 7 (5) batch rows.  The largest case, the backward,
takes about 44 GB of device memory."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, assert_close, say, to_dev, to_host

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
    yield
    torch.cuda.empty_cache()


def tiled(block, seqlen):
    """Device tensor of `block` (batch, period, ...) repeated along axis 1 to seqlen steps."""
    blk = to_dev(block)
    out = torch.empty((blk.shape[0], seqlen) + tuple(blk.shape[2:]), dtype=blk.dtype, device=blk.device)
    period = blk.shape[1]
    for s in range(0, seqlen, period):
        n = min(period, seqlen - s)
        out[:, s:s + n] = blk[:, :n]
    return out


def tiled_rows(block, n):
    """Device tensor of `block` (period, ...) repeated along axis 0 to n rows."""
    blk = to_dev(block)
    out = torch.empty((n,) + tuple(blk.shape[1:]), dtype=blk.dtype, device=blk.device)
    for s in range(0, n, blk.shape[0]):
        k = min(blk.shape[0], n - s)
        out[s:s + k] = blk[:k]
    return out


BATCH, L, DIM, PERIOD = 2, (1 << 20) + 37, 1040, 4099
PICKS = [(0, 0), (0, 517), (1, 0), (1, 63), (1, 1000), (1, DIM - 1)]


def test_scan_beyond_2_31_elements(o):
    import selective_state_space_61_amd as ssm
    assert BATCH * L * DIM > 2 ** 31
    t = W.long_scan_inputs(BATCH, L, DIM, 16, PERIOD, "bf16", seed=61100)
    say(f"[case] scan of {BATCH}x{L}x{DIM} bf16 ({BATCH * L * DIM} elements per tensor)")
    x, delta, z = tiled(t["x"], L), tiled(t["delta"], L), tiled(t["z"], L)
    y, st = ssm.ssm_scan_fwd(x, delta, to_dev(t["A"]), to_dev(t["B"]), to_dev(t["C"]), D=to_dev(t["D"]), z=z,
                             delta_bias=to_dev(t["delta_bias"]), delta_softplus=True)
    torch.cuda.synchronize()
    del x, delta, z
    for b, d in PICKS:
        cols = {k: W.repeat_in_time(t[k][b:b + 1, :, d:d + 1], L) for k in ("x", "delta", "z")}
        y_ref, st_ref = o.scan(cols["x"], cols["delta"], t["A"][d:d + 1], t["B"][b:b + 1], t["C"][b:b + 1],
                               D=t["D"][d:d + 1], z=cols["z"], delta_bias=t["delta_bias"][d:d + 1],
                               delta_softplus=True, nthreads=THREADS)
        assert_close(to_host(y[b, :, d]), y_ref[0, :, 0], TOL["bf16"], f"scan y (b={b}, d={d})")
        assert_close(to_host(st[b, d]), st_ref[0, 0], TOL["bf16"], f"scan last_state (b={b}, d={d})")


def test_conv1d_beyond_2_31_elements(o):
    import selective_state_space_61_amd as ssm
    t = W.conv_inputs(BATCH, PERIOD, DIM, 4, "bf16", seed=61102)
    say(f"[case] causal conv1d of {BATCH}x{L}x{DIM} bf16, width 4")
    x = tiled(t["x"], L)
    y, fin = ssm.ssm_causal_conv1d_fwd(x, to_dev(t["weight"]), to_dev(t["bias"]), silu=True,
                                       return_final_state=True)
    torch.cuda.synchronize()
    del x
    for b, d in PICKS:
        xs = W.repeat_in_time(t["x"][b:b + 1, :, d:d + 1], L)
        y_ref, fin_ref = o.causal_conv1d(xs, t["weight"][d:d + 1], t["bias"][d:d + 1], silu=True)
        assert_close(to_host(y[b, :, d]), y_ref[0, :, 0], TOL["bf16"], f"conv y (b={b}, d={d})")
        assert_close(to_host(fin[b, d]), fin_ref[0, 0], TOL["bf16"], f"conv final_state (b={b}, d={d})")


def test_ssd_beyond_2_31_elements(o):
    import selective_state_space_61_amd as ssm
    batch, seqlen, H, P, N, period = 1, (1 << 19) + 37, 64, 64, 128, 1031
    assert batch * seqlen * H * P > 2 ** 31
    t = W.long_ssd_inputs(batch, seqlen, H, P, N, period, seed=61101)
    say(f"[case] SSD layer of {batch}x{seqlen}x{H}x{P}, N {N} ({batch * seqlen * H * P} elements per tensor)")
    x, z = tiled(t["x"], seqlen), tiled(t["z"], seqlen)
    y, fin = ssm.ssm_ssd_fwd(x, to_dev(t["dt"]), to_dev(t["A"]), to_dev(t["B"]), to_dev(t["C"]), D=to_dev(t["D"]),
                             z=z, dt_bias=to_dev(t["dt_bias"]), dt_softplus=True)
    torch.cuda.synchronize()
    del x, z
    for h, p in [(0, 0), (31, 17), (63, 0), (63, 63)]:
        xs = W.repeat_in_time(t["x"][:, :, h:h + 1, p:p + 1], seqlen)
        zs = W.repeat_in_time(t["z"][:, :, h:h + 1, p:p + 1], seqlen)
        y_ref, fin_ref = o.ssd(xs, t["dt"][:, :, h:h + 1], t["A"][h:h + 1], t["B"], t["C"], D=t["D"][h:h + 1],
                               z=zs, dt_bias=t["dt_bias"][h:h + 1], dt_softplus=True, nthreads=THREADS)
        assert_close(to_host(y[0, :, h, p]), y_ref[0, :, 0, 0], TOL["bf16"], f"SSD y (h={h}, p={p})")
        assert_close(to_host(fin[0, h, p]), fin_ref[0, 0, 0], TOL["bf16"], f"SSD final_state (h={h}, p={p})")


def test_decode_state_beyond_2_31_elements(o):
    import selective_state_space_61_amd as ssm
    batch, dim, N, period = 2048, 65600, 16, 7
    assert batch * dim * N > 2 ** 31
    t = W.long_decode_inputs(batch, dim, N, period, seed=61103)
    say(f"[case] decode step, state {batch}x{dim}x{N} fp32 ({batch * dim * N} elements)")
    state = tiled_rows(t["state_block"], batch)
    y = ssm.ssm_state_update(state, to_dev(t["x"]), to_dev(t["delta"]), to_dev(t["A"]), to_dev(t["B"]),
                             to_dev(t["C"]), D=to_dev(t["D"]), z=to_dev(t["z"]),
                             delta_bias=to_dev(t["delta_bias"]), delta_softplus=True)
    torch.cuda.synchronize()
    for b in (0, 1500, batch - 2, batch - 1):
        y_ref, st_ref = o.state_update(t["state_block"][b % period][None], t["x"][b:b + 1], t["delta"][b:b + 1],
                                       t["A"], t["B"][b:b + 1], t["C"][b:b + 1], D=t["D"], z=t["z"][b:b + 1],
                                       delta_bias=t["delta_bias"], delta_softplus=True)
        assert_close(to_host(y[b]), y_ref[0], TOL["bf16"], f"decode y (row {b})")
        assert_close(to_host(state[b]), st_ref[0], TOL["bf16"], f"decode state (row {b})")
    del state


def test_ssd_decode_state_beyond_2_31_elements(o):
    import selective_state_space_61_amd as ssm
    batch, H, P, N, period = 4100, 64, 64, 128, 5
    assert batch * H * P * N > 2 ** 31
    t = W.long_ssd_decode_inputs(batch, H, P, N, period, seed=61104)
    say(f"[case] SSD decode step, state {batch}x{H}x{P}x{N} fp32 ({batch * H * P * N} elements)")
    state = tiled_rows(t["state_block"], batch)
    y = ssm.ssm_ssd_state_update(state, to_dev(t["x"]), to_dev(t["dt"]), to_dev(t["A"]), to_dev(t["B"]),
                                 to_dev(t["C"]), D=to_dev(t["D"]), z=to_dev(t["z"]), dt_bias=to_dev(t["dt_bias"]),
                                 dt_softplus=True)
    torch.cuda.synchronize()
    for b in (0, 2001, batch - 3, batch - 1):
        y_ref, fin_ref = o.ssd(t["x"][b:b + 1, None], t["dt"][b:b + 1, None], t["A"], t["B"][b:b + 1, None],
                               t["C"][b:b + 1, None], D=t["D"], z=t["z"][b:b + 1, None], dt_bias=t["dt_bias"],
                               dt_softplus=True, h0=t["state_block"][b % period][None])
        assert_close(to_host(y[b]), y_ref[0, 0], TOL["bf16"], f"SSD decode y (row {b})")
        assert_close(to_host(state[b]), fin_ref[0], TOL["bf16"], f"SSD decode state (row {b})")
    del state


def test_scan_bwd_beyond_2_31_elements(o):
    """The backward over the scan shape above: dx, ddelta and dz (past 2^31 elements each) and
    the per-channel dA, dD and ddelta_bias on sampled channels, from a single-channel oracle run
    over both batch rows.  dB and dC sum over every channel (their buffers stay below 2^31
    elements) and are covered by the full-width cases of test_bwd_gpu.py."""
    import selective_state_space_61_amd as ssm
    t = W.long_scan_inputs(BATCH, L, DIM, 16, PERIOD, "bf16", seed=61105)
    dy = W.f32_to_bf16_bits(np.random.default_rng(61105).standard_normal((BATCH, PERIOD, DIM)).astype(np.float32))
    say(f"[case] scan backward of {BATCH}x{L}x{DIM} bf16")
    x, delta, z, dyd = tiled(t["x"], L), tiled(t["delta"], L), tiled(t["z"], L), tiled(dy, L)
    g = ssm.ssm_scan_bwd(x, delta, to_dev(t["A"]), to_dev(t["B"]), to_dev(t["C"]), dyd, D=to_dev(t["D"]), z=z,
                         delta_bias=to_dev(t["delta_bias"]), delta_softplus=True)
    torch.cuda.synchronize()
    del x, delta, z, dyd
    for d in (0, 517, DIM - 1):
        cols = {k: W.repeat_in_time(src[:, :, d:d + 1], L)
                for k, src in (("x", t["x"]), ("delta", t["delta"]), ("z", t["z"]), ("dy", dy))}
        ref = o.scan_bwd(cols["x"], cols["delta"], t["A"][d:d + 1], t["B"], t["C"],
                         W.bf16_bits_to_f32(cols["dy"]).astype(np.float64), D=t["D"][d:d + 1], z=cols["z"],
                         delta_bias=t["delta_bias"][d:d + 1], delta_softplus=True)
        for k in ("dx", "ddelta", "dz"):
            assert_close(to_host(g[k][:, :, d]), ref[k][:, :, 0], TOL["bf16"], f"bwd {k} (d={d})")
        assert_close(to_host(g["dA"][d]), ref["dA"][0], 1e-3, f"bwd dA (d={d})")
        assert_close(to_host(g["dD"][d:d + 1]), ref["dD"], 1e-3, f"bwd dD (d={d})")
        assert_close(to_host(g["ddelta_bias"][d:d + 1]), ref["ddelta_bias"], 1e-3, f"bwd ddelta_bias (d={d})")
