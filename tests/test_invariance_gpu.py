"""A property of the discretisation, checked on the HIP path at full size, bit for bit.

The step enters the method only through delta A (the decay exp(delta A)) and delta B (the input
term delta B x of "Mamba 论文精读" sec. 3.3, and the exact hold (exp(delta A) - 1) / A B of
sec. 2.2).  So (delta, A, B) -> (2 delta, A / 2, B / 2) leaves every output unchanged.  Scaling by
two commutes with every rounding the kernels make (bf16 storage included), so the kernels must
return the same bits, whatever their order of operations: a kernel that mixed up which tensor
feeds which product, or dropped a factor of delta, would not.  The step is passed in its final
form (softplus applied on the host, no bias), since the map acts on the step itself.  These
tests need no oracle; the oracle side of the property is pinned in tests/pins.py."""
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_61_amd as ssm
    ssm.load_library()


def final_step(delta, bias):
    """softplus(delta + bias) in fp32, stored in delta's dtype (bf16 rounded to nearest even)."""
    v = delta.float() + (0.0 if bias is None else bias)
    return torch.nn.functional.softplus(v, threshold=20.0).to(delta.dtype)


def halved(t):
    return t / 2 if t.dtype == torch.float32 else (t.float() / 2).to(t.dtype)


def doubled(t):
    return t * 2 if t.dtype == torch.float32 else (t.float() * 2).to(t.dtype)


def assert_same_bits(a, b, what):
    assert a.shape == b.shape, f"{what}: shapes {a.shape} / {b.shape}"
    assert torch.all(torch.isfinite(a.float())), f"{what}: non-finite values"
    same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    if not same:
        diff = (a.float() - b.float()).abs().max().item()
        raise AssertionError(f"{what}: outputs differ under (2 delta, A / 2, B / 2), max |diff| {diff:.3e}")
    say(f"  {what}: {a.numel()} elements bit-identical")


def scan_pair(t, softplus=True, **kw):
    import selective_state_space_61_amd as ssm
    d = {k: to_dev(v) for k, v in t.items()}
    dt = final_step(d["delta"], d["delta_bias"]) if softplus else d["delta"]
    out = []
    for dtv, A, B in ((dt, d["A"], d["B"]), (doubled(dt), halved(d["A"]), halved(d["B"]))):
        y, st = ssm.ssm_scan_fwd(d["x"], dtv, A, B, d["C"], D=d["D"], z=d["z"], delta_softplus=False, **kw)
        out.append((y, st))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("workload,kw", [("mamba130m", {}), ("mamba130m", {"layout": "channel_lanes"}),
                                         ("mamba130m", {"zoh": True}), ("mamba2p8b", {})],
                         ids=["130m-auto", "130m-channel-lanes", "130m-zoh", "2p8b-auto"])
def test_scan_scale_invariance(workload, kw):
    w = W.WORKLOADS[workload]
    say(f"[case] scan {workload} {kw}: (2 delta, A / 2, B / 2)")
    (y0, s0), (y1, s1) = scan_pair(W.workload_inputs(w), **kw)
    assert_same_bits(y0, y1, f"{workload} {kw} y")
    assert_same_bits(s0, s1, f"{workload} {kw} last_state")


def test_scan_scale_invariance_split_sequence():
    """The genomics recipe (fp32, 256 channels) over 2^17 steps: few channels, so the sequence is
    split and the segments' carries composed with exp(A sum delta)."""
    t = W.scan_inputs(1, 1 << 17, 256, 16, dtype="f32", seed=61003, recipe="genomics", has_bias=False)
    say("[case] scan split sequence, genomics recipe 1 x 2^17 x 256 (delta passed as the step)")
    (y0, s0), (y1, s1) = scan_pair(t, softplus=False)
    assert_same_bits(y0, y1, "split-sequence y")
    assert_same_bits(s0, s1, "split-sequence last_state")


def test_decode_scale_invariance():
    import selective_state_space_61_amd as ssm
    w = W.WORKLOADS["decode"]
    t = W.workload_inputs(w)
    d = {k: to_dev(v) for k, v in t.items()}
    steps = 32
    say(f"[case] decode {w.batch} x {w.dim}, {steps} steps: (2 delta, A / 2, B / 2)")
    results = []
    for scale in (False, True):
        state = torch.zeros(w.batch, w.dim, w.dstate, device="cuda")
        ys = []
        for s in range(steps):
            dt = final_step(d["delta"][s], d["delta_bias"])
            A, B = d["A"], d["B"][s]
            if scale:
                dt, A, B = doubled(dt), halved(A), halved(B)
            ys.append(ssm.ssm_state_update(state, d["x"][s], dt, A, B, d["C"][s], D=d["D"], z=d["z"][s],
                                           delta_softplus=False))
        torch.cuda.synchronize()
        results.append((torch.stack(ys), state))
    assert_same_bits(results[0][0], results[1][0], "decode y")
    assert_same_bits(results[0][1], results[1][1], "decode state")


@pytest.mark.parametrize("workload", ["mamba2_layer_b8", "mamba2_layer"])
def test_ssd_scale_invariance(workload):
    """The SSD layer: the 8 x 2048 layer (C B^T computed once per group by the separate pass) and
    the 1 x 1024 example (the sequence split into segments whose states are composed)."""
    import selective_state_space_61_amd as ssm
    w = W.SSD_WORKLOADS[workload]
    t = W.ssd_workload_inputs(w)
    d = {k: to_dev(v) for k, v in t.items()}
    dt = final_step(d["dt"], d["dt_bias"])
    say(f"[case] SSD {workload}: (2 dt, A / 2, B / 2)")
    out = []
    for dtv, A, B in ((dt, d["A"], d["B"]), (doubled(dt), halved(d["A"]), halved(d["B"]))):
        out.append(ssm.ssm_ssd_fwd(d["x"], dtv, A, B, d["C"], D=d["D"], z=d["z"], dt_softplus=False))
    torch.cuda.synchronize()
    assert_same_bits(out[0][0], out[1][0], f"{workload} y")
    assert_same_bits(out[0][1], out[1][1], f"{workload} final_state")


# ---------------------------------------------------------------------------------------------------
# homogeneity in x: x enters only through the input term (delta x) and the skip (D x), and the gate
# depends on z alone, so y(2 x) = 2 y(x) and the final state doubles; doubling is exact in every
# rounding the kernels make.
# ---------------------------------------------------------------------------------------------------
def assert_doubled(a2, a1, what):
    assert_same_bits(a2, doubled(a1), what + ": twice the original")


@pytest.mark.parametrize("workload,kw", [("mamba130m", {}), ("mamba130m", {"layout": "channel_lanes"}),
                                         ("mamba130m", {"zoh": True})],
                         ids=["130m-auto", "130m-channel-lanes", "130m-zoh"])
def test_scan_homogeneous_in_x(workload, kw):
    import selective_state_space_61_amd as ssm
    t = W.workload_inputs(W.WORKLOADS[workload])
    d = {k: to_dev(v) for k, v in t.items()}
    say(f"[case] scan {workload} {kw}: x -> 2 x")
    out = [ssm.ssm_scan_fwd(x, d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], delta_bias=d["delta_bias"],
                            delta_softplus=True, **kw) for x in (d["x"], doubled(d["x"]))]
    torch.cuda.synchronize()
    assert_doubled(out[1][0], out[0][0], f"{workload} {kw} y")
    assert_doubled(out[1][1], out[0][1], f"{workload} {kw} last_state")


def test_ssd_homogeneous_in_x():
    import selective_state_space_61_amd as ssm
    t = W.ssd_workload_inputs(W.SSD_WORKLOADS["mamba2_layer_b8"])
    d = {k: to_dev(v) for k, v in t.items()}
    say("[case] SSD mamba2_layer_b8: x -> 2 x")
    out = [ssm.ssm_ssd_fwd(x, d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], dt_bias=d["dt_bias"],
                           dt_softplus=True) for x in (d["x"], doubled(d["x"]))]
    torch.cuda.synchronize()
    assert_doubled(out[1][0], out[0][0], "mamba2_layer_b8 y")
    assert_doubled(out[1][1], out[0][1], "mamba2_layer_b8 final_state")


# ---------------------------------------------------------------------------------------------------
# the backward under the same map: the loss sum(dy y) is unchanged by (delta, A, B) -> (2 delta,
# A / 2, B / 2), so at the mapped point dx, dC, dD and dz are unchanged, ddelta (with respect to the
# step) halves, and dA and dB double, bit for bit (every term of each gradient scales alike).
# The state-row backward adds dB and dC over channel blocks with atomics, in an order that varies
# from run to run, so there those two are compared to within their bf16 storage.
# ---------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("kw", [{}, {"layout": "channel_lanes"}, {"zoh": True}],
                         ids=["auto", "channel-lanes", "zoh"])
def test_backward_scale_covariance(kw):
    import selective_state_space_61_amd as ssm
    t = W.workload_inputs(W.WORKLOADS["mamba130m"])
    d = {k: to_dev(v) for k, v in t.items()}
    dt = final_step(d["delta"], d["delta_bias"])
    gen = torch.Generator(device="cuda").manual_seed(61)
    dy = torch.randn(d["x"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    say(f"[case] backward mamba130m {kw}: (2 delta, A / 2, B / 2)")
    g0 = ssm.ssm_scan_bwd(d["x"], dt, d["A"], d["B"], d["C"], dy, D=d["D"], z=d["z"], **kw)
    g1 = ssm.ssm_scan_bwd(d["x"], doubled(dt), halved(d["A"]), halved(d["B"]), d["C"], dy, D=d["D"], z=d["z"], **kw)
    torch.cuda.synchronize()
    atomics = kw.get("layout", "auto") == "auto" and not kw.get("zoh", False)
    for k, f in (("dx", None), ("dz", None), ("dD", None), ("ddelta", halved), ("dA", doubled),
                 ("dB", doubled), ("dC", None)):
        want = g0[k] if f is None else f(g0[k])
        if atomics and k in ("dB", "dC"):
            err = (g1[k].float() - want.float()).abs().max().item()
            scale = want.float().abs().max().item()
            say(f"  {k}: max |diff| {err:.3e} against max {scale:.3e} (atomic sums)")
            assert err <= 1e-2 * scale, f"{k}: {err:.3e} > 1e-2 x {scale:.3e}"
        else:
            assert_same_bits(g1[k], want, f"{k}{'' if f is None else ' (scaled)'}")


def test_ssd_decode_scale_invariance():
    """The SSD layer's single-token step on 64 rows x 64 heads x 64 channels, dstate 128, from a
    nonzero state over 8 tokens: the same bits under (2 dt, A / 2, B / 2)."""
    import selective_state_space_61_amd as ssm
    batch, H, P, N, steps = 64, 64, 64, 128, 8
    t = W.ssd_inputs(batch, steps, H, P, N, 1, seed=61009)
    d = {k: (None if v is None else to_dev(v)) for k, v in t.items()}
    gen = torch.Generator(device="cuda").manual_seed(9)
    h0 = torch.randn((batch, H, P, N), generator=gen, device="cuda") * 0.5
    dt = final_step(d["dt"], d["dt_bias"])
    say(f"[case] SSD decode {batch} x {H} x {P}, N {N}, {steps} tokens: (2 dt, A / 2, B / 2)")
    results = []
    for scale in (False, True):
        state = h0.clone()
        A = halved(d["A"]) if scale else d["A"]
        ys = []
        for s in range(steps):
            dts, B = dt[:, s].contiguous(), d["B"][:, s].contiguous()
            if scale:
                dts, B = doubled(dts), halved(B)
            ys.append(ssm.ssm_ssd_state_update(state, d["x"][:, s].contiguous(), dts, A, B, d["C"][:, s].contiguous(),
                                               D=d["D"], z=d["z"][:, s].contiguous()))
        torch.cuda.synchronize()
        results.append((torch.stack(ys), state))
    assert_same_bits(results[0][0], results[1][0], "SSD decode y")
    assert_same_bits(results[0][1], results[1][1], "SSD decode state")


def test_conv1d_homogeneous():
    """The depthwise causal convolution without bias or SiLU is linear in x and in the weights:
    doubling either (the entering state with x) doubles y and the final state, bit for bit, on
    the 8 x 2048 x 1536 bf16 shape."""
    import selective_state_space_61_amd as ssm
    t = W.conv_inputs(8, 2048, 1536, 4, "bf16", seed=61001, has_bias=False, has_init=True)
    d = {k: (None if v is None else to_dev(v)) for k, v in t.items()}
    say("[case] conv1d 8 x 2048 x 1536, width 4: x -> 2 x, weight -> 2 weight")

    def run(x, w, init):
        return ssm.ssm_causal_conv1d_fwd(x, w, None, initial_state=init, silu=False, return_final_state=True)
    y0, f0 = run(d["x"], d["weight"], d["init"])
    y1, f1 = run(doubled(d["x"]), d["weight"], doubled(d["init"]))
    y2, f2 = run(d["x"], d["weight"] * 2, d["init"])
    torch.cuda.synchronize()
    assert_doubled(y1, y0, "conv1d y")
    assert_doubled(f1, f0, "conv1d final_state")
    assert_doubled(y2, y0, "conv1d y (weights doubled)")
    assert_same_bits(f2, f0, "conv1d final_state (weights doubled: the inputs, unchanged)")


def test_checkpoint_pair_scale_covariance():
    """The training pair under (delta, A, B) -> (2 delta, A / 2, B / 2) at the 130M shape: the
    forward's checkpoints (states) are unchanged, and the backward from them transforms as the
    plain backward does (dB and dC are atomic sums there: compared within their bf16 storage)."""
    import selective_state_space_61_amd as ssm
    t = W.workload_inputs(W.WORKLOADS["mamba130m"])
    d = {k: to_dev(v) for k, v in t.items()}
    dt = final_step(d["delta"], d["delta_bias"])
    gen = torch.Generator(device="cuda").manual_seed(62)
    dy = torch.randn(d["x"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    say("[case] checkpoint pair mamba130m: (2 delta, A / 2, B / 2)")
    res = []
    for dtv, A, B in ((dt, d["A"], d["B"]), (doubled(dt), halved(d["A"]), halved(d["B"]))):
        y, st, ck = ssm.ssm_scan_fwd_ckpt(d["x"], dtv, A, B, d["C"], D=d["D"], z=d["z"])
        g = ssm.ssm_scan_bwd_ckpt(d["x"], dtv, A, B, d["C"], dy, ck, D=d["D"], z=d["z"])
        res.append((y, st, ck, g))
    torch.cuda.synchronize()
    assert_same_bits(res[1][0], res[0][0], "pair forward y")
    assert_same_bits(res[1][2], res[0][2], "checkpoints")
    g0, g1 = res[0][3], res[1][3]
    for k, f in (("dx", None), ("dz", None), ("dD", None), ("ddelta", halved), ("dA", doubled)):
        assert_same_bits(g1[k], g0[k] if f is None else f(g0[k]), f"pair {k}{'' if f is None else ' (scaled)'}")
    for k, f in (("dB", doubled), ("dC", None)):
        want = g0[k] if f is None else f(g0[k])
        err = (g1[k].float() - want.float()).abs().max().item()
        scale = want.float().abs().max().item()
        say(f"  pair {k}: max |diff| {err:.3e} against max {scale:.3e} (atomic sums)")
        assert err <= 1e-2 * scale, f"pair {k}: {err:.3e} > 1e-2 x {scale:.3e}"


# ---------------------------------------------------------------------------------------------------
# batch order: every batch row is computed by the same arithmetic whatever its position (and
# whichever workgroup and XCD the remapped grid gives it), so reversing the batch reverses the
# outputs bit for bit.  Gradients summed over the batch (dA, dD, the bias) change their order of
# summation and are left out; so are the state rows' atomically summed dB / dC.
# ---------------------------------------------------------------------------------------------------
def flipped(t):
    return None if t is None else torch.flip(t, dims=[0]).contiguous()


def test_scan_batch_reversal():
    import selective_state_space_61_amd as ssm
    t = W.workload_inputs(W.WORKLOADS["mamba130m"])
    d = {k: to_dev(v) for k, v in t.items()}
    say("[case] scan mamba130m: batch reversed")
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], delta_softplus=True)
    y0, s0 = ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], z=d["z"], **kw)
    y1, s1 = ssm.ssm_scan_fwd(flipped(d["x"]), flipped(d["delta"]), d["A"], flipped(d["B"]), flipped(d["C"]),
                              z=flipped(d["z"]), **kw)
    torch.cuda.synchronize()
    assert_same_bits(y1, flipped(y0), "scan y (batch reversed)")
    assert_same_bits(s1, flipped(s0), "scan last_state (batch reversed)")


def test_ssd_batch_reversal():
    import selective_state_space_61_amd as ssm
    t = W.ssd_workload_inputs(W.SSD_WORKLOADS["mamba2_layer_b8"])
    d = {k: to_dev(v) for k, v in t.items()}
    say("[case] SSD mamba2_layer_b8: batch reversed")
    kw = dict(D=d["D"], dt_bias=d["dt_bias"], dt_softplus=True)
    y0, f0 = ssm.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], z=d["z"], **kw)
    y1, f1 = ssm.ssm_ssd_fwd(flipped(d["x"]), flipped(d["dt"]), d["A"], flipped(d["B"]), flipped(d["C"]),
                             z=flipped(d["z"]), **kw)
    torch.cuda.synchronize()
    assert_same_bits(y1, flipped(y0), "SSD y (batch reversed)")
    assert_same_bits(f1, flipped(f0), "SSD final_state (batch reversed)")


@pytest.mark.parametrize("layout", ["auto", "channel_lanes"])
def test_backward_batch_reversal(layout):
    import selective_state_space_61_amd as ssm
    t = W.workload_inputs(W.WORKLOADS["mamba130m"])
    d = {k: to_dev(v) for k, v in t.items()}
    gen = torch.Generator(device="cuda").manual_seed(63)
    dy = torch.randn(d["x"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    say(f"[case] backward mamba130m ({layout}): batch reversed")
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], delta_softplus=True, layout=layout)
    g0 = ssm.ssm_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], dy, z=d["z"], **kw)
    g1 = ssm.ssm_scan_bwd(flipped(d["x"]), flipped(d["delta"]), d["A"], flipped(d["B"]), flipped(d["C"]),
                          flipped(dy), z=flipped(d["z"]), **kw)
    torch.cuda.synchronize()
    keys = ("dx", "ddelta", "dz") + (("dB", "dC") if layout == "channel_lanes" else ())
    for k in keys:
        assert_same_bits(g1[k], flipped(g0[k]), f"{k} (batch reversed)")
