"""The seeded input generators: bf16 rounding, reproducibility, recipe statistics."""
import numpy as np

import workloads as W


def test_bf16_round_to_nearest_even_bit_patterns():
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),            # exact tie, even mantissa stays
        (one + 3 * 2.0 ** -8, 0x3F82),        # exact tie, odd mantissa rounds up to even
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie rounds up
        (-2.0, 0xC000),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (np.inf, 0x7F80),
        (-np.inf, 0xFF80),
        (3.4028235e38, 0x7F80),               # max fp32 rounds to +inf in bf16
        (2.0 ** -133, 0x0001),                # smallest bf16 subnormal
        (1e-45, 0x0000),                      # fp32 denormal below half of it rounds to zero
    ]
    for v, bits in cases:
        got = int(W.f32_to_bf16_bits(np.array([v], np.float32))[0])
        assert got == bits, (v, hex(got), hex(bits))
    nan = W.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(W.bf16_bits_to_f32(nan))[0]


def test_bf16_widening_is_exact_and_roundtrips():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(bits)
    back = W.f32_to_bf16_bits(f)
    finite = np.isfinite(f) | np.isinf(f)
    assert np.array_equal(back[finite], bits[finite])


def test_reproducible_and_seed_dependent():
    a = W.scan_inputs(2, 33, 40, 8, "bf16", seed=5)
    b = W.scan_inputs(2, 33, 40, 8, "bf16", seed=5)
    c = W.scan_inputs(2, 33, 40, 8, "bf16", seed=6)
    for k in ("x", "delta", "B", "C", "z", "delta_bias"):
        assert np.array_equal(a[k], b[k]), k
        assert not np.array_equal(a[k], c[k]), k
    assert a["x"].dtype == np.uint16 and a["A"].dtype == np.float32


def test_default_recipe_statistics():
    t = W.scan_inputs(4, 512, 256, 16, "f32", seed=61000)
    assert abs(t["x"].mean()) < 0.01 and abs(t["x"].std() - 1.0) < 0.01
    assert abs(t["delta"].std() - 0.5) < 0.01
    assert np.array_equal(t["A"], -np.tile(np.arange(1, 17, dtype=np.float32), (256, 1)))
    assert np.all(t["D"] == 1.0)
    sp = np.logaddexp(0.0, t["delta_bias"].astype(np.float64))
    assert sp.min() >= 1e-3 * 0.999 and sp.max() <= 1e-1 * 1.001
    lg = np.log10(sp)
    assert abs(lg.mean() + 2.0) < 0.1   # log-uniform over [-3, -1]


def test_genomics_recipe():
    t = W.scan_inputs(1, 4096, 64, 16, "f32", seed=61003, recipe="genomics", has_bias=False)
    x = t["x"][0]
    rows = np.unique(x, axis=0)
    assert rows.shape[0] == 4                          # four symbols -> four distinct rows
    assert t["delta_bias"] is None
    assert t["delta"].min() >= 1e-4 * 0.999 and t["delta"].max() <= 1e-1 * 1.001
    assert abs(np.log10(t["delta"]).mean() + 2.5) < 0.05


def test_named_workloads_shapes():
    w = W.WORKLOADS
    assert (w["tiny"].batch, w["tiny"].seqlen, w["tiny"].dim, w["tiny"].dstate) == (1, 64, 16, 4)
    assert (w["mamba130m"].batch, w["mamba130m"].seqlen, w["mamba130m"].dim) == (8, 2048, 1536)
    assert (w["mamba2p8b"].batch, w["mamba2p8b"].seqlen, w["mamba2p8b"].dim) == (4, 2048, 5120)
    assert (w["genomics"].seqlen, w["genomics"].dim, w["genomics"].dtype) == (1 << 20, 256, "f32")
    assert (w["decode"].batch, w["decode"].dim, w["decode"].seqlen) == (64, 5120, 256)
    t = W.workload_inputs(w["tiny"])
    assert t["x"].shape == (1, 64, 16) and t["B"].shape == (1, 64, 4) and t["x"].dtype == np.float32
    small_decode = W.Workload("d", "decode", batch=3, seqlen=5, dim=7, dstate=4, dtype="bf16", seed=1)
    d = W.workload_inputs(small_decode)
    s = W.scan_inputs(3, 5, 7, 4, "bf16", seed=1)
    assert d["x"].shape == (5, 3, 7) and d["B"].shape == (5, 3, 4)
    assert np.array_equal(d["x"][2], s["x"][:, 2]) and np.array_equal(d["C"][4], s["C"][:, 4])


def test_long_inputs_repeat_a_block_in_time():
    t = W.long_scan_inputs(2, 1000, 40, 16, 37, "bf16", seed=5)
    assert t["x"].shape == (2, 37, 40) and t["B"].shape == (2, 1000, 16) and t["C"].shape == (2, 1000, 16)
    r = W.repeat_in_time(t["x"][:, :, 3:4], 1000)
    assert r.shape == (2, 1000, 1) and r.flags["C_CONTIGUOUS"]
    for step in (0, 36, 37, 500, 999):
        assert np.array_equal(r[:, step], t["x"][:, step % 37, 3:4])
    s = W.long_ssd_inputs(1, 500, 4, 8, 32, 31, seed=6)
    assert s["x"].shape == (1, 31, 4, 8) and s["dt"].shape == (1, 500, 4) and s["B"].shape == (1, 500, 1, 32)
    # B and C vary over the whole sequence, not with the block's period
    assert not np.array_equal(s["B"][:, 31:62], s["B"][:, 0:31])
    d = W.long_decode_inputs(20, 96, 16, 7, seed=3)
    assert d["state_block"].shape == (7, 96, 16) and d["x"].shape == (20, 96) and d["B"].shape == (20, 16)
    e = W.long_ssd_decode_inputs(12, 4, 8, 32, 5, seed=4)
    assert e["state_block"].shape == (5, 4, 8, 32) and e["x"].shape == (12, 4, 8) and e["B"].shape == (12, 1, 32)
