"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises AssertionError
when the oracle disagrees with the property.  None of them re-types the oracle's
loop: they use closed forms, an unrolled sum written with cumulative sums, the
convolution form of a time-invariant SSM, algebraic invariants, hand-derived
worked examples, and library routines (numpy.logaddexp, scipy.special.expit) for
softplus and the sigmoid.  ``tests/test_oracle_mutants.py`` shows that planted
mistakes in the oracle fail at least one pin.

Sources, by page title and section:
  * "Mamba 论文精读" (youngju.dev): sec. 2.2 recurrence and Abar = exp(delta A);
    sec. 3.3 selective_scan (Bbar x = delta B x, zero initial state, update then
    read out); sec. 3.1 softplus; sec. 3.4 bias, D skip, SiLU gate; sec. 6 O(1)
    decode with a fixed state.
  * "Mamba的基础知识" (weblog-19d): state space model section (D skip term) and
    the convolution section (kernel K = (CB, CAB, ..., CA^k B, ...) for a
    time-invariant SSM).
  * "mamba->jamba" (blog.csdn.net), sec. 2.3: a small step keeps the state and
    ignores the input; parallel scan over the linear recurrence.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------------------------
# helpers (test-side, independent of the oracle's C code)
# ----------------------------------------------------------------------------------------------
def _rand_case(seed, batch=2, L=7, dim=3, N=4, softplus=True, bias=True, z=True, D=True):
    """Small random float64 case with A varying over both d and n (so an index mix-up of A,
    B or C shows), a per-channel bias and D."""
    g = np.random.default_rng(seed)
    case = dict(
        x=g.normal(size=(batch, L, dim)),
        delta=g.normal(size=(batch, L, dim)) * 0.5 if softplus else g.uniform(0.05, 0.6, (batch, L, dim)),
        A=-g.uniform(0.2, 3.0, (dim, N)).astype(np.float32),
        B=g.normal(size=(batch, L, N)),
        C=g.normal(size=(batch, L, N)),
        D=g.normal(size=dim).astype(np.float32) if D else None,
        z=g.normal(size=(batch, L, dim)) if z else None,
        delta_bias=g.uniform(-3.0, 0.5, dim).astype(np.float32) if bias else None,
        delta_softplus=softplus,
    )
    return case


def _scan(o, c, **over):
    kw = dict(c)
    kw.update(over)
    return o.scan(kw["x"], kw["delta"], kw["A"], kw["B"], kw["C"], D=kw.get("D"), z=kw.get("z"),
                  delta_bias=kw.get("delta_bias"), delta_softplus=kw.get("delta_softplus", False),
                  h0=kw.get("h0"), zoh=kw.get("zoh", False))


def unrolled(c):
    """y_t = sum_{s<=t} sum_n C_t[n] exp(A[d,n] (Lam_t - Lam_s)) delta_s B_s[n] x_s + D x_t, then the
    gate; Lam is the running sum of delta.  This is the recurrence unrolled (the product of the
    per-step Abar between s and t is the exponential of A times the summed steps).  Returns
    (y, h_L) in float64."""
    x, C, B = c["x"], c["C"], c["B"]
    A = c["A"].astype(np.float64)
    v = c["delta"] + (0.0 if c.get("delta_bias") is None else c["delta_bias"].astype(np.float64))
    dt = np.logaddexp(0.0, v) if c.get("delta_softplus") else v
    batch, L, dim = x.shape
    N = A.shape[1]
    lam = np.cumsum(dt, axis=1)
    y = np.zeros((batch, L, dim))
    hL = np.zeros((batch, dim, N))
    for t in range(L):
        for s in range(t + 1):
            dec = np.exp(A[None] * (lam[:, t, :] - lam[:, s, :])[:, :, None])          # (b, d, n)
            contrib = dec * (dt[:, s, :] * x[:, s, :])[:, :, None] * B[:, s, None, :]    # (b, d, n)
            y[:, t, :] += np.einsum("bdn,bn->bd", contrib, C[:, t, :])
            if t == L - 1:
                hL += contrib
        if c.get("D") is not None:
            y[:, t, :] += c["D"].astype(np.float64) * x[:, t, :]
        if c.get("z") is not None:
            y[:, t, :] *= c["z"][:, t, :] * expit(c["z"][:, t, :])
    return y, hL


def _close(a, b, rtol, what):
    scale = max(float(np.max(np.abs(b))), 1e-300)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


# ----------------------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------------------
def pin_worked_examples(o):
    """Hand-derived examples (tests/golden/*.json); the pages print no numeric example."""
    for name in sorted(os.listdir(GOLDEN)):
        if not name.startswith("worked_example"):
            continue
        g = json.load(open(os.path.join(GOLDEN, name)))
        i = g["inputs"]
        arr = lambda k, dt=np.float64: None if k not in i else np.array(i[k], dt)  # noqa: E731
        y, st = o.scan(arr("x"), arr("delta"), arr("A", np.float32), arr("B"), arr("C"),
                       D=arr("D", np.float32), z=arr("z"), delta_bias=arr("delta_bias", np.float32),
                       delta_softplus=g["delta_softplus"])
        _close(y, np.array(g["expected"]["y"]), g["rtol"], f"{name} y")
        _close(st, np.array(g["expected"]["last_state"]), g["rtol"], f"{name} last_state")


def pin_unrolled_sum(o):
    """I-1: brute-force unrolled sum on tiny L, all options on and off."""
    for seed, opts in enumerate([{}, dict(softplus=False, bias=False), dict(z=False, D=False),
                                 dict(bias=False), dict(batch=3, L=5, dim=2, N=8)]):
        c = _rand_case(100 + seed, **opts)
        y, st = _scan(o, c)
        yr, hr = unrolled(c)
        _close(y, yr, 1e-12, f"unrolled y {opts}")
        _close(st, hr, 1e-12, f"unrolled last_state {opts}")


def pin_lti_convolution(o):
    """I-2: with delta, B, C constant in time (the S4 / LTI case) the scan is a causal convolution
    of x with K_k = sum_n C_n Abar_n^k Bbar_n, K = (CB, CAB, CA^2B, ...); for x = 1 it has the
    geometric closed form sum_n C_n Bbar_n (1 - Abar_n^(t+1)) / (1 - Abar_n)."""
    g = np.random.default_rng(7)
    batch, L, dim, N = 2, 48, 3, 5
    dt = g.uniform(0.05, 0.5, (batch, dim))
    Bc, Cc = g.normal(size=(batch, N)), g.normal(size=(batch, N))
    A = -g.uniform(0.1, 2.0, (dim, N)).astype(np.float32)
    x = g.normal(size=(batch, L, dim))
    delta = np.broadcast_to(dt[:, None, :], (batch, L, dim)).copy()
    Bt = np.broadcast_to(Bc[:, None, :], (batch, L, N)).copy()
    Ct = np.broadcast_to(Cc[:, None, :], (batch, L, N)).copy()
    y, _ = o.scan(x, delta, A, Bt, Ct)
    k = np.arange(L)
    for b in range(batch):
        for d in range(dim):
            abar = np.exp(dt[b, d] * A[d].astype(np.float64))                      # (N,)
            K = (Cc[b] * dt[b, d] * Bc[b])[None, :] * abar[None, :] ** k[:, None]  # (L, N)
            Kk = K.sum(axis=1)
            ref = np.convolve(x[b, :, d], Kk)[:L]
            _close(y[b, :, d], ref, 1e-12, f"LTI conv b={b} d={d}")
    ones = np.ones_like(x)
    y1, _ = o.scan(ones, delta, A, Bt, Ct)
    for b in range(batch):
        for d in range(dim):
            abar = np.exp(dt[b, d] * A[d].astype(np.float64))
            ref = np.array([np.sum(Cc[b] * dt[b, d] * Bc[b] * (1 - abar ** (t + 1)) / (1 - abar)) for t in range(L)])
            _close(y1[b, :, d], ref, 1e-12, f"LTI geometric b={b} d={d}")


def pin_linearity(o):
    """I-3: for fixed delta, B, C, z, D the output is linear in x."""
    c = _rand_case(11, L=9)
    g = np.random.default_rng(12)
    x1, x2 = g.normal(size=c["x"].shape), g.normal(size=c["x"].shape)
    al, be = 0.7, -1.9
    y1, s1 = _scan(o, c, x=x1)
    y2, s2 = _scan(o, c, x=x2)
    y3, s3 = _scan(o, c, x=al * x1 + be * x2)
    _close(y3, al * y1 + be * y2, 1e-12, "linearity y")
    _close(s3, al * s1 + be * s2, 1e-12, "linearity state")


def pin_channel_independence(o):
    """I-4: channels do not interact; a channel permutation permutes the outputs."""
    c = _rand_case(21, batch=2, L=6, dim=5)
    y0, s0 = _scan(o, c)
    x = c["x"].copy()
    x[:, :, 2] += 3.0
    y1, s1 = _scan(o, c, x=x)
    other = [0, 1, 3, 4]
    assert np.array_equal(y0[:, :, other], y1[:, :, other]), "perturbing channel 2 changed other channels"
    assert np.array_equal(s0[:, other, :], s1[:, other, :]), "perturbing channel 2 changed other states"
    assert not np.allclose(y0[:, :, 2], y1[:, :, 2]), "perturbing channel 2 did not change it"
    p = np.array([3, 0, 4, 1, 2])
    cp = dict(c, x=c["x"][:, :, p], delta=c["delta"][:, :, p], z=c["z"][:, :, p], A=c["A"][p],
              D=c["D"][p], delta_bias=c["delta_bias"][p])
    yp, sp = _scan(o, cp)
    assert np.array_equal(yp, y0[:, :, p]) and np.array_equal(sp, s0[:, p, :]), "channel permutation"
    # batches are independent too
    cb = dict(c, x=c["x"][::-1].copy(), delta=c["delta"][::-1].copy(), z=c["z"][::-1].copy(),
              B=c["B"][::-1].copy(), C=c["C"][::-1].copy())
    yb, sb = _scan(o, cb)
    assert np.array_equal(yb, y0[::-1]) and np.array_equal(sb, s0[::-1]), "batch permutation"


def pin_causality(o):
    """I-5: changing any input at step t0 leaves y_t, t < t0, unchanged."""
    c = _rand_case(31, L=10)
    y0, _ = _scan(o, c)
    t0 = 6
    for k in ("x", "delta", "B", "C", "z"):
        a = c[k].copy()
        a[:, t0:] += 0.5
        y1, _ = _scan(o, c, **{k: a})
        assert np.array_equal(y0[:, :t0], y1[:, :t0]), f"changing {k} at t>={t0} changed earlier outputs"
        assert not np.allclose(y0[:, t0:], y1[:, t0:]), f"changing {k} at t>={t0} had no effect"


def pin_zero_step(o):
    """I-6: delta = 0 gives Abar = I and a vanishing input term, so the state stays 0 and
    y = D x SiLU(z); a small step moves y away from that by O(delta)."""
    c = _rand_case(41, softplus=False, bias=False)
    zero = np.zeros_like(c["delta"])
    y, st = _scan(o, c, delta=zero)
    ref = c["D"].astype(np.float64) * c["x"] * c["z"] * expit(c["z"])
    _close(y, ref, 1e-15, "delta=0 output")
    assert np.all(st == 0.0), "delta=0 must leave the state at zero"
    diffs = []
    for eps in (1e-4, 5e-5, 2.5e-5):
        ye, _ = _scan(o, c, delta=np.full_like(c["delta"], eps))
        diffs.append(np.max(np.abs(ye - ref)))
    assert diffs[0] > 0 and abs(diffs[0] / diffs[1] - 2.0) < 1e-2 and abs(diffs[1] / diffs[2] - 2.0) < 1e-2, \
        f"y - Dx SiLU(z) is not linear in a small step: {diffs}"


def pin_impulse_long_carry(o):
    """I-7: an impulse at t=0 with delta_0 = 1, then delta = 0: the state is held exactly at
    delta_0 B_0 x_0, so y_t = (C_t . B_0 + D x_t) SiLU(z_t) for every t, over 2^20 steps."""
    g = np.random.default_rng(51)
    L, N = 1 << 20, 16
    x = g.normal(size=(1, L, 1)).astype(np.float32)
    x[0, 0, 0] = 1.0
    delta = np.zeros((1, L, 1), np.float32)
    delta[0, 0, 0] = 1.0
    B = g.normal(size=(1, L, N)).astype(np.float32)
    C = g.normal(size=(1, L, N)).astype(np.float32)
    z = g.normal(size=(1, L, 1)).astype(np.float32)
    A = -np.arange(1, N + 1, dtype=np.float32)[None]
    D = np.array([0.5], np.float32)
    y, st = o.scan(x, delta, A, B, C, D=D, z=z)
    h = B[0, 0].astype(np.float64)
    zz = z[0, :, 0].astype(np.float64)
    ref = (C[0].astype(np.float64) @ h + 0.5 * x[0, :, 0].astype(np.float64)) * zz * expit(zz)
    _close(y[0, :, 0], ref, 1e-13, "impulse carry")
    _close(st[0, 0], h, 1e-15, "impulse state")


def pin_decode_equals_scan(o):
    """I-8: L single-token updates from h=0 reproduce the scan's y_t and h_L; a scan resumed from
    its own last state equals the scan over the joined sequence."""
    c = _rand_case(61, batch=2, L=8, dim=3, N=4)
    y, st = _scan(o, c)
    h = np.zeros_like(st)
    for t in range(c["x"].shape[1]):
        yt, h = o.state_update(h, c["x"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                               D=c["D"], z=c["z"][:, t], delta_bias=c["delta_bias"],
                               delta_softplus=c["delta_softplus"])
        _close(yt, y[:, t], 1e-14, f"decode step {t}")
    _close(h, st, 1e-14, "decode final state")
    L1 = 5
    first = {k: (v[:, :L1] if isinstance(v, np.ndarray) and v.ndim == 3 else v) for k, v in c.items()}
    rest = {k: (v[:, L1:] if isinstance(v, np.ndarray) and v.ndim == 3 else v) for k, v in c.items()}
    ya, sa = _scan(o, first)
    yb, sb = _scan(o, rest, h0=sa)
    _close(np.concatenate([ya, yb], axis=1), y, 1e-14, "scan resumed from last_state")
    _close(sb, st, 1e-14, "resumed last_state")


def _compose(p, q):
    """The scan operator on (a, b) pairs: (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2)."""
    return (p[0] * q[0], q[0] * p[1] + q[1])


def _fold_random_tree(pairs, g):
    if len(pairs) == 1:
        return pairs[0]
    k = int(g.integers(1, len(pairs)))
    return _compose(_fold_random_tree(pairs[:k], g), _fold_random_tree(pairs[k:], g))


def pin_associative_scan(o):
    """I-9: the last state equals the fold of the per-step pairs (Abar_t, Bbar_t x_t) under the
    associative operator, for every bracketing (the parallel-scan view of the recurrence)."""
    c = _rand_case(71, batch=2, L=8, dim=3, N=4)
    _, st = _scan(o, c)
    v = c["delta"] + c["delta_bias"].astype(np.float64)
    dt = np.logaddexp(0.0, v)
    A = c["A"].astype(np.float64)
    a = np.exp(dt[..., None] * A[None, None])                          # (b, t, d, n)
    u = (dt * c["x"])[..., None] * c["B"][:, :, None, :]               # (b, t, d, n)
    pairs = [(a[:, t], u[:, t]) for t in range(a.shape[1])]
    g = np.random.default_rng(72)
    for _ in range(12):
        tot = _fold_random_tree(pairs, g)
        _close(tot[1], st, 1e-13, "bracketing of the scan operator")
        _close(tot[0], np.prod(a, axis=1), 1e-13, "decay product")


def pin_special_values(o):
    """I-10: softplus(0) = ln 2, softplus is log(1+e^v) at both tails, SiLU(0) = 0 and
    SiLU(1) = 1/(1+e^-1); a zero gate zeroes y; absent D or bias equal zero D or bias."""
    assert abs(o.softplus(0.0) - math.log(2.0)) <= 1e-16
    assert o.softplus(800.0) == 800.0 and o.softplus(-800.0) == 0.0
    for v in (-30.0, -5.0, -0.3, 0.7, 4.0, 25.0):
        assert abs(o.softplus(v) - float(np.logaddexp(0.0, v))) <= 1e-15 * max(1.0, abs(v)), v
    assert abs(o.softplus(-30.0) - math.exp(-30.0)) <= 1e-12 * math.exp(-30.0)
    assert o.silu(0.0) == 0.0
    assert abs(o.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-16
    for zv in (-40.0, -2.5, 0.3, 9.0):
        assert abs(o.silu(zv) - zv * float(expit(zv))) <= 1e-15 * max(1.0, abs(zv)), zv
    c = _rand_case(81)
    y, _ = _scan(o, c, z=np.zeros_like(c["z"]))
    assert np.all(y == 0.0), "z = 0 must zero the output"
    ya, sa = _scan(o, c, D=None)
    yb, sb = _scan(o, c, D=np.zeros_like(c["D"]))
    assert np.array_equal(ya, yb) and np.array_equal(sa, sb), "D=None differs from D=0"
    ya, sa = _scan(o, c, delta_bias=None)
    yb, sb = _scan(o, c, delta_bias=np.zeros_like(c["delta_bias"]))
    assert np.array_equal(ya, yb) and np.array_equal(sa, sb), "bias=None differs from bias=0"


def pin_storage_widening(o):
    """I-11: bf16 bit patterns and fp32 values widen exactly; a bf16-stored scan equals the same
    scan on the widened float64 values."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x8000, 0x3F81, 0x0080], np.uint16)
    ref = np.array([1.0, -2.0, 2.0 ** -133, np.inf, -np.inf, -0.0, 1.0 + 2.0 ** -7, 2.0 ** -126])
    w = o.widen(bits)
    assert np.array_equal(w, ref) and np.signbit(w[5]), f"bf16 widening {w}"
    assert np.isnan(o.widen(np.array([0x7FC0], np.uint16))[0])
    f = np.array([1.5, -3.25e-39, 3.4028235e38], np.float32)
    assert np.array_equal(o.widen(f), f.astype(np.float64))
    g = np.random.default_rng(91)
    shape = (2, 6, 3)
    to_bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncation
    wid = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)           # noqa: E731
    xb, db, zb = (to_bits(g.normal(size=shape)) for _ in range(3))
    Bb, Cb = (to_bits(g.normal(size=(2, 6, 4))) for _ in range(2))
    A = -g.uniform(0.2, 2.0, (3, 4)).astype(np.float32)
    y1, s1 = o.scan(xb, db, A, Bb, Cb, z=zb, delta_softplus=True)
    y2, s2 = o.scan(wid(xb), wid(db), A, wid(Bb), wid(Cb), z=wid(zb), delta_softplus=True)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2), "bf16 storage path differs"
    y3, s3 = o.scan(wid(xb).astype(np.float32), wid(db).astype(np.float32), A, wid(Bb).astype(np.float32),
                    wid(Cb).astype(np.float32), z=wid(zb).astype(np.float32), delta_softplus=True)
    assert np.array_equal(y1, y3) and np.array_equal(s1, s3), "fp32 storage path differs"


def pin_channel_selection(o):
    """scan_channels (used to sample full-size outputs) equals the full scan on those channels."""
    c = _rand_case(95, batch=3, L=9, dim=4)
    y, st = _scan(o, c)
    sb, sd = np.array([0, 2, 1, 2]), np.array([3, 0, 1, 3])
    yc, sc = o.scan_channels(c["x"], c["delta"], c["A"], c["B"], c["C"], sb, sd, D=c["D"], z=c["z"],
                             delta_bias=c["delta_bias"], delta_softplus=True)
    for k in range(len(sb)):
        assert np.array_equal(yc[k], y[sb[k], :, sd[k]]) and np.array_equal(sc[k], st[sb[k], sd[k]])


# ----------------------------------------------------------------------------------------------
# the depthwise causal convolution before the scan ("Mamba 论文精读" sec. 3.4, MambaBlock listing:
# Conv1d with groups = channels, padding K-1, first L outputs kept, then SiLU)
# ----------------------------------------------------------------------------------------------
def _conv_case(seed, batch=2, L=11, dim=5, K=4):
    g = np.random.default_rng(seed)
    return (g.normal(size=(batch, L, dim)), g.normal(size=(dim, K)).astype(np.float32),
            g.normal(size=dim).astype(np.float32))


def pin_conv_library_convolution(o):
    """Without SiLU and initial state, each channel is numpy.convolve of the input with the
    reversed kernel (Conv1d is a cross-correlation), cut to the first L outputs, plus the bias."""
    for K in (1, 2, 3, 4):
        x, w, bias = _conv_case(100 + K, K=K)
        y, _ = o.causal_conv1d(x, w, bias, silu=False)
        for b in range(x.shape[0]):
            for d in range(x.shape[2]):
                ref = np.convolve(x[b, :, d], w[d, ::-1].astype(np.float64))[: x.shape[1]] + float(bias[d])
                _close(y[b, :, d], ref, 1e-13, f"conv K={K} b={b} d={d}")


def pin_conv_impulse(o):
    """A unit impulse at t0 gives y[t0 + j] = bias + w[K-1-j] for j < K and bias elsewhere."""
    K, L, t0 = 4, 12, 5
    x = np.zeros((1, L, 2))
    x[0, t0, 1] = 1.0
    w = np.array([[1.0, 2.0, 3.0, 4.0], [0.5, -1.5, 2.5, -3.5]], np.float32)
    bias = np.array([0.0, 0.25], np.float32)
    y, fin = o.causal_conv1d(x, w, bias, silu=False)
    ref = np.full(L, 0.25)
    for j in range(K):
        ref[t0 + j] += float(w[1, K - 1 - j])
    _close(y[0, :, 1], ref, 0.0, "impulse response")
    _close(y[0, :, 0], np.zeros(L), 0.0, "silent channel")
    _close(fin[0, 1], x[0, L - 3:, 1], 0.0, "final state = last K-1 inputs")


def pin_conv_silu(o):
    """SiLU on the output is y * sigmoid(y) of the output without it (scipy.special.expit)."""
    x, w, bias = _conv_case(7)
    y0, _ = o.causal_conv1d(x, w, bias, silu=False)
    y1, _ = o.causal_conv1d(x, w, bias, silu=True)
    _close(y1, y0 * expit(y0), 1e-13, "silu(conv)")


def pin_conv_chaining(o):
    """Splitting the sequence and passing the final state of the first part as the initial
    state of the second gives the unsplit result; for L < K-1 the final state keeps the tail
    of the initial state."""
    x, w, bias = _conv_case(9, L=13, K=4)
    y, fin = o.causal_conv1d(x, w, bias, silu=True)
    for cut in (1, 2, 3, 7):
        y1, f1 = o.causal_conv1d(x[:, :cut], w, bias, silu=True)
        y2, f2 = o.causal_conv1d(x[:, cut:], w, bias, init_state=f1, silu=True)
        _close(np.concatenate([y1, y2], axis=1), y, 1e-13, f"chained at {cut}")
        _close(f2, fin, 0.0, f"final state chained at {cut}")
    init = np.random.default_rng(3).normal(size=(2, 5, 3))
    _, fs = o.causal_conv1d(x[:, :1], w, bias, init_state=init, silu=False)
    _close(fs[:, :, :2], init[:, :, 1:], 0.0, "short sequence keeps the initial state's tail")
    _close(fs[:, :, 2], x[:, 0, :], 0.0, "short sequence appends the input")


def pin_conv_decode_equals_fwd(o):
    """Feeding the tokens one by one through the decode update reproduces the full convolution
    (outputs and final state), from zeros and from a given initial state."""
    x, w, bias = _conv_case(11, L=9, K=4)
    init = np.random.default_rng(4).normal(size=(2, 5, 3))
    for st0 in (None, init):
        y, fin = o.causal_conv1d(x, w, bias, init_state=st0, silu=True)
        st = np.zeros((2, 5, 3)) if st0 is None else st0.copy()
        for t in range(x.shape[1]):
            yt, st = o.conv1d_update(st, x[:, t], w, bias, silu=True)
            _close(yt, y[:, t], 1e-13, f"decode step {t}")
        _close(st, fin, 0.0, "decode final state")


def pin_conv_causality(o):
    """Changing the input at t changes no output before t."""
    x, w, bias = _conv_case(13, L=10)
    y, _ = o.causal_conv1d(x, w, bias, silu=True)
    x2 = x.copy()
    x2[:, 6] += 3.0
    y2, _ = o.causal_conv1d(x2, w, bias, silu=True)
    _close(y2[:, :6], y[:, :6], 0.0, "outputs before the change")
    assert np.all(np.abs(y2[:, 6] - y[:, 6]) > 0), "the changed step must move its own output"


# ----------------------------------------------------------------------------------------------
# the backward pass: central finite differences of sum(dy * y) through the (pinned) forward
# ----------------------------------------------------------------------------------------------
def _fd_grad(o, c, dy, name, eps):
    """Central differences of sum(dy * y) w.r.t. every element of c[name]."""
    base = c[name]
    grad = np.zeros(base.shape)
    flat = grad.reshape(-1)
    for i in range(base.size):
        up, dn = base.copy(), base.copy()
        up.reshape(-1)[i] += eps
        dn.reshape(-1)[i] -= eps
        # parameters are stored in fp32: use the perturbation the storage actually holds
        h = float(up.reshape(-1)[i]) - float(dn.reshape(-1)[i])
        yu, _ = _scan(o, c, **{name: up})
        yd, _ = _scan(o, c, **{name: dn})
        flat[i] = float(np.sum(dy * (yu - yd))) / h
    return grad


def pin_backward_finite_differences(o):
    """Every gradient of the adjoint oracle matches central finite differences of the forward
    oracle (fp64 for the activations, the fp32-representable step for A, D and the bias)."""
    for seed, softplus, z, D, bias in ((21, True, True, True, True), (22, False, False, True, False),
                                        (23, True, True, False, False)):
        c = _rand_case(seed, batch=2, L=5, dim=3, N=3, softplus=softplus, bias=bias, z=z, D=D)
        dy = np.random.default_rng(seed + 100).normal(size=c["x"].shape)
        g = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy, D=c["D"], z=c["z"],
                       delta_bias=c["delta_bias"], delta_softplus=softplus)
        checks = [("x", "dx", 1e-6, 1e-6), ("delta", "ddelta", 1e-6, 1e-6), ("B", "dB", 1e-6, 1e-6),
                  ("C", "dC", 1e-6, 1e-6), ("A", "dA", 1e-3, 1e-5)]
        if z:
            checks.append(("z", "dz", 1e-6, 1e-6))
        if D:
            checks.append(("D", "dD", 1e-3, 1e-5))
        if bias:
            checks.append(("delta_bias", "ddelta_bias", 1e-3, 1e-5))
        for name, gname, eps, rtol in checks:
            fd = _fd_grad(o, c, dy, name, eps)
            _close(g[gname], fd, rtol, f"d{name} (seed {seed})")


def pin_backward_zoh_finite_differences(o):
    """The adjoint of the exact zero-order-hold forward ("Mamba 论文精读" sec. 2.2) matches central
    finite differences of that (pinned) forward: ordinary steps, steps small enough that
    dt * A is ~1e-3 (where (dt abar - phi) / A cancels), and a state with A = 0 exactly."""
    cases = [(41, True, True, True, True, None), (42, False, True, True, False, "small"),
             (43, True, False, False, True, "zero_a")]
    for seed, softplus, z, D, bias, kind in cases:
        c = _rand_case(seed, batch=2, L=5, dim=3, N=3, softplus=softplus, bias=bias, z=z, D=D)
        if kind == "small":
            c["delta"] = c["delta"] * 0.004
        if kind == "zero_a":
            c["A"][1, 2] = 0.0
        c["zoh"] = True
        dy = np.random.default_rng(seed + 100).normal(size=c["x"].shape)
        g = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy, D=c["D"], z=c["z"],
                       delta_bias=c["delta_bias"], delta_softplus=softplus, zoh=True)
        checks = [("x", "dx", 1e-6, 1e-6), ("delta", "ddelta", 1e-7 if kind == "small" else 1e-6, 1e-6),
                  ("B", "dB", 1e-6, 1e-6), ("C", "dC", 1e-6, 1e-6), ("A", "dA", 1e-3, 1e-5)]
        if z:
            checks.append(("z", "dz", 1e-6, 1e-6))
        if bias:
            checks.append(("delta_bias", "ddelta_bias", 1e-3, 1e-5))
        for name, gname, eps, rtol in checks:
            fd = _fd_grad(o, c, dy, name, eps)
            _close(g[gname], fd, rtol, f"ZOH d{name} (seed {seed}, {kind or 'ordinary'})")
        # and the ZOH adjoint is not the Delta B one
        g0 = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy, D=c["D"], z=c["z"],
                        delta_bias=c["delta_bias"], delta_softplus=softplus)
        assert np.max(np.abs(g0["dA"] - g["dA"])) > 1e-6 * np.max(np.abs(g["dA"])), "ZOH dA equals the Delta B dA"


def pin_backward_linear_in_dy(o):
    """The gradients are linear in dy."""
    c = _rand_case(31, batch=1, L=6, dim=2, N=3)
    g = np.random.default_rng(32)
    dy1, dy2 = g.normal(size=c["x"].shape), g.normal(size=c["x"].shape)
    kw = dict(D=c["D"], z=c["z"], delta_bias=c["delta_bias"], delta_softplus=True)
    r1 = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy1, **kw)
    r2 = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy2, **kw)
    r3 = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], 2.0 * dy1 - 3.0 * dy2, **kw)
    for k in r1:
        _close(r3[k], 2.0 * r1[k] - 3.0 * r2[k], 1e-12, f"linearity of {k}")


def pin_backward_euler_identities(o):
    """Euler's identity for homogeneous functions, on the loss l = sum(dy * y).  For fixed delta,
    A and z, y is linear in x (the input term and the D skip), and y - D x silu(z) is linear in B
    and, separately, in C (the state is linear in B; the read-out in C).  So, exactly:
        sum(x dx) = l,   sum(B dB) = sum(C dC) = l - l_D,   sum(D dD) = l_D,
    with l_D = sum(dy D x silu(z)).  This checks dx, dB, dC and dD against the forward oracle
    without finite differences, for both input terms (delta B and the exact zero-order hold)."""
    for seed, softplus, z, D, bias, zoh in ((51, True, True, True, True, False), (52, False, False, True, False, False),
                                             (53, True, True, False, True, False), (54, True, True, True, True, True)):
        c = _rand_case(seed, batch=2, L=6, dim=3, N=4, softplus=softplus, bias=bias, z=z, D=D)
        c["zoh"] = zoh
        dy = np.random.default_rng(seed + 200).normal(size=c["x"].shape)
        y, _ = _scan(o, c)
        g = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy, D=c["D"], z=c["z"],
                       delta_bias=c["delta_bias"], delta_softplus=softplus, zoh=zoh)
        gate = c["z"] * expit(c["z"]) if z else 1.0
        loss = float(np.sum(dy * y))
        loss_d = float(np.sum(dy * c["D"].astype(np.float64) * c["x"] * gate)) if D else 0.0
        scale = float(np.sum(np.abs(dy * y))) + abs(loss_d)
        what = f"seed {seed}{', ZOH' if zoh else ''}"
        for got, want, name in ((np.sum(c["x"] * g["dx"]), loss, "sum(x dx) = l"),
                                (np.sum(c["B"] * g["dB"]), loss - loss_d, "sum(B dB) = l - l_D"),
                                (np.sum(c["C"] * g["dC"]), loss - loss_d, "sum(C dC) = l - l_D")):
            assert abs(float(got) - want) <= 1e-12 * scale, f"{name} ({what}): {float(got):.15e} vs {want:.15e}"
        if D:
            got = float(np.sum(c["D"].astype(np.float64) * g["dD"]))
            assert abs(got - loss_d) <= 1e-12 * scale, f"sum(D dD) = l_D ({what}): {got:.15e} vs {loss_d:.15e}"


def pin_backward_closed_forms(o):
    """Exact identities for the gradients the homogeneity pin does not reach:
      * scale invariance: replacing (delta_eff, A, B) by (s delta_eff, A / s, B / s) leaves every
        decay exp(delta A) and every input term (delta B for "Mamba 论文精读" sec. 3.3; (exp(delta A)
        - 1) / A B for the exact hold of sec. 2.2) unchanged, so d/ds at s = 1 gives
        sum(delta_eff g_eff) = sum(A dA) + sum(B dB), g_eff = ddelta / softplus'(v) with softplus
        (the logistic function, scipy's expit) and ddelta without;
      * the gate: y = y0 silu(z) with y0 free of z, so dz = dy y (1 + z (1 - sigma(z))) / z;
      * the skip: dD[d] = sum over (b, t) of dy x silu(z);
      * the bias enters as delta does: ddelta_bias[d] = sum over (b, t) of ddelta."""
    for seed, softplus, zoh in ((61, True, False), (62, False, False), (63, True, True), (64, False, True)):
        c = _rand_case(seed, batch=2, L=6, dim=3, N=4, softplus=softplus, bias=True, z=True, D=True)
        c["zoh"] = zoh
        dy = np.random.default_rng(seed + 300).normal(size=c["x"].shape)
        y, _ = _scan(o, c)
        g = o.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], dy, D=c["D"], z=c["z"],
                       delta_bias=c["delta_bias"], delta_softplus=softplus, zoh=zoh)
        what = f"seed {seed}{', softplus' if softplus else ''}{', ZOH' if zoh else ''}"
        v = c["delta"] + c["delta_bias"].astype(np.float64)
        dt = np.logaddexp(0.0, v) if softplus else v
        g_eff = g["ddelta"] / expit(v) if softplus else g["ddelta"]
        A = c["A"].astype(np.float64)
        lhs = float(np.sum(dt * g_eff))
        rhs = float(np.sum(A * g["dA"]) + np.sum(c["B"] * g["dB"]))
        scale = float(np.sum(np.abs(dt * g_eff)) + np.sum(np.abs(A * g["dA"])) + np.sum(np.abs(c["B"] * g["dB"])))
        assert abs(lhs - rhs) <= 1e-12 * scale, f"scale invariance ({what}): {lhs:.15e} vs {rhs:.15e}"
        zz = c["z"]
        _close(g["dz"], dy * y * (1.0 + zz * (1.0 - expit(zz))) / zz, 1e-11, f"dz closed form ({what})")
        _close(g["dD"], np.sum(dy * c["x"] * zz * expit(zz), axis=(0, 1)), 1e-12, f"dD closed form ({what})")
        _close(g["ddelta_bias"], np.sum(g["ddelta"], axis=(0, 1)), 1e-12, f"ddelta_bias = sum ddelta ({what})")


# ----------------------------------------------------------------------------------------------
# the exact zero-order hold ("Mamba 论文精读" sec. 2.2: Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B)
# ----------------------------------------------------------------------------------------------
def _lti_zoh(o, x, dt, A, Bv, Cv):
    """One channel, constant Delta / B / C, as a (1, L, 1) scan with the ZOH flag."""
    L, N = x.size, A.size
    return o.scan(x.reshape(1, L, 1), np.full((1, L, 1), dt), A.reshape(1, N).astype(np.float32),
                  np.tile(Bv, (1, L, 1)), np.tile(Cv, (1, L, 1)), zoh=True)


def pin_zoh_steady_state(o):
    """Under a constant input x = 1 the exact ZOH state tends to the continuous fixed point
    -B/A, whatever the step (the Delta B form tends to Delta B / (1 - e^{Delta A}) instead)."""
    A = np.array([-0.5, -1.0, -2.0, -4.0])
    Bv = np.array([1.0, -2.0, 0.5, 3.0])
    Cv = np.ones(4)
    for dt in (0.01, 0.3, 2.0):
        L = int(60.0 / (dt * 0.5)) + 1
        _, st = _lti_zoh(o, np.ones(L), dt, A, Bv, Cv)
        _close(st[0, 0], -Bv / A, 1e-9, f"ZOH fixed point, dt={dt}")


def pin_zoh_semigroup(o):
    """ZOH is exact for piecewise-constant input: one step of 2 Delta equals two steps of Delta
    with the same input held."""
    A = np.array([-0.3, -1.7, -5.0])
    Bv, Cv = np.array([0.7, -1.1, 2.0]), np.array([1.0, 0.5, -2.0])
    for dt in (0.05, 0.8):
        _, one = _lti_zoh(o, np.array([1.3]), 2 * dt, A, Bv, Cv)
        _, two = _lti_zoh(o, np.array([1.3, 1.3]), dt, A, Bv, Cv)
        _close(one, two, 1e-12, f"ZOH semigroup, dt={dt}")


def pin_zoh_small_step_limit(o):
    """As Delta -> 0 the exact ZOH input term agrees with Delta B to first order: the states of
    the two forms differ by O(Delta^2 A) after one step."""
    A = np.array([-1.0, -3.0])
    Bv, Cv = np.array([2.0, -1.0]), np.array([1.0, 1.0])
    prev = None
    for dt in (1e-2, 1e-3, 1e-4):
        _, zoh = _lti_zoh(o, np.array([1.0]), dt, A, Bv, Cv)
        plain, _ = o.scan(np.ones((1, 1, 1)), np.full((1, 1, 1), dt), A.reshape(1, 2).astype(np.float32),
                          Bv.reshape(1, 1, 2), Cv.reshape(1, 1, 2))
        diff = float(np.max(np.abs(zoh[0, 0] - dt * Bv)))
        # expm1(dt a)/a - dt = dt^2 a / 2 + O(dt^3)
        ref = float(np.max(np.abs(dt * dt * A / 2 * Bv)))
        assert abs(diff - ref) <= 0.02 * ref, f"ZOH vs Delta B at dt={dt}: {diff} vs {ref}"
        if prev is not None:
            assert diff < prev / 50, "the ZOH / Delta B difference must shrink like Delta^2"
        prev = diff


def pin_zoh_decode_equals_scan(o):
    """The ZOH decode step run token by token equals the ZOH scan."""
    c = _rand_case(41, batch=2, L=6, dim=3, N=4)
    y, st = o.scan(c["x"], c["delta"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"], delta_bias=c["delta_bias"],
                   delta_softplus=True, zoh=True)
    s = np.zeros((2, 3, 4))
    for t in range(6):
        yt, s = o.state_update(s, c["x"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t], D=c["D"],
                               z=c["z"][:, t], delta_bias=c["delta_bias"], delta_softplus=True, zoh=True)
        _close(yt, y[:, t], 1e-12, f"ZOH decode step {t}")
    _close(s, st, 1e-12, "ZOH decode state")


# ----------------------------------------------------------------------------------------------
# Mamba-2 SSD ("Mamba 论文精读" sec. 4.1-4.2, 5.2)
# ----------------------------------------------------------------------------------------------
def _ssd_case(seed, batch=2, L=9, H=4, P=3, N=5, G=2, softplus=True):
    g = np.random.default_rng(seed)
    return dict(x=g.normal(size=(batch, L, H, P)), dt=g.normal(size=(batch, L, H)) * 0.5,
                A=-g.uniform(0.3, 3.0, H).astype(np.float32), B=g.normal(size=(batch, L, G, N)),
                C=g.normal(size=(batch, L, G, N)), D=g.normal(size=H).astype(np.float32),
                z=g.normal(size=(batch, L, H, P)), dt_bias=g.uniform(-2.0, 0.5, H).astype(np.float32),
                dt_softplus=softplus)


def pin_ssd_equals_selective_scan(o):
    """A Mamba-2 head is a selective scan whose channels share one dt, one scalar A and their
    group's B and C: mapping every head to headdim channels of the (pinned) scan oracle gives
    the same y and states."""
    c = _ssd_case(51)
    y, fin = o.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"], dt_bias=c["dt_bias"],
                   dt_softplus=True)
    batch, L, H, P = c["x"].shape
    G, N = c["B"].shape[2:]
    hpg = H // G
    for g in range(G):
        heads = range(g * hpg, (g + 1) * hpg)
        x1 = np.concatenate([c["x"][:, :, h, :] for h in heads], axis=2)
        d1 = np.concatenate([np.repeat(c["dt"][:, :, h:h + 1], P, axis=2) for h in heads], axis=2)
        z1 = np.concatenate([c["z"][:, :, h, :] for h in heads], axis=2)
        A1 = np.concatenate([np.full((P, N), c["A"][h], np.float32) for h in heads], axis=0)
        D1 = np.concatenate([np.full(P, c["D"][h], np.float32) for h in heads])
        b1 = np.concatenate([np.full(P, c["dt_bias"][h], np.float32) for h in heads])
        y1, st1 = o.scan(x1, d1, A1, c["B"][:, :, g, :], c["C"][:, :, g, :], D=D1, z=z1, delta_bias=b1,
                         delta_softplus=True)
        for i, h in enumerate(heads):
            _close(y[:, :, h, :], y1[:, :, i * P:(i + 1) * P], 1e-13, f"SSD head {h} vs selective scan")
            _close(fin[:, h], st1[:, i * P:(i + 1) * P, :], 1e-13, f"SSD state {h}")


def pin_ssd_dual_matrix_form(o):
    """The duality of sec. 4.1: without gate and skip, y = (L o C B^T)(dt x) per head, where
    L[i, j] = exp(sum_{k=j+1..i} dt_k A) for j <= i and 0 above the diagonal (a masked,
    semi-separable matrix), computed with numpy matmuls."""
    c = _ssd_case(52, L=11, softplus=False)
    c["dt"] = np.abs(c["dt"])
    y, _ = o.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"])
    batch, L, H, P = c["x"].shape
    G = c["B"].shape[2]
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            dt = c["dt"][b, :, h]
            cum = np.cumsum(dt * float(c["A"][h]))
            mask = np.tril(np.exp(cum[:, None] - cum[None, :]))
            M = mask * (c["C"][b, :, g, :] @ c["B"][b, :, g, :].T)
            ref = M @ (dt[:, None] * c["x"][b, :, h, :])
            _close(y[b, :, h, :], ref, 1e-12, f"SSD dual form b={b} h={h}")


def pin_ssd_resume_from_state(o):
    """Running the layer over L steps equals running it over the first k steps and then over the
    rest from the state it left (the state is the whole memory of the recurrence), for y and the
    final state; also with a nonzero entering state for the first part."""
    c = _ssd_case(53, L=13)
    g = np.random.default_rng(54)
    batch, L, H, P = c["x"].shape
    N = c["B"].shape[3]
    h0 = g.normal(size=(batch, H, P, N))
    kw = dict(D=c["D"], z=c["z"], dt_bias=c["dt_bias"], dt_softplus=True)
    y, fin = o.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], h0=h0, **kw)
    for k in (1, 6, 12):
        cut = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
        y1, f1 = o.ssd(cut(c["x"], 0, k), cut(c["dt"], 0, k), c["A"], cut(c["B"], 0, k), cut(c["C"], 0, k), h0=h0,
                       D=c["D"], z=cut(c["z"], 0, k), dt_bias=c["dt_bias"], dt_softplus=True)
        y2, f2 = o.ssd(cut(c["x"], k, L), cut(c["dt"], k, L), c["A"], cut(c["B"], k, L), cut(c["C"], k, L), h0=f1,
                       D=c["D"], z=cut(c["z"], k, L), dt_bias=c["dt_bias"], dt_softplus=True)
        _close(np.concatenate([y1, y2], axis=1), y, 1e-13, f"SSD resumed at {k}: y")
        _close(f2, fin, 1e-13, f"SSD resumed at {k}: final state")
    # and the entering state matters: a zero one gives a different result
    y0, _ = o.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], **kw)
    assert np.max(np.abs(y0 - y)) > 1e-3 * np.max(np.abs(y)), "the entering state had no effect"


def pin_discretisation_scale_invariance(o):
    """The discretisation depends on the step only through delta A (the decay exp(delta A)) and
    delta B (the input term delta B x of "Mamba 论文精读" sec. 3.3; the exact hold
    (exp(delta A) - 1) / A B of sec. 2.2 is the same under the map).  So replacing (delta, A, B)
    by (s delta, A / s, B / s) leaves y and the final state unchanged, for the selective scan with
    either input term and for the SSD layer (whose A is one scalar per head).  With s a power of
    two every product is unchanged bit for bit, so the results must be equal exactly.  Scaling
    delta alone must change them."""
    for s_ in (2.0, 0.25):
        for zoh in (False, True):
            c = _rand_case(71, batch=2, L=7, dim=3, N=4, softplus=False, bias=False, z=True, D=True)
            c["zoh"] = zoh
            y0, h0 = _scan(o, c)
            y1, h1 = _scan(o, c, delta=c["delta"] * s_, A=(c["A"] / np.float32(s_)).astype(np.float32), B=c["B"] / s_)
            assert np.array_equal(y0, y1) and np.array_equal(h0, h1), f"scan scale invariance (s {s_}, zoh {zoh})"
            y2, _ = _scan(o, c, delta=c["delta"] * s_)
            assert not np.allclose(y0, y2), "scaling delta alone left y unchanged"
        c = _ssd_case(72, softplus=False)
        c["dt"] = np.abs(c["dt"])
        kw = dict(D=c["D"], z=c["z"])
        y0, f0 = o.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], **kw)
        y1, f1 = o.ssd(c["x"], c["dt"] * s_, (c["A"] / np.float32(s_)).astype(np.float32), c["B"] / s_, c["C"], **kw)
        assert np.array_equal(y0, y1) and np.array_equal(f0, f1), f"SSD scale invariance (s {s_})"


ALL_PINS = [pin_worked_examples, pin_unrolled_sum, pin_lti_convolution, pin_linearity,
            pin_channel_independence, pin_causality, pin_zero_step, pin_impulse_long_carry,
            pin_decode_equals_scan, pin_associative_scan, pin_special_values, pin_storage_widening,
            pin_channel_selection, pin_conv_library_convolution, pin_conv_impulse, pin_conv_silu,
            pin_conv_chaining, pin_conv_decode_equals_fwd, pin_conv_causality, pin_backward_finite_differences,
            pin_backward_zoh_finite_differences, pin_backward_linear_in_dy, pin_backward_euler_identities, pin_backward_closed_forms, pin_zoh_steady_state, pin_zoh_semigroup, pin_zoh_small_step_limit,
            pin_zoh_decode_equals_scan, pin_ssd_equals_selective_scan, pin_ssd_dual_matrix_form,
            pin_ssd_resume_from_state, pin_discretisation_scale_invariance]
