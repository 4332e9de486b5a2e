"""The C ABI (include/ssm.h) on the host: the library loads, exports every declared symbol, and its
argument validation returns the documented statuses.  Every call here fails validation (or has
nothing to do) before any HIP call, so no GPU is needed; the pointers are never dereferenced."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_61_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3
F32, BF16 = 0, 1
P = 0x7F0000000000  # a 256-byte aligned fake device address; each tensor gets its own region
GAP = 1 << 32


def fake(i, off=0):
    return P + i * GAP + off


@pytest.fixture(scope="module")
def lib():
    from selective_state_space_61_amd import build as b
    if b.is_stale():
        b.build()
    return ssm.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SSM_API\s+[\w\s\*]*?\b(ssm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(ssm.EXPORTED)


def test_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ssm.LIBRARY], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT\s+(ssm_\w+)", out.stdout))
    assert set(declared_symbols()) <= exported
    # nothing else of ours leaks out of the library
    assert {s for s in exported if s.startswith("ssm")} == set(declared_symbols())


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define SSM_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.ssm_abi_version() == ver
    names = [lib.ssm_status_string(i).decode() for i in range(5)]
    assert names == ["SSM_OK", "SSM_ERR_INVALID_ARG", "SSM_ERR_UNSUPPORTED", "SSM_ERR_MISALIGNED", "SSM_ERR_HIP"]
    assert lib.ssm_status_string(99).decode() == "SSM_ERR_UNKNOWN"


def scan(lib, batch=2, seqlen=8, dim=16, dstate=16, dtype=F32, x=fake(0), delta=fake(1), A=fake(2), B=fake(3),
         C=fake(4), D=fake(5), z=fake(6), bias=fake(7), softplus=1, y=fake(8), state=fake(9), opts=None):
    if opts is None:
        return lib.ssm_scan_fwd(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, bias, softplus, y, state,
                                None)
    return lib.ssm_scan_fwd_ex(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, bias, softplus, y, state,
                               None, ctypes.byref(opts))


def update(lib, batch=2, dim=16, dstate=16, dtype=F32, state=fake(0), x=fake(1), delta=fake(2), A=fake(3),
           B=fake(4), C=fake(5), D=fake(6), z=fake(7), bias=fake(8), softplus=1, y=fake(9)):
    return lib.ssm_state_update(batch, dim, dstate, dtype, state, x, delta, A, B, C, D, z, bias, softplus, y, None)


def err(lib):
    return lib.ssm_last_error().decode()


@pytest.mark.parametrize("kw", [dict(batch=-1), dict(seqlen=-5), dict(dim=-2), dict(dstate=-4)])
def test_scan_negative_sizes(lib, kw):
    assert scan(lib, **kw) == INVALID and "negative" in err(lib)


@pytest.mark.parametrize("n", [3, 5, 12, 128, 0])
def test_scan_unsupported_dstate(lib, n):
    assert scan(lib, dstate=n) == UNSUPPORTED and "dstate" in err(lib)


def test_scan_unsupported_dtype(lib):
    assert scan(lib, dtype=7) == UNSUPPORTED


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "y"])
def test_scan_null_required(lib, name):
    assert scan(lib, **{name: None}) == INVALID and "NULL" in err(lib)


def test_scan_optional_may_be_null_but_nothing_to_do(lib):
    # batch == 0 or dim == 0: valid, nothing enqueued, even with NULL tensors
    assert scan(lib, batch=0, x=None, delta=None, A=None, B=None, C=None, D=None, z=None, bias=None, y=None,
                state=None) == OK
    assert scan(lib, dim=0) == OK


@pytest.mark.parametrize("name,dtype,off", [("x", F32, 2), ("delta", BF16, 1), ("A", F32, 2), ("y", F32, 1),
                                            ("state", F32, 2), ("D", F32, 1), ("bias", F32, 3), ("z", BF16, 1)])
def test_scan_misaligned(lib, name, dtype, off):
    base = {"x": 0, "delta": 1, "A": 2, "B": 3, "C": 4, "D": 5, "z": 6, "bias": 7, "y": 8, "state": 9}[name]
    assert scan(lib, dtype=dtype, **{name: fake(base, off)}) == MISALIGNED


def test_scan_bf16_bc_pairs_need_4_byte_alignment(lib):
    assert scan(lib, dtype=BF16, B=fake(3, 2)) == MISALIGNED and "B and C" in err(lib)
    assert scan(lib, dtype=BF16, C=fake(4, 2)) == MISALIGNED
    # with an odd dstate the pair path is not used; 2-byte alignment is enough (not launched: dim=0)
    assert scan(lib, dtype=BF16, dstate=1, B=fake(3, 2), dim=0) == OK


@pytest.mark.parametrize("a,b", [("y", "x"), ("y", "delta"), ("y", "z"), ("y", "B"), ("state", "A"),
                                 ("state", "y"), ("y", "D")])
def test_scan_output_overlap(lib, a, b):
    base = {"x": 0, "delta": 1, "A": 2, "B": 3, "C": 4, "D": 5, "z": 6, "bias": 7, "y": 8, "state": 9}
    assert scan(lib, **{a: fake(base[b], 4)}) == INVALID and "overlap" in err(lib)


def test_scan_opts_validation(lib):
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(3, 0)) == UNSUPPORTED
    assert scan(lib, dstate=4, opts=ssm.ScanOpts(8, 0)) == UNSUPPORTED     # more chains than states
    assert scan(lib, dstate=64, opts=ssm.ScanOpts(4, 0)) == UNSUPPORTED    # 16 scan waves: too many
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(1, 0)) == UNSUPPORTED    # 16 scan waves: too many
    assert "chains_per_lane" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(4, 0, 24)) == UNSUPPORTED and "chunk_steps" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(2, 0, 32)) == UNSUPPORTED  # 8 scan waves: 32-step tiles too big
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, -1, 0)) == INVALID
    bad = ssm.ScanOpts(0, 0, 0)
    bad.reserved[1] = 1
    assert scan(lib, dstate=16, opts=bad) == INVALID and "reserved" in err(lib)
    # the layout override: unknown values, the state-row layout's limits, channel groups with the
    # channel-lane layout
    rows, lanes = ssm.SSM_LAYOUT_STATE_ROWS, ssm.SSM_LAYOUT_CHANNEL_LANES
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, 0, 4)) == UNSUPPORTED and "layout" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, 0, rows, 7)) == UNSUPPORTED and "channel_groups" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, 0, rows, -1)) == UNSUPPORTED
    assert scan(lib, dstate=8, opts=ssm.ScanOpts(0, 0, 0, 0, rows)) == UNSUPPORTED and "STATE_ROWS" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, ssm.SSM_BBAR_ZOH, rows)) == UNSUPPORTED
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(2, 0, 0, 0, rows)) == UNSUPPORTED
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 3, 0, 0, rows)) == UNSUPPORTED
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, 0, lanes, 3)) == UNSUPPORTED and "channel_groups" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 32, 0, rows, 5)) == UNSUPPORTED and "chunk_steps" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, 2)) == UNSUPPORTED and "bbar_mode" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(4, 0, 32, ssm.SSM_BBAR_ZOH)) == UNSUPPORTED  # ZOH: 16-step tiles


def test_update_opts_validation(lib):
    def upd(opts):
        return lib.ssm_state_update_ex(2, 16, 16, F32, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                                       fake(7), fake(8), 1, fake(9), None, ctypes.byref(opts))
    assert upd(ssm.UpdateOpts(5)) == UNSUPPORTED and "bbar_mode" in err(lib)
    bad = ssm.UpdateOpts(0)
    bad.reserved[0] = 3
    assert upd(bad) == INVALID and "reserved" in err(lib)


def test_scan_size_overflow(lib):
    assert scan(lib, batch=1 << 40, seqlen=1 << 30, dim=1 << 20) == INVALID and "overflow" in err(lib)


@pytest.mark.parametrize("kw,code", [(dict(batch=-1), INVALID), (dict(dim=-1), INVALID), (dict(dstate=6), UNSUPPORTED),
                                     (dict(dtype=3), UNSUPPORTED), (dict(state=None), INVALID), (dict(y=None), INVALID),
                                     (dict(x=fake(1, 2)), MISALIGNED), (dict(state=fake(0, 2)), MISALIGNED),
                                     (dict(y=fake(0, 8)), INVALID), (dict(state=fake(1, 0)), INVALID)])
def test_update_validation(lib, kw, code):
    assert update(lib, **kw) == code
    assert err(lib)


def test_update_nothing_to_do(lib):
    assert update(lib, batch=0, state=None, x=None, delta=None, A=None, B=None, C=None, y=None) == OK


def test_error_string_is_thread_local(lib):
    import threading
    scan(lib, batch=-1)
    seen = {}

    def other():
        seen["before"] = err(lib)
        scan(lib, dstate=3)
        seen["after"] = err(lib)

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["before"] == "" and "dstate" in seen["after"]
    assert "negative" in err(lib)


def test_binding_raises_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("selective_state_space_61_amd")
    saved = mod._lib_handle
    mod._lib_handle = None
    try:
        with pytest.raises(RuntimeError, match="no fallback"):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        mod._lib_handle = saved


def conv(lib, batch=2, seqlen=8, dim=16, width=4, dtype=F32, x=fake(0), w=fake(1), bias=fake(2), init=fake(3),
         silu=1, y=fake(4), fin=fake(5)):
    return lib.ssm_causal_conv1d_fwd(batch, seqlen, dim, width, dtype, x, w, bias, init, silu, y, fin, None)


def conv_update(lib, batch=2, dim=16, width=4, dtype=F32, state=fake(0), x=fake(1), w=fake(2), bias=fake(3),
                silu=1, y=fake(4)):
    return lib.ssm_causal_conv1d_update(batch, dim, width, dtype, state, x, w, bias, silu, y, None)


@pytest.mark.parametrize("kw,code", [(dict(batch=-1), INVALID), (dict(seqlen=-1), INVALID), (dict(width=0), UNSUPPORTED),
                                     (dict(width=5), UNSUPPORTED), (dict(dtype=4), UNSUPPORTED),
                                     (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
                                     (dict(x=fake(0, 2)), MISALIGNED), (dict(fin=fake(5, 2)), MISALIGNED),
                                     (dict(w=fake(1, 2)), MISALIGNED), (dict(y=fake(0, 4)), INVALID),
                                     (dict(fin=fake(3, 0)), INVALID), (dict(fin=fake(4, 0)), INVALID)])
def test_conv_validation(lib, kw, code):
    assert conv(lib, **kw) == code
    assert err(lib)


def test_conv_nothing_to_do(lib):
    assert conv(lib, batch=0, x=None, w=None, y=None) == OK
    # seqlen == 0 without a final state: nothing to write
    assert conv(lib, seqlen=0, x=None, y=None, fin=None) == OK


@pytest.mark.parametrize("kw,code", [(dict(dim=-1), INVALID), (dict(width=7), UNSUPPORTED), (dict(state=None), INVALID),
                                     (dict(y=None), INVALID), (dict(state=fake(0, 2)), MISALIGNED),
                                     (dict(y=fake(1, 0)), INVALID), (dict(state=fake(2, 0)), INVALID)])
def test_conv_update_validation(lib, kw, code):
    assert conv_update(lib, **kw) == code
    assert err(lib)


def ssd(lib, batch=2, seqlen=8, nheads=4, headdim=64, dstate=128, ngroups=2, dtype=BF16, x=fake(0), dt=fake(1),
        A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), bias=fake(7), y=fake(8), fin=fake(9), init=None,
        opts=None):
    return lib.ssm_ssd_fwd(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, x, dt, A, B, C, D, z, bias, 1, init,
                           y, fin, None, opts)


def ssd_opts(slice_=0, reserved=0, segments=0, gram=0):
    o = ssm.SsdOpts(head_slice=slice_, segments=segments, gram=gram)
    o.reserved[3] = reserved
    return ctypes.byref(o)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), INVALID), (dict(seqlen=-1), INVALID), (dict(nheads=0), INVALID), (dict(headdim=0), INVALID),
    (dict(dstate=0), INVALID), (dict(ngroups=0), INVALID), (dict(ngroups=3), INVALID),
    (dict(dtype=F32), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED), (dict(dstate=16), UNSUPPORTED),
    (dict(dstate=96), UNSUPPORTED), (dict(dstate=512), UNSUPPORTED), (dict(headdim=40), UNSUPPORTED),
    (dict(x=None), INVALID), (dict(dt=None), INVALID), (dict(A=None), INVALID), (dict(B=None), INVALID),
    (dict(C=None), INVALID), (dict(y=None), INVALID),
    (dict(x=fake(0, 8)), MISALIGNED), (dict(z=fake(6, 8)), MISALIGNED), (dict(y=fake(8, 8)), MISALIGNED),
    (dict(B=fake(3, 8)), MISALIGNED), (dict(C=fake(4, 2)), MISALIGNED), (dict(dt=fake(1, 1)), MISALIGNED),
    (dict(A=fake(2, 2)), MISALIGNED), (dict(fin=fake(9, 4)), MISALIGNED),
    (dict(y=fake(0)), INVALID), (dict(y=fake(3)), INVALID), (dict(fin=fake(4)), INVALID), (dict(fin=fake(8)), INVALID),
    (dict(init=fake(10, 8)), MISALIGNED), (dict(init=fake(9)), INVALID), (dict(init=fake(8)), INVALID),
    (dict(opts=ssd_opts(8)), INVALID), (dict(opts=ssd_opts(48)), INVALID), (dict(headdim=32, opts=ssd_opts(64)), INVALID),
    (dict(opts=ssd_opts(0, reserved=1)), INVALID), (dict(opts=ssd_opts(0, segments=-2)), INVALID),
    (dict(opts=ssd_opts(0, gram=2)), INVALID), (dict(opts=ssd_opts(0, gram=-2)), INVALID),
    # the separate C B^T pass lays its tiles out for 64-channel slices
    (dict(opts=ssd_opts(32, gram=1)), UNSUPPORTED),
    # instantiated (dstate, waves) pairs: one wave only up to dstate 64, two up to 128
    (dict(opts=ssd_opts(16)), UNSUPPORTED), (dict(dstate=256, opts=ssd_opts(32)), UNSUPPORTED),
    (dict(dstate=256, headdim=32), UNSUPPORTED), (dict(dstate=128, headdim=16), UNSUPPORTED)])
def test_ssd_validation(lib, kw, code):
    assert ssd(lib, **kw) == code
    assert err(lib)


def test_ssd_nothing_to_do(lib):
    assert ssd(lib, batch=0, x=None, dt=None, B=None, C=None, y=None) == OK
    # seqlen == 0 without a final state: nothing to write
    assert ssd(lib, seqlen=0, x=None, dt=None, B=None, C=None, y=None, fin=None) == OK


def ssd_update(lib, batch=2, nheads=4, headdim=64, dstate=128, ngroups=2, dtype=BF16, state=fake(0), x=fake(1),
               dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), z=fake(7), bias=fake(8), y=fake(9)):
    return lib.ssm_ssd_state_update(batch, nheads, headdim, dstate, ngroups, dtype, state, x, dt, A, B, C, D, z, bias,
                                    1, y, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), INVALID), (dict(nheads=0), INVALID), (dict(ngroups=3), INVALID), (dict(dtype=F32), UNSUPPORTED),
    (dict(dstate=16), UNSUPPORTED), (dict(dstate=100), UNSUPPORTED), (dict(state=None), INVALID),
    (dict(x=None), INVALID), (dict(dt=None), INVALID), (dict(B=None), INVALID), (dict(y=None), INVALID),
    (dict(state=fake(0, 8)), MISALIGNED), (dict(B=fake(4, 4)), MISALIGNED), (dict(C=fake(5, 2)), MISALIGNED),
    (dict(x=fake(1, 1)), MISALIGNED), (dict(y=fake(1)), INVALID), (dict(state=fake(4)), INVALID),
    (dict(y=fake(0)), INVALID)])
def test_ssd_update_validation(lib, kw, code):
    assert ssd_update(lib, **kw) == code
    assert err(lib)


def test_ssd_update_nothing_to_do(lib):
    assert ssd_update(lib, batch=0, state=None, x=None, dt=None, B=None, C=None, y=None) == OK


def test_bwd_opts_validation(lib):
    def bwd(opts, dstate=16):
        args = [2, 8, 16, dstate, F32] + [fake(i) for i in range(8)] + [1] + [fake(8 + i) for i in range(9)] + [None]
        return lib.ssm_scan_bwd_ex(*args, ctypes.byref(opts))
    assert bwd(ssm.BwdOpts(2)) == UNSUPPORTED and "bbar_mode" in err(lib)
    bad = ssm.BwdOpts(0)
    bad.reserved[5] = 1
    assert bwd(bad) == INVALID and "reserved" in err(lib)
    assert bwd(ssm.BwdOpts(0), dstate=128) == UNSUPPORTED and "dstate" in err(lib)
    assert bwd(ssm.BwdOpts(0, 9)) == INVALID and "layout" in err(lib)
    assert bwd(ssm.BwdOpts(0, ssm.SSM_LAYOUT_TIME_SCAN)) == UNSUPPORTED and "TIME_SCAN" in err(lib)
    # the state-row backward takes bf16 only: fp32 is refused before any launch
    assert bwd(ssm.BwdOpts(0, ssm.SSM_LAYOUT_STATE_ROWS)) == UNSUPPORTED and "STATE_ROWS" in err(lib)
    assert bwd(ssm.BwdOpts(1, ssm.SSM_LAYOUT_STATE_ROWS)) == UNSUPPORTED and "STATE_ROWS" in err(lib)


def test_time_scan_opts_validation(lib):
    ts = ssm.SSM_LAYOUT_TIME_SCAN
    assert scan(lib, dstate=8, opts=ssm.ScanOpts(0, 0, 0, 0, ts)) == UNSUPPORTED and "TIME_SCAN" in err(lib)
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, ssm.SSM_BBAR_ZOH, ts)) == UNSUPPORTED
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 2, 0, 0, ts)) == UNSUPPORTED
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 0, 0, ts, 2)) == UNSUPPORTED
    assert scan(lib, dstate=16, opts=ssm.ScanOpts(0, 0, 128, 0, ts)) == UNSUPPORTED and "chunk_steps" in err(lib)


def test_checkpoint_pair_validation(lib):
    """ssm_scan_fwd_ckpt / ssm_scan_bwd_ckpt: the checkpoints are required when there is work,
    must be 16-byte aligned and must not overlap another argument; both need the state rows."""
    def fwd(ck=fake(10), dstate=16, dtype=BF16, batch=2, seqlen=8, dim=16, y=fake(8)):
        return lib.ssm_scan_fwd_ckpt(batch, seqlen, dim, dstate, dtype, fake(0), fake(1), fake(2), fake(3),
                                     fake(4), fake(5), fake(6), fake(7), 1, y, fake(9), ck, None)

    def bwd(ck=fake(20), dstate=16, dtype=BF16, batch=2, seqlen=8, dim=16):
        args = [batch, seqlen, dim, dstate, dtype] + [fake(i) for i in range(8)] + [1] + \
               [fake(8 + i) for i in range(9)]
        return lib.ssm_scan_bwd_ckpt(*args, ck, None)

    assert fwd(ck=None) == INVALID and "checkpoints" in err(lib)
    assert bwd(ck=None) == INVALID and "checkpoints" in err(lib)
    assert fwd(ck=None, batch=0) == OK  # nothing to compute
    assert bwd(ck=None, dim=0) == OK
    assert fwd(ck=fake(10, 2)) == MISALIGNED and "checkpoints" in err(lib)
    assert bwd(ck=fake(20, 2)) == MISALIGNED and "checkpoints" in err(lib)
    assert fwd(ck=fake(10, 8)) == MISALIGNED and "16-byte" in err(lib)
    assert bwd(ck=fake(20, 8)) == MISALIGNED and "16-byte" in err(lib)
    assert fwd(ck=fake(8)) == INVALID and "overlap" in err(lib)   # on y
    assert fwd(ck=fake(0)) == INVALID and "overlap" in err(lib)   # on x
    assert bwd(ck=fake(9)) == INVALID and "overlap" in err(lib)   # on dx (an output)
    assert fwd(dstate=8) == UNSUPPORTED and "state-row" in err(lib)
    assert bwd(dstate=8) == UNSUPPORTED
    assert bwd(dtype=F32) == UNSUPPORTED and "state-row" in err(lib)
    assert bwd(dim=12) == UNSUPPORTED and "state-row" in err(lib)
