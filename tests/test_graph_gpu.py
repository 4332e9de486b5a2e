"""The decode step captured in a HIP graph: every replay must equal the eager result.  Replays are
separated by eager work and synchronisations, and each one is checked."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def test_decode_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_61_amd as ssm
    w = W.Workload("graph", "decode", batch=8, seqlen=12, dim=320, dstate=16, dtype="bf16", seed=77)
    t = W.workload_inputs(w)
    d = {k: to_dev(v) for k, v in t.items()}
    steps = w.seqlen

    def run(state, ys):
        for s in range(steps):
            ssm.ssm_state_update(state, d["x"][s], d["delta"][s], d["A"], d["B"][s], d["C"][s], D=d["D"],
                                 z=d["z"][s], delta_bias=d["delta_bias"], delta_softplus=True, y=ys[s])

    st_e = torch.zeros(w.batch, w.dim, w.dstate, device="cuda")
    ys_e = torch.empty(steps, w.batch, w.dim, dtype=torch.bfloat16, device="cuda")
    run(st_e, ys_e)
    torch.cuda.synchronize()

    st_g = torch.zeros_like(st_e)
    ys_g = torch.empty_like(ys_e)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(st_g, ys_g)
    torch.cuda.synchronize()
    for rep in range(4):
        st_g.zero_()                     # reset the state (a fill kernel, outside the graph)
        ys_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st_g, st_e), f"replay {rep}: state differs from eager"
        assert torch.equal(ys_g, ys_e), f"replay {rep}: y differs from eager"
        # some eager work between replays
        tmp = torch.zeros_like(st_e)
        run(tmp, torch.empty_like(ys_e))
        torch.cuda.synchronize()
        say(f"  replay {rep} matches eager")


def test_split_scan_graph_survives_scratch_growth():
    """A split-sequence scan captured in a graph keeps working after a larger eager call on the
    same stream has replaced the stream's scratch buffer (the old buffer is retired, not freed)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_61_amd as ssm
    small = {k: to_dev(v) for k, v in W.scan_inputs(1, 900, 96, 16, "f32", seed=31).items()}
    large = {k: to_dev(v) for k, v in W.scan_inputs(2, 1500, 200, 16, "f32", seed=32).items()}

    def call(d, y, st):
        ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                         delta_bias=d["delta_bias"], delta_softplus=True, y=y, last_state=st, segments=4)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ys, ss = torch.empty_like(small["x"]), torch.empty(1, 96, 16, device="cuda")
    yl, sl = torch.empty_like(large["x"]), torch.empty(2, 200, 16, device="cuda")
    with torch.cuda.stream(side):
        call(small, ys, ss)                       # allocates the side stream's scratch
    torch.cuda.synchronize()
    ys_e, ss_e = ys.clone(), ss.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call(small, ys, ss)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        call(large, yl, sl)                       # needs more scratch: the buffer is replaced
    torch.cuda.synchronize()
    yl_e, sl_e = yl.clone(), sl.clone()
    for rep in range(3):
        ys.fill_(0)
        ss.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ys_e) and torch.equal(ss, ss_e), f"replay {rep} differs from eager"
        with torch.cuda.stream(side):
            call(large, yl, sl)
        torch.cuda.synchronize()
        assert torch.equal(yl, yl_e) and torch.equal(sl, sl_e), f"eager call after replay {rep} differs"
        say(f"  replay {rep} after scratch growth matches eager")
