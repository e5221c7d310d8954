"""The prefill and decode calls captured in a HIP graph: every replay equals
the eager call bit for bit.  Replays run with eager work and synchronisations
between them, and the outputs are cleared before each, so a replay that skips
or repeats work (or a recorded memset node that misbehaves after the first
replay) shows.  Inputs and outputs are allocated before capture; the binding's
workspace is allocated from the graph's pool during capture."""
import numpy as np
import pytest

from gated_delta_rule_90_amd import workloads
from tests._common import dev, say

pytestmark = pytest.mark.gpu
REPLAYS = 4


def _replay_equal(fn, outs):
    import torch
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()   # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(REPLAYS):
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)
    del g


@pytest.mark.parametrize("packed", [False, True])
def test_chunked_bf16_prefill_graph_replays(packed):
    import torch
    import gated_delta_rule_90_amd as kda
    if packed:
        inp = workloads.prefill_inputs(1, 0, 4, 128, 64, seed=500, lengths=[100, 0, 300, 37], init_state=True)
    else:
        inp = workloads.prefill_inputs(2, 200, 4, 128, 64, seed=501, init_state=True)
    bf, f = torch.bfloat16, torch.float32
    q, k, v = dev(inp.q, bf), dev(inp.k, bf), dev(inp.v, bf)
    g, beta, a_log, dtb = dev(inp.g, f), dev(inp.beta, f), dev(inp.a_log, f), dev(inp.dt_bias, f)
    s0 = dev(inp.initial_state, f)
    cu = dev(inp.cu_seqlens, torch.int32)
    o = torch.empty_like(v)
    fs = torch.empty_like(s0)
    say("graph: chunked bf16 prefill", "packed" if packed else "dense")
    _replay_equal(lambda: kda.prefill(q, k, v, g, beta, a_log, dtb, s0, cu, scale=inp.scale,
                                      lower_bound=inp.lower_bound, out=o, final_state=fs), [o, fs])


def test_float32_chunked_prefill_graph_replays():
    import torch
    import gated_delta_rule_90_amd as kda
    inp = workloads.prefill_inputs(2, 90, 3, 64, 32, seed=502, dtype="f32", init_state=True)
    f = torch.float32
    args = [dev(x, f) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.a_log, inp.dt_bias, inp.initial_state)]
    o = torch.empty_like(args[2])
    fs = torch.empty_like(args[7])
    say("graph: float32 chunked prefill")
    _replay_equal(lambda: kda.prefill(*args, scale=inp.scale, lower_bound=inp.lower_bound, out=o,
                                      final_state=fs), [o, fs])


def test_decode_graph_replays():
    """Each replay advances its own copy of the state from the same start."""
    import torch
    import gated_delta_rule_90_amd as kda
    d = workloads.decode_inputs(8, 4, 128, 128, seed=503)
    f = torch.float32
    q, k, v, g, beta, a_log, dtb = (dev(x, f) for x in (d.q, d.k, d.v, d.g, d.beta, d.a_log, d.dt_bias))
    S0 = dev(d.S, f)
    S = S0.clone()
    out = torch.empty((8, 4, 128), dtype=f, device="cuda")

    def step():
        S.copy_(S0)
        kda.decode_step(q, k, v, g, beta, a_log, dtb, S, scale=d.scale, out=out)

    say("graph: decode step")
    _replay_equal(step, [out, S])
