"""kda_prefill_noalloc: the same results as kda_prefill, with the chunked
path's scratch taken from the library's fixed device array instead of a
caller workspace.  Two calls in a row, the second smaller than the first (the
array keeps the first call's contents), each compared bit for bit with
kda_prefill on the same inputs and against the oracle to the bf16 bar."""
import numpy as np
import pytest

import gated_delta_rule_90_amd as kda
from gated_delta_rule_90_amd import workloads
from tests._common import dev, prefill_oracle, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _run(inp, noalloc):
    import torch
    io = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f = torch.float32
    B, T, H, _ = inp.q.shape
    dv = inp.v.shape[-1]
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    out = torch.full((B, T, H, dv), float("nan"), dtype=io, device="cuda")
    fs = torch.full((N, H, inp.q.shape[3], dv), float("nan"), dtype=f, device="cuda")
    fn = kda.prefill_noalloc if noalloc else kda.prefill
    fn(dev(inp.q, io), dev(inp.k, io), dev(inp.v, io), dev(inp.g, f), dev(inp.beta, f),
       None if inp.ejk else dev(inp.a_log, f), None if inp.ejk else dev(inp.dt_bias, f),
       dev(inp.initial_state, f), dev(inp.cu_seqlens, torch.int32), scale=inp.scale,
       lower_bound=inp.lower_bound, ejk=inp.ejk, out=out, final_state=fs)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), fs.cpu().numpy()


@pytest.mark.parametrize("ejk", [False, True], ids=["kda", "ejk"])
def test_noalloc_matches_kda_prefill_two_calls(ejk):
    big = workloads.prefill_inputs(2, 1000, 8, 128, 128, seed=1600 + ejk, ejk=ejk, init_state=True)
    small = workloads.prefill_inputs(1, 0, 4, 128, 64, seed=1602 + ejk, ejk=ejk, init_state=True,
                                     lengths=[300, 0, 77, 64])
    for name, inp in (("B2 T1000 H8", big), ("packed 300/0/77/64 H4 dv64", small)):
        say("noalloc", "EJK" if ejk else "KDA", name)
        o_n, s_n = _run(inp, noalloc=True)
        o_r, s_r = _run(inp, noalloc=False)
        np.testing.assert_array_equal(o_n, o_r)
        np.testing.assert_array_equal(s_n, s_r)
        ro, rs = prefill_oracle(inp)
        eo, es = rel_l2(o_n, ro), rel_l2(s_n, rs)
        say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= TOL and es <= TOL


@pytest.mark.parametrize("dk", [64, 128])
def test_noalloc_float32_two_kernel_route_two_calls(dk):
    """float32 inputs at dk 64 and 128 take the two-kernel float32 route, its
    operand blocks in the scratch array: two calls in a row, the second smaller,
    bit for bit kda_prefill's results and within the float32 bar of the oracle."""
    big = workloads.prefill_inputs(2, 700, 4, dk, 64, seed=1610 + dk, dtype="f32", init_state=True)
    small = workloads.prefill_inputs(1, 0, 3, dk, 32, seed=1611 + dk, dtype="f32", init_state=True,
                                     lengths=[70, 0, 33])
    for name, inp in (("B2 T700 H4", big), ("packed 70/0/33 H3 dv32", small)):
        say("noalloc float32", dk, name)
        o_n, s_n = _run(inp, noalloc=True)
        o_r, s_r = _run(inp, noalloc=False)
        np.testing.assert_array_equal(o_n, o_r)
        np.testing.assert_array_equal(s_n, s_r)
        ro, rs = prefill_oracle(inp)
        eo, es = rel_l2(o_n, ro), rel_l2(s_n, rs)
        say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
        assert eo <= 1e-5 and es <= 1e-5


def test_noalloc_dense_call_beyond_the_scratch_runs_in_segments():
    """One 32768-token sequence with 16 heads needs 541 MB of records, more than the
    scratch array: the dense call runs in segments of whole chunks inside it, the
    result the same bit for bit as kda_prefill with the whole workspace; then a
    smaller call in a row."""
    big = workloads.prefill_inputs(1, 32768, 16, 128, 128, seed=1620, init_state=True)
    small = workloads.prefill_inputs(2, 300, 4, 128, 64, seed=1621, init_state=True)
    assert kda.prefill_workspace_bytes(0, 1, 32768, 16, 128, 128, kda.QK_L2NORM | kda.CHUNKED) > (256 << 20)
    for name, inp in (("B1 T32768 H16", big), ("B2 T300 H4 dv64", small)):
        say("noalloc segments", name)
        o_n, s_n = _run(inp, noalloc=True)
        o_r, s_r = _run(inp, noalloc=False)
        np.testing.assert_array_equal(o_n, o_r)
        np.testing.assert_array_equal(s_n, s_r)
