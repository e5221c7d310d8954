"""Token-by-token prefill (use_chunked=False) against the oracle.

Bar: relative L2 <= 1e-5 for fp32 inputs and outputs; bf16 inputs are exact
in the oracle, so with fp32 output the same bar holds, and a bf16 output only
adds its own rounding (<= 2^-9 relative per element)."""
import numpy as np
import pytest

from gated_delta_rule_90_amd import workloads
from tests._common import prefill_gpu, prefill_oracle, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def test_recurrent_fp32_b1_t64_h2_d16():
    inp = workloads.recurrent_fp32_small()
    say("recurrent fp32 B=1 T=64 H=2 d=16")
    o, s = prefill_gpu(inp, use_chunked=False)
    ro, rs = prefill_oracle(inp)
    assert o.shape == (1, 64, 2, 16) and s.shape == (1, 2, 16, 16)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL, (rel_l2(o, ro), rel_l2(s, rs))


@pytest.mark.parametrize("dk,dv", [(16, 32), (32, 16), (64, 64), (128, 128), (128, 16), (16, 128)])
@pytest.mark.parametrize("ejk", [False, True])
def test_recurrent_shapes(dk, dv, ejk):
    inp = workloads.prefill_inputs(2, 37, 3, dk, dv, seed=dk * 7 + dv, dtype="f32", ejk=ejk,
                                   init_state=True)
    say("recurrent", dk, dv, "ejk" if ejk else "kda")
    o, s = prefill_gpu(inp, use_chunked=False)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL, (rel_l2(o, ro), rel_l2(s, rs))


def test_recurrent_bf16_inputs():
    import torch
    inp = workloads.prefill_inputs(1, 80, 2, 64, 64, seed=3, dtype="bf16", init_state=True)
    say("recurrent bf16 in")
    ro, rs = prefill_oracle(inp)
    o, s = prefill_gpu(inp, use_chunked=False, out_dtype=torch.float32)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL
    o16, s16 = prefill_gpu(inp, use_chunked=False)
    assert rel_l2(o16, ro) <= 4e-3 and rel_l2(s16, rs) <= TOL


def test_recurrent_no_l2norm_lower_bound_beyond_chunk_range():
    inp = workloads.prefill_inputs(1, 20, 2, 32, 32, seed=4, dtype="f32", lower_bound=-9.0,
                                   scale=0.2)
    say("recurrent no-l2norm lb=-9")
    o, s = prefill_gpu(inp, use_chunked=False, use_qk_l2norm=False)
    ro, rs = prefill_oracle(inp, use_qk_l2norm=False)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL


@pytest.mark.parametrize("dk,dv", [(64, 32), (16, 16), (32, 64)])
def test_recurrent_varlen_bitwise_equal_to_separate_runs(dk, dv):
    """Sequences start at arbitrary offsets; dk 16 and 32 take tokens in packs
    of 4 and 2 (the pack boundaries then fall at every possible phase)."""
    lens = [17, 0, 64, 1, 40, 3, 22]
    inp = workloads.prefill_inputs(1, 0, 3, dk, dv, seed=5 + dk, dtype="f32", lengths=lens,
                                   init_state=True)
    say("recurrent varlen", dk, dv, lens)
    o, s = prefill_gpu(inp, use_chunked=False)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            np.testing.assert_array_equal(s[n], inp.initial_state[n])
            continue
        sub = workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b],
                                      inp.g[:, a:b], inp.beta[:, a:b], inp.a_log, inp.dt_bias,
                                      inp.initial_state[n:n + 1], None, inp.dtype, inp.scale,
                                      inp.lower_bound)
        on, sn = prefill_gpu(sub, use_chunked=False)
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(s[n], sn[0])


def test_recurrent_split_resume_bitwise():
    inp = workloads.prefill_inputs(2, 50, 2, 32, 64, seed=6, dtype="f32", init_state=True)
    say("recurrent split")
    o, s = prefill_gpu(inp, use_chunked=False)
    cut = 23
    first = workloads.PrefillInputs(inp.q[:, :cut], inp.k[:, :cut], inp.v[:, :cut],
                                    inp.g[:, :cut], inp.beta[:, :cut], inp.a_log, inp.dt_bias,
                                    inp.initial_state, None, inp.dtype, inp.scale,
                                    inp.lower_bound)
    o1, s1 = prefill_gpu(first, use_chunked=False)
    second = workloads.PrefillInputs(inp.q[:, cut:], inp.k[:, cut:], inp.v[:, cut:],
                                     inp.g[:, cut:], inp.beta[:, cut:], inp.a_log, inp.dt_bias,
                                     s1, None, inp.dtype, inp.scale, inp.lower_bound)
    o2, s2 = prefill_gpu(second, use_chunked=False)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(s2, s)


def test_recurrent_zero_length_carries_state_and_in_place_alias():
    import torch
    from tests._common import dev
    import gated_delta_rule_90_amd as kda
    inp = workloads.prefill_inputs(2, 0, 2, 16, 16, seed=8, dtype="f32", init_state=True)
    say("recurrent T=0 passthrough")
    s0 = dev(inp.initial_state, torch.float32)
    f = torch.float32
    o, fs = kda.prefill(dev(inp.q, f), dev(inp.k, f), dev(inp.v, f), dev(inp.g, f),
                        dev(inp.beta, f), dev(inp.a_log, f), dev(inp.dt_bias, f), s0,
                        use_chunked=False, return_state=True)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 16)
    np.testing.assert_array_equal(fs.cpu().numpy(), inp.initial_state)
    # in-place carry: final_state aliases initial_state
    inp2 = workloads.prefill_inputs(2, 9, 2, 16, 16, seed=9, dtype="f32", init_state=True)
    ro, rs = prefill_oracle(inp2)
    st = dev(inp2.initial_state, f)
    kda.prefill(dev(inp2.q, f), dev(inp2.k, f), dev(inp2.v, f), dev(inp2.g, f),
                dev(inp2.beta, f), dev(inp2.a_log, f), dev(inp2.dt_bias, f), st,
                use_chunked=False, final_state=st)
    torch.cuda.synchronize()
    assert rel_l2(st.cpu().numpy(), rs) <= TOL


def test_decode_steps_equal_recurrent_prefill():
    """T decode calls (kda_tkg layout) == one token-by-token prefill on the GPU."""
    import torch
    from tests._common import dev
    import gated_delta_rule_90_amd as kda
    inp = workloads.prefill_inputs(3, 12, 4, 64, 32, seed=10, dtype="f32", init_state=True)
    say("decode steps vs recurrent prefill")
    o, s = prefill_gpu(inp, use_chunked=False)
    f = torch.float32
    S = dev(inp.initial_state, f)
    a_log, dtb = dev(inp.a_log[None, :], f), dev(inp.dt_bias, f)
    for t in range(12):
        out = kda.decode_step(dev(np.swapaxes(inp.q[:, t], 1, 2), f),
                              dev(np.swapaxes(inp.k[:, t], 1, 2), f), dev(inp.v[:, t], f),
                              dev(np.swapaxes(inp.g[:, t], 1, 2), f),
                              dev(inp.beta[:, t][:, None, :], f), a_log, dtb, S,
                              scale=inp.scale)
        torch.cuda.synchronize()
        assert rel_l2(out.cpu().numpy(), o[:, t]) <= TOL
    assert rel_l2(S.cpu().numpy(), s) <= TOL
