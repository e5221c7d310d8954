"""The chunked routes that compute in float32 (KDA_CHUNKED with float32 inputs,
or bf16 inputs with dk < 128) against the oracle, and their routing: with
H dk >= 128 and the workspace, two kernels on 16-token chunks (the operand
blocks of every chunk in parallel, then a scan per 16 state columns that forms
the output); otherwise one kernel (32-token chunks at dk <= 32, 16 above).

Bar: relative L2 <= 1e-5 for o and the final state (float32 path, as for the
token-by-token kernel); packed sequences and chunk-aligned splits bit for bit."""
import numpy as np
import pytest

from gated_delta_rule_90_amd import workloads
from tests._common import prefill_gpu, prefill_oracle, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _check(inp, **kw):
    o, s = prefill_gpu(inp, **kw)
    ro, rs = prefill_oracle(inp)
    eo, es = rel_l2(o, ro), rel_l2(s, rs)
    assert eo <= TOL and es <= TOL, (eo, es)
    return o, s


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 128])
@pytest.mark.parametrize("ejk", [False, True])
def test_chunked_f32_shapes(dk, dv, ejk):
    inp = workloads.prefill_inputs(2, 37, 3, dk, dv, seed=300 + dk + dv, dtype="f32", ejk=ejk,
                                   init_state=True)
    say("chunked f32", dk, dv, "ejk" if ejk else "kda")
    _check(inp)


def test_chunked_f32_small_fp32_workload():
    """B=1, T=64, H=2, dk=dv=16 (the small fp32 workload) through the chunked path."""
    inp = workloads.recurrent_fp32_small()
    say("chunked f32 B1 T64 H2 d16")
    o, s = _check(inp)
    orc, src = prefill_gpu(inp, use_chunked=False)
    assert rel_l2(o, orc) <= TOL and rel_l2(s, src) <= TOL


@pytest.mark.parametrize("ejk", [False, True])
def test_chunked_f32_long_strong_decay(ejk):
    """Many chunks, gates saturating at lower_bound = -5 (the factor range's edge)
    and, in EJK mode, decays of -2|N(0,1)| per token."""
    inp = workloads.prefill_inputs(1, 300, 2, 64, 32, seed=310, dtype="f32", ejk=ejk, init_state=True)
    if ejk:
        inp.g = (-2.0 * np.abs(np.random.default_rng(1).standard_normal(inp.g.shape))).astype(np.float32)
    else:
        inp.g = (inp.g + 8.0).astype(np.float32)   # sigmoid near 1: gamma near lower_bound
    say("chunked f32 strong decay", "ejk" if ejk else "kda")
    _check(inp)


def test_chunked_f32_without_l2norm_custom_scale_and_grouped_heads():
    inp = workloads.prefill_inputs(2, 45, 4, 32, 32, seed=320, dtype="f32", init_state=True, hkv=2,
                                   scale=0.3)
    say("chunked f32 grouped, custom scale")
    _check(inp)
    say("chunked f32 without l2 norm")
    o, s = prefill_gpu(inp, use_qk_l2norm=False)
    ro, rs = prefill_oracle(inp, use_qk_l2norm=False)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL


@pytest.mark.parametrize("ejk", [False, True])
def test_chunked_f32_varlen_bitwise_equal_to_separate_runs(ejk):
    lens = [17, 0, 64, 1, 40, 3, 22, 16]
    inp = workloads.prefill_inputs(1, 0, 3, 32, 32, seed=330, dtype="f32", lengths=lens, ejk=ejk,
                                   init_state=True)
    say("chunked f32 varlen", lens, "ejk" if ejk else "kda")
    o, s = _check(inp)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            np.testing.assert_array_equal(s[n], inp.initial_state[n])
            continue
        sub = workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b],
                                      None if inp.g is None else inp.g[:, a:b], inp.beta[:, a:b],
                                      inp.a_log, inp.dt_bias, inp.initial_state[n:n + 1], None,
                                      inp.dtype, inp.scale, inp.lower_bound, ejk=ejk)
        on, sn = prefill_gpu(sub)
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(s[n], sn[0])


def test_chunked_f32_split_at_chunk_boundary_bitwise():
    inp = workloads.prefill_inputs(2, 80, 2, 64, 32, seed=340, dtype="f32", init_state=True)
    say("chunked f32 split")
    o, s = prefill_gpu(inp)
    cut = 64   # a multiple of the kernel's 32-token chunk
    part = lambda x, a, b: x[:, a:b]
    first = workloads.PrefillInputs(part(inp.q, 0, cut), part(inp.k, 0, cut), part(inp.v, 0, cut),
                                    part(inp.g, 0, cut), part(inp.beta, 0, cut), inp.a_log, inp.dt_bias,
                                    inp.initial_state, None, inp.dtype, inp.scale, inp.lower_bound)
    o1, s1 = prefill_gpu(first)
    second = workloads.PrefillInputs(part(inp.q, cut, 80), part(inp.k, cut, 80), part(inp.v, cut, 80),
                                     part(inp.g, cut, 80), part(inp.beta, cut, 80), inp.a_log,
                                     inp.dt_bias, s1, None, inp.dtype, inp.scale, inp.lower_bound)
    o2, s2 = prefill_gpu(second)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(s2, s)


def test_chunked_f32_extremes():
    from tests.test_extremes_gpu import _extreme_prefill
    inp = workloads.prefill_inputs(2, 40, 3, 32, 32, seed=350, dtype="f32", init_state=True)
    inp = _extreme_prefill(inp, np.random.default_rng(3))
    say("chunked f32 extremes")
    o, s = _check(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))


def test_chunked_f32_in_place_alias_and_empty():
    import torch
    import gated_delta_rule_90_amd as kda
    from tests._common import dev
    inp = workloads.prefill_inputs(2, 33, 2, 16, 32, seed=360, dtype="f32", init_state=True)
    f = torch.float32
    st = dev(inp.initial_state, f)
    say("chunked f32 in-place carry")
    o = kda.prefill(dev(inp.q, f), dev(inp.k, f), dev(inp.v, f), dev(inp.g, f), dev(inp.beta, f),
                    dev(inp.a_log, f), dev(inp.dt_bias, f), st, scale=inp.scale,
                    lower_bound=inp.lower_bound, final_state=st)
    torch.cuda.synchronize()
    ro, rs = prefill_oracle(inp)
    assert rel_l2(o.cpu().numpy(), ro) <= TOL and rel_l2(st.cpu().numpy(), rs) <= TOL
    e = workloads.prefill_inputs(2, 0, 2, 16, 32, seed=361, dtype="f32", init_state=True)
    _, se = prefill_gpu(e)
    np.testing.assert_array_equal(se, e.initial_state)


def test_chunked_f32_routing_falls_back_to_token_by_token():
    """lower_bound < -5 (outside the factor range) and unaligned inputs take the
    token-by-token kernel: bit for bit its result."""
    import torch
    import gated_delta_rule_90_amd as kda
    inp = workloads.prefill_inputs(1, 30, 2, 32, 32, seed=370, dtype="f32", init_state=True,
                                   lower_bound=-7.0)
    say("chunked f32 routing: lower_bound -7")
    o, s = prefill_gpu(inp)
    orc, src = prefill_gpu(inp, use_chunked=False)
    np.testing.assert_array_equal(o, orc)
    np.testing.assert_array_equal(s, src)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(o, ro) <= TOL

    inp = workloads.prefill_inputs(1, 30, 2, 32, 32, seed=371, dtype="f32")
    f = torch.float32

    def unaligned(x):
        flat = torch.empty(x.size + 1, dtype=f, device="cuda")
        view = flat[1:].view(x.shape)          # 4 bytes past a 256-byte allocation boundary
        view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to("cuda"))
        return view

    args = [torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in
            (inp.v, inp.g, inp.beta, inp.a_log, inp.dt_bias)]
    say("chunked f32 routing: unaligned q")
    o_u, s_u = kda.prefill(unaligned(inp.q), unaligned(inp.k), *args, scale=inp.scale,
                           lower_bound=inp.lower_bound, return_state=True)
    o_r, s_r = kda.prefill(unaligned(inp.q), unaligned(inp.k), *args, scale=inp.scale,
                           lower_bound=inp.lower_bound, use_chunked=False, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o_u, o_r) and torch.equal(s_u, s_r)


@pytest.mark.parametrize("dk", [16, 32, 64])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("ejk", [False, True])
def test_chunked_float32_arithmetic_on_bf16_inputs(dk, out, ejk):
    """bf16 inputs with dk < 128 take the same kernel (float32 arithmetic on the
    widened inputs): the state meets the float32 bar, the output too unless it
    is rounded to bf16 (then the bf16-input bar)."""
    import torch
    inp = workloads.prefill_inputs(2, 45, 3, dk, 64, seed=380 + dk, ejk=ejk, init_state=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    say("chunked float32 arithmetic, bf16 inputs", dk, out, "ejk" if ejk else "kda")
    o, s = prefill_gpu(inp, out_dtype=od)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(s, rs) <= TOL, rel_l2(s, rs)
    assert rel_l2(o, ro) <= (2e-2 if out == "bf16" else TOL), rel_l2(o, ro)
    orc, src = prefill_gpu(inp, out_dtype=od, use_chunked=False)
    assert rel_l2(s, src) <= TOL


def test_chunked_float32_arithmetic_bf16_varlen_bitwise():
    lens = [33, 0, 80, 5, 16]
    inp = workloads.prefill_inputs(1, 0, 2, 64, 32, seed=390, lengths=lens, init_state=True)
    say("chunked float32 arithmetic, bf16 varlen", lens)
    o, s = prefill_gpu(inp)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(o, ro) <= 2e-2 and rel_l2(s, rs) <= TOL
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            np.testing.assert_array_equal(s[n], inp.initial_state[n])
            continue
        sub = workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b], inp.g[:, a:b],
                                      inp.beta[:, a:b], inp.a_log, inp.dt_bias, inp.initial_state[n:n + 1],
                                      None, inp.dtype, inp.scale, inp.lower_bound)
        on, sn = prefill_gpu(sub)
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(s[n], sn[0])


@pytest.mark.parametrize("dtype,use_chunked", [("f32", True), ("bf16", True), ("f32", False)])
def test_ejkernel_worked_example_shapes(dtype, use_chunked):
    """The ejkernel kda_attention example's shapes (tests/golden/ejkernel_example_shapes.json:
    batch 2, 64 tokens, 8 heads, head_dim 32, beta = sigmoid(N(0,1)), decay of scale -0.01, sign
    fixed to the documented <= 0) in EJK mode, through the chunked and token-by-token paths,
    returning the state: output [2, 64, 8, 32] and state [2, 8, 32, 32] against the oracle."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ejkernel_example_shapes.json")))
    B, T, H, d = gold["batch"], gold["seq_len"], gold["num_heads"], gold["head_dim"]
    inp = workloads.prefill_inputs(B, T, H, d, d, seed=2024, dtype=dtype, ejk=True)
    say("ejkernel example shapes", dtype, "chunked" if use_chunked else "token-by-token")
    o, s = prefill_gpu(inp, use_chunked=use_chunked)
    assert list(o.shape) == gold["output_shape"] and list(s.shape) == gold["state_shape"]
    ro, rs = prefill_oracle(inp)
    assert rel_l2(s, rs) <= TOL
    assert rel_l2(o, ro) <= (2e-2 if dtype == "bf16" else TOL)


# ---- the two-kernel route (dk 64 and 128 with the workspace)

def _separate_runs_bitwise(inp, o, s):
    """Each packed sequence run alone gives the packed call's rows and state bit for bit."""
    cu = inp.cu_seqlens
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            np.testing.assert_array_equal(s[n], inp.initial_state[n])
            continue
        sub = workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b],
                                      None if inp.g is None else inp.g[:, a:b], inp.beta[:, a:b],
                                      inp.a_log, inp.dt_bias, inp.initial_state[n:n + 1], None,
                                      inp.dtype, inp.scale, inp.lower_bound, ejk=inp.ejk)
        on, sn = prefill_gpu(sub)
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(s[n], sn[0])


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("ejk", [False, True])
def test_two_kernel_route_varlen_bitwise_equal_to_separate_runs(dk, ejk):
    lens = [17, 0, 100, 1, 48, 3, 250, 16]
    inp = workloads.prefill_inputs(1, 0, 8, dk, 32, seed=331 + dk, dtype="f32", lengths=lens, ejk=ejk,
                                   init_state=True)   # H dk >= 128: the two-kernel route
    say("two-kernel route varlen", dk, lens, "ejk" if ejk else "kda")
    o, s = _check(inp)
    _separate_runs_bitwise(inp, o, s)
    # without the final state (no state stores) the output is the same bit for bit
    import torch
    import gated_delta_rule_90_amd as kda
    from tests._common import dev
    f = torch.float32
    o2 = kda.prefill(dev(inp.q, f), dev(inp.k, f), dev(inp.v, f), dev(inp.g, f), dev(inp.beta, f),
                     None if ejk else dev(inp.a_log, f), None if ejk else dev(inp.dt_bias, f),
                     dev(inp.initial_state, f), dev(inp.cu_seqlens, torch.int32), scale=inp.scale,
                     lower_bound=inp.lower_bound, ejk=ejk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o2.cpu().numpy(), o)


@pytest.mark.parametrize("dtype,out,dk", [("f32", "f32", 128), ("f32", "f32", 32), ("bf16", "bf16", 64),
                                          ("bf16", "f32", 64), ("bf16", "f32", 16)])
@pytest.mark.parametrize("ejk", [False, True])
def test_two_kernel_route_many_chunks_grouped_heads(dtype, out, dk, ejk):
    """600 tokens (38 chunks, a ragged last one) over two sequences, grouped key and
    value heads, an initial state; H dk >= 128 (the two-kernel route) at every dk."""
    import torch
    inp = workloads.prefill_inputs(2, 600, max(4, 128 // dk), dk, 64, seed=392 + ejk, dtype=dtype, ejk=ejk,
                                   init_state=True, hkv=2)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    say("two-kernel route", dtype, "out", out, "dk", dk, "ejk" if ejk else "kda")
    o, s = prefill_gpu(inp, out_dtype=od)
    ro, rs = prefill_oracle(inp)
    eo, es = rel_l2(o, ro), rel_l2(s, rs)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert es <= TOL, es
    assert eo <= (2e-2 if out == "bf16" else TOL), eo


def test_two_kernel_route_split_at_16_token_boundary_bitwise():
    inp = workloads.prefill_inputs(2, 200, 2, 128, 32, seed=341, dtype="f32", init_state=True)
    say("two-kernel route split at 112")
    o, s = prefill_gpu(inp)
    cut = 112   # a multiple of the 16-token chunk
    part = lambda x, a, b: x[:, a:b]
    first = workloads.PrefillInputs(part(inp.q, 0, cut), part(inp.k, 0, cut), part(inp.v, 0, cut),
                                    part(inp.g, 0, cut), part(inp.beta, 0, cut), inp.a_log, inp.dt_bias,
                                    inp.initial_state, None, inp.dtype, inp.scale, inp.lower_bound)
    o1, s1 = prefill_gpu(first)
    second = workloads.PrefillInputs(part(inp.q, cut, 200), part(inp.k, cut, 200), part(inp.v, cut, 200),
                                     part(inp.g, cut, 200), part(inp.beta, cut, 200), inp.a_log,
                                     inp.dt_bias, s1, None, inp.dtype, inp.scale, inp.lower_bound)
    o2, s2 = prefill_gpu(second)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(s2, s)


@pytest.mark.parametrize("ejk", [False, True])
def test_without_workspace_the_one_kernel_route_serves_dk128(monkeypatch, ejk):
    """A call whose workspace cannot hold the operand blocks (here none) takes the
    one-kernel float32 route instead: no error, the same bar."""
    inp = workloads.prefill_inputs(2, 90, 3, 128, 32, seed=393 + ejk, dtype="f32", ejk=ejk, init_state=True)
    say("dk 128 without a workspace", "ejk" if ejk else "kda")
    import gated_delta_rule_90_amd as kda
    o_w, s_w = _check(inp)
    monkeypatch.setattr(kda, "prefill_workspace_bytes", lambda *a, **k: 0)
    o_1, s_1 = _check(inp)
    assert rel_l2(o_1, o_w) <= 2 * TOL and rel_l2(s_1, s_w) <= 2 * TOL


@pytest.mark.parametrize("dtype,dk,dv,H", [("f32", 128, 128, 8), ("bf16", 64, 64, 16), ("f32", 32, 32, 32)])
@pytest.mark.parametrize("ejk", [False, True])
def test_two_kernel_route_two_tiles_per_scan_workgroup(dtype, dk, dv, H, ejk):
    """Eight packed sequences (ragged, one empty) with H * 8 * dv / 32 >= 256, so that the
    scan carries two 16-column state tiles per workgroup: every (sequence, head) unit
    against the oracle, and each sequence run alone (few units: one tile per workgroup)
    equal to the packed call bit for bit."""
    import torch
    lens = [37, 16, 5, 64, 21, 0, 50, 33]
    assert H * len(lens) * (dv // 32) >= 256
    inp = workloads.prefill_inputs(1, 0, H, dk, dv, seed=400 + dk + ejk, dtype=dtype, lengths=lens,
                                   ejk=ejk, init_state=True)
    say("two-kernel route, two tiles per scan workgroup", dtype, "dk", dk, "dv", dv, "H", H,
        "ejk" if ejk else "kda")
    o, s = prefill_gpu(inp, out_dtype=torch.float32)
    ro, rs = prefill_oracle(inp)
    cu = inp.cu_seqlens
    worst_o = worst_s = 0.0
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            if b > a:
                worst_o = max(worst_o, rel_l2(o[0, a:b, h], ro[0, a:b, h]))
            worst_s = max(worst_s, rel_l2(s[n, h], rs[n, h]))
    say(f"  worst unit rel-L2 o={worst_o:.3e} S={worst_s:.3e}")
    assert worst_o <= TOL and worst_s <= TOL, (worst_o, worst_s)
    o2, s2 = prefill_gpu(inp)
    _separate_runs_bitwise(inp, o2, s2)
