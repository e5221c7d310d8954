"""MFMA chunked prefill (bf16 q/k/v, fp32 gates and state) against the oracle.

Bar: relative L2 <= 2e-2 for o and the final state (bf16-input path).
Packed varlen runs must equal per-sequence runs bitwise, and a split at a
chunk boundary with state passthrough must equal the unsplit run bitwise."""
import numpy as np
import pytest

import gated_delta_rule_90_amd as kda
from gated_delta_rule_90_amd import workloads
from tests._common import check_units, dev, prefill_gpu, prefill_oracle, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _check(inp, units=None, **kw):
    o, s = prefill_gpu(inp, **kw)
    ro, rs = prefill_oracle(inp, units=units, use_qk_l2norm=kw.get("use_qk_l2norm", True))
    if units is not None:
        H = inp.q.shape[2]
        sel_o = [(u // H, u % H) for u in units]
        if inp.cu_seqlens is None:
            o_s = np.stack([o[n, :, h] for n, h in sel_o])
            ro_s = np.stack([ro[n, :, h] for n, h in sel_o])
        else:
            cu = inp.cu_seqlens
            o_s = np.concatenate([o[0, cu[n]:cu[n + 1], h].ravel() for n, h in sel_o])
            ro_s = np.concatenate([ro[0, cu[n]:cu[n + 1], h].ravel() for n, h in sel_o])
        s_s = np.stack([s[n, h] for n, h in sel_o])
        rs_s = np.stack([rs[n, h] for n, h in sel_o])
    else:
        o_s, ro_s, s_s, rs_s = o, ro, s, rs
    eo, es = rel_l2(o_s, ro_s), rel_l2(s_s, rs_s)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= TOL and es <= TOL, (eo, es)
    return o, s


@pytest.mark.parametrize("T", [64, 200, 1, 130])
def test_chunked_ragged_small(T):
    inp = workloads.prefill_inputs(2, T, 3, 128, 128, seed=100 + T, init_state=True)
    say("chunked B=2 T=%d H=3" % T)
    _check(inp)


@pytest.mark.parametrize("dv", [16, 32, 64])
def test_chunked_dv_tiles(dv):
    inp = workloads.prefill_inputs(1, 150, 2, 128, dv, seed=200 + dv, init_state=True)
    say("chunked dv=%d" % dv)
    _check(inp)


def test_chunked_fp32_output_and_no_l2norm():
    import torch
    inp = workloads.prefill_inputs(2, 96, 2, 128, 64, seed=300, scale=0.05)
    say("chunked fp32 out, l2norm on")
    _check(inp, out_dtype=torch.float32)
    inp2 = workloads.prefill_inputs(1, 80, 2, 128, 32, seed=301, scale=0.02)
    inp2.q *= 0.1
    inp2.k *= 0.1
    inp2.q = workloads.round_to_bf16(inp2.q)
    inp2.k = workloads.round_to_bf16(inp2.k)
    say("chunked no l2norm")
    _check(inp2, use_qk_l2norm=False)


def test_chunked_strongest_decay():
    """lower_bound = -5 with saturated gates: in-chunk log-decay near -320."""
    inp = workloads.prefill_inputs(1, 256, 2, 128, 64, seed=400, init_state=True)
    inp.g = (inp.g + 20.0).astype(np.float32)
    say("chunked saturated gates")
    _check(inp)
    inp.g = (inp.g - 40.0).astype(np.float32)   # sigma ~ 0: almost no decay
    say("chunked almost no decay")
    _check(inp)


def test_chunked_determinism():
    inp = workloads.prefill_inputs(2, 300, 4, 128, 128, seed=500, init_state=True)
    say("chunked determinism")
    o1, s1 = prefill_gpu(inp)
    o2, s2 = prefill_gpu(inp)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_chunked_varlen_bitwise_and_zero_length():
    lens = [130, 0, 64, 1, 257, 63]
    inp = workloads.prefill_inputs(1, 0, 3, 128, 64, seed=600, lengths=lens, init_state=True)
    say("chunked varlen", lens)
    o, s = _check(inp)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            np.testing.assert_array_equal(s[n], inp.initial_state[n])
            continue
        sub = workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b], inp.g[:, a:b],
                                      inp.beta[:, a:b], inp.a_log, inp.dt_bias,
                                      inp.initial_state[n:n + 1], None, inp.dtype, inp.scale,
                                      inp.lower_bound)
        on, sn = prefill_gpu(sub)
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(s[n], sn[0])


def test_chunked_split_at_chunk_boundary_is_bitwise():
    inp = workloads.prefill_inputs(2, 384, 2, 128, 128, seed=700, init_state=True)
    say("chunked split at 192")
    o, s = prefill_gpu(inp)
    cut = 192

    def part(a, b, s0):
        return workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b],
                                       inp.g[:, a:b], inp.beta[:, a:b], inp.a_log, inp.dt_bias,
                                       s0, None, inp.dtype, inp.scale, inp.lower_bound)

    o1, s1 = prefill_gpu(part(0, cut, inp.initial_state))
    o2, s2 = prefill_gpu(part(cut, 384, s1))
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(s2, s)


@pytest.mark.parametrize("packed", [False, True])
def test_chunked_in_place_state_carry(packed):
    """initial_state passed again as final_state: the carried state and the output
    equal the out-of-place call bit for bit (each scan workgroup reads its state
    tile before it writes the same tile)."""
    import torch
    if packed:
        inp = workloads.prefill_inputs(1, 0, 4, 128, 128, seed=710, lengths=[70, 0, 200, 64], init_state=True)
    else:
        inp = workloads.prefill_inputs(3, 150, 4, 128, 128, seed=711, init_state=True)
    say("chunked in-place state carry", "packed" if packed else "dense")
    o_ref, s_ref = prefill_gpu(inp)
    bf, f = torch.bfloat16, torch.float32
    st = dev(inp.initial_state, f)
    o, fs = kda.prefill(dev(inp.q, bf), dev(inp.k, bf), dev(inp.v, bf), dev(inp.g, f), dev(inp.beta, f),
                        dev(inp.a_log, f), dev(inp.dt_bias, f), st, dev(inp.cu_seqlens, torch.int32),
                        scale=inp.scale, lower_bound=inp.lower_bound, return_state=True, final_state=st)
    torch.cuda.synchronize()
    assert fs is st
    np.testing.assert_array_equal(o.float().cpu().numpy(), o_ref)
    np.testing.assert_array_equal(st.cpu().numpy(), s_ref)


def test_chunked_matches_recurrent_kernel():
    import torch
    inp = workloads.prefill_inputs(1, 333, 2, 128, 128, seed=800, init_state=True)
    say("chunked vs recurrent")
    oc, sc = prefill_gpu(inp, out_dtype=torch.float32)
    orc, src = prefill_gpu(inp, use_chunked=False, out_dtype=torch.float32)
    assert rel_l2(oc, orc) <= TOL and rel_l2(sc, src) <= TOL


def test_chunked_full_size_b4_t4096_h16_every_unit(margin):
    """Launch shape of the benchmark: all 64 (batch, head) units against the
    oracle, each with its own relative L2."""
    inp = workloads.prefill_b4_t4096_h16_d128()
    say("chunked full size B=4 T=4096 H=16")
    o, s = prefill_gpu(inp)
    ro, rs = prefill_oracle(inp)
    check_units(o, ro, s, rs, TOL, margin, label="B4 T4096 H16")


def _packed_equals_separate(inp, o, s):
    """Each sequence of a packed batch run alone gives bitwise the packed result."""
    cu = inp.cu_seqlens
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b],
                                      None if inp.g is None else inp.g[:, a:b], inp.beta[:, a:b],
                                      inp.a_log, inp.dt_bias,
                                      None if inp.initial_state is None else inp.initial_state[n:n + 1],
                                      None, inp.dtype, inp.scale, inp.lower_bound, ejk=inp.ejk)
        on, sn = prefill_gpu(sub)
        assert np.array_equal(o[:, a:b], on), f"sequence {n}: packed o differs from the separate run"
        assert np.array_equal(s[n], sn[0]), f"sequence {n}: packed state differs from the separate run"


@pytest.mark.parametrize("ejk", [False, True], ids=["kda", "ejk"])
def test_chunked_varlen_8seq_every_sequence(ejk, margin):
    """The 8-sequence varlen batch: every (sequence, head) unit against the
    oracle, and every sequence run alone equal to the packed run bit for bit."""
    inp = workloads.prefill_varlen_8seq_h32_d128(ejk=ejk)
    say("chunked varlen 8 seqs", "EJK" if ejk else "KDA", inp.meta["lengths"])
    o, s = prefill_gpu(inp)
    ro, rs = prefill_oracle(inp)
    check_units(o, ro, s, rs, TOL, margin, cu=inp.cu_seqlens,
                label="varlen 8 seqs " + ("EJK" if ejk else "KDA"))
    del ro, rs
    say("  packed vs separate")
    _packed_equals_separate(inp, o, s)


@pytest.mark.parametrize("T", [64, 1, 200])
def test_chunked_ejk_ragged(T):
    """EJK ordering on the MFMA path: scalar per-head decay, beta as given,
    residual against the undecayed state."""
    inp = workloads.prefill_inputs(2, T, 3, 128, 128, seed=900 + T, ejk=True, init_state=True)
    say("chunked EJK B=2 T=%d H=3" % T)
    _check(inp)


def test_chunked_ejk_strong_and_no_decay():
    inp = workloads.prefill_inputs(1, 256, 2, 128, 64, seed=950, ejk=True, init_state=True)
    inp.g = (-20.0 * np.abs(inp.g) / np.maximum(np.abs(inp.g).max(), 1e-30) - 3.0).astype(np.float32)
    say("chunked EJK strong decay (cumulative past e^-190 in a chunk)")
    _check(inp)
    inp.g = None
    say("chunked EJK without decay")
    _check(inp)


def test_chunked_ejk_matches_recurrent_kernel():
    import torch
    inp = workloads.prefill_inputs(1, 333, 2, 128, 128, seed=960, ejk=True, init_state=True)
    say("chunked EJK vs recurrent")
    oc, sc = prefill_gpu(inp, out_dtype=torch.float32)
    orc, src = prefill_gpu(inp, use_chunked=False, out_dtype=torch.float32)
    assert rel_l2(oc, orc) <= TOL and rel_l2(sc, src) <= TOL


def test_chunked_long_context_t65536_h32_split_and_every_head(margin):
    """One 65536-token sequence, 32 heads, nonzero initial state: the call split
    at 32768 with the state passed through equals the unsplit call bitwise, and
    every head matches the oracle."""
    inp = workloads.prefill_long_t65536_h32_d128()
    say("chunked long context T=65536 H=32")
    o, s = prefill_gpu(inp)
    cut = 32768

    def part(a, b, s0):
        return workloads.PrefillInputs(inp.q[:, a:b], inp.k[:, a:b], inp.v[:, a:b],
                                       inp.g[:, a:b], inp.beta[:, a:b], inp.a_log, inp.dt_bias,
                                       s0, None, inp.dtype, inp.scale, inp.lower_bound)

    say("  split at 32768")
    o1, s1 = prefill_gpu(part(0, cut, inp.initial_state))
    o2, s2 = prefill_gpu(part(cut, 65536, s1))
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(s2, s)
    del o1, o2
    say("  oracle on all 32 heads")
    ro, rs = prefill_oracle(inp)
    check_units(o, ro, s, rs, TOL, margin, label="T65536 H32")


@pytest.mark.parametrize("nseq", [300, 2100])
def test_chunked_varlen_many_sequences(nseq):
    """Many packed sequences with repeated and zero lengths: the longest-first
    scan order (sorted up to 2048 sequences, identity beyond) must not change
    any result."""
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, 131, nseq)
    lens[::7] = 64                      # ties
    lens[3::11] = 0                     # empty sequences
    inp = workloads.prefill_inputs(1, 0, 2, 128, 32, seed=1200 + nseq, lengths=list(lens),
                                   init_state=True)
    say("chunked varlen", nseq, "sequences, total", int(lens.sum()))
    o, s = _check(inp)
    empty = np.flatnonzero(lens == 0)
    np.testing.assert_array_equal(s[empty], inp.initial_state[empty])


def test_chunked_bf16_routing_falls_back_to_token_by_token():
    """bf16 inputs at dk = 128 with lower_bound < -5, or with an unaligned
    pointer, take the token-by-token kernel: bit for bit its result, and
    within the bar of the oracle."""
    import torch
    inp = workloads.prefill_inputs(2, 150, 2, 128, 64, seed=1300, init_state=True, lower_bound=-7.0)
    say("chunked bf16 routing: lower_bound -7")
    o, s = prefill_gpu(inp)
    orc, src = prefill_gpu(inp, use_chunked=False)
    np.testing.assert_array_equal(o, orc)
    np.testing.assert_array_equal(s, src)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(o, ro) <= TOL and rel_l2(s, rs) <= TOL

    inp = workloads.prefill_inputs(1, 100, 2, 128, 128, seed=1301, init_state=True)
    bf, f = torch.bfloat16, torch.float32

    def unaligned(x, dtype):
        flat = torch.empty(x.size + 1, dtype=dtype, device="cuda")
        view = flat[1:].view(x.shape)          # 2 or 4 bytes past an allocation boundary
        view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to("cuda"))
        return view

    rest = [dev(x, f) for x in (inp.g, inp.beta, inp.a_log, inp.dt_bias, inp.initial_state)]
    for name in ("q", "v"):
        say("chunked bf16 routing: unaligned", name)
        q = unaligned(inp.q, bf) if name == "q" else dev(inp.q, bf)
        v = unaligned(inp.v, bf) if name == "v" else dev(inp.v, bf)
        k = dev(inp.k, bf)
        o_u, s_u = kda.prefill(q, k, v, *rest, scale=inp.scale, lower_bound=inp.lower_bound,
                               return_state=True)
        o_r, s_r = kda.prefill(q, k, v, *rest, scale=inp.scale, lower_bound=inp.lower_bound,
                               use_chunked=False, return_state=True)
        torch.cuda.synchronize()
        assert torch.equal(o_u, o_r) and torch.equal(s_u, s_r)


@pytest.mark.parametrize("ejk", [False, True], ids=["kda", "ejk"])
@pytest.mark.parametrize("return_state", [True, False], ids=["state", "no_state"])
def test_chunked_dense_workspace_below_the_call_runs_in_segments(monkeypatch, ejk, return_state):
    """A dense call given less workspace than its whole records runs in segments of
    whole 64-token chunks of every sequence (the state carried in final_state, or in
    the workspace without one): the result equals the one-segment call bit for bit.
    Here three chunks per segment over 1000 tokens (16 chunks, a ragged last one)."""
    import torch
    inp = workloads.prefill_inputs(2, 1000, 4, 128, 64, seed=1700 + ejk, ejk=ejk, init_state=True)
    say("dense segments", "EJK" if ejk else "KDA", "with state" if return_state else "output only")
    io, f = torch.bfloat16, torch.float32

    def call():
        r = kda.prefill(dev(inp.q, io), dev(inp.k, io), dev(inp.v, io), dev(inp.g, f), dev(inp.beta, f),
                        None if ejk else dev(inp.a_log, f), None if ejk else dev(inp.dt_bias, f),
                        dev(inp.initial_state, f), scale=inp.scale, lower_bound=inp.lower_bound, ejk=ejk,
                        return_state=return_state)
        torch.cuda.synchronize()
        return [x.float().cpu().numpy() for x in (r if return_state else (r,))]

    ref = call()
    carry = 0 if return_state else 2 * 4 * 128 * 64 * 4
    small = carry + 3 * 2 * 4 * 66048          # three chunks of records for every (sequence, head)
    real = kda.prefill_workspace_bytes
    assert real(0, 2, 1000, 4, 128, 64, kda.QK_L2NORM | kda.CHUNKED) > small
    monkeypatch.setattr(kda, "prefill_workspace_bytes", lambda *a, **k: small)
    seg = call()
    for x, y in zip(seg, ref):
        np.testing.assert_array_equal(x, y)
    ro, rs = prefill_oracle(inp)
    assert rel_l2(seg[0], ro) <= TOL
