"""kda_prefill_backward against the float64 backward oracle.

Every gradient (dq, dk, dv, dg, dbeta, da_log, ddt_bias, d_initial_state) is
compared with the oracle's by relative L2: <= 1e-5 with float32 inputs and
<= 2e-2 with bf16 inputs (the kernels compute in float32 either way, so the
bf16 cases land far inside their bar).  Cases: every dk in {16, 32, 64, 128}
with several dv, both orderings, ragged and packed sequences (with an empty
one), grouped heads, a nonzero initial state and final-state gradient, no L2
norm, strong decay."""
import numpy as np
import pytest

import gated_delta_rule_90_amd as kda
from gated_delta_rule_90_amd import workloads
from oracle import kda_oracle
from tests._common import dev, rel_l2, say

pytestmark = pytest.mark.gpu


def _run(inp, d_o, d_sf, use_qk_l2norm=True, do_bf16=False):
    import torch
    io = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f = torch.float32
    gr = kda.prefill_backward(
        dev(inp.q, io), dev(inp.k, io), dev(inp.v, io), dev(inp.g, f), dev(inp.beta, f),
        None if inp.ejk else dev(inp.a_log, f), None if inp.ejk else dev(inp.dt_bias, f),
        dev(inp.initial_state, f), dev(inp.cu_seqlens, torch.int32),
        dev(d_o, torch.bfloat16 if do_bf16 else f), dev(d_sf, f), scale=inp.scale,
        lower_bound=inp.lower_bound, use_qk_l2norm=use_qk_l2norm, ejk=inp.ejk)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in gr.items()}


def _check(inp, tol, use_qk_l2norm=True, seed=0, do_bf16=False, margin=None, label=""):
    r = np.random.default_rng(seed)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    d_o = r.normal(size=(B, T, H, dv)).astype(np.float32)
    if do_bf16:
        d_o = workloads.round_to_bf16(d_o)
    d_sf = r.normal(size=(N, H, dk, dv)).astype(np.float32)
    got = _run(inp, d_o, d_sf, use_qk_l2norm, do_bf16)
    ref = kda_oracle.backward(inp.q, inp.k, inp.v, inp.g, inp.beta,
                              None if inp.ejk else inp.a_log, None if inp.ejk else inp.dt_bias,
                              inp.initial_state, inp.cu_seqlens, d_o=d_o, d_final_state=d_sf,
                              scale=inp.scale, lower_bound=inp.lower_bound,
                              use_qk_l2norm=use_qk_l2norm, ejk=inp.ejk)
    errs = {}
    for name, want in ref.items():
        have = got[name]
        assert have.shape == want.shape, (name, have.shape, want.shape)
        assert np.all(np.isfinite(have)), name
        errs[name] = rel_l2(have, want)
    worst = max(errs, key=errs.get)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    if margin is not None:
        margin(f"{label} worst gradient ({worst})", errs[worst], tol)
    assert errs[worst] <= tol, errs


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
@pytest.mark.parametrize("ejk", [False, True], ids=["kda", "ejk"])
def test_backward_fp32_shapes(dk, dv, ejk, margin):
    inp = workloads.prefill_inputs(2, 45, 3, dk, dv, seed=1700 + dk + dv, dtype="f32", ejk=ejk,
                                   init_state=True)
    say("backward fp32", dk, dv, "EJK" if ejk else "KDA")
    _check(inp, 1e-5, seed=dk + dv, margin=margin, label=f"fp32 dk{dk} dv{dv}")


@pytest.mark.parametrize("ejk", [False, True], ids=["kda", "ejk"])
def test_backward_bf16_varlen_grouped(ejk, margin):
    inp = workloads.prefill_inputs(1, 0, 4, 128, 128, seed=1710 + ejk, ejk=ejk, init_state=True,
                                   lengths=[100, 0, 17, 64, 1], hkv=2)
    say("backward bf16 varlen grouped", "EJK" if ejk else "KDA")
    _check(inp, 2e-2, seed=5, do_bf16=True, margin=margin, label="bf16 varlen grouped")


def test_backward_fp32_varlen_grouped_tight(margin):
    inp = workloads.prefill_inputs(1, 0, 6, 64, 32, seed=1712, dtype="f32", init_state=True,
                                   lengths=[33, 0, 16, 70], hkv=3)
    say("backward fp32 varlen grouped")
    _check(inp, 1e-5, seed=6, margin=margin, label="fp32 varlen grouped")


def test_backward_no_l2norm_and_strong_decay(margin):
    inp = workloads.prefill_inputs(1, 90, 2, 64, 64, seed=1720, dtype="f32", init_state=True, scale=0.1)
    inp.q *= 0.2
    inp.k *= 0.2
    say("backward no l2 norm")
    _check(inp, 1e-5, use_qk_l2norm=False, seed=7, margin=margin, label="fp32 no l2 norm")
    inp = workloads.prefill_inputs(1, 90, 2, 128, 64, seed=1721, dtype="f32", init_state=True)
    inp.g = (inp.g + 8.0).astype(np.float32)      # gates near lower_bound = -5
    say("backward saturated gates")
    _check(inp, 1e-5, seed=8, margin=margin, label="fp32 saturated gates")
    inp = workloads.prefill_inputs(1, 90, 2, 128, 64, seed=1722, dtype="f32", ejk=True, init_state=True)
    inp.g = (-6.0 * np.abs(inp.g)).astype(np.float32)
    say("backward EJK strong decay")
    _check(inp, 1e-5, seed=9, margin=margin, label="fp32 EJK strong decay")


def test_backward_no_tokens_carries_the_state_gradient():
    import torch
    inp = workloads.prefill_inputs(2, 0, 2, 32, 32, seed=1730, dtype="f32", init_state=True)
    f = torch.float32
    d_sf = np.random.default_rng(1).normal(size=(2, 2, 32, 32)).astype(np.float32)
    say("backward with no tokens")
    gr = kda.prefill_backward(dev(inp.q, f), dev(inp.k, f), dev(inp.v, f), dev(inp.g, f), dev(inp.beta, f),
                              dev(inp.a_log, f), dev(inp.dt_bias, f), dev(inp.initial_state, f), None,
                              dev(np.zeros((2, 0, 2, 32), np.float32), f), dev(d_sf, f))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gr["d_initial_state"].cpu().numpy(), d_sf)
    assert torch.count_nonzero(gr["da_log"]) == 0 and torch.count_nonzero(gr["ddt_bias"]) == 0


def test_backward_b2_t1024_h8_d128_bf16(margin):
    """A training-sized call: every gradient against the oracle."""
    inp = workloads.prefill_inputs(2, 1024, 8, 128, 128, seed=1740, init_state=True)
    say("backward bf16 B2 T1024 H8 d128")
    _check(inp, 2e-2, seed=10, do_bf16=True, margin=margin, label="B2 T1024 H8")


@pytest.mark.parametrize("ejk", [False, True], ids=["kda", "ejk"])
def test_backward_two_tiles_per_scan_workgroup(ejk, margin):
    """Enough (sequence, head) units that each scan workgroup carries two
    16-column tiles over one shared copy of the chunk operands: 256 units at
    dv = 32 (float32), 256 at dv = 128 (bf16) and 64 packed sequences of 8
    heads with grouped keys (ragged, with empty ones)."""
    inp = workloads.prefill_inputs(4, 50, 64, 32, 32, seed=1760 + ejk, dtype="f32", ejk=ejk, init_state=True)
    say("backward fp32 B4 T50 H64 d32", "EJK" if ejk else "KDA")
    _check(inp, 1e-5, seed=12, margin=margin, label="fp32 B4 T50 H64 d32 (two tiles per scan workgroup)")
    inp = workloads.prefill_inputs(8, 80, 32, 128, 128, seed=1762 + ejk, ejk=ejk, init_state=True)
    say("backward bf16 B8 T80 H32 d128", "EJK" if ejk else "KDA")
    _check(inp, 2e-2, seed=13, do_bf16=True, margin=margin, label="B8 T80 H32 (two tiles per scan workgroup)")
    lengths = [int(x) for x in np.random.default_rng(1764 + ejk).integers(0, 70, size=64)]
    inp = workloads.prefill_inputs(1, 0, 8, 64, 64, seed=1766 + ejk, dtype="f32", ejk=ejk, init_state=True,
                                   lengths=lengths, hkv=2)
    say("backward fp32 64 packed sequences H8 Hkv2 d64", "EJK" if ejk else "KDA")
    _check(inp, 1e-5, seed=14, margin=margin, label="fp32 64 packed sequences (two tiles)")


def test_backward_unaligned_inputs_take_the_own_forward_scan():
    """A query 4 bytes past an allocation boundary: the first pass runs on the
    backward's own forward scan instead of the float32 chunked kernel (which
    needs 16-byte aligned rows); both against the oracle."""
    import torch
    inp = workloads.prefill_inputs(1, 70, 2, 64, 32, seed=1750, dtype="f32", init_state=True)
    r = np.random.default_rng(11)
    d_o = r.normal(size=(1, 70, 2, 32)).astype(np.float32)
    f = torch.float32
    flat = torch.empty(inp.q.size + 1, dtype=f, device="cuda")
    qu = flat[1:].view(inp.q.shape)
    qu.copy_(dev(inp.q, f))
    say("backward with an unaligned query")
    gr = kda.prefill_backward(qu, dev(inp.k, f), dev(inp.v, f), dev(inp.g, f), dev(inp.beta, f),
                              dev(inp.a_log, f), dev(inp.dt_bias, f), dev(inp.initial_state, f), None,
                              dev(d_o, f), None, scale=inp.scale, lower_bound=inp.lower_bound)
    torch.cuda.synchronize()
    ref = kda_oracle.backward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.a_log, inp.dt_bias, inp.initial_state,
                              None, d_o=d_o, scale=inp.scale, lower_bound=inp.lower_bound)
    for name, want in ref.items():
        assert rel_l2(gr[name].cpu().numpy(), want) <= 1e-5, name
