"""Grouped key/value heads on every kernel (ejkernel "recurrent" run(): key and
value carry num_kv_heads, query, gates, state and output num_heads; head h
reads key/value head h // (H // Hkv)).

Two checks per case:
- against the oracle, to the usual bars (relative L2 <= 1e-5 on the fp32
  paths, <= 2e-2 with bf16 inputs);
- bit for bit against the same kernel run without grouping on keys and
  values repeated per group: grouping changes which rows are read, not the
  arithmetic.
"""
import numpy as np
import pytest

from gated_delta_rule_90_amd import workloads
from tests._common import check_units, decode_gpu, decode_oracle, prefill_gpu, prefill_oracle, rel_l2, say

pytestmark = pytest.mark.gpu


def _expanded(inp):
    """The same inputs with k and v repeated per group (Hkv = H)."""
    import copy
    H, hkv = inp.q.shape[2], inp.k.shape[2]
    e = copy.copy(inp)
    e.k = np.ascontiguousarray(np.repeat(inp.k, H // hkv, axis=2))
    e.v = np.ascontiguousarray(np.repeat(inp.v, H // hkv, axis=2))
    return e


def _check_prefill(inp, tol, units=None, **kw):
    o, s = prefill_gpu(inp, **kw)
    oe, se = prefill_gpu(_expanded(inp), **kw)
    assert np.array_equal(o, oe) and np.array_equal(s, se)
    ro, rs = prefill_oracle(inp, units=units)
    if units is not None:
        H = inp.q.shape[2]
        sel = [(u // H, u % H) for u in units]
        o, ro = np.stack([o[n, :, h] for n, h in sel]), np.stack([ro[n, :, h] for n, h in sel])
        s, rs = np.stack([s[n, h] for n, h in sel]), np.stack([rs[n, h] for n, h in sel])
    eo, es = rel_l2(o, ro), rel_l2(s, rs)
    say(f"  rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("dk,dv,H,hkv", [(16, 16, 4, 2), (64, 32, 6, 3), (128, 128, 4, 1)])
def test_recurrent_grouped(dk, dv, H, hkv):
    inp = workloads.prefill_inputs(2, 37, H, dk, dv, seed=70 + dk, dtype="f32", init_state=True, hkv=hkv)
    say("recurrent grouped", dk, dv, H, hkv)
    _check_prefill(inp, 1e-5, use_chunked=False)


def test_recurrent_grouped_ejk_varlen():
    inp = workloads.prefill_inputs(1, 0, 4, 32, 32, seed=75, dtype="f32", ejk=True, init_state=True,
                                   lengths=[9, 0, 21], hkv=2)
    say("recurrent grouped EJK varlen")
    _check_prefill(inp, 1e-5, use_chunked=False)


@pytest.mark.parametrize("T,H,hkv,dv", [(200, 4, 2, 128), (130, 6, 1, 64), (64, 8, 4, 32)])
def test_chunked_grouped(T, H, hkv, dv):
    inp = workloads.prefill_inputs(2, T, H, 128, dv, seed=76 + T, init_state=True, hkv=hkv)
    say("chunked grouped", T, H, hkv, dv)
    _check_prefill(inp, 2e-2)


def test_chunked_grouped_ejk_varlen():
    inp = workloads.prefill_inputs(1, 0, 4, 128, 128, seed=79, ejk=True, init_state=True,
                                   lengths=[100, 1, 0, 257], hkv=2)
    say("chunked grouped EJK varlen")
    _check_prefill(inp, 2e-2)


def test_chunked_grouped_full_size_b4_t4096_h16_hkv4_every_unit(margin):
    """The grouped benchmark workload: bitwise equal to the ungrouped run on
    repeated keys and values, and all 64 (batch, head) units against the oracle."""
    inp = workloads.prefill_grouped_b4_t4096_h16_hkv4_d128()
    say("chunked grouped B=4 T=4096 H=16 Hkv=4")
    o, s = prefill_gpu(inp)
    oe, se = prefill_gpu(_expanded(inp))
    assert np.array_equal(o, oe) and np.array_equal(s, se)
    del oe, se
    ro, rs = prefill_oracle(inp)
    check_units(o, ro, s, rs, 2e-2, margin, label="grouped B4 T4096 H16 Hkv4")


@pytest.mark.parametrize("dk,dv,H,hkv,ejk", [(128, 128, 8, 2, False), (16, 64, 6, 3, False),
                                             (64, 128, 4, 1, True)])
def test_decode_grouped(dk, dv, H, hkv, ejk):
    inp = workloads.decode_inputs(5, H, dk, dv, seed=81 + dk, ejk=ejk, hkv=hkv)
    say("decode grouped", dk, dv, H, hkv, "ejk" if ejk else "kda")
    out, S = decode_gpu(inp)
    e = workloads.decode_inputs(5, H, dk, dv, seed=81 + dk, ejk=ejk, hkv=hkv)
    e.k = np.ascontiguousarray(np.repeat(e.k, H // hkv, axis=2))
    e.v = np.ascontiguousarray(np.repeat(e.v, H // hkv, axis=1))
    oute, Se = decode_gpu(e)
    assert np.array_equal(out, oute) and np.array_equal(S, Se)
    ro, rS = decode_oracle(inp)
    assert rel_l2(out, ro) <= 1e-5 and rel_l2(S, rS) <= 1e-5, (rel_l2(out, ro), rel_l2(S, rS))


def test_decode_grouped_full_size_b64_h32_hkv8(margin):
    inp = workloads.decode_grouped_b64_h32_hkv8_d128()
    say("decode grouped B=64 H=32 Hkv=8")
    out, S = decode_gpu(inp)
    ro, rS = decode_oracle(inp)
    check_units(out[:, None], ro[:, None], S, rS, 1e-5, margin, label="decode grouped B64 H32 Hkv8")
