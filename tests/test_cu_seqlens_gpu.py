"""cu_seqlens entries outside [0, T] or out of order, on every prefill path.

include/kda.h: device values are not inspected; out-of-range entries are
clamped to [0, T] and a decreasing pair is an empty sequence, so the kernels
never address memory outside the buffers.  Checked here:
  * out-of-range but non-overlapping entries give, bit for bit, the result of
    the clamped cu_seqlens;
  * overlapping ranges (each other sequence spans the whole batch), which on
    the bf16 chunked path count more chunks than the workspace has record
    slots: the call completes, the first sequence's output and state equal a
    run of that sequence alone, and the empty sequences keep their state."""
import numpy as np
import pytest

import gated_delta_rule_90_amd as kda
from gated_delta_rule_90_amd import workloads
from tests._common import dev, say

pytestmark = pytest.mark.gpu

PATHS = [("bf16", 128, True), ("f32", 64, True), ("f32", 32, False)]   # MFMA, float32 chunked, token by token


def _run(inp, cu, n_states, use_chunked, init=None):
    import torch
    io = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f = torch.float32
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    s0 = None if init is None else dev(init, f)
    fs = torch.zeros((n_states, H, dk, dv), dtype=f, device="cuda")
    o = torch.zeros((B, T, H, dv), dtype=f, device="cuda")
    kda.prefill(dev(inp.q, io), dev(inp.k, io), dev(inp.v, io), dev(inp.g, f), dev(inp.beta, f),
                dev(inp.a_log, f), dev(inp.dt_bias, f), s0, None if cu is None else dev(np.asarray(cu, np.int32)),
                scale=inp.scale, lower_bound=inp.lower_bound, use_chunked=use_chunked, out=o,
                final_state=fs, out_dtype=f)
    torch.cuda.synchronize()
    return o.cpu().numpy(), fs.cpu().numpy()


@pytest.mark.parametrize("dtype,dk,use_chunked", PATHS)
def test_out_of_range_entries_are_clamped(dtype, dk, use_chunked):
    inp = workloads.prefill_inputs(1, 100, 2, dk, 64, seed=600 + dk, dtype=dtype)
    init = np.random.default_rng(1).standard_normal((2, 2, dk, 64)).astype(np.float32) * 0.02
    say("cu_seqlens out of range", dtype, dk, use_chunked)
    o_bad, s_bad = _run(inp, [-5, 60, 250], 2, use_chunked, init)
    o_ok, s_ok = _run(inp, [0, 60, 100], 2, use_chunked, init)
    np.testing.assert_array_equal(o_bad, o_ok)
    np.testing.assert_array_equal(s_bad, s_ok)


@pytest.mark.parametrize("dtype,dk,use_chunked", PATHS)
def test_overlapping_ranges_stay_in_bounds(dtype, dk, use_chunked):
    # bf16 chunked path: 16 chunks per sequence and T / 64 + 5 = 21 record slots,
    # so the third sequence gets 5 (an odd count: the padded step stores nothing)
    # and the fifth none
    T = 1024
    inp = workloads.prefill_inputs(1, T, 2, dk, 64, seed=610 + dk, dtype=dtype)
    say("cu_seqlens overlapping", dtype, dk, use_chunked)
    o_bad, s_bad = _run(inp, [0, T, 0, T, 0, T], 5, use_chunked)
    o_one, s_one = _run(inp, None, 1, use_chunked)
    assert np.all(np.isfinite(o_bad)) and np.all(np.isfinite(s_bad))
    np.testing.assert_array_equal(s_bad[0], s_one[0])
    np.testing.assert_array_equal(o_bad, o_one)   # every writer of a row computes the same values
    assert np.all(s_bad[1] == 0) and np.all(s_bad[3] == 0)
