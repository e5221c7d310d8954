"""kda_decode_step (the kda_tkg-shaped single-token step) against the oracle.

Bar: relative L2 <= 1e-5 for out and the new state (fp32 path)."""
import numpy as np
import pytest

from gated_delta_rule_90_amd import workloads
from tests._common import decode_gpu, decode_oracle, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def test_decode_full_size_b64_h32_d128():
    inp = workloads.decode_b64_h32_d128()
    say("decode full size B=64 H=32 dk=dv=128")
    out, S = decode_gpu(inp)
    ro, rS = decode_oracle(inp)
    assert rel_l2(out, ro) <= TOL, rel_l2(out, ro)
    assert rel_l2(S, rS) <= TOL, rel_l2(S, rS)


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
@pytest.mark.parametrize("ejk", [False, True])
def test_decode_shapes(dk, dv, ejk):
    inp = workloads.decode_inputs(3, 5, dk, dv, seed=7 + dk + dv, ejk=ejk)
    say("decode B=3 H=5", dk, dv, "ejk" if ejk else "kda")
    out, S = decode_gpu(inp)
    ro, rS = decode_oracle(inp)
    assert rel_l2(out, ro) <= TOL and rel_l2(S, rS) <= TOL, (rel_l2(out, ro), rel_l2(S, rS))


def test_decode_without_l2norm_and_custom_scale():
    inp = workloads.decode_inputs(2, 3, 64, 32, seed=11, scale=0.3, lower_bound=-2.0)
    say("decode no l2norm")
    out, S = decode_gpu(inp, use_qk_l2norm=False)
    ro, rS = decode_oracle(inp, use_qk_l2norm=False)
    assert rel_l2(out, ro) <= TOL and rel_l2(S, rS) <= TOL


def test_decode_ejk_null_decay_means_no_decay():
    inp = workloads.decode_inputs(2, 4, 32, 32, seed=12, ejk=True)
    inp.g = None
    say("decode ejk g=None")
    out, S = decode_gpu(inp)
    ro, rS = decode_oracle(inp)
    assert rel_l2(out, ro) <= TOL and rel_l2(S, rS) <= TOL


def test_decode_steps_chain_and_determinism():
    """Eight chained steps on the device state stay within tolerance of the
    oracle's chain, and rerunning gives bitwise identical results."""
    base = workloads.decode_inputs(4, 6, 128, 128, seed=13)
    S_ref = base.S.astype(np.float64)
    import torch
    from tests._common import dev
    import gated_delta_rule_90_amd as kda
    f = torch.float32
    S_gpu = dev(base.S, f)
    S_gpu2 = dev(base.S, f)
    for step in range(8):
        inp = workloads.decode_inputs(4, 6, 128, 128, seed=100 + step)
        say("decode chain step", step)
        args = [dev(x, f) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.a_log, inp.dt_bias)]
        o1 = kda.decode_step(*args, S_gpu, scale=inp.scale)
        o2 = kda.decode_step(*args, S_gpu2, scale=inp.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S_gpu, S_gpu2)
        ro, S_ref = decode_oracle(inp, S=S_ref)
        assert rel_l2(o1.cpu().numpy(), ro) <= TOL
    assert rel_l2(S_gpu.cpu().numpy(), S_ref) <= TOL


def test_decode_empty_batch():
    import torch
    import gated_delta_rule_90_amd as kda
    f = torch.float32
    z = lambda *s: torch.zeros(*s, dtype=f, device="cuda")
    out = kda.decode_step(z(0, 16, 2), z(0, 16, 2), z(0, 2, 16), z(0, 16, 2), z(0, 1, 2),
                          z(1, 2), z(16, 2), z(0, 2, 16, 16))
    assert out.shape == (0, 2, 16)
