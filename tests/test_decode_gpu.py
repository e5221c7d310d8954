"""kda_decode_step (the kda_tkg-shaped single-token step) against the oracle.

Bar: relative L2 <= 1e-5 for out and the new state (fp32 path)."""
import numpy as np
import pytest

from gated_delta_rule_90_amd import workloads
from tests._common import check_units, decode_gpu, decode_oracle, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def test_decode_full_size_b64_h32_d128(margin):
    """The benchmark step: every (request, head) unit against the oracle."""
    inp = workloads.decode_b64_h32_d128()
    say("decode full size B=64 H=32 dk=dv=128")
    out, S = decode_gpu(inp)
    ro, rS = decode_oracle(inp)
    # out [B, H, dv] viewed as one token per request
    check_units(out[:, None], ro[:, None], S, rS, TOL, margin, label="decode B64 H32")


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


def test_decode_state_beyond_2e31_elements():
    """A batch whose state holds more than 2^31 elements (B=4100, H=32, dk=dv=128:
    8.6 GB of fp32 state): items past element 2^31 are advanced like the first.
    The state is drawn on the device from a seeded generator; the sampled items'
    incoming states are copied back before the call and given to the oracle."""
    import torch
    import gated_delta_rule_90_amd as kda
    from oracle import kda_oracle
    from tests._common import dev
    B, H, dk, dv = 4100, 32, 128, 128
    assert B * H * dk * dv > 2 ** 31
    rng = np.random.default_rng(4100)
    q = rng.standard_normal((B, dk, H), dtype=np.float32)
    k = rng.standard_normal((B, dk, H), dtype=np.float32)
    g = rng.standard_normal((B, dk, H), dtype=np.float32)
    v = rng.standard_normal((B, H, dv), dtype=np.float32)
    beta = rng.standard_normal((B, 1, H), dtype=np.float32)
    a_log = rng.uniform(-1.0, 1.0, size=(1, H)).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal((dk, H))).astype(np.float32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4100)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda").normal_(0.0, 0.02, generator=gen)
    # item b * H + h starts at element (b * H + h) * dk * dv: (4096, 0) starts exactly at 2^31
    items = [(0, 0), (2049, 7), (4095, 31), (4096, 0), (4099, 17), (B - 1, H - 1)]
    before = {it: S[it[0], it[1]].cpu().numpy() for it in items}
    say("decode B=4100 H=32 dk=dv=128 (state > 2^31 elements)")
    f = torch.float32
    out = kda.decode_step(dev(q, f), dev(k, f), dev(v, f), dev(g, f), dev(beta, f), dev(a_log, f),
                          dev(dt_bias, f), S, scale=1.0 / np.sqrt(dk), lower_bound=-5.0)
    torch.cuda.synchronize()
    for b, h in items:
        ro, rS = kda_oracle.decode(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], g[b:b + 1, :, h:h + 1],
                                   v[b:b + 1, h:h + 1], beta[b:b + 1, :, h:h + 1], a_log[:, h:h + 1],
                                   dt_bias[:, h:h + 1], before[(b, h)][None, None],
                                   scale=1.0 / np.sqrt(dk), lower_bound=-5.0)
        eo = rel_l2(out[b, h].cpu().numpy(), ro[0, 0])
        es = rel_l2(S[b, h].cpu().numpy(), rS[0, 0])
        assert eo <= TOL and es <= TOL, (b, h, eo, es)
    del S
    torch.cuda.empty_cache()
