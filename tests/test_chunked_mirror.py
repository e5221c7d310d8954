"""The chunk-parallel algebra of the prefill kernel, checked in float64 against
the oracle before any kernel runs: sub-block decay factorisation, blocked
triangular inverse and the WY state carry reproduce the token recurrence to
rounding, including ragged tails, varlen packing and the strongest decay the
chunked path accepts (lower_bound = -5)."""
import numpy as np
import pytest

from oracle import kda_oracle
from tests import chunked_mirror


def _rel(a, b):
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


@pytest.mark.parametrize("T", [64, 100, 7, 128])
def test_mirror_matches_oracle_dense(T):
    rng = np.random.default_rng(T)
    B, H, dk, dv = 2, 2, 32, 16
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v, g = rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, T, H, dk))
    beta = rng.standard_normal((B, T, H))
    a_log, dtb = rng.uniform(-1, 1, H), 0.1 * rng.standard_normal((dk, H))
    s0 = 0.02 * rng.standard_normal((B, H, dk, dv))
    o, s = chunked_mirror.prefill(q, k, v, g, beta, a_log, dtb, s0)
    ro, rs = kda_oracle.prefill(q, k, v, g, beta, a_log, dtb, s0)
    assert _rel(o, ro) < 1e-11 and _rel(s, rs) < 1e-11


def test_mirror_strongest_decay_and_saturated_gates():
    """lower_bound = -5 with large gate logits: in-chunk cumulative decay
    reaches ~ -320, far past fp32's exp range; the factorisation must stay
    finite and exact."""
    rng = np.random.default_rng(1)
    T, H, dk, dv = 192, 1, 16, 8
    q, k = rng.standard_normal((1, T, H, dk)), rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    g = 20.0 + rng.standard_normal((1, T, H, dk))  # sigma ~ 1: gamma ~ lb per step
    beta = rng.standard_normal((1, T, H))
    a_log, dtb = np.zeros(H), np.zeros((dk, H))
    s0 = rng.standard_normal((1, H, dk, dv))
    o, s = chunked_mirror.prefill(q, k, v, g, beta, a_log, dtb, s0, lower_bound=-5.0)
    ro, rs = kda_oracle.prefill(q, k, v, g, beta, a_log, dtb, s0, lower_bound=-5.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert _rel(o, ro) < 1e-11
    np.testing.assert_allclose(s, rs, atol=1e-300, rtol=1e-9)


def test_mirror_varlen_and_no_l2norm():
    rng = np.random.default_rng(2)
    lens = [70, 0, 64, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    N = int(cu[-1])
    H, dk, dv = 2, 16, 16
    q, k = rng.standard_normal((1, N, H, dk)), 0.3 * rng.standard_normal((1, N, H, dk))
    v, g = rng.standard_normal((1, N, H, dv)), rng.standard_normal((1, N, H, dk))
    beta = rng.standard_normal((1, N, H))
    a_log, dtb = rng.uniform(-1, 1, H), 0.1 * rng.standard_normal((dk, H))
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    for l2 in (True, False):
        o, s = chunked_mirror.prefill(q, k, v, g, beta, a_log, dtb, s0, cu_seqlens=cu,
                                      use_qk_l2norm=l2, scale=0.3)
        ro, rs = kda_oracle.prefill(q, k, v, g, beta, a_log, dtb, s0, cu_seqlens=cu,
                                    use_qk_l2norm=l2, scale=0.3)
        assert _rel(o, ro) < 1e-11 and _rel(s, rs) < 1e-11


@pytest.mark.parametrize("decay", ["mild", "strong", "none"])
def test_mirror_ejk_matches_oracle(decay):
    """EJK: scalar per-head decay, beta as given, residual against the
    undecayed state.  'strong' takes the cumulative decay in a chunk past
    e^-1000 (every scaled factor underflows cleanly to zero)."""
    rng = np.random.default_rng(11)
    lens = [130, 64, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    N = int(cu[-1])
    H, dk, dv = 2, 16, 8
    q, k = rng.standard_normal((1, N, H, dk)), rng.standard_normal((1, N, H, dk))
    v = rng.standard_normal((1, N, H, dv))
    beta = rng.uniform(0.0, 1.0, (1, N, H))
    if decay == "none":
        d = None
    elif decay == "mild":
        d = -0.05 * np.abs(rng.standard_normal((1, N, H)))
    else:
        d = -20.0 * np.abs(rng.standard_normal((1, N, H)))
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    o, s = chunked_mirror.prefill(q, k, v, d, beta, initial_state=s0, cu_seqlens=cu, ejk=True)
    ro, rs = kda_oracle.prefill(q, k, v, d, beta, None, None, s0, cu_seqlens=cu, ejk=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert _rel(o, ro) < 1e-11 and _rel(s, rs) < 1e-11
