"""The chunk-level backward algebra (tests/chunked_bwd_mirror.py, float64)
against the token-by-token backward oracle: equal to rounding on ragged
chunks, packed sequences, strong decay and both orderings."""
import numpy as np
import pytest

from oracle import kda_oracle
from tests import chunked_bwd_mirror as M


@pytest.mark.parametrize("ejk,l2norm,strong", [(False, True, False), (True, True, False),
                                               (False, False, False), (False, True, True),
                                               (True, True, True)])
def test_chunk_backward_equals_token_backward(ejk, l2norm, strong):
    r = np.random.default_rng(40 + 2 * ejk + strong)
    lengths = [37, 0, 16, 5]
    T, H, dk, dv = sum(lengths), 2, 8, 6
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v = r.normal(size=(1, T, H, dk)), r.normal(size=(1, T, H, dk)), r.normal(size=(1, T, H, dv))
    if ejk:
        g = -(3.0 if strong else 0.05) * np.abs(r.normal(size=(1, T, H)))
        beta = 1 / (1 + np.exp(-r.normal(size=(1, T, H))))
    else:
        g = r.normal(size=(1, T, H, dk)) + (8.0 if strong else 0.0)   # strong: sigmoid near 1
        beta = r.normal(size=(1, T, H))
    a_log, dtb = r.uniform(-1, 1, H), r.normal(0, 0.1, (dk, H))
    S0 = r.normal(0, 0.3, (len(lengths), H, dk, dv))
    dO, dSf = r.normal(size=(1, T, H, dv)), r.normal(size=(len(lengths), H, dk, dv))
    sc, lb = 0.4, -5.0
    ref = kda_oracle.backward(q, k, v, g, beta, a_log, dtb, S0, cu, d_o=dO, d_final_state=dSf, scale=sc,
                              lower_bound=lb, use_qk_l2norm=l2norm, ejk=ejk)
    got = M.backward(q, k, v, g, beta, a_log, dtb, S0, cu, dO, dSf, sc, lb, l2norm, ejk)
    pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
             ("d_initial_state", "dS0")]
    if not ejk:
        pairs += [("da_log", "da_log"), ("ddt_bias", "ddt_bias")]
    for a, b in pairs:
        err = np.linalg.norm(got[b] - ref[a]) / max(np.linalg.norm(ref[a]), 1e-300)
        assert err < 1e-10, (a, err)
