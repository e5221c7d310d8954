"""Pins of the float64 backward oracle (oracle.kda_oracle.backward), on the CPU.

The reverse sweep is checked against things it does not share code with:
- central finite differences of the forward oracle, for every element of
  every input (KDA and EJK, packed sequences with an empty one, grouped
  heads, a nonzero initial state and final-state gradient, with and without
  the L2 norm);
- closed forms: pure decay (beta = 0), where the state is the initial state
  scaled by the running product of the gates, and the first token from a zero
  state, o_1 = beta (kh . qh) v;
- linearity of the gradients in (dO, dS_T).
"""
import numpy as np
import pytest

from oracle import kda_oracle

RNG = np.random.default_rng


def _case(ejk, l2norm=True, seed=0, lengths=(3, 0, 4), H=2, hkv=1, dk=4, dv=3):
    r = RNG(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    x = dict(q=r.normal(size=(1, T, H, dk)), k=r.normal(size=(1, T, hkv, dk)),
             v=r.normal(size=(1, T, hkv, dv)),
             g=(-0.3 * np.abs(r.normal(size=(1, T, H))) if ejk else r.normal(size=(1, T, H, dk))),
             beta=(1 / (1 + np.exp(-r.normal(size=(1, T, H)))) if ejk else r.normal(size=(1, T, H))),
             a_log=r.uniform(-1, 1, H), dt_bias=r.normal(0, 0.3, (dk, H)),
             initial_state=r.normal(0, 0.5, (N, H, dk, dv)))
    kw = dict(cu_seqlens=cu, scale=0.7, lower_bound=-3.0, ejk=ejk, use_qk_l2norm=l2norm)
    W_o = r.normal(size=(1, T, H, dv))
    W_s = r.normal(size=(N, H, dk, dv))
    return x, kw, W_o, W_s


def _loss(x, kw, W_o, W_s):
    o, s = kda_oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["a_log"], x["dt_bias"],
                              x["initial_state"], **kw)
    return float(np.sum(o * W_o) + np.sum(s * W_s))


def _grads(x, kw, W_o, W_s):
    return kda_oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["a_log"], x["dt_bias"],
                               x["initial_state"], d_o=W_o, d_final_state=W_s, **kw)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "a_log": "da_log",
         "dt_bias": "ddt_bias", "initial_state": "d_initial_state"}


@pytest.mark.parametrize("ejk,l2norm,hkv", [(False, True, 1), (True, True, 2), (False, False, 2),
                                            (True, False, 1)])
def test_backward_matches_central_differences(ejk, l2norm, hkv):
    x, kw, W_o, W_s = _case(ejk, l2norm, seed=3 + ejk, hkv=hkv)
    gr = _grads(x, kw, W_o, W_s)
    h = 1e-6
    for name, gname in NAMES.items():
        if ejk and name in ("a_log", "dt_bias"):
            continue
        a = x[name]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + h
            lp = _loss(x, kw, W_o, W_s)
            a[idx] = old - h
            lm = _loss(x, kw, W_o, W_s)
            a[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(gr[gname] - fd))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), (name, err)


def test_pure_decay_closed_form():
    """beta = 0: S_t = Diag(prod_{s<=t} e^{gamma_s}) S0 and o_t = S_t^T qh_t, so
    dS0 = sum_t Diag(P_t) qh_t dO_t^T + Diag(P_T) dS_T, dqh_t = S_t dO_t,
    dv = 0, and dgamma_{t,i} = sum_{t'>=t} (S_t' qh_t' dO_t'^T summed over j)_i
    + (S_T * dS_T summed over j)_i."""
    r = RNG(11)
    T, H, dk, dv = 6, 1, 3, 2
    q, k, v = r.normal(size=(1, T, H, dk)), r.normal(size=(1, T, H, dk)), r.normal(size=(1, T, H, dv))
    g = r.normal(size=(1, T, H, dk))
    beta = np.full((1, T, H), -np.inf)
    a_log, dtb = np.array([0.3]), r.normal(0, 0.2, (dk, H))
    S0 = r.normal(size=(1, H, dk, dv))
    dO, dST = r.normal(size=(1, T, H, dv)), r.normal(size=(1, H, dk, dv))
    lb, sc = -2.0, 0.9
    gr = kda_oracle.backward(q, k, v, g, beta, a_log, dtb, S0, d_o=dO, d_final_state=dST, scale=sc,
                             lower_bound=lb, use_qk_l2norm=False)
    x = np.exp(a_log[0]) * (g[0, :, 0] + dtb[:, 0])
    gam = lb / (1 + np.exp(-x))                      # [T, dk]
    P = np.exp(np.cumsum(gam, axis=0))               # running products
    S = [P[t][:, None] * S0[0, 0] for t in range(T)]
    qh = sc * q[0, :, 0]
    dS0 = sum(P[t][:, None] * np.outer(qh[t], dO[0, t, 0]) for t in range(T)) + P[-1][:, None] * dST[0, 0]
    np.testing.assert_allclose(gr["d_initial_state"][0, 0], dS0, rtol=1e-12, atol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(gr["dq"][0, t, 0], sc * (S[t] @ dO[0, t, 0]), rtol=1e-12, atol=1e-12)
    assert np.all(gr["dv"] == 0) and np.all(gr["dbeta"] == 0)
    term = [np.sum(S[t] * np.outer(qh[t], dO[0, t, 0]), axis=1) for t in range(T)]
    fin = np.sum(S[-1] * dST[0, 0], axis=1)
    for t in range(T):
        dgam = sum(term[t:]) + fin
        sg = 1 / (1 + np.exp(-x[t]))
        np.testing.assert_allclose(gr["dg"][0, t, 0], dgam * lb * sg * (1 - sg) * np.exp(a_log[0]),
                                   rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("ejk", [False, True])
def test_first_token_closed_form(ejk):
    """One token from a zero state: o = beta (kh . qh) v, S = beta kh v^T."""
    r = RNG(12 + ejk)
    dk, dv = 5, 3
    q, k, v = r.normal(size=(1, 1, 1, dk)), r.normal(size=(1, 1, 1, dk)), r.normal(size=(1, 1, 1, dv))
    g = -0.2 * np.ones((1, 1, 1)) if ejk else r.normal(size=(1, 1, 1, dk))
    bl = r.normal(size=(1, 1, 1))
    beta = 1 / (1 + np.exp(-bl)) if ejk else bl
    dO = r.normal(size=(1, 1, 1, dv))
    gr = kda_oracle.backward(q, k, v, g, beta, np.zeros(1), None, None, d_o=dO, scale=1.0, ejk=ejk,
                             use_qk_l2norm=False)
    b = float(beta.ravel()[0]) if ejk else 1 / (1 + np.exp(-float(bl.ravel()[0])))
    kq = float(k.ravel() @ q.ravel())
    np.testing.assert_allclose(gr["dv"].ravel(), b * kq * dO.ravel(), rtol=1e-12)
    db = kq * float(v.ravel() @ dO.ravel())
    want = db if ejk else db * b * (1 - b)
    np.testing.assert_allclose(gr["dbeta"].ravel(), [want], rtol=1e-12)
    np.testing.assert_allclose(gr["dq"].ravel(), b * k.ravel() * float(v.ravel() @ dO.ravel()), rtol=1e-12)
    # the decay acts on the zero state only: no gradient
    assert np.all(gr["dg"] == 0)


def test_gradients_are_linear_in_the_output_gradients():
    x, kw, W_o, W_s = _case(False, seed=21, lengths=(5, 2))
    r = RNG(22)
    W_o2, W_s2 = r.normal(size=W_o.shape), r.normal(size=W_s.shape)
    g1, g2 = _grads(x, kw, W_o, W_s), _grads(x, kw, W_o2, W_s2)
    g12 = _grads(x, kw, W_o + 2 * W_o2, W_s + 2 * W_s2)
    for name in g1:
        np.testing.assert_allclose(g12[name], g1[name] + 2 * g2[name], rtol=1e-10, atol=1e-12)
