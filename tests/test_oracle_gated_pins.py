"""Pins of the gated recurrent attention oracle (oracle.kda_oracle.gated_recurrent),
on the CPU, against computations that share nothing with its token loop:
- no gates and a zero state: causal linear attention, o = scale * (lower(Q K^T)) V;
- all gates and an initial state: the parallel form, each token's k v^T and
  the initial state decayed by the sum of the log-gates of the steps after it;
- reverse = the forward operator on each sequence read backwards;
- packed sequences = separate runs; grouped heads = heads repeated."""
import numpy as np
import pytest

from oracle import kda_oracle

RNG = np.random.default_rng


def _inputs(seed, B=2, T=9, H=2, hkv=2, dk=5, dv=3):
    r = RNG(seed)
    return dict(q=r.normal(size=(B, T, H, dk)), k=r.normal(size=(B, T, hkv, dk)),
                v=r.normal(size=(B, T, hkv, dv)), g=0.3 * r.normal(size=(B, T, H, dk)),
                g_gamma=-0.2 * np.abs(r.normal(size=(B, H))), gk=-0.5 * np.abs(r.normal(size=(B, T, H, dk))),
                gv=-0.5 * np.abs(r.normal(size=(B, T, H, dv))), initial_state=r.normal(size=(B, H, dk, dv)))


def test_no_gates_is_causal_linear_attention():
    x = _inputs(1)
    o, s = kda_oracle.gated_recurrent(x["q"], x["k"], x["v"], scale=0.7)
    B, T, H, dk = x["q"].shape
    for b in range(B):
        for h in range(H):
            A = np.tril(x["q"][b, :, h] @ x["k"][b, :, h].T)
            np.testing.assert_allclose(o[b, :, h], 0.7 * A @ x["v"][b, :, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(s[b, h], x["k"][b, :, h].T @ x["v"][b, :, h], rtol=1e-12, atol=1e-12)


def test_all_gates_match_the_parallel_form():
    x = _inputs(2)
    sc = 0.45
    o, s = kda_oracle.gated_recurrent(x["q"], x["k"], x["v"], x["g"], x["g_gamma"], x["gk"], x["gv"],
                                      x["initial_state"], scale=sc)
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    for b in range(B):
        for h in range(H):
            # L[t, i, j] = sum_{u <= t} (gk_ui + gv_uj + gamma): log-decay of steps 1..t
            L = np.cumsum(x["gk"][b, :, h][:, :, None] + x["gv"][b, :, h][:, None, :] + x["g_gamma"][b, h], 0)
            qt = sc * np.exp(x["g"][b, :, h]) * x["q"][b, :, h]
            for t in range(T):
                st = x["initial_state"][b, h] * np.exp(L[t])
                for s_ in range(t + 1):
                    st = st + np.outer(x["k"][b, s_, h], x["v"][b, s_, h]) * np.exp(L[t] - L[s_])
                np.testing.assert_allclose(o[b, t, h], qt[t] @ st, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(s[b, h], st, rtol=1e-11, atol=1e-12)


def test_reverse_is_the_forward_operator_on_reversed_sequences():
    x = _inputs(3, B=1, T=11)
    cu = np.array([0, 4, 4, 11])
    args = [x[n] for n in ("g", "g_gamma", "gk", "gv")]
    s0 = RNG(4).normal(size=(3, 2, 5, 3))
    o, s = kda_oracle.gated_recurrent(x["q"], x["k"], x["v"], *args, s0, cu, scale=0.3, reverse=True)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        f = lambda t: None if t is None else t[:, a:b][:, ::-1]
        on, sn = kda_oracle.gated_recurrent(f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), x["g_gamma"],
                                            f(x["gk"]), f(x["gv"]), s0[n:n + 1], scale=0.3)
        np.testing.assert_allclose(o[:, a:b], on[:, ::-1], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(s[n], sn[0], rtol=1e-12, atol=1e-13)


def test_packed_equals_separate_and_grouped_equals_repeated():
    x = _inputs(5, B=1, T=12, H=4, hkv=2)
    cu = np.array([0, 5, 12])
    args = [x[n] for n in ("g", "g_gamma", "gk", "gv")]
    s0 = RNG(6).normal(size=(2, 4, 5, 3))
    o, s = kda_oracle.gated_recurrent(x["q"], x["k"], x["v"], *args, s0, cu)
    for n in range(2):
        a, b = cu[n], cu[n + 1]
        cut = lambda t: t[:, a:b]
        on, sn = kda_oracle.gated_recurrent(cut(x["q"]), cut(x["k"]), cut(x["v"]), cut(x["g"]), x["g_gamma"],
                                            cut(x["gk"]), cut(x["gv"]), s0[n:n + 1])
        np.testing.assert_allclose(o[:, a:b], on, rtol=1e-13)
        np.testing.assert_allclose(s[n], sn[0], rtol=1e-13)
    rep = lambda t: np.repeat(t, 2, axis=2)
    oe, se = kda_oracle.gated_recurrent(x["q"], rep(x["k"]), rep(x["v"]), *args, s0, cu)
    np.testing.assert_array_equal(o, oe)
    np.testing.assert_array_equal(s, se)
