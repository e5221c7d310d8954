"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here runs on the CPU.  The oracle (C, float64) and its NumPy twin
are compared with values that do not come from either of them: a worked
example done by hand, closed forms of special cases, invariants of the
recurrence and brute-force Kronecker products.  A plausible slip in the oracle
(dropped decay, decay applied after the residual, S k instead of S^T k,
sigmoid sign, dt_bias transposed, a_log not exponentiated, beta not
activated, wrong varlen offset) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

from oracle import kda_np, kda_oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
LN2, LN3 = np.log(2.0), np.log(3.0)
IMPLS = [kda_oracle, kda_np]


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


@pytest.fixture(scope="module", autouse=True)
def _build():
    kda_oracle.build(force=False)


# ---------------------------------------------------------------- golden ---
@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_hand_example_kda(impl):
    d = json.load(open(os.path.join(GOLD, "kda_hand_example.json")))
    q = np.array(d["q"], float).reshape(1, 2, 1, 2)
    k = np.array(d["k"], float).reshape(1, 2, 1, 2)
    v = np.array(d["v"], float).reshape(1, 2, 1, 2)
    g = (np.array(d["g_kda_over_ln3"], float) * LN3).reshape(1, 2, 1, 2)
    beta = (np.array(d["beta_logit_over_ln3"], float) * LN3).reshape(1, 2, 1)
    s0 = np.array(d["S0"], float).reshape(1, 1, 2, 2)
    o, s = impl.prefill(q, k, v, g, beta, a_log=np.zeros(1), dt_bias=np.zeros((2, 1)),
                        initial_state=s0, scale=1.0, lower_bound=-4 * LN2, use_qk_l2norm=False)
    np.testing.assert_allclose(o.reshape(2, 2), d["kda_o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(s.reshape(2, 2), d["kda_S"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_hand_example_ejk(impl):
    d = json.load(open(os.path.join(GOLD, "kda_hand_example.json")))
    q = np.array(d["q"], float).reshape(1, 2, 1, 2)
    k = np.array(d["k"], float).reshape(1, 2, 1, 2)
    v = np.array(d["v"], float).reshape(1, 2, 1, 2)
    dd = (np.array(d["ejk_d_over_ln2"], float) * LN2).reshape(1, 2, 1)
    beta = np.array(d["ejk_beta"], float).reshape(1, 2, 1)
    s0 = np.array(d["S0"], float).reshape(1, 1, 2, 2)
    o, s = impl.prefill(q, k, v, dd, beta, initial_state=s0, scale=1.0,
                        use_qk_l2norm=False, ejk=True)
    np.testing.assert_allclose(o.reshape(2, 2), d["ejk_o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(s.reshape(2, 2), d["ejk_S"], rtol=0, atol=1e-14)


def test_page_example_shapes():
    d = json.load(open(os.path.join(GOLD, "ejkernel_example_shapes.json")))
    B, T, H, D = d["batch"], d["seq_len"], d["num_heads"], d["head_dim"]
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    dec = rng.standard_normal((B, T, H)) * d["decay_scale"]
    o, s = kda_oracle.prefill(q, k, v, dec, beta, ejk=True)
    assert list(o.shape) == d["output_shape"]
    assert list(s.shape) == d["state_shape"]
    assert np.all(np.isfinite(o))


# --------------------------------------------------------- closed forms ---
def _unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_gate_closed_forms_pure_decay(impl):
    """beta logit = -inf gives beta = 0 exactly: the state only decays, per key
    channel, by exp(lb * sigma) with sigma in {1/4, 1/2, 3/4} built from
    a_log, dt_bias[i, h] and g so that each factor is checked."""
    H, dk, dv, T = 2, 3, 4, 3
    lb = -1.7
    a_log = np.array([0.0, LN2])           # head 1: exp(a_log) = 2
    # target pre-activation x[h, i] (after the exp(a_log) multiply)
    x = np.array([[0.0, LN3, -LN3], [LN3, 0.0, -LN3]])
    sig = np.array([[0.5, 0.75, 0.25], [0.75, 0.5, 0.25]])
    dt_bias = np.array([[0.3, -0.2], [0.1, 0.4], [-0.5, 0.25]])    # [dk, H], asymmetric
    g = np.zeros((1, T, H, dk))
    for h in range(H):
        g[0, :, h, :] = x[h] / np.exp(a_log[h]) - dt_bias[:, h]
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, T, H, dk))
    k = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    s0 = rng.standard_normal((1, H, dk, dv))
    beta = np.full((1, T, H), -np.inf)
    o, s = impl.prefill(q, k, v, g, beta, a_log=a_log, dt_bias=dt_bias, initial_state=s0,
                        scale=0.5, lower_bound=lb)
    for h in range(H):
        for t in range(T):
            St = np.exp((t + 1) * lb * sig[h])[:, None] * s0[0, h]
            qh = 0.5 * q[0, t, h] / np.sqrt(np.sum(q[0, t, h] ** 2) + kda_oracle.EPS)
            np.testing.assert_allclose(o[0, t, h], St.T @ qh, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(s[0, h], np.exp(T * lb * sig[h])[:, None] * s0[0, h],
                                   rtol=1e-13, atol=0)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_zero_params_gives_half_lower_bound(impl):
    """a_log = dt_bias = g = 0: gamma = lb / 2 on every channel; lb = 0: no decay."""
    rng = np.random.default_rng(2)
    H, dk, dv, T = 3, 4, 2, 5
    s0 = rng.standard_normal((1, H, dk, dv))
    args = [rng.standard_normal((1, T, H, dk)), rng.standard_normal((1, T, H, dk)),
            rng.standard_normal((1, T, H, dv)), np.zeros((1, T, H, dk)),
            np.full((1, T, H), -np.inf)]
    for lb in (-3.0, 0.0):
        _, s = impl.prefill(*args, a_log=np.zeros(H), dt_bias=np.zeros((dk, H)),
                            initial_state=s0, lower_bound=lb)
        np.testing.assert_allclose(s, np.exp(T * lb / 2) * s0, rtol=1e-14, atol=0)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
@pytest.mark.parametrize("ejk", [False, True])
def test_first_token_from_zero_state(impl, ejk):
    """S1 = beta k^ v^T and o1 = beta (k^ . q^) v; dk != dv pins the orientation."""
    dk, dv = 3, 5
    q = np.array([3.0, 0.0, 4.0])      # ||q|| = 5
    k = np.array([0.0, 6.0, 8.0])      # ||k|| = 10
    v = np.array([1.0, -2.0, 0.5, 3.0, -1.0])
    scale = 0.7
    qh = scale * q / np.sqrt(25.0 + kda_oracle.EPS)
    kh = k / np.sqrt(100.0 + kda_oracle.EPS)
    if ejk:
        g, beta, b = np.array([[[-0.3]]]), np.array([[[0.75]]]), 0.75
    else:
        g, beta, b = np.array([[[[0.2, -1.0, 3.0]]]]), np.array([[[LN3]]]), 0.75
    o, s = impl.prefill(q.reshape(1, 1, 1, dk), k.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv),
                        g, beta, a_log=np.zeros(1), dt_bias=np.zeros((dk, 1)), scale=scale,
                        ejk=ejk)
    np.testing.assert_allclose(s[0, 0], b * np.outer(kh, v), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], b * (kh @ qh) * v, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_delta_rule_recall_kda(impl):
    """KDA, beta = 1, q = k, scale = 1, any gates: S_t^T k^_t = v_t after every
    step, so o_t = v_t.  Fails if the residual is taken before the decay."""
    rng = np.random.default_rng(3)
    T, H, dk, dv = 7, 2, 6, 5
    # large-norm keys: the L2-norm epsilon then moves ||k^|| by < 1e-12
    k = 1e4 * rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    g = rng.standard_normal((1, T, H, dk))
    s0 = rng.standard_normal((1, H, dk, dv))
    o, _ = impl.prefill(k, k, v, g, np.full((1, T, H), np.inf), a_log=rng.uniform(-1, 1, H),
                        dt_bias=0.3 * rng.standard_normal((dk, H)), initial_state=s0, scale=1.0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_delta_rule_recall_ejk_differs_by_decay(impl):
    """EJK with beta = 1, q = k, scale = 1: S_t^T k^ = v_t + (e^d - 1) S_{t-1}^T k^,
    so o_t = v_t only when d = 0.  Separates the two orderings."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 4, 1, 4, 3
    k = 1e4 * rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    d = -np.abs(rng.standard_normal((1, T, H)))
    s0 = rng.standard_normal((1, H, dk, dv))
    beta = np.ones((1, T, H))
    o, _ = impl.prefill(k, k, v, d, beta, initial_state=s0, scale=1.0, ejk=True)
    for t in range(T):
        if t == 0:
            sp = s0[0, 0]
        else:
            _, sp = impl.prefill(k[:, :t], k[:, :t], v[:, :t], d[:, :t], beta[:, :t],
                                 initial_state=s0, scale=1.0, ejk=True)
            sp = sp[0, 0]
        kh = k[0, t, 0] / np.sqrt(np.sum(k[0, t, 0] ** 2) + kda_oracle.EPS)
        expect = v[0, t, 0] + (np.exp(d[0, t, 0]) - 1.0) * (sp.T @ kh)
        np.testing.assert_allclose(o[0, t, 0], expect, rtol=1e-12, atol=1e-12)
        assert np.linalg.norm(o[0, t, 0] - v[0, t, 0]) > 1e-3


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_orthonormal_keys_store_every_value(impl):
    """No decay (lb = 0), beta = 1, orthonormal keys: after n tokens the state
    returns every stored value, S^T k_s = v_s for all s."""
    rng = np.random.default_rng(5)
    dk, dv, n = 8, 3, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:n]
    big = 1e4 * keys                   # normalised back to the orthonormal rows
    v = rng.standard_normal((1, n, 1, dv))
    q = rng.standard_normal((1, n, 1, dk))
    _, s = impl.prefill(q, big.reshape(1, n, 1, dk), v, rng.standard_normal((1, n, 1, dk)),
                        np.full((1, n, 1), np.inf), a_log=np.zeros(1), lower_bound=0.0)
    np.testing.assert_allclose(keys @ s[0, 0], v[0, :, 0], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ invariants ---
@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
@pytest.mark.parametrize("ejk", [False, True])
def test_non_expansion(impl, ejk):
    """v = 0, gates <= 0, beta in [0, 1], unit keys: ||S_t||_F never grows."""
    rng = np.random.default_rng(6)
    T, dk, dv = 12, 5, 4
    k = rng.standard_normal((1, T, 1, dk))
    q = rng.standard_normal((1, T, 1, dk))
    v = np.zeros((1, T, 1, dv))
    s0 = rng.standard_normal((1, 1, dk, dv))
    if ejk:
        g, beta = -np.abs(rng.standard_normal((1, T, 1))), rng.uniform(0, 1, (1, T, 1))
    else:
        g, beta = rng.standard_normal((1, T, 1, dk)), rng.standard_normal((1, T, 1))
    norms = [np.linalg.norm(s0)]
    for t in range(1, T + 1):
        _, s = impl.prefill(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t],
                            a_log=np.zeros(1), dt_bias=np.zeros((dk, 1)), initial_state=s0,
                            ejk=ejk)
        norms.append(np.linalg.norm(s))
    assert all(b <= a * (1 + 1e-14) for a, b in zip(norms, norms[1:]))
    assert norms[-1] < norms[0]


@pytest.mark.parametrize("ejk", [False, True])
def test_linearity_in_values_and_state(ejk):
    rng = np.random.default_rng(7)
    T, H, dk, dv = 9, 2, 4, 3
    q, k = rng.standard_normal((1, T, H, dk)), rng.standard_normal((1, T, H, dk))
    g = -np.abs(rng.standard_normal((1, T, H))) if ejk else rng.standard_normal((1, T, H, dk))
    beta = rng.uniform(0, 1, (1, T, H)) if ejk else rng.standard_normal((1, T, H))
    v1, v2 = rng.standard_normal((2, 1, T, H, dv))
    s1, s2 = rng.standard_normal((2, 1, H, dk, dv))
    kw = dict(a_log=rng.uniform(-1, 1, H), dt_bias=0.1 * rng.standard_normal((dk, H)), ejk=ejk)
    oa, sa = kda_oracle.prefill(q, k, v1 + 2 * v2, g, beta, initial_state=s1 + 2 * s2, **kw)
    o1, f1 = kda_oracle.prefill(q, k, v1, g, beta, initial_state=s1, **kw)
    o2, f2 = kda_oracle.prefill(q, k, v2, g, beta, initial_state=s2, **kw)
    np.testing.assert_allclose(oa, o1 + 2 * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sa, f1 + 2 * f2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ejk", [False, True])
def test_brute_force_kronecker(ejk):
    """vec(S_t) = (I_dv kron M_t) vec(S_{t-1}) + beta_t (v_t kron k_t), with
    M_t = (I - beta k k^T) Diag(exp gamma) (KDA) or exp(d) I - beta k k^T (EJK),
    o_t = (I_dv kron q_t^T) vec(S_t).  Prologue made trivial (no L2 norm,
    scale 1, exact sigmoid values) so this pins the step itself."""
    rng = np.random.default_rng(8 + ejk)
    T, dk, dv = 5, 3, 4
    lb = -2.0
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk)) * 0.5
    v = rng.standard_normal((1, T, 1, dv))
    s0 = rng.standard_normal((1, 1, dk, dv))
    choice = rng.integers(0, 3, size=(T, dk))
    xs, sg = np.array([0.0, LN3, -LN3]), np.array([0.5, 0.75, 0.25])
    bchoice = rng.integers(0, 3, size=T)
    if ejk:
        g = -np.abs(rng.standard_normal((1, T, 1)))
        beta = sg[bchoice].reshape(1, T, 1)
    else:
        g = xs[choice].reshape(1, T, 1, dk)
        beta = xs[bchoice].reshape(1, T, 1)
    o, s = kda_oracle.prefill(q, k, v, g, beta, a_log=np.zeros(1), dt_bias=np.zeros((dk, 1)),
                              initial_state=s0, scale=1.0, lower_bound=lb,
                              use_qk_l2norm=False, ejk=ejk)
    vec = s0[0, 0].reshape(-1, order="F")
    for t in range(T):
        kt, qt, bt = k[0, t, 0], q[0, t, 0], sg[bchoice[t]]
        if ejk:
            M = np.exp(g[0, t, 0]) * np.eye(dk) - bt * np.outer(kt, kt)
        else:
            M = (np.eye(dk) - bt * np.outer(kt, kt)) @ np.diag(np.exp(lb * sg[choice[t]]))
        vec = np.kron(np.eye(dv), M) @ vec + bt * np.kron(v[0, t, 0], kt)
        ot = np.kron(np.eye(dv), qt.reshape(1, -1)) @ vec
        np.testing.assert_allclose(o[0, t, 0], ot, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s[0, 0], vec.reshape(dk, dv, order="F"), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------- plumbing pins -------
def _rand_case(seed, B=2, T=11, H=3, dk=4, dv=5, ejk=False):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    if ejk:
        g, beta = -np.abs(rng.standard_normal((B, T, H))), rng.uniform(0, 1, (B, T, H))
    else:
        g, beta = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H))
    kw = dict(a_log=rng.uniform(-1, 1, H), dt_bias=0.1 * rng.standard_normal((dk, H)),
              initial_state=0.1 * rng.standard_normal((B, H, dk, dv)), ejk=ejk)
    return (q, k, v, g, beta), kw


@pytest.mark.parametrize("ejk", [False, True])
@pytest.mark.parametrize("l2", [True, False])
def test_twin_agreement(ejk, l2):
    args, kw = _rand_case(10 + ejk, ejk=ejk)
    oc, sc = kda_oracle.prefill(*args, use_qk_l2norm=l2, scale=0.3, **kw)
    on, sn = kda_np.prefill(*args, use_qk_l2norm=l2, scale=0.3, **kw)
    assert _rel(oc, on) < 1e-12 and _rel(sc, sn) < 1e-12


@pytest.mark.parametrize("ejk", [False, True])
def test_split_and_resume(ejk):
    args, kw = _rand_case(20 + ejk, T=16, ejk=ejk)
    o, s = kda_oracle.prefill(*args, **kw)
    first = [a[:, :7] for a in args]
    second = [a[:, 7:] for a in args]
    o1, s1 = kda_oracle.prefill(*first, **kw)
    kw2 = dict(kw, initial_state=s1)
    o2, s2 = kda_oracle.prefill(*second, **kw2)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, s, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
@pytest.mark.parametrize("ejk", [False, True])
def test_decode_steps_equal_prefill(impl, ejk):
    """T single-token decode calls in kda_tkg layouts == one prefill."""
    args, kw = _rand_case(30 + ejk, B=3, T=6, H=2, dk=4, dv=3, ejk=ejk)
    q, k, v, g, beta = args
    o, s = kda_oracle.prefill(*args, scale=0.4, lower_bound=-3.0, **kw)
    S = kw["initial_state"]
    for t in range(q.shape[1]):
        gd = (g[:, t][:, None, :] if ejk else np.swapaxes(g[:, t], 1, 2))
        out, S = impl.decode(np.swapaxes(q[:, t], 1, 2), np.swapaxes(k[:, t], 1, 2), gd,
                             v[:, t], beta[:, t][:, None, :], kw["a_log"][None, :],
                             kw["dt_bias"], S, scale=0.4, lower_bound=-3.0, ejk=ejk)
        np.testing.assert_allclose(out, o[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, s, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
def test_varlen_equals_separate_runs(impl):
    rng = np.random.default_rng(40)
    H, dk, dv = 2, 4, 3
    lens = [5, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(cu[-1])
    q, k = rng.standard_normal((1, N, H, dk)), rng.standard_normal((1, N, H, dk))
    v, g = rng.standard_normal((1, N, H, dv)), rng.standard_normal((1, N, H, dk))
    beta = rng.standard_normal((1, N, H))
    a_log, dtb = rng.uniform(-1, 1, H), 0.1 * rng.standard_normal((dk, H))
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    o, s = impl.prefill(q, k, v, g, beta, a_log=a_log, dt_bias=dtb, initial_state=s0,
                        cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if a == b:
            np.testing.assert_array_equal(s[n], s0[n])
            continue
        on, sn = kda_oracle.prefill(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                                    a_log=a_log, dt_bias=dtb, initial_state=s0[n:n + 1])
        np.testing.assert_allclose(o[:, a:b], on, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(s[n], sn[0], rtol=1e-13, atol=1e-14)


def test_head_permutation_equivariance():
    args, kw = _rand_case(50, H=4)
    perm = np.array([2, 0, 3, 1])
    o, s = kda_oracle.prefill(*args, **kw)
    pa = [a[:, :, perm] for a in args]
    pkw = dict(kw, a_log=kw["a_log"][perm], dt_bias=kw["dt_bias"][:, perm],
               initial_state=kw["initial_state"][:, perm])
    op, sp = kda_oracle.prefill(*pa, **pkw)
    np.testing.assert_allclose(op, o[:, :, perm], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sp, s[:, perm], rtol=1e-14, atol=1e-15)


def test_unit_subset_matches_full_run():
    args, kw = _rand_case(60, B=2, H=3)
    o, s = kda_oracle.prefill(*args, **kw)
    units = [4, 1]
    os_, ss = kda_oracle.prefill(*args, units=units, **kw)
    for u in units:
        n, h = divmod(u, 3)
        np.testing.assert_array_equal(os_[n, :, h], o[n, :, h])
        np.testing.assert_array_equal(ss[n, h], s[n, h])


def test_default_scale_is_inverse_sqrt_dk():
    args, kw = _rand_case(70, dk=16)
    o1, _ = kda_oracle.prefill(*args, scale=None, **kw)
    o2, _ = kda_oracle.prefill(*args, scale=0.25, **kw)
    np.testing.assert_array_equal(o1, o2)


def test_zero_vector_normalises_to_zero():
    """An all-zero key contributes nothing (no NaN): S1 = 0 from a zero state."""
    q = np.ones((1, 1, 1, 4))
    k = np.zeros((1, 1, 1, 4))
    v = np.ones((1, 1, 1, 2))
    o, s = kda_oracle.prefill(q, k, v, np.zeros((1, 1, 1, 4)), np.zeros((1, 1, 1)),
                              a_log=np.zeros(1))
    assert np.all(s == 0) and np.all(o == 0)


# --------------------------------------------------------- grouped heads ---
# ejkernel "recurrent" run(): query, gates and state carry num_heads, key and
# value num_kv_heads.  Reading taken: consecutive heads share a key/value head
# (head h reads head h // (H // Hkv)).  A grouped run must equal the ungrouped
# run on keys and values repeated that way, exactly: the grouping is indexing.
@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
@pytest.mark.parametrize("ejk", [False, True])
def test_grouped_heads_equal_repeated_kv(impl, ejk):
    args, kw = _rand_case(80 + ejk, B=2, T=9, H=6, dk=5, dv=4, ejk=ejk)
    q, k, v, g, beta = args
    grp = 3                                   # Hkv = 2
    kg, vg = k[:, :, ::grp].copy(), v[:, :, ::grp].copy()
    o_g, s_g = impl.prefill(q, kg, vg, g, beta, **kw)
    o_r, s_r = kda_oracle.prefill(q, np.repeat(kg, grp, axis=2), np.repeat(vg, grp, axis=2), g, beta, **kw)
    np.testing.assert_allclose(o_g, o_r, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(s_g, s_r, rtol=1e-14, atol=1e-15)
    # and it is not the interleaved grouping (head h reading h % Hkv)
    o_i, _ = kda_oracle.prefill(q, np.tile(kg, (1, 1, grp, 1)), np.tile(vg, (1, 1, grp, 1)), g, beta, **kw)
    assert _rel(o_g, o_i) > 1e-3


@pytest.mark.parametrize("impl", IMPLS, ids=["c", "numpy"])
@pytest.mark.parametrize("ejk", [False, True])
def test_grouped_decode_equals_repeated_kv(impl, ejk):
    rng = np.random.default_rng(90 + ejk)
    B, H, Hkv, dk, dv = 3, 4, 2, 5, 3
    q, g = rng.standard_normal((B, dk, H)), rng.standard_normal((B, dk, H))
    k, v = rng.standard_normal((B, dk, Hkv)), rng.standard_normal((B, Hkv, dv))
    beta = rng.standard_normal((B, 1, H))
    if ejk:
        g = -0.1 * np.abs(rng.standard_normal((B, 1, H)))
        beta = 1.0 / (1.0 + np.exp(-beta))
    a_log, dtb = rng.uniform(-1, 1, (1, H)), 0.1 * rng.standard_normal((dk, H))
    S = rng.standard_normal((B, H, dk, dv))
    o_g, s_g = impl.decode(q, k, g, v, beta, a_log, dtb, S, ejk=ejk)
    o_r, s_r = kda_oracle.decode(q, np.repeat(k, 2, axis=2), g, np.repeat(v, 2, axis=1), beta, a_log, dtb, S,
                                 ejk=ejk)
    np.testing.assert_allclose(o_g, o_r, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(s_g, s_r, rtol=1e-14, atol=1e-15)
