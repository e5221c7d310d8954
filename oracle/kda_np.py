"""NumPy float64 twin of the C oracle, written independently of it.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It is
the same plain definition as ``kda_oracle.c`` - prologue of the kda_tkg page
(AWS Neuron "KDA TKG Kernel API Reference", parameters q, k, g, beta, scale,
lower_bound), KDA step "decay, delta update against the decayed state,
output from the updated state", and the ejkernel ordering of
"kernel_delta_attention" ("The core recurrence") as the EJK variant - but
written as whole-vector NumPy operations looping over tokens only, so that a
slip in one of the two implementations shows up as a disagreement.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def normalise(x, use_l2norm, mult, eps=EPS):
    """x [..., d] -> mult * x / ||x|| (row-wise), or mult * x without the norm."""
    x = np.asarray(x, dtype=np.float64)
    if use_l2norm:
        return mult * x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    return mult * x


def gate(g, a_log, dt_bias, lower_bound):
    """g [..., H, dk], a_log [H], dt_bias [dk, H] -> gamma [..., H, dk]."""
    ea = np.exp(np.asarray(a_log, dtype=np.float64))[:, None]          # [H, 1]
    db = 0.0 if dt_bias is None else np.asarray(dt_bias, np.float64).T  # [H, dk]
    return lower_bound * sigmoid(ea * (np.asarray(g, np.float64) + db))


def step(S, qh, kh, v, gamma_or_d, beta, ejk):
    """Vectorised over a leading batch of heads: S [n, dk, dv], qh/kh [n, dk],
    v [n, dv], gamma [n, dk] (KDA) or d [n] (EJK), beta [n]."""
    if not ejk:
        S = np.exp(gamma_or_d)[:, :, None] * S
        u = np.einsum("nij,ni->nj", S, kh)
        S = S + beta[:, None, None] * kh[:, :, None] * (v - u)[:, None, :]
    else:
        u = np.einsum("nij,ni->nj", S, kh)
        S = np.exp(gamma_or_d)[:, None, None] * S + \
            beta[:, None, None] * kh[:, :, None] * (v - u)[:, None, :]
    o = np.einsum("nij,ni->nj", S, qh)
    return S, o


def prefill(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None, cu_seqlens=None,
            scale=None, lower_bound=-5.0, use_qk_l2norm=True, ejk=False, eps=EPS):
    """q [B, T, H, dk]; k [B, T, Hkv, dk], v [B, T, Hkv, dv]: query head h
    uses key/value head h // (H // Hkv) (ejkernel "recurrent", num_kv_heads)."""
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    grp = H // np.shape(k)[2]
    k = np.repeat(np.asarray(k, np.float64), grp, axis=2)
    v = np.repeat(np.asarray(v, np.float64), grp, axis=2)
    dv = v.shape[-1]
    if scale is None or not (scale > 0):
        scale = 1.0 / np.sqrt(dk)
    if a_log is None:
        a_log = np.zeros(H)
    a_log = np.reshape(np.asarray(a_log, np.float64), (H,))
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        assert B == 1
        cu = np.asarray(cu_seqlens, np.int64)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(cu.shape[0] - 1)]
    o = np.zeros((B, T, H, dv))
    fs = np.zeros((len(seqs), H, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        S = np.zeros((H, dk, dv)) if initial_state is None else \
            np.array(initial_state[n], dtype=np.float64)
        for t in range(t0, t1):
            qh = normalise(q[b, t], use_qk_l2norm, scale, eps)
            kh = normalise(k[b, t], use_qk_l2norm, 1.0, eps)
            if not ejk:
                gd = gate(g[b, t], a_log, dt_bias, lower_bound)
                bt = sigmoid(np.asarray(beta[b, t], np.float64))
            else:
                gd = np.zeros(H) if g is None else np.asarray(g[b, t], np.float64)
                bt = np.asarray(beta[b, t], np.float64)
            S, o[b, t] = step(S, qh, kh, v[b, t], gd, bt, ejk)
        fs[n] = S
    return o, fs


def decode(q, k, g, v, beta, a_log, dt_bias, S, scale=None, lower_bound=-5.0,
           use_qk_l2norm=True, ejk=False, eps=EPS):
    """kda_tkg layouts: q, g [B, dk, H]; k [B, dk, Hkv]; v [B, Hkv, dv];
    beta [B, 1, H]."""
    q = np.swapaxes(np.asarray(q, np.float64), 1, 2)   # [B, H, dk]
    B, H, dk = q.shape
    grp = H // np.shape(k)[2]
    k = np.repeat(np.swapaxes(np.asarray(k, np.float64), 1, 2), grp, axis=1)
    v = np.repeat(np.asarray(v, np.float64), grp, axis=1)
    if scale is None or not (scale > 0):
        scale = 1.0 / np.sqrt(dk)
    a_log = np.reshape(np.asarray(a_log, np.float64), (H,))
    beta = np.reshape(np.asarray(beta, np.float64), (B, H))
    S = np.array(S, dtype=np.float64)
    out = np.zeros((B, H, np.shape(v)[-1]))
    for b in range(B):
        qh = normalise(q[b], use_qk_l2norm, scale, eps)
        kh = normalise(k[b], use_qk_l2norm, 1.0, eps)
        if not ejk:
            gd = gate(np.swapaxes(np.asarray(g, np.float64), 1, 2)[b], a_log, dt_bias, lower_bound)
            bt = sigmoid(beta[b])
        else:
            gd = np.zeros(H) if g is None else np.reshape(np.asarray(g, np.float64), (B, H))[b]
            bt = beta[b]
        S[b], out[b] = step(S[b], qh, kh, np.asarray(v[b], np.float64), gd, bt, ejk)
    return out, S
