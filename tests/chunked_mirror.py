"""Float64 NumPy mirror of the chunk-parallel algebra used by the MFMA prefill
kernel (test helper; it is not the oracle and the oracle does not use it).

Within a chunk of C = 64 tokens, with b_r = sum_{s<=r} gamma_s (per key
channel, restarting at the chunk start) and the state S0 entering the chunk,
the token recurrence (decay, residual against the decayed state, update)
is exactly
    A_rs = beta_r sum_i kh_ri kh_si e^{b_ri - b_si}      (s < r)
    P_rs = sum_i qh_ri kh_si e^{b_ri - b_si}             (s <= r)
    T    = (I + A)^{-1}
    W    = T diag(beta) Kg,   Kg_r = e^{b_r} * kh_r
    U~   = T diag(beta) V
    U    = U~ - W S0
    O    = Qg S0 + P U,       Qg_r = e^{b_r} * qh_r
    S    = Diag(e^{b_C}) S0 + Kc^T U,   Kc_s = e^{b_C - b_s} * kh_s
The mirror evaluates A and P the way the kernel does, on 16-row sub-blocks
with reference rows chosen so that no factor overflows, and inverts I + A by
16x16 diagonal inverses merged 16 -> 32 -> 64.

EJK variant (scalar per-head decay d_t, beta as given, residual against the
undecayed state): with b_r = sum_{s<=r} d_s, the residual of row r sees the
state decayed only up to row r-1, so
    A_rs = beta_r e^{b_{r-1} - b_s} kh_r . kh_s           (s < r, b_{-1} = 0)
    Kg_r = e^{b_{r-1}} kh_r
and P, Qg, Kc and the carry are as above with the scalar b.  With d <= 0
every factor is at most 1, so the kernel scales the plain Gram products
instead of factorising.
"""
from __future__ import annotations

import numpy as np

C, BLK = 64, 16


def _prologue(q, k, g, beta, a_log_h, dtb_h, scale, lb, l2norm, eps=1e-6):
    if l2norm:
        qh = scale * q / np.sqrt(np.sum(q * q, -1, keepdims=True) + eps)
        kh = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + eps)
    else:
        qh, kh = scale * q, k
    gam = lb / (1.0 + np.exp(-np.exp(a_log_h) * (g + dtb_h)))
    bt = 1.0 / (1.0 + np.exp(-beta))
    return qh, kh, gam, bt


def _blocked_unit_lower_inverse(A):
    """(I + A)^{-1} for strictly lower A (64 x 64): diagonal 16x16 blocks by
    forward substitution, then T10 = -T11 A10 T00 (and T32), then the 32x32
    lower-left block -T_B A_low T_A."""
    n = A.shape[0]
    T = np.zeros_like(A)
    for I in range(n // BLK):
        sl = slice(BLK * I, BLK * (I + 1))
        a = A[sl, sl]
        t = np.zeros((BLK, BLK))
        for j in range(BLK):
            t[j, j] = 1.0
            for r in range(j + 1, BLK):
                t[r, j] = -a[r, j:r] @ t[j:r, j]
        T[sl, sl] = t
    for I in (1, 3):
        r, c = slice(BLK * I, BLK * (I + 1)), slice(BLK * (I - 1), BLK * I)
        T[r, c] = -T[r, r] @ (A[r, c] @ T[c, c])
    lo, hi = slice(0, 32), slice(32, 64)
    T[hi, lo] = -T[hi, hi] @ (A[hi, lo] @ T[lo, lo])
    return T


def chunk_step(S0, qh, kh, v, gam, bt):
    """One chunk (rows beyond the sequence padded with qh = kh = v = 0,
    gamma = 0, beta = 0).  Returns (O [C, dv], S_new)."""
    b = np.cumsum(gam, axis=0)                       # [C, dk]
    nb = C // BLK
    first = b[0::BLK]                                 # b at the first row of each block
    last = b[BLK - 1::BLK]                            # b at the last row of each block
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for I in range(nb):
        rI = slice(BLK * I, BLK * (I + 1))
        Lr = np.exp(b[rI] - first[I])                 # <= 1
        for J in range(I + 1):
            sJ = slice(BLK * J, BLK * (J + 1))
            if I == J:
                Rs = np.exp(first[I] - b[sJ])         # >= 1, <= e^{15 |lb|}
            else:
                # e^{b_fI - b_s} = e^{b_fI - b_eJ} * e^{b_eJ - b_s}, both <= 1
                Rs = np.exp(first[I] - last[J]) * np.exp(last[J] - b[sJ])
            A[rI, sJ] = (kh[rI] * Lr) @ (kh[sJ] * Rs).T
            P[rI, sJ] = (qh[rI] * Lr) @ (kh[sJ] * Rs).T
    r_idx = np.arange(C)
    A = np.where(r_idx[:, None] > r_idx[None, :], A, 0.0) * bt[:, None]
    P = np.where(r_idx[:, None] >= r_idx[None, :], P, 0.0)
    T = _blocked_unit_lower_inverse(A)
    Tb = T * bt[None, :]
    Kg = np.exp(b) * kh
    Qg = np.exp(b) * qh
    Kc = np.exp(b[-1] - b) * kh
    W = Tb @ Kg
    U = Tb @ v - W @ S0
    O = Qg @ S0 + P @ U
    S = np.exp(b[-1])[:, None] * S0 + Kc.T @ U
    return O, S


def chunk_step_ejk(S0, qh, kh, v, d, bt):
    """EJK chunk: d [C] scalar log-decays, bt [C] betas as given (padding rows
    d = 0, beta = 0)."""
    b = np.cumsum(d)
    bx = np.concatenate([[0.0], b[:-1]])               # b_{r-1}
    r_idx = np.arange(C)
    lower = r_idx[:, None] > r_idx[None, :]
    A = np.where(lower, np.exp(np.where(lower, bx[:, None] - b[None, :], 0.0)), 0.0)
    A = A * (kh @ kh.T) * bt[:, None]
    lower_eq = r_idx[:, None] >= r_idx[None, :]
    P = np.where(lower_eq, np.exp(np.where(lower_eq, b[:, None] - b[None, :], 0.0)), 0.0)
    P = P * (qh @ kh.T)
    T = _blocked_unit_lower_inverse(A)
    Tb = T * bt[None, :]
    W = Tb @ (np.exp(bx)[:, None] * kh)
    U = Tb @ v - W @ S0
    O = (np.exp(b)[:, None] * qh) @ S0 + P @ U
    S = np.exp(b[-1]) * S0 + (np.exp(b[-1] - b)[:, None] * kh).T @ U
    return O, S


def prefill(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None, cu_seqlens=None,
            scale=None, lower_bound=-5.0, use_qk_l2norm=True, ejk=False):
    """Same arguments and returns as the oracle's prefill (EJK: g [B, T, H]
    log-decays or None, beta used as given)."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g = None if g is None else np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, dv))
    fs = np.zeros((len(seqs), H, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else \
                np.array(initial_state[n, h], np.float64)
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                m = c1 - c0
                pad = lambda x: np.concatenate([x, np.zeros((C - m,) + x.shape[1:])])
                if ejk:
                    qh, kh, _, _ = _prologue(q[b, c0:c1, h], k[b, c0:c1, h], 0.0, 0.0, 0.0, 0.0,
                                             scale, 0.0, use_qk_l2norm)
                    d = np.zeros(m) if g is None else g[b, c0:c1, h]
                    O, S = chunk_step_ejk(S, pad(qh), pad(kh), pad(v[b, c0:c1, h]), pad(d),
                                          pad(beta[b, c0:c1, h]))
                else:
                    qh, kh, gam, bt = _prologue(q[b, c0:c1, h], k[b, c0:c1, h], g[b, c0:c1, h],
                                                beta[b, c0:c1, h], a_log[h], dt_bias[:, h], scale,
                                                lower_bound, use_qk_l2norm)
                    O, S = chunk_step(S, pad(qh), pad(kh), pad(v[b, c0:c1, h]), pad(gam), pad(bt))
                o[b, c0:c1, h] = O[:m]
            fs[n, h] = S
    return o, fs
