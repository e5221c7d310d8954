"""Float64 NumPy mirror of the chunk-level backward algebra used by the HIP
backward kernels (test helper: it is not the oracle, and the oracle does not
use it).  It pins the derivation before and apart from the kernels.

Within a chunk of C = 16 tokens, with b_r = sum_{s<=r} gamma_s (per key
channel for KDA, one scalar per token for EJK, restarting at the chunk
start), b' = b for KDA and b'_r = b_{r-1} (b'_0 = 0) for EJK, and the state
S0 entering the chunk, the forward chunk map is
    GA_rs = sum_i kh_ri kh_si e^{b'_ri - b_si},  A = strict_lower(diag(beta) GA)
    GP_rs = sum_i qh_ri kh_si e^{b_ri - b_si},   P = lower(GP)
    Kg = e^{b'} kh,  Qg = e^{b} qh,  Kc = e^{b_C - b} kh   (b_C: last row)
    Y = V - Kg S0,   (I + A) U = diag(beta) Y
    O = Qg S0 + P U,   S1 = Diag(e^{b_C}) S0 + Kc^T U
and, given dO and dS1 = dL/dS1, its adjoint is
    dU = P^T dO + Kc dS1,   (I + A)^T Z = dU,   dY = diag(beta) Z,   dV = dY
    dS0 = Qg^T dO + Diag(e^{b_C}) dS1 - Kg^T dY
    dA = -strict_lower(Z U^T),   dP = lower(dO U^T),   dbeta_r = Z_r . Y_r + dA_r . GA_r
    dQg = dO S0^T,   dKg = -dY S0^T,   dKc = U dS1^T
then through the Gram products (a row and a column role each) and the
elementwise decay factors into dqh, dkh and db, db' (db' folds into db: same
row for KDA, the row before for EJK), and dgamma = the reverse cumulative sum
of db, plus the carry's e^{b_C} term on every row and the Kc terms summed over
the rows before (pair terms whose two roles fall on the same b are left out
of db: they cancel exactly, and in float32 would leave rounding of the size of
the undecayed terms).  Chunks are chained
by the forward states S0 (forward over chunks) and the state gradients dS1
(backward over chunks).
"""
from __future__ import annotations

import numpy as np

C = 16


def _rows(q, k, g, beta, a_log_h, dtb_h, scale, lb, l2norm, ejk, eps=1e-6):
    """The prologue of every row, with what its backward needs."""
    nq = np.sqrt(np.sum(q * q, -1, keepdims=True) + eps)
    nk = np.sqrt(np.sum(k * k, -1, keepdims=True) + eps)
    qh = scale * q / nq if l2norm else scale * q
    kh = k / nk if l2norm else k
    if ejk:
        gam = np.zeros(q.shape[0]) if g is None else g.copy()
        bt = beta.copy()
        sg = x = None
    else:
        x = np.exp(a_log_h) * (g + dtb_h)
        sg = 1.0 / (1.0 + np.exp(-x))
        gam = lb * sg
        bt = 1.0 / (1.0 + np.exp(-beta))
    return dict(q=q, k=k, qh=qh, kh=kh, nq=nq, nk=nk, gam=gam, bt=bt, sg=sg, x=x)


def _chunk_fwd(R, V, S0, ejk):
    n, dk = R["kh"].shape
    qh, kh, bt = R["qh"], R["kh"], R["bt"]
    b = np.cumsum(R["gam"], axis=0)                        # [n, dk] or [n]
    bp = b.copy() if not ejk else np.concatenate([[0.0], b[:-1]])
    bC = b[-1]
    if ejk:
        DA = np.exp(np.minimum(bp[:, None] - b[None, :], 0.0))[:, :, None] * np.ones(dk)
        DP = np.exp(np.minimum(b[:, None] - b[None, :], 0.0))[:, :, None] * np.ones(dk)
        eb, ebp, eC, ecb = (np.exp(b)[:, None] * np.ones(dk), np.exp(bp)[:, None] * np.ones(dk),
                            np.exp(bC) * np.ones(dk), np.exp(bC - b)[:, None] * np.ones(dk))
    else:
        DA = np.exp(np.minimum(bp[:, None, :] - b[None, :, :], 0.0))
        DP = np.exp(np.minimum(b[:, None, :] - b[None, :, :], 0.0))
        eb, ebp, eC, ecb = np.exp(b), np.exp(bp), np.exp(bC), np.exp(bC - b)
    low = np.tril(np.ones((n, n)), -1)
    lowi = np.tril(np.ones((n, n)))
    GA = np.einsum("ri,si,rsi->rs", kh, kh, DA) * low
    GP = np.einsum("ri,si,rsi->rs", qh, kh, DP) * lowi
    A = bt[:, None] * GA
    Kg, Qg, Kc = ebp * kh, eb * qh, ecb * kh
    Y = V - Kg @ S0
    U = np.linalg.solve(np.eye(n) + A, bt[:, None] * Y)
    O = Qg @ S0 + GP @ U
    S1 = eC[:, None] * S0 + Kc.T @ U
    return dict(b=b, bp=bp, DA=DA, DP=DP, eb=eb, ebp=ebp, eC=eC, ecb=ecb, GA=GA, GP=GP, A=A,
                Kg=Kg, Qg=Qg, Kc=Kc, Y=Y, U=U, O=O, S1=S1)


def _chunk_dS0(F, dO, dS1, bt):
    n = F["A"].shape[0]
    dU = F["GP"].T @ dO + F["Kc"] @ dS1
    Z = np.linalg.solve((np.eye(n) + F["A"]).T, dU)
    dY = bt[:, None] * Z
    return Z, dY, F["Qg"].T @ dO + F["eC"][:, None] * dS1 - F["Kg"].T @ dY


def _chunk_local(R, F, S0, dO, dS1, ejk):
    bt, qh, kh = R["bt"], R["qh"], R["kh"]
    n = kh.shape[0]
    Z, dY, _ = _chunk_dS0(F, dO, dS1, bt)
    U = F["U"]
    dA = -np.tril(Z @ U.T, -1)
    dP = np.tril(dO @ U.T)
    dbt = np.sum(Z * F["Y"], 1) + np.sum(dA * F["GA"], 1)
    dGA = bt[:, None] * dA
    dQg, dKg, dKc = dO @ S0.T, -dY @ S0.T, U @ dS1.T
    # Gram products: row and column roles
    rowA = np.einsum("rs,si,rsi->ri", dGA, kh, F["DA"])
    colA = np.einsum("rs,ri,rsi->si", dGA, kh, F["DA"])
    rowP = np.einsum("rs,si,rsi->ri", dP, kh, F["DP"])
    colP = np.einsum("rs,ri,rsi->si", dP, qh, F["DP"])
    dqh = rowP + F["eb"] * dQg
    dkh = rowA + colA + colP + F["ebp"] * dKg + F["ecb"] * dKc
    # dgamma_u collects, from each pair term of a Gram product, the pairs whose
    # row-role index rho and column-role index kappa straddle it (kappa < u <=
    # rho); pairs with rho == kappa (the diagonal of P; for EJK the first
    # sub-diagonal of A, whose row role sits on b_{r-1}) contribute nothing and
    # are left out, and the Kc terms (kappa = s, rho = the last row) are summed
    # as the prefix over s < u: no large terms that cancel.
    dPd = np.diag(dP)
    rowP_nd = rowP - dPd[:, None] * kh
    colP_nd = colP - dPd[:, None] * qh
    rowA_nd, colA_nd = rowA.copy(), colA.copy()
    if ejk:
        sub = np.diag(dGA, -1)                      # dGA[r, r-1], with DA = 1 there
        rowA_nd[1:] -= sub[:, None] * kh[:-1]
        colA_nd[:-1] -= sub[:, None] * kh[1:]
    db = qh * rowP_nd - kh * colA_nd - kh * colP_nd + F["Qg"] * dQg
    dbp = kh * rowA_nd + F["Kg"] * dKg
    kcd = F["Kc"] * dKc
    dbC = F["eC"] * np.sum(S0 * dS1, 1)
    if ejk:
        db, dbp, kcd, dbC = db.sum(1), dbp.sum(1), kcd.sum(1), dbC.sum()
        db[:-1] += dbp[1:]
    else:
        db = db + dbp
    pre = np.concatenate([np.zeros_like(kcd[:1]), np.cumsum(kcd, axis=0)[:-1]])
    dgam = np.cumsum(db[::-1], axis=0)[::-1] + dbC + pre
    return dict(dqh=dqh, dkh=dkh, dV=dY, dgam=dgam, dbt=dbt)


def _prologue_bwd(R, G, scale, lb, l2norm, ejk, a_log_h):
    q, k, nq, nk = R["q"], R["k"], R["nq"], R["nk"]
    if l2norm:
        dq = scale * (G["dqh"] / nq - q * np.sum(q * G["dqh"], -1, keepdims=True) / nq ** 3)
        dk = G["dkh"] / nk - k * np.sum(k * G["dkh"], -1, keepdims=True) / nk ** 3
    else:
        dq, dk = scale * G["dqh"], G["dkh"]
    if ejk:
        return dq, dk, G["dgam"], G["dbt"], None
    dx = G["dgam"] * lb * R["sg"] * (1 - R["sg"])
    dg = dx * np.exp(a_log_h)
    dl = G["dbt"] * R["bt"] * (1 - R["bt"])
    return dq, dk, dg, dl, dx


def backward(q, k, v, g, beta, a_log, dt_bias, S0, cu, dO, dSf, scale, lb, l2norm=True, ejk=False):
    """Gradients of one packed batch ([1, T, H, *] inputs, cu [N + 1]) by the
    chunk algebra; Hkv = H.  Returns dq, dk, dv, dg, dbeta, da_log, ddt_bias, dS0."""
    _, T, H, dk = q.shape
    dv = v.shape[-1]
    N = len(cu) - 1
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros((1, T, H) if ejk else (1, T, H, dk)), dbeta=np.zeros((1, T, H)),
               da_log=np.zeros(H), ddt_bias=np.zeros((dk, H)), dS0=np.zeros((N, H, dk, dv)))
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            s = np.zeros((dk, dv)) if S0 is None else S0[n, h].copy()
            chunks = []
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                R = _rows(q[0, c0:c1, h], k[0, c0:c1, h], None if g is None else g[0, c0:c1, h],
                          beta[0, c0:c1, h], a_log[h] if not ejk else 0.0,
                          dt_bias[:, h] if not ejk else 0.0, scale, lb, l2norm, ejk)
                F = _chunk_fwd(R, v[0, c0:c1, h], s, ejk)
                chunks.append((c0, c1, R, F, s))
                s = F["S1"]
            ds = np.zeros((dk, dv)) if dSf is None else dSf[n, h].copy()
            for c0, c1, R, F, s0 in reversed(chunks):
                G = _chunk_local(R, F, s0, dO[0, c0:c1, h], ds, ejk)
                dq, dkk, dgg, dbb, dx = _prologue_bwd(R, G, scale, lb, l2norm, ejk, a_log[h] if not ejk else 0)
                out["dq"][0, c0:c1, h], out["dk"][0, c0:c1, h], out["dv"][0, c0:c1, h] = dq, dkk, G["dV"]
                out["dg"][0, c0:c1, h], out["dbeta"][0, c0:c1, h] = dgg, dbb
                if not ejk:
                    out["ddt_bias"][:, h] += dgg.sum(0)
                    out["da_log"][h] += np.sum(dx * R["x"])
                ds = _chunk_dS0(F, dO[0, c0:c1, h], ds, R["bt"])[2]
            out["dS0"][n, h] = ds
    return out
