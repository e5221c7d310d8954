"""Python front end of the plain float64 C oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the library and its Python
binding never do.  It shares no code with the HIP path.

Every input is converted exactly to float64 before the call (bf16 and fp32
values are exactly representable), so the oracle sees the very values the
GPU receives.  See ``kda_oracle.c`` for the recurrence and its citations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

EPS = 1e-6  # L2-norm epsilon: x / sqrt(sum x^2 + EPS) (not given by the pages)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(ctypes.c_double)
        I = ctypes.c_int
        D = ctypes.c_double
        lib.kda_oracle_prefill.argtypes = [P, P, P, P, P, P, P, P,
                                           ctypes.POINTER(ctypes.c_int64), I, I, I, I, I, D, D, D,
                                           I, I, ctypes.POINTER(ctypes.c_int32), I, P, P, I]
        lib.kda_oracle_prefill.restype = I
        lib.kda_oracle_decode.argtypes = [P, P, P, P, P, P, P, D, D, D, I, I, I, I, I, I, I, P, P, I]
        lib.kda_oracle_decode.restype = I
        lib.kda_oracle_max_threads.restype = I
        lib.kda_oracle_backward.argtypes = [P, P, P, P, P, P, P, P, ctypes.POINTER(ctypes.c_int64), I, I, I,
                                            I, I, D, D, D, I, I, P, P, P, P, P, P, P, P, P, P, I]
        lib.kda_oracle_backward.restype = I
        lib.kda_oracle_gated_recurrent.argtypes = [P, P, P, P, P, I, P, P, P, ctypes.POINTER(ctypes.c_int64),
                                                   I, I, I, I, I, D, I, P, P, I]
        lib.kda_oracle_gated_recurrent.restype = I
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None, cu_seqlens=None,
            scale=None, lower_bound=-5.0, use_qk_l2norm=True, ejk=False, units=None,
            threads=0, eps=EPS):
    """Token-by-token float64 recurrence over every (sequence, head).

    q: [B, T, H, dk]; k: [B, T, Hkv, dk]; v: [B, T, Hkv, dv] (Hkv divides H;
    head h uses key/value head h // (H // Hkv)); g: [B, T, H, dk] raw gate (KDA) or
    [B, T, H] log-decay / None (EJK); beta: [B, T, H] logits (KDA) or
    activated (EJK); a_log [H]; dt_bias [dk, H]; initial_state [N, H, dk, dv].
    With cu_seqlens ([N+1]) the batch must be 1 and sequences are packed.
    ``units`` restricts the work to a list of (seq * H + head) items; outputs
    of the other items are left as zeros.
    Returns (o [B, T, H, dv], final_state [N, H, dk, dv]) in float64.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires batch 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = cu.shape[0] - 1
    g = _f64(g)
    beta = _f64(beta)
    a_log = _f64(np.zeros(H) if a_log is None else np.reshape(a_log, (H,)))
    dt_bias = _f64(dt_bias)
    s0 = _f64(initial_state)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    fs = np.zeros((n, H, dk, dv), dtype=np.float64)
    if units is None:
        uptr, nu = ctypes.POINTER(ctypes.c_int32)(), 0
        uarr = None
    else:
        uarr = np.ascontiguousarray(np.asarray(units, dtype=np.int32))
        uptr, nu = uarr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(uarr.size)
    sc = -1.0 if scale is None else float(scale)
    rc = lib.kda_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(a_log),
                                _ptr(dt_bias), _ptr(s0),
                                cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, H, Hkv, dk, dv,
                                sc, float(lower_bound), float(eps), int(bool(use_qk_l2norm)),
                                int(bool(ejk)), uptr, nu, _ptr(o), _ptr(fs), int(threads))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return o, fs


def decode(q, k, g, v, beta, a_log, dt_bias, S, scale=None, lower_bound=-5.0,
           use_qk_l2norm=True, ejk=False, threads=0, eps=EPS):
    """One step for each of B requests, kda_tkg layouts.

    q, g: [B, dk, H] (EJK: g is [B, 1, H] log-decay or None); k: [B, dk, Hkv];
    v: [B, Hkv, dv];
    beta: [B, 1, H]; a_log: [1, H]; dt_bias: [dk, H]; S: [B, H, dk, dv].
    Returns (out [B, H, dv], S_new) without touching the caller's S.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, dk, H = q.shape
    Hkv = k.shape[2]
    dv = v.shape[-1]
    g = _f64(g)
    beta = _f64(beta)
    a_log = _f64(np.zeros(H) if a_log is None else np.reshape(a_log, (H,)))
    dt_bias = _f64(dt_bias)
    S_new = np.array(S, dtype=np.float64, copy=True, order="C")
    out = np.zeros((B, H, dv), dtype=np.float64)
    sc = -1.0 if scale is None else float(scale)
    rc = lib.kda_oracle_decode(_ptr(q), _ptr(k), _ptr(g), _ptr(v), _ptr(beta), _ptr(a_log),
                               _ptr(dt_bias), sc, float(lower_bound), float(eps), B, H, Hkv, dk, dv,
                               int(bool(use_qk_l2norm)), int(bool(ejk)), _ptr(out), _ptr(S_new),
                               int(threads))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return out, S_new


def backward(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None, cu_seqlens=None,
             d_o=None, d_final_state=None, scale=None, lower_bound=-5.0, use_qk_l2norm=True,
             ejk=False, threads=0, eps=EPS):
    """Gradients of the prefill (o and the final state) with respect to every
    input, by a float64 reverse sweep of the token recurrence (see
    kda_oracle_backward in kda_oracle.c).  Arguments as prefill(); d_o
    [B, T, H, dv] is dL/do and d_final_state [N, H, dk, dv] dL/d(final state)
    (None = 0).  Returns a dict with dq, dk, dv (shapes of q, k, v), dg (shape
    of g: the raw gate for KDA, the decay for EJK, given even where g is None),
    dbeta (dL/d beta logit for KDA, dL/d beta for EJK), da_log [H],
    ddt_bias [dk, H] (KDA) and d_initial_state [N, H, dk, dv]."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires batch 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = cu.shape[0] - 1
    g = _f64(g)
    beta = _f64(beta)
    a_log = _f64(np.zeros(H) if a_log is None else np.reshape(a_log, (H,)))
    dt_bias = _f64(dt_bias)
    s0 = _f64(initial_state)
    do = _f64(np.zeros((B, T, H, dv)) if d_o is None else d_o)
    dsf = _f64(d_final_state)
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, Hkv, dk)), "dv": np.zeros((B, T, Hkv, dv)),
           "dg": np.zeros((B, T, H) if ejk else (B, T, H, dk)), "dbeta": np.zeros((B, T, H)),
           "da_log": np.zeros(H), "ddt_bias": np.zeros((dk, H)), "d_initial_state": np.zeros((n, H, dk, dv))}
    sc = -1.0 if scale is None else float(scale)
    rc = lib.kda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(a_log), _ptr(dt_bias),
                                 _ptr(s0), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, H, Hkv, dk,
                                 dv, sc, float(lower_bound), float(eps), int(bool(use_qk_l2norm)),
                                 int(bool(ejk)), _ptr(do), _ptr(dsf), _ptr(out["dq"]), _ptr(out["dk"]),
                                 _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["da_log"]),
                                 _ptr(out["ddt_bias"]), _ptr(out["d_initial_state"]), int(threads))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    if ejk:
        del out["da_log"], out["ddt_bias"]
    return out


def gated_recurrent(q, k, v, g=None, g_gamma=None, gk=None, gv=None, initial_state=None,
                    cu_seqlens=None, scale=None, reverse=False, threads=0):
    """The gated recurrent attention of the ejkernel "recurrent" page, token by
    token in float64 (see kda_oracle_gated_recurrent in kda_oracle.c for the
    reading of the gates).  q [B, T, H, dk]; k [B, T, Hkv, dk]; v
    [B, T, Hkv, dv]; g, gk [B, T, H, dk]; gv [B, T, H, dv]; g_gamma [B, H];
    initial_state [N, H, dk, dv].  Returns (o [B, T, H, dv], final_state)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires batch 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = cu.shape[0] - 1
    gg = _f64(g_gamma)
    rows = 0 if gg is None else gg.reshape(-1, H).shape[0]
    o = np.zeros((B, T, H, dv))
    fs = np.zeros((n, H, dk, dv))
    sc = -1.0 if scale is None else float(scale)
    rc = lib.kda_oracle_gated_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(_f64(g)), _ptr(gg), int(rows),
                                        _ptr(_f64(gk)), _ptr(_f64(gv)), _ptr(_f64(initial_state)),
                                        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, H, Hkv, dk, dv,
                                        sc, int(bool(reverse)), _ptr(o), _ptr(fs), int(threads))
    if rc != 0:
        raise ValueError("oracle gated_recurrent rejected its arguments")
    return o, fs
