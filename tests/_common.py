"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the binding, run the oracle on the same values, and
compare with the relative L2 metric in float64."""
from __future__ import annotations

import sys

import numpy as np

import gated_delta_rule_90_amd as kda
from oracle import kda_oracle


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def say(*a):
    """Name the case on stdout (flushed) before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda").contiguous()


def prefill_gpu(inp, use_chunked=True, out_dtype=None, initial_state="inputs", cu="inputs",
                return_numpy=True, **kw):
    import torch
    io = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    s0 = inp.initial_state if isinstance(initial_state, str) else initial_state
    cu_np = inp.cu_seqlens if isinstance(cu, str) else cu
    o, fs = kda.prefill(dev(inp.q, io), dev(inp.k, io), dev(inp.v, io),
                        dev(inp.g, torch.float32), dev(inp.beta, torch.float32),
                        None if inp.ejk else dev(inp.a_log, torch.float32),
                        None if inp.ejk else dev(inp.dt_bias, torch.float32),
                        dev(s0, torch.float32), dev(cu_np, torch.int32),
                        scale=inp.scale, lower_bound=inp.lower_bound, use_chunked=use_chunked,
                        ejk=inp.ejk, return_state=True, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    if not return_numpy:
        return o, fs
    return o.float().cpu().numpy(), fs.cpu().numpy()


def prefill_oracle(inp, units=None, initial_state="inputs", cu="inputs", **kw):
    s0 = inp.initial_state if isinstance(initial_state, str) else initial_state
    cu_np = inp.cu_seqlens if isinstance(cu, str) else cu
    return kda_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta,
                              None if inp.ejk else inp.a_log, None if inp.ejk else inp.dt_bias,
                              s0, cu_np, scale=inp.scale, lower_bound=inp.lower_bound,
                              ejk=inp.ejk, units=units, **kw)


def decode_gpu(inp, S=None, **kw):
    import torch
    f = torch.float32
    St = dev(inp.S if S is None else S, f)
    out = kda.decode_step(dev(inp.q, f), dev(inp.k, f), dev(inp.v, f), dev(inp.g, f),
                          dev(inp.beta, f), dev(inp.a_log, f), dev(inp.dt_bias, f), St,
                          scale=inp.scale, lower_bound=inp.lower_bound, ejk=inp.ejk, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), St.cpu().numpy()


def decode_oracle(inp, S=None, **kw):
    return kda_oracle.decode(inp.q, inp.k, inp.g, inp.v, inp.beta, inp.a_log, inp.dt_bias,
                             inp.S if S is None else S, scale=inp.scale,
                             lower_bound=inp.lower_bound, ejk=inp.ejk, **kw)


def unit_errors(o, ro, s, rs, cu=None):
    """Relative L2 of every (sequence, head) unit, for o and the final state.

    o, ro: [B, T, H, dv] (with cu, B == 1 and sequence n is rows cu[n]:cu[n+1]);
    s, rs: [N, H, dk, dv].  Returns (eo [N, H], es [N, H]); an empty sequence
    has eo = 0."""
    N, H = rs.shape[:2]
    eo = np.zeros((N, H))
    es = np.zeros((N, H))
    for n in range(N):
        if cu is None:
            on, ron = o[n], ro[n]
        else:
            a, b = int(cu[n]), int(cu[n + 1])
            on, ron = o[0, a:b], ro[0, a:b]
        for h in range(H):
            if on.shape[0]:
                eo[n, h] = rel_l2(on[:, h], ron[:, h])
            es[n, h] = rel_l2(s[n, h], rs[n, h])
    return eo, es


def check_units(o, ro, s, rs, tol, margin=None, cu=None, label=""):
    """Assert the worst per-unit relative L2 of o and of the state; record it."""
    eo, es = unit_errors(o, ro, s, rs, cu)
    wo, ws = np.unravel_index(np.argmax(eo), eo.shape), np.unravel_index(np.argmax(es), es.shape)
    msg = (f"{label} worst unit o={eo[wo]:.3e} at (seq, head) {tuple(int(x) for x in wo)}, "
           f"S={es[ws]:.3e} at {tuple(int(x) for x in ws)}; {eo.size} units, bar {tol:g}")
    say("  " + msg)
    if margin is not None:
        margin(f"{label} o".strip(), eo[wo], tol)
        margin(f"{label} S".strip(), es[ws], tol)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s)), msg
    assert eo[wo] <= tol and es[ws] <= tol, msg
    return eo, es
