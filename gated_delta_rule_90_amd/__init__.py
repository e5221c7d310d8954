"""MI355X-native Kimi Delta Attention (KDA) gated delta-rule recurrence.

Thin Python binding over ``libkda.so`` (see ``include/kda.h``): it checks and
marshals torch tensors into device pointers and the current HIP stream, and
allocates outputs with torch.  Every step of the computation runs in the HIP
kernels; there is no CPU or PyTorch fallback - if the library is missing the
calls raise.

    prefill(q, k, v, g, beta, a_log, dt_bias, initial_state=None, cu_seqlens=None,
            scale=None, lower_bound=-5.0, chunk_size=64, use_qk_l2norm=True,
            use_chunked=True, ejk=False, return_state=False)
        mirrors ejkernel kernel_delta_attention's run() (plus cu_seqlens, as in
        ejkernel's recurrent run()), returning o or (o, final_state).
    decode_step(q, k, v, g, beta, a_log, dt_bias, S, scale=None, lower_bound=-5.0)
        mirrors the kda_tkg kernel: fills out [B, H, dv] and advances S in place.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = ["prefill", "prefill_noalloc", "prefill_backward", "recurrent_attention", "decode_step", "KdaError", "lib", "LIB_PATH",
           "QK_L2NORM", "CHUNKED", "EJK", "F32", "BF16", "prefill_workspace_bytes"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

# values of include/kda.h
KDA_OK, KDA_EINVAL, KDA_EUNSUPPORTED, KDA_EHIP = 0, 1, 2, 3
F32, BF16 = 0, 1
QK_L2NORM, CHUNKED, EJK = 1 << 0, 1 << 1, 1 << 2

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libkda status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libkda.so and declare its C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i32, u32, f32 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    L.kda_prefill.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, fp, fp, ip, i32, i32, i32,
                              i32, i32, i32, i32, f32, f32, i32, u32, vp, ctypes.c_int, fp, vp,
                              ctypes.c_size_t, vp]
    L.kda_prefill.restype = ctypes.c_int
    L.kda_prefill_noalloc.argtypes = L.kda_prefill.argtypes[:24] + [vp]
    L.kda_prefill_noalloc.restype = ctypes.c_int
    L.kda_prefill_backward.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, fp, fp, ip, i32, i32, i32, i32,
                                       i32, i32, i32, f32, f32, u32, vp, ctypes.c_int, fp, fp, fp, fp, fp,
                                       fp, fp, fp, fp, vp, ctypes.c_size_t, vp]
    L.kda_prefill_backward.restype = ctypes.c_int
    L.kda_prefill_backward_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.kda_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
    L.kda_recurrent_attention.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, fp, fp, ip, i32, i32, i32,
                                          i32, i32, i32, i32, f32, i32, vp, ctypes.c_int, fp, vp,
                                          ctypes.c_size_t, vp]
    L.kda_recurrent_attention.restype = ctypes.c_int
    L.kda_recurrent_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.kda_recurrent_attention_workspace_bytes.restype = ctypes.c_size_t
    L.kda_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int, u32]
    L.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.kda_decode_step.argtypes = [fp, fp, fp, fp, fp, fp, fp, f32, f32, i32, i32, i32, i32, i32, u32,
                                  fp, fp, vp]
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_last_error.argtypes = []
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_abi_version.argtypes = []
    L.kda_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != KDA_OK:
        raise KdaError(status, lib().kda_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(name, t, dtypes, device):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device, stream):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Make `stream` current while outputs and the workspace are allocated, so
    torch's caching allocator ties those blocks to the stream the kernels run
    on: the workspace freed on return is then reused only by work ordered
    after them on that stream."""
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def prefill_workspace_bytes(num_seqs, B, T, H, dk, dv, flags, in_dtype=BF16) -> int:
    return int(lib().kda_prefill_workspace_bytes(num_seqs, B, T, H, dk, dv, in_dtype, flags))


def prefill(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None, cu_seqlens=None, *,
            scale=None, lower_bound=-5.0, chunk_size=64, use_qk_l2norm=True, use_chunked=True,
            ejk=False, return_state=False, out_dtype=None, out=None, final_state=None,
            stream=None, _noalloc=False):
    """KDA over whole sequences.  q [B, T, H, dk], k [B, T, Hkv, dk] and
    v [B, T, Hkv, dv] in bf16 or fp32 (Hkv divides H: head h reads the key and
    value of head h // (H // Hkv)); g [B, T, H, dk] raw gate (EJK: [B, T, H]
    log-decay or None);
    beta [B, T, H] (KDA logits / EJK activated); a_log [H]; dt_bias [dk, H];
    initial_state [N, H, dk, dv]; cu_seqlens [N + 1] int32 with B == 1.
    Returns o, or (o, final_state) when return_state (final_state may be passed
    in, also as the initial_state tensor itself for an in-place carry)."""
    import torch
    dev = q.device
    io = (torch.bfloat16, torch.float32)
    f = (torch.float32,)
    _dev("q", q, io, dev)
    _dev("k", k, (q.dtype,), dev)
    _dev("v", v, (q.dtype,), dev)
    _dev("g", g, f, dev)
    _dev("beta", beta, f, dev)
    _dev("a_log", a_log, f, dev)
    _dev("dt_bias", dt_bias, f, dev)
    _dev("initial_state", initial_state, f, dev)
    _dev("cu_seqlens", cu_seqlens, (torch.int32,), dev)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape[:2] != q.shape[:2] or \
            k.shape[3] != q.shape[3] or v.shape[:3] != k.shape[:3] or q.shape[2] % k.shape[2] != 0:
        raise ValueError("q must be [B, T, H, dk], k [B, T, Hkv, dk] and v [B, T, Hkv, dv], Hkv dividing H")
    B, T, H, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if beta.shape != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    if g is not None:
        want = (B, T, H) if ejk else (B, T, H, dk)
        if tuple(g.shape) != want:
            raise ValueError(f"g must be {list(want)}")
    if a_log is not None and a_log.numel() != H:
        raise ValueError("a_log must hold H values")
    if dt_bias is not None and tuple(dt_bias.shape) != (dk, H):
        raise ValueError("dt_bias must be [dk, H]")
    if initial_state is not None and tuple(initial_state.shape) != (N, H, dk, dv):
        raise ValueError(f"initial_state must be [{N}, {H}, {dk}, {dv}]")
    odt = q.dtype if out_dtype is None else out_dtype
    with _on(stream):
        if out is None:
            out = torch.empty((B, T, H, dv), dtype=odt, device=dev)
        else:
            _dev("out", out, (odt,), dev)
            if tuple(out.shape) != (B, T, H, dv):
                raise ValueError("out must be [B, T, H, dv]")
        if return_state and final_state is None:
            final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        elif final_state is not None:
            _dev("final_state", final_state, f, dev)
            if tuple(final_state.shape) != (N, H, dk, dv):
                raise ValueError("final_state must be [N, H, dk, dv]")
        flags = (QK_L2NORM if use_qk_l2norm else 0) | (CHUNKED if use_chunked else 0) | \
            (EJK if ejk else 0)
        nseq = N if cu_seqlens is not None else 0
        idt = BF16 if q.dtype == torch.bfloat16 else F32
        sc = -1.0 if scale is None else float(scale)
        common = (_ptr(q), _ptr(k), _ptr(v), idt,
                  _ptr(g), _ptr(beta), _ptr(a_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_seqlens),
                  nseq, B, T, H, Hkv, dk, dv, sc, float(lower_bound), int(chunk_size), flags,
                  _ptr(out), BF16 if odt == torch.bfloat16 else F32, _ptr(final_state))
        if _noalloc:
            _check(lib().kda_prefill_noalloc(*common, _stream(dev, stream)))
        else:
            wsb = prefill_workspace_bytes(nseq, B, T, H, dk, dv, flags, idt)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb > 0 else None
            _check(lib().kda_prefill(*common, _ptr(ws), wsb, _stream(dev, stream)))
    if return_state:
        return out, final_state
    return out


def prefill_noalloc(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None,
                    cu_seqlens=None, **kw):
    """prefill() through kda_prefill_noalloc: the library call allocates
    nothing; the chunked path's scratch is the library's fixed device array of
    KDA_NOALLOC_SCRATCH_BYTES per GPU (shared by every call on that GPU, so
    calls that overlap in time on one GPU race).  Pass ``out`` (and
    ``final_state``) to keep this wrapper from allocating them with torch."""
    return prefill(q, k, v, g, beta, a_log, dt_bias, initial_state, cu_seqlens, _noalloc=True, **kw)


def prefill_backward(q, k, v, g, beta, a_log=None, dt_bias=None, initial_state=None, cu_seqlens=None,
                     d_o=None, d_final_state=None, *, scale=None, lower_bound=-5.0, use_qk_l2norm=True,
                     ejk=False, stream=None):
    """Gradients of prefill() (kda_prefill_backward).  Inputs as prefill();
    d_o [B, T, H, dv] (float32 or bf16) is dL/do and d_final_state
    [N, H, dk, dv] dL/d(final state) (None = 0).  Returns a dict of float32
    tensors: dq, dk, dv (shapes of q, k, v), dg (shape of g: [B, T, H, dk]
    for KDA, [B, T, H] for EJK), dbeta ([B, T, H]: dL/d logit for KDA,
    dL/d beta for EJK), d_initial_state [N, H, dk, dv] and, for KDA,
    da_log [H] and ddt_bias [dk, H]."""
    import torch
    dev = q.device
    io = (torch.bfloat16, torch.float32)
    f = (torch.float32,)
    _dev("q", q, io, dev)
    _dev("k", k, (q.dtype,), dev)
    _dev("v", v, (q.dtype,), dev)
    _dev("g", g, f, dev)
    _dev("beta", beta, f, dev)
    _dev("a_log", a_log, f, dev)
    _dev("dt_bias", dt_bias, f, dev)
    _dev("initial_state", initial_state, f, dev)
    _dev("cu_seqlens", cu_seqlens, (torch.int32,), dev)
    _dev("d_o", d_o, io, dev)
    _dev("d_final_state", d_final_state, f, dev)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape[:2] != q.shape[:2] or \
            k.shape[3] != q.shape[3] or v.shape[:3] != k.shape[:3] or q.shape[2] % k.shape[2] != 0:
        raise ValueError("q must be [B, T, H, dk], k [B, T, Hkv, dk] and v [B, T, Hkv, dv], Hkv dividing H")
    B, T, H, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if d_o is None or tuple(d_o.shape) != (B, T, H, dv):
        raise ValueError("d_o must be [B, T, H, dv]")
    if beta.shape != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    if g is not None and tuple(g.shape) != ((B, T, H) if ejk else (B, T, H, dk)):
        raise ValueError("g must be [B, T, H, dk] (EJK: [B, T, H])")
    for name, t, shp in (("initial_state", initial_state, (N, H, dk, dv)),
                         ("d_final_state", d_final_state, (N, H, dk, dv)), ("dt_bias", dt_bias, (dk, H))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {list(shp)}")
    if a_log is not None and a_log.numel() != H:
        raise ValueError("a_log must hold H values")
    with _on(stream):
        e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
        out = {"dq": e(B, T, H, dk), "dk": e(B, T, Hkv, dk), "dv": e(B, T, Hkv, dv),
               "dg": e(B, T, H) if ejk else e(B, T, H, dk), "dbeta": e(B, T, H),
               "d_initial_state": e(N, H, dk, dv)}
        if not ejk:
            out["da_log"] = e(H)
            out["ddt_bias"] = e(dk, H)
        nseq = N if cu_seqlens is not None else 0
        wsb = int(lib().kda_prefill_backward_workspace_bytes(nseq, B, T, H, Hkv, dk, dv))
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        flags = (QK_L2NORM if use_qk_l2norm else 0) | (EJK if ejk else 0)
        sc = -1.0 if scale is None else float(scale)
        idt = BF16 if q.dtype == torch.bfloat16 else F32
        _check(lib().kda_prefill_backward(
            _ptr(q), _ptr(k), _ptr(v), idt, _ptr(g), _ptr(beta), _ptr(a_log), _ptr(dt_bias),
            _ptr(initial_state), _ptr(cu_seqlens), nseq, B, T, H, Hkv, dk, dv, sc, float(lower_bound), flags,
            _ptr(d_o), BF16 if d_o.dtype == torch.bfloat16 else F32, _ptr(d_final_state),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
            _ptr(out.get("da_log")), _ptr(out.get("ddt_bias")), _ptr(out["d_initial_state"]), _ptr(ws), wsb,
            _stream(dev, stream)))
    return out


def recurrent_attention(query, key, value, g=None, g_gamma=None, gk=None, gv=None, initial_state=None,
                        cu_seqlens=None, *, softmax_scale=None, reverse=False, return_state=False,
                        out_dtype=None, out=None, final_state=None, stream=None):
    """The gated recurrent attention of the ejkernel "recurrent" page
    (kda_recurrent_attention): query [B, T, H, dk], key [B, T, Hkv, dk],
    value [B, T, Hkv, dv] (bf16 or float32); g, gk [B, T, H, dk], gv
    [B, T, H, dv], g_gamma [B, H] float32 log-space gates (None = absent);
    initial_state [N, H, dk, dv]; cu_seqlens [N + 1] int32 with B == 1.
    Returns o, or (o, final_state) when return_state."""
    import torch
    q, k, v = query, key, value
    dev = q.device
    io = (torch.bfloat16, torch.float32)
    f = (torch.float32,)
    _dev("query", q, io, dev)
    _dev("key", k, (q.dtype,), dev)
    _dev("value", v, (q.dtype,), dev)
    for name, t in (("g", g), ("g_gamma", g_gamma), ("gk", gk), ("gv", gv), ("initial_state", initial_state)):
        _dev(name, t, f, dev)
    _dev("cu_seqlens", cu_seqlens, (torch.int32,), dev)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape[:2] != q.shape[:2] or \
            k.shape[3] != q.shape[3] or v.shape[:3] != k.shape[:3] or q.shape[2] % k.shape[2] != 0:
        raise ValueError("query must be [B, T, H, dk], key [B, T, Hkv, dk] and value [B, T, Hkv, dv]")
    B, T, H, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    for name, t, shp in (("g", g, (B, T, H, dk)), ("gk", gk, (B, T, H, dk)), ("gv", gv, (B, T, H, dv)),
                         ("g_gamma", g_gamma, (B, H)), ("initial_state", initial_state, (N, H, dk, dv))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {list(shp)}")
    odt = q.dtype if out_dtype is None else out_dtype
    with _on(stream):
        if out is None:
            out = torch.empty((B, T, H, dv), dtype=odt, device=dev)
        else:
            _dev("out", out, (odt,), dev)
            if tuple(out.shape) != (B, T, H, dv):
                raise ValueError("out must be [B, T, H, dv]")
        if return_state and final_state is None:
            final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        elif final_state is not None:
            _dev("final_state", final_state, f, dev)
            if tuple(final_state.shape) != (N, H, dk, dv):
                raise ValueError("final_state must be [N, H, dk, dv]")
        sc = -1.0 if softmax_scale is None else float(softmax_scale)
        nseq = N if cu_seqlens is not None else 0
        wsb = int(lib().kda_recurrent_attention_workspace_bytes(nseq, B, T, H, dk, dv))
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        _check(lib().kda_recurrent_attention(
            _ptr(q), _ptr(k), _ptr(v), BF16 if q.dtype == torch.bfloat16 else F32, _ptr(g), _ptr(g_gamma),
            _ptr(gk), _ptr(gv), _ptr(initial_state), _ptr(cu_seqlens), nseq,
            B, T, H, Hkv, dk, dv, sc, int(bool(reverse)), _ptr(out), BF16 if odt == torch.bfloat16 else F32,
            _ptr(final_state), _ptr(ws), wsb, _stream(dev, stream)))
    if return_state:
        return out, final_state
    return out


def decode_step(q, k, v, g, beta, a_log, dt_bias, S, *, scale=None, lower_bound=-5.0,
                use_qk_l2norm=True, ejk=False, out=None, stream=None):
    """One token for each of B requests, kda_tkg layouts (all fp32):
    q, g [B, dk, H] (EJK: g [B, 1, H] or None); k [B, dk, Hkv]; v [B, Hkv, dv]
    (Hkv divides H); beta [B, 1, H];
    a_log [1, H]; dt_bias [dk, H]; S [B, H, dk, dv] advanced in place.
    Returns out [B, H, dv]."""
    import torch
    dev = q.device
    f = (torch.float32,)
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("a_log", a_log),
                    ("dt_bias", dt_bias), ("S", S)):
        _dev(name, t, f, dev)
    if q.dim() != 3 or k.dim() != 3 or k.shape[:2] != q.shape[:2] or q.shape[2] % k.shape[2] != 0:
        raise ValueError("q must be [B, dk, H] and k [B, dk, Hkv], Hkv dividing H")
    B, dk, H = q.shape
    Hkv = k.shape[2]
    if S.dim() != 4 or tuple(S.shape[:3]) != (B, H, dk):
        raise ValueError("S must be [B, H, dk, dv]")
    dv = S.shape[3]
    if tuple(v.shape) != (B, Hkv, dv) or beta.numel() != B * H:
        raise ValueError("v must be [B, Hkv, dv] and beta [B, 1, H]")
    if g is not None and g.numel() != (B * H if ejk else B * dk * H):
        raise ValueError("g must be [B, dk, H] (EJK: [B, 1, H])")
    if not ejk and g is None:
        raise ValueError("KDA mode needs g")
    if a_log is not None and a_log.numel() != H:
        raise ValueError("a_log must hold H values")
    if dt_bias is not None and tuple(dt_bias.shape) != (dk, H):
        raise ValueError("dt_bias must be [dk, H]")
    with _on(stream):
        if out is None:
            out = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
        else:
            _dev("out", out, f, dev)
            if tuple(out.shape) != (B, H, dv):
                raise ValueError("out must be [B, H, dv]")
    flags = (QK_L2NORM if use_qk_l2norm else 0) | (EJK if ejk else 0)
    sc = -1.0 if scale is None else float(scale)
    _check(lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(g), _ptr(v), _ptr(beta), _ptr(a_log),
                                 _ptr(dt_bias), sc, float(lower_bound), B, H, Hkv, dk, dv, flags,
                                 _ptr(out), _ptr(S), _stream(dev, stream)))
    return out
