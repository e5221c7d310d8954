"""Seeded synthetic inputs shaped like the pages' KDA workloads.

This module only draws random numbers and casts them: it contains none of the
recurrence's arithmetic, and both the HIP path (tests, benchmark) and the CPU
oracle take their inputs from it.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per input set):
  * draw order: [lengths], q, k, v, g, beta, a_log, dt_bias, initial_state
    (absent tensors are skipped; varlen lengths are drawn first because they
    fix the other shapes);
  * q, k, v, g and beta logits ~ N(0, 1); a_log ~ U(-1, 1); dt_bias ~ N(0, sd 0.1);
    initial states ~ N(0, sd 0.02);
  * normals are drawn directly in float32; "bf16" tensors are then rounded to
    bfloat16 with round-to-nearest-even and kept as float32 arrays whose values
    are exactly representable in bf16 (so the GPU cast is exact);
  * EJK inputs follow the ejkernel page's worked example: beta = logistic of a
    N(0, 1) draw (already activated) and a per-head log-decay
    d = -0.01 * |N(0, 1)| (the example's scale, sign fixed to the documented
    "decay <= 0");
  * varlen lengths: 8 iid integers U{512..8192}, the whole set redrawn until
    30720 <= sum <= 34816.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def round_to_bf16(x) -> np.ndarray:
    """float32 array -> float32 array rounded to the nearest bf16 (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + (np.uint32(0x7FFF) + lsb)) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _normal(rng, shape, sd=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sd != 1.0:
        x *= np.float32(sd)
    return x


@dataclass
class PrefillInputs:
    q: np.ndarray            # [B, T, H, dk]  (bf16-exact float32 when dtype == "bf16")
    k: np.ndarray            # [B, T, H, dk]
    v: np.ndarray            # [B, T, H, dv]
    g: np.ndarray | None     # KDA: raw gate [B, T, H, dk]; EJK: log-decay [B, T, H]
    beta: np.ndarray         # KDA: logits [B, T, H]; EJK: activated [B, T, H]
    a_log: np.ndarray        # [H]
    dt_bias: np.ndarray      # [dk, H]
    initial_state: np.ndarray | None   # [N, H, dk, dv]
    cu_seqlens: np.ndarray | None      # [N + 1] int32
    dtype: str               # "bf16" or "f32": the storage type of q, k, v
    scale: float
    lower_bound: float
    ejk: bool = False
    meta: dict = field(default_factory=dict)


@dataclass
class DecodeInputs:
    q: np.ndarray            # [B, dk, H]
    k: np.ndarray            # [B, dk, Hkv]
    v: np.ndarray            # [B, Hkv, dv]
    g: np.ndarray | None     # KDA: [B, dk, H]; EJK: [B, 1, H]
    beta: np.ndarray         # [B, 1, H]
    a_log: np.ndarray        # [1, H]
    dt_bias: np.ndarray      # [dk, H]
    S: np.ndarray            # [B, H, dk, dv]
    scale: float
    lower_bound: float
    ejk: bool = False


def varlen_lengths(rng, n=8, lo=512, hi=8192, total_lo=30720, total_hi=34816):
    while True:
        lens = rng.integers(lo, hi + 1, size=n)
        if total_lo <= int(lens.sum()) <= total_hi:
            return lens.astype(np.int64)


def prefill_inputs(B, T, H, dk, dv, seed, dtype="bf16", ejk=False, init_state=False,
                   lengths=None, zero_params=False, lower_bound=-5.0, scale=None, hkv=None):
    """Inputs of one prefill call.  With ``lengths`` (a list, or "varlen" for the
    8-sequence recipe) the batch is packed: B must be 1 and T is the sum.  With
    ``hkv`` the key and value carry hkv heads (grouped heads)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = None
    if lengths is not None:
        if isinstance(lengths, str):
            lengths = varlen_lengths(rng)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(lengths.size + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T = 1, int(cu[-1])
    n_state = (lengths.size if lengths is not None else B)
    hkv = H if hkv is None else hkv
    q = _normal(rng, (B, T, H, dk))
    k = _normal(rng, (B, T, hkv, dk))
    v = _normal(rng, (B, T, hkv, dv))
    if not ejk:
        g = _normal(rng, (B, T, H, dk))
        beta = _normal(rng, (B, T, H))
    else:
        g = -np.float32(0.01) * np.abs(_normal(rng, (B, T, H)))
        z = _normal(rng, (B, T, H)).astype(np.float64)
        beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    if zero_params:
        a_log = np.zeros(H, dtype=np.float32)
        dt_bias = np.zeros((dk, H), dtype=np.float32)
    else:
        a_log = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
        dt_bias = _normal(rng, (dk, H), sd=0.1)
    s0 = _normal(rng, (n_state, H, dk, dv), sd=0.02) if init_state else None
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    return PrefillInputs(q, k, v, g, beta, a_log, dt_bias, s0, cu, dtype, float(scale),
                         float(lower_bound), ejk,
                         meta={"seed": seed, "lengths": None if lengths is None else
                               [int(x) for x in lengths]})


def decode_inputs(B, H, dk, dv, seed, ejk=False, lower_bound=-5.0, scale=None, hkv=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    hkv = H if hkv is None else hkv
    q = _normal(rng, (B, dk, H))
    k = _normal(rng, (B, dk, hkv))
    v = _normal(rng, (B, hkv, dv))
    if not ejk:
        g = _normal(rng, (B, dk, H))
        beta = _normal(rng, (B, 1, H))
    else:
        g = -np.float32(0.01) * np.abs(_normal(rng, (B, 1, H)))
        z = _normal(rng, (B, 1, H)).astype(np.float64)
        beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    a_log = rng.uniform(-1.0, 1.0, size=(1, H)).astype(np.float32)
    dt_bias = _normal(rng, (dk, H), sd=0.1)
    S = _normal(rng, (B, H, dk, dv), sd=0.02)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    return DecodeInputs(q, k, v, g, beta, a_log, dt_bias, S, float(scale), float(lower_bound), ejk)


# The five workloads, by what they are.  Seeds 1001..1005.
def recurrent_fp32_small():
    """B=1, T=64, H=2, dk=dv=16, fp32, a_log=0, dt_bias=0, lb=-5, scale=1/4."""
    return prefill_inputs(1, 64, 2, 16, 16, seed=1001, dtype="f32", zero_params=True, scale=0.25)


def prefill_fp32_b1_t4096_h16_d128():
    """One 4096-token sequence, H=16, dk=dv=128, float32 inputs (the float32
    kernels at a prefill size), otherwise as the bf16 chunked workload."""
    return prefill_inputs(1, 4096, 16, 128, 128, seed=1008, dtype="f32")


def decode_b64_h32_d128():
    """kda_tkg-shaped decode: B=64 requests, H=32, dk=dv=128, fp32."""
    return decode_inputs(64, 32, 128, 128, seed=1002)


def prefill_b4_t4096_h16_d128():
    """Chunked prefill: B=4, T=4096, H=16, dk=dv=128, bf16 q/k/v, fp32 gates."""
    return prefill_inputs(4, 4096, 16, 128, 128, seed=1003)


def prefill_long_t65536_h32_d128():
    """Long-context prefill: B=1, T=65536, H=32, dk=dv=128, nonzero initial state."""
    return prefill_inputs(1, 65536, 32, 128, 128, seed=1004, init_state=True)


def prefill_grouped_b4_t4096_h16_hkv4_d128():
    """Grouped key/value heads: the chunked-prefill shape with 4 key/value heads."""
    return prefill_inputs(4, 4096, 16, 128, 128, seed=1006, hkv=4)


def decode_grouped_b64_h32_hkv8_d128():
    """Grouped key/value heads: the decode shape with 8 key/value heads."""
    return decode_inputs(64, 32, 128, 128, seed=1007, hkv=8)


def prefill_varlen_8seq_h32_d128(ejk=False):
    """Packed varlen prefill: 8 sequences, lengths U{512..8192}, sum ~32768, H=32."""
    return prefill_inputs(1, 0, 32, 128, 128, seed=1005, lengths="varlen", ejk=ejk)
