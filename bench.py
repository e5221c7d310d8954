"""Benchmark of the KDA hot path on one MI355X.

Headline (``value``): single-token decode steps/s for B=64 requests, H=32,
dk=dv=128, fp32 (the kda_tkg-shaped workload): one step is one
kda_decode_step call - prologue, state decay, delta update and output for all
64 x 32 (request, head) items.  Inputs are resident in HBM before timing; the
state rotates over 5 buffers (640 MiB) so that the 256 MB Infinity Cache
cannot hold it between steps.

The same JSON line also carries:
  roofline      the decode kernel against MI355X's 8 TB/s HBM (algorithmic
                bytes per launch / mean launch time from HIP events)
  cpu_baseline  the float64 CPU oracle timed on the host on a bounded sample
                (decode here; the prefill entry carries its own), with the
                parity (relative L2) of the GPU results of the benchmarked
                configuration on that sample
  prefill       chunked prefill tokens/s for B=4, T=4096, H=16, dk=dv=128
                (bf16 inputs) with its own roofline fractions (--no-prefill
                skips it)
  configs       the other workloads, each timed the same way: the fp32
                token-by-token kernel at B=1, T=64, H=2, d=16 (latency bound),
                one 65536-token sequence with 32 heads (also split at 32768
                with the state passed through, checked bitwise against the
                unsplit call), and 8 packed sequences of 512..8192 tokens with
                32 heads, in KDA and EJK mode (--no-configs skips them)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-configs] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + decode steps/s; % MFMA peak / % HBM BW peak"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFS = 2500.0

# decode, B=64 H=32 dk=dv=128: state read + write, q/g [B,dk,H], k [B,dk,Hkv],
# v [B,Hkv,dv], out [B,H,dv], beta [B,1,H], a_log [1,H], dt_bias [dk,H] - all fp32
def decode_bytes(B, H, dk, dv, hkv=None):
    hkv = H if hkv is None else hkv
    return 4 * (2 * B * H * dk * dv + 2 * B * dk * H + B * dk * hkv + B * hkv * dv + B * H * dv
                + B * H + H + dk * H)


def decode_flops(B, H, dk, dv):
    # decay (1), S^T k (2), S^T q (2), rank-1 update (2) per state element
    return 7 * B * H * dk * dv


def prefill_bytes(ntok, H, dk, dv, n_states, init_state, ejk=False, io_bytes=2, hkv=None):
    # q (H heads), k, v (Hkv heads) in; g (KDA: [dk] per token-head, EJK: one decay)
    # and beta fp32; o out; final states written, initial states read when given;
    # a_log, dt_bias (KDA)
    hkv = H if hkv is None else hkv
    gate = 4 if ejk else dk * 4
    per_tok = H * (dk * io_bytes + gate + 4 + dv * io_bytes) + hkv * (dk + dv) * io_bytes
    states = n_states * H * dk * dv * 4 * (2 if init_state else 1)
    return ntok * per_tok + states + (0 if ejk else H * 4 + dk * H * 4)


def prefill_flops(ntok, H, dk, dv, C=64):
    # triangle-aware: intra-chunk Gram and output terms + the three state products
    return ntok * H * (C * (3 * dk + 2 * dv) + 6 * dk * dv)


def _code_only(text):
    """Source text without comments and blank space, so that a counter summary
    stays tied to the code it was taken on, not to the comments around it."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.strip() for line in text.splitlines() if line.strip())


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_90_amd", "csrc", n), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _profile_kv(name, src_hash):
    """The "key: value" lines of a committed rocprofv3 --pmc summary
    (profiles/<name>_pmc.txt) if it was taken on the current kernel source;
    else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_pmc.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv if kv.get("src_hash") == src_hash else None


def _counter_traffic(name, src_hash):
    """HBM bytes per launch from a committed counter summary taken on the
    current kernel source; else None."""
    kv = _profile_kv(name, src_hash)
    try:
        return int(float(kv["hbm_bytes_per_launch"])) if kv else None
    except (KeyError, ValueError):
        return None


def prefill_counters(ms, name="chunked_prefill_b4_t4096_h16_d128", alg_bytes=None):
    """Counter figures of a chunked prefill workload from its committed summary
    (profiles/<name>_pmc.txt: HBM traffic, executed bf16 MFMA flops, MFMA busy
    fraction), with the executed flops turned into a fraction of peak over this
    run's time and the traffic into a ratio to the algorithmic bytes; all None
    once the kernel source has changed since they were taken."""
    sh = _src_hash("kda_chunked.hip", "kda_device.h")
    kv = _profile_kv(name, sh)
    res = {"traffic": None, "traffic_over_alg": None, "mfma_flops": None, "mfma_frac": None,
           "mfma_busy_frac": None, "src_hash": sh, "source": f"profiles/{name}_pmc.txt"}
    if kv:
        try:
            tr = int(float(kv["hbm_bytes_per_call"]))
            res["traffic"] = tr
            if alg_bytes:
                res["traffic_over_alg"] = round(tr / alg_bytes, 3)
            fl = int(float(kv["mfma_bf16_flops_per_call"]))
            res.update(mfma_flops=fl, mfma_frac=round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS, 4),
                       mfma_busy_frac=float(kv["mfma_busy_frac"]))
        except (KeyError, ValueError):
            pass
    return res


def bench_decode(steps, warmup, nbuf=5):
    from gated_delta_rule_90_amd import workloads
    return _decode_run(workloads.decode_b64_h32_d128(), steps, warmup, nbuf)


def _decode_run(inp, steps, warmup, nbuf=5):
    """Time kda.decode_step with the state rotating over nbuf buffers."""
    import torch
    import gated_delta_rule_90_amd as kda
    f = torch.float32
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", f)
    q, k, v, g, beta = d(inp.q), d(inp.k), d(inp.v), d(inp.g), d(inp.beta)
    a_log, dtb = d(inp.a_log), d(inp.dt_bias)
    S0 = d(inp.S)
    states = [S0.clone() for _ in range(nbuf)]
    B, dk, H = inp.q.shape
    hkv = inp.k.shape[2]
    dv = inp.v.shape[-1]
    out = torch.empty((B, H, dv), dtype=f, device="cuda")   # [B, H, dv]: v has Hkv heads

    def step(i):
        kda.decode_step(q, k, v, g, beta, a_log, dtb, states[i % nbuf], scale=inp.scale,
                        lower_bound=inp.lower_bound, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    # One more untimed step goes in first, so that e0's timestamp is taken when
    # it ends with the first timed step already queued behind it: the device
    # time of the K steps does not include the host's latency to submit the
    # first one after the synchronisation (the wall time below does).
    step(warmup)
    e0.record()
    for i in range(steps):
        step(warmup + 1 + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    nbytes = decode_bytes(B, H, dk, dv, hkv)
    achieved = nbytes / (ms * 1e-3) / 1e9
    # one more step from the initial state, outside the timed region: its output
    # and new state are compared with the oracle by the CPU leg
    S1 = S0.clone()
    out1 = kda.decode_step(q, k, v, g, beta, a_log, dtb, S1, scale=inp.scale, lower_bound=inp.lower_bound)
    torch.cuda.synchronize()
    check = (out1.cpu().numpy(), S1.cpu().numpy())
    del S1, states
    sh = _src_hash("kda_decode.hip", "kda_device.h")
    traffic = _counter_traffic("decode_b64_h32_d128", sh)
    return inp, {
        "check": check,
        "ms": ms, "wall_s": wall, "steps_per_s": 1e3 / ms, "bytes": nbytes,
        "flops": decode_flops(B, H, dk, dv),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "decode_kernel<128,128,false>",
                     "bytes_per_launch": nbytes, "src_hash": sh},
    }


def rel_l2(x, ref):
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _unit_worst(o, ro, s, rs, cu=None):
    """Worst relative L2 over (sequence, head) units, for o [B, T, H, dv] (packed:
    B = 1, sequence n is rows cu[n]:cu[n+1]) and states [N, H, dk, dv]."""
    N, H = rs.shape[:2]
    wo = ws = 0.0
    for n in range(N):
        if cu is None:
            on, ron = o[n], ro[n]
        else:
            on, ron = o[0, int(cu[n]):int(cu[n + 1])], ro[0, int(cu[n]):int(cu[n + 1])]
        for h in range(H):
            if on.shape[0]:
                wo = max(wo, rel_l2(on[:, h], ron[:, h]))
            ws = max(ws, rel_l2(s[n, h], rs[n, h]))
    return wo, ws


# float32 prefill workloads: (input generator in workloads, chunked route, kernel sources)
FP32_CONFIGS = {
    "recurrent_fp32_b1_t64_h2_d16": ("recurrent_fp32_small", False, ("kda_recurrent.hip", "kda_device.h")),
    "chunked_fp32_b1_t64_h2_d16": ("recurrent_fp32_small", True, ("kda_chunked_f32.hip", "kda_device.h")),
    "prefill_fp32_b1_t4096_h16_d128_token_by_token": ("prefill_fp32_b1_t4096_h16_d128", False,
                                                      ("kda_recurrent.hip", "kda_device.h")),
    "prefill_fp32_b1_t4096_h16_d128_chunked": ("prefill_fp32_b1_t4096_h16_d128", True,
                                               ("kda_backward.hip", "kda_device.h")),
}


def kernel_counters(name, sources, alg_bytes):
    """HBM traffic per call of a workload from its committed counter summary
    (profiles/<name>_pmc.txt, taken on the current source of `sources`) and
    its ratio to the algorithmic bytes; None once the source has changed."""
    sh = _src_hash(*sources)
    kv = _profile_kv(name, sh)
    res = {"traffic": None, "traffic_over_alg": None, "src_hash": sh, "source": f"profiles/{name}_pmc.txt"}
    if kv:
        try:
            tr = int(float(kv["hbm_bytes_per_call"]))
            res.update(traffic=tr, traffic_over_alg=round(tr / alg_bytes, 3) if alg_bytes else None)
        except (KeyError, ValueError):
            pass
    return res


def cpu_info():
    """Host figures reported with every CPU leg: logical CPUs of the machine,
    its CPU model, and the oracle's OpenMP thread count (the cores it uses)."""
    from oracle import kda_oracle
    kda_oracle.build(force=False)
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = None
    return {"cores": kda_oracle.max_threads(), "threads": kda_oracle.max_threads(),
            "nproc": os.cpu_count(), "cpus_available": avail, "cpu_model": model}


def _median3(fn, runs=3):
    """Wall times of `runs` calls of fn (steady clock); (median, all)."""
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), [round(t, 3) for t in ts]


def cpu_decode_baseline(inp, budget_s=10.0, check=None):
    """The float64 oracle on full decode steps: a sample of n steps, timed three
    times, median reported (n set so the three take about budget_s).  With
    check = (out, S_new) of the GPU's step from the same state, the first
    oracle step also gives the parity of the benchmarked configuration."""
    from oracle import kda_oracle
    info = cpu_info()
    t0 = time.perf_counter()
    ro, rS = kda_oracle.decode(inp.q, inp.k, inp.g, inp.v, inp.beta, inp.a_log, inp.dt_bias, inp.S,
                               scale=inp.scale, lower_bound=inp.lower_bound)
    one = time.perf_counter() - t0
    parity = None
    if check is not None:
        parity = {"rel_l2_out": rel_l2(check[0], ro), "rel_l2_state": rel_l2(check[1], rS), "bar": 1e-5,
                  "sample": "one step of all 64 x 32 (request, head) items"}
        parity["ok"] = parity["rel_l2_out"] <= 1e-5 and parity["rel_l2_state"] <= 1e-5
    reps = max(1, int(budget_s / 3 / max(one, 1e-3)))

    def run():
        for _ in range(reps):
            kda_oracle.decode(inp.q, inp.k, inp.g, inp.v, inp.beta, inp.a_log, inp.dt_bias, inp.S,
                              scale=inp.scale, lower_bound=inp.lower_bound)

    el, runs = _median3(run)
    res = dict({"value": round(reps / el, 3), "unit": "decode steps/s", "kind": "oracle",
                "sample": f"{reps} full decode steps (B=64, H=32, dk=dv=128, float64) per run; "
                          f"median of 3 runs {runs} s"}, **info)
    if parity is not None:
        res["parity"] = parity
    return res


def _cpu_prefill_leg(inp, heads, runs, what, check=None):
    """The float64 oracle on the given heads of a prefill workload (every
    sequence of it), timed `runs` times; reported as tokens/s over all heads
    (the sample's time scaled by H / len(heads)).  With check = (o, final
    state) of the GPU call on the same inputs, the first run also gives the
    parity of those heads, per (sequence, head) unit."""
    from oracle import kda_oracle
    info = cpu_info()
    H = inp.q.shape[2]
    hs = list(heads)
    hkv = inp.k.shape[2]
    kv = sorted({h // (H // hkv) for h in hs})
    kmap = [kv.index(h // (H // hkv)) for h in hs]
    if len(hs) % len(kv) or kmap != [i // (len(hs) // len(kv)) for i in range(len(hs))]:
        raise ValueError("sampled heads must be whole, equal groups of their key/value heads")
    args = (inp.q[:, :, hs], inp.k[:, :, kv], inp.v[:, :, kv],
            None if inp.g is None else inp.g[:, :, hs], inp.beta[:, :, hs],
            None if inp.ejk else inp.a_log[hs], None if inp.ejk else inp.dt_bias[:, hs],
            None if inp.initial_state is None else inp.initial_state[:, hs], inp.cu_seqlens)
    kw = dict(scale=inp.scale, lower_bound=inp.lower_bound, ejk=inp.ejk)
    out = {}

    def run():
        out["r"] = kda_oracle.prefill(*args, **kw)

    el, times = _median3(run, runs)
    ntok = int(inp.q.shape[0] * inp.q.shape[1])
    res = dict({"value": round(ntok / (el * H / len(hs)), 1), "unit": f"prefill tokens/s (all {H} heads)",
                "kind": "oracle",
                "sample": f"{what}, heads {hs[0]}..{hs[-1]} ({len(hs)} of {H}), float64; "
                          + (f"median of {runs} runs {times} s" if runs > 1 else f"one run {times} s")}, **info)
    if check is not None:
        ro, rs = out["r"]
        o_gpu, s_gpu = check
        wo, ws = _unit_worst(o_gpu[:, :, hs], ro, s_gpu[:, hs], rs, inp.cu_seqlens)
        bar = 2e-2 if inp.dtype == "bf16" else 1e-5
        res["parity"] = {"worst_unit_rel_l2_o": wo, "worst_unit_rel_l2_state": ws, "bar": bar,
                         "ok": wo <= bar and ws <= bar,
                         "sample": "every (sequence, head) unit of the sampled heads of the timed call"}
    return res


def cpu_prefill_baseline(budget_s=5.0, check=None):
    """The float64 oracle on a bounded sample of the B4 T4096 H16 workload: all
    four sequences of the first few heads (enough (sequence, head) units for
    every core), median of three runs; reported as tokens/s over all 16 heads."""
    from gated_delta_rule_90_amd import workloads
    from oracle import kda_oracle
    kda_oracle.build(force=False)
    threads = kda_oracle.max_threads()
    inp = workloads.prefill_b4_t4096_h16_d128()
    B, T, H, _ = inp.q.shape
    nh = min(H, max(1, -(-threads // B)))
    return _cpu_prefill_leg(inp, range(nh), 3, "4 sequences x 4096 tokens", check)


def _prefill_run(inp, steps, warmup, nsets=1, split=None, graph=False, keep=False, use_chunked=None):
    """Time kda.prefill on one workload (inputs resident in HBM, nsets input
    copies used in turn so the Infinity Cache cannot hold them)."""
    import torch
    import gated_delta_rule_90_amd as kda
    io = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f = torch.float32
    d = lambda x, t: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(t)
    sets = [[d(inp.q, io), d(inp.k, io), d(inp.v, io), d(inp.g, f), d(inp.beta, f)]
            for _ in range(nsets)]
    a_log = None if inp.ejk else d(inp.a_log, f)
    dtb = None if inp.ejk else d(inp.dt_bias, f)
    s0 = d(inp.initial_state, f)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to("cuda")
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    nst = B if cu is None else cu.numel() - 1
    o = torch.empty((B, T, H, dv), dtype=io, device="cuda")
    fs = torch.empty((nst, H, dk, dv), dtype=f, device="cuda")

    def call(i, q=None, k=None, v=None, g=None, beta=None, init=s0, out=o, fin=fs, use_chunked=True):
        qq, kk, vv, gg, bb = sets[i % nsets]
        return kda.prefill(qq if q is None else q, kk if k is None else k, vv if v is None else v,
                           gg if g is None else g, bb if beta is None else beta, a_log, dtb, init,
                           cu, scale=inp.scale, lower_bound=inp.lower_bound, ejk=inp.ejk,
                           use_chunked=use_chunked, out=out, final_state=fin)

    # bf16 inputs: the chunked kernels (the MFMA one at dk = 128, the float32 one
    # below); float32 inputs: the token-by-token kernel unless use_chunked asks
    # for the float32 chunked one
    chunked = (inp.dtype == "bf16") if use_chunked is None else use_chunked
    mfma = chunked and inp.dtype == "bf16" and dk == 128
    for i in range(warmup):
        call(i, use_chunked=chunked)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    call(warmup, use_chunked=chunked)   # untimed lead call: see _decode_run
    e0.record()
    for i in range(steps):
        call(warmup + 1 + i, use_chunked=chunked)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    ntok = B * T if cu is None else int(inp.cu_seqlens[-1])
    io_bytes = 2 if inp.dtype == "bf16" else 4
    nbytes = prefill_bytes(ntok, H, dk, dv, nst, s0 is not None, inp.ejk, io_bytes, inp.k.shape[2])
    res = {"tokens_per_s": round(ntok / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
           "wall_ms_per_call": round(wall * 1e3 / (steps + 1), 4), "alg_bytes": nbytes, "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "path": "chunked MFMA" if mfma else (
               ("chunked float32, two kernels (16-token operand blocks, then the scan)" if H * dk >= 128
                else "chunked float32, one kernel") if chunked else "token-by-token")}
    if mfma:
        fl = prefill_flops(ntok, H, dk, dv)
        tfs = fl / (ms * 1e-3) / 1e12
        floor_ms = max(nbytes / (HBM_PEAK_GBS * 1e9), fl / (BF16_MFMA_PEAK_TFS * 1e12)) * 1e3
        res.update({"alg_flops_tri": fl, "mfma_frac": round(tfs / BF16_MFMA_PEAK_TFS, 4),
                    "roofline_frac": round(floor_ms / ms, 4),
                    "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1), "achieved_TFs": round(tfs, 2)})
    if graph:
        # a call this small is bound by the host's per-call overhead; captured
        # in a HIP graph (GRAPH_CALLS calls per replay) it shows the device time.
        # Each replay's output must equal the eager call's bitwise.
        GRAPH_CALLS = 20
        call(0, use_chunked=chunked)
        torch.cuda.synchronize()
        o_ref, fs_ref = o.clone(), fs.clone()
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(0, use_chunked=chunked)   # warm the side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for _ in range(GRAPH_CALLS):
                call(0, use_chunked=chunked)
        same = True
        for _ in range(3):
            o.zero_()
            fs.zero_()
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            same = same and bool(torch.equal(o, o_ref) and torch.equal(fs, fs_ref))
        reps = max(1, steps // GRAPH_CALLS)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            gr.replay()
        g1.record()
        torch.cuda.synchronize()
        res["graph_ms_per_call"] = round(g0.elapsed_time(g1) / (reps * GRAPH_CALLS), 4)
        res["graph_replay_bitwise_equal"] = same
        del gr
    if split is not None:
        # the same call in two halves with the state passed through: bitwise equal?
        call(0, use_chunked=chunked)
        torch.cuda.synchronize()
        o_ref, fs_ref = o.clone(), fs.clone()
        qq, kk, vv, gg, bb = sets[0]
        o1 = torch.empty_like(o[:, :split])
        o2 = torch.empty_like(o[:, split:])
        mid = torch.empty_like(fs)
        fin = torch.empty_like(fs)
        part = lambda x, a, b: None if x is None else x[:, a:b].contiguous()
        call(0, part(qq, 0, split), part(kk, 0, split), part(vv, 0, split), part(gg, 0, split),
             part(bb, 0, split), s0, o1, mid, use_chunked=chunked)
        call(0, part(qq, split, T), part(kk, split, T), part(vv, split, T), part(gg, split, T),
             part(bb, split, T), mid, o2, fin, use_chunked=chunked)
        torch.cuda.synchronize()
        res["split_at"] = split
        res["split_bitwise_equal"] = bool(torch.equal(torch.cat([o1, o2], 1), o_ref) and
                                          torch.equal(fin, fs_ref))
    if keep:
        # every input set holds the same values, so o and fs are the outputs of one call
        res["check"] = (o.float().cpu().numpy(), fs.cpu().numpy())
    del sets
    return res


def bench_prefill(steps, warmup):
    from gated_delta_rule_90_amd import workloads
    inp = workloads.prefill_b4_t4096_h16_d128()
    res = _prefill_run(inp, steps, warmup, nsets=2, keep=True)   # 2 x 408 MB: more than the Infinity Cache
    res.pop("path")
    res["rocprof"] = prefill_counters(res["ms_per_call"], alg_bytes=res["alg_bytes"])
    return dict({"workload": "kda_chunked_prefill_b4_t4096_h16_d128_bf16"}, **res)


def _mfma_configs():
    """The bf16 chunked-prefill workloads timed as configs:
    name -> (input maker, timing options, CPU-leg heads, CPU-leg runs, CPU-leg description)."""
    from gated_delta_rule_90_amd import workloads
    return {
        "prefill_long_t65536_h32_d128": (workloads.prefill_long_t65536_h32_d128, {"split": 32768},
                                         "threads", 1, "1 sequence x 65536 tokens"),
        "prefill_varlen_8seq_h32_d128": (workloads.prefill_varlen_8seq_h32_d128, {}, "threads/8", 3,
                                         "8 packed sequences"),
        "prefill_varlen_8seq_h32_d128_ejk": (lambda: workloads.prefill_varlen_8seq_h32_d128(ejk=True), {},
                                             "threads/8", 3, "8 packed sequences, EJK"),
        "prefill_grouped_b4_t4096_h16_hkv4_d128": (workloads.prefill_grouped_b4_t4096_h16_hkv4_d128,
                                                   {"nsets": 2}, "threads/4", 3, "4 sequences x 4096 tokens"),
    }


def bench_one_mfma_config(name, steps, warmup, cpu=True, extras=True):
    """Time one bf16 chunked-prefill workload; with cpu, also its sampled CPU
    oracle leg (and the parity of the sampled heads of the timed call).
    extras=False leaves out the calls beyond the timed ones (the split check),
    so that a profiler run sees only full calls."""
    import gc
    from oracle import kda_oracle
    make, kw, heads, runs, what = _mfma_configs()[name]
    if not extras:
        kw = {k: v for k, v in kw.items() if k != "split"}
    inp = make()
    res = _prefill_run(inp, steps, warmup, keep=cpu, **kw)
    if inp.cu_seqlens is not None:
        res["lengths"] = inp.meta["lengths"]
    res["rocprof"] = prefill_counters(res["ms_per_call"], name, res["alg_bytes"])
    if cpu:
        check = res.pop("check")
        H = inp.q.shape[2]
        th = kda_oracle.max_threads()
        nseq = inp.q.shape[0] if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
        nh = min(H, max(1, th if heads == "threads" else -(-th // nseq)))
        hkv = inp.k.shape[2]
        nh = -(-nh // (H // hkv)) * (H // hkv)          # whole groups of key/value heads
        res["cpu_baseline"] = _cpu_prefill_leg(inp, range(min(nh, H)), runs, what, check)
        del check
    del inp
    gc.collect()
    return res


def backward_bytes(ntok, H, dk, dv, io_bytes=2, do_bytes=2):
    """Algorithmic bytes of one prefill backward: q, k, v (input dtype), g, beta
    and dO read; dq, dk, dv, dg, dbeta written (float32)."""
    return ntok * H * ((2 * dk + dv) * io_bytes + 4 * dk + 4 + dv * do_bytes + 4 * (3 * dk + dv) + 4)


def bench_backward(steps, warmup, cpu=True):
    """kda_prefill_backward on the B4 T4096 H16 bf16 workload (dO bf16, no
    final-state gradient), with a sampled CPU oracle leg."""
    import torch
    import gated_delta_rule_90_amd as kda
    from gated_delta_rule_90_amd import workloads
    inp = workloads.prefill_b4_t4096_h16_d128()
    bf, f = torch.bfloat16, torch.float32
    d = lambda x, t: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(t)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    d_o_np = workloads.round_to_bf16(np.random.default_rng(1003).standard_normal((B, T, H, dv), np.float32))
    args = (d(inp.q, bf), d(inp.k, bf), d(inp.v, bf), d(inp.g, f), d(inp.beta, f), d(inp.a_log, f),
            d(inp.dt_bias, f), None, None, d(d_o_np, bf))

    def call():
        return kda.prefill_backward(*args, scale=inp.scale, lower_bound=inp.lower_bound)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = backward_bytes(B * T, H, dk, dv)
    res = {"workload": "kda_prefill_backward_b4_t4096_h16_d128_bf16", "tokens_per_s": round(B * T / (ms * 1e-3), 1),
           "ms_per_call": round(ms, 4), "alg_bytes": nbytes,
           "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "note": "float32 arithmetic; chunks of 16 tokens: chunk operands formed once, forward state "
                   "scan, reverse state-gradient scan, chunk-parallel local gradients",
           "rocprof": kernel_counters("backward_b4_t4096_h16_d128_bf16", ("kda_backward.hip", "kda_device.h"),
                                      nbytes)}
    if cpu:
        from oracle import kda_oracle
        gr = call()
        torch.cuda.synchronize()
        hs = list(range(min(H, max(1, -(-kda_oracle.max_threads() // B)))))
        sub = lambda x: x[:, :, hs]
        t0 = time.perf_counter()
        ref = kda_oracle.backward(sub(inp.q), sub(inp.k), sub(inp.v), sub(inp.g), sub(inp.beta),
                                  inp.a_log[hs], inp.dt_bias[:, hs], None, None, d_o=sub(d_o_np),
                                  scale=inp.scale, lower_bound=inp.lower_bound)
        el = time.perf_counter() - t0
        # every one of these has the head axis third: [B, T, H, ...]
        worst = max(rel_l2(gr[n][:, :, hs].cpu().numpy(), ref[n]) for n in ("dq", "dk", "dv", "dg", "dbeta"))
        res["cpu_baseline"] = dict({"value": round(B * T / (el * H / len(hs)), 1),
                                    "unit": f"backward tokens/s (all {H} heads)", "kind": "oracle",
                                    "sample": f"4 sequences x 4096 tokens, heads 0..{hs[-1]}, float64; one run {el:.2f} s",
                                    "parity": {"worst_rel_l2": worst, "bar": 2e-2, "ok": worst <= 2e-2,
                                               "over": "dq, dk, dv, dg, dbeta of the sampled heads"}},
                                   **cpu_info())
    return res


def gated_bytes(ntok, H, dk, dv, gates, io_bytes=2):
    """Algorithmic bytes of one gated recurrent attention call: q, k, v in,
    the given per-token gates (float32), o out."""
    per = (2 * dk + dv) * io_bytes + dv * io_bytes
    per += 4 * dk * (("g" in gates) + ("gk" in gates)) + 4 * dv * ("gv" in gates)
    return ntok * H * per + (4 * H if "g_gamma" in gates else 0)


GATED_CONFIGS = ["gated_recurrent_b4_t4096_h16_d128_bf16_gk", "gated_recurrent_b4_t4096_h16_d128_bf16_all"]


def bench_gated(steps, warmup, cpu=True, only=None):
    """recurrent_attention on the B4 T4096 H16 bf16 workload, with the key
    gate alone and with all four gates; each with a sampled CPU oracle leg
    (the float64 token loop on the first heads, every sequence) that also
    gives the parity of those heads."""
    import torch
    import gated_delta_rule_90_amd as kda
    from gated_delta_rule_90_amd import workloads
    inp = workloads.prefill_b4_t4096_h16_d128()
    bf, f = torch.bfloat16, torch.float32
    d = lambda x, t: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(t)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    rng = np.random.default_rng(1008)
    gk = -np.abs(0.05 * rng.standard_normal((B, T, H, dk), np.float32))
    gv = -np.abs(0.05 * rng.standard_normal((B, T, H, dv), np.float32))
    g = 0.1 * rng.standard_normal((B, T, H, dk), np.float32)
    gg = -np.abs(0.01 * rng.standard_normal((B, H), np.float32))
    q, k, v = d(inp.q, bf), d(inp.k, bf), d(inp.v, bf)
    out = {}
    for name, gates_np in (("gk", {"gk": gk}), ("all", {"g": g, "gk": gk, "gv": gv, "g_gamma": gg})):
        key = f"gated_recurrent_b4_t4096_h16_d128_bf16_{name}"
        if only is not None and key != only:
            continue
        gates = {n: d(x, f) for n, x in gates_np.items()}
        call = lambda: kda.recurrent_attention(q, k, v, **gates)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes = gated_bytes(B * T, H, dk, dv, gates)
        res = {"tokens_per_s": round(B * T / (ms * 1e-3), 1), "ms_per_call": round(ms, 4), "alg_bytes": nbytes,
               "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "gates": sorted(gates),
               "path": "16-token chunks, float32 (MFMA)",
               "rocprof": kernel_counters(key, ("kda_gated.hip", "kda_device.h"), nbytes)}
        if cpu:
            from oracle import kda_oracle
            o_gpu = call().float().cpu().numpy()
            hs = list(range(min(H, max(1, -(-kda_oracle.max_threads() // B)))))
            sub = lambda x: None if x is None else x[:, :, hs]
            qs, ks, vs = (workloads.round_to_bf16(x[:, :, hs]) for x in (inp.q, inp.k, inp.v))
            kw = dict(g=sub(gates_np.get("g")), gk=sub(gates_np.get("gk")), gv=sub(gates_np.get("gv")),
                      g_gamma=None if "g_gamma" not in gates_np else gates_np["g_gamma"][:, hs])
            box = {}

            def run():
                box["o"], _ = kda_oracle.gated_recurrent(qs, ks, vs, **kw)

            el, times = _median3(run, 3)
            worst = max(rel_l2(o_gpu[bb, :, h], box["o"][bb, :, j]) for bb in range(B) for j, h in enumerate(hs))
            res["cpu_baseline"] = dict({"value": round(B * T / (el * H / len(hs)), 1),
                                        "unit": f"tokens/s (all {H} heads)", "kind": "oracle",
                                        "sample": f"4 sequences x 4096 tokens, heads 0..{hs[-1]} ({len(hs)} of "
                                                  f"{H}), float64; median of 3 runs {times} s",
                                        "parity": {"worst_unit_rel_l2_o": worst, "bar": 2e-2, "ok": worst <= 2e-2,
                                                   "sample": "every (sequence, head) unit of the sampled heads"}},
                                       **cpu_info())
        out[key] = res
    return out


def bench_configs(steps, warmup, cpu=True):
    """The other workloads: each is generated on the host (seeded), uploaded,
    then timed; inputs are freed before the next one."""
    import gc
    from gated_delta_rule_90_amd import workloads
    out = {}
    inp = workloads.recurrent_fp32_small()
    r = _prefill_run(inp, 10 * steps, warmup, graph=True, keep=cpu)
    c1 = r.pop("check", None)
    out["recurrent_fp32_b1_t64_h2_d16"] = dict(r, note="64 dependent token steps per call: latency bound; "
                                                       "ms_per_call includes the host's per-call overhead, "
                                                       "graph_ms_per_call is the device time")
    # the same workload through the float32 chunked kernel (2 chunks of 32 tokens)
    r2 = _prefill_run(inp, 10 * steps, warmup, graph=True, use_chunked=True, keep=cpu)
    c2 = r2.pop("check", None)
    out["chunked_fp32_b1_t64_h2_d16"] = dict(r2, note="2 dependent 32-token chunks per call; graph_ms_per_call "
                                                      "is the device time")
    if cpu:
        # the whole workload (both heads)
        for key, ck in (("recurrent_fp32_b1_t64_h2_d16", c1), ("chunked_fp32_b1_t64_h2_d16", c2)):
            out[key]["cpu_baseline"] = _cpu_prefill_leg(inp, range(inp.q.shape[2]), 3, "the whole workload",
                                                        check=ck)
    # a larger float32 prefill on both float32 kernels
    inp = workloads.prefill_fp32_b1_t4096_h16_d128()
    out["prefill_fp32_b1_t4096_h16_d128_token_by_token"] = _prefill_run(inp, steps, warmup, keep=cpu)
    out["prefill_fp32_b1_t4096_h16_d128_chunked"] = _prefill_run(inp, steps, warmup, use_chunked=True, keep=cpu)
    if cpu:
        from oracle import kda_oracle
        nh = min(inp.q.shape[2], max(1, kda_oracle.max_threads()))
        for key in ("prefill_fp32_b1_t4096_h16_d128_token_by_token", "prefill_fp32_b1_t4096_h16_d128_chunked"):
            out[key]["cpu_baseline"] = _cpu_prefill_leg(inp, range(nh), 3, "1 sequence x 4096 tokens",
                                                        check=out[key].pop("check"))
    del inp
    for key, (_, _, sources) in FP32_CONFIGS.items():
        out[key]["rocprof"] = kernel_counters(key, sources, out[key].get("alg_bytes"))
    gc.collect()
    for name in _mfma_configs():
        out[name] = bench_one_mfma_config(name, steps, warmup, cpu)
    out["backward_b4_t4096_h16_d128_bf16"] = bench_backward(max(3, steps // 4), 1, cpu)
    gc.collect()
    out.update(bench_gated(max(3, steps // 4), 1, cpu))
    gc.collect()
    # a decode step takes ~50 us: 20x the steps of the prefill configs, so that the
    # mean is not set by the first few calls
    ginp = workloads.decode_grouped_b64_h32_hkv8_d128()
    _, dres = _decode_run(ginp, 20 * steps, 2 * warmup)
    out["decode_grouped_b64_h32_hkv8_d128"] = {
        "steps_per_s": round(dres["steps_per_s"], 2), "ms_per_step": round(dres["ms"], 5),
        "alg_bytes": dres["bytes"], "hbm_frac": dres["roofline"]["frac"],
        "rocprof": kernel_counters("decode_grouped_b64_h32_hkv8_d128", ("kda_decode.hip", "kda_device.h"),
                                   dres["bytes"])}
    if cpu:
        out["decode_grouped_b64_h32_hkv8_d128"]["cpu_baseline"] = cpu_decode_baseline(ginp, 5.0,
                                                                                      check=dres.get("check"))
    return out


def copy_calibration(mib=256):
    """One device-to-device copy of a known size (read and write `mib` MiB each),
    so that profiler byte counters can be scaled against a known amount."""
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--config", default=None,
                    help="time only this bf16 chunked-prefill workload (for profiler runs)")
    ap.add_argument("--calib", action="store_true",
                    help="run a 256 MiB device copy first (profiler counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the KDA path runs on one GPU only (asked for --gpus {args.gpus}); "
              "the KDA kernels use no collectives and the pass does not shard", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calib:
        copy_calibration()
    if args.config:
        # one workload alone (profiling runs): its own timing only
        if args.config == "prefill_b4_t4096_h16_d128":
            res = bench_prefill(max(20, args.steps), args.warmup)
            res.pop("check", None)
        elif args.config in _mfma_configs():
            res = bench_one_mfma_config(args.config, max(10, args.steps), args.warmup, cpu=False,
                                        extras=False)
        elif args.config in FP32_CONFIGS:
            from gated_delta_rule_90_amd import workloads
            gen, chunked, _ = FP32_CONFIGS[args.config]
            res = _prefill_run(getattr(workloads, gen)(), max(10, args.steps), args.warmup, use_chunked=chunked)
            res.pop("check", None)
        elif args.config == "decode_grouped_b64_h32_hkv8_d128":
            from gated_delta_rule_90_amd import workloads
            _, dres = _decode_run(workloads.decode_grouped_b64_h32_hkv8_d128(), 20 * max(1, args.steps), args.warmup)
            res = {"steps_per_s": round(dres["steps_per_s"], 2), "ms_per_step": round(dres["ms"], 5),
                   "alg_bytes": dres["bytes"]}
        elif args.config == "backward_b4_t4096_h16_d128_bf16":
            res = bench_backward(args.steps, args.warmup, cpu=False)
        elif args.config in GATED_CONFIGS:
            res = bench_gated(args.steps, args.warmup, cpu=False, only=args.config)[args.config]
        else:
            print(f"bench.py: unknown --config {args.config}; one of prefill_b4_t4096_h16_d128, "
                  + ", ".join(list(_mfma_configs()) + list(FP32_CONFIGS) + ["decode_grouped_b64_h32_hkv8_d128",
                              "backward_b4_t4096_h16_d128_bf16"] + GATED_CONFIGS),
                  file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"config": args.config, **res}), flush=True)
        return
    inp, dec = bench_decode(args.steps, args.warmup)
    line = {
        "metric": METRIC,
        "value": round(dec["steps_per_s"], 2),
        "unit": "decode steps/s (B=64 requests x H=32 heads, dk=dv=128)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "kda_decode_b64_h32_d128_fp32", "B": 64, "H": 32, "dk": 128,
                   "dv": 128, "state_buffers": 5, "seed": 1002},
        "request_tokens_per_s": round(64 * dec["steps_per_s"], 1),
        "roofline": dec["roofline"],
    }
    pcheck = None
    if not args.no_prefill:
        # at least 20 calls (~5 ms of timed work) whatever --steps says
        line["prefill"] = bench_prefill(max(20, args.steps), max(2, args.warmup // 2))
        pcheck = line["prefill"].pop("check")
    if not args.no_configs:
        line["configs"] = bench_configs(max(10, args.steps // 2), max(2, args.warmup // 2),
                                        cpu=not args.no_cpu)
    dcheck = dec.pop("check")
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_decode_baseline(inp, args.cpu_budget, check=dcheck)
        if "prefill" in line:
            line["prefill"]["cpu_baseline"] = cpu_prefill_baseline(args.cpu_budget / 2, check=pcheck)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
