"""Host checks of bench.py: the algorithmic byte and flop counts behind its
roofline fractions, the one-GPU refusal, and the committed counter lookup.

The expected counts are rebuilt here tensor by tensor (or term by term of the
chunk algebra), not by calling the formulas under test."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_b64_h32_d128():
    B, H, dk, dv, f32 = 64, 32, 128, 128, 4
    tensors = {
        "state in": B * H * dk * dv * f32,
        "state out": B * H * dk * dv * f32,
        "q": B * dk * H * f32, "k": B * dk * H * f32, "g": B * dk * H * f32,
        "v": B * H * dv * f32, "out": B * H * dv * f32,
        "beta": B * H * f32, "a_log": H * f32, "dt_bias": dk * H * f32,
    }
    assert sum(tensors.values()) == 273_703_040
    assert bench.decode_bytes(B, H, dk, dv) == 273_703_040


def test_prefill_bytes_b4_t4096_h16_d128_bf16():
    B, T, H, dk, dv, bf16, f32 = 4, 4096, 16, 128, 128, 2, 4
    ntok = B * T
    tensors = {
        "q": ntok * H * dk * bf16, "k": ntok * H * dk * bf16, "v": ntok * H * dv * bf16,
        "g": ntok * H * dk * f32, "beta": ntok * H * f32, "o": ntok * H * dv * bf16,
        "final state": B * H * dk * dv * f32, "a_log": H * f32, "dt_bias": dk * H * f32,
    }
    assert sum(tensors.values()) == 407_904_320
    assert bench.prefill_bytes(ntok, H, dk, dv, B, False) == 407_904_320


def test_prefill_bytes_initial_state_and_ejk():
    # an initial state is read as well as the final one written; EJK has one
    # decay per token and head and no a_log / dt_bias
    ntok, H, dk, dv, N = 100, 2, 128, 64, 3
    base = bench.prefill_bytes(ntok, H, dk, dv, N, False)
    assert bench.prefill_bytes(ntok, H, dk, dv, N, True) - base == N * H * dk * dv * 4
    ejk = bench.prefill_bytes(ntok, H, dk, dv, N, False, ejk=True)
    assert base - ejk == ntok * H * (dk - 1) * 4 + H * 4 + dk * H * 4


def test_grouped_bytes():
    # grouped key/value heads: k and v are read once per key/value head
    B, H, hkv, dk, dv, f32 = 64, 32, 8, 128, 128, 4
    assert bench.decode_bytes(B, H, dk, dv) - bench.decode_bytes(B, H, dk, dv, hkv) == \
        (B * dk + B * dv) * (H - hkv) * f32
    ntok, bf16 = 4 * 4096, 2
    assert bench.prefill_bytes(ntok, 16, dk, dv, 4, False) - \
        bench.prefill_bytes(ntok, 16, dk, dv, 4, False, hkv=4) == ntok * (16 - 4) * (dk + dv) * bf16


def test_prefill_flops_per_token_head():
    # per chunk of C tokens (lower-triangular products count half): A = K K^T,
    # P = Q K^T and W = T' Kg each C^2 dk; U~ = T' V and P U each C^2 dv; the
    # state products W S0, Qg S0 and Kc^T U each 2 C dk dv
    C, dk, dv = 64, 128, 128
    per_chunk = 3 * C * C * dk + 2 * C * C * dv + 3 * (2 * C * dk * dv)
    assert per_chunk // C == 139_264
    assert bench.prefill_flops(C, 1, dk, dv) == per_chunk


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_counter_traffic_only_for_matching_source():
    sh = bench._src_hash("kda_decode.hip", "kda_device.h")
    good = bench._counter_traffic("decode_b64_h32_d128", sh)
    if good is None:
        pytest.skip("committed counter summary predates the current decode source")
    # within 1% of the algorithmic bytes: the state stream is read and written once
    assert abs(good - 273_703_040) / 273_703_040 < 0.01
    assert bench._counter_traffic("decode_b64_h32_d128", "0" * 16) is None


def test_prefill_counters_only_for_matching_source(monkeypatch):
    res = bench.prefill_counters(0.2574)
    if res["mfma_flops"] is None:
        pytest.skip("committed prefill counter summary predates the current chunked source")
    # executed bf16 MFMA work lies between the triangle-aware algorithmic count
    # and the count with every masked tile executed
    tri = bench.prefill_flops(4 * 4096, 16, 128, 128)
    dense = 4 * 4096 * 16 * (64 * (6 * 128 + 4 * 128) + 6 * 128 * 128)
    assert tri <= res["mfma_flops"] <= dense
    assert res["mfma_frac"] == round(res["mfma_flops"] / 0.2574e-3 / 1e12 / 2500.0, 4)
    # the record round trip: more HBM traffic than the algorithmic bytes, within 3x
    assert 407_904_320 < res["traffic"] < 3 * 407_904_320
    monkeypatch.setattr(bench, "_src_hash", lambda *names: "0" * 16)
    stale = bench.prefill_counters(0.2574)
    assert stale["traffic"] is None and stale["mfma_frac"] is None


def test_cpu_decode_leg_reports_parity_of_the_given_step():
    from gated_delta_rule_90_amd import workloads
    from oracle import kda_oracle
    inp = workloads.decode_inputs(2, 3, 16, 16, seed=5)
    ro, rS = kda_oracle.decode(inp.q, inp.k, inp.g, inp.v, inp.beta, inp.a_log, inp.dt_bias, inp.S,
                               scale=inp.scale, lower_bound=inp.lower_bound)
    good = bench.cpu_decode_baseline(inp, budget_s=0.05, check=(ro.astype(np.float32), rS.astype(np.float32)))
    assert good["parity"]["ok"] and good["parity"]["rel_l2_out"] < 1e-6
    bad_out = ro.copy()
    bad_out[0, 0, 0] += 0.01 * np.linalg.norm(ro)      # a 1% error in one element
    bad = bench.cpu_decode_baseline(inp, budget_s=0.05, check=(bad_out, rS))
    assert not bad["parity"]["ok"] and abs(bad["parity"]["rel_l2_out"] - 0.01) < 1e-3
    assert "parity" not in bench.cpu_decode_baseline(inp, budget_s=0.05)


def test_cpu_info_and_prefill_leg_on_a_sample():
    """The CPU prefill leg times the oracle on the sampled heads (median of the
    runs), reports the host (cores, nproc, CPU model) and, with the GPU's
    outputs, the worst per-unit parity of those heads."""
    from gated_delta_rule_90_amd import workloads
    from oracle import kda_oracle
    info = bench.cpu_info()
    assert info["cores"] == kda_oracle.max_threads() and info["nproc"] >= 1
    inp = workloads.prefill_inputs(1, 0, 4, 16, 16, seed=9, lengths=[20, 0, 7], init_state=True, hkv=2)
    ro, rs = kda_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.a_log, inp.dt_bias,
                                inp.initial_state, inp.cu_seqlens, scale=inp.scale,
                                lower_bound=inp.lower_bound)
    res = bench._cpu_prefill_leg(inp, range(2), 3, "3 packed sequences",
                                 check=(ro.astype(np.float32), rs.astype(np.float32)))
    assert res["kind"] == "oracle" and res["value"] > 0 and "median of 3" in res["sample"]
    assert res["parity"]["ok"] and res["parity"]["worst_unit_rel_l2_o"] < 1e-6
    bad = ro.copy()
    bad[0, 25, 1] *= 1.5                                 # one token of sequence 2, head 1
    res = bench._cpu_prefill_leg(inp, range(2), 1, "3 packed sequences", check=(bad, rs))
    assert not res["parity"]["ok"]
    with pytest.raises(ValueError):
        bench._cpu_prefill_leg(inp, [0, 1, 2], 1, "uneven groups")   # 2 + 1 heads per key/value head
