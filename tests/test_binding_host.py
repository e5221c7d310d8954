"""Host checks of the Python binding: every tensor a kernel reads or writes is
shape-checked before the library is called, so a caller's wrong buffer raises
instead of reaching the GPU.  CPU tensors only; no library call is made."""
import pytest
import torch

import gated_delta_rule_90_amd as kda


def _decode_args(B=3, H=4, hkv=2, dk=16, dv=8):
    f = torch.float32
    return dict(q=torch.zeros(B, dk, H, dtype=f), k=torch.zeros(B, dk, hkv, dtype=f),
                v=torch.zeros(B, hkv, dv, dtype=f), g=torch.zeros(B, dk, H, dtype=f),
                beta=torch.zeros(B, 1, H, dtype=f), a_log=torch.zeros(1, H, dtype=f),
                dt_bias=torch.zeros(dk, H, dtype=f), S=torch.zeros(B, H, dk, dv, dtype=f))


def _decode(**over):
    a = _decode_args()
    a.update(over)
    return kda.decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["a_log"], a["dt_bias"], a["S"],
                           out=a.get("out"))


@pytest.mark.parametrize("over,msg", [
    (dict(out=torch.zeros(3, 2, 8)), "out must be"),          # shaped like v: [B, Hkv, dv]
    (dict(a_log=torch.zeros(1, 3)), "a_log"),
    (dict(dt_bias=torch.zeros(4, 16)), "dt_bias"),
    (dict(k=torch.zeros(3, 16, 3)), "Hkv dividing H"),
    (dict(v=torch.zeros(3, 4, 8)), "v must be"),
    (dict(g=None), "needs g"),
    (dict(S=torch.zeros(3, 2, 16, 8)), "S must be"),
])
def test_decode_step_rejects_wrong_shapes(over, msg):
    with pytest.raises(ValueError, match=msg):
        _decode(**over)


def _prefill_args(B=2, T=5, H=4, hkv=2, dk=16, dv=8):
    f, bf = torch.float32, torch.bfloat16
    return dict(q=torch.zeros(B, T, H, dk, dtype=bf), k=torch.zeros(B, T, hkv, dk, dtype=bf),
                v=torch.zeros(B, T, hkv, dv, dtype=bf), g=torch.zeros(B, T, H, dk, dtype=f),
                beta=torch.zeros(B, T, H, dtype=f), a_log=torch.zeros(H, dtype=f),
                dt_bias=torch.zeros(dk, H, dtype=f))


@pytest.mark.parametrize("over,msg", [
    (dict(out=torch.zeros(2, 5, 2, 8, dtype=torch.bfloat16)), "out must be"),
    (dict(k=torch.zeros(2, 5, 3, 16, dtype=torch.bfloat16)), "Hkv dividing H"),
    (dict(v=torch.zeros(2, 5, 4, 8, dtype=torch.bfloat16)), "Hkv dividing H"),
    (dict(beta=torch.zeros(2, 5, 2)), "beta"),
    (dict(a_log=torch.zeros(2)), "a_log"),
    (dict(dt_bias=torch.zeros(4, 16)), "dt_bias"),
    (dict(initial_state=torch.zeros(2, 2, 16, 8)), "initial_state"),
])
def test_prefill_rejects_wrong_shapes(over, msg):
    a = _prefill_args()
    out = over.pop("out", None)
    init = over.pop("initial_state", None)
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        kda.prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["a_log"], a["dt_bias"], init, out=out)
