"""The Python binding's own checks, on the CPU: a caller-supplied output buffer of the wrong
shape is rejected before anything reaches the library. (The device checks are bypassed here,
since there is no GPU; the library entry points are replaced by a stub that fails if called.)"""

import pytest
import torch

import gated_delta_rule_13_amd as kda


@pytest.fixture
def no_device(monkeypatch):
    monkeypatch.setattr(kda, "_check", lambda *a, **k: None)
    monkeypatch.setattr(kda, "_stream", lambda dev: 0)

    def must_not_run(*a, **k):
        raise AssertionError("reached the library with a wrong output shape")
    for name in ("kda_chunk_fwd", "kda_gdr2_chunk_fwd", "kda_recurrent_step",
                 "kda_gdr2_recurrent_step"):
        monkeypatch.setattr(kda, name, must_not_run)


def chunk_inputs(B=1, H=2, T=8, dk=64, dv=64):
    bf = torch.bfloat16
    return (torch.zeros(B, H, T, dk, dtype=bf), torch.zeros(B, H, T, dk, dtype=bf),
            torch.zeros(B, H, T, dv, dtype=bf), torch.zeros(B, H, T, dk),
            torch.zeros(B, H, T))


@pytest.mark.parametrize("o_shape", [(1, 2, 7, 64), (1, 2, 8, 32), (2, 2, 8, 64)])
def test_chunk_fwd_rejects_wrong_o(no_device, o_shape):
    q, k, v, g, beta = chunk_inputs()
    with pytest.raises(ValueError, match="o must be"):
        kda.chunk_fwd(q, k, v, g, beta, o=torch.zeros(o_shape, dtype=torch.bfloat16))


@pytest.mark.parametrize("s_shape", [(1, 2, 64, 32), (2, 2, 64, 64), (1, 1, 64, 64)])
def test_chunk_fwd_rejects_wrong_final_state(no_device, s_shape):
    q, k, v, g, beta = chunk_inputs()
    with pytest.raises(ValueError, match="final_state must be"):
        kda.chunk_fwd(q, k, v, g, beta, final_state=torch.zeros(s_shape))


def test_gdr2_chunk_fwd_rejects_wrong_o(no_device):
    q, k, v, g, _ = chunk_inputs()
    erase, write = torch.zeros(1, 2, 8, 64), torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError, match="o must be"):
        kda.gdr2_chunk_fwd(q, k, v, g, erase, write,
                           o=torch.zeros(1, 2, 8, 63, dtype=torch.bfloat16))


def test_recurrent_step_rejects_wrong_o(no_device):
    bf = torch.bfloat16
    q, k, v = (torch.zeros(3, 2, 64, dtype=bf) for _ in range(3))
    g, beta, state = torch.zeros(3, 2, 64), torch.zeros(3, 2), torch.zeros(3, 2, 64, 64)
    with pytest.raises(ValueError, match="o must be"):
        kda.recurrent_step(q, k, v, g, beta, state, o=torch.zeros(3, 2, 32, dtype=bf))
