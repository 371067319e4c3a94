"""GPU parity of kda_recurrent_step against the fp64 oracle (through the C ABI).

The full decode workload (256 sequences x 32 heads, dk = dv = 128, 512 steps on a
resident fp32 state) runs in full on the GPU; the oracle follows a seeded sample of
512 chains over all 512 steps and checks their outputs at every step and their
final states. Small cases cover both dtypes, gate modes and head sizes, and T
decode steps are checked against one chunked forward over the same T tokens.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
import oracle
from kda_workloads import CONFIGS, decode_initial_state, decode_step_inputs, make_chunk_inputs
from tests.gpu_util import DT, TOL, assert_close, note, up

pytestmark = pytest.mark.gpu


def test_decode_workload_sampled_chains():
    cfg = CONFIGS[4]
    note(f"decode parity {cfg.name}: {cfg.T} steps, sampled chains")
    N, H = cfg.B, cfg.H
    rng = np.random.default_rng(99)
    pick = np.sort(rng.choice(N * H, size=512, replace=False))
    S0 = decode_initial_state(cfg)
    state = up(S0)
    ref_state = S0.reshape(N * H, cfg.dk, cfg.dv)[pick].astype(np.float64)
    got_o, want_o = [], []
    for step in range(cfg.T):
        d = decode_step_inputs(cfg, step)
        o = kda.recurrent_step(up(d.q, torch.bfloat16), up(d.k, torch.bfloat16),
                               up(d.v, torch.bfloat16), up(d.g), up(d.beta), state)
        flat = lambda a: a.reshape(N * H, *a.shape[2:])[pick]  # noqa: E731
        ro, ref_state = oracle.kda_chains(
            flat(d.q), flat(d.k), flat(d.v), flat(d.g), flat(d.beta),
            np.arange(len(pick)), np.ones(len(pick), np.int64), s0=ref_state)
        got_o.append(o.float().cpu().numpy().reshape(N * H, -1)[pick])
        want_o.append(ro)
    torch.cuda.synchronize()
    eo = assert_close(np.stack(got_o), np.stack(want_o), TOL["bf16"], "decode outputs")
    got_s = state.cpu().numpy().reshape(N * H, cfg.dk, cfg.dv)[pick]
    es = assert_close(got_s, ref_state, TOL["bf16"], "decode final states")
    print(f"decode: err o={eo:.2e} S={es:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(dtype, gate, dk, dv):
    cfg = CONFIGS[4].replace(dtype=dtype, gate=gate, dk=dk, dv=dv, B=5, H=3, seed=31)
    note(f"decode small {dtype} {gate} {dk}x{dv}")
    S = decode_initial_state(cfg)
    state = up(S)
    ref = S.astype(np.float64)
    for step in range(6):
        d = decode_step_inputs(cfg, step)
        o = kda.recurrent_step(up(d.q, DT[dtype]), up(d.k, DT[dtype]), up(d.v, DT[dtype]),
                               up(d.g), up(d.beta), state)
        ro, ref = oracle.kda_decode_step(ref, d.q, d.k, d.v, d.g, d.beta)
        assert_close(o.float().cpu().numpy(), ro, TOL[dtype], f"step {step} outputs")
    assert_close(state.cpu().numpy(), ref, TOL[dtype], "final states")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_steps_equal_chunk_forward(dtype):
    """T calls of the decode step equal one chunked forward over the same T tokens."""
    cfg = CONFIGS[1].replace(dtype=dtype, B=2, H=3, T=70, seed=15)
    x = make_chunk_inputs(cfg)
    dt = DT[dtype]
    note(f"decode steps vs chunk forward {dtype}")
    o_chunk, s_chunk = kda.chunk_fwd(up(x.q, dt), up(x.k, dt), up(x.v, dt), up(x.g),
                                     up(x.beta), initial_state=up(x.s0))
    state = up(x.s0)
    outs = []
    for t in range(cfg.T):
        sl = lambda a: np.ascontiguousarray(a[:, :, t])  # noqa: E731
        outs.append(kda.recurrent_step(up(sl(x.q), dt), up(sl(x.k), dt), up(sl(x.v), dt),
                                       up(sl(x.g)), up(sl(x.beta)), state))
    torch.cuda.synchronize()
    o_steps = torch.stack(outs, dim=2).float().cpu().numpy()
    tol = TOL[dtype]
    assert_close(o_steps, o_chunk.float().cpu().numpy(), tol, "steps vs chunk outputs")
    assert_close(state.cpu().numpy(), s_chunk.cpu().numpy(), tol, "steps vs chunk states")
