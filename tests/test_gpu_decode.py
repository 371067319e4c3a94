"""GPU parity of kda_recurrent_step against the fp64 oracle (through the C ABI).

The full decode workload (256 sequences x 32 heads, dk = dv = 128, 512 steps on a
resident fp32 state) runs in full on the GPU, and the oracle follows all 8192 chains
over the 512 steps: their outputs at every step and their final states. Small cases cover both dtypes, gate modes and head sizes, and T
decode steps are checked against one chunked forward over the same T tokens.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
import oracle
from kda_workloads import (KDA_B2_H16_T4096, KDA_DECODE_N256_H32, decode_initial_state,
                           decode_step_inputs, make_chunk_inputs)
from tests.gpu_util import DT, TOL, assert_close, note, up

pytestmark = pytest.mark.gpu


def test_decode_workload_all_chains():
    cfg = KDA_DECODE_N256_H32
    note(f"decode parity {cfg.name}: {cfg.T} steps, all chains")
    N, H, T, dk, dv = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv
    S0 = decode_initial_state(cfg)
    state = up(S0)
    dev = state.device
    # every step's inputs stay on the GPU ([T, N, H, d]) for the oracle's chains below
    qs = torch.empty((T, N, H, dk), dtype=torch.bfloat16, device=dev)
    ks, vs = torch.empty_like(qs), torch.empty((T, N, H, dv), dtype=torch.bfloat16, device=dev)
    gs = torch.empty((T, N, H, dk), dtype=torch.float32, device=dev)
    bs = torch.empty((T, N, H), dtype=torch.float32, device=dev)
    os_ = torch.empty((T, N, H, dv), dtype=torch.bfloat16, device=dev)
    for step in range(T):
        d = decode_step_inputs(cfg, step)
        qs[step], ks[step], vs[step] = (up(a, torch.bfloat16) for a in (d.q, d.k, d.v))
        gs[step], bs[step] = up(d.g), up(d.beta)
        os_[step] = kda.recurrent_step(qs[step], ks[step], vs[step], gs[step], bs[step], state)
    torch.cuda.synchronize()
    got_s = state.cpu().numpy().reshape(N * H, dk, dv)
    S0f = S0.reshape(N * H, dk, dv)
    worst = (0.0, 0.0)
    per = 1024  # chains per oracle call (bounds the host memory)
    for c0 in range(0, N * H, per):
        sl = slice(c0, c0 + per)
        # rows of chain c are its T steps: [T, chains, d] -> [chains * T, d]
        rows = lambda t: t.reshape(T, N * H, *t.shape[3:])[:, sl].transpose(0, 1).reshape(  # noqa: E731
            -1, *t.shape[3:]).float().cpu().numpy()
        n = min(per, N * H - c0)
        ro, rs = oracle.kda_chains(rows(qs), rows(ks), rows(vs), rows(gs), rows(bs),
                                   np.arange(n) * T, np.full(n, T), s0=S0f[sl])
        eo = assert_close(rows(os_), ro, TOL["bf16"], f"decode outputs, chains {c0}..")
        es = assert_close(got_s[sl], rs, TOL["bf16"], f"decode final states, chains {c0}..")
        worst = (max(worst[0], eo), max(worst[1], es))
    print(f"decode: all {N * H} chains x {T} steps, err o={worst[0]:.2e} S={worst[1]:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(dtype, gate, dk, dv):
    cfg = KDA_DECODE_N256_H32.replace(dtype=dtype, gate=gate, dk=dk, dv=dv, B=5, H=3, seed=31)
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
    cfg = KDA_B2_H16_T4096.replace(dtype=dtype, B=2, H=3, T=70, seed=15)
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


def test_decode_steps_in_a_replayed_graph():
    """Eight decode steps captured once in a HIP graph and replayed three times, with eager
    work and synchronisations between the replays: every replay gives the eager outputs
    and final state bit for bit."""
    cfg = KDA_DECODE_N256_H32.replace(B=16, H=4, T=8, seed=61)
    note("decode steps in a HIP graph")
    N, H, T = cfg.B, cfg.H, cfg.T
    S0 = up(decode_initial_state(cfg))
    steps = [decode_step_inputs(cfg, s) for s in range(T)]
    ins = [(up(d.q, torch.bfloat16), up(d.k, torch.bfloat16), up(d.v, torch.bfloat16),
            up(d.g), up(d.beta)) for d in steps]
    outs = [torch.empty((N, H, cfg.dv), dtype=torch.bfloat16, device=S0.device) for _ in range(T)]
    state = S0.clone()
    for s in range(T):
        kda.recurrent_step(*ins[s], state, o=outs[s])
    torch.cuda.synchronize()
    want_o = [o.clone() for o in outs]
    want_s = state.clone()
    state.copy_(S0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(T):
            kda.recurrent_step(*ins[s], state, o=outs[s])
    for rep in range(3):
        state.copy_(S0)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(T):
            assert torch.equal(outs[s], want_o[s]), f"replay {rep}, step {s}: outputs differ"
        assert torch.equal(state, want_s), f"replay {rep}: final state differs"
