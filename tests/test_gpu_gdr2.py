"""GPU parity of the Gated Delta Rule-2 entry points (kda_gdr2_chunk_fwd,
kda_gdr2_recurrent_step) against the fp64 oracle, through the C ABI.

The erase gate b [.., dk] and the write gate w [.., dv] are drawn as sigmoid(N(0, 1))
per element. Checked: every dtype, gate mode and head size on ragged sequences; the
B2 H16 T4096 workload in full; the packed varlen T=65536 workload (the benchmark's
launch configuration) on all chains; edge lengths; b = w = beta 1 against the
KDA entry point; decode steps against the oracle and against one chunked forward.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
import oracle
from kda_workloads import (KDA_B2_H16_T4096, KDA_DECODE_N256_H32, KDA_VARLEN_H32_T65536,
                           decode_initial_state, decode_step_inputs, make_chunk_inputs)
from tests.gpu_util import (DT, TOL, assert_close, check_chains, note, oracle_chains, run_chunk,
                            up)

pytestmark = pytest.mark.gpu

SMALL = [(dtype, gate, dk, dv) for dtype in ("f32", "bf16") for gate in ("channel", "head")
         for dk, dv in ((64, 64), (128, 128), (64, 128), (128, 64))]


@pytest.mark.parametrize("dtype,gate,dk,dv", SMALL)
def test_gdr2_small_ragged(dtype, gate, dk, dv):
    cfg = KDA_B2_H16_T4096.replace(dtype=dtype, gate=gate, dk=dk, dv=dv, B=2, H=3, T=200, seed=78,
                                   gates="gdr2")
    note(f"gdr2 small {dtype} {gate} dk={dk} dv={dv}")
    x = make_chunk_inputs(cfg)
    o, sT = run_chunk(x, dtype)
    check_chains(x, o, sT, oracle_chains(x), TOL[dtype], f"gdr2 small {dtype} {gate} {dk}x{dv}")


def test_gdr2_b2_h16_t4096_full():
    cfg = KDA_B2_H16_T4096.replace(name="gdr2_bf16_b2_h16_t4096", gates="gdr2")
    note(f"gdr2 parity {cfg.name}")
    x = make_chunk_inputs(cfg)
    o, sT = run_chunk(x, "bf16")
    eo, es = check_chains(x, o, sT, oracle_chains(x), TOL["bf16"], cfg.name)
    print(f"{cfg.name}: err o={eo:.2e} S={es:.2e}")


def test_gdr2_varlen_t65536_all_chains():
    cfg = KDA_VARLEN_H32_T65536.replace(name="gdr2_bf16_varlen_h32_t65536", gates="gdr2")
    note(f"gdr2 parity {cfg.name} (all chains)")
    x = make_chunk_inputs(cfg)
    o, sT = run_chunk(x, "bf16", o_fill=float("nan"))
    assert np.all(np.isfinite(o)), "some output position was not written"
    worst = (0.0, 0.0)
    for h0 in range(0, cfg.H, 8):
        chains = [(n, h) for n in range(x.n_seqs) for h in range(h0, min(h0 + 8, cfg.H))]
        eo, es = check_chains(x, o, sT, oracle_chains(x, chains), TOL["bf16"],
                              f"{cfg.name} heads {h0}..{h0 + 7}")
        worst = (max(worst[0], eo), max(worst[1], es))
    print(f"{cfg.name}: all {x.n_seqs * cfg.H} chains, err o={worst[0]:.2e} S={worst[1]:.2e}")


@pytest.mark.parametrize("dv", [128, 64])
def test_gdr2_segmented_matches_oracle_and_whole_chains(dv):
    """Few chains for the device: long sequences are cut into segments. dv = 128, the segment
    plan: the later segments run from the zero state and as transitions (zero values, so the
    write gate leaves them untouched) and their outputs are corrected. dv = 64: segments of
    equal length get their end states from zero and their transitions, a chain over them
    gives every start state, and every segment is re-run from it."""
    lens = [5000, 3000, 800, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=int(cu[-1]), dv=dv, num_seqs=0, pin_frac=0.05,
                                        seed=57, gates="gdr2")
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(5).standard_normal((len(lens), 2, 128, dv)).astype(
        np.float32) * np.float32(0.02)
    ws = kda.kda_chunk_fwd_workspace_size(1, 2, int(cu[-1]), 128, dv, len(lens), kda.KDA_BF16)
    assert ws > 128 * 128 * 4, "expected a segmented path"
    note(f"gdr2 segmented dv={dv}")
    o1, s1 = run_chunk(x, "bf16", schedule=True)
    o0, s0 = run_chunk(x, "bf16", schedule=False)
    check_chains(x, o1, s1, oracle_chains(x), TOL["bf16"], "gdr2 segmented")
    assert_close(o1, o0, TOL["bf16"], "gdr2 segmented vs whole outputs")
    assert_close(s1, s0, TOL["bf16"], "gdr2 segmented vs whole states")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdr2_varlen_edge_lengths(dtype):
    lens = [0, 1, 63, 64, 65, 130, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(dtype=dtype, H=2, T=int(cu[-1]) + 3, num_seqs=0,
                                        pin_frac=0.05, seed=6, gates="gdr2")
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(4).standard_normal((len(lens), 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    note(f"gdr2 varlen edges {dtype}")
    o, sT = run_chunk(x, dtype, o_fill=float("nan"))
    assert np.all(np.isnan(o[0, :, cu[-1]:])), "tokens outside every sequence were written"
    check_chains(x, o, sT, oracle_chains(x), TOL[dtype], f"gdr2 varlen edges {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdr2_with_beta_gates_matches_kda(dtype):
    """b = beta 1 and w = beta 1 reduce Gated Delta Rule-2 to KDA: both entry points agree
    (to the rounding of the bf16 operands, which the two paths form differently)."""
    cfg = KDA_B2_H16_T4096.replace(dtype=dtype, B=1, H=4, T=333, seed=13, random_s0=True)
    note(f"gdr2 = kda with beta gates {dtype}")
    x = make_chunk_inputs(cfg)
    o_kda, s_kda = run_chunk(x, dtype)
    x.erase = np.repeat(x.beta[..., None], cfg.dk, axis=-1)
    x.write = np.repeat(x.beta[..., None], cfg.dv, axis=-1)
    o_g, s_g = run_chunk(x, dtype)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert_close(o_g, o_kda, tol, f"outputs {dtype}")
    assert_close(s_g, s_kda, tol, f"states {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_gdr2_decode_small(dtype, gate, dk, dv):
    cfg = KDA_DECODE_N256_H32.replace(dtype=dtype, gate=gate, dk=dk, dv=dv, B=5, H=3, T=6, seed=31,
                                      gates="gdr2")
    note(f"gdr2 decode {dtype} {gate} dk={dk} dv={dv}")
    S0 = decode_initial_state(cfg)
    state = up(S0)
    ref = S0.astype(np.float64)
    for step in range(cfg.T):
        d = decode_step_inputs(cfg, step)
        o = kda.gdr2_recurrent_step(up(d.q, DT[dtype]), up(d.k, DT[dtype]), up(d.v, DT[dtype]),
                                    up(d.g), up(d.erase), up(d.write), state)
        ro, ref = oracle.kda_decode_step(ref, d.q, d.k, d.v, d.g, d.beta, erase=d.erase,
                                         write=d.write)
        assert_close(o.float().cpu().numpy(), ro, TOL[dtype], f"decode o step {step}")
    torch.cuda.synchronize()
    assert_close(state.cpu().numpy(), ref, TOL[dtype], "decode state")


def test_gdr2_decode_steps_equal_chunk_forward():
    """T decode steps on the same tokens equal one chunked forward (the state is the
    whole context), for the bf16 matrix-core chunk path."""
    B, H, T, dk, dv = 2, 4, 70, 128, 128
    cfg = KDA_B2_H16_T4096.replace(B=B, H=H, T=T, seed=55, random_s0=True, gates="gdr2")
    note("gdr2 decode steps vs chunk forward")
    x = make_chunk_inputs(cfg)
    o_chunk, s_chunk = run_chunk(x, "bf16")
    bf = torch.bfloat16
    state = up(x.s0)
    outs = []
    for t in range(T):
        sl = (slice(None), slice(None), t)
        outs.append(kda.gdr2_recurrent_step(
            up(x.q[sl], bf), up(x.k[sl], bf), up(x.v[sl], bf), up(x.g[sl]),
            up(x.erase[sl]), up(x.write[sl]), state).float().cpu().numpy())
    o_steps = np.stack(outs, axis=2)
    assert_close(o_steps, o_chunk, TOL["bf16"], "outputs")
    assert_close(state.cpu().numpy(), s_chunk, TOL["bf16"], "state")
