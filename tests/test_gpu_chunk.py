"""GPU parity of kda_chunk_fwd against the fp64 oracle (through the C ABI).

Full-size workloads: the tiny fp32 case, KDA B2 H16 T4096, GDN B1 H16 T8192 are
checked on every output and final state; the packed varlen T=65536 H32 case runs in
full on the GPU (the launch configuration the benchmark times) and is checked on all
its chains as well. Smaller cases
cover several chunks with a ragged tail for every dtype, gate mode and head size,
and the edge cases: empty and one-token sequences, lengths at and around the chunk
size, the decay floor g = -5 everywhere, no decay, beta = 0 and beta = 1.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
from kda_workloads import (GDN_B1_H16_T8192, KDA_B2_H16_T4096, KDA_VARLEN_H32_T65536,
                           TINY_KDA_F32, bf16_round, make_chunk_inputs)
from tests.gpu_util import (TOL, assert_close, check_chains, dev, note, oracle_chains,
                            run_chunk, up)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [TINY_KDA_F32, KDA_B2_H16_T4096, GDN_B1_H16_T8192],
                         ids=lambda c: c.name)
def test_workload_full_parity(cfg):
    note(f"chunk parity {cfg.name}")
    x = make_chunk_inputs(cfg)
    o, sT = run_chunk(x, cfg.dtype)
    ref = oracle_chains(x)
    eo, es = check_chains(x, o, sT, ref, TOL[cfg.dtype], cfg.name)
    print(f"{cfg.name}: normwise err o={eo:.2e} S={es:.2e}")


def test_varlen_t65536_all_chains():
    """The packed varlen T = 65536 workload in the benchmark's launch configuration (with
    its workspace: the segment plan): every output row is written, and all 256 chains
    match the oracle (checked eight heads at a time to bound the host memory)."""
    cfg = KDA_VARLEN_H32_T65536
    note(f"chunk parity {cfg.name} (all chains)")
    x = make_chunk_inputs(cfg)
    o, sT = run_chunk(x, cfg.dtype, o_fill=float("nan"))
    assert np.all(np.isfinite(o)), "some output position was not written"
    worst = (0.0, 0.0)
    for h0 in range(0, cfg.H, 8):
        chains = [(n, h) for n in range(x.n_seqs) for h in range(h0, min(h0 + 8, cfg.H))]
        eo, es = check_chains(x, o, sT, oracle_chains(x, chains), TOL["bf16"],
                              f"{cfg.name} heads {h0}..{h0 + 7}")
        worst = (max(worst[0], eo), max(worst[1], es))
    print(f"{cfg.name}: all {x.n_seqs * cfg.H} chains, err o={worst[0]:.2e} S={worst[1]:.2e}")


@pytest.mark.parametrize("ws_kind", ["work_list", "64MiB", "recommended", "1GiB"])
def test_varlen_t65536_within_given_workspace(ws_kind):
    """The packed varlen T = 65536 workload through the C ABI with workspaces of several sizes:
    the work list's size (the smallest accepted: no segments), 64 MiB (too small for the
    segments' matrices: the halves work list), the recommended size and 1 GiB (segments).
    Every call plans within what it is given; 8 heads of every sequence match the oracle."""
    cfg = KDA_VARLEN_H32_T65536
    x = make_chunk_inputs(cfg)
    dt = torch.bfloat16
    q, k, v, g, beta = up(x.q, dt), up(x.k, dt), up(x.v, dt), up(x.g), up(x.beta)
    cu = up(x.cu_seqlens, torch.int32)
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    N = x.n_seqs
    rec = kda.kda_chunk_fwd_workspace_size(B, H, T, dk, dv, N, kda.KDA_BF16)
    sizes = {"work_list": 4 * (1 + 2 * N * H), "64MiB": 64 << 20, "recommended": rec,
             "1GiB": 1 << 30}
    nbytes = -(-sizes[ws_kind] // 256) * 256
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    o = torch.full(tuple(x.v.shape), float("nan"), dtype=dt, device=dev())
    sT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev())
    note(f"chunk varlen T65536 with a {ws_kind} workspace ({nbytes} bytes)")
    st = kda.kda_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                           beta.data_ptr(), None, sT.data_ptr(), o.data_ptr(), cu.data_ptr(), N,
                           B, H, T, dk, dv, kda.KDA_BF16, kda.KDA_GATE_PER_CHANNEL,
                           ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    assert st == kda.KDA_OK, kda.kda_status_string(st)
    torch.cuda.synchronize()
    of = o.float().cpu().numpy()
    assert np.all(np.isfinite(of)), "some output position was not written"
    chains = [(n, h) for n in range(N) for h in range(0, H, 4)]
    check_chains(x, of, sT.cpu().numpy(), oracle_chains(x, chains, initial_state=False),
                 TOL["bf16"], f"varlen T65536, {ws_kind} workspace")


def test_workspace_below_the_work_list_is_rejected():
    """A packed call with a workspace below its work list's size is an argument error."""
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=4096)
    x = make_chunk_inputs(cfg)
    dt = torch.bfloat16
    q, k, v, g, beta = up(x.q, dt), up(x.k, dt), up(x.v, dt), up(x.g), up(x.beta)
    cu = up(x.cu_seqlens, torch.int32)
    B, H, T, dk = x.q.shape
    o = torch.empty(tuple(x.v.shape), dtype=dt, device=dev())
    ws = torch.empty(64, dtype=torch.uint8, device=dev())
    st = kda.kda_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                           beta.data_ptr(), None, None, o.data_ptr(), cu.data_ptr(), x.n_seqs,
                           B, H, T, dk, dk, kda.KDA_BF16, kda.KDA_GATE_PER_CHANNEL,
                           ws.data_ptr(), 64, torch.cuda.current_stream().cuda_stream)
    assert st == kda.KDA_ERR_INVALID_ARG


SMALL = []
for dtype in ("f32", "bf16"):
    for gate in ("channel", "head"):
        for dk, dv in ((64, 64), (128, 128), (64, 128), (128, 64)):
            SMALL.append((dtype, gate, dk, dv))


@pytest.mark.parametrize("dtype,gate,dk,dv", SMALL)
def test_small_ragged(dtype, gate, dk, dv):
    cfg = KDA_B2_H16_T4096.replace(dtype=dtype, gate=gate, dk=dk, dv=dv, B=2, H=3, T=200, seed=77)
    note(f"chunk small {dtype} {gate} dk={dk} dv={dv}")
    x = make_chunk_inputs(cfg)
    o, sT = run_chunk(x, dtype)
    check_chains(x, o, sT, oracle_chains(x), TOL[dtype], f"small {dtype} {gate} {dk}x{dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_edge_lengths(dtype):
    lens = [0, 1, 63, 64, 65, 130, 0, 7, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) + 5   # tokens past the last sequence must stay untouched
    cfg = KDA_VARLEN_H32_T65536.replace(dtype=dtype, H=2, T=T, num_seqs=0, pin_frac=0.05, seed=5)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(3).standard_normal((len(lens), 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    note(f"chunk varlen edges {dtype}")
    o, sT = run_chunk(x, dtype, o_fill=float("nan"))
    assert np.all(np.isnan(o[0, :, cu[-1]:])), "tokens outside every sequence were written"
    assert np.all(np.isfinite(o[0, :, :cu[-1]]))
    ref = oracle_chains(x)
    check_chains(x, o, sT, ref, TOL[dtype], f"varlen edges {dtype}")
    for n, ln in enumerate(lens):
        if ln == 0:   # an empty sequence returns its initial state
            np.testing.assert_array_equal(sT[n], x.s0[n])


@pytest.mark.parametrize("case", ["floor", "no_decay", "beta0", "beta1"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_gates(case, dtype):
    cfg = KDA_B2_H16_T4096.replace(dtype=dtype, B=1, H=2, T=300, seed=9)
    x = make_chunk_inputs(cfg)
    if case == "floor":
        x.g[...] = -5.0
    elif case == "no_decay":
        x.g[...] = 0.0
    elif case == "beta0":
        x.beta[...] = 0.0
    else:
        x.beta[...] = 1.0
    note(f"chunk degenerate {case} {dtype}")
    o, sT = run_chunk(x, dtype)
    check_chains(x, o, sT, oracle_chains(x), TOL[dtype], f"{case} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token(dtype):
    cfg = KDA_B2_H16_T4096.replace(dtype=dtype, B=3, H=2, T=1, seed=4)
    x = make_chunk_inputs(cfg)
    note(f"chunk T=1 {dtype}")
    o, sT = run_chunk(x, dtype)
    check_chains(x, o, sT, oracle_chains(x), TOL[dtype], f"T=1 {dtype}")


@pytest.mark.parametrize("mode", ["channel", "head", "gdr2"])
def test_correlated_keys(mode, norm=1.0):
    """Unit keys that point nearly the same way (a shared direction plus small noise) make
    the strictly lower part N of a block's (I + N) large (up to about 0.9), so the terms of
    the block inverse's product form grow and cancel; the results must still match the
    oracle."""
    cfg = KDA_B2_H16_T4096.replace(B=1, H=3, T=333, seed=31, gate="head" if mode == "head"
                                   else "channel", gates="gdr2" if mode == "gdr2" else "beta")
    x = make_chunk_inputs(cfg)
    rng = np.random.default_rng(99)
    base = rng.standard_normal((1, cfg.H, 1, cfg.dk))
    kk = base + 0.25 * rng.standard_normal(x.k.shape)
    kk = norm * kk / np.linalg.norm(kk, axis=-1, keepdims=True)
    x.k[...] = bf16_round(kk.astype(np.float32))
    if mode == "gdr2":
        x.erase[...] = np.maximum(x.erase, 0.9)
    else:
        x.beta[...] = np.maximum(x.beta, 0.8)
    note(f"chunk correlated keys |k| = {norm}, {mode}")
    o, sT = run_chunk(x, "bf16")
    check_chains(x, o, sT, oracle_chains(x), TOL["bf16"], f"correlated keys {mode} {norm}")


def test_split_resume_and_aliasing():
    """[0, T) in one call equals [0, T1) then [T1, T) resumed from the returned state;
    the resumed call passes the same buffer as initial and final state."""
    import gated_delta_rule_13_amd as kda
    cfg = KDA_B2_H16_T4096.replace(B=2, H=4, T=640, seed=21)
    x = make_chunk_inputs(cfg)
    dt = torch.bfloat16
    q, k, v, g, beta, s0 = (up(x.q, dt), up(x.k, dt), up(x.v, dt), up(x.g), up(x.beta),
                            up(x.s0))
    note("chunk split/resume")
    o_full, s_full = kda.chunk_fwd(q, k, v, g, beta, initial_state=s0)
    T1 = 197
    sl = lambda t, a, b: t[:, :, a:b].contiguous()  # noqa: E731
    state = s0.clone()
    o1, _ = kda.chunk_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1),
                          sl(beta, 0, T1), initial_state=state, final_state=state)
    o2, _ = kda.chunk_fwd(sl(q, T1, 640), sl(k, T1, 640), sl(v, T1, 640), sl(g, T1, 640),
                          sl(beta, T1, 640), initial_state=state, final_state=state)
    torch.cuda.synchronize()
    o_split = torch.cat([o1, o2], dim=2).float().cpu().numpy()
    assert_close(o_split, o_full.float().cpu().numpy(), 1e-2, "split outputs")
    assert_close(state.cpu().numpy(), s_full.cpu().numpy(), 1e-2, "split state")


def test_split_resume_and_aliasing_segmented():
    """The same with one long chain, so that every call is cut into segments: the first
    segment reads the initial state and the segment chain writes the final state into the
    same buffer; outputs and states match the one-call run and the oracle."""
    import gated_delta_rule_13_amd as kda
    cfg = KDA_B2_H16_T4096.replace(B=1, H=1, T=5000, seed=22, random_s0=True)
    x = make_chunk_inputs(cfg)
    dt = torch.bfloat16
    q, k, v, g, beta, s0 = (up(x.q, dt), up(x.k, dt), up(x.v, dt), up(x.g), up(x.beta),
                            up(x.s0))
    note("chunk split/resume, segmented")
    o_full, s_full = kda.chunk_fwd(q, k, v, g, beta, initial_state=s0)
    T1 = 2100
    sl = lambda t, a, b: t[:, :, a:b].contiguous()  # noqa: E731
    state = s0.clone()
    o1, _ = kda.chunk_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1),
                          sl(beta, 0, T1), initial_state=state, final_state=state)
    o2, _ = kda.chunk_fwd(sl(q, T1, 5000), sl(k, T1, 5000), sl(v, T1, 5000),
                          sl(g, T1, 5000), sl(beta, T1, 5000), initial_state=state,
                          final_state=state)
    torch.cuda.synchronize()
    o_split = torch.cat([o1, o2], dim=2).float().cpu().numpy()
    assert_close(o_split, o_full.float().cpu().numpy(), 1e-2, "split outputs")
    assert_close(state.cpu().numpy(), s_full.cpu().numpy(), 1e-2, "split state")
    check_chains(x, o_split, state.cpu().numpy(), oracle_chains(x), TOL["bf16"],
                 "split, segmented")


def test_deterministic():
    cfg = KDA_B2_H16_T4096.replace(B=2, H=4, T=1000, seed=8)
    x = make_chunk_inputs(cfg)
    note("chunk determinism")
    o1, s1 = run_chunk(x, "bf16")
    o2, s2 = run_chunk(x, "bf16")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("gates", ["beta", "gdr2"])
def test_deterministic_segment_plan(gates):
    """The packed varlen T = 65536 workload (all 32 heads for KDA, 8 for Gated Delta Rule-2)
    through the segment plan (planner, items, chain, corrections): two calls give
    bit-identical outputs and final states."""
    H = 32 if gates == "beta" else 8
    x = make_chunk_inputs(KDA_VARLEN_H32_T65536.replace(H=H, gates=gates))
    note(f"chunk determinism, segment plan ({gates})")
    o1, s1 = run_chunk(x, "bf16")
    o2, s2 = run_chunk(x, "bf16")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_gdn_equals_broadcast_kda():
    cfg = GDN_B1_H16_T8192.replace(H=4, T=700, seed=12)
    x = make_chunk_inputs(cfg)
    note("chunk GDN vs broadcast KDA")
    o1, s1 = run_chunk(x, "bf16")
    x.g = np.ascontiguousarray(np.repeat(x.g[..., None], cfg.dk, axis=-1))
    o2, s2 = run_chunk(x, "bf16")
    assert_close(o1, o2, 1e-2, "GDN vs KDA outputs")
    assert_close(s1, s2, 1e-2, "GDN vs KDA states")


@pytest.mark.parametrize("dv", [128, 64])
def test_schedule_is_bitwise_neutral(dv):
    """The work list (longest sequences first, value columns of the longest chains split
    over two workgroups) changes only where each column is computed, not how: outputs and
    final states equal the one-workgroup-per-chain run bit for bit, and match the oracle."""
    # 6 sequences x 48 heads: on a 256-CU device the planner splits the value columns of
    # the longest chains (its bound for segments is 11% higher), so no segments are cut
    lens = [957, 795, 643, 621, 513, 494]
    H = 48
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=H, T=int(cu[-1]), dv=dv, num_seqs=0, pin_frac=0.05,
                                        seed=21)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(8).standard_normal((len(lens), H, 128, dv)).astype(
        np.float32) * np.float32(0.02)
    note(f"chunk schedule neutrality dv={dv}")
    o1, s1 = run_chunk(x, "bf16", schedule=True)
    o0, s0 = run_chunk(x, "bf16", schedule=False)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(s1, s0)
    check_chains(x, o1, s1, oracle_chains(x), TOL["bf16"], f"scheduled dv={dv}")


SEG_CASES = [  # (name, lens or None for equal lengths, B, H, T, dv, gate)
    ("varlen_dv128", [3000, 90, 700, 0, 1300, 33, 64], 1, 4, None, 128, "channel"),
    ("varlen_dv64_head", [2500, 513, 511, 1700], 1, 3, None, 64, "head"),
    ("equal_b2_h2", None, 2, 2, 2100, 128, "channel"),
    # one chain: about twenty segments, a chain of that many steps and many correction units
    ("one_long_h1", [20000], 1, 1, None, 128, "channel"),
    # one decay per head; sequences of 1 and 0 tokens among cut ones
    ("varlen_head_gate", [5000, 4000, 64, 1, 0, 2500], 1, 2, None, 128, "head"),
]


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: c[0])
def test_segmented_matches_oracle_and_whole_chains(case):
    """Few chains for the device: long sequences are cut into segments. dv = 128: the later
    segments run from the zero state and as transitions, the start states are chained and
    the outputs corrected; dv = 64: every segment is re-run from its exact start state.
    Outputs and final states match the oracle, and the whole-chain run to rounding."""
    name, lens, B, H, T, dv, gate = case
    if lens is not None:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        cfg = KDA_VARLEN_H32_T65536.replace(H=H, T=int(cu[-1]), dv=dv, gate=gate, num_seqs=0,
                                            pin_frac=0.05, seed=23)
    else:
        cfg = KDA_B2_H16_T4096.replace(B=B, H=H, T=T, dv=dv, gate=gate, seed=23, random_s0=True)
    x = make_chunk_inputs(cfg)
    if lens is not None:
        x.cu_seqlens = cu
        x.s0 = np.random.default_rng(9).standard_normal((len(lens), H, 128, dv)).astype(
            np.float32) * np.float32(0.02)
    ns = x.n_seqs if lens is not None else 0
    ws = kda.kda_chunk_fwd_workspace_size(x.q.shape[0], H, x.q.shape[2], 128, dv, ns,
                                          kda.KDA_BF16)
    assert ws > 128 * 128 * 4, f"{name}: expected the segmented path"
    note(f"segmented chunk {name}")
    o1, s1 = run_chunk(x, "bf16", schedule=True)
    o0, s0 = run_chunk(x, "bf16", schedule=False)
    check_chains(x, o1, s1, oracle_chains(x), TOL["bf16"], f"segmented {name}")
    assert_close(o1, o0, TOL["bf16"], f"{name}: segmented vs whole outputs")
    assert_close(s1, s0, TOL["bf16"], f"{name}: segmented vs whole states")


def test_segmented_without_initial_or_final_state():
    """The segment plan with no initial state (the first segment starts from zero) and no
    final state requested (the segment chain writes none): outputs match the oracle."""
    lens = [6000, 2500, 700]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=int(cu[-1]), num_seqs=0, pin_frac=0.05, seed=31)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = None
    note("segmented chunk without initial / final state")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16)
               for a in (x.q, x.k, x.v))
    g, beta = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in (x.g, x.beta))
    o, sT = kda.chunk_fwd(q, k, v, g, beta, cu_seqlens=torch.from_numpy(cu).to("cuda"),
                          output_final_state=False)
    torch.cuda.synchronize()
    assert sT is None
    ref = oracle_chains(x, initial_state=False)
    on = o.float().cpu().numpy()
    got = [on[b, h, t0:t0 + ln] for (n, h) in ref for (b, t0, ln) in [x.chain_rows(n, h)]]
    assert_close(np.concatenate(got), np.concatenate([ro for ro, _ in ref.values()]),
                 TOL["bf16"], "segmented, no states: outputs")


def test_segmented_one_long_among_many():
    """300 packed sequences, 299 of 64 tokens and at index 287 one of 20,000 tokens, which the
    planner cuts into many segments: the 1024-thread planner, a segment chain of many steps,
    and the final-state step of the corrections launch, which finds the one cut sequence
    among hundreds. Every chain matches the oracle and the whole-chain run."""
    lens = [64] * 300
    lens[287] = 20000
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    ws = kda.kda_chunk_fwd_workspace_size(1, 2, T, 128, 128, len(lens), kda.KDA_BF16)
    assert ws > kda.kda_chunk_fwd_workspace_size(1, 2, T, 128, 64, len(lens), kda.KDA_BF16), \
        "expected the segment plan"
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=T, num_seqs=0, pin_frac=0.05, seed=41)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(42).standard_normal((len(lens), 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    note("segmented chunk: one long sequence among 300")
    o1, s1 = run_chunk(x, "bf16", o_fill=float("nan"))
    assert np.all(np.isfinite(o1)), "some output position was not written"
    o0, s0 = run_chunk(x, "bf16", schedule=False)
    check_chains(x, o1, s1, oracle_chains(x), TOL["bf16"], "one long among 300")
    assert_close(o1, o0, TOL["bf16"], "one long among 300: segmented vs whole outputs")
    assert_close(s1, s0, TOL["bf16"], "one long among 300: segmented vs whole states")


RANDOM_SHAPES = list(range(40))


@pytest.mark.parametrize("case", RANDOM_SHAPES)
def test_random_packed_shapes(case):
    """Seeded random packed batches (1 to 12 sequences of 0 to 6000 tokens, 1 to 8 heads,
    dv 64 or 128, per-channel or per-head decay, KDA or Gated Delta Rule-2 gates, with or
    without an initial state) through the scheduled path: whatever the planner picks
    (halves, segments, or neither), every chain matches the oracle."""
    rng = np.random.default_rng(1000 + case)
    n = int(rng.integers(1, 13))
    lens = [int(v) for v in rng.integers(0, 6001, size=n)]
    if sum(lens) == 0:
        lens[0] = 1
    H = int(rng.choice([1, 2, 3, 5, 8]))
    dv = int(rng.choice([64, 128]))
    gate = str(rng.choice(["channel", "head"]))
    gates = str(rng.choice(["beta", "gdr2"]))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=H, T=int(cu[-1]), dv=dv, gate=gate, num_seqs=0,
                                        pin_frac=0.05, seed=2000 + case, gates=gates)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    if rng.random() < 0.5:
        x.s0 = rng.standard_normal((n, H, 128, dv)).astype(np.float32) * np.float32(0.02)
    else:
        x.s0 = None
    note(f"random packed case {case}: lens={lens} H={H} dv={dv} {gate} {gates}")
    o, sT = run_chunk(x, "bf16", o_fill=float("nan"))
    assert np.all(np.isfinite(o)), "some output position was not written"
    check_chains(x, o, sT, oracle_chains(x), TOL["bf16"], f"random case {case}")


def test_more_sequences_than_one_plan_sorts():
    """1,100 packed sequences of 0 to 40 tokens (more than the 1,024 that one planning
    workgroup sorts): no workspace is asked for, the chains run one workgroup each in chain
    order, every output row is written and every chain matches the oracle."""
    rng = np.random.default_rng(77)
    lens = [int(v) for v in rng.integers(0, 41, size=1100)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    assert kda.kda_chunk_fwd_workspace_size(1, 2, T, 128, 128, len(lens), kda.KDA_BF16) == 0
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=T, num_seqs=0, pin_frac=0.05, seed=78)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = rng.standard_normal((len(lens), 2, 128, 128)).astype(np.float32) * np.float32(0.02)
    note("chunk with 1100 packed sequences")
    o, sT = run_chunk(x, "bf16", o_fill=float("nan"))
    assert np.all(np.isfinite(o)), "some output position was not written"
    check_chains(x, o, sT, oracle_chains(x), TOL["bf16"], "1100 sequences")


@pytest.mark.parametrize("T", [(1 << 22) - 64, (1 << 22) + 64], ids=["bf16-whole-chains", "fp32"])
def test_longest_t_axis(T):
    """The longest T axis the bf16 kernel takes with whole-chain items (a chain's per-channel
    decay, T x dk fp32, must stay under 2^31 bytes: T < 2^22) and one just past it, which
    (about 14,000 packed sequences, more than one segment plan holds) the fp32 matrix-core
    kernel takes, as packed sequences of 200 to 400 tokens: sampled sequences at the start,
    the middle and the end of the axis (byte offsets past 2^31) match the oracle. The inputs
    are a 65,536-token draw repeated along T."""
    rng = np.random.default_rng(92)
    lens = []
    while sum(lens) < T:
        lens.append(int(rng.integers(200, 401)))
    lens[-1] -= sum(lens) - T
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    base = make_chunk_inputs(KDA_VARLEN_H32_T65536.replace(H=1, T=65536, num_seqs=0,
                                                           pin_frac=0.05, seed=93))
    reps = -(-T // 65536)
    x = base
    for name in ("q", "k", "v", "g"):
        tiled = np.tile(getattr(base, name), (1, 1, reps, 1))[:, :, :T]
        setattr(x, name, np.ascontiguousarray(tiled))
    x.beta = np.ascontiguousarray(np.tile(base.beta, (1, 1, reps))[:, :, :T])
    x.cu_seqlens = cu
    x.s0 = None
    n = len(lens)
    note(f"chunk longest T axis {T}: {n} sequences")
    o, sT = run_chunk(x, "bf16")
    sample = [0, 1, n // 2, n // 2 + 1, n - 3, n - 2, n - 1]
    ref = oracle_chains(x, chains=[(i, 0) for i in sample], initial_state=False)
    check_chains(x, o, sT, ref, TOL["bf16"], f"T = {T}")


def test_forward_in_a_replayed_graph():
    """The segment plan's launches (planner, items, chain, corrections) captured once in a
    HIP graph and replayed three times, with eager work and synchronisations between the
    replays: every replay gives the eager outputs and final states bit for bit."""
    lens = [20000, 3000, 500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=int(cu[-1]), num_seqs=0, pin_frac=0.05, seed=98)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(99).standard_normal((3, 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    ws = kda.kda_chunk_fwd_workspace_size(1, 2, int(cu[-1]), 128, 128, 3, kda.KDA_BF16)
    assert ws > 128 * 128 * 4, "expected the segment plan"
    note("chunk forward in a HIP graph")
    bf = torch.bfloat16
    q, k, v = up(x.q, bf), up(x.k, bf), up(x.v, bf)
    g, beta, s0 = up(x.g), up(x.beta), up(x.s0)
    cut = up(cu, torch.int32)
    o = torch.empty(tuple(x.v.shape), dtype=bf, device=q.device)
    sT = torch.empty((3, 2, 128, 128), dtype=torch.float32, device=q.device)
    kda.chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cut, o=o, final_state=sT)
    torch.cuda.synchronize()
    want_o, want_s = o.clone(), sT.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cut, o=o, final_state=sT)
    for rep in range(3):
        o.fill_(float("nan"))
        sT.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), f"replay {rep}: outputs differ"
        assert torch.equal(sT, want_s), f"replay {rep}: final states differ"
