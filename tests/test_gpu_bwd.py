"""GPU parity of the backward pass (kda_chunk_bwd) against the fp64 backward oracle
(oracle/kda_oracle_bwd.c, itself pinned to finite differences of the forward), through
the C ABI.

Every gradient (dq, dk, dv, dg, dbeta, dS0) is compared chain by chain with the normwise
bound max |got - want| <= 2e-2 max |want| of bf16 inputs with fp32 accumulation, each
tensor separately. Checked: both gate modes and value head sizes on ragged sequences with
and without an initial state and a final-state cotangent; key head size 64 (the dk = 128
kernels on zero-padded key channels); sequence lengths around the
16- and 64-token block edges (packed); the B2 H16 T4096 workload in full; the packed
H32 T65536 workload on all 256 chains; tokens outside every sequence left untouched; and
the Gated Delta Rule-2 backward (erase and write gates: their gradients replace dbeta), on
the packed H32 T65536 workload for every sequence on two heads.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
import oracle
from kda_workloads import (GDN_B1_H16_T8192, KDA_B2_H16_T4096, KDA_VARLEN_H32_T65536,
                           make_chunk_inputs, make_cotangents)
from tests.gpu_util import TOL, assert_close, note, up

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def run_bwd(x, ct, initial_state=True, final_cotangent=True, fill=None):
    bf = torch.bfloat16
    q, k, v, do = up(x.q, bf), up(x.k, bf), up(x.v, bf), up(ct.do, bf)
    s0 = up(x.s0) if (initial_state and x.s0 is not None) else None
    dsT = up(ct.dsT) if final_cotangent else None
    cu = up(x.cu_seqlens, torch.int32) if x.cu_seqlens is not None else None
    if fill is None:
        out = kda.chunk_bwd(q, k, v, up(x.g), up(x.beta), do, initial_state=s0,
                            grad_final_state=dsT, cu_seqlens=cu)
    else:   # pre-filled outputs through the raw entry point (untouched-token check)
        B, H, T, dk = x.q.shape
        dv = x.v.shape[-1]
        outs = [torch.full(x.q.shape, fill, dtype=bf, device=q.device) for _ in range(2)]
        outs.append(torch.full(x.v.shape, fill, dtype=bf, device=q.device))
        outs.append(torch.full(x.g.shape, fill, dtype=torch.float32, device=q.device))
        outs.append(torch.full(x.beta.shape, fill, dtype=torch.float32, device=q.device))
        N = x.n_seqs
        ds0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
        ns = 0 if cu is None else N
        gm = kda.KDA_GATE_PER_CHANNEL if x.g.ndim == 4 else kda.KDA_GATE_PER_HEAD
        wsb = kda.kda_chunk_bwd_workspace_size(B, H, T, dk, dv, ns, kda.KDA_BF16)
        ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
        g, beta = up(x.g), up(x.beta)
        st = kda.kda_chunk_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                               beta.data_ptr(), s0.data_ptr() if s0 is not None else None,
                               do.data_ptr(), dsT.data_ptr() if dsT is not None else None,
                               *[o.data_ptr() for o in outs], ds0.data_ptr(),
                               cu.data_ptr() if cu is not None else None, ns, B, H, T, dk, dv,
                               kda.KDA_BF16, gm, ws.data_ptr(), wsb,
                               torch.cuda.current_stream().cuda_stream)
        assert st == kda.KDA_OK, kda.kda_status_string(st)
        out = (*outs, ds0)
    torch.cuda.synchronize()
    return {name: t.float().cpu().numpy() for name, t in zip(NAMES + ("ds0",), out)}


def oracle_grads(x, ct, chains=None, initial_state=True, final_cotangent=True):
    return oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, ct.do,
                               s0=x.s0 if initial_state else None,
                               dsT=ct.dsT if final_cotangent else None,
                               cu_seqlens=x.cu_seqlens, chains=chains)


def check(x, got, ref, what, tol=TOL["bf16"]):
    errs = {}
    for name in NAMES + ("ds0",):
        g_parts, w_parts = [], []
        for (n, h), r in ref.items():
            if name == "ds0":
                g_parts.append(got["ds0"][n, h])
            else:
                b, t0, ln = x.chain_rows(n, h)
                g_parts.append(got[name][b, h, t0:t0 + ln])
            w_parts.append(r[name])
        gg = np.concatenate([a.ravel() for a in g_parts])
        ww = np.concatenate([a.ravel() for a in w_parts])
        errs[name] = assert_close(gg, ww, tol, f"{what}: {name}")
    return errs


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dv", [128, 64])
def test_bwd_small_ragged(gate, dv):
    cfg = KDA_B2_H16_T4096.replace(gate=gate, dv=dv, B=2, H=3, T=200, seed=81, random_s0=True)
    note(f"bwd small {gate} dv={dv}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    errs = check(x, run_bwd(x, ct), oracle_grads(x, ct), f"bwd {gate} dv={dv}")
    print({k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("initial_state,final_cotangent", [(False, False), (True, False),
                                                            (False, True)])
def test_bwd_optional_states(initial_state, final_cotangent):
    cfg = KDA_B2_H16_T4096.replace(B=1, H=2, T=150, seed=82, random_s0=True)
    note(f"bwd s0={initial_state} dsT={final_cotangent}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    got = run_bwd(x, ct, initial_state, final_cotangent)
    check(x, got, oracle_grads(x, ct, initial_state=initial_state,
                               final_cotangent=final_cotangent), "bwd optional states")


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_bwd_varlen_edge_lengths(gate):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 130, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(gate=gate, H=2, T=int(cu[-1]) + 5, num_seqs=0,
                                        pin_frac=0.05, seed=83)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(8).standard_normal((len(lens), 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, len(lens))
    note(f"bwd varlen edges {gate}")
    got = run_bwd(x, ct, fill=float("nan"))
    for name in NAMES:
        tail = got[name][0, :, cu[-1]:]
        assert np.all(np.isnan(tail)), f"{name}: tokens outside every sequence were written"
    check(x, got, oracle_grads(x, ct), f"bwd varlen edges {gate}")


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dv", [128, 64])
def test_bwd_dk64_small_ragged(gate, dv):
    """dk = 64 (the dk = 128 kernels on copies padded with zero key channels): every gradient
    of ragged sequences with an initial state and a final-state cotangent matches the oracle,
    which runs at dk = 64."""
    cfg = KDA_B2_H16_T4096.replace(gate=gate, dk=64, dv=dv, B=2, H=3, T=200, seed=86,
                                   random_s0=True)
    note(f"bwd dk=64 small {gate} dv={dv}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    errs = check(x, run_bwd(x, ct), oracle_grads(x, ct), f"bwd dk=64 {gate} dv={dv}")
    print({k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_bwd_dk64_varlen_edge_lengths(gate):
    """dk = 64, packed sequences around the block edges, through the raw entry point with
    pre-filled outputs: tokens outside every sequence keep their values through the padded
    copies, and every chain matches the oracle."""
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 130, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(gate=gate, dk=64, dv=128, H=2, T=int(cu[-1]) + 5,
                                        num_seqs=0, pin_frac=0.05, seed=87)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(11).standard_normal((len(lens), 2, 64, 128)).astype(
        np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, len(lens))
    note(f"bwd dk=64 varlen edges {gate}")
    got = run_bwd(x, ct, fill=float("nan"))
    for name in NAMES:
        tail = got[name][0, :, cu[-1]:]
        assert np.all(np.isnan(tail)), f"{name}: tokens outside every sequence were written"
    check(x, got, oracle_grads(x, ct), f"bwd dk=64 varlen edges {gate}")


def test_bwd_dk64_b2_h16_t4096():
    """dk = 64 at B2 H16 T4096 (dv = 128): every chain matches the oracle."""
    cfg = KDA_B2_H16_T4096.replace(name="kda_bf16_dk64_b2_h16_t4096", dk=64, seed=88)
    note(f"bwd parity {cfg.name}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    errs = check(x, run_bwd(x, ct), oracle_grads(x, ct), cfg.name)
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_b2_h16_t4096_full():
    cfg = KDA_B2_H16_T4096
    note(f"bwd parity {cfg.name}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    errs = check(x, run_bwd(x, ct), oracle_grads(x, ct), cfg.name)
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_gdn_b1_h16_t8192_all_chains():
    cfg = GDN_B1_H16_T8192
    note(f"bwd parity {cfg.name} (all chains)")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    errs = check(x, run_bwd(x, ct), oracle_grads(x, ct), cfg.name)
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_varlen_t65536_all_chains():
    """All 256 chains of the packed T = 65536 workload (in the benchmark's launch
    configuration), checked against the oracle eight heads at a time to bound host memory."""
    cfg = KDA_VARLEN_H32_T65536
    note(f"bwd parity {cfg.name} (all chains)")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    got = run_bwd(x, ct)
    worst = {}
    for h0 in range(0, cfg.H, 8):
        chains = [(n, h) for n in range(x.n_seqs) for h in range(h0, h0 + 8)]
        errs = check(x, got, oracle_grads(x, ct, chains), f"{cfg.name} heads {h0}..{h0 + 7}")
        worst = {k: max(v, worst.get(k, 0.0)) for k, v in errs.items()}
    print(cfg.name, "all chains", {k: f"{v:.2e}" for k, v in worst.items()})


@pytest.mark.parametrize("case", range(16))
def test_bwd_random_packed_shapes(case):
    """Seeded random packed batches (1 to 8 sequences of 0 to 2500 tokens, 1 to 4 heads, dv
    64 or 128, per-channel or per-head decay, with or without an initial state and a
    final-state cotangent): every chain's gradients match the oracle."""
    rng = np.random.default_rng(3000 + case)
    n = int(rng.integers(1, 9))
    lens = [int(v) for v in rng.integers(0, 2501, size=n)]
    if sum(lens) == 0:
        lens[0] = 1
    H = int(rng.integers(1, 5))
    dv = int(rng.choice([64, 128]))
    gate = str(rng.choice(["channel", "head"]))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=H, T=int(cu[-1]), dv=dv, gate=gate, num_seqs=0,
                                        pin_frac=0.05, seed=4000 + case)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = rng.standard_normal((n, H, 128, dv)).astype(np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, n)
    init, fin = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    note(f"bwd random case {case}: lens={lens} H={H} dv={dv} {gate} s0={init} dsT={fin}")
    errs = check(x, run_bwd(x, ct, initial_state=init, final_cotangent=fin),
                 oracle_grads(x, ct, initial_state=init, final_cotangent=fin),
                 f"bwd random case {case}")
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_more_sequences_than_one_plan_sorts():
    """1,100 packed sequences of 0 to 30 tokens (more than one planning workgroup sorts):
    the workspace holds the two histories only, the chain passes run in chain order, and
    every chain's gradients match the oracle."""
    rng = np.random.default_rng(79)
    lens = [int(v) for v in rng.integers(0, 31, size=1100)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    one = kda.kda_chunk_bwd_workspace_size(1, 1, T, 128, 128, len(lens), kda.KDA_BF16)
    cfg = KDA_VARLEN_H32_T65536.replace(H=1, T=T, num_seqs=0, pin_frac=0.05, seed=80)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = rng.standard_normal((len(lens), 1, 128, 128)).astype(np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, len(lens))
    note(f"bwd with 1100 packed sequences (workspace {one} bytes)")
    errs = check(x, run_bwd(x, ct), oracle_grads(x, ct), "bwd 1100 sequences")
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_longest_t_axis():
    """The longest T axis the backward takes at dv = 128 (one chain's bf16 history, one
    matrix per pair of blocks, (T + 64) x 8 x dv bytes, must stay under 2^31: T = 2^21 - 65),
    as packed sequences of 200 to 400 tokens: sampled sequences at the start, the middle and
    the end of the axis match the oracle. The inputs are a 65,536-token draw repeated
    along T."""
    T = (1 << 21) - 65
    rng = np.random.default_rng(94)
    lens = []
    while sum(lens) < T:
        lens.append(int(rng.integers(200, 401)))
    lens[-1] -= sum(lens) - T
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=1, T=65536, num_seqs=0, pin_frac=0.05, seed=95)
    x = make_chunk_inputs(cfg)
    reps = -(-T // 65536)
    for name in ("q", "k", "v", "g"):
        tiled = np.tile(getattr(x, name), (1, 1, reps, 1))[:, :, :T]
        setattr(x, name, np.ascontiguousarray(tiled))
    x.beta = np.ascontiguousarray(np.tile(x.beta, (1, 1, reps))[:, :, :T])
    x.cu_seqlens = cu
    x.s0 = None
    n = len(lens)
    ct = make_cotangents(cfg.replace(T=T), n)
    note(f"bwd longest T axis {T}: {n} sequences")
    got = run_bwd(x, ct)
    sample = [(i, 0) for i in (0, 1, n // 2, n // 2 + 1, n - 3, n - 2, n - 1)]
    errs = check(x, got, oracle_grads(x, ct, chains=sample), f"bwd T = {T}")
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_deterministic():
    """Packed sequences through the three launches (the state history on the second stream
    beside the reverse carry): two calls give bit-identical gradients."""
    lens = [9000, 4100, 2500, 777, 64, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=4, T=int(cu[-1]), num_seqs=0, pin_frac=0.05, seed=96)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(97).standard_normal((len(lens), 4, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, len(lens))
    note("bwd determinism")
    a, b = run_bwd(x, ct), run_bwd(x, ct)
    for name in NAMES + ("ds0",):
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def test_bwd_in_a_replayed_graph():
    """The backward's launches (work list, state history on the second stream beside the
    reverse carry, gradients) captured once in a HIP graph and replayed three times, with
    eager work and synchronisations between the replays: every replay gives the eager
    gradients bit for bit."""
    lens = [3000, 1100, 65, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=int(cu[-1]), num_seqs=0, pin_frac=0.05, seed=100)
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(101).standard_normal((len(lens), 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, len(lens))
    note("bwd in a HIP graph")
    bf = torch.bfloat16
    args = (up(x.q, bf), up(x.k, bf), up(x.v, bf), up(x.g), up(x.beta), up(ct.do, bf))
    kw = dict(initial_state=up(x.s0), grad_final_state=up(ct.dsT),
              cu_seqlens=up(cu, torch.int32))
    want = [t.clone() for t in kda.chunk_bwd(*args, **kw)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = kda.chunk_bwd(*args, **kw)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, w in zip(NAMES + ("ds0",), outs, want):
            assert torch.equal(got, w), f"replay {rep}: {name} differs"


def test_bwd_on_two_streams_at_once():
    """Two backward calls enqueued back to back on two streams of the device, which share
    the library's second stream for their state histories: each gives the gradients of the
    same call run alone, bit for bit."""
    cases = []
    for i, lens in enumerate(([2500, 700, 64], [1800, 1800, 5, 300])):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=int(cu[-1]), num_seqs=0, pin_frac=0.05,
                                            seed=102 + i)
        x = make_chunk_inputs(cfg)
        ct = make_cotangents(cfg, len(lens))
        bf = torch.bfloat16
        args = (up(x.q, bf), up(x.k, bf), up(x.v, bf), up(x.g), up(x.beta), up(ct.do, bf))
        kw = dict(grad_final_state=up(ct.dsT), cu_seqlens=up(cu, torch.int32))
        cases.append((args, kw))
    note("bwd on two streams")
    alone = []
    for args, kw in cases:
        alone.append([t.clone() for t in kda.chunk_bwd(*args, **kw)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (args, kw), st in zip(cases, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(kda.chunk_bwd(*args, **kw))
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(outs, alone)):
        for name, a, b in zip(NAMES + ("ds0",), got, want):
            assert torch.equal(a, b), f"call {i}: {name} differs"


GDR2_NAMES = ("dq", "dk", "dv", "dg", "derase", "dwrite", "ds0")


def run_gdr2_bwd(x, ct):
    bf = torch.bfloat16
    cu = up(x.cu_seqlens, torch.int32) if x.cu_seqlens is not None else None
    out = kda.gdr2_chunk_bwd(up(x.q, bf), up(x.k, bf), up(x.v, bf), up(x.g), up(x.erase),
                             up(x.write), up(ct.do, bf),
                             initial_state=up(x.s0) if x.s0 is not None else None,
                             grad_final_state=up(ct.dsT), cu_seqlens=cu)
    torch.cuda.synchronize()
    return {name: t.float().cpu().numpy() for name, t in zip(GDR2_NAMES, out)}


def check_gdr2(x, got, ref, what):
    errs = {}
    for name in GDR2_NAMES:
        g_parts, w_parts = [], []
        for (n, h), r in ref.items():
            if name == "ds0":
                g_parts.append(got["ds0"][n, h])
            else:
                b, t0, ln = x.chain_rows(n, h)
                g_parts.append(got[name][b, h, t0:t0 + ln])
            w_parts.append(r[name])
        errs[name] = assert_close(np.concatenate([a.ravel() for a in g_parts]),
                                  np.concatenate([a.ravel() for a in w_parts]), TOL["bf16"],
                                  f"{what}: {name}")
    return errs


@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dv", [128, 64])
def test_gdr2_bwd_small_ragged(gate, dv, dk):
    cfg = KDA_B2_H16_T4096.replace(gate=gate, dk=dk, dv=dv, B=2, H=3, T=200, seed=84,
                                   random_s0=True, gates="gdr2")
    note(f"gdr2 bwd small {gate} dk={dk} dv={dv}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    ref = oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, ct.do, s0=x.s0, dsT=ct.dsT,
                              erase=x.erase, write=x.write)
    errs = check_gdr2(x, run_gdr2_bwd(x, ct), ref, f"gdr2 bwd {gate} dk={dk} dv={dv}")
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_gdr2_bwd_varlen_edges():
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 130, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = KDA_VARLEN_H32_T65536.replace(H=2, T=int(cu[-1]) + 5, num_seqs=0, pin_frac=0.05, seed=85,
                                        gates="gdr2")
    x = make_chunk_inputs(cfg)
    x.cu_seqlens = cu
    x.s0 = np.random.default_rng(10).standard_normal((len(lens), 2, 128, 128)).astype(
        np.float32) * np.float32(0.02)
    ct = make_cotangents(cfg, len(lens))
    note("gdr2 bwd varlen edges")
    ref = oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, ct.do, s0=x.s0, dsT=ct.dsT,
                              cu_seqlens=cu, erase=x.erase, write=x.write)
    check_gdr2(x, run_gdr2_bwd(x, ct), ref, "gdr2 bwd varlen edges")


def test_gdr2_bwd_b2_h16_t4096_full():
    cfg = KDA_B2_H16_T4096.replace(name="gdr2_bf16_b2_h16_t4096", gates="gdr2")
    note(f"gdr2 bwd parity {cfg.name}")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    ref = oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, ct.do, s0=x.s0, dsT=ct.dsT,
                              erase=x.erase, write=x.write)
    errs = check_gdr2(x, run_gdr2_bwd(x, ct), ref, cfg.name)
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_gdr2_bwd_varlen_t65536_every_sequence():
    """The Gated Delta Rule-2 backward on the packed T = 65536 workload (the shape the
    benchmark times): every sequence on two heads (16 chains) against the oracle."""
    cfg = KDA_VARLEN_H32_T65536.replace(name="gdr2_bf16_varlen_h32_t65536", gates="gdr2")
    note(f"gdr2 bwd parity {cfg.name} (two heads of every sequence)")
    x = make_chunk_inputs(cfg)
    ct = make_cotangents(cfg, x.n_seqs)
    chains = [(n, (5 * n + j * 17) % cfg.H) for n in range(x.n_seqs) for j in range(2)]
    got = run_gdr2_bwd(x, ct)
    ref = oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, ct.do, s0=None, dsT=ct.dsT,
                              cu_seqlens=x.cu_seqlens, chains=chains, erase=x.erase,
                              write=x.write)
    errs = check_gdr2(x, got, ref, cfg.name)
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})
