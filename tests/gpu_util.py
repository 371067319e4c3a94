"""Helpers of the GPU parity tests: upload seeded inputs, call the C ABI through the
binding, and compare with the fp64 oracle under the normwise tolerance
max |got - want| <= tol * max |want|, applied to outputs and to final states
separately (2e-2 for bf16 inputs with fp32 accumulation, 1e-4 for fp32 inputs)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import gated_delta_rule_13_amd as kda
import oracle

TOL = {"bf16": 2e-2, "f32": 1e-4}
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def note(msg: str) -> None:
    """Names the case before a GPU step, so a failure can be traced."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev():
    return torch.device("cuda:0")


def up(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev(), dtype)


def normwise_err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    scale = np.max(np.abs(want)) if want.size else 0.0
    return float(np.max(np.abs(got - want)) / scale) if scale > 0 else float(np.max(np.abs(got)))


def assert_close(got, want, tol, what):
    e = normwise_err(got, want)
    assert e <= tol, f"{what}: normwise error {e:.3e} > {tol:.1e}"
    return e


def run_chunk(x, dtype: str, initial_state=True, o_fill=None, schedule=True):
    """Runs kda_chunk_fwd on inputs ``x`` (kda_workloads.ChunkInputs).
    Returns (o float32 numpy [B,H,T,dv], final state numpy [N,H,dk,dv])."""
    dt = DT[dtype]
    q, k, v = up(x.q, dt), up(x.k, dt), up(x.v, dt)
    g, beta = up(x.g), up(x.beta)
    s0 = up(x.s0) if (initial_state and x.s0 is not None) else None
    cu = up(x.cu_seqlens, torch.int32) if x.cu_seqlens is not None else None
    o = None
    if o_fill is not None:
        o = torch.full(tuple(x.v.shape), o_fill, dtype=dt, device=dev())
    if x.erase is not None:   # Gated Delta Rule-2 gates
        o, sT = kda.gdr2_chunk_fwd(q, k, v, g, up(x.erase), up(x.write), initial_state=s0,
                                   cu_seqlens=cu, o=o, schedule=schedule)
    else:
        o, sT = kda.chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu, o=o,
                              schedule=schedule)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), sT.cpu().numpy()


def oracle_chains(x, chains=None, initial_state=True):
    return oracle.kda_forward(x.q, x.k, x.v, x.g, x.beta,
                              s0=x.s0 if initial_state else None,
                              cu_seqlens=x.cu_seqlens, chains=chains,
                              erase=x.erase, write=x.write)


def check_chains(x, o, sT, ref, tol, what):
    """Compares the chains in ``ref`` ({(n, h): (o, S)}) with the GPU result."""
    got_o, want_o, got_s, want_s = [], [], [], []
    for (n, h), (ro, rs) in ref.items():
        b, t0, ln = x.chain_rows(n, h)
        got_o.append(o[b, h, t0:t0 + ln])
        want_o.append(ro)
        got_s.append(sT[n, h])
        want_s.append(rs)
    eo = assert_close(np.concatenate(got_o), np.concatenate(want_o), tol, f"{what} outputs")
    es = assert_close(np.stack(got_s), np.stack(want_s), tol, f"{what} final states")
    return eo, es
