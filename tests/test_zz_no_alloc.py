"""kda_chunk_fwd_noalloc (the forward without a workspace argument, for callers that cannot
allocate) against kda_chunk_fwd with its recommended workspace, through the C ABI: two calls
in a row on the library's shared scratch array, the second with a smaller input, each within
the bf16 tolerance (normwise 2e-2) of the workspace call and of the oracle."""

import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as kda
from kda_workloads import KDA_B2_H16_T4096, KDA_VARLEN_H32_T65536, make_chunk_inputs
from tests.gpu_util import TOL, assert_close, check_chains, dev, note, oracle_chains, up

pytestmark = pytest.mark.gpu


def call(x, noalloc):
    bf = torch.bfloat16
    q, k, v, g, beta = up(x.q, bf), up(x.k, bf), up(x.v, bf), up(x.g), up(x.beta)
    s0 = up(x.s0) if x.s0 is not None else None
    cu = up(x.cu_seqlens, torch.int32) if x.cu_seqlens is not None else None
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    o = torch.full(tuple(x.v.shape), float("nan"), dtype=bf, device=dev())
    sT = torch.empty((x.n_seqs, H, dk, dv), dtype=torch.float32, device=dev())
    ns = x.n_seqs if cu is not None else 0
    gm = kda.KDA_GATE_PER_CHANNEL if x.g.ndim == 4 else kda.KDA_GATE_PER_HEAD
    ptr = lambda a: a.data_ptr() if a is not None else None  # noqa: E731
    stream = torch.cuda.current_stream().cuda_stream
    args = (ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(s0), ptr(sT), ptr(o), ptr(cu), ns,
            B, H, T, dk, dv, kda.KDA_BF16, gm)
    if noalloc:
        st = kda.kda_chunk_fwd_noalloc(*args, stream)
    else:
        wsb = kda.kda_chunk_fwd_workspace_size(B, H, T, dk, dv, ns, kda.KDA_BF16)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev())
        st = kda.kda_chunk_fwd(*args, ptr(ws), wsb, stream)
    assert st == kda.KDA_OK, kda.kda_status_string(st)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), sT.cpu().numpy()


def test_noalloc_matches_workspace_call_twice():
    cases = [
        # packed sequences of unequal length: the segment plan fits the scratch array
        ("packed H8 T16384", KDA_VARLEN_H32_T65536.replace(H=8, T=16384, seed=61)),
        # then a smaller, unpacked batch: the array still holds the first call's plan
        ("batch B2 H4 T1500", KDA_B2_H16_T4096.replace(B=2, H=4, T=1500, seed=62)),
    ]
    for name, cfg in cases:
        x = make_chunk_inputs(cfg)
        note(f"no-alloc forward: {name}")
        o_n, s_n = call(x, noalloc=True)
        o_w, s_w = call(x, noalloc=False)
        assert np.all(np.isfinite(o_n)), "some output position was not written"
        assert_close(o_n, o_w, TOL["bf16"], f"{name} outputs against kda_chunk_fwd")
        assert_close(s_n, s_w, TOL["bf16"], f"{name} states against kda_chunk_fwd")
        check_chains(x, o_n, s_n, oracle_chains(x), TOL["bf16"], f"{name} against the oracle")


def test_noalloc_headline_within_scratch():
    """The packed T = 65536, H = 32 workload needs more than the 64 MiB array for its
    segments: the call plans within it and still matches kda_chunk_fwd."""
    x = make_chunk_inputs(KDA_VARLEN_H32_T65536)
    note("no-alloc forward: packed H32 T65536")
    o_n, s_n = call(x, noalloc=True)
    o_w, s_w = call(x, noalloc=False)
    assert np.all(np.isfinite(o_n))
    assert_close(o_n, o_w, TOL["bf16"], "outputs against kda_chunk_fwd")
    assert_close(s_n, s_w, TOL["bf16"], "states against kda_chunk_fwd")
