"""The C-ABI library on the CPU: it loads, exports every symbol include/kda.h declares,
and rejects invalid arguments with the documented status codes before launching
anything (no compute call is made here: there is no GPU in this environment)."""

import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_13_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(kda_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(kda.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = kda.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for sym in declared_symbols():
        assert sym in exported, sym
        assert getattr(lib, sym) is not None


def test_status_strings():
    for code in range(5):
        assert kda.kda_status_string(code).startswith("KDA_")
    assert kda.kda_status_string(kda.KDA_ERR_PRECONDITION).startswith("KDA_ERR_PRECONDITION")
    assert "UNKNOWN" in kda.kda_status_string(99)


def test_debug_library_exports_every_declared_symbol():
    """The KDA_DEBUG build (device-side precondition checks) has the same boundary."""
    if not os.path.exists(kda.DEBUG_LIB_PATH):
        from gated_delta_rule_13_amd.build import build
        build(debug=True)
    lib = kda.open_library(kda.DEBUG_LIB_PATH)
    out = subprocess.run(["nm", "-D", "--defined-only", kda.DEBUG_LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for sym in declared_symbols():
        assert sym in exported, sym
    assert lib.kda_status_string(kda.KDA_ERR_PRECONDITION).startswith(b"KDA_ERR_PRECONDITION")
    # the host-side argument checks come first in the debug build too (nothing launches)
    assert chunk_call_on(lib, q=None) == kda.KDA_ERR_INVALID_ARG
    assert chunk_call_on(lib, dk=96) == kda.KDA_ERR_UNSUPPORTED


def plan_words_bytes(N, H, S):
    words = 8 + (N + 1) + 2 * (S + 1) + 4 * H * S
    return -(-4 * words // 256) * 256


def long_chain_slots(N, T, packed):
    """Slots kda.h requires for T axes of 2^22 tokens or more (0 below)."""
    if T < 1 << 22:
        return 0
    m = -(-T // (1 << 21))
    return (2 * N + 2 * m if packed else 2 * m * N) + 1


def segment_plan_bytes(B, H, T, N, packed, dk=128, cus=256):
    """The segment plan's recommended workspace as kda.h states it: plan words for a capacity
    of S slots, the states and transitions of S segments per head, and rows of carried-back
    queries per head (a whole T axis per sequence with fewer chains than compute units or
    past 2^22 tokens, else a quarter of the T axis)."""
    C = -(-T // 64)
    xmin = min(1 << 15, max(8, -(-C // 64)))
    S_all = min(1024, N + N // 8 + -(-C // xmin) + 1)
    S = max(long_chain_slots(N, T, packed), N, min(S_all, N + -(-cus // H) + 1))
    rows = (T if packed else N * T) if N * H < cus or T >= 1 << 22 else -(-T // 4)
    return plan_words_bytes(N, H, S) + 3 * S * H * dk * dk * 4 + rows * H * dk * 2


def long_chain_min_bytes(H, T, N, packed, dk=128):
    """The smallest workspace kda.h states for T axes of 2^22 tokens or more."""
    S = long_chain_slots(N, T, packed)
    rows = T if packed else N * T
    return plan_words_bytes(N, H, S) + 3 * S * H * dk * dk * 4 + rows * H * dk * 2


def test_workspace_size():
    # (sizes for a 256-CU device; without a GPU the library assumes 256 compute units)
    # dv = dk, packed sequences: the segment plan (the T = 65536 workload: 230 MiB)
    assert kda.kda_chunk_fwd_workspace_size(1, 32, 65536, 128, 128, 8, kda.KDA_BF16) == \
        segment_plan_bytes(1, 32, 65536, 8, True) == 241181440
    assert kda.kda_chunk_fwd_workspace_size(1, 4, 5000, 128, 128, 7, kda.KDA_BF16) == \
        segment_plan_bytes(1, 4, 5000, 7, True)
    # dv = dk, equal lengths with fewer chains than compute units: the segment plan
    assert kda.kda_chunk_fwd_workspace_size(2, 16, 4096, 128, 128, 0, kda.KDA_BF16) == \
        segment_plan_bytes(2, 16, 4096, 2, False)
    assert kda.kda_chunk_fwd_workspace_size(1, 2, 1000, 128, 128, 0, kda.KDA_BF16) == \
        segment_plan_bytes(1, 2, 1000, 1, False)
    # dv = 64, few chains: segments; per segment two dk x dv states and one dk x dk
    # transition (fp32); 2 sequences x 16 heads: 8 segments of 512 tokens
    assert kda.kda_chunk_fwd_workspace_size(1, 16, 4096, 128, 64, 2, kda.KDA_BF16) == \
        32 * 8 * (2 * 128 * 64 + 128 * 128) * 4
    # dv = 64, packed sequences with enough chains: a work list of 1 + 2 N H words
    # (rounded up to 256 bytes)
    assert kda.kda_chunk_fwd_workspace_size(1, 32, 65536, 128, 64, 8, kda.KDA_BF16) == 2304
    # equal lengths with enough chains: scheduled on the host, no workspace
    assert kda.kda_chunk_fwd_workspace_size(8, 32, 4096, 128, 128, 0, kda.KDA_BF16) == 0
    # no schedule: fp32, dk = 64, more than 1024 sequences, invalid sizes
    assert kda.kda_chunk_fwd_workspace_size(1, 32, 65536, 128, 128, 8, kda.KDA_F32) == 0
    assert kda.kda_chunk_fwd_workspace_size(1, 32, 65536, 64, 128, 8, kda.KDA_BF16) == 0
    assert kda.kda_chunk_fwd_workspace_size(1, 4, 65536, 128, 128, 1025, kda.KDA_BF16) == 0
    assert kda.kda_chunk_fwd_workspace_size(0, 4, 64, 128, 128, 0, kda.KDA_BF16) == 0
    # num_seqs > 0 describes a packed call, which has B = 1: any other B gets no workspace
    assert kda.kda_chunk_fwd_workspace_size(4, 1, 2048, 128, 128, 4, kda.KDA_BF16) == 0
    assert kda.kda_chunk_fwd_workspace_size(2, 4, 8192, 128, 128, 2, kda.KDA_BF16) == 0


@pytest.mark.parametrize("B,H,T,N,packed", [
    (1, 1, (1 << 22) + 5000, 1, True),      # one sequence past the whole-chain bound
    (1, 32, (1 << 22) + 64, 8, True),       # packed: S = 2 N + 2 m + 1 exceeds the usual cap
    (2, 4, (1 << 22) + 64, 2, False),       # equal lengths: S = 2 m N + 1, rows N T
    (1, 2, 1 << 24, 3, True),               # Xmin at its bound of 2^15 chunks
])
def test_workspace_size_long_chains(B, H, T, N, packed):
    """T axes of 2^22 tokens or more: the segment plan with items of at most 2^21 tokens;
    the recommendation covers kda.h's minimum."""
    got = kda.kda_chunk_fwd_workspace_size(B, H, T, 128, 128, N if packed else 0, kda.KDA_BF16)
    assert got == segment_plan_bytes(B, H, T, N, packed)
    assert got >= long_chain_min_bytes(H, T, N, packed)


def test_workspace_size_long_chains_fp32_path():
    """Long chains the segment plan cannot take get no workspace (the float32 path): dv = 64,
    fp32, and plans whose minimum exceeds 1024 slots."""
    T = (1 << 22) + 64
    assert kda.kda_chunk_fwd_workspace_size(1, 4, T, 128, 64, 1, kda.KDA_BF16) == 0
    assert kda.kda_chunk_fwd_workspace_size(1, 4, T, 128, 128, 1, kda.KDA_F32) == 0
    assert long_chain_slots(600, T, True) > 1024
    assert kda.kda_chunk_fwd_workspace_size(1, 1, T, 128, 128, 600, kda.KDA_BF16) == 0
    # just below the bound, whole chains as before
    assert kda.kda_chunk_fwd_workspace_size(1, 1, (1 << 22) - 64, 128, 128, 1, kda.KDA_BF16) == \
        segment_plan_bytes(1, 1, (1 << 22) - 64, 1, True)


DUMMY = 0x1000  # never dereferenced: every call below is rejected on the host


def chunk_call_on(lib, **over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, beta=DUMMY, initial_state=None,
                final_state=None, o=DUMMY, cu_seqlens=None, num_seqs=0, B=1, H=2, T=64,
                dk=128, dv=128, dt=kda.KDA_BF16, gm=kda.KDA_GATE_PER_CHANNEL, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(over)
    return lib.kda_chunk_fwd(*args.values())


def chunk_call(**over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, beta=DUMMY, initial_state=None,
                final_state=None, o=DUMMY, cu_seqlens=None, num_seqs=0, B=1, H=2, T=64,
                dk=128, dv=128, dt=kda.KDA_BF16, gm=kda.KDA_GATE_PER_CHANNEL, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(over)
    return kda.kda_chunk_fwd(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(beta=None), kda.KDA_ERR_INVALID_ARG),
    (dict(B=0), kda.KDA_ERR_INVALID_ARG),
    (dict(T=-3), kda.KDA_ERR_INVALID_ARG),
    (dict(dt=7), kda.KDA_ERR_INVALID_ARG),
    (dict(gm=5), kda.KDA_ERR_INVALID_ARG),
    (dict(cu_seqlens=DUMMY, num_seqs=2, B=2), kda.KDA_ERR_INVALID_ARG),
    (dict(cu_seqlens=DUMMY, num_seqs=0), kda.KDA_ERR_INVALID_ARG),
    (dict(num_seqs=3), kda.KDA_ERR_INVALID_ARG),
    # packed sequences need a work list: a buffer below its size, or a size without a buffer
    (dict(cu_seqlens=DUMMY, num_seqs=2, workspace=DUMMY, workspace_bytes=16),
     kda.KDA_ERR_INVALID_ARG),
    (dict(cu_seqlens=DUMMY, num_seqs=2, workspace=None, workspace_bytes=4096),
     kda.KDA_ERR_INVALID_ARG),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=256, dv=256), kda.KDA_ERR_UNSUPPORTED),
    # row arrays must be 16-byte aligned
    (dict(q=DUMMY + 8), kda.KDA_ERR_INVALID_ARG),
    (dict(v=DUMMY + 2), kda.KDA_ERR_INVALID_ARG),
    (dict(g=DUMMY + 4), kda.KDA_ERR_INVALID_ARG),
    (dict(o=DUMMY + 8, dt=kda.KDA_F32), kda.KDA_ERR_INVALID_ARG),
])
def test_chunk_fwd_rejects(over, code):
    assert chunk_call(**over) == code


def gdr2_chunk_call(**over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, erase=DUMMY, write=DUMMY,
                initial_state=None, final_state=None, o=DUMMY, cu_seqlens=None, num_seqs=0,
                B=1, H=2, T=64, dk=128, dv=128, dt=kda.KDA_BF16, gm=kda.KDA_GATE_PER_CHANNEL,
                workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return kda.kda_gdr2_chunk_fwd(*args.values())


def gdr2_step_call(**over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, erase=DUMMY, write=DUMMY, state=DUMMY,
                o=DUMMY, N=4, H=2, dk=128, dv=128, dt=kda.KDA_BF16,
                gm=kda.KDA_GATE_PER_CHANNEL, stream=None)
    args.update(over)
    return kda.kda_gdr2_recurrent_step(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(erase=None), kda.KDA_ERR_INVALID_ARG),
    (dict(write=None), kda.KDA_ERR_INVALID_ARG),
    (dict(q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(T=0), kda.KDA_ERR_INVALID_ARG),
    (dict(dv=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(erase=DUMMY + 4), kda.KDA_ERR_INVALID_ARG),
    (dict(write=DUMMY + 8), kda.KDA_ERR_INVALID_ARG),
])
def test_gdr2_chunk_fwd_rejects(over, code):
    assert gdr2_chunk_call(**over) == code


@pytest.mark.parametrize("over,code", [
    (dict(erase=None), kda.KDA_ERR_INVALID_ARG),
    (dict(write=None), kda.KDA_ERR_INVALID_ARG),
    (dict(state=None), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=256), kda.KDA_ERR_UNSUPPORTED),
])
def test_gdr2_recurrent_step_rejects(over, code):
    assert gdr2_step_call(**over) == code


def step_call(**over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, beta=DUMMY, state=DUMMY, o=DUMMY, N=4,
                H=2, dk=128, dv=128, dt=kda.KDA_BF16, gm=kda.KDA_GATE_PER_CHANNEL,
                stream=None)
    args.update(over)
    return kda.kda_recurrent_step(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(state=None), kda.KDA_ERR_INVALID_ARG),
    (dict(k=None), kda.KDA_ERR_INVALID_ARG),
    (dict(N=0), kda.KDA_ERR_INVALID_ARG),
    (dict(H=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(dt=2), kda.KDA_ERR_INVALID_ARG),
    (dict(gm=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=100), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
])
def test_recurrent_step_rejects(over, code):
    assert step_call(**over) == code


def test_python_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, torch.zeros(1, 1, 4, 64), torch.zeros(1, 1, 4))


def prologue_call(**over):
    args = dict(q_in=DUMMY, k_in=DUMMY, u=DUMMY, A_log=DUMMY, dt_bias=DUMMY, beta_in=None,
                q_out=DUMMY, k_out=DUMMY, g_out=DUMMY, beta_out=None, B=1, H=2, T=8, dk=128,
                dt=kda.KDA_BF16, stream=None)
    args.update(over)
    return kda.kda_prologue(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(u=None), kda.KDA_ERR_INVALID_ARG),
    (dict(A_log=None), kda.KDA_ERR_INVALID_ARG),
    (dict(g_out=None), kda.KDA_ERR_INVALID_ARG),
    (dict(beta_in=DUMMY), kda.KDA_ERR_INVALID_ARG),        # beta_in without beta_out
    (dict(beta_out=DUMMY), kda.KDA_ERR_INVALID_ARG),
    (dict(T=0), kda.KDA_ERR_INVALID_ARG),
    (dict(dt=3), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(q_in=DUMMY + 8), kda.KDA_ERR_INVALID_ARG),     # not 16-byte aligned
    (dict(g_out=DUMMY + 4), kda.KDA_ERR_INVALID_ARG),
    (dict(dt_bias=DUMMY + 4), kda.KDA_ERR_INVALID_ARG),
])
def test_prologue_rejects(over, code):
    assert prologue_call(**over) == code


def epilogue_call(**over):
    args = dict(o_in=DUMMY, z=DUMMY, weight=None, eps=1e-6, o_out=DUMMY, B=1, H=2, T=8, dv=128,
                dt=kda.KDA_BF16, stream=None)
    args.update(over)
    return kda.kda_epilogue(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(z=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o_out=None), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=0.0), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=float("inf")), kda.KDA_ERR_INVALID_ARG),
    (dict(B=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(dv=200), kda.KDA_ERR_UNSUPPORTED),
    (dict(z=DUMMY + 8), kda.KDA_ERR_INVALID_ARG),        # not 16-byte aligned
    (dict(weight=DUMMY + 4), kda.KDA_ERR_INVALID_ARG),
])
def test_epilogue_rejects(over, code):
    assert epilogue_call(**over) == code


def test_bwd_workspace_size():
    # two bf16 histories of dk * dv / 16 bytes per padded token (one matrix per pair of
    # 16-token blocks): 2 x 32 x (4096 + 64 * 2) x 1024
    # (packed sequences: plus the 768-byte work list of 2 x 32 chains)
    one = 32 * (4096 + 64 * 2) * 1024
    assert kda.kda_chunk_bwd_workspace_size(1, 32, 4096, 128, 128, 2, kda.KDA_BF16) == \
        2 * one + 768
    # equal lengths: B sequences padded to 64 tokens each
    one = 16 * 2 * 4096 * 512
    assert kda.kda_chunk_bwd_workspace_size(2, 16, 4096, 128, 64, 0, kda.KDA_BF16) == 2 * one
    assert kda.kda_chunk_bwd_workspace_size(2, 16, 4096, 128, 128, 0, kda.KDA_F32) == 0
    assert kda.kda_chunk_bwd_workspace_size(2, 16, 4096, 96, 128, 0, kda.KDA_BF16) == 0
    # dk = 64: the dk = 128 workspace behind padded copies of the key-side arrays and states
    # (q, k, dq, dk bf16 and g, erase, dg, d erase fp32 of 128 channels per row; s0, dS_T,
    # dS_0 of 128 x dv fp32 per chain)
    rows, nh = 2 * 16 * 4096, 2 * 16
    pads = rows * 128 * (4 * 2 + 4 * 4) + 3 * nh * 128 * 128 * 4
    assert kda.kda_chunk_bwd_workspace_size(2, 16, 4096, 64, 128, 0, kda.KDA_BF16) == \
        pads + kda.kda_chunk_bwd_workspace_size(2, 16, 4096, 128, 128, 0, kda.KDA_BF16)
    assert kda.kda_chunk_bwd_workspace_size(0, 16, 4096, 128, 128, 0, kda.KDA_BF16) == 0
    # the longest T axis of the backward: (T + 64) 8 dv < 2^31
    assert kda.kda_chunk_bwd_workspace_size(1, 1, (1 << 21) - 65, 128, 128, 1, kda.KDA_BF16) > 0
    assert kda.kda_chunk_bwd_workspace_size(1, 1, (1 << 21) - 64, 128, 128, 1, kda.KDA_BF16) == 0


def bwd_call(**over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, beta=DUMMY, initial_state=None,
                grad_o=DUMMY, grad_final_state=None, grad_q=DUMMY, grad_k=DUMMY, grad_v=DUMMY,
                grad_g=DUMMY, grad_beta=DUMMY, grad_initial_state=None, cu_seqlens=None,
                num_seqs=0, B=1, H=2, T=64, dk=128, dv=128, dt=kda.KDA_BF16,
                gm=kda.KDA_GATE_PER_CHANNEL, workspace=DUMMY, workspace_bytes=0, stream=None)
    args.update(over)
    return kda.kda_chunk_bwd(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(grad_o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(grad_q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(grad_g=None), kda.KDA_ERR_INVALID_ARG),
    (dict(grad_beta=None), kda.KDA_ERR_INVALID_ARG),
    (dict(beta=None), kda.KDA_ERR_INVALID_ARG),
    (dict(T=0), kda.KDA_ERR_INVALID_ARG),
    (dict(gm=7), kda.KDA_ERR_INVALID_ARG),
    (dict(cu_seqlens=DUMMY, num_seqs=0), kda.KDA_ERR_INVALID_ARG),
    (dict(workspace_bytes=100), kda.KDA_ERR_INVALID_ARG),     # smaller than the size
    (dict(workspace=None, workspace_bytes=1 << 30), kda.KDA_ERR_INVALID_ARG),
    (dict(dt=kda.KDA_F32), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=64), kda.KDA_ERR_INVALID_ARG),   # supported, but the workspace is too small
    (dict(dv=96), kda.KDA_ERR_UNSUPPORTED),
    # one chain's history must be addressable by a buffer descriptor: (T + 64) 8 dv < 2^31
    (dict(T=(1 << 21) - 64), kda.KDA_ERR_UNSUPPORTED),
    (dict(T=(1 << 22) - 64, dv=64), kda.KDA_ERR_UNSUPPORTED),
])
def test_bwd_rejects(over, code):
    assert bwd_call(**over) == code


def gdr2_bwd_call(**over):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, erase=DUMMY, write=DUMMY,
                initial_state=None, grad_o=DUMMY, grad_final_state=None, grad_q=DUMMY,
                grad_k=DUMMY, grad_v=DUMMY, grad_g=DUMMY, grad_erase=DUMMY, grad_write=DUMMY,
                grad_initial_state=None, cu_seqlens=None, num_seqs=0, B=1, H=2, T=64, dk=128,
                dv=128, dt=kda.KDA_BF16, gm=kda.KDA_GATE_PER_CHANNEL, workspace=DUMMY,
                workspace_bytes=0, stream=None)
    args.update(over)
    return kda.kda_gdr2_chunk_bwd(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(erase=None), kda.KDA_ERR_INVALID_ARG),
    (dict(write=None), kda.KDA_ERR_INVALID_ARG),
    (dict(grad_erase=None), kda.KDA_ERR_INVALID_ARG),
    (dict(grad_write=None), kda.KDA_ERR_INVALID_ARG),
    (dict(grad_g=None), kda.KDA_ERR_INVALID_ARG),
    (dict(workspace_bytes=100), kda.KDA_ERR_INVALID_ARG),
    (dict(dt=kda.KDA_F32), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=32), kda.KDA_ERR_UNSUPPORTED),
])
def test_gdr2_bwd_rejects(over, code):
    assert gdr2_bwd_call(**over) == code
