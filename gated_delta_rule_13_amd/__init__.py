"""Python binding of libkda.so, the MI355X (gfx950) gated delta rule forward library.

The binding only marshals arguments: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/kda.h``. PyTorch provides device memory and the
current stream. There is no CPU fallback: if the library is not built, or a tensor is
not on the GPU, the call raises.

  chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
            output_final_state=True)               -> (o, final_state or None)
  recurrent_step(q, k, v, g, beta, state)         -> o      (state updated in place)

The raw entry points ``kda_chunk_fwd``, ``kda_recurrent_step``,
``kda_chunk_fwd_workspace_size`` and ``kda_status_string`` are exposed with the C
names and C argument order (pointers as integers).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_ERR_PRECONDITION = 4   # KDA_DEBUG builds (libkda_debug.so) only
DEBUG_LIB_PATH = os.path.join(HERE, "libkda_debug.so")
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_PER_CHANNEL, KDA_GATE_PER_HEAD = 0, 1

EXPORTED_SYMBOLS = ("kda_chunk_fwd", "kda_recurrent_step", "kda_chunk_fwd_workspace_size",
                    "kda_status_string", "kda_gdr2_chunk_fwd", "kda_gdr2_recurrent_step",
                    "kda_prologue", "kda_epilogue", "kda_chunk_bwd",
                    "kda_chunk_bwd_workspace_size", "kda_gdr2_chunk_bwd",
                    "kda_chunk_fwd_noalloc")

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kda_status_string(status)}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libkda.so (built by ``gated_delta_rule_13_amd/build.py``) as the library behind
    every function of this module; raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A separate handle on a build of the library (e.g. ``DEBUG_LIB_PATH``), with the C
    signatures set; the module's functions keep using ``load_library``'s."""
    if not os.path.exists(path):
        raise RuntimeError(f"{os.path.basename(path)} is not built ({path}); "
                           "run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P,
                                  ctypes.c_size_t, P]
    lib.kda_chunk_fwd.restype = I
    lib.kda_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.kda_chunk_fwd_noalloc.restype = I
    lib.kda_recurrent_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.kda_recurrent_step.restype = I
    lib.kda_gdr2_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                       I, P, ctypes.c_size_t, P]
    lib.kda_gdr2_chunk_fwd.restype = I
    lib.kda_gdr2_recurrent_step.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.kda_gdr2_recurrent_step.restype = I
    lib.kda_prologue.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.kda_prologue.restype = I
    lib.kda_epilogue.argtypes = [P, P, P, ctypes.c_float, P, I, I, I, I, I, P]
    lib.kda_epilogue.restype = I
    lib.kda_chunk_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I,
                                  I, I, I, I, P, ctypes.c_size_t, P]
    lib.kda_chunk_bwd.restype = I
    lib.kda_gdr2_chunk_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, I,
                                       I, I, I, I, I, I, I, P, ctypes.c_size_t, P]
    lib.kda_gdr2_chunk_bwd.restype = I
    lib.kda_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.kda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_status_string.argtypes = [I]
    lib.kda_status_string.restype = ctypes.c_char_p
    return lib


# ----------------------------------------------------------------------------- raw ABI
def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_chunk_fwd_workspace_size(B, H, T, dk, dv, num_seqs, dt) -> int:
    return int(load_library().kda_chunk_fwd_workspace_size(B, H, T, dk, dv, num_seqs, dt))


def kda_chunk_fwd(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, num_seqs,
                  B, H, T, dk, dv, dt, gm, workspace, workspace_bytes, stream) -> int:
    return int(load_library().kda_chunk_fwd(q, k, v, g, beta, initial_state, final_state, o,
                                            cu_seqlens, num_seqs, B, H, T, dk, dv, dt, gm,
                                            workspace, workspace_bytes, stream))


def kda_chunk_fwd_noalloc(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens,
                          num_seqs, B, H, T, dk, dv, dt, gm, stream) -> int:
    return int(load_library().kda_chunk_fwd_noalloc(q, k, v, g, beta, initial_state,
                                                    final_state, o, cu_seqlens, num_seqs, B, H,
                                                    T, dk, dv, dt, gm, stream))


def kda_recurrent_step(q, k, v, g, beta, state, o, N, H, dk, dv, dt, gm, stream) -> int:
    return int(load_library().kda_recurrent_step(q, k, v, g, beta, state, o, N, H, dk, dv,
                                                 dt, gm, stream))


def kda_gdr2_chunk_fwd(q, k, v, g, erase, write, initial_state, final_state, o, cu_seqlens,
                       num_seqs, B, H, T, dk, dv, dt, gm, workspace, workspace_bytes,
                       stream) -> int:
    return int(load_library().kda_gdr2_chunk_fwd(q, k, v, g, erase, write, initial_state,
                                                 final_state, o, cu_seqlens, num_seqs, B, H,
                                                 T, dk, dv, dt, gm, workspace,
                                                 workspace_bytes, stream))


def kda_gdr2_recurrent_step(q, k, v, g, erase, write, state, o, N, H, dk, dv, dt, gm,
                            stream) -> int:
    return int(load_library().kda_gdr2_recurrent_step(q, k, v, g, erase, write, state, o, N,
                                                      H, dk, dv, dt, gm, stream))


def kda_chunk_bwd_workspace_size(B, H, T, dk, dv, num_seqs, dt) -> int:
    return int(load_library().kda_chunk_bwd_workspace_size(B, H, T, dk, dv, num_seqs, dt))


def kda_chunk_bwd(q, k, v, g, beta, initial_state, grad_o, grad_final_state, grad_q, grad_k,
                  grad_v, grad_g, grad_beta, grad_initial_state, cu_seqlens, num_seqs, B, H, T,
                  dk, dv, dt, gm, workspace, workspace_bytes, stream) -> int:
    return int(load_library().kda_chunk_bwd(
        q, k, v, g, beta, initial_state, grad_o, grad_final_state, grad_q, grad_k, grad_v,
        grad_g, grad_beta, grad_initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv, dt, gm,
        workspace, workspace_bytes, stream))


def kda_gdr2_chunk_bwd(q, k, v, g, erase, write, initial_state, grad_o, grad_final_state,
                       grad_q, grad_k, grad_v, grad_g, grad_erase, grad_write,
                       grad_initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv, dt, gm,
                       workspace, workspace_bytes, stream) -> int:
    return int(load_library().kda_gdr2_chunk_bwd(
        q, k, v, g, erase, write, initial_state, grad_o, grad_final_state, grad_q, grad_k,
        grad_v, grad_g, grad_erase, grad_write, grad_initial_state, cu_seqlens, num_seqs, B, H,
        T, dk, dv, dt, gm, workspace, workspace_bytes, stream))


def kda_prologue(q_in, k_in, u, A_log, dt_bias, beta_in, q_out, k_out, g_out, beta_out, B, H, T,
                 dk, dt, stream) -> int:
    return int(load_library().kda_prologue(q_in, k_in, u, A_log, dt_bias, beta_in, q_out,
                                           k_out, g_out, beta_out, B, H, T, dk, dt, stream))


def kda_epilogue(o_in, z, weight, eps, o_out, B, H, T, dv, dt, stream) -> int:
    return int(load_library().kda_epilogue(o_in, z, weight, float(eps), o_out, B, H, T, dv, dt,
                                           stream))


# ----------------------------------------------------------------------- torch helpers
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _chunk(q, k, v, g, gates, initial_state, cu_seqlens, output_final_state, o, final_state,
           schedule):
    """Shared argument checks and call of kda_chunk_fwd / kda_gdr2_chunk_fwd.
    ``gates`` is (beta,) or (erase, write)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    _check(g, "g", torch.float32, dev)
    _check(initial_state, "initial_state", torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("inconsistent q/k/v shapes")
    if len(gates) == 1:
        _check(gates[0], "beta", torch.float32, dev)
        if gates[0].shape != (B, H, T):
            raise ValueError(f"beta must be {(B, H, T)}")
    else:
        _check(gates[0], "erase", torch.float32, dev)
        _check(gates[1], "write", torch.float32, dev)
        if gates[0].shape != (B, H, T, dk) or gates[1].shape != (B, H, T, dv):
            raise ValueError(f"erase must be {(B, H, T, dk)} and write {(B, H, T, dv)}")
    if g.shape == (B, H, T, dk):
        gm = KDA_GATE_PER_CHANNEL
    elif g.shape == (B, H, T):
        gm = KDA_GATE_PER_HEAD
    else:
        raise ValueError(f"g must be [B,H,T,dk] or [B,H,T], got {tuple(g.shape)}")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None and initial_state.shape != (N, H, dk, dv):
        raise ValueError(f"initial_state must be {(N, H, dk, dv)}")
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, dev)
    if tuple(o.shape) != (B, H, T, dv):
        raise ValueError(f"o must be {(B, H, T, dv)}, got {tuple(o.shape)}")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", torch.float32, dev)
    if final_state is not None and tuple(final_state.shape) != (N, H, dk, dv):
        raise ValueError(f"final_state must be {(N, H, dk, dv)}, got {tuple(final_state.shape)}")
    num_seqs = 0 if cu_seqlens is None else N
    ws_bytes = kda_chunk_fwd_workspace_size(B, H, T, dk, dv, num_seqs, dt) if schedule else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    common = (_ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(cu_seqlens), num_seqs,
              B, H, T, dk, dv, dt, gm, _ptr(ws), ws_bytes, _stream(dev))
    if len(gates) == 1:
        st = kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gates[0]), *common)
        where = "kda_chunk_fwd"
    else:
        st = kda_gdr2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gates[0]),
                                _ptr(gates[1]), *common)
        where = "kda_gdr2_chunk_fwd"
    if st != KDA_OK:
        raise KDAError(st, where)
    return o, final_state


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, output_final_state: bool = True,
              o: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
              schedule: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked forward over [B, H, T, d] head-major tensors (see ``kda_chunk_fwd``).

    g: float32 [B, H, T, dk] (per key channel, KDA) or [B, H, T] (per head, Gated
    DeltaNet); beta: float32 [B, H, T]; initial_state: float32 [N, H, dk, dv] or None;
    cu_seqlens: int32 [N + 1] on the GPU (B must be 1) or None. ``o`` and ``final_state``
    may be given to reuse buffers; ``final_state`` may be ``initial_state``.
    ``schedule=False`` passes no workspace (one workgroup per chain, no column split).
    """
    return _chunk(q, k, v, g, (beta,), initial_state, cu_seqlens, output_final_state, o,
                  final_state, schedule)


def gdr2_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   erase: torch.Tensor, write: torch.Tensor,
                   initial_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, output_final_state: bool = True,
                   o: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                   schedule: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated Delta Rule-2 chunked forward (see ``kda_gdr2_chunk_fwd``): ``chunk_fwd`` with
    beta replaced by erase float32 [B, H, T, dk] and write float32 [B, H, T, dv]."""
    return _chunk(q, k, v, g, (erase, write), initial_state, cu_seqlens, output_final_state,
                  o, final_state, schedule)


def _step(q, k, v, g, gates, state, o):
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    _check(g, "g", torch.float32, dev)
    _check(state, "state", torch.float32, dev)
    if k.shape != q.shape or v.shape[:2] != (N, H) or state.shape != (N, H, dk, dv):
        raise ValueError("inconsistent decode shapes")
    if len(gates) == 1:
        _check(gates[0], "beta", torch.float32, dev)
        if gates[0].shape != (N, H):
            raise ValueError("beta must be [N, H]")
    else:
        _check(gates[0], "erase", torch.float32, dev)
        _check(gates[1], "write", torch.float32, dev)
        if gates[0].shape != (N, H, dk) or gates[1].shape != (N, H, dv):
            raise ValueError("erase must be [N, H, dk] and write [N, H, dv]")
    if g.shape == (N, H, dk):
        gm = KDA_GATE_PER_CHANNEL
    elif g.shape == (N, H):
        gm = KDA_GATE_PER_HEAD
    else:
        raise ValueError(f"g must be [N,H,dk] or [N,H], got {tuple(g.shape)}")
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, dev)
    if tuple(o.shape) != (N, H, dv):
        raise ValueError(f"o must be {(N, H, dv)}, got {tuple(o.shape)}")
    if len(gates) == 1:
        st = kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gates[0]),
                                _ptr(state), _ptr(o), N, H, dk, dv, dt, gm, _stream(dev))
        where = "kda_recurrent_step"
    else:
        st = kda_gdr2_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gates[0]),
                                     _ptr(gates[1]), _ptr(state), _ptr(o), N, H, dk, dv, dt,
                                     gm, _stream(dev))
        where = "kda_gdr2_recurrent_step"
    if st != KDA_OK:
        raise KDAError(st, where)
    return o


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   beta: torch.Tensor, state: torch.Tensor,
                   o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step (see ``kda_recurrent_step``): q, k [N, H, dk]; v [N, H, dv];
    g float32 [N, H, dk] or [N, H]; beta float32 [N, H]; state float32 [N, H, dk, dv],
    updated in place. Returns o [N, H, dv]."""
    return _step(q, k, v, g, (beta,), state, o)


def gdr2_recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        erase: torch.Tensor, write: torch.Tensor, state: torch.Tensor,
                        o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gated Delta Rule-2 decode step (see ``kda_gdr2_recurrent_step``): erase float32
    [N, H, dk], write float32 [N, H, dv] in place of beta."""
    return _step(q, k, v, g, (erase, write), state, o)


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, grad_o: torch.Tensor,
              initial_state: Optional[torch.Tensor] = None,
              grad_final_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, grad_initial_state: bool = True):
    """Backward of ``chunk_fwd`` (see ``kda_chunk_bwd``): returns (dq, dk, dv, dg, dbeta,
    dS0 or None) for the loss gradients grad_o [B, H, T, dv] and grad_final_state
    [N, H, dk, dv] (None = 0). bf16 q/k/v/grad_o, dk in {64, 128}, dv in {64, 128}."""
    return _bwd(q, k, v, g, (beta,), grad_o, initial_state, grad_final_state, cu_seqlens,
                grad_initial_state)


def gdr2_chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   erase: torch.Tensor, write: torch.Tensor, grad_o: torch.Tensor,
                   initial_state: Optional[torch.Tensor] = None,
                   grad_final_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, grad_initial_state: bool = True):
    """Backward of ``gdr2_chunk_fwd`` (see ``kda_gdr2_chunk_bwd``): returns (dq, dk, dv, dg,
    d_erase, d_write, dS0 or None)."""
    return _bwd(q, k, v, g, (erase, write), grad_o, initial_state, grad_final_state,
                cu_seqlens, grad_initial_state)


def _bwd(q, k, v, g, gates, grad_o, initial_state, grad_final_state, cu_seqlens,
         grad_initial_state):
    """Shared checks and call of kda_chunk_bwd / kda_gdr2_chunk_bwd; ``gates`` is (beta,)
    or (erase, write)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (grad_o, "grad_o")):
        _check(t, n, q.dtype, dev)
    for t, n in ((g, "g"), (initial_state, "initial_state"),
                 (grad_final_state, "grad_final_state")) + tuple((x, "gate") for x in gates):
        _check(t, n, torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or grad_o.shape != v.shape:
        raise ValueError("inconsistent q/k/v/grad_o shapes")
    if len(gates) == 1 and gates[0].shape != (B, H, T):
        raise ValueError(f"beta must be {(B, H, T)}")
    if len(gates) == 2 and (gates[0].shape != (B, H, T, dk) or gates[1].shape != (B, H, T, dv)):
        raise ValueError(f"erase must be {(B, H, T, dk)} and write {(B, H, T, dv)}")
    if g.shape == (B, H, T, dk):
        gm = KDA_GATE_PER_CHANNEL
    elif g.shape == (B, H, T):
        gm = KDA_GATE_PER_HEAD
    else:
        raise ValueError(f"g must be [B,H,T,dk] or [B,H,T], got {tuple(g.shape)}")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    for t, n in ((initial_state, "initial_state"), (grad_final_state, "grad_final_state")):
        if t is not None and t.shape != (N, H, dk, dv):
            raise ValueError(f"{n} must be {(N, H, dk, dv)}")
    num_seqs = 0 if cu_seqlens is None else N
    ws_bytes = kda_chunk_bwd_workspace_size(B, H, T, dk, dv, num_seqs, dt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g)
    dgates = tuple(torch.empty_like(x) for x in gates)
    ds0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) \
        if grad_initial_state else None
    common = (_ptr(cu_seqlens), num_seqs, B, H, T, dk, dv, dt, gm, _ptr(ws), ws_bytes,
              _stream(dev))
    if len(gates) == 1:
        st = kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gates[0]),
                           _ptr(initial_state), _ptr(grad_o), _ptr(grad_final_state), _ptr(dq),
                           _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(dgates[0]), _ptr(ds0), *common)
        where = "kda_chunk_bwd"
    else:
        st = kda_gdr2_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gates[0]),
                                _ptr(gates[1]), _ptr(initial_state), _ptr(grad_o),
                                _ptr(grad_final_state), _ptr(dq), _ptr(dk_), _ptr(dv_),
                                _ptr(dg), _ptr(dgates[0]), _ptr(dgates[1]), _ptr(ds0), *common)
        where = "kda_gdr2_chunk_bwd"
    if st != KDA_OK:
        raise KDAError(st, where)
    return (dq, dk_, dv_, dg) + dgates + (ds0,)


def prologue(q_in: torch.Tensor, k_in: torch.Tensor, u: torch.Tensor, A_log: torch.Tensor,
             dt_bias: torch.Tensor, beta_in: Optional[torch.Tensor] = None,
             inplace: bool = False):
    """Fused prologue (see ``kda_prologue``): q_in, k_in [B, H, T, dk] (bf16 or fp32),
    u float32 [B, H, T, dk], A_log float32 [H], dt_bias float32 [H, dk] (or [H * dk]),
    beta_in float32 [B, H, T] or None. Returns (q, k, g, beta); with ``inplace`` q, k, g
    and beta overwrite q_in, k_in, u and beta_in."""
    B, H, T, dk = q_in.shape
    dev = q_in.device
    dt = _dtype_code(q_in)
    _check(q_in, "q_in", q_in.dtype, dev)
    _check(k_in, "k_in", q_in.dtype, dev)
    for t, n in ((u, "u"), (A_log, "A_log"), (dt_bias, "dt_bias")):
        _check(t, n, torch.float32, dev)
    _check(beta_in, "beta_in", torch.float32, dev)
    if k_in.shape != q_in.shape or u.shape != q_in.shape or A_log.numel() != H \
            or dt_bias.numel() != H * dk or (beta_in is not None and beta_in.shape != (B, H, T)):
        raise ValueError("inconsistent prologue shapes")
    q = q_in if inplace else torch.empty_like(q_in)
    k = k_in if inplace else torch.empty_like(k_in)
    g = u if inplace else torch.empty_like(u)
    beta = None if beta_in is None else (beta_in if inplace else torch.empty_like(beta_in))
    st = kda_prologue(_ptr(q_in), _ptr(k_in), _ptr(u), _ptr(A_log), _ptr(dt_bias), _ptr(beta_in),
                      _ptr(q), _ptr(k), _ptr(g), _ptr(beta), B, H, T, dk, dt, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_prologue")
    return q, k, g, beta


def epilogue(o_in: torch.Tensor, z: torch.Tensor, weight: Optional[torch.Tensor] = None,
             eps: float = 1e-6, inplace: bool = False) -> torch.Tensor:
    """Fused epilogue (see ``kda_epilogue``): Sigmoid(z) * RMSNorm(o_in) * weight per head
    over dv. o_in, z [B, H, T, dv] (same dtype); weight float32 [dv] or None."""
    B, H, T, dv = o_in.shape
    dev = o_in.device
    dt = _dtype_code(o_in)
    _check(o_in, "o_in", o_in.dtype, dev)
    _check(z, "z", o_in.dtype, dev)
    _check(weight, "weight", torch.float32, dev)
    if z.shape != o_in.shape or (weight is not None and weight.numel() != dv):
        raise ValueError("inconsistent epilogue shapes")
    out = o_in if inplace else torch.empty_like(o_in)
    st = kda_epilogue(_ptr(o_in), _ptr(z), _ptr(weight), eps, _ptr(out), B, H, T, dv, dt,
                      _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_epilogue")
    return out
