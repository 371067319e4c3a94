"""fp64 CPU oracle for the gated delta rule forward (KDA / Gated DeltaNet).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. It shares no code with the
HIP library (``gated_delta_rule_13_amd``) and never imports it; the HIP library
never imports this package.

Two independent implementations live here:
  * ``kda_oracle.c`` (through ``kda_chains`` / ``kda_forward`` / ``kda_decode_step``):
    the token recurrence in plain C, fp64, parallel over chains. This is the oracle
    the GPU path is compared with. ``kda_oracle_bwd.c`` (``kda_chains_bwd`` /
    ``kda_backward``) is its backward pass: the chain rule through the same token
    step in reverse order.
  * ``reference.py``: the same recurrence written with numpy (for small cases), the
    pages' chunked (WY / UT transform) form, the pages' WY recursions and brute-force
    unrolled products, and the backward twin ``recurrence_bwd``. These exist to pin the
    oracle to the pages (the backward to finite differences of the forward).

Every function here has at least one pin in ``tests/test_oracle_pins.py``; none is
"parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

from .build import LIB, build_oracle

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = LIB if os.path.exists(LIB) else build_oracle(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.oracle_kda_chains.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P,
                                          P, P, P, P, ctypes.c_int, P, P, P, P, P, P, P, P,
                                          ctypes.c_int]
        lib.oracle_kda_chains.restype = ctypes.c_int
        lib.oracle_kda_chains_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P,
                                              P, P, P, P, ctypes.c_int, P, P, P, P, P, P, P,
                                              P, P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_kda_chains_bwd.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def kda_chains(q, k, v, g, beta, row_off, row_len, s0=None, erase=None, write=None,
               threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Runs independent chains whose tokens are rows of flat arrays.

    q, k: [rows, dk]; v: [rows, dv]; g: [rows, dk] (per channel) or [rows] (per head);
    beta: [rows]. The optional erase / write gates are scalars per row ([rows], used by
    the pins) or the Gated Delta Rule-2 vectors (erase [rows, dk], write [rows, dv]).
    Chain c covers rows row_off[c] .. row_off[c] + row_len[c] - 1. s0: [chains, dk, dv].
    Returns (o [rows, dv], final states [chains, dk, dv]), both float64.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    erase, write, s0 = _f64(erase), _f64(write), _f64(s0)
    erase_vec = erase if erase is not None and erase.ndim == 2 else None
    write_vec = write if write is not None and write.ndim == 2 else None
    erase = None if erase_vec is not None else erase
    write = None if write_vec is not None else write
    rows, dk = q.shape
    dv = v.shape[1]
    per_channel = 1 if g.ndim == 2 else 0
    off = np.ascontiguousarray(row_off, dtype=np.int64)
    ln = np.ascontiguousarray(row_len, dtype=np.int64)
    n = len(off)
    assert k.shape == (rows, dk) and v.shape[0] == rows and beta.shape == (rows,)
    assert erase_vec is None or erase_vec.shape == (rows, dk)
    assert write_vec is None or write_vec.shape == (rows, dv)
    assert erase is None or erase.shape == (rows,)
    assert write is None or write.shape == (rows,)
    assert np.all(off >= 0) and np.all(ln >= 0) and np.all(off + ln <= rows)
    if s0 is not None:
        assert s0.shape == (n, dk, dv)
    o = np.zeros((rows, dv), np.float64)
    sf = np.zeros((n, dk, dv), np.float64)
    rc = _load().oracle_kda_chains(n, dk, dv, _ptr(off), _ptr(ln), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(g), per_channel, _ptr(beta), _ptr(erase), _ptr(write),
                                   _ptr(erase_vec), _ptr(write_vec), _ptr(s0), _ptr(o),
                                   _ptr(sf), int(threads))
    if rc != 0:
        raise MemoryError("oracle_kda_chains could not allocate its work buffers")
    return o, sf


def kda_chains_bwd(q, k, v, g, beta, row_off, row_len, do, s0=None, dsT=None, erase=None,
                   write=None, threads: int = 0) -> Dict[str, np.ndarray]:
    """Gradients of ``kda_chains`` (kda_oracle_bwd.c): given do [rows, dv] and dsT
    [chains, dk, dv] (None = 0), the gradients of sum(do * o) + sum(dsT * S_T) with respect
    to q, k, v, g, beta (or the Gated Delta Rule-2 gates erase [rows, dk] / write
    [rows, dv]) and s0. Returns a dict of float64 arrays: dq, dk, dv, dg, ds0 and dbeta or
    derase / dwrite."""
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    erase, write, s0, dsT = _f64(erase), _f64(write), _f64(s0), _f64(dsT)
    rows, dk = q.shape
    dv = v.shape[1]
    off = np.ascontiguousarray(row_off, dtype=np.int64)
    ln = np.ascontiguousarray(row_len, dtype=np.int64)
    n = len(off)
    gdr2 = erase is not None
    assert (write is not None) == gdr2
    assert k.shape == (rows, dk) and v.shape == (rows, dv) and do.shape == (rows, dv)
    assert beta.shape == (rows,) and g.shape in ((rows, dk), (rows,))
    assert not gdr2 or (erase.shape == (rows, dk) and write.shape == (rows, dv))
    assert np.all(off >= 0) and np.all(ln >= 0) and np.all(off + ln <= rows)
    for x in (s0, dsT):
        assert x is None or x.shape == (n, dk, dv)
    out = {"dq": np.zeros((rows, dk)), "dk": np.zeros((rows, dk)), "dv": np.zeros((rows, dv)),
           "dg": np.zeros(g.shape), "ds0": np.zeros((n, dk, dv))}
    if gdr2:
        out["derase"], out["dwrite"] = np.zeros((rows, dk)), np.zeros((rows, dv))
    else:
        out["dbeta"] = np.zeros(rows)
    rc = _load().oracle_kda_chains_bwd(
        n, dk, dv, _ptr(off), _ptr(ln), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        1 if g.ndim == 2 else 0, _ptr(beta), _ptr(erase), _ptr(write), _ptr(s0), _ptr(do),
        _ptr(dsT), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
        _ptr(out.get("dbeta")), _ptr(out.get("derase")), _ptr(out.get("dwrite")),
        _ptr(out["ds0"]), int(threads))
    if rc != 0:
        raise MemoryError("oracle_kda_chains_bwd could not allocate its work buffers")
    return out


def pack_chains(q, k, v, g, beta, s0=None, cu_seqlens=None,
                chains: Optional[Iterable[Tuple[int, int]]] = None, erase=None, write=None):
    """Gathers the rows of the selected (sequence n, head h) chains of head-major inputs
    [B, H, T, ...] (B = 1 with ``cu_seqlens``) into the flat float64 arrays of
    ``kda_chains``; ``erase`` [B, H, T, dk] and ``write`` [B, H, T, dv] are the Gated
    Delta Rule-2 gates. Returns (chains, args, kwargs) with ``kda_chains(*args, **kwargs)``."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        N = len(cu) - 1
        spans = [(0, int(cu[n]), int(cu[n + 1] - cu[n])) for n in range(N)]
    else:
        N = B
        spans = [(n, 0, T) for n in range(N)]
    if chains is None:
        chains = [(n, h) for n in range(N) for h in range(H)]
    chains = list(chains)
    per_channel = g.ndim == 4
    offs, lens = [], []
    row = 0
    for (n, h) in chains:
        offs.append(row)
        lens.append(spans[n][2])
        row += spans[n][2]

    def gather(x, width):
        out = np.empty((row,) + ((width,) if width else ()), np.float64)
        for c, (n, h) in enumerate(chains):
            b, t0, ln = spans[n]
            out[offs[c]:offs[c] + ln] = x[b, h, t0:t0 + ln]
        return out

    args = (gather(q, dk), gather(k, dk), gather(v, dv), gather(g, dk if per_channel else 0),
            gather(beta, 0), offs, lens)
    kwargs = {"s0": np.stack([s0[n, h] for (n, h) in chains]) if s0 is not None else None}
    if erase is not None:
        kwargs["erase"] = gather(erase, dk)
    if write is not None:
        kwargs["write"] = gather(write, dv)
    return chains, args, kwargs


def kda_forward(q, k, v, g, beta, s0=None, cu_seqlens=None,
                chains: Optional[Iterable[Tuple[int, int]]] = None,
                threads: int = 0, erase=None,
                write=None) -> Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]]:
    """Forward over head-major inputs [B, H, T, ...] (B = 1 with ``cu_seqlens``).

    Each (sequence n, head h) is an independent chain. ``chains`` selects a subset
    (default: all). ``erase`` [B, H, T, dk] and ``write`` [B, H, T, dv] select Gated
    Delta Rule-2 (beta is then unused). Returns {(n, h): (o [len, dv], final state
    [dk, dv])}, float64.
    """
    chains, args, kwargs = pack_chains(q, k, v, g, beta, s0, cu_seqlens, chains, erase, write)
    o, sf = kda_chains(*args, **kwargs, threads=threads)
    offs, lens = args[5], args[6]
    return {ch: (o[offs[c]:offs[c] + lens[c]], sf[c]) for c, ch in enumerate(chains)}


def kda_backward(q, k, v, g, beta, do, s0=None, dsT=None, cu_seqlens=None,
                 chains: Optional[Iterable[Tuple[int, int]]] = None, threads: int = 0,
                 erase=None, write=None) -> Dict[Tuple[int, int], Dict[str, np.ndarray]]:
    """Backward over head-major inputs [B, H, T, ...] (B = 1 with ``cu_seqlens``): do
    [B, H, T, dv] and dsT [N, H, dk, dv] (None = 0) are the loss's gradients with respect
    to o and the final states. Returns {(n, h): {name: gradient}} with dq, dk [len, dk],
    dv [len, dv], dg [len, dk] or [len], ds0 [dk, dv] and dbeta [len] (or derase [len, dk]
    / dwrite [len, dv] for Gated Delta Rule-2), float64."""
    chains, args, kwargs = pack_chains(q, k, v, g, beta, s0, cu_seqlens, chains, erase, write)
    # the rows of do, in the packed order of the chains
    _, dargs, _ = pack_chains(q, k, do, g, beta, None, cu_seqlens, chains)
    dsT_c = np.stack([dsT[n, h] for (n, h) in chains]) if dsT is not None else None
    offs, lens = args[5], args[6]
    out = kda_chains_bwd(*args[:5], offs, lens, dargs[2], s0=kwargs["s0"], dsT=dsT_c,
                         erase=kwargs.get("erase"), write=kwargs.get("write"), threads=threads)
    res = {}
    for c, ch in enumerate(chains):
        sl = slice(offs[c], offs[c] + lens[c])
        res[ch] = {name: (a[c] if name == "ds0" else a[sl]) for name, a in out.items()}
    return res


def kda_decode_step(state, q, k, v, g, beta, threads: int = 0, erase=None,
                    write=None) -> Tuple[np.ndarray, np.ndarray]:
    """One single-token step for every (sequence, head): state [N, H, dk, dv];
    q, k [N, H, dk]; v [N, H, dv]; g [N, H, dk] or [N, H]; beta [N, H]; optional Gated
    Delta Rule-2 gates erase [N, H, dk] and write [N, H, dv].
    Returns (o [N, H, dv], new state [N, H, dk, dv]) in float64."""
    N, H, dk, dv = state.shape
    rows = N * H
    o, sf = kda_chains(q.reshape(rows, dk), k.reshape(rows, dk), v.reshape(rows, dv),
                       g.reshape(rows, -1) if g.ndim == 3 else g.reshape(rows),
                       beta.reshape(rows), np.arange(rows), np.ones(rows, np.int64),
                       s0=state.reshape(rows, dk, dv), threads=threads,
                       erase=None if erase is None else np.reshape(erase, (rows, dk)),
                       write=None if write is None else np.reshape(write, (rows, dv)))
    return o.reshape(N, H, dv), sf.reshape(N, H, dk, dv)
