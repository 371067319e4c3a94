"""Seeded generators for the five benchmark workloads and for smaller test cases.

All arrays are numpy float32 (or int32 for ``cu_seqlens``). When a workload is
bf16, every value that the kernel receives as bf16 (q, k, v) is rounded here to
the nearest bf16 value (round to nearest, ties to even), so that the float32
array holds exactly what the device sees and the oracle can upcast it without
any further rounding. g, beta and the initial state stay float32.

Layouts are head-major, as the boundary expects:
  q, k : [B, H, T, dk]      v : [B, H, T, dv]
  g    : [B, H, T, dk] (per-key-channel decay) or [B, H, T] (one decay per head)
  beta : [B, H, T]          s0 : [N, H, dk, dv]
With packed variable-length sequences B is 1 and ``cu_seqlens`` (int32, N+1
entries, starting at 0 and ending at T) marks where each sequence starts.

Distributions (the same for every workload unless stated):
  q, k  ~ N(0, 1) per element, then L2-normalised per (b, h, t) vector
  v     ~ N(0, 1)
  beta  = sigmoid(x), x ~ N(0, 1)
  g     = max(-5, -exp(x)), x ~ N(-3, 1)   (log of the decay alpha, per token)
  s0    ~ N(0, 0.02^2) where a workload has a random initial state
  erase, write (gates = "gdr2" only) = sigmoid(x), x ~ N(0, 1) per element:
        the Gated Delta Rule-2 gates, erase [B, H, T, dk] and write [B, H, T, dv]
  prologue / epilogue pre-activations: see make_gate_inputs
Every tensor is drawn in blocks of one (batch row, head) from its own counter-style
seeded stream, numpy.random.default_rng([seed, tensor id, batch row, head]), so the
values do not depend on how many threads fill the blocks; the sequence lengths and
the pinned rows have streams of their own.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

G_FLOOR = -5.0  # lower bound of the per-token log-decay


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    kind: str            # "chunk" (prefill forward) or "decode" (single-token steps)
    dtype: str           # "f32" or "bf16": element type of q, k, v and o
    B: int
    H: int
    T: int               # tokens per sequence (chunk) or steps (decode)
    dk: int
    dv: int
    gate: str = "channel"   # "channel" (KDA) or "head" (Gated DeltaNet)
    random_s0: bool = False
    num_seqs: int = 0       # > 0: packed variable-length sequences (B must be 1)
    pin_frac: float = 0.0   # fraction of (head, token) rows whose log-decay is pinned at -5
    seed: int = 0
    gates: str = "beta"     # "beta" (one gate per token) or "gdr2" (erase [.., dk], write [.., dv])

    @property
    def n_chains(self) -> int:
        n = self.num_seqs if self.num_seqs else self.B
        return n * self.H

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


TINY_KDA_F32 = WorkloadConfig("tiny_kda_f32", "chunk", "f32", B=1, H=2, T=256, dk=64, dv=64,
                              seed=0)
KDA_B2_H16_T4096 = WorkloadConfig("kda_bf16_b2_h16_t4096", "chunk", "bf16", B=2, H=16, T=4096,
                                  dk=128, dv=128, random_s0=True, seed=1)
GDN_B1_H16_T8192 = WorkloadConfig("gdn_bf16_b1_h16_t8192", "chunk", "bf16", B=1, H=16, T=8192,
                                  dk=128, dv=128, gate="head", seed=2)
KDA_VARLEN_H32_T65536 = WorkloadConfig("kda_bf16_varlen_h32_t65536", "chunk", "bf16", B=1, H=32,
                                       T=65536, dk=128, dv=128, num_seqs=8, pin_frac=0.05, seed=3)
# decode: B = independent sequences, T = consecutive single-token steps
KDA_DECODE_N256_H32 = WorkloadConfig("kda_decode_n256_h32", "decode", "bf16", B=256, H=32, T=512,
                                     dk=128, dv=128, random_s0=True, seed=4)
# every workload: the four chunked-forward shapes, then the decode workload
WORKLOADS = (TINY_KDA_F32, KDA_B2_H16_T4096, GDN_B1_H16_T8192, KDA_VARLEN_H32_T65536,
             KDA_DECODE_N256_H32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 value (ties to even), kept as
    float32. (For finite inputs the 32-bit sum below cannot overflow.)"""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("...i,...i->...", x, x))[..., None]
    x /= n
    return x


_THREADS = max(1, min(16, os.cpu_count() or 1))


def _blocks(seed: int, tid: int, lead, tail, fill):
    """Array of shape lead + tail; block (i, j) of the two leading axes is filled by
    fill(rng, tail) with rng = default_rng([seed, tid, i, j])."""
    out = np.empty(tuple(lead) + tuple(tail), np.float32)

    def one(ij):
        i, j = ij
        out[i, j] = fill(np.random.default_rng([seed, tid, i, j]), tail)

    jobs = [(i, j) for i in range(lead[0]) for j in range(lead[1])]
    if len(jobs) == 1 or int(np.prod(tail)) < 65536:
        for ij in jobs:
            one(ij)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(one, jobs))
    return out


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _unit_normal(rng, shape):
    return _l2_normalise(rng.standard_normal(shape, dtype=np.float32))


def _sigmoid_normal(rng, shape):
    return _sigmoid(rng.standard_normal(shape, dtype=np.float32))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _log_decay(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    x -= np.float32(3.0)
    np.exp(x, out=x)
    np.negative(x, out=x)
    np.maximum(x, np.float32(G_FLOOR), out=x)
    return x


def varlen_lengths(rng: np.random.Generator, num_seqs: int, total: int,
                   lo: int = 1024, hi: int = 16384, chunk: int = 64) -> np.ndarray:
    """Sequence lengths drawn uniformly from [lo, hi], rescaled to sum to ``total``.

    Rescaling floors each length; the remainder adds one token to the first
    sequences. A length that is a multiple of ``chunk`` moves one token to the
    next sequence (cyclically), so that every sequence ends in a partial chunk.
    """
    raw = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int64)
    lens = np.floor(raw * (total / raw.sum())).astype(np.int64)
    rem = total - int(lens.sum())
    lens[:rem] += 1
    for _ in range(4 * num_seqs):
        bad = np.nonzero(lens % chunk == 0)[0]
        if bad.size == 0:
            break
        i = int(bad[0])
        lens[i] -= 1
        lens[(i + 1) % num_seqs] += 1
    assert lens.sum() == total and np.all(lens > 0)
    return lens


@dataclass
class ChunkInputs:
    cfg: WorkloadConfig
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    s0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    erase: Optional[np.ndarray] = None   # [B, H, T, dk] (Gated Delta Rule-2)
    write: Optional[np.ndarray] = None   # [B, H, T, dv]

    @property
    def n_seqs(self) -> int:
        return len(self.cu_seqlens) - 1 if self.cu_seqlens is not None else self.q.shape[0]

    def chain_rows(self, n: int, h: int):
        """(batch index, first token, length) of sequence n, head h."""
        if self.cu_seqlens is not None:
            a, b = int(self.cu_seqlens[n]), int(self.cu_seqlens[n + 1])
            return 0, a, b - a
        return n, 0, self.q.shape[2]


def make_chunk_inputs(cfg: WorkloadConfig) -> ChunkInputs:
    """Inputs of a prefill workload (or of a smaller case built with ``cfg.replace``)."""
    assert cfg.kind == "chunk"
    B, H, T, dk, dv, sd = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.seed
    q = _blocks(sd, 0, (B, H), (T, dk), _unit_normal)
    k = _blocks(sd, 1, (B, H), (T, dk), _unit_normal)
    v = _blocks(sd, 2, (B, H), (T, dv), _normal)
    if cfg.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    beta = _blocks(sd, 3, (B, H), (T,), _sigmoid_normal)
    g = _blocks(sd, 4, (B, H), (T, dk) if cfg.gate == "channel" else (T,), _log_decay)
    n_seqs = cfg.num_seqs if cfg.num_seqs else B
    s0 = None
    if cfg.random_s0:
        s0 = _blocks(sd, 5, (n_seqs, H), (dk, dv), _normal)
        s0 *= np.float32(0.02)
    cu = None
    if cfg.num_seqs:
        assert B == 1
        lens = varlen_lengths(np.random.default_rng([sd, 6]), cfg.num_seqs, T)
        cu = np.zeros(cfg.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
    if cfg.pin_frac > 0:
        pin = np.random.default_rng([sd, 7]).random((B, H, T)) < cfg.pin_frac
        g[pin] = np.float32(G_FLOOR)
    erase = write = None
    if cfg.gates == "gdr2":
        erase = _blocks(sd, 8, (B, H), (T, dk), _sigmoid_normal)
        write = _blocks(sd, 9, (B, H), (T, dv), _sigmoid_normal)
    return ChunkInputs(cfg, q, k, v, g, beta, s0, cu, erase, write)


@dataclass
class DecodeInputs:
    q: np.ndarray      # [N, H, dk]
    k: np.ndarray      # [N, H, dk]
    v: np.ndarray      # [N, H, dv]
    g: np.ndarray      # [N, H, dk] or [N, H]
    beta: np.ndarray   # [N, H]
    erase: Optional[np.ndarray] = None   # [N, H, dk] (Gated Delta Rule-2)
    write: Optional[np.ndarray] = None   # [N, H, dv]


def decode_initial_state(cfg: WorkloadConfig) -> np.ndarray:
    """Resident fp32 state [N, H, dk, dv] ~ N(0, 0.02^2) (zeros if the workload has none)."""
    N, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    if not cfg.random_s0:
        return np.zeros((N, H, dk, dv), np.float32)
    s = _blocks(cfg.seed, 5, (N, H), (dk, dv), _normal)
    s *= np.float32(0.02)
    return s


def decode_step_inputs(cfg: WorkloadConfig, step: int) -> DecodeInputs:
    """Inputs of decode step ``step`` (0-based); each step has its own seeded streams."""
    assert cfg.kind == "decode"
    rng = lambda tid: np.random.default_rng([cfg.seed, 100 + tid, step])  # noqa: E731
    N, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = _unit_normal(rng(0), (N, H, dk))
    k = _unit_normal(rng(1), (N, H, dk))
    v = _normal(rng(2), (N, H, dv))
    if cfg.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    beta = _sigmoid_normal(rng(3), (N, H))
    g = _log_decay(rng(4), (N, H, dk) if cfg.gate == "channel" else (N, H))
    erase = write = None
    if cfg.gates == "gdr2":
        erase = _sigmoid_normal(rng(5), (N, H, dk))
        write = _sigmoid_normal(rng(6), (N, H, dv))
    return DecodeInputs(q, k, v, g, beta, erase, write)


@dataclass
class GateInputs:
    """Pre-activations of the prologue and the epilogue (head-major, float32; the q / k /
    z values are bf16-rounded for bf16 workloads)."""
    q_in: np.ndarray      # [B, H, T, dk] before L2Norm
    k_in: np.ndarray
    u: np.ndarray         # [B, H, T, dk] decay pre-activation
    A_log: np.ndarray     # [H]
    dt_bias: np.ndarray   # [H, dk]
    beta_in: np.ndarray   # [B, H, T]
    z: np.ndarray         # [B, H, T, dv] output-gate pre-activation
    weight: np.ndarray    # [dv] RMSNorm weight


def make_gate_inputs(cfg: WorkloadConfig) -> GateInputs:
    """Synthetic pre-activations in the ranges of a Mamba-style parameterization: raw q, k,
    u, z and the beta pre-activation ~ N(0, 1); dt_bias = log(expm1(dt)) with dt
    log-uniform in [1e-3, 1e-1]; A_log = log U[1, 16]; weight = 1 + N(0, 0.1^2). With these
    the prologue's log-decay has median about -0.09, 95% of it in [-1.6, 0], and about
    0.5% of it on the lower bound -5."""
    B, H, T, dk, dv, sd = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.seed
    q_in = _blocks(sd, 10, (B, H), (T, dk), _normal)
    k_in = _blocks(sd, 11, (B, H), (T, dk), _normal)
    z = _blocks(sd, 12, (B, H), (T, dv), _normal)
    if cfg.dtype == "bf16":
        q_in, k_in, z = bf16_round(q_in), bf16_round(k_in), bf16_round(z)
    u = _blocks(sd, 13, (B, H), (T, dk), _normal)
    beta_in = _blocks(sd, 14, (B, H), (T,), _normal)
    rng = np.random.default_rng([sd, 15])
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(H, dk)))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    weight = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    return GateInputs(q_in, k_in, u, A_log, dt_bias, beta_in, z, weight)


@dataclass
class Cotangents:
    """Gradients of a loss with respect to the forward's outputs, for the backward pass."""
    do: np.ndarray      # [B, H, T, dv], ~ N(0, 1) (bf16-rounded for bf16 workloads)
    dsT: np.ndarray     # [N, H, dk, dv], ~ N(0, 0.1^2)


def make_cotangents(cfg: WorkloadConfig, n_seqs: int) -> Cotangents:
    """Seeded cotangents of a prefill workload (tensor ids 16 and 17)."""
    B, H, T, dk, dv, sd = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.seed
    do = _blocks(sd, 16, (B, H), (T, dv), _normal)
    if cfg.dtype == "bf16":
        do = bf16_round(do)
    dsT = (np.float32(0.1) * _blocks(sd, 17, (n_seqs, H), (dk, dv), _normal)).astype(np.float32)
    return Cotangents(do, dsT)


@dataclass
class LongChainInputs:
    """Device tensors of one packed axis of T tokens (B = 1): q, k, v bf16 [1, H, T, 128],
    g float32 [1, H, T, 128], beta float32 [1, H, T] (KDA) or erase / write float32
    [1, H, T, 128] (Gated Delta Rule-2), s0 float32 [N, H, 128, 128] or None."""
    q: object
    k: object
    v: object
    g: object
    beta: object
    erase: object
    write: object
    s0: object


def make_long_chain_inputs(T: int, H: int, seed: int, device, gdr2: bool = False,
                           n_seqs: int = 1, random_s0: bool = True,
                           gate: str = "channel") -> LongChainInputs:
    """Inputs of the long-chain cases, drawn on ``device`` with torch's seeded generator (an
    axis of millions of tokens takes too long to draw on the host). Same distributions as
    ``make_chunk_inputs``: q and k unit-norm rows of normals, v normals (the three rounded to
    bf16), beta and the Gated Delta Rule-2 gates sigmoids of normals, g the per-channel log
    decay -exp(N(0, 1) - 3) floored at G_FLOOR ([1, H, T, 128], or [1, H, T] with
    gate="head"), s0 normals times 0.02. Callers place runs of g = G_FLOOR themselves
    (``set_floor``)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(*shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    def unit_rows():
        x = normal(1, H, T, 128)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(torch.bfloat16)

    q = unit_rows()
    k = unit_rows()
    v = normal(1, H, T, 128).to(torch.bfloat16)
    g = normal(1, H, T, 128) if gate == "channel" else normal(1, H, T)
    g -= 3.0
    g.exp_().neg_().clamp_(min=G_FLOOR)
    beta = erase = write = None
    if gdr2:
        erase = torch.sigmoid(normal(1, H, T, 128))
        write = torch.sigmoid(normal(1, H, T, 128))
    else:
        beta = torch.sigmoid(normal(1, H, T))
    s0 = normal(n_seqs, H, 128, 128) * 0.02 if random_s0 else None
    return LongChainInputs(q, k, v, g, beta, erase, write, s0)


def set_floor(g, start: int, length: int) -> None:
    """Sets g = G_FLOOR on every head (and channel) of tokens start .. start + length - 1 of a
    [1, H, T, dk] or [1, H, T] log-decay tensor (in place)."""
    g[:, :, start:start + length] = G_FLOOR
