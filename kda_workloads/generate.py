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
Draw order: q, k, v, beta, g, s0, then sequence lengths and pinned rows.
"""

from __future__ import annotations

import dataclasses
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

    @property
    def n_chains(self) -> int:
        n = self.num_seqs if self.num_seqs else self.B
        return n * self.H

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = [
    WorkloadConfig("tiny_kda_f32", "chunk", "f32", B=1, H=2, T=256, dk=64, dv=64, seed=0),
    WorkloadConfig("kda_bf16_b2_h16_t4096", "chunk", "bf16", B=2, H=16, T=4096, dk=128, dv=128,
                   random_s0=True, seed=1),
    WorkloadConfig("gdn_bf16_b1_h16_t8192", "chunk", "bf16", B=1, H=16, T=8192, dk=128, dv=128,
                   gate="head", seed=2),
    WorkloadConfig("kda_bf16_varlen_h32_t65536", "chunk", "bf16", B=1, H=32, T=65536, dk=128,
                   dv=128, num_seqs=8, pin_frac=0.05, seed=3),
    # decode: B = independent sequences, T = consecutive single-token steps
    WorkloadConfig("kda_decode_n256_h32", "decode", "bf16", B=256, H=32, T=512, dk=128, dv=128,
                   random_s0=True, seed=4),
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _log_decay(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32) - np.float32(3.0)
    return np.maximum(np.float32(G_FLOOR), -np.exp(x)).astype(np.float32)


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
    rng = np.random.default_rng(cfg.seed)
    B, H, T, dk, dv = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv
    q = _l2_normalise(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if cfg.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    beta = _sigmoid(rng.standard_normal((B, H, T), dtype=np.float32))
    g = _log_decay(rng, (B, H, T, dk) if cfg.gate == "channel" else (B, H, T))
    n_seqs = cfg.num_seqs if cfg.num_seqs else B
    s0 = None
    if cfg.random_s0:
        s0 = (rng.standard_normal((n_seqs, H, dk, dv), dtype=np.float32) * np.float32(0.02))
    cu = None
    if cfg.num_seqs:
        assert B == 1
        lens = varlen_lengths(rng, cfg.num_seqs, T)
        cu = np.zeros(cfg.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
    if cfg.pin_frac > 0:
        pin = rng.random((B, H, T)) < cfg.pin_frac
        g[pin] = np.float32(G_FLOOR)
    return ChunkInputs(cfg, q, k, v, g, beta, s0, cu)


@dataclass
class DecodeInputs:
    q: np.ndarray      # [N, H, dk]
    k: np.ndarray      # [N, H, dk]
    v: np.ndarray      # [N, H, dv]
    g: np.ndarray      # [N, H, dk] or [N, H]
    beta: np.ndarray   # [N, H]


def decode_initial_state(cfg: WorkloadConfig) -> np.ndarray:
    """Resident fp32 state [N, H, dk, dv] ~ N(0, 0.02^2) (zeros if the workload has none)."""
    shape = (cfg.B, cfg.H, cfg.dk, cfg.dv)
    if not cfg.random_s0:
        return np.zeros(shape, np.float32)
    rng = np.random.default_rng([cfg.seed, 0])
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)


def decode_step_inputs(cfg: WorkloadConfig, step: int) -> DecodeInputs:
    """Inputs of decode step ``step`` (0-based); each step has its own seeded stream."""
    assert cfg.kind == "decode"
    rng = np.random.default_rng([cfg.seed, step + 1])
    N, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = _l2_normalise(rng.standard_normal((N, H, dk), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((N, H, dk), dtype=np.float32))
    v = rng.standard_normal((N, H, dv), dtype=np.float32)
    if cfg.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    beta = _sigmoid(rng.standard_normal((N, H), dtype=np.float32))
    g = _log_decay(rng, (N, H, dk) if cfg.gate == "channel" else (N, H))
    return DecodeInputs(q, k, v, g, beta)
