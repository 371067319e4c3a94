"""Seeded synthetic inputs for the gated delta rule forward (KDA / Gated DeltaNet).

This package is shared by the fp64 oracle's tests and by the GPU path's tests and
benchmark. It only draws random numbers and shapes them (normal draws, L2
normalisation of query/key vectors, sigmoid for the write strength, the clipped
log-decay, bf16 rounding of values handed to a bf16 kernel). It contains none of
the method's arithmetic: no decay, no state update, no chunking.
"""

from .generate import (  # noqa: F401
    GDN_B1_H16_T8192,
    KDA_B2_H16_T4096,
    KDA_DECODE_N256_H32,
    KDA_VARLEN_H32_T65536,
    TINY_KDA_F32,
    WORKLOADS,
    ChunkInputs,
    Cotangents,
    DecodeInputs,
    GateInputs,
    LongChainInputs,
    WorkloadConfig,
    bf16_round,
    decode_step_inputs,
    decode_initial_state,
    make_chunk_inputs,
    make_cotangents,
    make_gate_inputs,
    make_long_chain_inputs,
    set_floor,
    varlen_lengths,
)
