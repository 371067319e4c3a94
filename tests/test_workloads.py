"""The seeded input generator: determinism, shapes, bf16 rounding and the varlen recipe."""

import numpy as np
import pytest
import torch

from kda_workloads import (KDA_DECODE_N256_H32, KDA_VARLEN_H32_T65536, WORKLOADS, bf16_round,
                           decode_step_inputs, make_chunk_inputs, varlen_lengths)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # ties round to even
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(x), want)


def test_small_cases_are_deterministic_and_shaped():
    for cfg in WORKLOADS[:4]:
        small = cfg.replace(T=192 if not cfg.num_seqs else 1000, H=2, B=min(cfg.B, 2))
        a, b = make_chunk_inputs(small), make_chunk_inputs(small)
        for x, y in zip((a.q, a.k, a.v, a.g, a.beta), (b.q, b.k, b.v, b.g, b.beta)):
            np.testing.assert_array_equal(x, y)
        B, H, T = small.B, small.H, small.T
        assert a.q.shape == (B, H, T, small.dk) and a.v.shape == (B, H, T, small.dv)
        assert a.g.shape == ((B, H, T, small.dk) if small.gate == "channel" else (B, H, T))
        assert np.all(a.g >= -5.0) and np.all(a.g < 0.0)
        assert np.all((a.beta > 0) & (a.beta < 1))
        np.testing.assert_allclose(np.linalg.norm(a.q, axis=-1), 1.0, atol=1e-2)
        if small.dtype == "bf16":
            np.testing.assert_array_equal(a.q, bf16_round(a.q))
            np.testing.assert_array_equal(a.v, bf16_round(a.v))


def test_varlen_recipe():
    for seed in range(20):
        lens = varlen_lengths(np.random.default_rng(seed), 8, 65536)
        assert lens.sum() == 65536 and len(lens) == 8
        assert np.all(lens % 64 != 0)
        # rescaling keeps the ratio of any two lengths within 16384 / 1024
        assert lens.max() <= 16 * lens.min() + 16


def test_pinned_rows_fraction():
    cfg = KDA_VARLEN_H32_T65536.replace(T=20000)
    x = make_chunk_inputs(cfg)
    pinned = np.all(x.g == -5.0, axis=-1)
    assert 0.04 < pinned.mean() < 0.06
    assert x.cu_seqlens[0] == 0 and x.cu_seqlens[-1] == 20000


@pytest.mark.parametrize("step", [0, 7])
def test_decode_steps_differ_and_repeat(step):
    cfg = KDA_DECODE_N256_H32.replace(B=4, H=3)
    a, b = decode_step_inputs(cfg, step), decode_step_inputs(cfg, step)
    c = decode_step_inputs(cfg, step + 1)
    np.testing.assert_array_equal(a.q, b.q)
    assert not np.array_equal(a.q, c.q)
    assert a.g.shape == (4, 3, 128) and a.beta.shape == (4, 3)
