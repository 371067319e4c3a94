"""The oracle against its pins (closed forms, the pages' other equations, brute force,
the page-4 worked example and invariants), on the C oracle and on its numpy twin."""

import numpy as np
import pytest

import oracle
from oracle import reference as ref
from tests import pins


def c_oracle(q, k, v, g, beta, s0=None, erase=None, write=None):
    T = k.shape[0]
    o, sf = oracle.kda_chains(q, k, v, g, beta, [0], [T],
                              s0=None if s0 is None else np.asarray(s0)[None],
                              erase=erase, write=write, threads=1)
    return o, sf[0]


def numpy_twin(q, k, v, g, beta, s0=None, erase=None, write=None):
    return ref.recurrence(q, k, v, g, beta, s0=s0, erase=erase, write=write)


IMPLS = {"c_oracle": c_oracle, "numpy_twin": numpy_twin}


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("impl", list(IMPLS), ids=str)
def test_pin(pin, impl):
    pin(IMPLS[impl])


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_c_oracle_matches_numpy_twin(gate):
    q, k, v, g, beta, s0 = pins.case(200, 16, 12, seed=41, gate=gate, strong=True)
    e = np.random.default_rng(2).random(200)
    w = np.random.default_rng(3).random(200)
    ev = np.random.default_rng(4).random((200, 16))   # Gated Delta Rule-2 vector gates
    wv = np.random.default_rng(6).random((200, 12))
    for kw in ({}, {"s0": s0}, {"s0": s0, "erase": e, "write": w},
               {"s0": s0, "erase": ev, "write": wv}):
        o1, S1 = c_oracle(q, k, v, g, beta, **kw)
        o2, S2 = numpy_twin(q, k, v, g, beta, **kw)
        np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-12)


def test_forward_varlen_equals_separate_chains():
    """Packed sequences are independent: one call over cu_seqlens equals per-chain calls,
    and the head-major indexing picks the right rows for every (sequence, head)."""
    rng = np.random.default_rng(5)
    H, T, dk, dv = 3, 90, 8, 6
    q = pins._unit(rng.standard_normal((1, H, T, dk)))
    k = pins._unit(rng.standard_normal((1, H, T, dk)))
    v = rng.standard_normal((1, H, T, dv))
    g = -rng.random((1, H, T, dk))
    beta = rng.random((1, H, T))
    cu = np.array([0, 17, 17 + 40, T])
    s0 = rng.standard_normal((3, H, dk, dv))
    res = oracle.kda_forward(q, k, v, g, beta, s0=s0, cu_seqlens=cu)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            o, S = ref.recurrence(q[0, h, a:b], k[0, h, a:b], v[0, h, a:b], g[0, h, a:b],
                                  beta[0, h, a:b], s0=s0[n, h])
            np.testing.assert_allclose(res[(n, h)][0], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res[(n, h)][1], S, rtol=1e-12, atol=1e-12)
    sub = oracle.kda_forward(q, k, v, g, beta, s0=s0, cu_seqlens=cu, chains=[(2, 1)])
    np.testing.assert_array_equal(sub[(2, 1)][0], res[(2, 1)][0])


def test_decode_step_equals_one_token_forward():
    rng = np.random.default_rng(6)
    N, H, dk, dv = 3, 2, 8, 5
    S = rng.standard_normal((N, H, dk, dv))
    q = pins._unit(rng.standard_normal((N, H, dk)))
    k = pins._unit(rng.standard_normal((N, H, dk)))
    v = rng.standard_normal((N, H, dv))
    g = -rng.random((N, H, dk))
    beta = rng.random((N, H))
    o, S1 = oracle.kda_decode_step(S, q, k, v, g, beta)
    for n in range(N):
        for h in range(H):
            oo, SS = ref.recurrence(q[n, h][None], k[n, h][None], v[n, h][None],
                                    g[n, h][None], beta[n, h][None], s0=S[n, h])
            np.testing.assert_allclose(o[n, h], oo[0], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S1[n, h], SS, rtol=1e-12, atol=1e-12)


def test_gates_pins():
    pins.pins_gates()


@pytest.mark.parametrize("kind", ["channel", "head", "gdr2"])
def test_a_floor_run_forgets_the_state(kind):
    """The premise of the long-chain GPU checks, on the oracle: after 32 tokens of the floor
    decay g = -5 on every channel, the outputs no longer depend on the state that entered the
    run (each token map has norm at most 2 e^-5 for unit keys and gates in [0, 1], so the
    entering state is scaled by less than 1e-60), while before the run's end they still do.
    The large initial state (Frobenius norm about 4000) makes any leak visible."""
    q, k, v, g, beta, s0 = pins.case(260, 128, 128, seed=77, gate="channel" if kind != "head"
                                     else "head")
    s0 = s0 * 100.0
    rng = np.random.default_rng(78)
    ew = {} if kind != "gdr2" else {"erase": rng.random((260, 128)), "write": rng.random((260, 128))}
    g = g.copy()
    g[100:132] = -5.0
    o_full, S_full = c_oracle(q, k, v, g, beta, s0=s0, **ew)
    cut = {n: (a[100:] if a.ndim else a) for n, a in ew.items()}
    o_cut, S_cut = c_oracle(q[100:], k[100:], v[100:], g[100:], beta[100:], **cut)
    after, during = o_full[132:], o_full[100:132]
    scale = float(np.max(np.abs(after)))
    assert np.max(np.abs(after - o_cut[32:])) <= 1e-12 * scale
    assert np.max(np.abs(S_full - S_cut)) <= 1e-12 * float(np.max(np.abs(S_full)))
    # not vacuous: inside the run the entering state still shows
    assert np.max(np.abs(during - o_cut[:32])) > 1e-6 * float(np.max(np.abs(during)))
