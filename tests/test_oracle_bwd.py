"""The backward oracle (kda_oracle_bwd.c and its numpy twin) against its pins: finite
differences of the pinned forward recurrence, closed forms, linearity; and plausible
mistakes planted in a copy of the numpy twin each fail at least one of them."""

import numpy as np
import pytest

import oracle
from oracle import reference as ref
from tests import pins


def c_oracle_bwd(q, k, v, g, beta, do, s0=None, dsT=None, erase=None, write=None):
    T = k.shape[0]
    out = oracle.kda_chains_bwd(q, k, v, g, beta, [0], [T], do,
                                s0=None if s0 is None else np.asarray(s0)[None],
                                dsT=None if dsT is None else np.asarray(dsT)[None],
                                erase=erase, write=write, threads=1)
    out["ds0"] = out["ds0"][0]
    return out


IMPLS = {"c_oracle": c_oracle_bwd, "numpy_twin": ref.recurrence_bwd}


@pytest.mark.parametrize("pin", pins.BWD_PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("impl", list(IMPLS), ids=str)
def test_bwd_pin(pin, impl):
    pin(IMPLS[impl])


@pytest.mark.parametrize("mode", ["channel", "head", "gdr2"])
def test_c_oracle_bwd_matches_numpy_twin(mode):
    """Several checkpoint segments (T = 150 > 2 x 64), an initial state."""
    q, k, v, g, beta, s0 = pins.case(150, 12, 9, seed=71, gate="head" if mode == "head" else
                                     "channel", strong=True)
    rng = np.random.default_rng(72)
    do, dsT = rng.standard_normal((150, 9)), rng.standard_normal((12, 9))
    gates = {"erase": rng.random((150, 12)), "write": rng.random((150, 9))} if mode == "gdr2" \
        else {}
    a = c_oracle_bwd(q, k, v, g, beta, do, s0=s0, dsT=dsT, **gates)
    b = ref.recurrence_bwd(q, k, v, g, beta, do, s0=s0, dsT=dsT, **gates)
    assert sorted(a) == sorted(b)
    for name in a:
        np.testing.assert_allclose(a[name], b[name], rtol=1e-11, atol=1e-12, err_msg=name)


def test_backward_varlen_equals_separate_chains():
    """kda_backward over packed sequences equals one call per chain, and dsT = None is a
    zero cotangent."""
    rng = np.random.default_rng(73)
    H, T, dk, dv = 2, 80, 6, 5
    q = pins._unit(rng.standard_normal((1, H, T, dk)))
    k = pins._unit(rng.standard_normal((1, H, T, dk)))
    v = rng.standard_normal((1, H, T, dv))
    g = -rng.random((1, H, T, dk))
    beta = rng.random((1, H, T))
    do = rng.standard_normal((1, H, T, dv))
    cu = np.array([0, 30, 31, T])
    s0 = rng.standard_normal((3, H, dk, dv))
    res = oracle.kda_backward(q, k, v, g, beta, do, s0=s0, cu_seqlens=cu)
    for n in range(3):
        for h in range(H):
            sl = slice(cu[n], cu[n + 1])
            want = ref.recurrence_bwd(q[0, h, sl], k[0, h, sl], v[0, h, sl], g[0, h, sl],
                                      beta[0, h, sl], do[0, h, sl], s0=s0[n, h])
            for name, x in want.items():
                np.testing.assert_allclose(res[(n, h)][name], x, rtol=1e-11, atol=1e-12,
                                           err_msg=f"{name} chain {(n, h)}")


def _mutant(mut):
    """A copy of the numpy backward with one planted mistake."""
    def bwd(q, k, v, g, beta, do, s0=None, dsT=None, erase=None, write=None):
        T, dk = k.shape
        dv = v.shape[1]
        g = np.asarray(g, float)
        a = np.exp(g if g.ndim == 2 else np.repeat(g[:, None], dk, axis=1))
        gdr2 = erase is not None
        E = erase if gdr2 else np.repeat(beta[:, None], dk, axis=1)
        W = write if gdr2 else np.repeat(beta[:, None], dv, axis=1)
        S = np.zeros((dk, dv)) if s0 is None else np.array(s0, float)
        St, D = [], []
        for t in range(T):
            S = a[t][:, None] * S
            St.append(S.copy())
            D.append(W[t] * v[t] - S.T @ (E[t] * k[t]))
            S = S + np.outer(k[t], D[t])
        dq, dkk, dvv, dg = np.zeros((T, dk)), np.zeros((T, dk)), np.zeros((T, dv)), np.zeros((T, dk))
        de, dw = np.zeros((T, dk)), np.zeros((T, dv))
        dS = np.zeros((dk, dv)) if dsT is None else np.array(dsT, float)
        for t in reversed(range(T)):
            Sp = St[t] + np.outer(k[t], D[t])
            if mut != "output_gradient_after_readout":
                dS = dS + np.outer(q[t], do[t])
            dq[t] = (St[t] if mut == "dq_from_decayed_state" else Sp) @ do[t]
            dd = dS.T @ k[t]
            dkk[t] = dS @ D[t]
            dw[t] = dd * v[t]
            dvv[t] = dd * (1.0 if mut == "dv_without_write_gate" else W[t])
            if mut != "drop_prediction_term":
                sign = 1.0 if mut == "prediction_sign" else -1.0
                dS = dS + sign * np.outer(E[t] * k[t], dd)
            r = -St[t] @ dd
            if mut != "dk_without_read_term":
                dkk[t] += E[t] * r
            de[t] = k[t] * r
            dg[t] = np.sum(dS * (Sp if mut == "dg_from_updated_state" else St[t]), axis=1)
            if mut != "undecayed_state_gradient":
                dS = a[t][:, None] * dS
            if mut == "output_gradient_after_readout":
                dS = dS + np.outer(q[t], do[t])
        out = {"dq": dq, "dk": dkk, "dv": dvv,
               "dg": dg if g.ndim == 2 else dg.sum(axis=1), "ds0": dS}
        if gdr2:
            out["derase"], out["dwrite"] = de, dw
        elif mut == "dbeta_write_part_only":
            out["dbeta"] = dw.sum(axis=1)
        else:
            out["dbeta"] = de.sum(axis=1) + dw.sum(axis=1)
        return out
    return bwd


BWD_MUTANTS = ["output_gradient_after_readout", "dq_from_decayed_state", "dv_without_write_gate",
               "drop_prediction_term", "prediction_sign", "dk_without_read_term",
               "dg_from_updated_state", "undecayed_state_gradient", "dbeta_write_part_only"]


def test_unmutated_backward_copy_passes():
    for pin in pins.BWD_PINS:
        pin(_mutant(None))


@pytest.mark.parametrize("mut", BWD_MUTANTS)
def test_backward_mutant_fails_a_pin(mut):
    failed = []
    for pin in pins.BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_mutant(mut))
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"backward mutant {mut} passed every pin"
