"""Plants plausible mistakes in a copy of the oracle's recurrence (on the CPU) and
checks that every one of them fails at least one pin: the pins are sharp enough to
catch a dropped term, a wrong sign, a wrong order or a transposed operand."""

import numpy as np
import pytest

from tests import pins


def _make(mut):
    def impl(q, k, v, g, beta, s0=None, erase=None, write=None):
        q, k, v = (np.asarray(x, float) for x in (q, k, v))
        T, dk = k.shape
        dv = v.shape[1]
        gg = np.asarray(g, float)
        gg = gg if gg.ndim == 2 else np.repeat(gg[:, None], dk, axis=1)
        e = beta if erase is None else erase
        w = beta if write is None else write
        S = np.zeros((dk, dv)) if s0 is None else np.array(s0, float)
        o = np.zeros((T, dv))
        G = np.zeros(dk)
        for t in range(T):
            a = np.exp(gg[t])
            G = G + gg[t]
            if mut == "decay_after_update":
                S = S + np.outer(k[t], w[t] * v[t] - S.T @ (e[t] * k[t]))
                S = a[:, None] * S
            elif mut == "predict_from_undecayed":
                p = S.T @ (e[t] * k[t])
                S = a[:, None] * S + np.outer(k[t], w[t] * v[t] - p)
            elif mut == "cumulative_decay":
                S = np.exp(G)[:, None] * S
                S = S + np.outer(k[t], w[t] * v[t] - S.T @ (e[t] * k[t]))
            else:
                S = a[:, None] * S if mut != "no_decay" else S
                p = S.T @ k[t]
                pe = S.T @ (e[t] * k[t])   # read along the erase-gated key
                if mut == "erase_without_beta":
                    S = S + np.outer(k[t], w[t] * v[t] - p)
                elif mut == "erase_sign":
                    S = S + np.outer(k[t], w[t] * v[t] + pe)
                elif mut == "predict_with_query":
                    S = S + np.outer(k[t], w[t] * v[t] - S.T @ (e[t] * q[t]))
                elif mut == "write_without_beta":
                    S = S + np.outer(k[t], v[t] - pe)
                elif mut == "erase_gate_on_write_factor":   # b on the left factor
                    S = S + np.outer(e[t] * k[t], w[t] * v[t] - p)
                elif mut == "write_gate_on_residual":       # w on the whole residual
                    S = S + np.outer(k[t], w[t] * (v[t] - pe))
                else:
                    S = S + np.outer(k[t], w[t] * v[t] - pe)
            if mut == "readout_before_update_order":
                o[t] = (S - np.outer(k[t], w[t] * v[t])).T @ q[t]
            elif mut == "readout_with_key":
                o[t] = S.T @ k[t]
            elif mut == "readout_transposed_gate":
                o[t] = S.T @ (q[t] * np.exp(gg[t]))
            else:
                o[t] = S.T @ q[t]
        return o, S
    return impl


MUTANTS = ["decay_after_update", "predict_from_undecayed", "cumulative_decay", "no_decay",
           "erase_without_beta", "erase_sign", "predict_with_query", "write_without_beta",
           "readout_before_update_order", "readout_with_key", "readout_transposed_gate",
           "erase_gate_on_write_factor", "write_gate_on_residual"]


def test_unmutated_copy_passes_all_pins():
    impl = _make(None)
    for pin in pins.ALL_PINS:
        pin(impl)


@pytest.mark.parametrize("mut", MUTANTS)
def test_mutant_fails_a_pin(mut):
    impl = _make(mut)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {mut} passed every pin"


GATE_MUTANTS = {
    "l2norm_without_sqrt": ("l2norm", lambda G: lambda x: np.asarray(x, float) / (
        np.sum(np.asarray(x, float) ** 2, axis=-1, keepdims=True) + G.EPS_L2)),
    "softplus_as_relu": ("softplus", lambda G: lambda x: np.maximum(np.asarray(x, float), 0.0)),
    "decay_without_lower_bound": ("decay_gate", lambda G: lambda u, A_log, dt_bias: -np.exp(
        np.asarray(A_log, float)).reshape(1, -1, 1, 1) * G.softplus(np.asarray(u, float) + np.asarray(
            dt_bias, float).reshape(1, len(A_log), 1, -1))),
    "rms_as_sum": ("epilogue", lambda G: lambda o, z, w, eps: G.sigmoid(z) * np.asarray(o) / np.sqrt(
        np.sum(np.asarray(o) ** 2, axis=-1, keepdims=True) + eps) * w),
    "gate_on_input": ("epilogue", lambda G: lambda o, z, w, eps: G.sigmoid(o) * np.asarray(z) / np.sqrt(
        np.mean(np.asarray(z) ** 2, axis=-1, keepdims=True) + eps) * w),
}


@pytest.mark.parametrize("mut", sorted(GATE_MUTANTS))
def test_gate_mutant_fails_a_pin(mut, monkeypatch):
    from oracle import gates as G
    name, make = GATE_MUTANTS[mut]
    monkeypatch.setattr(G, name, make(G))
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            pins.pins_gates()
