"""fp64 definitions of the steps on either side of the operator: the prologue that
turns per-token pre-activations into the operator's inputs and the epilogue that gates
and normalises its output.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): only the tests, the smoke check and the
benchmark's CPU baseline use this module; it shares nothing with the HIP library.

Sources ("Token Mixer I", section "The Kimi Linear Model Architecture", neural
parameterization; page "阅读笔记: Kimi Delta Attention", section 6, model architecture):
  q, k   = L2Norm(.) of the (short-convolved, Swish-activated) projections, per head and
           token, over the key channels;
  log a  = max(-exp(A_log) * softplus(u + dt_bias), g_min), u the low-rank projection of
           the token, A_log [H], dt_bias [H * dk]; computed in fp32 before the operator
           ("Token Mixer I", section "Gated DeltaNet-2", decay parameterization), with the
           lower bound g_min = -5 of KDA's decay (page "【轻量化复刻大模型】线性注意力（Linear
           Attention）", knowledge map of section 3.1, item 7a);
  beta   = Sigmoid(.) of its projection;
  out    = Sigmoid(z) * RMSNorm(o), per head over the value channels, z the low-rank
           projection of the output gate.
The pages print no epsilon for L2Norm or RMSNorm and no RMSNorm weight: L2Norm uses
x / sqrt(sum x^2 + eps_l2) with eps_l2 = 1e-6, RMSNorm uses o / sqrt(mean o^2 + eps) * w
with eps and the weight w [dv] as arguments.
"""

from __future__ import annotations

import numpy as np

EPS_L2 = 1e-6
G_MIN = -5.0


def l2norm(x):
    """x / sqrt(sum(x^2) + EPS_L2) over the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS_L2)


def softplus(x):
    """log(1 + exp(x)), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def decay_gate(u, A_log, dt_bias):
    """log-decay g = max(-exp(A_log[h]) * softplus(u + dt_bias[h, c]), G_MIN) for
    u [B, H, T, dk], A_log [H], dt_bias [H * dk] (head-major)."""
    u = np.asarray(u, dtype=np.float64)
    B, H, T, dk = u.shape
    a = np.exp(np.asarray(A_log, dtype=np.float64)).reshape(1, H, 1, 1)
    b = np.asarray(dt_bias, dtype=np.float64).reshape(1, H, 1, dk)
    return np.maximum(-a * softplus(u + b), G_MIN)


def prologue(q_in, k_in, u, A_log, dt_bias, beta_in):
    """(q, k, g, beta) from the pre-activations: L2Norm, decay gate, Sigmoid."""
    return l2norm(q_in), l2norm(k_in), decay_gate(u, A_log, dt_bias), sigmoid(beta_in)


def epilogue(o, z, weight, eps):
    """Sigmoid(z) * o / sqrt(mean(o^2) + eps) * weight over the last axis (dv)."""
    o = np.asarray(o, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return sigmoid(z) * o * r * np.asarray(weight, dtype=np.float64)
