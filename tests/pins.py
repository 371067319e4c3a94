"""Pins of the oracle: checks against what the pages and the mathematics fix.

Each pin takes an implementation ``impl(q, k, v, g, beta, s0=None, erase=None,
write=None) -> (o [T, dv], S_T [dk, dv])`` of one chain and raises AssertionError
if it disagrees. The pins are written independently of the oracle's own code:
closed forms, other equations of the pages, brute-force products and invariants.
``tests/test_oracle_pins.py`` runs them on the C oracle and on its numpy twin;
``tests/test_oracle_mutants.py`` shows that plausible mistakes fail at least one.
"""

from __future__ import annotations

import os

import numpy as np

from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(T, dk, dv, seed, gate="channel", strong=False):
    """Small random chain: unit q, k; v ~ N(0,1); beta in (0,1); g in [-5, 0]."""
    rng = np.random.default_rng(seed)
    q = _unit(rng.standard_normal((T, dk)))
    k = _unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    shape = (T, dk) if gate == "channel" else (T,)
    if strong:
        g = -5.0 * rng.random(shape)
    else:
        g = np.maximum(-5.0, -np.exp(rng.standard_normal(shape) - 2.0))
    s0 = 0.3 * rng.standard_normal((dk, dv))
    return q, k, v, g, beta, s0


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * scale, f"{what}: max |diff| {err:.3e} > {tol:.1e} * {scale:.3g}"


def states_by_steps(impl, q, k, v, g, beta, s0, erase=None, write=None):
    """States after every token, by calling ``impl`` one token at a time."""
    S = s0
    out = []
    for t in range(k.shape[0]):
        sl = slice(t, t + 1)
        _, S = impl(q[sl], k[sl], v[sl], g[sl], beta[sl], s0=S,
                    erase=None if erase is None else erase[sl],
                    write=None if write is None else write[sl])
        out.append(S)
    return out


# ---------------------------------------------------------------------------------
def pin_basis_key_overwrite(impl):
    """Closed form for a basis key k = e_i (boxed KDA recurrence, "Token Mixer I",
    section "Kimi Delta Attention"): (I - beta e_i e_i^T) Diag(alpha) S + beta e_i v^T
    keeps every row j != i at alpha_j S[j] and sets row i to (1 - beta) alpha_i S[i] + beta v.
    The read-out is o = S^T q."""
    rng = np.random.default_rng(11)
    dk, dv = 6, 5
    for i, b in [(0, 0.3), (3, 1.0), (5, 0.0), (2, 0.75)]:
        S0 = rng.standard_normal((dk, dv))
        g = -rng.random(dk) * 3.0
        k = np.zeros(dk)
        k[i] = 1.0
        v = rng.standard_normal(dv)
        q = rng.standard_normal(dk)
        o, S = impl(q[None], k[None], v[None], g[None], np.array([b]), s0=S0)
        a = np.exp(g)
        want = a[:, None] * S0
        want[i] = (1.0 - b) * a[i] * S0[i] + b * v
        _close(S, want, 1e-12, "basis-key state")
        _close(o[0], want.T @ q, 1e-12, "basis-key read-out")


def pin_chunked_equals_recurrence(impl):
    """The pages' chunkwise form (WY representation + UT transform, "Token Mixer I",
    section "Kimi Delta Attention") equals the recurrence, for several chunk sizes and
    a partial last chunk, per-channel and per-head decay, with an initial state."""
    for gate in ("channel", "head"):
        q, k, v, g, beta, s0 = case(150, 12, 7, seed=3, gate=gate, strong=True)
        o, S = impl(q, k, v, g, beta, s0=s0)
        for C in (16, 37, 64):
            oc, Sc = ref.chunked(q, k, v, g, beta, s0=s0, C=C)
            _close(o, oc, 1e-10, f"chunked C={C} outputs ({gate})")
            _close(S, Sc, 1e-10, f"chunked C={C} final state ({gate})")


def pin_deltanet_alpha_one(impl):
    """alpha = 1 (g = 0) gives DeltaNet. Compared with the DeltaNet chunk algorithm of
    "Token Mixer I", section "Delta Networks" (UT transform, state in the transposed
    R^{dv x dk} orientation):
      T = [I + StrictLower(diag(beta) K K^T)]^-1 diag(beta), W = T K, U = T V,
      O = Q S^T + (Q K^T ⊙ M)(U - W S^T),  S <- S + (U - W S^T)^T K,
    and with one step of the SGD view of section "Linear Attention and the Gated Delta
    Rule": S <- S - beta grad_S 1/2 ||S^T k - v||^2."""
    q, k, v, _, beta, s0 = case(96, 10, 6, seed=5)
    g = np.zeros((96, 10))
    o, S = impl(q, k, v, g, beta, s0=s0)
    St = s0.T.copy()   # dv x dk
    C = 32
    out = np.zeros_like(o)
    for c0 in range(0, 96, C):
        sl = slice(c0, c0 + C)
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = K.shape[0]
        Tm = np.linalg.inv(np.eye(n) + np.tril(np.diag(b) @ K @ K.T, -1)) @ np.diag(b)
        W, U = Tm @ K, Tm @ V
        Vp = U - W @ St.T
        out[sl] = Q @ St.T + np.tril(Q @ K.T) @ Vp
        St = St + Vp.T @ K
    _close(o, out, 1e-10, "DeltaNet chunk outputs")
    _close(S, St.T, 1e-10, "DeltaNet chunk final state")
    # one SGD step on the online regression loss
    S1 = s0.copy()
    _, S_impl = impl(q[:1], k[:1], v[:1], g[:1], beta[:1], s0=S1)
    grad = np.outer(k[0], S1.T @ k[0] - v[0])
    _close(S_impl, S1 - beta[0] * grad, 1e-12, "SGD step")


def pin_gdn_scalar_gate(impl):
    """One decay per head gives Gated DeltaNet, "Token Mixer I", section "Linear
    Attention and the Gated Delta Rule": S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
    + beta_t k_t v_t^T (explicit dk x dk matrices here). A per-channel decay that is
    the same on every channel must give the same result."""
    q, k, v, g, beta, s0 = case(40, 8, 5, seed=7, gate="head", strong=True)
    o, S = impl(q, k, v, g, beta, s0=s0)
    St = s0.copy()
    want = np.zeros_like(o)
    for t in range(40):
        St = np.exp(g[t]) * (np.eye(8) - beta[t] * np.outer(k[t], k[t])) @ St \
            + beta[t] * np.outer(k[t], v[t])
        want[t] = St.T @ q[t]
    _close(o, want, 1e-11, "GDN outputs")
    _close(S, St, 1e-11, "GDN final state")
    ob, Sb = impl(q, k, v, np.repeat(g[:, None], 8, axis=1), beta, s0=s0)
    _close(ob, o, 1e-12, "broadcast per-channel decay outputs")
    _close(Sb, S, 1e-12, "broadcast per-channel decay state")


def pin_linear_attention(impl):
    """With erase 0, write 1 and alpha = 1 the update is plain linear attention,
    "Token Mixer I", section "Mamba2: Linear Attention with Decay": O = (Q K^T ⊙ M) V
    with M the inclusive causal mask (plus Q S_0 for an initial state). With the tied
    gate beta = 0 the state is frozen (o_t = S_0^T q_t), and with a decay it only decays:
    S_T = Diag(gamma_T) S_0."""
    T, dk, dv = 30, 7, 4
    q, k, v, _, beta, s0 = case(T, dk, dv, seed=9)
    zero = np.zeros(T)
    o, S = impl(q, k, v, np.zeros((T, dk)), beta, s0=s0, erase=zero, write=np.ones(T))
    M = np.tril(np.ones((T, T)))
    _close(o, (q @ k.T * M) @ v + q @ s0, 1e-11, "linear attention outputs")
    _close(S, s0 + k.T @ v, 1e-11, "linear attention final state")
    o0, S0 = impl(q, k, v, np.zeros((T, dk)), zero, s0=s0)
    _close(o0, q @ s0, 1e-12, "frozen-state outputs")
    _close(S0, s0, 1e-12, "frozen state")
    g = -np.random.default_rng(1).random((T, dk))
    _, Sd = impl(q, k, v, g, zero, s0=s0)
    _close(Sd, np.exp(g.sum(0))[:, None] * s0, 1e-12, "pure decay")


def pin_decayed_linear_attention(impl):
    """Erase 0, write 1 with decay: "Token Mixer I", section "Mamba2": o_t = sum_{i<=t}
    v_i (q_t^T Diag(gamma_t / gamma_i) k_i) + (Diag(gamma_t) S_0)^T q_t per channel, and
    O = ((Q K^T) ⊙ Gamma) V with Gamma_ij = gamma_i / gamma_j (i >= j) for one decay per head."""
    T, dk, dv = 24, 6, 5
    q, k, v, g, beta, s0 = case(T, dk, dv, seed=13, strong=True)
    e, w = np.zeros(T), np.ones(T)
    o, _ = impl(q, k, v, g, beta, s0=s0, erase=e, write=w)
    G = np.cumsum(g, axis=0)
    want = np.zeros((T, dv))
    for t in range(T):
        for i in range(t + 1):
            want[t] += v[i] * (q[t] @ (np.exp(G[t] - G[i]) * k[i]))
        want[t] += (np.exp(G[t])[:, None] * s0).T @ q[t]
    _close(o, want, 1e-11, "per-channel decayed linear attention")
    gh = g[:, 0]
    oh, _ = impl(q, k, v, gh, beta, erase=e, write=w)
    Gh = np.cumsum(gh)
    Gam = np.tril(np.exp(Gh[:, None] - Gh[None, :]))
    _close(oh, ((q @ k.T) * Gam) @ v, 1e-11, "scalar-decay linear attention")


def pin_exact_overwrite(impl):
    """"Token Mixer I", section "Gated DeltaNet-2 / Preliminary": with ||k|| = 1 and
    beta = 1 the write overwrites the association of k, so S_t^T k_t = v_t; in general
    S_t^T k_t = (1 - beta) (Diag(alpha) S_{t-1})^T k_t + beta v_t."""
    T, dk, dv = 12, 9, 4
    q, k, v, g, beta, s0 = case(T, dk, dv, seed=17)
    sts = states_by_steps(impl, q, k, v, g, np.ones(T), s0)
    for t in range(T):
        _close(sts[t].T @ k[t], v[t], 1e-12, "beta=1 overwrite")
    sts = states_by_steps(impl, q, k, v, g, beta, s0)
    prev = s0
    for t in range(T):
        dec = np.exp(g[t])[:, None] * prev
        _close(sts[t].T @ k[t], (1 - beta[t]) * dec.T @ k[t] + beta[t] * v[t], 1e-12,
               "partial overwrite")
        prev = sts[t]


def pin_brute_force_products(impl):
    """Brute force on T <= 16: the states equal S^r = P^r S_0 + H^r with the explicit
    unrolled products of "Token Mixer I", section "Kimi Delta Attention", and the WY
    forms of the same section give the same P^r and H^r."""
    T, dk, dv = 16, 5, 3
    q, k, v, g, beta, s0 = case(T, dk, dv, seed=19, strong=True)
    sts = states_by_steps(impl, q, k, v, g, beta, s0)
    w, u, G = ref.wy_factors(k, v, g, beta)
    for r in range(1, T + 1):
        P, H = ref.brute_force_products(k, v, g, beta, r)
        _close(sts[r - 1], P @ s0 + H, 1e-12, f"unrolled products r={r}")
        Pw, Hw = ref.wy_products(k, w, u, G, r)
        _close(Pw, P, 1e-12, f"WY P r={r}")
        _close(Hw, H, 1e-12, f"WY H r={r}")


def pin_split_resume(impl):
    """The state is the whole context (page "【轻量化复刻大模型】线性注意力（Linear
    Attention）", section 4.0.1: each step reads S, modifies S, returns the output):
    running [0, T) equals running [0, T1) and then [T1, T) from the returned state."""
    q, k, v, g, beta, s0 = case(70, 8, 6, seed=23)
    o, S = impl(q, k, v, g, beta, s0=s0)
    T1 = 29
    o1, S1 = impl(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], s0=s0)
    o2, S2 = impl(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], s0=S1)
    _close(np.concatenate([o1, o2]), o, 1e-12, "split outputs")
    _close(S2, S, 1e-12, "split final state")


def pin_page4_capacity_demo(impl):
    """Page "【轻量化复刻大模型】线性注意力（Linear Attention）", section 4.1.8: the printed
    read-back of a 1-D state after five writes (fixture tests/golden/page4_capacity_demo.txt).
    beta = 0.5 and (1 - beta) alpha = 0.076 are inferred from the table (smoke pin)."""
    rows = np.loadtxt(os.path.join(GOLDEN, "page4_capacity_demo.txt"))
    vals, printed = rows[:, 0], rows[:, 1]
    n = len(vals)
    q = np.ones((n, 1))
    k = np.ones((n, 1))
    g = np.full((n, 1), np.log(0.076 / 0.5))
    o, _ = impl(q, k, vals[:, None], g, np.full(n, 0.5))
    assert np.array_equal(np.round(o[:, 0], 3), printed), (o[:, 0], printed)


def pin_invariants(impl):
    """Properties of the boxed recurrence ("Token Mixer I", section "Kimi Delta
    Attention"): linear in (V, S_0) jointly; permuting the key channels of q, k and g
    together permutes the rows of S and leaves O unchanged; value columns are
    independent; ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t|| for unit keys."""
    T, dk, dv = 20, 6, 5
    q, k, v, g, beta, s0 = case(T, dk, dv, seed=29, strong=True)
    rng = np.random.default_rng(31)
    v2, s2 = rng.standard_normal(v.shape), rng.standard_normal(s0.shape)
    o1, S1 = impl(q, k, v, g, beta, s0=s0)
    o2, S2 = impl(q, k, v2, g, beta, s0=s2)
    o3, S3 = impl(q, k, 2.0 * v - 0.5 * v2, g, beta, s0=2.0 * s0 - 0.5 * s2)
    _close(o3, 2.0 * o1 - 0.5 * o2, 1e-12, "linearity outputs")
    _close(S3, 2.0 * S1 - 0.5 * S2, 1e-12, "linearity state")
    perm = rng.permutation(dk)
    op, Sp = impl(q[:, perm], k[:, perm], v, g[:, perm], beta, s0=s0[perm])
    _close(op, o1, 1e-12, "channel permutation outputs")
    _close(Sp, S1[perm], 1e-12, "channel permutation state")
    cols = [4, 1]
    oc, Sc = impl(q, k, v[:, cols], g, beta, s0=s0[:, cols])
    _close(oc, o1[:, cols], 1e-12, "value-column independence outputs")
    _close(Sc, S1[:, cols], 1e-12, "value-column independence state")
    sts = states_by_steps(impl, q, k, v, g, beta, s0)
    prev = s0
    for t in range(T):
        assert np.linalg.norm(sts[t]) <= np.linalg.norm(prev) + beta[t] * np.linalg.norm(v[t]) \
            + 1e-12
        prev = sts[t]


# ---------------------------------------------------------------------------------
# Gated Delta Rule-2 ("Token Mixer I", section "Gated DeltaNet-2: Decoupling Erase and
# Write"): erase gate b_t in [0,1]^dk on the key side, write gate w_t in [0,1]^dv on the
# value side.

def _gdr2_gates(T, dk, dv, seed):
    rng = np.random.default_rng(seed)
    return rng.random((T, dk)), rng.random((T, dv))


def pin_gdr2_reduces_to_kda(impl):
    """The section states that b_t = beta_t 1 and w_t = beta_t 1 give KDA exactly."""
    q, k, v, g, beta, s0 = case(40, 12, 10, seed=61)
    o1, S1 = impl(q, k, v, g, beta, s0=s0)
    o2, S2 = impl(q, k, v, g, beta, s0=s0, erase=np.repeat(beta[:, None], 12, axis=1),
                  write=np.repeat(beta[:, None], 10, axis=1))
    _close(o2, o1, 1e-12, "b = w = beta 1 outputs")
    _close(S2, S1, 1e-12, "b = w = beta 1 state")


def pin_gdr2_write_only(impl):
    """With b = 0 nothing is erased: S_t = Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T, whose
    unrolled (parallel) form is the decayed linear attention of "Token Mixer I", section
    "Mamba2: Linear Attention with Decay", with per-channel decay and gated values:
    o_t = (q_t * gamma_t)^T S_0 + sum_{j<=t} (sum_c q_t[c] k_j[c] gamma_t[c] / gamma_j[c]) w_j * v_j,
    gamma_t = exp(sum_{s<=t} g_s)."""
    T, dk, dv = 14, 9, 7
    q, k, v, g, beta, s0 = case(T, dk, dv, seed=62)
    _, w = _gdr2_gates(T, dk, dv, 63)
    o, S = impl(q, k, v, g, beta, s0=s0, erase=np.zeros((T, dk)), write=w)
    G = np.cumsum(g, axis=0)
    z = w * v
    want = np.zeros((T, dv))
    for t in range(T):
        want[t] = (q[t] * np.exp(G[t])) @ s0
        for j in range(t + 1):
            want[t] += np.sum(q[t] * k[j] * np.exp(G[t] - G[j])) * z[j]
    _close(o, want, 1e-10, "write-only outputs")
    S_want = np.exp(G[-1])[:, None] * s0 + sum(
        np.outer(k[j] * np.exp(G[-1] - G[j]), z[j]) for j in range(T))
    _close(S, S_want, 1e-10, "write-only state")


def pin_gdr2_erase_direction(impl):
    """One token, no decay, nothing written: the erase matrix keeps k_t as its left factor
    and takes b_t * k_t as its right factor (the read direction), so
    S_1 = (I - k (b * k)^T) S_0 and o = S_1^T q. Zeroing one channel of b leaves the
    component of S_0 along that channel unread."""
    dk, dv = 8, 6
    q, k, v, g, beta, s0 = case(1, dk, dv, seed=64)
    b, _ = _gdr2_gates(1, dk, dv, 65)
    b[0, 3] = 0.0
    o, S = impl(q, k, v, np.zeros_like(g), beta, s0=s0, erase=b, write=np.zeros((1, dv)))
    S_want = (np.eye(dk) - np.outer(k[0], b[0] * k[0])) @ s0
    _close(S, S_want, 1e-12, "erase state")
    _close(o[0], S_want.T @ q[0], 1e-12, "erase output")
    s_mod = s0.copy()
    s_mod[3] += 1.0   # channel 3 is not read: changing its row moves S only along that row
    _, S2 = impl(q, k, v, np.zeros_like(g), beta, s0=s_mod, erase=b, write=np.zeros((1, dv)))
    d = S2 - S
    _close(np.delete(d, 3, axis=0), np.zeros((dk - 1, dv)), 1e-12, "unread channel")


# ---------------------------------------------------------------------------------
# Prologue / epilogue (oracle/gates.py): closed forms and special cases.

def pins_gates():
    """Pins of oracle/gates.py (raises AssertionError)."""
    from oracle import gates as G
    # L2Norm: a 3-4-5 triangle, unit length, scale invariance, the zero vector stays 0
    _close(G.l2norm(np.array([3.0, 4.0])), np.array([0.6, 0.8]), 1e-7, "l2norm 3-4-5")
    x = np.random.default_rng(71).standard_normal((5, 128)) * 7.0
    _close(np.linalg.norm(G.l2norm(x), axis=-1), np.ones(5), 1e-9, "l2norm unit")
    _close(G.l2norm(3.5 * x), G.l2norm(x), 1e-9, "l2norm scale")
    assert np.all(G.l2norm(np.zeros(8)) == 0.0)
    # softplus: log 2 at 0, -> x for large x, -> exp(x) for very negative x, odd part x
    _close(G.softplus(0.0), np.log(2.0), 1e-15, "softplus(0)")
    _close(G.softplus(60.0), 60.0, 1e-15, "softplus(60)")
    _close(G.softplus(-40.0), np.exp(-40.0), 1e-15, "softplus(-40)")
    t = np.linspace(-30, 30, 61)
    _close(G.softplus(t) - G.softplus(-t), t, 1e-12, "softplus(x) - softplus(-x) = x")
    # decay gate: -exp(A_log) softplus(dt_bias) at u = 0; never positive; head scaling
    A_log = np.log(np.array([0.5, 2.0]))
    dt_bias = np.linspace(-3, 1.5, 2 * 4)  # keeps every g at u = 0 above the bound
    g = G.decay_gate(np.zeros((1, 2, 3, 4)), A_log, dt_bias)
    want = -np.array([0.5, 2.0])[:, None] * np.log1p(np.exp(dt_bias.reshape(2, 4)))
    _close(g[0, :, 0, :], want, 1e-12, "decay gate at u = 0")
    u = np.random.default_rng(72).standard_normal((2, 2, 5, 4)) * 10
    gu = G.decay_gate(u, A_log, dt_bias)
    assert np.all(gu <= 0.0) and np.all(gu >= -5.0)
    # the lower bound g_min = -5: a large pre-activation saturates at exactly -5
    _close(G.decay_gate(np.full((1, 2, 1, 4), 50.0), A_log, dt_bias), np.full((1, 2, 1, 4), -5.0),
           0.0, "decay gate lower bound")
    # sigmoid: 1/2 at 0, symmetry, the logistic function
    _close(G.sigmoid(0.0), 0.5, 1e-15, "sigmoid(0)")
    _close(G.sigmoid(t) + G.sigmoid(-t), np.ones_like(t), 1e-12, "sigmoid symmetry")
    _close(G.sigmoid(1.3), 1.0 / (1.0 + np.exp(-1.3)), 1e-15, "sigmoid(1.3)")
    # epilogue: a constant row c gives sign(c) w / sqrt(1 + eps / c^2) * sigmoid(z);
    # z = 0 halves; invariant to the scale of o (up to eps); RMS of the result = weight
    w = np.linspace(0.5, 1.5, 16)
    o = np.full((1, 16), -3.0)
    _close(G.epilogue(o, np.zeros((1, 16)), w, 1e-6), -0.5 * w / np.sqrt(1 + 1e-6 / 9),
           1e-12, "epilogue constant row")
    o = np.random.default_rng(73).standard_normal((4, 16))
    z = np.random.default_rng(74).standard_normal((4, 16))
    _close(G.epilogue(o * 40.0, z, w, 0.0), G.epilogue(o, z, w, 0.0), 1e-12, "epilogue scale")
    y = G.epilogue(o, np.full_like(z, 50.0), np.ones(16), 0.0)
    _close(np.sqrt(np.mean(y * y, axis=-1)), np.ones(4), 1e-12, "epilogue unit RMS")
    # an all-zero row with eps > 0 maps to exactly 0 (0 / sqrt(eps)), whatever the gate
    y = G.epilogue(np.zeros((2, 16)), z[:2], w, 1e-6)
    assert np.all(y == 0.0), "epilogue zero row"


ALL_PINS = [
    pin_basis_key_overwrite,
    pin_chunked_equals_recurrence,
    pin_deltanet_alpha_one,
    pin_gdn_scalar_gate,
    pin_linear_attention,
    pin_decayed_linear_attention,
    pin_exact_overwrite,
    pin_brute_force_products,
    pin_split_resume,
    pin_page4_capacity_demo,
    pin_invariants,
    pin_gdr2_reduces_to_kda,
    pin_gdr2_write_only,
    pin_gdr2_erase_direction,
]


# ------------------------------------------------------------------ backward pass
# Each backward pin takes ``bwd(q, k, v, g, beta, do, s0=None, dsT=None, erase=None,
# write=None) -> dict`` (the gradients of sum(do * o) + sum(dsT * S_T); see
# oracle.reference.recurrence_bwd) and checks it against the definition of a derivative
# or against closed forms, using only the forward recurrence (pinned above).

def _loss(q, k, v, g, beta, do, s0, dsT, erase=None, write=None):
    o, S = ref.recurrence(q, k, v, g, beta, s0=s0, erase=erase, write=write)
    return float(np.sum(do * o) + np.sum(dsT * S))


def pin_bwd_finite_differences(bwd):
    """Central differences of the loss with respect to every input element (fp64, step
    1e-6: truncation and cancellation both below 1e-9 of the gradient's scale), for
    per-channel and per-head decay, with an initial state, and for the Gated Delta
    Rule-2 gates."""
    h = 1e-6
    for mode in ("channel", "head", "gdr2"):
        T, dk, dv = 9, 5, 4
        q, k, v, g, beta, s0 = case(T, dk, dv, seed=61, gate="head" if mode == "head" else
                                    "channel", strong=True)
        rng = np.random.default_rng(62)
        do = rng.standard_normal((T, dv))
        dsT = rng.standard_normal((dk, dv))
        gates = {}
        if mode == "gdr2":
            gates = {"erase": rng.random((T, dk)), "write": rng.random((T, dv))}
        got = bwd(q, k, v, g, beta, do, s0=s0, dsT=dsT, **gates)
        inputs = {"dq": q, "dk": k, "dv": v, "dg": g, "ds0": s0}
        if mode == "gdr2":
            inputs.update(derase=gates["erase"], dwrite=gates["write"])
        else:
            inputs["dbeta"] = beta
        for name, x in inputs.items():
            fd = np.zeros(x.shape)
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + h
                lp = _loss(q, k, v, g, beta, do, s0, dsT, **gates)
                x[idx] = keep - h
                lm = _loss(q, k, v, g, beta, do, s0, dsT, **gates)
                x[idx] = keep
                fd[idx] = (lp - lm) / (2 * h)
            _close(got[name], fd, 1e-7, f"finite differences {name} ({mode})")


def pin_bwd_linear_attention(bwd):
    """Erase 0, write 1, alpha = 1 is linear attention, o_t = sum_{s<=t} (q_t.k_s) v_s +
    S0^T q_t and S_T = S0 + K^T V ("Token Mixer I", section "Mamba2"); its gradients in
    closed form: dQ = (dO V^T ⊙ M) K + dO S0^T, dK = (dO V^T ⊙ M)^T Q + V dS_T^T,
    dV = (Q K^T ⊙ M)^T dO + K dS_T, dS0 = Q^T dO + dS_T, M the inclusive causal mask,
    and the write gate's gradient dW = dV ⊙ V (since dV = dd * 1)."""
    T, dk, dv = 14, 6, 5
    q, k, v, _, beta, s0 = case(T, dk, dv, seed=63)
    rng = np.random.default_rng(64)
    do = rng.standard_normal((T, dv))
    dsT = rng.standard_normal((dk, dv))
    M = np.tril(np.ones((T, T)))
    got = bwd(q, k, v, np.zeros((T, dk)), beta, do, s0=s0, dsT=dsT,
              erase=np.zeros((T, dk)), write=np.ones((T, dv)))
    _close(got["dq"], (do @ v.T * M) @ k + do @ s0.T, 1e-12, "linear attention dq")
    _close(got["dk"], (do @ v.T * M).T @ q + v @ dsT.T, 1e-12, "linear attention dk")
    dV = (q @ k.T * M).T @ do + k @ dsT
    _close(got["dv"], dV, 1e-12, "linear attention dv")
    _close(got["ds0"], q.T @ do + dsT, 1e-12, "linear attention ds0")
    _close(got["dwrite"], dV * v, 1e-12, "linear attention dwrite")


def pin_bwd_pure_decay(bwd):
    """With the tied gate beta = 0 and do = 0 the state only decays, S_T = Diag(exp sum_t
    g_t) S0: dS0 = Diag(exp sum_t g_t) dS_T, every token's dg_t = rowsum(dS_T ⊙ S_T) (the
    sum over channels for one decay per head), and dq = dv = 0."""
    T, dk, dv = 11, 6, 4
    for gate in ("channel", "head"):
        q, k, v, g, _, s0 = case(T, dk, dv, seed=65, gate=gate, strong=True)
        dsT = np.random.default_rng(66).standard_normal((dk, dv))
        got = bwd(q, k, v, g, np.zeros(T), np.zeros((T, dv)), s0=s0, dsT=dsT)
        gs = g.sum(axis=0) if gate == "channel" else np.full(dk, g.sum())
        ST = np.exp(gs)[:, None] * s0
        _close(got["ds0"], np.exp(gs)[:, None] * dsT, 1e-12, f"pure decay ds0 ({gate})")
        row = np.sum(dsT * ST, axis=1)
        want = np.tile(row, (T, 1)) if gate == "channel" else np.full(T, row.sum())
        _close(got["dg"], want, 1e-12, f"pure decay dg ({gate})")
        _close(got["dq"], np.zeros((T, dk)), 0.0, "pure decay dq")
        _close(got["dv"], np.zeros((T, dv)), 0.0, "pure decay dv")


def pin_bwd_linear_in_cotangents(bwd):
    """The gradients are linear in (do, dS_T): bwd(a do1 + b do2, a ds1 + b ds2) =
    a bwd(do1, ds1) + b bwd(do2, ds2), and zero cotangents give zero gradients."""
    T, dk, dv = 70, 8, 6   # crosses the oracle's 64-token checkpoint segments
    q, k, v, g, beta, s0 = case(T, dk, dv, seed=67, strong=True)
    rng = np.random.default_rng(68)
    do1, do2 = rng.standard_normal((2, T, dv))
    ds1, ds2 = rng.standard_normal((2, dk, dv))
    r1 = bwd(q, k, v, g, beta, do1, s0=s0, dsT=ds1)
    r2 = bwd(q, k, v, g, beta, do2, s0=s0, dsT=ds2)
    r3 = bwd(q, k, v, g, beta, 2.0 * do1 - 0.5 * do2, s0=s0, dsT=2.0 * ds1 - 0.5 * ds2)
    for name in r1:
        _close(r3[name], 2.0 * r1[name] - 0.5 * r2[name], 1e-12, f"linearity {name}")
    r0 = bwd(q, k, v, g, beta, np.zeros((T, dv)), s0=s0, dsT=np.zeros((dk, dv)))
    for name in r0:
        assert np.all(r0[name] == 0.0), f"zero cotangents give nonzero {name}"


BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_linear_attention,
    pin_bwd_pure_decay,
    pin_bwd_linear_in_cotangents,
]
