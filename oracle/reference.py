"""numpy fp64 forms of the gated delta rule, used to pin the C oracle to the pages.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). Every function works on one
chain (one sequence of one head) with row-per-token arrays:
  q, k : [T, dk]   v : [T, dv]   g : [T, dk] (per key channel) or [T] (one per head)
  beta : [T]       state S : [dk, dv] (rows = key channels)
"""

from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _gate(g: np.ndarray, dk: int) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g if g.ndim == 2 else np.repeat(g[:, None], dk, axis=1)


def recurrence(q, k, v, g, beta, s0=None, erase=None, write=None, states=False):
    """Token-by-token recurrence, the numpy twin of ``kda_oracle.c``.

    "Token Mixer I", section "Kimi Delta Attention: Improving Delta Rule with
    Fine-grained Gating", boxed recurrence, evaluated in the decay-then-delta order of
    the page "KDA 与 Gated DeltaNet：线性注意力怎样读写有限状态", section 2:
      S~ = Diag(exp g_t) S;  S = S~ + k_t (w_t v_t - e_t S~^T k_t)^T;  o_t = S^T q_t,
    with e_t = w_t = beta_t (None) for the method. ``erase`` [T, dk] and ``write``
    [T, dv] are the per-channel gates of Gated Delta Rule-2 ("Token Mixer I", section
    "Gated DeltaNet-2"): S = S~ + k_t (w_t * v_t - S~^T (e_t * k_t))^T. Returns
    (o [T, dv], S_T) and, with ``states``, also the list of states after every token.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, dk = k.shape
    dv = v.shape[1]
    a = np.exp(_gate(g, dk))
    beta = np.asarray(beta, dtype=np.float64)
    e = beta if erase is None else np.asarray(erase, dtype=np.float64)
    w = beta if write is None else np.asarray(write, dtype=np.float64)
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((T, dv))
    hist = []
    for t in range(T):
        S = a[t][:, None] * S
        p = S.T @ (e[t] * k[t])
        S = S + np.outer(k[t], w[t] * v[t] - p)
        o[t] = S.T @ q[t]
        if states:
            hist.append(S.copy())
    return (o, S, hist) if states else (o, S)


def chunked(q, k, v, g, beta, s0=None, C=64):
    """The pages' chunkwise form (WY representation + UT transform), chunk size C.

    "Token Mixer I", section "Kimi Delta Attention", equations after the WY
    representation: per chunk with local cumulative log-decay G_r (gamma^r = exp G_r),
      M = (I + StrictTril(Diag(beta) (Gamma ⊙ K)(K / Gamma)^T))^-1 Diag(beta),
      W = M (Gamma ⊙ K),  U = M V,
      S' = Diag(gamma^C) S + (Gamma^{i->C} ⊙ K)^T (U - W S),
      O  = (Gamma ⊙ Q) S + Tril((Gamma ⊙ Q)(K / Gamma)^T) (U - W S),
    where Gamma^{i->C} row i is gamma^C / gamma^i. The products with K / Gamma are
    formed from exact pairwise exponent differences exp(G_i - G_j) (fp64), so no
    factor is ever divided by a small number. A last chunk shorter than C is
    processed with its own length. Returns (o [T, dv], S_T).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, dk = k.shape
    dv = v.shape[1]
    gg = _gate(g, dk)
    beta = np.asarray(beta, dtype=np.float64)
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = K.shape[0]
        G = np.cumsum(gg[sl], axis=0)                      # [n, dk], inclusive
        D = np.exp(G[:, None, :] - G[None, :, :])           # D[i, j, c] = gamma^i_c / gamma^j_c
        Akk = np.einsum("ic,jc,ijc->ij", K, K, D)           # (Gamma⊙K)(K/Gamma)^T
        Aqk = np.einsum("ic,jc,ijc->ij", Q, K, D)           # (Gamma⊙Q)(K/Gamma)^T
        L = np.eye(n) + np.tril(b[:, None] * Akk, -1)
        KG = K * np.exp(G)                                   # Gamma^{1->C} ⊙ K
        W = solve_triangular(L, b[:, None] * KG, lower=True, unit_diagonal=True)
        U = solve_triangular(L, b[:, None] * V, lower=True, unit_diagonal=True)
        Vp = U - W @ S                                       # pseudo-value
        o[sl] = (Q * np.exp(G)) @ S + np.tril(Aqk) @ Vp
        Kdec = K * np.exp(G[-1][None, :] - G)                # Gamma^{i->C} ⊙ K
        S = np.exp(G[-1])[:, None] * S + Kdec.T @ Vp
    return o, S


def brute_force_products(k, v, g, beta, r):
    """Explicit dk x dk products of the chunk expansion, first r tokens.

    "Token Mixer I", section "Kimi Delta Attention", chunk expansion:
      S^r = P^r S^0 + H^r,  P^r = prod_{i=r..1} [(I - beta_i k_i k_i^T) Diag(alpha_i)],
      H^r = sum_i (prod_{j=r..i+1} [(I - beta_j k_j k_j^T) Diag(alpha_j)]) beta_i k_i v_i^T,
    where later factors multiply on the left.
    """
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    dk, dv = k.shape[1], v.shape[1]
    gg = _gate(g, dk)
    P = np.eye(dk)
    H = np.zeros((dk, dv))
    for i in range(r):
        F = (np.eye(dk) - beta[i] * np.outer(k[i], k[i])) @ np.diag(np.exp(gg[i]))
        P = F @ P
        H = F @ H + beta[i] * np.outer(k[i], v[i])
    return P, H


def wy_factors(k, v, g, beta):
    """The WY auxiliaries w_r, u_r of "Token Mixer I", section "Kimi Delta Attention",
    WY representation (recursions written with gamma^{i->r} = prod_{j=i+1..r} alpha_j):
      w_r = beta_r (Diag(gamma^r) k_r - sum_{i<r} w_i (k_i^T Diag(gamma^{i->r}) k_r)),
      u_r = beta_r (v_r - sum_{i<r} u_i (k_i^T Diag(gamma^{i->r}) k_r)).
    Returns (w [T, dk], u [T, dv], G [T, dk]) with G the inclusive cumulative log-decay."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    T, dk = k.shape
    G = np.cumsum(_gate(g, dk), axis=0)
    w = np.zeros_like(k)
    u = np.zeros_like(v)
    for r in range(T):
        acc_w = np.exp(G[r]) * k[r]
        acc_u = v[r].copy()
        for i in range(r):
            c = k[i] @ (np.exp(G[r] - G[i]) * k[r])
            acc_w -= w[i] * c
            acc_u -= u[i] * c
        w[r] = beta[r] * acc_w
        u[r] = beta[r] * acc_u
    return w, u, G


def wy_products(k, w, u, G, r):
    """P^r = Diag(gamma^r) - sum_{i<=r} Diag(gamma^{i->r}) k_i w_i^T and
    H^r = sum_{i<=r} Diag(gamma^{i->r}) k_i u_i^T (same page and section)."""
    dk = k.shape[1]
    P = np.diag(np.exp(G[r - 1]))
    H = np.zeros((dk, u.shape[1]))
    for i in range(r):
        d = np.exp(G[r - 1] - G[i])
        P -= np.outer(d * k[i], w[i])
        H += np.outer(d * k[i], u[i])
    return P, H


def recurrence_bwd(q, k, v, g, beta, do, s0=None, dsT=None, erase=None, write=None):
    """Gradients of sum(do * o) + sum(dsT * S_T) for ``recurrence``, the numpy twin of
    ``kda_oracle_bwd.c``: the chain rule through the token step S~ = Diag(a) S,
    p = S~^T (e * k), d = w * v - p, S' = S~ + k d^T, o = S'^T q, in reverse token order
    (every state kept). Returns a dict with dq, dk, dv, dg (shaped like g), ds0 and
    dbeta (e = w = beta) or derase [T, dk] / dwrite [T, dv] (Gated Delta Rule-2)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    T, dk = k.shape
    dv = v.shape[1]
    g = np.asarray(g, dtype=np.float64)
    a = np.exp(_gate(g, dk))
    beta = np.asarray(beta, dtype=np.float64)
    gdr2 = erase is not None
    E = np.asarray(erase, np.float64) if gdr2 else np.repeat(beta[:, None], dk, axis=1)
    W = np.asarray(write, np.float64) if gdr2 else np.repeat(beta[:, None], dv, axis=1)
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    St, D = [], []
    for t in range(T):                       # forward, keeping S~ and d of every token
        S = a[t][:, None] * S
        St.append(S.copy())
        d = W[t] * v[t] - S.T @ (E[t] * k[t])
        D.append(d)
        S = S + np.outer(k[t], d)
    out = {"dq": np.zeros((T, dk)), "dk": np.zeros((T, dk)), "dv": np.zeros((T, dv)),
           "dg": np.zeros((T, dk))}
    de, dw = np.zeros((T, dk)), np.zeros((T, dv))
    dS = np.zeros((dk, dv)) if dsT is None else np.array(dsT, dtype=np.float64)
    for t in reversed(range(T)):
        Sp = St[t] + np.outer(k[t], D[t])    # S' of token t
        dS = dS + np.outer(q[t], do[t])
        out["dq"][t] = Sp @ do[t]
        dd = dS.T @ k[t]
        out["dk"][t] = dS @ D[t]
        dw[t] = dd * v[t]
        out["dv"][t] = dd * W[t]
        dS = dS - np.outer(E[t] * k[t], dd)  # dS~
        r = -St[t] @ dd
        out["dk"][t] += E[t] * r
        de[t] = k[t] * r
        out["dg"][t] = np.sum(dS * St[t], axis=1)
        dS = a[t][:, None] * dS
    if g.ndim == 1:
        out["dg"] = out["dg"].sum(axis=1)
    out["ds0"] = dS
    if gdr2:
        out["derase"], out["dwrite"] = de, dw
    else:
        out["dbeta"] = de.sum(axis=1) + dw.sum(axis=1)
    return out
