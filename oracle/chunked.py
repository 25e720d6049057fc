"""Chunkwise KDA forward in fp64 NumPy -- TEST INFRASTRUCTURE.

This is the second, independent oracle implementation. It follows the
chunkwise derivation on the Doubleword page "You Could Have Come Up with Kimi
Delta Attention", section 6, equation by equation, for one (sequence, head):

  6.1  D_i = Diag(alpha_i); D_{0:i} = D_0..D_i; D_{j+1:i} = D_{j+1}..D_i.
       Stored as prefix sums of log-decays (section 6.6): G_i = sum_{m<=i} g_m,
       so D_{0:i} = Diag(exp G_i) and D_{j+1:i} = Diag(exp(G_i - G_j)).
  6.2  provisional errors  ebar_i = beta_i (v_i - S_c D_{0:i} k_i)
  6.3  rho_ij = beta_i <k_j| D_{j+1:i} |k_i>  (j < i), R strictly lower,
       A^kk = (I + R)^-1, and the causal substitution
       e_i = ebar_i - sum_{j<i} rho_ij e_j   (forward substitution)
  6.4  S_{c+1} = S_c D_{0:last} + E_c K^end,  K^end rows <k_j| D_{j+1:last}
  6.5  chi_ij = s <k_j| D_{j+1:i} |q_i>  (j <= i),
       O_c = s S_c Q^bnd + E_c (A^qk)^T,  Q^bnd columns D_{0:i} q_i

The page says the chunkwise form must give exactly the same states and outputs
as the token recurrence, which is what the tests check against the C token
oracle. A partial last chunk simply has fewer tokens; "last" is its last real
token.

Section 6.6 also names a "WY pseudo-key / pseudo-value" form without defining
it. The reading used here: stacking the errors as rows,
    E = A^kk Diag(beta) (V - K_b S_c^T) = U - W S_c^T
with  U = A^kk Diag(beta) V  and  W = A^kk Diag(beta) K_b,  K_b rows
D_{0:i} k_i. These are emitted as intermediates (not used to produce the
outputs, which follow 6.2-6.5 literally), and a test checks U - W S_c^T
against the literal substitution.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module. It shares nothing with the GPU library.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    """Logistic function 1/(1+e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def activations(q, k, g_raw, beta_raw, lower_bound, eps):
    """Gate, write-strength and normalisation in front of the recurrence.

    FlashKDA pages (instagit summary "Chunked Token Processing"; DocSearch
    digest, "Configure fla_chunk_kda"): g = lower_bound * sigmoid(g_raw) is the
    per-channel log-decay (alpha = exp g), beta = sigmoid(beta_raw), and q, k
    are L2-normalised per token (x / sqrt(sum x^2 + eps)).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    qn = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    kn = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    g = lower_bound * sigmoid(g_raw)
    beta = sigmoid(beta_raw)
    return qn, kn, g, beta


def chunk_step(S, q, k, v, g, beta, scale):
    """Advance one chunk of L <= C tokens (section 6 of the Doubleword page).

    S: [V,K] incoming state S_c. q,k,g: [L,K]. v: [L,V]. beta: [L].
    Returns (O [L,V], S_next [V,K], intermediates dict).
    """
    L, K = k.shape
    G = np.cumsum(g, axis=0)                      # 6.6: prefix sums of log-decay
    # 6.2 provisional errors, as columns ebar_i (stored here as rows)
    ebar = np.empty_like(v)
    for i in range(L):
        ebar[i] = beta[i] * (v[i] - S @ (np.exp(G[i]) * k[i]))
    # 6.3 causal key-key coefficients and forward substitution
    R = np.zeros((L, L))
    for i in range(L):
        for j in range(i):
            R[i, j] = beta[i] * np.dot(k[j] * np.exp(G[i] - G[j]), k[i])
    E = np.empty_like(ebar)
    for i in range(L):
        E[i] = ebar[i] - sum((R[i, j] * E[j] for j in range(i)), np.zeros(v.shape[1]))
    Akk = np.linalg.inv(np.eye(L) + R)
    # 6.4 fast-forward the state
    last = L - 1
    Kend = np.stack([k[j] * np.exp(G[last] - G[j]) for j in range(L)])
    S_next = S * np.exp(G[last])[None, :] + E.T @ Kend
    # 6.5 outputs: chi_ij = s <k_j|D_{j+1:i}|q_i> for j <= i
    Aqk = np.zeros((L, L))
    for i in range(L):
        for j in range(i + 1):
            Aqk[i, j] = scale * np.dot(k[j] * np.exp(G[i] - G[j]), q[i])
    Qbnd = np.stack([np.exp(G[i]) * q[i] for i in range(L)])   # rows D_{0:i} q_i
    O = scale * (Qbnd @ S.T) + Aqk @ E
    # WY reading of section 6.6 (see module docstring)
    Kb = np.stack([np.exp(G[i]) * k[i] for i in range(L)])
    W = Akk @ (beta[:, None] * Kb)
    U = Akk @ (beta[:, None] * v)
    inter = dict(G=G, R=R, Akk=Akk, Aqk=Aqk, Qbnd=Qbnd, Kend=Kend, Kb=Kb,
                 W=W, U=U, E=E, gamma=np.exp(G[last]), beta=beta, S_in=S.copy())
    return O, S_next, inter


def forward_pair(q, k, v, g, beta, S0, scale, chunk=16, keep=False):
    """Chunkwise forward for one (sequence, head) on activated inputs.

    Chunks start at the sequence start; the last one may be partial.
    Returns (o [T,V], S_T [V,K], list of per-chunk intermediates or None).
    """
    T = k.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    inters = [] if keep else None
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        O, S, inter = chunk_step(S, q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], scale)
        o[c0:c1] = O
        if keep:
            inters.append(inter)
    return o, S, inters


def forward(q, k, v, g_raw, beta_raw, seq_offsets, initial_state=None,
            lower_bound=-5.0, scale=None, eps=1e-6, chunk=16, keep=False):
    """Chunkwise forward on the packed layout [T_tot,H,D] with N+1 offsets.

    Returns (o [T_tot,H,V], final_state [N,H,V,K], intermediates) where
    intermediates[(n, h)] is the per-chunk list when keep=True.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T_tot, H, K = k.shape
    V = v.shape[2]
    if scale is None:
        scale = K ** -0.5
    qn, kn, g, beta = activations(q, k, np.asarray(g_raw, np.float64),
                                  np.asarray(beta_raw, np.float64), lower_bound, eps)
    offs = [int(x) for x in seq_offsets]
    N = len(offs) - 1
    o = np.zeros((T_tot, H, V))
    fin = np.zeros((N, H, V, K))
    inters = {}
    for n in range(N):
        a, b = offs[n], offs[n + 1]
        for h in range(H):
            S0 = np.zeros((V, K)) if initial_state is None else np.asarray(initial_state[n, h], np.float64)
            on, Sn, it = forward_pair(qn[a:b, h], kn[a:b, h], v[a:b, h], g[a:b, h],
                                      beta[a:b, h], S0, scale, chunk, keep)
            o[a:b, h] = on
            fin[n, h] = Sn
            if keep:
                inters[(n, h)] = it
    return o, fin, inters


def unit_lower_inverse_substitution(R):
    """(I + R)^-1 for strictly lower-triangular R by forward substitution.

    Column by column: row i of X = (I+R)^-1 satisfies X_i = e_i - sum_{j<i} R_ij X_j,
    the same causal substitution section 6.3 applies to the error kets.
    """
    n = R.shape[0]
    X = np.zeros((n, n))
    for i in range(n):
        X[i] = np.eye(n)[i] - sum((R[i, j] * X[j] for j in range(i)), np.zeros(n))
    return X


def unit_lower_inverse_neumann(R):
    """(I + R)^-1 = sum_{m=0}^{n-1} (-R)^m, exact because R^n = 0 (nilpotent).

    The FlashKDA pages (deep-dive section 1; review section 2.1) invert the
    16 x 16 matrix by this series.
    """
    n = R.shape[0]
    X = np.eye(n)
    P = np.eye(n)
    for _ in range(1, n):
        P = P @ (-R)
        X = X + P
    return X
