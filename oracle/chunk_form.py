"""Chunk-form (WY / UT) model of the gated delta recurrence, fp64 NumPy.

TEST INFRASTRUCTURE ONLY.  It is a second, independently written algorithm
for the same recurrence as ``gdn_oracle.c``; the tests require the two to agree
to ~1e-12, which pins the chunk identities the GPU prefill is built on.  It
shares no code with the GPU library.

Row convention: H = S^T (row = key dim, column = value dim).  The Qwen3.8-Flash-
Next model card's chunk state line (state * chunk_decay + key^T @ v_new) is
this convention.  Within one chunk with entering state H0, tokens r = 0..C-1,
log-decays g_r = log alpha_r, G_r = g_0 + ... + g_r (chunk-local cumsum):

    L[i, j] = beta_i * exp(G_i - G_j) * (k_i . k_j)        for j < i, else 0
    Tinv    = (I + L)^-1
    W       = Tinv diag(beta * exp(G)) K
    Utilde  = Tinv diag(beta) V
    U       = Utilde - W H0                      ("v_new" of the model card)
    M[i, j] = exp(G_i - G_j) * (q_i . k_j)                 for j <= i, else 0
    O       = diag(exp(G)) Q H0 + M U
    H_C     = exp(G_{C-1}) H0 + Khat^T U,   Khat_r = exp(G_{C-1} - G_r) k_r

These follow by unrolling the field guide's six update steps over a chunk:
H_r = exp(G_r) H0 + sum_{s<=r} exp(G_r - G_s) k_s u_s^T with
u_s = beta_s (v_s - alpha_s H_{s-1}^T k_s), which is triangular in u.
"""
from __future__ import annotations

import numpy as np


def chunk_recurrence(g, beta, q, k, v, H0=None, chunk=64):
    """Chunked recurrence of one head.

    g: [T] log-decays (alpha = exp(g)); beta: [T]; q, k: [T, Dk]; v: [T, Dv];
    H0: [Dk, Dv] or None.  Returns (y [T, Dv], H_T [Dk, Dv]).
    """
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Dk = k.shape
    Dv = v.shape[1]
    H = np.zeros((Dk, Dv)) if H0 is None else np.array(H0, dtype=np.float64)
    y = np.empty((T, Dv))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        C = c1 - c0
        G = np.cumsum(g[c0:c1])
        Kc, Qc, Vc, bc = k[c0:c1], q[c0:c1], v[c0:c1], beta[c0:c1]
        diff = G[:, None] - G[None, :]
        lower = np.tril(np.ones((C, C), dtype=bool), -1)
        lower_eq = np.tril(np.ones((C, C), dtype=bool), 0)
        # exponentiate only non-positive differences (the masked-out ones are set to -inf)
        decay_strict = np.exp(np.where(lower, diff, -np.inf))
        decay_incl = np.exp(np.where(lower_eq, diff, -np.inf))
        L = bc[:, None] * decay_strict * (Kc @ Kc.T)
        Tinv = np.linalg.inv(np.eye(C) + L)
        gam = np.exp(G)
        W = Tinv @ ((bc * gam)[:, None] * Kc)
        Ut = Tinv @ (bc[:, None] * Vc)
        U = Ut - W @ H
        M = decay_incl * (Qc @ Kc.T)
        y[c0:c1] = gam[:, None] * (Qc @ H) + M @ U
        Khat = np.exp(G[-1] - G)[:, None] * Kc
        H = gam[-1] * H + Khat.T @ U
    return y, H
