"""Closed forms of tree GDN verification and commit, NumPy fp64.

TEST INFRASTRUCTURE ONLY (imported by tests to pin ``gdn_oracle.c``).

This is a second, independent route to the same numbers as the node-by-node
recurrence: no state is ever updated.  Everything is written in this
package's d_v x d_k orientation (o = S q); the Bole review stores the state
transposed (d_k x d_v, o^T = q^T S), so its S is our S^T and its K S_pre is our
(S_pre K^T)^T.

* Path decay P_i: product of the decay gates over the root-to-i path
  (Bole review, Sec. 3.1).
* Lemma 1 / Eq. (3): S_i = P_i S_pre + sum_{j on path(i)} (P_i / P_j) u_j k_j^T.
* Lemma 2 / Eq. (5): (I + G) U = R with
  G_ij = beta_i (P_i / P_j) k_i . k_j for j a strict ancestor of i, and
  R_i  = beta_i (v_i - P_i S_pre k_i).
* Eq. (4) / Theorem 1: o_i = P_i S_pre q_i + sum_{j on path(i)} (P_i/P_j)(q_i . k_j) u_j.
* Lemma 3 / Eq. (6): G is nilpotent, G^{d+1} = 0 for d the largest number of
  strict ancestors, so (I + G)^{-1} = sum_{m=0}^{d} (-G)^m.
* Eq. (10) (factorized commit): S_new = P_a S_pre + sum_{j in path(a)} (P_a/P_j) u_j k_j^T.
* TreeWY, Sec. 3 gives the same system with g for the path decay and the
  pseudo-values V~ in place of U.
"""
from __future__ import annotations

import numpy as np


def ancestors(parent):
    """Strict ancestor list of every node, root-level first (Bole review, Sec.
    3.1: A(i) is the set of draft nodes on the root-to-i path without i)."""
    parent = list(int(p) for p in parent)
    out = []
    for i in range(len(parent)):
        chain = []
        p = parent[i]
        while p >= 0:
            chain.append(p)
            p = parent[p]
        out.append(chain[::-1])
    return out


def path_decay(parent, alpha):
    """P_i = product of alpha over A(i) and i (Bole review, Algorithm 1 step 1)."""
    anc = ancestors(parent)
    P = np.empty(len(parent))
    for i, a in enumerate(anc):
        P[i] = np.prod([alpha[j] for j in a + [i]])
    return P


def masks(parent):
    """Strict-ancestor mask M- (M-[i,j] = 1 iff j in A(i)) and M+ = M- + I
    (Bole review, Algorithm 1 step 4)."""
    N = len(parent)
    Mm = np.zeros((N, N))
    for i, a in enumerate(ancestors(parent)):
        for j in a:
            Mm[i, j] = 1.0
    return Mm, Mm + np.eye(N)


def g_matrix(parent, alpha, beta, K):
    """G = D_beta D_P [(K K^T) o M-] D_P^{-1} (Bole review, Eq. (5), Algorithm 1 step 4)."""
    P = path_decay(parent, alpha)
    Mm, _ = masks(parent)
    return (beta * P)[:, None] * ((K @ K.T) * Mm) / P[None, :]


def solve_tree(parent, alpha, beta, Q, K, V, S_pre, use_neumann=False):
    """Outputs O [N][d_v] and corrections U [N][d_v] of one (request, head) by
    Theorem 1 (Bole review, Eq. (2)), with a dense solve of (I+G)U=R or, with
    ``use_neumann``, the finite Neumann series of Eq. (6).  Q, K: [N][d_k]
    (already normalised if the caller normalises), V: [N][d_v], S_pre [d_v][d_k].
    """
    N = len(parent)
    P = path_decay(parent, alpha)
    _, Mp = masks(parent)
    G = g_matrix(parent, alpha, beta, K)
    R = beta[:, None] * (V - P[:, None] * (K @ S_pre.T))
    if use_neumann:
        d = max((len(a) for a in ancestors(parent)), default=0)
        U = R.copy()
        Z = R.copy()
        for _ in range(d):
            Z = -G @ Z
            U = U + Z
    else:
        U = np.linalg.solve(np.eye(N) + G, R)
    Cm = P[:, None] * ((Q @ K.T) * Mp) / P[None, :]
    O = P[:, None] * (Q @ S_pre.T) + Cm @ U
    return O, U


def commit_factorized(parent, alpha, path, K, U, S_pre):
    """Eq. (10) of the Bole review in d_v x d_k orientation:
    S_new = P_a S_pre + sum_{j in path} (P_a / P_j) u_j k_j^T; an empty path
    returns S_pre unchanged (Algorithm 2 step 8)."""
    if len(path) == 0:
        return S_pre.copy()
    P = path_decay(parent, alpha)
    a = path[-1]
    S = P[a] * S_pre
    for j in path:
        S = S + (P[a] / P[j]) * np.outer(U[j], K[j])
    return S


def treewy_states(parent, alpha, beta, K, V, S0):
    """State of every node from TreeWY's pseudo-values (TreeWY, Sec. 3):
    (I + diag(beta) G~) V~ = R~ with G~[t,i] = (g_t/g_i) k_t.k_i [i strict
    ancestor of t], R~[t] = beta_t v_t - beta_t g_t S_0 k_t, and
    S_a = g_a S_0 + sum_{i on path(a)} (g_a / g_i) v~_i k_i^T."""
    N = len(parent)
    g = path_decay(parent, alpha)
    Mm, _ = masks(parent)
    Gt = g[:, None] * ((K @ K.T) * Mm) / g[None, :]
    Rt = beta[:, None] * V - (beta * g)[:, None] * (K @ S0.T)
    Vt = np.linalg.solve(np.eye(N) + beta[:, None] * Gt, Rt)
    anc = ancestors(parent)
    states = []
    for a_node in range(N):
        S = g[a_node] * S0
        for i in anc[a_node] + [a_node]:
            S = S + (g[a_node] / g[i]) * np.outer(Vt[i], K[i])
        states.append(S)
    return np.stack(states)
