"""Ancestry-aware tree attention and the accepted path's KV publication, in
fp64 (TEST INFRASTRUCTURE ONLY: see the package docstring for who may
import it).

LumoTree, Sec. III-C and V-B: query rows stay in logical node order; the
candidates' keys and values sit in the KV cache after the committed prefix
at physical slots given by the slot map (node_row), and the ancestry mask
names which of those a node sees -- its root path (its ancestors and
itself); every node also sees the whole committed prefix.  Publication
moves the accepted path's entries through the same slot map to the native
continuation positions right after the prefix, in path order.

Layouts (the device calls use the same):
  q        [B][N][Hq][D]      logical node rows
  k, v     [B][S][Hkv][D]     KV cache; positions [0, ctx_len[b]) are the
                              committed prefix, ctx_len[b] + r the candidate
                              in physical row r (0 <= r < R)
  out      [B][N][Hq][D]      NaN where nothing is written
Query head h reads kv head h // (Hq / Hkv).
"""
from __future__ import annotations

import numpy as np

EV_PARENT, EV_ROW, EV_STATE, EV_PATH, EV_CTX = 1, 2, 4, 8, 16


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def root_path(parent, i):
    """Node i's root path as a list, root-level node first (ends with i)."""
    path = []
    while i >= 0:
        path.append(int(i))
        i = int(parent[i])
    return path[::-1]


def tree_attention(parent, node_row, status, q, k, v, ctx_len, R: int, Hq: int, Hkv: int,
                   scale: float, shared: bool = False, nodes=None):
    """o[b, i, h] = sum_j softmax_j(scale * q[b, i, h] . k_j) v_j over the keys
    node i sees: prefix positions 0 .. ctx_len[b]-1 and ctx_len[b] +
    node_row[b, a] for every node a on i's root path (LumoTree, Sec. V-B:
    the ancestry mask over physically placed candidate keys).  Requests whose
    tree is malformed (status != 0, reported by the descriptor build) or whose
    ctx_len is outside [0, S - R] (EV_CTX) get no output.  With ``nodes``
    (pairs (b, i)) only those rows are computed (the rest stay NaN).
    Returns (out float64, err)."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, N = q64.shape[0], q64.shape[1]
    S = k64.shape[1]
    D = q64.shape[-1]
    G = Hq // Hkv
    parent = np.atleast_2d(parent)
    node_row = np.atleast_2d(node_row)
    status = np.atleast_1d(status)
    out = np.full((B, N, Hq, D), np.nan)
    err = 0
    for b in range(B):
        t = 0 if shared else b
        if status[t] != 0:
            continue
        L = int(ctx_len[b])
        if L < 0 or L + R > S:
            err |= EV_CTX
            continue
        for i in range(N):
            if nodes is not None and (b, i) not in nodes:
                continue
            cand = [L + int(node_row[t, a]) for a in root_path(parent[t], i)]
            for h in range(Hq):
                g = h // G
                # the prefix keys, then the root path's candidates
                s = scale * np.concatenate([k64[b, :L, g, :] @ q64[b, i, h], k64[b, cand, g, :] @ q64[b, i, h]])
                w = np.exp(s - s.max())
                out[b, i, h] = (w[:L] @ v64[b, :L, g, :] + w[L:] @ v64[b, cand, g, :]) / w.sum()
    return out, err


def kv_publish(path_rows, path_n, k, v, ctx_len, R: int):
    """The accepted path's KV entries moved to the continuation positions: for
    n = path_n[b] > 0, position ctx_len[b] + j receives the entry at
    ctx_len[b] + path_rows[b, j] for j < n (every source read before any
    destination is written; LumoTree, Sec. V-B: publication translates the
    selected nodes through the slot map into native continuation positions).
    path_n <= 0 leaves the request alone; ctx_len outside [0, S - R] is EV_CTX.
    Returns (k_new, v_new, err) as copies of the inputs' dtype."""
    k2, v2 = np.array(k, copy=True), np.array(v, copy=True)
    S = k2.shape[1]
    err = 0
    for b in range(k2.shape[0]):
        n = int(path_n[b])
        if n <= 0:
            continue
        L = int(ctx_len[b])
        if L < 0 or L + R > S:
            err |= EV_CTX
            continue
        src = [L + int(path_rows[b, j]) for j in range(n)]
        ks, vs = k2[b, src].copy(), v2[b, src].copy()
        k2[b, L:L + n] = ks
        v2[b, L:L + n] = vs
    return k2, v2, err
