"""Seeded synthetic inputs for tree GDN verify / commit / conv.

This is the one module both the HIP path's callers (tests, bench) and the
oracle's callers use.  It draws random numbers and lays them out; it holds
none of the method's arithmetic (no decay, delta update, readout or
convolution).  Every array is NumPy on the host; bf16 operands are returned as
uint16 bit patterns (round-to-nearest-even from float32).

Workloads.  The pages measure their GDN component on synthetic operands with
a fixed tree geometry (LumoTree, Sec. VII-D and VII-H: 48 instances, 28 active
nodes packed in 32 rows).  The five configurations below stand in for those
component workloads; their shapes and value distributions are stated with
each configuration below.

Random streams: NumPy PCG64 seeded with SeedSequence([seed, cfg, layer,
stream]).  Trees use layer 0 so that every layer of a multi-layer config
shares one tree per request.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# random stream ids
_S_ROWS, _S_Q, _S_K, _S_V, _S_A, _S_B, _S_POOL, _S_IDX, _S_PATH = range(1, 10)
_S_X, _S_HIST, _S_W = 10, 11, 12
_S_RAW_A, _S_RAW_B, _S_GATE_P = 13, 14, 15
_S_BIAS = 16
_S_ATT_Q, _S_ATT_K, _S_ATT_V, _S_ATT_ROWS = 17, 18, 19, 20
ATTN_CFG = 100  # generator id of the attention inputs
_S_TREE0 = 1_000_000  # + request index


def rng(seed: int, cfg: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, layer, stream])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even; NaN stays NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, BF16_NAN, r)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  ``depth_max`` counts edges below the root
    node; the longest accepted path therefore has depth_max + 1 nodes."""
    name: str
    cfg_id: int
    B: int
    N: int
    R: int
    Hv: int
    Hqk: int
    D: int
    dtype: str              # "bf16" or "f32" for q/k/v
    tree: str               # "binary7" | "chain" | "random"
    bmax: int = 0           # max children per node ("random" trees)
    depth_max: int = 0      # max edges below the root ("random" trees)
    s_std: float = 0.05     # std of the committed state
    gates: str = "softplus"  # "uniform": a~U(0.9,1), b~U(0,1); "softplus": a=exp(-softplus(n)), b=sigmoid(n)
    path: str = "uniform_len"  # "leaf_full" | "full" | "uniform_len"
    conv_W: int = 0         # 0: q/k/v given directly; >0: q/k/v = conv(x)
    conv_C: int = 0
    act: int = 1            # conv activation: 0 none, 1 SiLU
    norm_qk: bool = False   # q/k normalised inside verify/commit
    layers: int = 1
    w_std: float = 0.02

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def C(self) -> int:
        return self.conv_C

    @property
    def Lmax(self) -> int:
        if self.tree == "chain":
            return self.N
        if self.tree == "binary7":
            return 3
        return self.depth_max + 1


CONFIGS = {
    1: Config("binary7_d32_f32", 1, B=1, N=7, R=8, Hv=1, Hqk=1, D=32, dtype="f32",
              tree="binary7", s_std=0.1, gates="uniform", path="leaf_full"),
    2: Config("chain8_b64_h16", 2, B=64, N=8, R=8, Hv=16, Hqk=16, D=128, dtype="bf16",
              tree="chain", s_std=0.05, path="full"),
    3: Config("tree27_b32_h32", 3, B=32, N=27, R=32, Hv=32, Hqk=16, D=128, dtype="bf16",
              tree="random", bmax=3, depth_max=6, s_std=0.05),
    4: Config("tree27_b128_h32_conv4", 4, B=128, N=27, R=32, Hv=32, Hqk=16, D=128,
              dtype="bf16", tree="random", bmax=3, depth_max=6, s_std=0.05,
              conv_W=4, conv_C=8192, act=1, norm_qk=True),
    5: Config("tree64_b256_h32_l48", 5, B=256, N=64, R=64, Hv=32, Hqk=16, D=128,
              dtype="bf16", tree="random", bmax=4, depth_max=8, s_std=0.05, layers=48),
}


# --------------------------------------------------------------------------
# trees, row packing, accepted paths
# --------------------------------------------------------------------------

def random_tree(g: np.random.Generator, N: int, bmax: int, depth_max: int) -> np.ndarray:
    """Node 0 is the single root-level node (parent -1); node i >= 1 takes a
    parent uniformly from {j < i : children(j) < bmax, edges(j) < depth_max},
    which keeps parent[i] < i."""
    parent = np.full(N, -1, np.int32)
    children = np.zeros(N, np.int64)
    edges = np.zeros(N, np.int64)
    for i in range(1, N):
        cand = [j for j in range(i) if children[j] < bmax and edges[j] < depth_max]
        if not cand:
            raise ValueError("tree shape cannot hold N nodes")
        p = int(cand[g.integers(len(cand))])
        parent[i] = p
        children[p] += 1
        edges[i] = edges[p] + 1
    return parent


def tree_for(cfg: Config, seed: int, b: int) -> np.ndarray:
    if cfg.tree == "binary7":
        return np.array([-1, 0, 0, 1, 1, 2, 2], np.int32)
    if cfg.tree == "chain":
        return np.arange(-1, cfg.N - 1, dtype=np.int32)
    return random_tree(rng(seed, cfg.cfg_id, 0, _S_TREE0 + b), cfg.N, cfg.bmax, cfg.depth_max)


def path_lengths(parent: np.ndarray) -> np.ndarray:
    """Number of nodes on each node's root chain (bookkeeping for the path
    draw; the descriptor builders compute their own)."""
    L = np.zeros(len(parent), np.int64)
    for i, p in enumerate(parent):
        L[i] = 1 if p < 0 else L[p] + 1
    return L


def root_chain(parent: np.ndarray, node: int) -> list:
    chain = []
    while node >= 0:
        chain.append(int(node))
        node = int(parent[node])
    return chain[::-1]


def random_rows(g: np.random.Generator, N: int, R: int) -> np.ndarray:
    """Seeded injective logical->physical map into [0, R)."""
    return g.permutation(R)[:N].astype(np.int32)


def bfs_rows(parent: np.ndarray) -> np.ndarray:
    """Breadth-first packing: row order by (depth, index).  The previous
    physical row is usually a sibling or cousin, not the parent (the packed
    buffer trap of the GDN Tree-Scan review's worked example)."""
    L = path_lengths(parent)
    order = sorted(range(len(parent)), key=lambda i: (L[i], i))
    rows = np.empty(len(parent), np.int32)
    for r, i in enumerate(order):
        rows[i] = r
    return rows


def draw_path(g: np.random.Generator, parent: np.ndarray, mode: str):
    L = path_lengths(parent)
    if mode == "full":          # chain: the whole chain
        node = int(np.argmax(L))
    elif mode == "leaf_full":   # a uniformly drawn leaf, full root chain
        has_child = np.zeros(len(parent), bool)
        for p in parent:
            if p >= 0:
                has_child[p] = True
        leaves = np.nonzero(~has_child)[0]
        node = int(leaves[g.integers(len(leaves))])
    else:                       # L ~ U{1..max}, then a uniform node at that length
        Lb = int(g.integers(1, int(L.max()) + 1))
        cand = np.nonzero(L == Lb)[0]
        node = int(cand[g.integers(len(cand))])
    return root_chain(parent, node)


# --------------------------------------------------------------------------
# operands
# --------------------------------------------------------------------------

def _unit_rows(g: np.random.Generator, shape) -> np.ndarray:
    x = g.standard_normal(shape, dtype=np.float32)
    n = np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True))
    return (x / n).astype(np.float32)


def _gates(g_a, g_b, cfg: Config, shape):
    if cfg.gates == "uniform":
        a = g_a.uniform(0.9, 1.0, shape).astype(np.float32)
        b = g_b.uniform(0.0, 1.0, shape).astype(np.float32)
    else:
        na = g_a.standard_normal(shape)
        nb = g_b.standard_normal(shape)
        a = np.exp(-np.logaddexp(0.0, na)).astype(np.float32)
        b = (1.0 / (1.0 + np.exp(-nb))).astype(np.float32)
    return a, b


def make_case(cfg: Config, seed: int = 2026, layer: int = 0, B: int | None = None,
              packing: str = "perm", extra_slots: int = 0, poison: bool = True,
              with_pool: bool = True, conv_values: str = "normal") -> dict:
    """All inputs of one layer of ``cfg`` (optionally with a smaller batch B).

    Returns a dict of host arrays:
      parent, node_row [B][N] int32; path [B][Lmax], path_len [B] int32;
      q, k [B][R][Hqk][D] and v [B][R][Hv][D] (uint16 bf16 bits or float32) --
        or, for conv configs, x [B][R][C], hist [P][W-1][C], w [C][W] (uint16);
      alpha, beta [B][R][Hv] float32; pool [P][Hv][D][D] float32;
      state_idx [B] int32 (a seeded permutation of pool slots).
    Padding rows (rows no node maps to) and unused pool slots hold NaN.

    conv_values="dyadic" draws x and hist from {k/8 : |k| <= 16} and w from
    {j/64 : |j| <= 8} instead of the normal distributions: every product is
    a multiple of 2^-9 and every W-tap sum stays below 2^4 in magnitude, so
    any fp32 or fp64 summation of the taps is exact and both sides round the
    same value to bf16 (conv parity without rounding straddles; use it with
    act = 0).
    """
    B = cfg.B if B is None else B
    N, R, D, Hv, Hqk = cfg.N, cfg.R, cfg.D, cfg.Hv, cfg.Hqk
    cid = cfg.cfg_id
    parents = np.stack([tree_for(cfg, seed, b) for b in range(B)]).astype(np.int32)
    g_rows = rng(seed, cid, 0, _S_ROWS)
    if packing == "bfs":
        rows = np.stack([bfs_rows(parents[b]) for b in range(B)])
    else:
        rows = np.stack([random_rows(g_rows, N, R) for _ in range(B)])
    used = np.zeros((B, R), bool)
    for b in range(B):
        used[b, rows[b]] = True
    g_path = rng(seed, cid, layer, _S_PATH)
    Lmax = cfg.Lmax
    path = np.full((B, Lmax), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        p = draw_path(g_path, parents[b], cfg.path)
        path[b, :len(p)] = p
        plen[b] = len(p)
    out = dict(cfg=cfg, seed=seed, layer=layer, B=B, parent=parents, node_row=rows.astype(np.int32),
               path=path, path_len=plen)

    P = B + extra_slots
    if cfg.conv_W > 0:
        C, W = cfg.conv_C, cfg.conv_W
        if conv_values == "dyadic":
            x = rng(seed, cid, layer, _S_X).integers(-16, 17, (B, R, C)).astype(np.float32) / 8
            hist = rng(seed, cid, layer, _S_HIST).integers(-16, 17, (P, W - 1, C)).astype(np.float32) / 8
            w = rng(seed, cid, layer, _S_W).integers(-8, 9, (C, W)).astype(np.float32) / 64
        else:
            x = rng(seed, cid, layer, _S_X).standard_normal((B, R, C), dtype=np.float32)
            hist = rng(seed, cid, layer, _S_HIST).standard_normal((P, W - 1, C), dtype=np.float32)
            w = (rng(seed, cid, layer, _S_W).standard_normal((C, W), dtype=np.float32) * np.float32(cfg.w_std))
        if poison:
            x[~used] = np.nan
        out.update(x=f32_to_bf16_bits(x), hist=f32_to_bf16_bits(hist), w=f32_to_bf16_bits(w))
    else:
        q = _unit_rows(rng(seed, cid, layer, _S_Q), (B, R, Hqk, D))
        k = _unit_rows(rng(seed, cid, layer, _S_K), (B, R, Hqk, D))
        v = rng(seed, cid, layer, _S_V).standard_normal((B, R, Hv, D), dtype=np.float32)
        if poison:
            q[~used] = np.nan
            k[~used] = np.nan
            v[~used] = np.nan
        if cfg.dtype == "bf16":
            q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        out.update(q=q, k=k, v=v)
    a, bt = _gates(rng(seed, cid, layer, _S_A), rng(seed, cid, layer, _S_B), cfg, (B, R, Hv))
    if poison:
        a[~used] = np.nan
        bt[~used] = np.nan
    out.update(alpha=a, beta=bt)
    perm = rng(seed, cid, layer, _S_IDX).permutation(P)[:B].astype(np.int32)
    out["state_idx"] = perm
    out["P"] = P
    if with_pool:
        pool = (rng(seed, cid, layer, _S_POOL).standard_normal((P, Hv, D, D), dtype=np.float32)
                * np.float32(cfg.s_std))
        if poison and extra_slots:
            mask = np.ones(P, bool)
            mask[perm] = False
            pool[mask] = np.nan
        out["pool"] = pool
    return out


def with_raw_gates(case: dict, gate_params: np.ndarray | None = None) -> dict:
    """A copy of ``case`` whose gates are raw inputs (for GDN_F_RAW_GATES):
    alpha and beta become a, b ~ N(0, 1) float32, NaN where the case's gates
    are NaN (rows no node uses), and gate_params float32 [2][Hv] holds the
    per-head A_log ~ U(0, log 16) and dt_bias ~ U(-7, -2) (so exp(A_log) lies
    in [1, 16] and softplus(a + dt_bias) mostly between 1e-3 and 0.3).  Pass
    the first step's gate_params to later steps of the same layer."""
    cfg = case["cfg"]
    seed, layer = case["seed"], case["layer"]
    shape = case["alpha"].shape
    a = rng(seed, cfg.cfg_id, layer, _S_RAW_A).standard_normal(shape, dtype=np.float32)
    b = rng(seed, cfg.cfg_id, layer, _S_RAW_B).standard_normal(shape, dtype=np.float32)
    pad = np.isnan(case["alpha"])
    a[pad] = np.nan
    b[pad] = np.nan
    if gate_params is None:
        g = rng(seed, cfg.cfg_id, layer, _S_GATE_P)
        gate_params = np.stack([g.uniform(0.0, np.log(16.0), cfg.Hv),
                                g.uniform(-7.0, -2.0, cfg.Hv)]).astype(np.float32)
    out = dict(case)
    out.update(alpha=a, beta=b, gate_params=np.asarray(gate_params, np.float32))
    return out


def conv_bias(cfg: Config, seed: int, layer: int = 0, dyadic: bool = False) -> np.ndarray:
    """A conv bias float32 [C] for the layer: N(0, 0.1^2), or with ``dyadic``
    multiples of 1/64 up to 1/4 in magnitude (exact in every fp32 tap sum,
    like the dyadic conv inputs)."""
    g = rng(seed, cfg.cfg_id, layer, _S_BIAS)
    if dyadic:
        return (g.integers(-16, 17, cfg.conv_C) / 64.0).astype(np.float32)
    return (g.standard_normal(cfg.conv_C) * 0.1).astype(np.float32)


def make_attention_case(seed: int, B: int, N: int, R: int, Hq: int, Hkv: int, D: int, ctx, S: int,
                        bmax: int = 3, depth_max: int = 6, packing: str = "perm",
                        poison: bool = True, shared: bool = False) -> dict:
    """Inputs of one tree-attention layer: B trees of N nodes (the random-tree
    rule above) with physical rows in [0, R) (a seeded injective map, or
    breadth-first); q [B][N][Hq][D] and the KV cache k, v [B][S][Hkv][D] as
    bf16 bit patterns of N(0, 1) values; ctx [B] committed prefix lengths.
    With ``poison`` the cache positions past ctx + R and the candidate rows no
    node occupies hold NaN (nothing may read them).  With ``shared`` every
    request has request 0's tree and rows."""
    ctx = np.asarray(ctx, np.int32)
    parents = np.stack([random_tree(rng(seed, ATTN_CFG, 0 if shared else b, _S_TREE0), N, bmax, depth_max)
                        for b in range(B)]).astype(np.int32)
    g_rows = rng(seed, ATTN_CFG, 0, _S_ATT_ROWS)
    if packing == "bfs":
        rows = np.stack([bfs_rows(parents[b]) for b in range(B)])
    else:
        rows = np.stack([random_rows(g_rows, N, R) for _ in range(B)])
    if shared:
        rows = np.repeat(rows[:1], B, axis=0)
    q = rng(seed, ATTN_CFG, 0, _S_ATT_Q).standard_normal((B, N, Hq, D), dtype=np.float32)
    k = rng(seed, ATTN_CFG, 0, _S_ATT_K).standard_normal((B, S, Hkv, D), dtype=np.float32)
    v = rng(seed, ATTN_CFG, 0, _S_ATT_V).standard_normal((B, S, Hkv, D), dtype=np.float32)
    if poison:
        for b in range(B):
            L = int(ctx[b])
            if L < 0 or L + R > S:
                continue
            k[b, L + R:] = np.nan
            v[b, L + R:] = np.nan
            unused = np.setdiff1d(np.arange(R), rows[b])
            k[b, L + unused] = np.nan
            v[b, L + unused] = np.nan
    return dict(parent=parents, node_row=rows.astype(np.int32), q=f32_to_bf16_bits(q),
                k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v), ctx=ctx, B=B, N=N, R=R, Hq=Hq,
                Hkv=Hkv, D=D, S=S)
