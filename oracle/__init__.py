"""fp64 CPU oracle for tree GDN verify / commit / ancestry-gathered conv1d.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``tree_speculative_verification_gdn_amd``) and
neither imports the other; the seeded input generators in ``gdn_inputs`` are
the only thing both sides use.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, node by
node from each node's parent state).  This module builds it with gcc, loads it
with ctypes and converts inputs: bf16 bit patterns (uint16) and fp32 arrays
become float64 exactly.  ``closed_form`` holds an independent NumPy
re-derivation used only to pin the C code.

Every function cites the passage it follows in its docstring; the page titles
are the ones in the reference pages (LumoTree; TreeWY; the Bole review; the
GDN Tree-Scan review).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_NAME = "libgdn_oracle.so"

EV_PARENT, EV_ROW, EV_STATE, EV_PATH = 1, 2, 4, 8

_lock = threading.Lock()
_lib = None


def build(force: bool = False, mutation: int = 0, outdir: str | None = None) -> str:
    """Compile ``gdn_oracle.c`` with gcc -O2 -fopenmp and return the .so path.

    ``mutation`` > 0 builds a variant with one planted mistake (see the C
    file); such variants go to ``outdir`` and are used only by the tests that
    show the pins catch them.
    """
    outdir = outdir or _HERE
    name = _LIB_NAME if mutation == 0 else f"libgdn_oracle_m{mutation}.so"
    path = os.path.join(outdir, name)
    if (not force and os.path.exists(path)
            and os.path.getmtime(path) >= os.path.getmtime(_SRC)):
        return path
    tmp = path + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           f"-DORA_MUTATION={int(mutation)}", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


def _bind(lib):
    i32p = ctypes.POINTER(ctypes.c_int32)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    f64p = ctypes.POINTER(ctypes.c_double)
    ci = ctypes.c_int
    lib.ora_threads.restype = ci
    lib.ora_threads.argtypes = []
    lib.ora_set_threads.restype = None
    lib.ora_set_threads.argtypes = [ci]
    lib.ora_desc_build.restype = ci
    lib.ora_desc_build.argtypes = [ci, ci, ci, ci, i32p, i32p, i32p, u64p, i32p, i32p]
    lib.ora_conv.restype = ci
    lib.ora_conv.argtypes = [ci, ci, ci, ci, ci, ci, i32p, i32p, i32p, f64p, f64p,
                             ci, i32p, f64p, f64p, ci, f64p]
    lib.ora_verify.restype = ci
    lib.ora_verify.argtypes = [ci, ci, ci, ci, i32p, i32p, i32p, f64p, f64p, f64p,
                               f64p, f64p, f64p, ci, i32p, ci, ci, ci, ci, f64p, f64p, f64p]
    lib.ora_commit.restype = ci
    lib.ora_commit.argtypes = [ci, ci, ci, ci, i32p, i32p, i32p, i32p, i32p, ci,
                               f64p, f64p, f64p, f64p, f64p, ci, i32p, ci, ci, ci,
                               ci, f64p, f64p, ci, ci]
    return lib


def load(path: str | None = None):
    """Load (building if needed) the oracle library.  With ``path`` given, a
    fresh handle to that file is returned (used for planted-mistake variants)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            _lib = _bind(ctypes.CDLL(build()))
        return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(load().ora_threads())


def set_threads(n: int) -> None:
    """Set the OpenMP threads of the oracle's parallel loops (calling thread)."""
    load().ora_set_threads(int(n))


# --------------------------------------------------------------------------
# input conversion (exact) and the oracle's own bf16 rounding
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (the 16 bits are the top
    half of an IEEE binary32)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Operand array -> float64.  uint16 arrays are bf16 bit patterns; float32
    and float64 arrays are converted exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def round_f64_to_bf16_bits(d: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 (ties to even), returned as uint16
    bit patterns.  Direct rounding of the double value: a plain
    double->float->bf16 chain can round twice, so the one case where the float
    lands exactly on a bf16 halfway point is decided from the double."""
    d = np.ascontiguousarray(d, dtype=np.float64)
    f = d.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    keep = u >> 16
    # ordinary round-half-even on the float's bits
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & 1) == 1))
    # float sits exactly on a bf16 halfway point but the double does not
    tie = (low == 0x8000) & (f.astype(np.float64) != d)
    mag_above = np.abs(d) > np.abs(f.astype(np.float64))
    up = np.where(tie, mag_above, up)
    res = (keep + up.astype(np.uint64)) & 0xFFFF
    nan = np.isnan(d)
    res = np.where(nan, (keep | 0x40) & 0xFFFF, res)
    return res.astype(np.uint16)


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# --------------------------------------------------------------------------
# oracle entry points
# --------------------------------------------------------------------------

def desc_build(parent, node_row, R: int, W: int, lib=None):
    """Descriptor for T trees (arrays [T][N]): validation, depth, strict-ancestor
    mask and conv tap sources.

    LumoTree, Sec. III-C (one logical topology drives every stage) and Sec.
    V-C (static gather indices derived from the topology); Bole review, Sec.
    3.1 (strict ancestors A(i), parent map) and Algorithm 1 (ancestor mask).
    Returns dict(depth, anc (uint64 bitmask), conv_src [T][N][W-1], status, err).
    """
    lib = lib or load()
    parent = _i32(np.atleast_2d(parent))
    node_row = _i32(np.atleast_2d(node_row))
    T, N = parent.shape
    H = W - 1
    depth = np.zeros((T, N), np.int32)
    anc = np.zeros((T, N), np.uint64)
    conv_src = np.zeros((T, N, max(H, 1)), np.int32)
    status = np.zeros((T,), np.int32)
    err = lib.ora_desc_build(T, N, R, W, _p(parent, ctypes.c_int32),
                             _p(node_row, ctypes.c_int32), _p(depth, ctypes.c_int32),
                             _p(anc, ctypes.c_uint64), _p(conv_src, ctypes.c_int32),
                             _p(status, ctypes.c_int32))
    return dict(depth=depth, anc=anc, conv_src=conv_src[:, :, :H], status=status,
                err=int(err))


def conv(node_row, conv_src, status, x, hist, state_idx, w, bias, act: int,
         R: int, C: int, W: int, shared: bool = False, lib=None):
    """Ancestry-gathered causal conv1d, fp64, unrounded output [B][R][C] (rows
    not written stay NaN).

    LumoTree, Sec. V-C: windows gathered from prior conv history and candidate
    inputs along ancestry, taps in order, unused history positions keep their
    padding.  y_i[c] = act(sum_{t<W-1} w[c][t] X(src_i[t])[c] + w[c][W-1] x_i[c]).
    """
    lib = lib or load()
    x64 = as_f64(x)
    B = x64.shape[0]
    N = np.atleast_2d(node_row).shape[-1]
    h64 = as_f64(hist)
    P = h64.shape[0]
    w64 = as_f64(w)
    b64 = None if bias is None else as_f64(bias)
    y = np.full((B, R, C), np.nan, np.float64)
    H = W - 1
    cs = _i32(conv_src).reshape(-1)
    if cs.size == 0:
        cs = np.zeros(1, np.int32)
    err = lib.ora_conv(B, N, R, C, W, int(shared), _p(_i32(node_row), ctypes.c_int32),
                       _p(cs, ctypes.c_int32), _p(_i32(status), ctypes.c_int32),
                       _p(x64, ctypes.c_double), _p(h64, ctypes.c_double), P,
                       _p(_i32(state_idx), ctypes.c_int32), _p(w64, ctypes.c_double),
                       None if b64 is None else _p(b64, ctypes.c_double), int(act),
                       _p(y, ctypes.c_double))
    return y, int(err)


def verify(parent, node_row, status, q, k, v, alpha, beta, pool, state_idx,
           Hqk: int, Hv: int, norm: bool, shared: bool = False,
           want_states: bool = False, want_u: bool = False, lib=None):
    """Tree verify in fp64: for every node i (topological order) and value head
    h, start from the parent's state (the committed state for parent -1), apply
    the gated delta update with node i's operands, read out o_i = S_i q_i.

    TreeWY, Sec. 1 (the gated delta rule and readout); Bole review, Sec. 1 Eq.
    (1) and Sec. 3.1 (node i uses the state of pi(i)); GDN Tree-Scan review,
    "Background" (the parent is not the previous packed row).
    q, k: [B][R][Hqk][D]; v: [B][R][Hv][D]; alpha, beta: [B][R][Hv];
    pool: [P][Hv][D][D] (d_v x d_k, row-major); out: [B][R][Hv][D], NaN where
    no node writes.  With ``want_states`` also returns S_i as [B][N][Hv][D][D];
    with ``want_u`` (last) every node's delta correction
    u_i = beta_i (v_i - alpha_i S_parent k_i) as [B][R][Hv][D] (Bole review,
    Lemma 2: the rows of U in (I + G) U = R).
    """
    lib = lib or load()
    q64, k64, v64 = as_f64(q), as_f64(k), as_f64(v)
    a64, b64 = as_f64(alpha), as_f64(beta)
    p64 = as_f64(pool)
    B, R = v64.shape[0], v64.shape[1]
    D = v64.shape[-1]
    N = np.atleast_2d(node_row).shape[-1]
    P = p64.shape[0]
    out = np.full((B, R, Hv, D), np.nan, np.float64)
    states = np.full((B, N, Hv, D, D), np.nan, np.float64) if want_states else None
    u = np.full((B, R, Hv, D), np.nan, np.float64) if want_u else None
    err = lib.ora_verify(B, N, R, int(shared), _p(_i32(parent), ctypes.c_int32),
                         _p(_i32(node_row), ctypes.c_int32), _p(_i32(status), ctypes.c_int32),
                         _p(q64, ctypes.c_double), _p(k64, ctypes.c_double),
                         _p(v64, ctypes.c_double), _p(a64, ctypes.c_double),
                         _p(b64, ctypes.c_double), _p(p64, ctypes.c_double), P,
                         _p(_i32(state_idx), ctypes.c_int32), Hqk, Hv, D, int(norm),
                         _p(out, ctypes.c_double),
                         None if states is None else _p(states, ctypes.c_double),
                         None if u is None else _p(u, ctypes.c_double))
    res = (out, int(err))
    if want_states:
        res = res + (states,)
    if want_u:
        res = res + (u,)
    return res


def commit(parent, node_row, status, path, path_len, k, v, alpha, beta, pool,
           state_idx, Hqk: int, Hv: int, norm: bool, x=None, hist=None, W: int = 1,
           shared: bool = False, lib=None):
    """Accepted-path commit in fp64.  Starting from the committed state, replay
    the gated delta update for path[b][0..len-1] (root-level node first), write
    the state back in place; publish the conv history as the last W-1 entries
    of (old history ++ the accepted rows' conv inputs).  len 0 leaves both
    untouched; a malformed path or a bad / shared state slot leaves that
    request untouched and sets an error bit.

    LumoTree, Sec. IV-B (replay of recorded accepted operands into the fp32
    state in place) and Sec. V-A (one device path drives recurrent replay and
    convolution publication; padded path entries never advance state); Bole
    review, Algorithm 2 step 8 (no accepted draft -> state unchanged).
    Returns (pool_new float64, hist_new float64 or None, err).
    """
    lib = lib or load()
    k64, v64 = as_f64(k), as_f64(v)
    a64, b64 = as_f64(alpha), as_f64(beta)
    pool64 = as_f64(pool).copy()
    B, R = v64.shape[0], v64.shape[1]
    D = v64.shape[-1]
    N = np.atleast_2d(node_row).shape[-1]
    P = pool64.shape[0]
    path = _i32(path)
    Lmax = path.shape[1] if path.ndim == 2 and path.shape[1] > 0 else 1
    if path.size == 0:
        path = np.zeros((B, 1), np.int32)
    x64 = None if x is None else as_f64(x)
    h64 = None if hist is None else as_f64(hist).copy()
    C = 0 if x64 is None else x64.shape[-1]
    err = lib.ora_commit(B, N, R, int(shared), _p(_i32(parent), ctypes.c_int32),
                         _p(_i32(node_row), ctypes.c_int32), _p(_i32(status), ctypes.c_int32),
                         _p(path, ctypes.c_int32), _p(_i32(path_len), ctypes.c_int32), Lmax,
                         _p(k64, ctypes.c_double), _p(v64, ctypes.c_double),
                         _p(a64, ctypes.c_double), _p(b64, ctypes.c_double),
                         _p(pool64, ctypes.c_double), P, _p(_i32(state_idx), ctypes.c_int32),
                         Hqk, Hv, D, int(norm),
                         None if x64 is None else _p(x64, ctypes.c_double),
                         None if h64 is None else _p(h64, ctypes.c_double), C, W)
    return pool64, h64, int(err)
