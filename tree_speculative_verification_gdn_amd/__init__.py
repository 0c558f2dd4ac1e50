"""tree_speculative_verification_gdn_amd: tree-structured gated-delta-rule
verification and accepted-path commit for AMD Instinct MI355X (gfx950).

This module is the thin Python binding of the C ABI in ``include/gdn_tree.h``
(``libgdntree.so``, built from ``csrc/`` by ``_build.py``).  It marshals torch
device tensors into pointers, sizes and the caller's HIP stream; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
the shared library is missing, every call raises.

Entry points (same names as the C ABI):
    gdn_tree_desc_build, conv_ancestry_gather, gdn_tree_verify, gdn_tree_commit,
    the fused steady-state step: conv_ancestry_gather_publish,
    gdn_tree_commit_verify; and one launch per layer: gdn_path_resolve or
    gdn_step_prepare (once per step) + gdn_layer_step (once per layer)
Helper: TreeDesc (owns the descriptor's device arrays and the C struct).
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "GDN_OK", "GDN_ERR_ARG", "GDN_ERR_UNSUPPORTED", "GDN_ERR_HIP",
    "GDN_EV_PARENT", "GDN_EV_ROW", "GDN_EV_STATE", "GDN_EV_PATH", "GDN_EV_CTX",
    "GDN_DT_BF16", "GDN_DT_F32", "GDN_F_NORM_QK", "GDN_F_OUT_BF16", "GDN_F_VALU", "GDN_F_RAW_GATES",
    "GDN_F_DUMP_STATES",
    "GDN_ACT_NONE", "GDN_ACT_SILU", "GdnError", "TreeDesc", "library_path", "load_library",
    "gdn_tree_desc_build", "conv_ancestry_gather", "gdn_tree_verify", "gdn_tree_commit",
    "gdn_tree_commit_layers", "conv_ancestry_gather_publish", "gdn_tree_commit_verify",
    "gdn_tree_verify_store_u", "gdn_tree_commit_factored",
    "gdn_path_resolve", "gdn_step_prepare", "gdn_layer_step", "gdn_tree_attention_workspace_bytes",
    "gdn_tree_attention", "gdn_tree_attention_noalloc", "GDN_ATTN_NOALLOC_SCRATCH_BYTES", "gdn_tree_kv_publish",
]

# values mirror include/gdn_tree.h
GDN_OK, GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, -1, -4, -5
GDN_EV_PARENT, GDN_EV_ROW, GDN_EV_STATE, GDN_EV_PATH, GDN_EV_CTX = 1, 2, 4, 8, 16
GDN_DT_BF16, GDN_DT_F32 = 0, 1
GDN_F_NORM_QK, GDN_F_OUT_BF16, GDN_F_VALU, GDN_F_RAW_GATES, GDN_F_DUMP_STATES = 1, 2, 4, 8, 16
GDN_ACT_NONE, GDN_ACT_SILU = 0, 1
GDN_ATTN_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024

EXPORTED = ("gdn_tree_desc_build", "conv_ancestry_gather", "gdn_tree_verify",
            "gdn_tree_verify_store_u", "gdn_tree_commit_factored",
            "gdn_tree_commit", "gdn_tree_commit_layers", "conv_ancestry_gather_publish", "gdn_tree_commit_verify",
            "gdn_path_resolve", "gdn_step_prepare", "gdn_layer_step",
            "gdn_tree_attention_workspace_bytes", "gdn_tree_attention", "gdn_tree_attention_noalloc",
            "gdn_tree_kv_publish",
            "gdn_status_string", "gdn_abi_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_lib = None


class GdnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: status {code} ({_status_string(code)})")
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, "libgdntree.so")


class gdn_tree_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("R", ctypes.c_int32),
        ("W", ctypes.c_int32), ("shared", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("parent", ctypes.c_void_p), ("node_row", ctypes.c_void_p), ("depth", ctypes.c_void_p),
        ("anc", ctypes.c_void_p), ("conv_src", ctypes.c_void_p), ("status", ctypes.c_void_p),
    ]


def load_library():
    """Load libgdntree.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing; build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950)")
        lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        dp = ctypes.POINTER(gdn_tree_desc)
        lib.gdn_tree_desc_build.restype = i32
        lib.gdn_tree_desc_build.argtypes = [dp, vp, vp]
        lib.conv_ancestry_gather.restype = i32
        lib.conv_ancestry_gather.argtypes = [dp, vp, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp]
        lib.gdn_tree_verify.restype = i32
        lib.gdn_tree_verify.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp, vp, i32, vp, vp,
                                        i32, i32, i32, i32, i32, i32, vp, vp, vp]
        lib.gdn_tree_verify_store_u.restype = i32
        lib.gdn_tree_verify_store_u.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp, vp, i32, vp, vp, vp, vp,
                                                i32, i32, i32, i32, i32, i32, vp, vp, vp]
        lib.gdn_tree_commit_factored.restype = i32
        lib.gdn_tree_commit_factored.argtypes = [dp, vp, vp, i32, vp, i64, vp, vp, vp, i32, vp, i32, i32,
                                                 i32, i32, i32, vp, vp, vp]
        lib.gdn_tree_commit.restype = i32
        lib.gdn_tree_commit.argtypes = [dp, vp, vp, i32, vp, vp, i64, i64, vp, vp, vp, i32, vp,
                                        vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
        lib.gdn_tree_commit_layers.restype = i32
        lib.gdn_tree_commit_layers.argtypes = [dp, vp, vp, i32, i32, vp, vp, i64, i64, i64, i64,
                                               vp, vp, i64, vp, i64, i32, vp, i32, i32, i32, i32,
                                               i32, i32, vp, vp, vp]
        lib.conv_ancestry_gather_publish.restype = i32
        lib.conv_ancestry_gather_publish.argtypes = [dp, vp, vp, i32, vp, vp, vp, vp, i32, i32,
                                                     dp, vp, vp, i32, vp, vp, vp]
        lib.gdn_tree_commit_verify.restype = i32
        lib.gdn_tree_commit_verify.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp, vp, i32, vp, vp,
                                               dp, vp, vp, i32, vp, vp, i64, i64, vp, vp,
                                               i32, i32, i32, i32, i32, i32, vp, vp, vp]
        lib.gdn_path_resolve.restype = i32
        lib.gdn_path_resolve.argtypes = [dp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
        lib.gdn_step_prepare.restype = i32
        lib.gdn_step_prepare.argtypes = [dp, dp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
        lib.gdn_layer_step.restype = i32
        lib.gdn_layer_step.argtypes = [dp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                       dp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                       vp, vp, vp]
        lib.gdn_tree_attention_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn_tree_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.gdn_tree_attention.restype = i32
        lib.gdn_tree_attention.argtypes = [dp, vp, vp, vp, i32, vp, vp, vp, ctypes.c_size_t, i32, i32,
                                           i32, i32, ctypes.c_float, i32, vp, vp]
        lib.gdn_tree_attention_noalloc.restype = i32
        lib.gdn_tree_attention_noalloc.argtypes = [dp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32,
                                                   ctypes.c_float, i32, vp, vp]
        lib.gdn_tree_kv_publish.restype = i32
        lib.gdn_tree_kv_publish.argtypes = [dp, vp, vp, i32, vp, vp, i32, vp, i32, i32, vp, vp]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_status_string.argtypes = [i32]
        lib.gdn_abi_version.restype = i32
        lib.gdn_abi_version.argtypes = []
        _lib = lib
        return lib


def _status_string(code: int) -> str:
    try:
        return load_library().gdn_status_string(int(code)).decode()
    except Exception:  # pragma: no cover
        return "?"


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_DT_BF16
    if t.dtype == torch.float32:
        return GDN_DT_F32
    raise ValueError(f"unsupported operand dtype {t.dtype}")


def _rows_view(t, name):
    """(row stride in elements, heads, head dim) of a [B, R, H, D] view whose
    element (b, r, h, d) sits at (b*R + r)*row_stride + h*D + d."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, R, H, D]")
    B, R, H, D = t.shape
    s0, s1, s2, s3 = t.stride()
    if s3 != 1 or s2 != D or (B > 1 and s0 != R * s1):
        raise ValueError(f"{name}: layout not expressible as rows of stride {s1}")
    return s1, H, D


def _gate_flags(flags, gate_params):
    """flags, with GDN_F_RAW_GATES set when gate parameters are passed: alpha
    and beta then hold raw gate inputs, gate_params the per-head A_log and
    dt_bias (float32 [2, Hv], or [L, 2, Hv] for the layer-batched commit)."""
    return int(flags) | (GDN_F_RAW_GATES if gate_params is not None else 0)


def _check(code, what, raise_on_error):
    if raise_on_error and code < 0:
        raise GdnError(code, what)
    return code


class TreeDesc:
    """Descriptor of B requests' draft trees (one per request, or one shared).

    Holds the input arrays (parent, node_row: int32 [T][N] on the device) and
    the device outputs gdn_tree_desc_build fills (depth, anc, conv_src,
    status), plus the C struct pointing at them.  Allocation is torch's.
    """

    def __init__(self, parent, node_row, R: int, W: int = 1, B: int | None = None,
                 shared: bool = False):
        import torch
        if parent.dtype != torch.int32 or node_row.dtype != torch.int32:
            raise ValueError("parent and node_row must be int32")
        self.parent = parent.contiguous()
        self.node_row = node_row.contiguous()
        T, N = self.parent.shape
        self.B = int(B if B is not None else T)
        self.N, self.R, self.W, self.shared = int(N), int(R), int(W), bool(shared)
        dev = self.parent.device
        self.depth = torch.zeros((T, N), dtype=torch.int32, device=dev)
        self.anc = torch.zeros((T, N), dtype=torch.int64, device=dev)
        self.conv_src = torch.zeros((T, N, max(W - 1, 1)), dtype=torch.int32, device=dev)
        self.status = torch.zeros((T,), dtype=torch.int32, device=dev)
        self.c = gdn_tree_desc(self.B, self.N, self.R, self.W, int(self.shared), 0,
                               self.parent.data_ptr(), self.node_row.data_ptr(),
                               self.depth.data_ptr(), self.anc.data_ptr(),
                               self.conv_src.data_ptr() if W > 1 else None,
                               self.status.data_ptr())

    def ref(self):
        return ctypes.byref(self.c)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def gdn_tree_desc_build(desc: TreeDesc, err, stream=None, raise_on_error=True) -> int:
    """Validate trees and build depth / ancestor mask / conv sources / status."""
    code = load_library().gdn_tree_desc_build(desc.ref(), _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_desc_build", raise_on_error)


def conv_ancestry_gather(desc: TreeDesc, x, hist, state_idx, w, bias, y, act: int, err,
                         stream=None, raise_on_error=True) -> int:
    """Ancestry-gathered causal conv1d: x [B][R][C] bf16, hist [P][W-1][C] bf16,
    w [C][W] bf16, bias fp32 [C] or None -> y [B][R][C] bf16."""
    C = int(x.shape[-1])
    P = int(hist.shape[0]) if hist is not None else 1
    code = load_library().conv_ancestry_gather(desc.ref(), _ptr(x), _ptr(hist), P,
                                               _ptr(state_idx), _ptr(w), _ptr(bias), _ptr(y),
                                               C, int(act), _ptr(err), _stream(stream))
    return _check(code, "conv_ancestry_gather", raise_on_error)


def gdn_tree_verify(desc: TreeDesc, q, k, v, alpha, beta, state_pool, state_idx, out, err,
                    flags: int = 0, stream=None, raise_on_error=True, gate_params=None) -> int:
    """Every node's output.  q, k: [B, R, Hqk, D] views (row-strided), v: [B, R, Hv, D],
    alpha/beta fp32 [B, R, Hv], state_pool fp32 [P, Hv, D, D], state_idx int32 [B],
    out [B, R, Hv, D] fp32 (bf16 with GDN_F_OUT_BF16)."""
    rs_qk, Hqk, dk = _rows_view(q, "q")
    rs_k, Hk, dk2 = _rows_view(k, "k")
    rs_v, Hv, dv = _rows_view(v, "v")
    if rs_k != rs_qk or Hk != Hqk or dk2 != dk or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q and k must share layout and dtype with v")
    P = int(state_pool.shape[0])
    code = load_library().gdn_tree_verify(desc.ref(), _ptr(q), _ptr(k), _ptr(v), rs_qk, rs_v,
                                          _ptr(alpha), _ptr(beta), _ptr(state_pool), P,
                                          _ptr(state_idx), _ptr(out), Hqk, Hv, dk, dv,
                                          _dtype_code(q), _gate_flags(flags, gate_params),
                                          _ptr(gate_params), _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_verify", raise_on_error)


def gdn_tree_verify_store_u(desc: TreeDesc, q, k, v, alpha, beta, state_pool, state_idx, out, u, err,
                            flags: int = 0, stream=None, raise_on_error=True, gate_params=None,
                            dump=None) -> int:
    """gdn_tree_verify, plus every node's delta correction into u (fp32
    [B, R, Hv, D], the layout of out).  With ``dump`` (fp32 [B, N, Hv, D, D],
    debug) GDN_F_DUMP_STATES is set and every node's state is written there."""
    if dump is not None:
        flags |= GDN_F_DUMP_STATES
    rs_qk, Hqk, dk = _rows_view(q, "q")
    rs_k, Hk, dk2 = _rows_view(k, "k")
    rs_v, Hv, dv = _rows_view(v, "v")
    if rs_k != rs_qk or Hk != Hqk or dk2 != dk or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q and k must share layout and dtype with v")
    P = int(state_pool.shape[0])
    code = load_library().gdn_tree_verify_store_u(desc.ref(), _ptr(q), _ptr(k), _ptr(v), rs_qk, rs_v,
                                                  _ptr(alpha), _ptr(beta), _ptr(state_pool), P,
                                                  _ptr(state_idx), _ptr(out), _ptr(u), _ptr(dump), Hqk, Hv,
                                                  dk, dv,
                                                  _dtype_code(q), _gate_flags(flags, gate_params),
                                                  _ptr(gate_params), _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_verify_store_u", raise_on_error)


def gdn_tree_commit_factored(desc: TreeDesc, path, path_len, k, u, alpha, state_pool, state_idx, err,
                             flags: int = 0, stream=None, raise_on_error=True, gate_params=None) -> int:
    """Commit path [B, Lmax] (len path_len [B]) into state_pool in place from
    the stored corrections u [B, R, Hv, 128] (S = P_a S_pre + sum (P_a/P_j)
    u_j k_j^T) and the bf16 k rows [B, R, Hqk, 128]."""
    rs_qk, Hqk, dk = _rows_view(k, "k")
    Hv = int(u.shape[2])
    P = int(state_pool.shape[0])
    Lmax = int(path.shape[1])
    code = load_library().gdn_tree_commit_factored(desc.ref(), _ptr(path), _ptr(path_len), Lmax, _ptr(k),
                                                   rs_qk, _ptr(u), _ptr(alpha), _ptr(state_pool), P,
                                                   _ptr(state_idx), Hqk, Hv, dk, int(u.shape[3]),
                                                   _gate_flags(flags, gate_params), _ptr(gate_params),
                                                   _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_commit_factored", raise_on_error)


def gdn_tree_commit(desc: TreeDesc, path, path_len, k, v, alpha, beta, state_pool, state_idx,
                    err, Hqk: int | None = None, flags: int = 0, x=None, hist=None,
                    stream=None, raise_on_error=True, gate_params=None) -> int:
    """Replay path [B, Lmax] (len path_len [B]) into state_pool in place; with
    x / hist also publish the conv history."""
    rs_qk, Hk, dk = _rows_view(k, "k")
    rs_v, Hv, dv = _rows_view(v, "v")
    Hqk = Hk if Hqk is None else Hqk
    P = int(state_pool.shape[0])
    Lmax = int(path.shape[1])
    C = int(x.shape[-1]) if x is not None else 0
    code = load_library().gdn_tree_commit(desc.ref(), _ptr(path), _ptr(path_len), Lmax, _ptr(k),
                                          _ptr(v), rs_qk, rs_v, _ptr(alpha), _ptr(beta),
                                          _ptr(state_pool), P, _ptr(state_idx), _ptr(x),
                                          _ptr(hist), C, Hqk, Hv, dk, dv, _dtype_code(k),
                                          _gate_flags(flags, gate_params), _ptr(gate_params),
                                          _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_commit", raise_on_error)


def _layer_stride(t, name, L):
    if t.dim() < 1 or int(t.shape[0]) != L:
        raise ValueError(f"{name} must have the layer count {L} as its first dimension")
    return int(t.stride(0)) if L > 1 else 0


def gdn_tree_commit_layers(desc: TreeDesc, path, path_len, k, v, alpha, beta, state_pool,
                           state_idx, err, Hqk: int | None = None, flags: int = 0, stream=None,
                           raise_on_error=True, gate_params=None) -> int:
    """Replay path [B, Lmax] into every layer's state in one launch: k
    [L, B, R, Hqk, dk], v [L, B, R, Hv, dv], alpha / beta [L, B, R, Hv],
    state_pool [L, P, Hv, dv, dk]; layer l is gdn_tree_commit on the l-th
    slices."""
    L = int(k.shape[0])
    rs_qk, Hk, dk = _rows_view(k[0], "k")
    rs_v, Hv, dv = _rows_view(v[0], "v")
    Hqk = Hk if Hqk is None else Hqk
    for t, name in ((alpha, "alpha"), (beta, "beta")):
        if t.dim() != 4 or not t[0].is_contiguous():
            raise ValueError(f"{name} must be [L, B, R, Hv] with contiguous layers")
    if alpha.stride(0) != beta.stride(0):
        raise ValueError("alpha and beta need the same layer stride")
    if not state_pool[0].is_contiguous():
        raise ValueError("state_pool must be [L, P, Hv, dv, dk] with contiguous layers")
    P = int(state_pool.shape[1])
    Lmax = int(path.shape[1])
    code = load_library().gdn_tree_commit_layers(
        desc.ref(), _ptr(path), _ptr(path_len), Lmax, L, _ptr(k), _ptr(v), rs_qk, rs_v,
        _layer_stride(k, "k", L), _layer_stride(v, "v", L), _ptr(alpha), _ptr(beta),
        _layer_stride(alpha, "alpha", L), _ptr(state_pool),
        _layer_stride(state_pool, "state_pool", L), P, _ptr(state_idx), Hqk, Hv, dk, dv,
        _dtype_code(k), _gate_flags(flags, gate_params), _ptr(gate_params), _ptr(err),
        _stream(stream))
    return _check(code, "gdn_tree_commit_layers", raise_on_error)


def conv_ancestry_gather_publish(desc: TreeDesc, x, hist, state_idx, w, bias, y, act: int,
                                 prev: TreeDesc, path_rows, path_n, x_prev, err, stream=None,
                                 raise_on_error=True) -> int:
    """Publish the conv history of the previous step's accepted path (prev's
    tree; the path resolved by gdn_path_resolve into path_rows [B, Lmax] and
    path_n [B]; its conv input x_prev [B, prev R, C]), then convolve desc's
    tree as conv_ancestry_gather does."""
    C = int(x.shape[-1])
    P = int(hist.shape[0]) if hist is not None else 1
    Lmax = int(path_rows.shape[1])
    code = load_library().conv_ancestry_gather_publish(
        desc.ref(), _ptr(x), _ptr(hist), P, _ptr(state_idx), _ptr(w), _ptr(bias), _ptr(y), C,
        int(act), prev.ref(), _ptr(path_rows), _ptr(path_n), Lmax, _ptr(x_prev), _ptr(err),
        _stream(stream))
    return _check(code, "conv_ancestry_gather_publish", raise_on_error)


def gdn_tree_commit_verify(desc: TreeDesc, q, k, v, alpha, beta, state_pool, state_idx, out,
                           prev: TreeDesc, path_rows, path_n, k_prev, v_prev, alpha_prev,
                           beta_prev, err, flags: int = 0, stream=None,
                           raise_on_error=True, gate_params=None) -> int:
    """Commit the previous step's accepted path (prev's tree; the path resolved
    into path_rows / path_n; its recorded k_prev, v_prev, alpha_prev,
    beta_prev) into state_pool, then verify desc's tree from the committed
    state into out (layouts as in gdn_tree_verify)."""
    rs_qk, Hqk, dk = _rows_view(q, "q")
    rs_k, Hk, dk2 = _rows_view(k, "k")
    rs_v, Hv, dv = _rows_view(v, "v")
    if rs_k != rs_qk or Hk != Hqk or dk2 != dk or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q and k must share layout and dtype with v")
    rs_qkp, Hkp, _ = _rows_view(k_prev, "k_prev")
    rs_vp, Hvp, _ = _rows_view(v_prev, "v_prev")
    if Hkp != Hqk or Hvp != Hv or k_prev.dtype != q.dtype or v_prev.dtype != q.dtype:
        raise ValueError("previous operands must match the new ones in heads and dtype")
    P = int(state_pool.shape[0])
    Lmax = int(path_rows.shape[1])
    code = load_library().gdn_tree_commit_verify(
        desc.ref(), _ptr(q), _ptr(k), _ptr(v), rs_qk, rs_v, _ptr(alpha), _ptr(beta),
        _ptr(state_pool), P, _ptr(state_idx), _ptr(out), prev.ref(), _ptr(path_rows), _ptr(path_n),
        Lmax, _ptr(k_prev), _ptr(v_prev), rs_qkp, rs_vp, _ptr(alpha_prev), _ptr(beta_prev), Hqk,
        Hv, dk, dv, _dtype_code(q), _gate_flags(flags, gate_params), _ptr(gate_params), _ptr(err),
        _stream(stream))
    return _check(code, "gdn_tree_commit_verify", raise_on_error)


def gdn_tree_attention_workspace_bytes(B: int, N: int, Hq: int, D: int, splits: int) -> int:
    return int(load_library().gdn_tree_attention_workspace_bytes(B, N, Hq, D, splits))


def gdn_tree_attention(desc: TreeDesc, q, k_cache, v_cache, ctx_len, out, workspace, err,
                       splits: int, scale: float | None = None, flags: int = 0, stream=None,
                       raise_on_error=True) -> int:
    """Tree attention: q [B, N, Hq, D] (logical node rows), k_cache / v_cache
    [B, S, Hkv, D] with the candidates at ctx_len[b] + node_row, out
    [B, N, Hq, D]; workspace: a device buffer of at least
    gdn_tree_attention_workspace_bytes(...) bytes."""
    B, N, Hq, D = (int(x) for x in q.shape)
    S, Hkv = int(k_cache.shape[1]), int(k_cache.shape[2])
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    scale = 1.0 / float(D) ** 0.5 if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    code = load_library().gdn_tree_attention(desc.ref(), _ptr(q), _ptr(k_cache), _ptr(v_cache), S,
                                             _ptr(ctx_len), _ptr(out), _ptr(workspace), nbytes,
                                             int(splits), Hq, Hkv, D, scale, int(flags), _ptr(err),
                                             _stream(stream))
    return _check(code, "gdn_tree_attention", raise_on_error)


def gdn_tree_attention_noalloc(desc: TreeDesc, q, k_cache, v_cache, ctx_len, out, err, splits: int,
                               scale: float | None = None, flags: int = 0, stream=None,
                               raise_on_error=True) -> int:
    """gdn_tree_attention without a workspace: the split partials go to the
    library's own scratch (GDN_ATTN_NOALLOC_SCRATCH_BYTES per GPU); the call
    allocates nothing.  Calls that overlap on one GPU share that scratch."""
    B, N, Hq, D = (int(x) for x in q.shape)
    S, Hkv = int(k_cache.shape[1]), int(k_cache.shape[2])
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    scale = 1.0 / float(D) ** 0.5 if scale is None else float(scale)
    code = load_library().gdn_tree_attention_noalloc(desc.ref(), _ptr(q), _ptr(k_cache), _ptr(v_cache), S,
                                                     _ptr(ctx_len), _ptr(out), int(splits), Hq, Hkv, D,
                                                     scale, int(flags), _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_attention_noalloc", raise_on_error)


def gdn_tree_kv_publish(prev: TreeDesc, path_rows, path_n, k_cache, v_cache, ctx_len, err,
                        stream=None, raise_on_error=True) -> int:
    """Move the accepted path's KV entries (resolved rows path_rows [B, Lmax],
    counts path_n [B]) to the positions right after each request's prefix."""
    S, Hkv, D = int(k_cache.shape[1]), int(k_cache.shape[2]), int(k_cache.shape[3])
    Lmax = int(path_rows.shape[1])
    code = load_library().gdn_tree_kv_publish(prev.ref(), _ptr(path_rows), _ptr(path_n), Lmax,
                                              _ptr(k_cache), _ptr(v_cache), S, _ptr(ctx_len), Hkv,
                                              D, _ptr(err), _stream(stream))
    return _check(code, "gdn_tree_kv_publish", raise_on_error)


def gdn_path_resolve(prev: TreeDesc, path, path_len, state_idx, P: int, path_rows, path_n, err,
                     stream=None, raise_on_error=True) -> int:
    """Validate the previous step's accepted path (path [B, Lmax], path_len
    [B]) against prev's tree; write its physical rows (path_rows int32 [B,
    Lmax]) and the number of nodes each layer commits (path_n int32 [B]; -1
    for a request whose slot is out of range or shared)."""
    Lmax = int(path.shape[1])
    code = load_library().gdn_path_resolve(prev.ref(), _ptr(path), _ptr(path_len), Lmax,
                                           _ptr(state_idx), int(P), _ptr(path_rows),
                                           _ptr(path_n), _ptr(err), _stream(stream))
    return _check(code, "gdn_path_resolve", raise_on_error)


def gdn_step_prepare(desc: TreeDesc, prev: TreeDesc, path, path_len, state_idx, P: int, path_rows,
                     path_n, err, stream=None, raise_on_error=True) -> int:
    """gdn_tree_desc_build(desc) and gdn_path_resolve(prev, ...) in one launch."""
    Lmax = int(path.shape[1])
    code = load_library().gdn_step_prepare(desc.ref(), prev.ref(), _ptr(path), _ptr(path_len), Lmax,
                                           _ptr(state_idx), int(P), _ptr(path_rows), _ptr(path_n),
                                           _ptr(err), _stream(stream))
    return _check(code, "gdn_step_prepare", raise_on_error)


def gdn_layer_step(desc: TreeDesc, x, w, bias, act: int, hist_in, hist_out, alpha, beta,
                   state_pool, state_idx, out, prev: TreeDesc, x_prev, alpha_prev, beta_prev,
                   path_rows, path_n, err, Hqk: int, flags: int = 0, y=None, stream=None,
                   gate_params=None,
                   raise_on_error=True) -> int:
    """One GDN layer's step in one launch: commit the previous path (resolved
    by gdn_path_resolve) with its k/v recomputed from x_prev and hist_in,
    write the new conv history to hist_out, convolve desc's tree (x [B, R, C],
    channels [q | k | v]) and verify it into out [B, R, Hv, 128].  y, if
    given, receives the conv output [B, R, C] (bf16)."""
    P, Hv, dv, dk = (int(d) for d in state_pool.shape)
    Lmax = int(path_rows.shape[1])
    code = load_library().gdn_layer_step(
        desc.ref(), _ptr(x), _ptr(w), _ptr(bias), int(act), _ptr(hist_in), _ptr(hist_out),
        _ptr(alpha), _ptr(beta), _ptr(state_pool), P, _ptr(state_idx), _ptr(out), _ptr(y),
        prev.ref(), _ptr(x_prev), _ptr(alpha_prev), _ptr(beta_prev), _ptr(path_rows),
        _ptr(path_n), Lmax, int(Hqk), Hv, dk, dv, _gate_flags(flags, gate_params), _ptr(gate_params),
        _ptr(err), _stream(stream))
    return _check(code, "gdn_layer_step", raise_on_error)
