"""The C-ABI library loads on the CPU host and exports every entry point that
include/gdn_tree.h declares; argument checks return their codes before any
device work (no kernel is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

import tree_speculative_verification_gdn_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_tree.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.library_path()):
        pytest.skip("libgdntree.so not built")
    return g.load_library()


def test_header_declares_the_entry_points():
    decl = declared_functions()
    for name in ("gdn_tree_desc_build", "conv_ancestry_gather", "gdn_tree_verify", "gdn_tree_commit",
                 "gdn_tree_commit_layers", "conv_ancestry_gather_publish", "gdn_tree_commit_verify",
                 "gdn_path_resolve", "gdn_step_prepare", "gdn_layer_step", "gdn_tree_attention",
                 "gdn_tree_kv_publish", "gdn_tree_verify_store_u", "gdn_tree_commit_factored"):
        assert name in decl
    assert set(decl) == set(g.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", g.library_path()], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name


def test_status_strings_and_version(lib):
    assert lib.gdn_abi_version() == 8
    assert lib.gdn_status_string(0) == b"ok"
    assert lib.gdn_status_string(-1) == b"invalid argument"
    assert lib.gdn_status_string(-4) == b"unsupported size"


def _desc(**kw):
    base = dict(B=2, N=7, R=8, W=4, shared=0, reserved=0, parent=16, node_row=32, depth=48,
                anc=64, conv_src=80, status=96)
    base.update(kw)
    return g.gdn_tree_desc(**base)


def test_argument_checks_fail_before_launch(lib):
    # fake (never dereferenced) device addresses: validation rejects before any launch
    err = ctypes.c_void_p(128)
    assert lib.gdn_tree_desc_build(None, err, None) == g.GDN_ERR_ARG
    assert lib.gdn_tree_desc_build(ctypes.byref(_desc(N=65)), err, None) == g.GDN_ERR_UNSUPPORTED
    assert lib.gdn_tree_desc_build(ctypes.byref(_desc(N=0)), err, None) == g.GDN_ERR_UNSUPPORTED
    assert lib.gdn_tree_desc_build(ctypes.byref(_desc(R=5)), err, None) == g.GDN_ERR_ARG
    assert lib.gdn_tree_desc_build(ctypes.byref(_desc(W=5)), err, None) == g.GDN_ERR_UNSUPPORTED
    assert lib.gdn_tree_desc_build(ctypes.byref(_desc(conv_src=None)), err, None) == g.GDN_ERR_ARG
    assert lib.gdn_tree_desc_build(ctypes.byref(_desc()), None, None) == g.GDN_ERR_ARG
    d = ctypes.byref(_desc())
    p = ctypes.c_void_p(256)
    # verify: bad head ratio, d_k != d_v, bad dtype, unknown flag, short row stride
    V = lib.gdn_tree_verify
    assert V(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, 3, 32, 128, 128, 0, 0, None, err, None) == g.GDN_ERR_ARG
    assert V(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, 16, 32, 128, 64, 0, 0, None, err, None) == g.GDN_ERR_UNSUPPORTED
    assert V(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, 16, 32, 96, 96, 0, 0, None, err, None) == g.GDN_ERR_UNSUPPORTED
    assert V(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, 16, 32, 128, 128, 7, 0, None, err, None) == g.GDN_ERR_ARG
    assert V(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, 16, 32, 128, 128, 0, 64, None, err, None) == g.GDN_ERR_ARG
    assert V(d, p, p, p, 100, 4096, p, p, p, 4, p, p, 16, 32, 128, 128, 0, 0, None, err, None) == g.GDN_ERR_ARG
    assert V(d, None, p, p, 2048, 4096, p, p, p, 4, p, p, 16, 32, 128, 128, 0, 0, None, err, None) == g.GDN_ERR_ARG
    # commit: Lmax out of range, x without hist
    Cm = lib.gdn_tree_commit
    assert Cm(d, p, p, 0, p, p, 2048, 4096, p, p, p, 4, p, None, None, 0, 16, 32, 128, 128, 0, 0, None, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Cm(d, p, p, 65, p, p, 2048, 4096, p, p, p, 4, p, None, None, 0, 16, 32, 128, 128, 0, 0, None, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Cm(d, p, p, 7, p, p, 2048, 4096, p, p, p, 4, p, p, None, 8, 16, 32, 128, 128, 0, 0, None, err, None) == g.GDN_ERR_ARG
    # stored-U verify: no u buffer, misaligned u, unknown flag; the state
    # dump without its buffer, misaligned, or at fp32 / d != 128
    VU = lib.gdn_tree_verify_store_u
    DS = g.GDN_F_DUMP_STATES
    assert VU(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, None, None, 16, 32, 128, 128, 0, 0, None, err,
              None) == g.GDN_ERR_ARG
    assert VU(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, ctypes.c_void_p(258), None, 16, 32, 128, 128, 0, 0, None,
              err, None) == g.GDN_ERR_ARG
    assert VU(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, p, None, 16, 32, 128, 128, 0, 64, None, err,
              None) == g.GDN_ERR_ARG
    assert VU(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, p, None, 16, 32, 128, 128, 0, DS, None, err,
              None) == g.GDN_ERR_ARG
    assert VU(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, p, ctypes.c_void_p(264), 16, 32, 128, 128, 0, DS, None, err,
              None) == g.GDN_ERR_ARG
    assert VU(d, p, p, p, 2048, 4096, p, p, p, 4, p, p, p, p, 16, 32, 128, 128, 1, DS, None, err,
              None) == g.GDN_ERR_UNSUPPORTED
    assert VU(d, p, p, p, 1024, 2048, p, p, p, 4, p, p, p, p, 16, 32, 64, 64, 0, DS, None, err,
              None) == g.GDN_ERR_UNSUPPORTED
    CF = lib.gdn_tree_commit_factored
    assert CF(d, p, p, 7, p, 2048, p, p, p, 4, p, 16, 32, 64, 64, 0, None, err, None) == g.GDN_ERR_UNSUPPORTED
    assert CF(d, p, p, 7, p, 2048, p, p, p, 4, p, 16, 32, 128, 128, g.GDN_F_OUT_BF16, None, err, None) == g.GDN_ERR_ARG
    assert CF(d, p, p, 65, p, 2048, p, p, p, 4, p, 16, 32, 128, 128, 0, None, err, None) == g.GDN_ERR_UNSUPPORTED
    assert CF(d, p, p, 7, p, 2048, ctypes.c_void_p(264), p, p, 4, p, 16, 32, 128, 128, 0, None, err,
              None) == g.GDN_ERR_ARG
    assert CF(d, p, p, 7, p, 2046, p, p, p, 4, p, 16, 32, 128, 128, 0, None, err, None) == g.GDN_ERR_ARG
    # commit over layers (B = 2, R = 8: 16 rows; P = 4): no layers, overlapping
    # layer strides, an unknown flag, a pool stride that breaks alignment
    Cl = lib.gdn_tree_commit_layers
    ok = (16 * 2048, 16 * 4096, 16 * 32, 4 * 32 * 128 * 128)

    def cl(layers=3, strides=ok, flags=0, Lmax=7, gp=None):
        return Cl(d, p, p, Lmax, layers, p, p, 2048, 4096, strides[0], strides[1], p, p, strides[2], p,
                  strides[3], 4, p, 16, 32, 128, 128, 0, flags, gp, err, None)
    assert cl(layers=0) == g.GDN_ERR_ARG
    assert cl(strides=(15 * 2048,) + ok[1:]) == g.GDN_ERR_ARG
    assert cl(strides=ok[:1] + (16 * 4096 - 1,) + ok[2:]) == g.GDN_ERR_ARG
    assert cl(strides=ok[:2] + (16 * 31,) + ok[3:]) == g.GDN_ERR_ARG
    assert cl(strides=ok[:3] + (ok[3] - 4,)) == g.GDN_ERR_ARG
    assert cl(strides=ok[:3] + (ok[3] + 2,)) == g.GDN_ERR_ARG
    assert cl(flags=g.GDN_F_OUT_BF16) == g.GDN_ERR_ARG
    assert cl(Lmax=65) == g.GDN_ERR_UNSUPPORTED
    assert cl(flags=g.GDN_F_RAW_GATES) == g.GDN_ERR_ARG      # raw gates without parameters
    assert cl(flags=g.GDN_F_RAW_GATES, gp=ctypes.c_void_p(258)) == g.GDN_ERR_ARG  # misaligned
    # conv: channel count not a multiple of 4, bad activation
    Cv = lib.conv_ancestry_gather
    assert Cv(d, p, p, 4, p, p, None, p, 8190, 1, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Cv(d, p, p, 4, p, p, None, p, 8192, 2, err, None) == g.GDN_ERR_ARG


def test_fused_step_argument_checks_fail_before_launch(lib):
    err = ctypes.c_void_p(128)
    d = ctypes.byref(_desc())
    other_b = ctypes.byref(_desc(B=3))
    other_w = ctypes.byref(_desc(W=2))
    p = ctypes.c_void_p(256)
    # conv with publication: previous tree of another batch or conv width,
    # Lmax out of range, missing previous input
    Cp = lib.conv_ancestry_gather_publish
    assert Cp(d, p, p, 4, p, p, None, p, 8192, 1, other_b, p, p, 7, p, err, None) == g.GDN_ERR_ARG
    assert Cp(d, p, p, 4, p, p, None, p, 8192, 1, other_w, p, p, 7, p, err, None) == g.GDN_ERR_ARG
    assert Cp(d, p, p, 4, p, p, None, p, 8192, 1, d, p, p, 0, p, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Cp(d, p, p, 4, p, p, None, p, 8192, 1, d, p, p, 7, None, err, None) == g.GDN_ERR_ARG
    assert Cp(d, p, p, 4, p, p, None, p, 8192, 1, None, p, p, 7, p, err, None) == g.GDN_ERR_ARG
    # commit + verify: previous tree of another batch, Lmax out of range, short
    # previous row stride, missing previous gates, unknown flag
    F = lib.gdn_tree_commit_verify
    args = dict(q=p, k=p, v=p, rqk=2048, rv=4096, a=p, b=p, pool=p, P=4, sidx=p, out=p, prev=d,
                path=p, plen=p, Lmax=7, kp=p, vp=p, rqkp=2048, rvp=4096, ap=p, bp=p, Hqk=16, Hv=32,
                dk=128, dv=128, dt=0, fl=0)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return F(d, a["q"], a["k"], a["v"], a["rqk"], a["rv"], a["a"], a["b"], a["pool"], a["P"],
                 a["sidx"], a["out"], a["prev"], a["path"], a["plen"], a["Lmax"], a["kp"], a["vp"],
                 a["rqkp"], a["rvp"], a["ap"], a["bp"], a["Hqk"], a["Hv"], a["dk"], a["dv"], a["dt"],
                 a["fl"], a.get("gp"), err, None)
    assert call(prev=other_b) == g.GDN_ERR_ARG
    assert call(Lmax=65) == g.GDN_ERR_UNSUPPORTED
    assert call(fl=g.GDN_F_RAW_GATES) == g.GDN_ERR_ARG      # raw gates without parameters
    assert call(rqkp=100) == g.GDN_ERR_ARG
    assert call(bp=None) == g.GDN_ERR_ARG
    assert call(fl=64) == g.GDN_ERR_ARG
    assert call(Hqk=3) == g.GDN_ERR_ARG
    assert call(pool=ctypes.c_void_p(260)) == g.GDN_ERR_ARG  # state pool not 16-byte aligned


def test_layer_step_argument_checks_fail_before_launch(lib):
    err = ctypes.c_void_p(128)
    d = ctypes.byref(_desc(N=27, R=32))
    other_b = ctypes.byref(_desc(B=3, N=27, R=32))
    big = ctypes.byref(_desc(N=33, R=40))
    p = ctypes.c_void_p(256)
    # path resolve: missing outputs, Lmax out of range, no slots
    Rz = lib.gdn_path_resolve
    assert Rz(d, p, p, 7, p, 4, p, None, err, None) == g.GDN_ERR_ARG
    assert Rz(d, p, p, 0, p, 4, p, p, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Rz(d, p, p, 65, p, 4, p, p, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Rz(d, p, p, 7, p, 0, p, p, err, None) == g.GDN_ERR_ARG
    assert Rz(None, p, p, 7, p, 4, p, p, err, None) == g.GDN_ERR_ARG
    # step prepare: previous tree of another batch, Lmax out of range, missing rows
    Sp = lib.gdn_step_prepare
    assert Sp(d, other_b, p, p, 7, p, 4, p, p, err, None) == g.GDN_ERR_ARG
    assert Sp(d, d, p, p, 65, p, 4, p, p, err, None) == g.GDN_ERR_UNSUPPORTED
    assert Sp(d, d, p, p, 7, p, 4, None, p, err, None) == g.GDN_ERR_ARG
    # layer step: C = 2*16*128 + 32*128 = 8192 channels, history bytes P*(W-1)*C*2
    L = lib.gdn_layer_step
    hbytes = 4 * 3 * 8192 * 2
    args = dict(d=d, x=p, w=p, bias=None, act=1, hin=ctypes.c_void_p(1 << 20),
                hout=ctypes.c_void_p((1 << 20) + hbytes), a=p, b=p, pool=p, P=4, sidx=p, out=p,
                y=None, prev=d, xp=p, ap=p, bp=p, prow=p, pn=p, Lmax=7, Hqk=16, Hv=32, dk=128,
                dv=128, fl=1)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L(a["d"], a["x"], a["w"], a["bias"], a["act"], a["hin"], a["hout"], a["a"], a["b"],
                 a["pool"], a["P"], a["sidx"], a["out"], a["y"], a["prev"], a["xp"], a["ap"], a["bp"],
                 a["prow"], a["pn"], a["Lmax"], a["Hqk"], a["Hv"], a["dk"], a["dv"], a["fl"], a.get("gp"),
                 err, None)
    assert call(prev=other_b) == g.GDN_ERR_ARG              # previous tree of another batch
    assert call(d=big) == g.GDN_ERR_UNSUPPORTED             # N > 32
    assert call(dk=64, dv=64) == g.GDN_ERR_UNSUPPORTED      # d != 128
    assert call(Lmax=65) == g.GDN_ERR_UNSUPPORTED
    assert call(act=2) == g.GDN_ERR_ARG
    assert call(fl=4) == g.GDN_ERR_ARG                      # only NORM_QK, OUT_BF16, RAW_GATES
    assert call(fl=1 | g.GDN_F_RAW_GATES) == g.GDN_ERR_ARG  # raw gates without parameters
    assert call(hout=None) == g.GDN_ERR_ARG
    assert call(hout=args["hin"]) == g.GDN_ERR_ARG          # history buffers overlap
    assert call(hout=ctypes.c_void_p((1 << 20) + hbytes - 16)) == g.GDN_ERR_ARG
    assert call(x=ctypes.c_void_p(264)) == g.GDN_ERR_ARG    # x not 16-byte aligned
    assert call(xp=None) == g.GDN_ERR_ARG
    assert call(pn=None) == g.GDN_ERR_ARG
    assert call(Hqk=3) == g.GDN_ERR_ARG


def test_attention_argument_checks_fail_before_launch(lib):
    err = ctypes.c_void_p(128)
    d = ctypes.byref(_desc(N=27, R=32))
    big_r = ctypes.byref(_desc(N=27, R=65))
    p = ctypes.c_void_p(256)
    W = lib.gdn_tree_attention_workspace_bytes
    assert W(2, 27, 16, 256, 8) == 9 * 2 * 16 * 27 * 258 * 4
    assert W(0, 27, 16, 256, 8) == 0
    A = lib.gdn_tree_attention
    ws = W(2, 27, 16, 256, 8)
    args = dict(d=d, q=p, k=p, v=p, S=4096, ctx=p, out=p, ws=p, wsb=ws, splits=8, Hq=16, Hkv=2, D=256,
                scale=0.0625, fl=0)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return A(a["d"], a["q"], a["k"], a["v"], a["S"], a["ctx"], a["out"], a["ws"], a["wsb"], a["splits"],
                 a["Hq"], a["Hkv"], a["D"], a["scale"], a["fl"], err, None)
    assert call(D=64) == g.GDN_ERR_UNSUPPORTED
    assert call(Hq=15) == g.GDN_ERR_ARG                      # Hq not a multiple of Hkv
    assert call(splits=0) == g.GDN_ERR_UNSUPPORTED
    assert call(wsb=ws - 4) == g.GDN_ERR_ARG                 # workspace too small
    assert call(S=31) == g.GDN_ERR_ARG                       # cache shorter than the candidates
    assert call(scale=0.0) == g.GDN_ERR_ARG
    assert call(scale=float("nan")) == g.GDN_ERR_ARG
    assert call(scale=float("inf")) == g.GDN_ERR_ARG
    assert call(scale=3.0e38) == g.GDN_ERR_ARG                 # scale * log2(e) overflows fp32
    assert call(fl=g.GDN_F_NORM_QK) == g.GDN_ERR_ARG
    assert call(d=big_r) == g.GDN_ERR_UNSUPPORTED            # R > 64
    assert call(k=ctypes.c_void_p(264)) == g.GDN_ERR_ARG     # not 16-byte aligned
    assert call(ctx=None) == g.GDN_ERR_ARG
    # the no-alloc variant: the same checks, and a request past its scratch
    Z = lib.gdn_tree_attention_noalloc

    def call_z(**kw):
        a = dict(args)
        a.update(kw)
        return Z(a["d"], a["q"], a["k"], a["v"], a["S"], a["ctx"], a["out"], a["splits"], a["Hq"], a["Hkv"],
                 a["D"], a["scale"], a["fl"], err, None)
    assert call_z(D=64) == g.GDN_ERR_UNSUPPORTED
    assert call_z(Hq=15) == g.GDN_ERR_ARG
    assert call_z(scale=0.0) == g.GDN_ERR_ARG
    assert call_z(scale=float("inf")) == g.GDN_ERR_ARG
    assert call_z(out=None) == g.GDN_ERR_ARG
    assert W(2, 27, 16, 256, 1024) > g.GDN_ATTN_NOALLOC_SCRATCH_BYTES
    assert call_z(splits=1024) == g.GDN_ERR_UNSUPPORTED       # partials past the scratch
    K = lib.gdn_tree_kv_publish
    assert K(d, p, p, 0, p, p, 4096, p, 2, 256, err, None) == g.GDN_ERR_UNSUPPORTED
    assert K(d, p, p, 8, p, p, 4096, p, 2, 64, err, None) == g.GDN_ERR_UNSUPPORTED
    assert K(d, p, None, 8, p, p, 4096, p, 2, 256, err, None) == g.GDN_ERR_ARG
    assert K(d, p, p, 8, p, p, 16, p, 2, 256, err, None) == g.GDN_ERR_ARG


def test_binding_refuses_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        g.load_library()
