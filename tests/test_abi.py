"""The C ABI without a GPU: the library loads, exports every function that
include/dit_attn.h declares, and rejects bad arguments on the host before
any HIP call (so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import diffusion_transformer_attention_amd as dta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dta.LIB_PATH):
        pytest.fail("libditattn.so not built: run __graft_entry__.build()")
    return dta.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(dta.EXPORTED)


def test_one_library_per_process(lib):
    assert dta.load_library() is lib
    assert dta.load_library(dta.LIB_PATH) is lib
    with pytest.raises(RuntimeError, match="already loaded"):
        dta.load_library(os.path.join(ROOT, "elsewhere", "libditattn.so"))


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert lib.dit_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert lib.dit_strerror(code)
    assert b"scratch" in lib.dit_strerror(dta.DIT_ESCRATCH)


V = ctypes.c_void_p
A = V(0x10000)       # 16-byte aligned stand-in address: never dereferenced here
MIS = V(0x10008)     # 8-byte aligned, not 16
NULL = V(0)
S = V(0)             # stream


def fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=2, N=64, D=128, scale=0.125, dt=0):
    return lib.dit_attn_fwd(q, k, v, o, lse, B, H, N, D, ctypes.c_float(scale), dt, S)


def blk(lib, Nq=64, Nkv=64, ind=0, od=1, lse=A, D=128, scale=0.125):
    return lib.dit_attn_fwd_block(A, A, A, A, lse, 1, 2, Nq, Nkv, D, ctypes.c_float(scale), ind, od, S)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), dta.DIT_EINVAL), (dict(k=NULL), dta.DIT_EINVAL), (dict(v=NULL), dta.DIT_EINVAL),
    (dict(o=NULL), dta.DIT_EINVAL), (dict(B=-1), dta.DIT_EINVAL), (dict(N=-5), dta.DIT_EINVAL),
    (dict(scale=0.0), dta.DIT_EINVAL), (dict(scale=-1.0), dta.DIT_EINVAL),
    (dict(scale=float("inf")), dta.DIT_EINVAL), (dict(scale=float("nan")), dta.DIT_EINVAL),
    (dict(D=96), dta.DIT_EUNSUPPORTED), (dict(D=256), dta.DIT_EUNSUPPORTED),
    (dict(D=0), dta.DIT_EINVAL), (dict(dt=2), dta.DIT_EUNSUPPORTED),
    (dict(q=MIS), dta.DIT_EALIGN), (dict(o=MIS), dta.DIT_EALIGN), (dict(lse=V(0x10002)), dta.DIT_EALIGN),
    (dict(B=0), dta.DIT_OK), (dict(H=0, q=NULL), dta.DIT_OK), (dict(N=0), dta.DIT_OK),
    (dict(B=1 << 30, H=1 << 30), dta.DIT_ERANGE),
])
def test_attn_fwd_validation(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_block_validation(lib):
    assert blk(lib, lse=NULL) == dta.DIT_EINVAL          # the ring partial needs its LSE
    assert blk(lib, Nkv=0) == dta.DIT_EINVAL             # empty key set
    assert blk(lib, ind=1, od=0) == dta.DIT_EUNSUPPORTED  # f32 in -> bf16 out not built
    assert blk(lib, Nq=0) == dta.DIT_OK                  # nothing to compute


def test_balanced_workspace_and_validation(lib):
    n = ctypes.c_size_t(7)
    size = lambda B=1, H=10, Nq=75600, Nkv=75600, D=128, slots=256: (
        lib.dit_attn_fwd_balanced_workspace(B, H, Nq, Nkv, D, slots, ctypes.byref(n)), n.value)
    assert size(Nq=32768, Nkv=32768) == (dta.DIT_OK, 0)   # 1280 tiles: five whole waves of 256
    rc, need = size()                                      # 2960 tiles: 11.56 waves, tail split
    assert rc == dta.DIT_OK and need > 0 and need % (4 * 129) == 0
    assert size(Nkv=64) == (dta.DIT_OK, 0)                 # one key tile: nothing to split
    assert size(Nq=0) == (dta.DIT_OK, 0)
    assert size(H=1 << 20, Nq=1 << 20, Nkv=128, D=32) == (dta.DIT_OK, 0)  # 2^32 tiles: no plan
    assert size(D=96)[0] == dta.DIT_EUNSUPPORTED
    assert size(slots=-1)[0] == dta.DIT_EINVAL
    assert size(Nkv=0)[0] == dta.DIT_EINVAL
    assert lib.dit_attn_fwd_balanced_workspace(1, 1, 64, 64, 128, 256, None) == dta.DIT_EINVAL
    bal = lambda ws=A, nb=need, o=A, od=0, Nq=75600, Nkv=75600, scale=0.125, slots=256: \
        lib.dit_attn_fwd_balanced(A, A, A, o, A, 1, 10, Nq, Nkv, 128, ctypes.c_float(scale), od,
                                  slots, ws, nb, S)
    assert bal(nb=need - 1) == dta.DIT_EINVAL              # workspace too small
    assert bal(ws=NULL) == dta.DIT_EINVAL
    assert bal(ws=MIS) == dta.DIT_EALIGN
    assert bal(o=NULL) == dta.DIT_EINVAL
    assert bal(od=5) == dta.DIT_EUNSUPPORTED
    assert bal(scale=0.0) == dta.DIT_EINVAL
    assert bal(Nkv=0) == dta.DIT_EINVAL
    assert bal(slots=-2) == dta.DIT_EINVAL
    assert bal(Nq=0, ws=NULL) == dta.DIT_OK                # nothing to compute


def test_balanced_noalloc_validation(lib):
    """The no-allocation balanced forward: argument errors as the workspace
    form, and a plan whose partials exceed the static scratch is refused on
    the host before any HIP call."""
    nb = lambda o=A, od=0, B=1, H=10, Nq=75600, Nkv=75600, scale=0.125, slots=256, lse=A: \
        lib.dit_attn_fwd_balanced_noalloc(A, A, A, o, lse, B, H, Nq, Nkv, 128, ctypes.c_float(scale),
                                          od, slots, S)
    assert nb(o=NULL) == dta.DIT_EINVAL
    assert nb(o=MIS) == dta.DIT_EALIGN
    assert nb(lse=V(0x10002)) == dta.DIT_EALIGN
    assert nb(od=5) == dta.DIT_EUNSUPPORTED
    assert nb(scale=float("nan")) == dta.DIT_EINVAL
    assert nb(Nkv=0) == dta.DIT_EINVAL
    assert nb(slots=-1) == dta.DIT_EINVAL
    assert nb(Nq=0, o=NULL) == dta.DIT_OK
    # 5120 tiles on 2048 slots: 1024 tail tiles in two key chunks, 270 MB of partials
    n = ctypes.c_size_t(0)
    assert lib.dit_attn_fwd_balanced_workspace(1, 40, 32768, 32768, 128, 2048, ctypes.byref(n)) == 0
    assert n.value > dta.DIT_SCRATCH_BYTES
    assert nb(H=40, Nq=32768, Nkv=32768, slots=2048) == dta.DIT_ESCRATCH
    # the long-video plan on 256 compute units fits the scratch
    assert lib.dit_attn_fwd_balanced_workspace(1, 10, 75600, 75600, 128, 256, ctypes.byref(n)) == 0
    assert 0 < n.value <= dta.DIT_SCRATCH_BYTES


def test_merge_validation(lib):
    m = lambda nblk=4, o=A, op=A, lp=A, D=128, od=0, N=64: lib.dit_attn_merge(
        op, lp, nblk, o, A, 1, 2, N, D, od, S)
    assert m(nblk=0) == dta.DIT_EINVAL
    assert m(op=NULL) == dta.DIT_EINVAL
    assert m(D=48) == dta.DIT_EUNSUPPORTED
    assert m(od=5) == dta.DIT_EUNSUPPORTED
    assert m(op=MIS) == dta.DIT_EALIGN
    assert m(N=0) == dta.DIT_OK


def test_fused_ulysses_validation(lib):
    u = lambda P=4, r=0, H=8, N=512, D=128, dt=0, q=A, o=A, lse=A, scale=0.125: \
        lib.dit_attn_fwd_ulysses(q, A, A, o, lse, P, r, 1, H, N, D, ctypes.c_float(scale), dt, S)
    assert u(r=4) == dta.DIT_EINVAL          # rank outside [0, P)
    assert u(r=-1) == dta.DIT_EINVAL
    assert u(P=0) == dta.DIT_EINVAL
    assert u(H=6) == dta.DIT_EINVAL          # heads not divisible by P
    assert u(N=514) == dta.DIT_EINVAL        # tokens not divisible by P
    assert u(N=4 * 48) == dta.DIT_EUNSUPPORTED  # shards shorter than a key tile and not whole tiles
    # ragged shards more than 2^31 bytes apart (the next shard out of 32-bit offset reach)
    assert u(H=4096, N=4 * 20001) == dta.DIT_EUNSUPPORTED
    assert u(dt=1) == dta.DIT_EUNSUPPORTED   # bf16 only
    assert u(D=80) == dta.DIT_EUNSUPPORTED
    assert u(scale=0.0) == dta.DIT_EINVAL
    assert u(q=NULL) == dta.DIT_EINVAL
    assert u(o=MIS) == dta.DIT_EALIGN
    assert u(lse=V(0x10002)) == dta.DIT_EALIGN
    assert u(N=0) == dta.DIT_OK              # nothing to compute


def test_backward_validation(lib):
    def b(B=1, Nq=64, Nkv=64, D=128, dt=0, gdt=1, q=A, lse=A, delta=A, dq=A, scale=0.125):
        return lib.dit_attn_bwd(q, A, A, A, A, lse, delta, dq, A, A, B, 2, Nq, Nkv, D,
                                ctypes.c_float(scale), dt, gdt, S)
    assert b(D=80) == dta.DIT_EUNSUPPORTED     # head dims 32, 64, 128 only
    assert b(D=256) == dta.DIT_EUNSUPPORTED
    assert b(dt=1) == dta.DIT_EUNSUPPORTED     # bf16 inputs only
    assert b(gdt=0) == dta.DIT_EUNSUPPORTED    # float32 gradients only
    assert b(Nq=0) == dta.DIT_EINVAL           # gradients of an empty problem are not a no-op
    assert b(Nkv=0) == dta.DIT_EINVAL
    assert b(B=0) == dta.DIT_OK
    assert b(q=NULL) == dta.DIT_EINVAL
    assert b(lse=NULL) == dta.DIT_EINVAL
    assert b(delta=NULL) == dta.DIT_EINVAL
    assert b(dq=MIS) == dta.DIT_EALIGN
    assert b(lse=V(0x10002)) == dta.DIT_EALIGN
    assert b(scale=float("nan")) == dta.DIT_EINVAL
    assert b(Nq=-1) == dta.DIT_EINVAL


def test_rope_pack_validation(lib):
    def r(xt=A, xi=A, ct=A, st=A, ci=A, si=A, out=A, B=1, H=2, Ht=8, h0=2, Nt=16, Ni=64, D=128):
        return lib.dit_rope_pack(xt, xi, ct, st, ci, si, out, B, H, Ht, h0, Nt, Ni, D, S)
    assert r(h0=7) == dta.DIT_EINVAL           # text heads 7, 8 past Ht = 8
    assert r(h0=-1) == dta.DIT_EINVAL
    assert r(Ht=1) == dta.DIT_EINVAL           # fewer text heads than the launch covers
    # no text (image): its pointer and heads are not looked at; the misaligned
    # output then fails the last check, so no call here reaches a launch
    assert r(Nt=0, Ht=0, h0=0, xt=NULL, out=MIS) == dta.DIT_EALIGN
    assert r(Ni=0, xi=NULL, out=MIS) == dta.DIT_EALIGN
    assert r(xt=NULL) == dta.DIT_EINVAL
    assert r(xi=NULL) == dta.DIT_EINVAL
    assert r(out=NULL) == dta.DIT_EINVAL
    assert r(ct=NULL) == dta.DIT_EINVAL        # cos without sin
    assert r(si=NULL) == dta.DIT_EINVAL
    assert r(ct=MIS) == dta.DIT_EALIGN
    assert r(xi=MIS) == dta.DIT_EALIGN
    assert r(out=MIS) == dta.DIT_EALIGN
    assert r(D=96) == dta.DIT_EUNSUPPORTED
    assert r(Nt=-1) == dta.DIT_EINVAL
    assert r(Nt=0, Ni=0) == dta.DIT_OK         # nothing to pack
    assert r(B=0) == dta.DIT_OK
    assert r(Nt=2 ** 30, Ni=2 ** 30) == dta.DIT_ERANGE


def test_joint_validation(lib):
    def j(q=A, ws=A, o=A, lse=A, ct=A, st=A, Ht=4, h0=0, Nt=16, Ni=64, D=128, scale=0.125):
        return lib.dit_attn_fwd_joint(q, A, A, q, A, A, ct, st, A, A, ws, o, lse, 1, 4, Ht, h0,
                                      Nt, Ni, D, ctypes.c_float(scale), S)
    assert j(ws=NULL) == dta.DIT_EINVAL
    assert j(o=NULL) == dta.DIT_EINVAL
    assert j(q=NULL) == dta.DIT_EINVAL
    assert j(ct=NULL) == dta.DIT_EINVAL
    assert j(ct=NULL, st=NULL, o=MIS) == dta.DIT_EALIGN
    assert j(ws=MIS) == dta.DIT_EALIGN
    assert j(lse=V(0x10002)) == dta.DIT_EALIGN
    assert j(scale=0.0) == dta.DIT_EINVAL
    assert j(h0=1) == dta.DIT_EINVAL           # heads 1..4 of a 4-head text tensor
    assert j(D=16) == dta.DIT_EUNSUPPORTED
    assert j(Nt=0, Ni=0) == dta.DIT_OK


def test_quant_fp8_validation(lib):
    def qz(x=A, c=A, ds=A, B=1, H=2, N=64, D=128):
        return lib.dit_quant_fp8(x, c, ds, B, H, N, D, S)
    assert qz(D=96) == dta.DIT_EUNSUPPORTED
    assert qz(ds=NULL) == dta.DIT_EINVAL
    assert qz(x=NULL) == dta.DIT_EINVAL
    assert qz(c=NULL) == dta.DIT_EINVAL
    assert qz(c=V(0x10004)) == dta.DIT_EALIGN    # codes need 8-byte alignment
    assert qz(x=MIS) == dta.DIT_EALIGN
    assert qz(ds=V(0x10002)) == dta.DIT_EALIGN
    assert qz(N=-1) == dta.DIT_EINVAL
    assert qz(B=0) == dta.DIT_OK
    assert qz(B=2 ** 20, H=2 ** 12, N=1, D=32) == dta.DIT_ERANGE


def test_quant_fp8_qk_validation(lib):
    def qk(q=A, k=A, qc=A, kc=A, qd=A, kd=A, B=1, H=2, Nq=64, Nkv=32, D=128):
        return lib.dit_quant_fp8_qk(q, k, qc, kc, qd, kd, B, H, Nq, Nkv, D, S)
    assert qk(D=96) == dta.DIT_EUNSUPPORTED
    assert qk(qd=NULL) == dta.DIT_EINVAL
    assert qk(kd=NULL) == dta.DIT_EINVAL
    assert qk(k=NULL) == dta.DIT_EINVAL
    assert qk(qc=NULL) == dta.DIT_EINVAL
    assert qk(kc=V(0x10004)) == dta.DIT_EALIGN
    assert qk(q=MIS) == dta.DIT_EALIGN
    assert qk(kd=V(0x10002)) == dta.DIT_EALIGN
    assert qk(Nkv=-1) == dta.DIT_EINVAL
    assert qk(B=0) == dta.DIT_OK
    assert qk(B=2 ** 20, H=2 ** 12, Nq=1, Nkv=1, D=32) == dta.DIT_ERANGE


def test_attn_fp8_validation(lib):
    def f(q=A, qd=A, kd=A, o=A, lse=A, Nq=64, Nkv=64, D=128, scale=0.125, od=0):
        return lib.dit_attn_fwd_fp8(q, A, A, qd, kd, o, lse, 1, 2, Nq, Nkv, D,
                                    ctypes.c_float(scale), od, S)
    assert f(D=64) == dta.DIT_EUNSUPPORTED
    assert f(od=5) == dta.DIT_EUNSUPPORTED
    assert f(qd=NULL) == dta.DIT_EINVAL
    assert f(kd=NULL) == dta.DIT_EINVAL
    assert f(Nkv=0) == dta.DIT_EINVAL
    assert f(scale=-1.0) == dta.DIT_EINVAL
    assert f(q=MIS) == dta.DIT_EALIGN
    assert f(kd=V(0x10002)) == dta.DIT_EALIGN
    assert f(lse=V(0x10002)) == dta.DIT_EALIGN
    assert f(Nq=0) == dta.DIT_OK


def test_quant_fp8_qk_mx_validation(lib):
    def qk(q=A, k=A, qc=A, kc=A, qd=A, kd=A, B=1, H=2, Nq=64, Nkv=32, D=128, scale=0.125):
        return lib.dit_quant_fp8_qk_mx(q, k, qc, kc, qd, kd, B, H, Nq, Nkv, D,
                                       ctypes.c_float(scale), S)
    assert qk(D=96) == dta.DIT_EUNSUPPORTED
    assert qk(scale=0.0) == dta.DIT_EINVAL
    assert qk(scale=float("inf")) == dta.DIT_EINVAL
    assert qk(qd=NULL) == dta.DIT_EINVAL
    assert qk(k=NULL) == dta.DIT_EINVAL
    assert qk(kc=V(0x10004)) == dta.DIT_EALIGN
    assert qk(q=MIS) == dta.DIT_EALIGN
    assert qk(Nkv=-1) == dta.DIT_EINVAL
    assert qk(B=0) == dta.DIT_OK
    assert qk(B=2 ** 20, H=2 ** 12, Nq=1, Nkv=1, D=32) == dta.DIT_ERANGE


def test_attn_fp8_mx_validation(lib):
    def f(q=A, qd=A, kd=A, o=A, lse=A, Nq=64, Nkv=64, D=128, od=0):
        return lib.dit_attn_fwd_fp8_mx(q, A, A, qd, kd, o, lse, 1, 2, Nq, Nkv, D, od, S)
    assert f(D=64) == dta.DIT_EUNSUPPORTED
    assert f(od=5) == dta.DIT_EUNSUPPORTED
    assert f(qd=NULL) == dta.DIT_EINVAL
    assert f(Nkv=0) == dta.DIT_EINVAL
    assert f(q=MIS) == dta.DIT_EALIGN
    assert f(kd=V(0x10002)) == dta.DIT_EALIGN
    assert f(Nq=0) == dta.DIT_OK


@pytest.mark.parametrize("fn", ["ulysses_seq2head", "ulysses_head2seq"])
def test_permute_validation(lib, fn):
    f = getattr(lib, fn)
    call = lambda P=4, H=8, N=64, eb=2, i=A, o=A: f(i, o, P, 1, H, N, 32, eb, S)
    assert call(H=6) == dta.DIT_EINVAL        # heads not divisible by P
    assert call(N=66) == dta.DIT_EINVAL       # tokens not divisible by P
    assert call(P=0) == dta.DIT_EINVAL
    assert call(eb=3) == dta.DIT_EUNSUPPORTED
    assert call(i=NULL) == dta.DIT_EINVAL
    assert call(eb=4, i=V(0x10002)) == dta.DIT_EALIGN
    assert call(N=0) == dta.DIT_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        dta.dit_attn_fwd(x, x, x)
