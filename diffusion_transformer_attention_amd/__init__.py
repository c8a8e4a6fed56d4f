"""MI355X-native attention hot path of Ulysses / Ring sequence parallelism.

Thin ctypes binding over libditattn.so (C ABI in include/dit_attn.h).  The
functions carry the C entry points' names and take torch tensors on the
current HIP device; they only check shapes, dtypes and contiguity, pass data
pointers and the current stream, and raise on a non-zero return.  Every step
of the computation runs in the library's HIP kernels: there is no fallback,
and importing the binding fails loudly if the library has not been built
(``python -m diffusion_transformer_attention_amd.build``).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libditattn.so")

DIT_BF16, DIT_F32 = 0, 1
DIT_OK, DIT_EINVAL, DIT_EUNSUPPORTED, DIT_EALIGN, DIT_ELAUNCH, DIT_ERANGE = 0, -1, -2, -3, -4, -5
DIT_ESCRATCH = -6
DIT_SCRATCH_BYTES = 160 << 20   # static device scratch behind dit_attn_fwd_balanced_noalloc
EXPORTED = ("dit_attn_fwd", "dit_attn_fwd_block", "dit_attn_fwd_balanced",
            "dit_attn_fwd_balanced_workspace", "dit_attn_fwd_balanced_noalloc",
            "dit_attn_fwd_ulysses", "dit_attn_bwd",
            "dit_attn_merge", "dit_rope_pack", "dit_attn_fwd_joint", "dit_quant_fp8",
            "dit_quant_fp8_qk", "dit_attn_fwd_fp8", "dit_quant_fp8_qk_mx", "dit_attn_fwd_fp8_mx",
            "ulysses_seq2head", "ulysses_head2seq", "dit_strerror", "dit_abi_version")

_lib = None
_lib_path = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libditattn.so (the in-tree build unless `path` names another) and
    declare its prototypes (no device call is made).

    One library per process: without a path, the one already loaded is
    returned; a later call naming another path raises."""
    global _lib, _lib_path
    if _lib is not None:
        if path is not None and os.path.realpath(path) != _lib_path:
            raise RuntimeError(f"{_lib_path} is already loaded; cannot switch to {path}")
        return _lib
    path = LIB_PATH if path is None else path
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m diffusion_transformer_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.dit_attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P]
    lib.dit_attn_fwd_block.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.dit_attn_fwd_ulysses.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P]
    lib.dit_attn_fwd_balanced.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, P,
                                          ctypes.c_size_t, P]
    lib.dit_attn_fwd_balanced_workspace.argtypes = [I, I, I, I, I, I,
                                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.dit_attn_fwd_balanced_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.dit_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.dit_attn_merge.argtypes = [P, P, I, P, P, I, I, I, I, I, P]
    lib.dit_quant_fp8.argtypes = [P, P, P, I, I, I, I, P]
    lib.dit_quant_fp8_qk.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
    lib.dit_attn_fwd_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.dit_quant_fp8_qk_mx.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, P]
    lib.dit_attn_fwd_fp8_mx.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.dit_rope_pack.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.dit_attn_fwd_joint.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P,
                                       I, I, I, I, I, I, I, F, P]
    lib.ulysses_seq2head.argtypes = [P, P, I, I, I, I, I, I, P]
    lib.ulysses_head2seq.argtypes = [P, P, I, I, I, I, I, I, P]
    for name in ("dit_attn_fwd", "dit_attn_fwd_block", "dit_attn_fwd_balanced",
                 "dit_attn_fwd_balanced_workspace", "dit_attn_fwd_balanced_noalloc",
                 "dit_attn_fwd_ulysses", "dit_attn_bwd",
                 "dit_attn_merge", "dit_rope_pack", "dit_attn_fwd_joint", "dit_quant_fp8",
                 "dit_quant_fp8_qk", "dit_attn_fwd_fp8", "dit_quant_fp8_qk_mx", "dit_attn_fwd_fp8_mx",
                 "ulysses_seq2head", "ulysses_head2seq", "dit_abi_version"):
        getattr(lib, name).restype = ctypes.c_int
    lib.dit_strerror.argtypes = [ctypes.c_int]
    lib.dit_strerror.restype = ctypes.c_char_p
    lib.dit_abi_version.argtypes = []
    _lib, _lib_path = lib, os.path.realpath(path)
    return lib


def dit_strerror(code: int) -> str:
    return load_library().dit_strerror(int(code)).decode()


def dit_abi_version() -> int:
    return load_library().dit_abi_version()


class DitError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {dit_strerror(code)} (code {code})")
        self.code = code


def _check(rc: int, where: str):
    if rc != DIT_OK:
        raise DitError(rc, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return DIT_BF16
    if dt == torch.float32:
        return DIT_F32
    raise TypeError(f"unsupported dtype {dt}")


def _need(t, name, dims):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def dit_attn_fwd(q, k, v, scale=None, out=None, lse=None, return_lse=True):
    """Attention over all N tokens of each (b, h): q, k, v [B,H,N,D] (bf16 or f32).

    Returns (O [B,H,N,D] in the input dtype, LSE float32 [B,H,N] or None).
    """
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", 4)
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be float32 [B,H,N]")
    rc = lib.dit_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D,
                          ctypes.c_float(scale), _dtype_code(q.dtype), _stream())
    _check(rc, "dit_attn_fwd")
    return o, lse


def dit_attn_fwd_block(q, k, v, scale=None, out_dtype=torch.float32, out=None, lse=None):
    """One Ring step: q [B,H,Nq,D] against one K/V block k, v [B,H,Nkv,D].

    Returns (O [B,H,Nq,D] in out_dtype, LSE float32 [B,H,Nq]).
    """
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != D:
        raise ValueError("k, v must be [B,H,Nkv,D] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share dtype")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, D), device=q.device, dtype=out_dtype) if out is None else out
    _need(o, "out", 4)
    if lse is None:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    _need(lse, "lse", 3)
    rc = lib.dit_attn_fwd_block(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nkv, D,
                                ctypes.c_float(scale), _dtype_code(q.dtype),
                                _dtype_code(o.dtype), _stream())
    _check(rc, "dit_attn_fwd_block")
    return o, lse


def dit_attn_fwd_balanced_workspace(B, H, Nq, Nkv, D, slots=0):
    """Workspace bytes dit_attn_fwd_balanced needs (0: no split for these sizes)."""
    n = ctypes.c_size_t(0)
    _check(load_library().dit_attn_fwd_balanced_workspace(B, H, Nq, Nkv, D, int(slots),
                                                         ctypes.byref(n)),
           "dit_attn_fwd_balanced_workspace")
    return int(n.value)


def dit_attn_fwd_balanced(q, k, v, scale=None, out_dtype=torch.bfloat16, out=None, lse=None,
                          return_lse=True, slots=0, workspace=None):
    """Work-balanced forward of bf16 q [B,H,Nq,D] against k, v [B,H,Nkv,D].

    ``workspace``: a uint8 device tensor of at least
    dit_attn_fwd_balanced_workspace(...) bytes, allocated here when None.
    Returns (O [B,H,Nq,D] in out_dtype, LSE float32 [B,H,Nq] or None).
    """
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != D:
        raise ValueError("k, v must be [B,H,Nkv,D] matching q")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("q, k, v must be bf16")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, D), device=q.device, dtype=out_dtype) if out is None else out
    _need(o, "out", 4)
    if tuple(o.shape) != (B, H, Nq, D):
        raise ValueError("out must be [B,H,Nq,D]")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be float32 [B,H,Nq]")
    if workspace is None:
        nbytes = dit_attn_fwd_balanced_workspace(B, H, Nq, Nkv, D, slots)
        workspace = torch.empty((max(nbytes, 1),), device=q.device, dtype=torch.uint8)
    _need(workspace, "workspace", 1)
    rc = lib.dit_attn_fwd_balanced(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nkv,
                                   D, ctypes.c_float(scale), _dtype_code(o.dtype), int(slots),
                                   _ptr(workspace),
                                   ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                   _stream())
    _check(rc, "dit_attn_fwd_balanced")
    return o, lse


def dit_attn_fwd_balanced_noalloc(q, k, v, out, lse=None, scale=None, slots=0):
    """dit_attn_fwd_balanced with the library's static device scratch instead
    of a workspace: the caller passes the outputs ``out`` ([B,H,Nq,D], bf16 or
    float32) and ``lse`` (float32 [B,H,Nq] or None) and nothing is allocated.
    Raises DitError (DIT_ESCRATCH) when the plan needs more than
    DIT_SCRATCH_BYTES.  Returns (out, lse)."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != D:
        raise ValueError("k, v must be [B,H,Nkv,D] matching q")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("q, k, v must be bf16")
    if tuple(out.shape) != (B, H, Nq, D):
        raise ValueError("out must be [B,H,Nq,D]")
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be float32 [B,H,Nq]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = lib.dit_attn_fwd_balanced_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq,
                                           Nkv, D, ctypes.c_float(scale), _dtype_code(out.dtype),
                                           int(slots), _stream())
    _check(rc, "dit_attn_fwd_balanced_noalloc")
    return out, lse


def dit_attn_fwd_ulysses(q, k, v, r, scale=None, out=None, lse=None, return_lse=True):
    """Attention of Ulysses head group r read from / written to token shards.

    q, k, v: bf16 [P,B,H,N/P,D] token shards.  Writes heads [r*H/P, (r+1)*H/P)
    of every shard of `out` (allocated as zeros when None) and returns
    (out [P,B,H,N/P,D], LSE float32 [B,H/P,N] or None).
    """
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 5)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    P, B, H, Ns, D = q.shape
    if P == 0 or H % P:
        raise ValueError("H must be divisible by P")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.zeros_like(q) if out is None else out
    _need(o, "out", 5)
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, H // P, Ns * P), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H // P, Ns * P):
            raise ValueError("lse must be float32 [B,H/P,N]")
    rc = lib.dit_attn_fwd_ulysses(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), P, int(r), B, H,
                                  Ns * P, D, ctypes.c_float(scale), _dtype_code(q.dtype),
                                  _stream())
    _check(rc, "dit_attn_fwd_ulysses")
    return o, lse


def dit_attn_bwd(q, k, v, o, dout, lse, scale=None, dq=None, dk=None, dv=None, delta=None):
    """Attention backward: q, o, dout bf16 [B,H,Nq,D]; k, v bf16 [B,H,Nkv,D] (D = 32,
    64 or 128); lse float32 [B,H,Nq] from the forward.

    Returns (dq [B,H,Nq,D], dk, dv [B,H,Nkv,D], delta [B,H,Nq]), all float32.
    """
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, 4)
    _need(lse, "lse", 3)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must match q")
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != D:
        raise ValueError("k, v must be [B,H,Nkv,D] matching q")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise ValueError("q, k, v, o, dout must share dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be float32 [B,H,Nq]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    f32 = dict(device=q.device, dtype=torch.float32)
    dq = torch.empty((B, H, Nq, D), **f32) if dq is None else dq
    dk = torch.empty((B, H, Nkv, D), **f32) if dk is None else dk
    dv = torch.empty((B, H, Nkv, D), **f32) if dv is None else dv
    delta = torch.empty((B, H, Nq), **f32) if delta is None else delta
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, 4)
    _need(delta, "delta", 3)
    rc = lib.dit_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta),
                          _ptr(dq), _ptr(dk), _ptr(dv), B, H, Nq, Nkv, D, ctypes.c_float(scale),
                          _dtype_code(q.dtype), _dtype_code(dq.dtype), _stream())
    _check(rc, "dit_attn_bwd")
    return dq, dk, dv, delta


def dit_attn_merge(o_parts, lse_parts, out_dtype=torch.bfloat16, out=None, lse=None,
                   return_lse=True):
    """Exact LSE merge: o_parts float32 [nblk,B,H,N,D], lse_parts float32 [nblk,B,H,N].

    Returns (O [B,H,N,D] in out_dtype, LSE float32 [B,H,N] or None).
    """
    lib = load_library()
    _need(o_parts, "o_parts", 5)
    _need(lse_parts, "lse_parts", 4)
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("partials must be float32")
    nblk, B, H, N, D = o_parts.shape
    if tuple(lse_parts.shape) != (nblk, B, H, N):
        raise ValueError("lse_parts must be [nblk,B,H,N]")
    o = torch.empty((B, H, N, D), device=o_parts.device, dtype=out_dtype) if out is None else out
    _need(o, "out", 4)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), device=o_parts.device, dtype=torch.float32)
    rc = lib.dit_attn_merge(_ptr(o_parts), _ptr(lse_parts), nblk, _ptr(o), _ptr(lse), B, H, N, D,
                            _dtype_code(o.dtype), _stream())
    _check(rc, "dit_attn_merge")
    return o, lse


def _joint_shapes(x_txt, x_img, h0):
    _need(x_txt, "text tensor", 4)
    _need(x_img, "image tensor", 4)
    if x_txt.dtype != torch.bfloat16 or x_img.dtype != torch.bfloat16:
        raise ValueError("text and image tensors must be bf16")
    B, Ht, Nt, D = x_txt.shape
    Bi, H, Ni, Di = x_img.shape
    if B != Bi or D != Di:
        raise ValueError("text [B,Ht,Nt,D] and image [B,H,Ni,D] must share B and D")
    if Nt and not (0 <= h0 and h0 + H <= Ht):
        raise ValueError("text heads h0 .. h0+H-1 must lie in [0, Ht)")
    return B, H, Ht, Nt, Ni, D


def _tables(c, s, n, half, what):
    if (c is None) != (s is None):
        raise ValueError(f"{what}: give both cos and sin tables or neither")
    for t, name in ((c, "cos"), (s, "sin")):
        if t is not None:
            _need(t, f"{what} {name}", 2)
            if t.dtype != torch.float32 or tuple(t.shape) != (n, half):
                raise ValueError(f"{what} {name} must be float32 [{n}, {half}]")


def dit_rope_pack(x_txt, x_img, cos_txt=None, sin_txt=None, cos_img=None, sin_img=None, h0=0,
                  out=None):
    """Joint sequence of one tensor: text bf16 [B,Ht,Nt,D] (heads h0 .. h0+H-1
    used) then image bf16 [B,H,Ni,D], each part turned by its rotary tables
    (float32 [N, D/2]) when given.  Returns out bf16 [B,H,Nt+Ni,D]."""
    lib = load_library()
    B, H, Ht, Nt, Ni, D = _joint_shapes(x_txt, x_img, h0)
    _tables(cos_txt, sin_txt, Nt, D // 2, "text")
    _tables(cos_img, sin_img, Ni, D // 2, "image")
    o = torch.empty((B, H, Nt + Ni, D), device=x_img.device, dtype=torch.bfloat16) \
        if out is None else out
    _need(o, "out", 4)
    if tuple(o.shape) != (B, H, Nt + Ni, D) or o.dtype != torch.bfloat16:
        raise ValueError("out must be bf16 [B,H,Nt+Ni,D]")
    rc = lib.dit_rope_pack(_ptr(x_txt), _ptr(x_img), _ptr(cos_txt), _ptr(sin_txt), _ptr(cos_img),
                           _ptr(sin_img), _ptr(o), B, H, Ht, int(h0), Nt, Ni, D, _stream())
    _check(rc, "dit_rope_pack")
    return o


def dit_attn_fwd_joint(q_txt, k_txt, v_txt, q_img, k_img, v_img, cos_txt=None, sin_txt=None,
                       cos_img=None, sin_img=None, h0=0, scale=None, workspace=None, out=None,
                       lse=None, return_lse=True):
    """Joint text + image attention with RoPE on q and k.

    Text q/k/v bf16 [B,Ht,Nt,D] (heads h0 .. h0+H-1 used), image q/k/v bf16
    [B,H,Ni,D], rotary tables float32 [Nt, D/2] / [Ni, D/2] or None.  Returns
    (O bf16 [B,H,Nt+Ni,D] with the text rows first, LSE float32 [B,H,Nt+Ni]
    or None).  ``workspace`` (bf16 [3,B,H,Nt+Ni,D]) is allocated when None.
    """
    lib = load_library()
    B, H, Ht, Nt, Ni, D = _joint_shapes(q_txt, q_img, h0)
    for t, r in ((k_txt, q_txt), (v_txt, q_txt), (k_img, q_img), (v_img, q_img)):
        _need(t, "k/v", 4)
        if t.shape != r.shape or t.dtype != r.dtype:
            raise ValueError("text (image) q, k, v must share shape and dtype")
    _tables(cos_txt, sin_txt, Nt, D // 2, "text")
    _tables(cos_img, sin_img, Ni, D // 2, "image")
    N = Nt + Ni
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q_img.device
    ws = torch.empty((3, B, H, N, D), device=dev, dtype=torch.bfloat16) \
        if workspace is None else workspace
    _need(ws, "workspace", 5)
    if tuple(ws.shape) != (3, B, H, N, D) or ws.dtype != torch.bfloat16:
        raise ValueError("workspace must be bf16 [3,B,H,Nt+Ni,D]")
    o = torch.empty((B, H, N, D), device=dev, dtype=torch.bfloat16) if out is None else out
    _need(o, "out", 4)
    if tuple(o.shape) != (B, H, N, D) or o.dtype != torch.bfloat16:
        raise ValueError("out must be bf16 [B,H,Nt+Ni,D]")
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be float32 [B,H,Nt+Ni]")
    rc = lib.dit_attn_fwd_joint(_ptr(q_txt), _ptr(k_txt), _ptr(v_txt), _ptr(q_img), _ptr(k_img),
                                _ptr(v_img), _ptr(cos_txt), _ptr(sin_txt), _ptr(cos_img),
                                _ptr(sin_img), _ptr(ws), _ptr(o), _ptr(lse), B, H, Ht, int(h0),
                                Nt, Ni, D, ctypes.c_float(scale), _stream())
    _check(rc, "dit_attn_fwd_joint")
    return o, lse


def _codes(t, name):
    _need(t, name, 4)
    if t.element_size() != 1 or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")


def dit_quant_fp8(x, codes=None, descale=None):
    """Per-(b, h) E4M3 quantization of bf16 x [B,H,N,D].

    Returns (codes uint8 [B,H,N,D], descale float32 [B,H]) with
    x ~= decode(codes) * descale[b, h].
    """
    lib = load_library()
    _need(x, "x", 4)
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    B, H, N, D = x.shape
    c = torch.empty((B, H, N, D), device=x.device, dtype=torch.uint8) if codes is None else codes
    _codes(c, "codes")
    if tuple(c.shape) != (B, H, N, D):
        raise ValueError("codes must match x")
    ds = torch.empty((B, H), device=x.device, dtype=torch.float32) if descale is None else descale
    _need(ds, "descale", 2)
    if ds.dtype != torch.float32 or tuple(ds.shape) != (B, H):
        raise ValueError("descale must be float32 [B,H]")
    rc = lib.dit_quant_fp8(_ptr(x), _ptr(c), _ptr(ds), B, H, N, D, _stream())
    _check(rc, "dit_quant_fp8")
    return c, ds


def _quant_qk_outputs(q, k, q_codes, k_codes, q_descale, k_descale):
    """Shape checks and outputs of the paired quantizers."""
    for t, n in ((q, "q"), (k, "k")):
        _need(t, n, 4)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
    B, H, Nq, D = q.shape
    if k.shape[:2] != q.shape[:2] or k.shape[3] != D:
        raise ValueError("k must be [B,H,Nkv,D] matching q")
    Nkv = k.shape[2]
    out = []
    for c, x, n in ((q_codes, q, "q_codes"), (k_codes, k, "k_codes")):
        c = torch.empty(x.shape, device=x.device, dtype=torch.uint8) if c is None else c
        _codes(c, n)
        if c.shape != x.shape:
            raise ValueError(f"{n} must match its input")
        out.append(c)
    ds = []
    for d, n in ((q_descale, "q_descale"), (k_descale, "k_descale")):
        d = torch.empty((B, H), device=q.device, dtype=torch.float32) if d is None else d
        _need(d, n, 2)
        if d.dtype != torch.float32 or tuple(d.shape) != (B, H):
            raise ValueError(f"{n} must be float32 [B,H]")
        ds.append(d)
    return (B, H, Nq, Nkv, D), out, ds


def dit_quant_fp8_qk(q, k, q_codes=None, k_codes=None, q_descale=None, k_descale=None):
    """dit_quant_fp8 of q [B,H,Nq,D] and k [B,H,Nkv,D] (bf16) in one call.

    Returns (q_codes, k_codes, q_descale, k_descale).
    """
    lib = load_library()
    (B, H, Nq, Nkv, D), out, ds = _quant_qk_outputs(q, k, q_codes, k_codes, q_descale, k_descale)
    rc = lib.dit_quant_fp8_qk(_ptr(q), _ptr(k), _ptr(out[0]), _ptr(out[1]), _ptr(ds[0]), _ptr(ds[1]),
                              B, H, Nq, Nkv, D, _stream())
    _check(rc, "dit_quant_fp8_qk")
    return out[0], out[1], ds[0], ds[1]


def dit_quant_fp8_qk_mx(q, k, scale=None, q_codes=None, k_codes=None, q_descale=None,
                        k_descale=None):
    """q [B,H,Nq,D] and k [B,H,Nkv,D] (bf16) to E4M3 codes with power-of-two
    descales, q first multiplied by scale * log2(e) (scale defaults to
    1/sqrt(D)), for dit_attn_fwd_fp8_mx.

    Returns (q_codes, k_codes, q_descale, k_descale).
    """
    lib = load_library()
    (B, H, Nq, Nkv, D), out, ds = _quant_qk_outputs(q, k, q_codes, k_codes, q_descale, k_descale)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = lib.dit_quant_fp8_qk_mx(_ptr(q), _ptr(k), _ptr(out[0]), _ptr(out[1]), _ptr(ds[0]),
                                 _ptr(ds[1]), B, H, Nq, Nkv, D, ctypes.c_float(scale), _stream())
    _check(rc, "dit_quant_fp8_qk_mx")
    return out[0], out[1], ds[0], ds[1]


def dit_attn_fwd_fp8(q, k, v, q_descale, k_descale, scale=None, out_dtype=torch.bfloat16,
                     out=None, lse=None, return_lse=True):
    """Attention with E4M3 q [B,H,Nq,128] and k [B,H,Nkv,128] (codes, with
    float32 [B,H] descales) and bf16 v [B,H,Nkv,128].

    Returns (O [B,H,Nq,D] in out_dtype, LSE float32 [B,H,Nq] or None).
    """
    lib = load_library()
    _codes(q, "q")
    _codes(k, "k")
    _need(v, "v", 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if k.shape[:2] != q.shape[:2] or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k, v must be [B,H,Nkv,D] matching q")
    if v.dtype != torch.bfloat16:
        raise ValueError("v must be bf16")
    for t, n in ((q_descale, "q_descale"), (k_descale, "k_descale")):
        _need(t, n, 2)
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H):
            raise ValueError(f"{n} must be float32 [B,H]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, D), device=q.device, dtype=out_dtype) if out is None else out
    _need(o, "out", 4)
    if tuple(o.shape) != (B, H, Nq, D):
        raise ValueError("out must be [B,H,Nq,D]")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be float32 [B,H,Nq]")
    rc = lib.dit_attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(o),
                              _ptr(lse), B, H, Nq, Nkv, D, ctypes.c_float(scale),
                              _dtype_code(o.dtype), _stream())
    _check(rc, "dit_attn_fwd_fp8")
    return o, lse


def dit_attn_fwd_fp8_mx(q, k, v, q_descale, k_descale, out_dtype=torch.bfloat16, out=None,
                        lse=None, return_lse=True):
    """Attention of codes from dit_quant_fp8_qk_mx (q [B,H,Nq,128], k
    [B,H,Nkv,128], power-of-two float32 [B,H] descales; the softmax scale is
    in the query codes) and bf16 v [B,H,Nkv,128]: base-2 scores
    q_descale * k_descale * (q . k).

    Returns (O [B,H,Nq,D] in out_dtype, LSE float32 [B,H,Nq] (natural log) or None).
    """
    lib = load_library()
    _codes(q, "q")
    _codes(k, "k")
    _need(v, "v", 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if k.shape[:2] != q.shape[:2] or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k, v must be [B,H,Nkv,D] matching q")
    if v.dtype != torch.bfloat16:
        raise ValueError("v must be bf16")
    for t, n in ((q_descale, "q_descale"), (k_descale, "k_descale")):
        _need(t, n, 2)
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H):
            raise ValueError(f"{n} must be float32 [B,H]")
    o = torch.empty((B, H, Nq, D), device=q.device, dtype=out_dtype) if out is None else out
    _need(o, "out", 4)
    if tuple(o.shape) != (B, H, Nq, D):
        raise ValueError("out must be [B,H,Nq,D]")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", 3)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be float32 [B,H,Nq]")
    rc = lib.dit_attn_fwd_fp8_mx(_ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale),
                                 _ptr(o), _ptr(lse), B, H, Nq, Nkv, D, _dtype_code(o.dtype),
                                 _stream())
    _check(rc, "dit_attn_fwd_fp8_mx")
    return o, lse


def ulysses_seq2head(shards, out=None):
    """[P,B,H,N/P,D] token shards -> [P,B,H/P,N,D] head groups (bit-exact, any dtype)."""
    lib = load_library()
    _need(shards, "shards", 5)
    P, B, H, Ns, D = shards.shape
    if P == 0 or H % P:
        raise ValueError("H must be divisible by P")
    o = torch.empty((P, B, H // P, Ns * P, D), device=shards.device, dtype=shards.dtype) \
        if out is None else out
    _need(o, "out", 5)
    rc = lib.ulysses_seq2head(_ptr(shards), _ptr(o), P, B, H, Ns * P, D, shards.element_size(),
                              _stream())
    _check(rc, "ulysses_seq2head")
    return o


def ulysses_head2seq(groups, out=None):
    """[P,B,H/P,N,D] head groups -> [P,B,H,N/P,D] token shards (bit-exact, any dtype)."""
    lib = load_library()
    _need(groups, "groups", 5)
    P, B, g, N, D = groups.shape
    if P == 0 or N % P:
        raise ValueError("N must be divisible by P")
    o = torch.empty((P, B, g * P, N // P, D), device=groups.device, dtype=groups.dtype) \
        if out is None else out
    _need(o, "out", 5)
    rc = lib.ulysses_head2seq(_ptr(groups), _ptr(o), P, B, g * P, N, D, groups.element_size(),
                              _stream())
    _check(rc, "ulysses_head2seq")
    return o


__all__ = ["dit_attn_fwd", "dit_attn_fwd_block", "dit_attn_fwd_ulysses", "dit_attn_bwd",
           "dit_attn_merge", "dit_rope_pack", "dit_attn_fwd_joint", "dit_quant_fp8",
           "dit_attn_fwd_fp8", "ulysses_seq2head",
           "ulysses_head2seq", "dit_strerror", "dit_abi_version", "load_library", "DitError",
           "LIB_PATH", "EXPORTED", "DIT_BF16", "DIT_F32"]
