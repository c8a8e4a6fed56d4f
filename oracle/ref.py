"""Plain CPU oracle for one GPU's share of DiT sequence-parallel attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py use it.  It shares no code with the HIP
library or its Python binding.

Everything is float64 numpy on the exact input values (bf16 inputs are
widened exactly; fp32 inputs likewise).  It is written to be checked by eye,
not to be fast: each function is the plain definition of what the hot path
computes, with no fusion or reordering beyond what that definition states.

Sources (web pages; sections named, not quoted):
* "Multi-GPU parallelism: spreading one step over several cards" (AI infra
  handbook), section "Sequence parallelism: Ulysses and Ring": Ulysses cuts
  the tokens into one slice per card and trades slices for head groups
  before attention and back after it; Ring runs local attention on each
  K/V block and merges the blocks with a log-sum-exp.
* "Feat: USP sequence parallelism (Ulysses x Ring) via SequenceParallelPlan"
  (miles_diffusion pull request), Design / "Ring kernel selection": ring
  kernels must return the LSE; "Limitations": no mask, dropout, causal flag
  or explicit scale under SP, head count divisible by the Ulysses degree,
  sequence length divisible by the SP degree.
* "Parallelism Acceleration Guide" (vLLM-Omni docs), "How to parallelize a
  new model": joint attention over concatenated text and image tokens, text
  replicated on every sequence-parallel rank, image rotary tables cut along
  the token axis.

Readings where the pages are silent:
* LSE is the natural log of sum_j exp(scale * q.k_j) (the scale included).
* Default scale is 1/sqrt(D), the scaled_dot_product_attention default the
  simulation relies on.
* Merge: blocks whose LSE is -inf get weight 0; if every block is -inf the
  result is O = 0, LSE = -inf (cannot happen without a mask).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


# --------------------------------------------------------------------------
# Attention (handbook, "Sequence parallelism: Ulysses and Ring": every card
# runs full, non-causal scaled-dot-product attention over its heads).
# --------------------------------------------------------------------------
def attention(q, k, v, scale=None, row_block=256):
    """softmax(scale * Q K^T) V and its per-row log-sum-exp.

    q: [B,H,Nq,D], k and v: [B,H,Nkv,D].  Returns (O [B,H,Nq,D] float64,
    LSE [B,H,Nq] float64).  For each row: S = scale * q K^T, m = max S,
    E = exp(S - m), l = sum E, O = (E V) / l, LSE = m + ln l.  Rows are
    independent; they are taken ``row_block`` at a time only to bound memory.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, D = q.shape
    scale = default_scale(D) if scale is None else float(scale)
    O = np.empty((B, H, Nq, v.shape[-1]), dtype=np.float64)
    L = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                S = scale * (q[b, h, r0:r1] @ k[b, h].T)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                O[b, h, r0:r1] = (E @ v[b, h]) / l
                L[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])
    return O, L


def attention_rows(q, k, v, rows, scale=None):
    """``attention`` for the query rows ``rows`` only (same rows in every head).

    Returns (O [B,H,len(rows),D], LSE [B,H,len(rows)]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    return attention(np.asarray(q)[:, :, rows], k, v, scale)


def probabilities(q, k, scale=None):
    """The softmax matrix softmax(scale * Q K^T) itself, [B,H,Nq,Nkv]."""
    q, k = _f64(q), _f64(k)
    scale = default_scale(q.shape[-1]) if scale is None else float(scale)
    S = scale * np.einsum("bhnd,bhmd->bhnm", q, k)
    E = np.exp(S - S.max(axis=-1, keepdims=True))
    return E / E.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Backward (pull request, "Ring kernel selection": the ring kernels pair with
# a real backward kernel, timed forward + backward; Validation: dQ/dK/dV are
# compared against a full-sequence reference).  The pages give no formulas;
# these are the chain rule applied to the definition above, for the scalar
# sum(dO * O):
#   P = softmax_row(scale Q K^T),  O = P V
#   dV = P^T dO,  dP = dO V^T,  delta_i = sum_d dO_id O_id (= sum_j P_ij dP_ij)
#   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q
# --------------------------------------------------------------------------
def attention_backward(q, k, v, dout, scale=None, row_block=256):
    """Gradients of sum(dout * attention(q, k, v)[0]) with respect to q, k, v.

    q, dout: [B,H,Nq,D]; k, v: [B,H,Nkv,D].  Returns (dq, dk, dv, delta), all
    float64, delta [B,H,Nq] = rowsum(dout * O).  Query rows are independent
    in P, dP and dq; dk and dv sum over them, ``row_block`` rows at a time.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Nq, D = q.shape
    scale = default_scale(D) if scale is None else float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                S = scale * (q[b, h, r0:r1] @ k[b, h].T)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                O = P @ v[b, h]
                dO = dout[b, h, r0:r1]
                dl = (dO * O).sum(axis=1)
                dP = dO @ v[b, h].T
                dS = P * (dP - dl[:, None])
                dq[b, h, r0:r1] = scale * (dS @ k[b, h])
                dk[b, h] += scale * (dS.T @ q[b, h, r0:r1])
                dv[b, h] += P.T @ dO
                delta[b, h, r0:r1] = dl
    return dq, dk, dv, delta


def attention_backward_rows(q, k, v, dout, rows, scale=None):
    """``attention_backward``'s dq and delta for the query rows ``rows`` only
    (a query row's gradient depends on that row alone)."""
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(q)
    kz = np.asarray(k)
    dq, _, _, delta = attention_backward(q[:, :, rows], kz, v, np.asarray(dout)[:, :, rows], scale)
    return dq, delta


def attention_backward_keys(q, k, v, dout, keys, scale=None):
    """``attention_backward``'s dk and dv for the key rows ``keys`` only.

    A key's gradients sum over every query row, each needing that row's LSE
    and delta, so those are computed for all rows first (with ``attention``);
    then for the chosen keys: P_ij = exp(scale q_i.k_j - LSE_i), dP_ij =
    dO_i.v_j, dS_ij = P_ij (dP_ij - delta_i), dk_j = scale sum_i dS_ij q_i,
    dv_j = sum_i P_ij dO_i.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    keys = np.asarray(keys, dtype=np.int64)
    scale = default_scale(q.shape[-1]) if scale is None else float(scale)
    O, L = attention(q, k, v, scale)
    delta = (dout * O).sum(axis=-1)
    B, H = q.shape[:2]
    dk = np.empty((B, H, len(keys), k.shape[-1]))
    dv = np.empty((B, H, len(keys), v.shape[-1]))
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h, keys].T)           # [Nq, nkeys]
            P = np.exp(S - L[b, h][:, None])
            dP = dout[b, h] @ v[b, h, keys].T
            dS = P * (dP - delta[b, h][:, None])
            dk[b, h] = scale * (dS.T @ q[b, h])
            dv[b, h] = P.T @ dout[b, h]
    return dk, dv


# --------------------------------------------------------------------------
# Ring share (handbook, Ring paragraph: attention over each arriving K/V block,
# merged by log-sum-exp; pull request, "Ring kernel selection": the block
# kernel returns its LSE so the merge is exact).
# --------------------------------------------------------------------------
def split_kv(k, v, nblk):
    """Contiguous token blocks of K and V: block i holds tokens
    [i*Nkv/nblk, (i+1)*Nkv/nblk)."""
    Nkv = k.shape[2]
    if Nkv % nblk:
        raise ValueError("Nkv must divide into nblk blocks")
    s = Nkv // nblk
    return [(k[:, :, i * s:(i + 1) * s], v[:, :, i * s:(i + 1) * s]) for i in range(nblk)]


def merge(o_parts, lse_parts):
    """Exact log-sum-exp merge of attention over disjoint key blocks.

    o_parts: [nblk,B,H,N,D], lse_parts: [nblk,B,H,N].
    M = max_i LSE_i; LSE = M + ln sum_i exp(LSE_i - M); O = sum_i exp(LSE_i - LSE) O_i.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    M = lse_parts.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w_un = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Msafe[None]), 0.0)
    tot = w_un.sum(axis=0)
    lse = np.where(finite, Msafe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    w = np.where(finite[None], w_un / np.where(finite, tot, 1.0)[None], 0.0)
    O = (w[..., None] * o_parts).sum(axis=0)
    return O, lse


def ring_attention(q, k, v, nblk, scale=None):
    """Attention as a ring rank computes it: per-block partials, then merge."""
    parts = [attention(q, kb, vb, scale) for kb, vb in split_kv(k, v, nblk)]
    return merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


# --------------------------------------------------------------------------
# Ulysses layout exchange on one device (handbook, "Sequence parallelism:
# Ulysses and Ring": before attention every card trades its token slice of
# all heads for all tokens of its head group, and trades back afterwards).
# Buffers are rank-stacked: axis 0 is the rank.  With n = N/P tokens per
# slice and g = H/P heads per group, the two exchanges are the index maps
#   seq->head:  out[r, b, h', s*n + i, d] = in[s, b, r*g + h', i, d]
#   head->seq:  out[s, b, r*g + h', i, d] = in[r, b, h', s*n + i, d]
# for ranks r, s < P, h' < g, i < n.  Each function below writes its map as
# a split of one axis into (rank, index) plus an axis permutation, so a
# reader can check it against the map letter by letter.  Pure data
# movement, exact in any dtype.
# --------------------------------------------------------------------------
def shard_tokens(x, P):
    """[B,H,N,D] -> [P,B,H,N/P,D]:  out[r, b, h, i, d] = x[b, h, r*n + i, d].

    Rank r holds every head of tokens [r*n, (r+1)*n), n = N/P.
    """
    x = np.asarray(x)
    B, H, N, D = x.shape
    if N % P:
        raise ValueError("N must be divisible by P")
    # token axis N -> (r, i); then move r to the front
    return np.ascontiguousarray(x.reshape(B, H, P, N // P, D).transpose(2, 0, 1, 3, 4))


def unshard_tokens(shards):
    """[P,B,H,N/P,D] -> [B,H,N,D]:  out[b, h, r*n + i, d] = shards[r, b, h, i, d]."""
    shards = np.asarray(shards)
    P, B, H, n, D = shards.shape
    return np.ascontiguousarray(shards.transpose(1, 2, 0, 3, 4)).reshape(B, H, P * n, D)


def seq2head(shards):
    """[P,B,H,N/P,D] token slices -> [P,B,H/P,N,D] head groups.

    out[r, b, h', s*n + i, d] = in[s, b, r*g + h', i, d]: rank r ends up with
    head group r (heads [r*g, (r+1)*g)) over all N tokens, the slice that
    came from rank s landing at tokens [s*n, (s+1)*n).
    """
    x = np.asarray(shards)
    P, B, H, n, D = x.shape
    if H % P:
        raise ValueError("H must be divisible by P")
    g = H // P
    # in axes (s, b, r, h', i, d) with the head axis split as r*g + h'
    t = x.reshape(P, B, P, g, n, D)
    # out axes (r, b, h', s, i, d); (s, i) then merge into the token s*n + i
    t = t.transpose(2, 1, 3, 0, 4, 5)
    return np.ascontiguousarray(t).reshape(P, B, g, P * n, D)


def head2seq(groups):
    """[P,B,H/P,N,D] head groups -> [P,B,H,N/P,D] token slices (inverse of seq2head).

    out[s, b, r*g + h', i, d] = in[r, b, h', s*n + i, d]: rank s gets back
    token slice s of every head, the group from rank r landing at heads
    [r*g, (r+1)*g).
    """
    x = np.asarray(groups)
    P, B, g, N, D = x.shape
    if N % P:
        raise ValueError("N must be divisible by P")
    n = N // P
    # in axes (r, b, h', s, i, d) with the token axis split as s*n + i
    t = x.reshape(P, B, g, P, n, D)
    # out axes (s, b, r, h', i, d); (r, h') then merge into the head r*g + h'
    t = t.transpose(3, 1, 0, 2, 4, 5)
    return np.ascontiguousarray(t).reshape(P, B, P * g, n, D)


def ulysses_attention(q, k, v, P, scale=None):
    """Attention as the P Ulysses ranks compute it together: every tensor is
    cut into token slices and exchanged to head groups, each rank runs
    ``attention`` on its group, and the outputs are exchanged back and the
    token slices joined."""
    grouped = [seq2head(shard_tokens(t, P)) for t in (q, k, v)]
    outs = np.stack([attention(grouped[0][r], grouped[1][r], grouped[2][r], scale)[0]
                     for r in range(P)])
    return unshard_tokens(head2seq(outs))


def ulysses_send_bytes_per_rank(B, H, N, D, P, elem_bytes, ntensors=3):
    """Bytes one rank sends in one seq->head exchange of ``ntensors`` tensors:
    it keeps 1/P of each [B,H,N/P,D] shard and sends the other (P-1)/P."""
    return ntensors * B * H * (N // P) * D * elem_bytes * (P - 1) // P


# --------------------------------------------------------------------------
# Joint text + image attention with rotary position embedding ("Parallelism
# Acceleration Guide", vLLM-Omni docs, "How to parallelize a new model": a dual-stream
# model attends jointly over the concatenated text and image tokens; under
# sequence parallelism the text stays whole on every rank, and the image
# rotary tables are cut along the token axis together with the image tokens).
# The pages name the rotary tables but not the rotation itself; the reading
# taken is the rotary position embedding of RoFormer in its interleaved form:
# channels (2i, 2i+1) of a token are one pair, turned by that token's angle
# for pair i, given as cos and sin tables [N, D/2].  Text tokens come first
# in the joint sequence.
# --------------------------------------------------------------------------
def rope(x, cos, sin):
    """Turn each channel pair (2i, 2i+1) of token n by the angle whose cosine
    and sine are cos[n, i] and sin[n, i]:
        y[2i]   = x[2i] cos - x[2i+1] sin
        y[2i+1] = x[2i] sin + x[2i+1] cos
    x: [..., N, D]; cos, sin: [N, D/2].  Returns float64 [..., N, D]."""
    x, c, s = _f64(x), _f64(cos), _f64(sin)
    even, odd = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = even * c - odd * s
    y[..., 1::2] = even * s + odd * c
    return y


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (8 significant bits),
    ties to even; zero stays zero.  Finite inputs in bfloat16's normal range."""
    x = _f64(x)
    out = np.zeros_like(x)
    nz = x != 0
    ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(x[nz]))).astype(np.int64) - 7)
    out[nz] = np.round(x[nz] / ulp) * ulp   # numpy rounds halves to even
    return out


def joint_sequence(x_txt, x_img, cos_txt=None, sin_txt=None, cos_img=None, sin_img=None,
                   to_bf16=False):
    """[B,H,Nt,D] text and [B,H,Ni,D] image tokens -> [B,H,Nt+Ni,D], text
    first, each part turned by its own rotary tables when they are given.
    to_bf16: round the result to bfloat16, the type the attention takes its
    inputs in (the reading for a bf16 model: the turned tokens are handed to
    attention in the model's type)."""
    t = _f64(x_txt) if cos_txt is None else rope(x_txt, cos_txt, sin_txt)
    i = _f64(x_img) if cos_img is None else rope(x_img, cos_img, sin_img)
    y = np.concatenate([t, i], axis=2)
    return round_bf16(y) if to_bf16 else y


def joint_attention(q_txt, k_txt, v_txt, q_img, k_img, v_img, cos_txt=None, sin_txt=None,
                    cos_img=None, sin_img=None, scale=None, rows=None, to_bf16=False):
    """Attention of every text and image query over every text and image key,
    with RoPE on queries and keys (not values).  Returns (O, LSE) of the joint
    sequence [B,H,Nt+Ni,...]; ``rows`` restricts the queries to those joint
    rows; ``to_bf16`` rounds the turned queries and keys to bfloat16 first."""
    q = joint_sequence(q_txt, q_img, cos_txt, sin_txt, cos_img, sin_img, to_bf16)
    k = joint_sequence(k_txt, k_img, cos_txt, sin_txt, cos_img, sin_img, to_bf16)
    v = joint_sequence(v_txt, v_img)
    if rows is not None:
        q = q[:, :, np.asarray(rows, dtype=np.int64)]
    return attention(q, k, v, scale)


# --------------------------------------------------------------------------
# FP8 attention.  The handbook ("Multi-GPU parallelism: spreading one step
# over several cards", section "Combining: what xDiT does") stacks FP8 low
# precision on top of the parallel split and caching, without saying which
# tensors are 8-bit.  The reading taken: queries and keys are quantized to the
# OCP 8-bit floating-point format E4M3 (1 sign, 4 exponent bits with bias 7,
# 3 mantissa bits, subnormals, largest finite 448, no infinities, S.1111.111
# is NaN), one scale per (b, h) from the tensor's largest magnitude; the
# scores are their exact product times both scales; P and V stay in the
# model's type.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """E4M3 codes (uint8) -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_round(x):
    """Nearest E4M3 value to each finite float64 x, ties to even, magnitudes
    beyond 448 clamped to 448.  The spacing is 2**(e-3) in the binade
    [2**e, 2**(e+1)) for e >= -6 and 2**-9 below 2**-6 (subnormals)."""
    x = _f64(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a >= 2.0 ** -6, np.ldexp(1.0, (e - 3).astype(np.int64)), 2.0 ** -9)
    r = np.round(a / ulp) * ulp                      # halves to even
    return np.copysign(np.minimum(r, E4M3_MAX), x)


def e4m3_encode(x):
    """Codes of e4m3_round(x) (uint8); -0 encodes as 0x80."""
    v = e4m3_round(x)
    a = np.abs(v)
    sub = a < 2.0 ** -6
    e = np.floor(np.log2(np.where(sub, 1.0, a)))
    m_norm = np.round((a / np.ldexp(1.0, e.astype(np.int64)) - 1.0) * 8.0)
    m_sub = np.round(a / 2.0 ** -9)
    code = np.where(sub, m_sub, ((e + 7) * 8 + m_norm))
    return (code.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8))


def quantize_fp8(x):
    """Per-(b, h) E4M3 quantization of x [B,H,N,D] (float32 values).

    descale[b,h] = amax / 448 in float32 (1 when the head is all zeros);
    code = E4M3 rounding of the float32 quotient x / descale, clamped to
    +-448.  Returns (codes uint8 [B,H,N,D], descale float32 [B,H]).  The
    quotient is taken in float32, the type the scale is kept in, so both the
    scale and each code are fixed by float32 arithmetic."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=(2, 3)) if x32.size else np.zeros(x32.shape[:2], np.float32)
    descale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quotient = x32 / descale[:, :, None, None]
    return e4m3_encode(quotient.astype(np.float64)), descale


def attention_fp8(q_codes, k_codes, v, q_descale, k_descale, scale=None, rows=None):
    """Attention of E4M3 queries and keys: q = decode(q_codes) * q_descale[b,h],
    likewise k; v as given.  ``scale`` defaults to 1/sqrt(D)."""
    q = e4m3_decode(q_codes) * _f64(q_descale)[:, :, None, None]
    k = e4m3_decode(k_codes) * _f64(k_descale)[:, :, None, None]
    if rows is not None:
        q = q[:, :, np.asarray(rows, dtype=np.int64)]
    return attention(q, k, v, scale)


# --------------------------------------------------------------------------
# FP8 attention, second reading: the scaling done by the fp8 matrix
# instruction itself.  The same step ("Multi-GPU parallelism ...", "Combining:
# what xDiT does": FP8 low precision on top of the split) read for hardware
# whose fp8 products take power-of-two (E8M0) scales: each head of q and of k
# gets a power-of-two scale, the smallest that brings its largest magnitude
# within E4M3's 448, and the queries are first multiplied in float32 by the
# softmax constant scale * log2(e), so that the scaled products are the
# scores in base 2.  P and V stay in the model's type.
# --------------------------------------------------------------------------
LOG2E_F32 = np.float32(1.4426950408889634)


def pow2_descale(amax):
    """Per-head power-of-two scale for largest magnitudes ``amax`` (float32):
    the smallest 2**e with amax <= 448 * 2**e, e >= -126; 1 where amax is 0."""
    a = np.asarray(amax, dtype=np.float64)
    safe = np.where(a > 0, a, E4M3_MAX)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # exact correction of the floating-point log: 448 * 2**e is exact in float64
    e = np.where(E4M3_MAX * np.ldexp(1.0, e) < safe, e + 1, e)
    e = np.where(E4M3_MAX * np.ldexp(1.0, e - 1) >= safe, e - 1, e)
    e = np.maximum(e, -126)
    return np.where(a > 0, np.ldexp(1.0, e), 1.0).astype(np.float32)


def quantize_fp8_mx(q, k, scale=None):
    """Queries and keys [B,H,N,D] (float32 values) of one attention call ->
    (q_codes, k_codes, q_descale, k_descale).

    q' = float32(q * c0) with c0 = float32(scale) * float32(log2 e) (the
    float32 product); k' = k.  Per (b, h): d = pow2_descale(max |x'|), codes =
    E4M3 of x' / d (exact: d is a power of two).  ``scale`` defaults to
    1/sqrt(D)."""
    q32 = np.asarray(q, dtype=np.float32)
    k32 = np.asarray(k, dtype=np.float32)
    scale = default_scale(q32.shape[-1]) if scale is None else scale
    c0 = np.float32(np.float32(scale) * LOG2E_F32)
    out = []
    for x in (q32 * c0, k32):
        amax = np.abs(x).max(axis=(2, 3)) if x.size else np.zeros(x.shape[:2], np.float32)
        d = pow2_descale(amax)
        out.append((e4m3_encode(x.astype(np.float64) / d.astype(np.float64)[:, :, None, None]), d))
    return out[0][0], out[1][0], out[0][1], out[1][1]


def attention_fp8_mx(q_codes, k_codes, v, q_descale, k_descale, rows=None):
    """Attention whose scores are in base 2: s_ij = q_descale * k_descale *
    (q_i . k_j) of the decoded codes, P_ij = 2**s_ij / sum_j 2**s_ij, O = P V,
    LSE (natural log) = ln 2 * log2 sum_j 2**s_ij."""
    q = e4m3_decode(q_codes) * _f64(q_descale)[:, :, None, None]
    k = e4m3_decode(k_codes) * _f64(k_descale)[:, :, None, None]
    if rows is not None:
        q = q[:, :, np.asarray(rows, dtype=np.int64)]
    s2 = np.einsum("bhid,bhjd->bhij", q, k)
    m = s2.max(axis=-1, keepdims=True)
    w = np.exp2(s2 - m)
    den = w.sum(axis=-1, keepdims=True)
    O = np.einsum("bhij,bhjd->bhid", w / den, _f64(v))
    lse = np.log(2.0) * (m[..., 0] + np.log2(den[..., 0]))
    return O, lse
