"""Sizes past 2^31 elements per tensor: 64-bit addressing in every kernel.

B1 H2050 N8192 D128 bf16 holds 2.15e9 elements (4.3 GB) per tensor, so the
offsets of the later heads exceed a 32-bit element index (and, in bytes,
any 32-bit range).  Inputs are drawn on the device by torch's seeded
generator; the oracle gets the heads it checks copied back.  Checked: the
forward on sampled rows of the first, a middle and the last head; the
work-balanced forward (65600 query tiles: its key-split tail is the last
64, the last two heads) on sampled tail rows, with the whole-wave rows bit-identical to
the forward; the backward's dq on sampled rows and dk, dv on sampled keys
of the last head; the Ulysses exchange on sampled (rank, shard, head,
token) runs, bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
import diffusion_transformer_attention_amd as dta
from _helpers import assert_bf16_close, to_f64

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 2050, 8192, 128
GRAD_REL_RMS, GRAD_MAX_ABS_REL = 1e-2, 3e-2


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def head64(t, h):
    return t[:, h:h + 1].float().cpu().double().numpy()


@pytest.fixture(scope="module")
def qkv():
    say(f"drawing q, k, v [{B},{H},{N},{D}] bf16 on the device")
    assert B * H * N * D > 2 ** 31
    t = [datagen.device_normal_bf16((B, H, N, D), seed) for seed in (11, 12, 13)]
    yield t
    del t
    torch.cuda.empty_cache()


def test_forward_large(qkv):
    q, k, v = qkv
    say("forward, 2.15e9 elements per tensor")
    O, L = dta.dit_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    rows = datagen.sample_rows(N, 16, 2001)
    ri = torch.from_numpy(rows).cuda()
    for h in (0, 1025, H - 1):
        Oref, Lref = oracle.attention_rows(head64(q, h), head64(k, h), head64(v, h), rows)
        assert_bf16_close(to_f64(O[:, h:h + 1, ri]), to_f64(L[:, h:h + 1, ri]), Oref, Lref,
                          f"head {h}")
    say("work-balanced forward at the same size")
    nbytes = dta.dit_attn_fwd_balanced_workspace(B, H, N, N, D)
    assert nbytes > 0
    ws = torch.empty((nbytes,), device="cuda", dtype=torch.uint8)
    Ob, Lb = dta.dit_attn_fwd_balanced(q, k, v, workspace=ws)
    slots = torch.cuda.get_device_properties(0).multi_processor_count
    total = B * H * (N // 256)
    r0 = (total // slots * slots) * 256                   # N is a multiple of the tile
    assert torch.equal(Ob.reshape(-1, D)[:r0], O.reshape(-1, D)[:r0])
    assert torch.equal(Lb.reshape(-1)[:r0], L.reshape(-1)[:r0])
    h0, n0 = divmod(r0, N)
    assert h0 >= H - 2                                    # the 64 tail tiles: the last two heads
    rng = np.random.default_rng(2002)
    for h in range(h0, H):
        lo = n0 if h == h0 else 0
        rows = np.unique(np.concatenate([[lo, N - 1], rng.integers(lo, N, 14)]))
        ri = torch.from_numpy(rows).cuda()
        Oref, Lref = oracle.attention_rows(head64(q, h), head64(k, h), head64(v, h), rows)
        assert_bf16_close(to_f64(Ob[:, h:h + 1, ri]), to_f64(Lb[:, h:h + 1, ri]), Oref, Lref,
                          f"balanced tail head {h}")
    del O, L, Ob, Lb, ws
    torch.cuda.empty_cache()


def test_backward_large(qkv):
    q, k, v = qkv
    say("backward, 2.15e9 elements per tensor")
    dout = datagen.device_normal_bf16((B, H, N, D), 14)
    O, L = dta.dit_attn_fwd(q, k, v)
    dq, dk, dv, delta = dta.dit_attn_bwd(q, k, v, O, dout, L)
    torch.cuda.synchronize()
    h = H - 1
    rows = datagen.sample_rows(N, 8, 2003)
    keys = datagen.sample_rows(N, 8, 2004)
    ri, ki = torch.from_numpy(rows).cuda(), torch.from_numpy(keys).cuda()
    q64, k64, v64, do64 = (head64(t, h) for t in (q, k, v, dout))
    rq, rd = oracle.attention_backward_rows(q64, k64, v64, do64, rows)
    rk, rv = oracle.attention_backward_keys(q64, k64, v64, do64, keys)
    for got, ref, n in ((dq[:, h:h + 1, ri], rq, "dq"), (dk[:, h:h + 1, ki], rk, "dk"),
                        (dv[:, h:h + 1, ki], rv, "dv"), (delta[:, h:h + 1, ri], rd, "delta")):
        err = to_f64(got) - ref
        rr = float(np.linalg.norm(err.ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))
        assert rr <= GRAD_REL_RMS, f"{n} rel-RMS {rr:.3e}"
        if n != "delta":
            ma = float(np.abs(err).max() / max(np.abs(ref).max(), 1e-300))
            assert ma <= GRAD_MAX_ABS_REL, f"{n} max-abs {ma:.3e}"
    del dout, O, L, dq, dk, dv, delta
    torch.cuda.empty_cache()


def test_permutes_large(qkv):
    q = qkv[0]
    P = 2
    say(f"seq2head / head2seq of [{P}][{B},{H},{N // P},{D}] shards")
    shards = torch.stack(q.chunk(P, dim=2)).contiguous()
    groups = dta.ulysses_seq2head(shards)
    back = dta.ulysses_head2seq(groups)
    torch.cuda.synchronize()
    assert torch.equal(back, shards)
    rng = np.random.default_rng(2005)
    hg, ns = H // P, N // P
    for _ in range(16):   # out[r][b, h', s*N/P + n] == in[s][b, r*H/P + h', n]
        r, s_, hh = int(rng.integers(P)), int(rng.integers(P)), int(rng.integers(hg))
        n = int(rng.integers(ns))
        assert torch.equal(groups[r, 0, hh, s_ * ns + n], shards[s_, 0, r * hg + hh, n])
    del shards, groups, back
    torch.cuda.empty_cache()
