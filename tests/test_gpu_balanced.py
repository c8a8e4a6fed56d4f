"""GPU parity of the work-balanced forward (dit_attn_fwd_balanced).

The query tiles that fill whole waves of the planned workgroup slots must
equal the plain forward (dit_attn_fwd_block) bit for bit; the rows of the
key-split tail tiles, computed as float32 chunk partials merged by
log-sum-exp, must meet the bf16 tolerances against the fp64 oracle (in full
at small sizes, on sampled rows of the tail at the long-video shape); two
calls give the same bits; nothing outside O and LSE is written.  The
workspace is filled with NaN before each call, so a partial the merge read
before the split kernel wrote it would show.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
import diffusion_transformer_attention_amd as dta
from _helpers import assert_bf16_close, bits_to_torch_bf16, to_f64

pytestmark = pytest.mark.gpu

GUARD = 4096
BM = 256  # query rows per tile


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def f64(bits):
    return datagen.bf16_to_f32(bits).astype(np.float64)


def _slots(slots):
    return slots if slots > 0 else torch.cuda.get_device_properties(0).multi_processor_count


def _tail_row0(B, H, Nq, slots):
    """First flat query row of the key-split tail (the whole waves come first)."""
    nqt = -(-Nq // BM)
    total = B * H * nqt
    whole = total // slots * slots
    return (whole // nqt) * Nq + (whole % nqt) * BM


def _run(q, k, v, out_dtype, slots, with_lse=True):
    B, H, Nq, D = q.shape
    nbytes = dta.dit_attn_fwd_balanced_workspace(B, H, Nq, k.shape[2], D, slots)
    assert nbytes > 0, "these sizes should take the key-split path"
    ws = torch.full((nbytes // 4,), float("nan"), device="cuda", dtype=torch.float32)
    obuf = torch.full((B * H * Nq * D + 2 * GUARD,), -12345.0, device="cuda", dtype=out_dtype)
    O = obuf[GUARD:GUARD + B * H * Nq * D].view(B, H, Nq, D)
    lbuf = torch.full((B * H * Nq + 2 * GUARD,), -12345.0, device="cuda", dtype=torch.float32)
    L = lbuf[GUARD:GUARD + B * H * Nq].view(B, H, Nq) if with_lse else None
    dta.dit_attn_fwd_balanced(q, k, v, out_dtype=out_dtype, out=O, lse=L, return_lse=with_lse,
                              slots=slots, workspace=ws.view(torch.uint8))
    torch.cuda.synchronize()
    for buf in (obuf, lbuf):
        s = torch.full((GUARD,), -12345.0, device="cuda", dtype=buf.dtype)
        assert torch.equal(buf[:GUARD], s) and torch.equal(buf[-GUARD:], s), "write outside O/LSE"
    if not with_lse:
        assert torch.equal(lbuf[GUARD:-GUARD], torch.full_like(lbuf[GUARD:-GUARD], -12345.0))
    return O, L


@pytest.mark.parametrize("B,H,Nq,Nkv,D,slots,out,with_lse", [
    (1, 3, 700, 3000, 128, 4, torch.bfloat16, True),   # 8 whole tiles + 1 split, partial tiles
    (2, 2, 300, 2500, 64, 7, torch.float32, True),     # tail tile in the second batch
    (1, 5, 256, 2049, 32, 2, torch.bfloat16, True),    # one key past a tile: a 1-key last chunk tile
    (1, 2, 600, 3000, 128, 4, torch.bfloat16, False),  # no LSE
    (1, 2, 1000, 2000, 128, 0, torch.bfloat16, True),  # the device's slots: every tile split
    (1, 1, 1, 4000, 128, 0, torch.float32, True),      # a single query row
])
def test_balanced_small(B, H, Nq, Nkv, D, slots, out, with_lse):
    say(f"balanced B{B} H{H} Nq{Nq} Nkv{Nkv} D{D} slots {slots} {out} lse {with_lse}")
    qb, kb, vb = datagen.small_bf16(B, H, Nq, D, seed=Nq + Nkv + D, Nkv=Nkv)
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    O, L = _run(q, k, v, out, slots, with_lse)
    Oref, Lref = oracle.attention(f64(qb), f64(kb), f64(vb))
    assert_bf16_close(to_f64(O), to_f64(L) if with_lse else None, Oref, Lref, "balanced")
    # whole-wave rows: the plain kernel's bits
    Op, Lp = dta.dit_attn_fwd_block(q, k, v, out_dtype=out)
    r0 = _tail_row0(B, H, Nq, _slots(slots))
    assert torch.equal(O.reshape(-1, D)[:r0], Op.reshape(-1, D)[:r0])
    if with_lse:
        assert torch.equal(L.reshape(-1)[:r0], Lp.reshape(-1)[:r0])
    # repeatable
    O2, L2 = _run(q, k, v, out, slots, with_lse)
    assert torch.equal(O, O2) and (not with_lse or torch.equal(L, L2))


def test_balanced_image_share_full():
    say("balanced image share B1 H24 N4096 D128, full compare")
    qb, kb, vb = datagen.workload_inputs("image_share")
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    O, L = _run(q, k, v, torch.bfloat16, 0)
    Oref, Lref = oracle.attention(f64(qb), f64(kb), f64(vb))
    assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "balanced image share")
    Op, Lp = dta.dit_attn_fwd(q, k, v)
    r0 = _tail_row0(1, 24, 4096, _slots(0))
    assert torch.equal(O.reshape(-1, 128)[:r0], Op.reshape(-1, 128)[:r0])
    assert torch.equal(L.reshape(-1)[:r0], Lp.reshape(-1)[:r0])


def test_balanced_long_video():
    say("balanced long video B1 H10 N75600 D128: whole rows bitwise, tail rows sampled")
    qb, kb, vb = datagen.workload_inputs("long_video")
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    O, L = _run(q, k, v, torch.bfloat16, 0)
    Op, Lp = dta.dit_attn_fwd(q, k, v)
    r0 = _tail_row0(1, 10, 75600, _slots(0))
    assert 0 < r0 < 10 * 75600
    assert torch.equal(O.reshape(-1, 128)[:r0], Op.reshape(-1, 128)[:r0])
    assert torch.equal(L.reshape(-1)[:r0], Lp.reshape(-1)[:r0])
    # sampled tail rows (they all lie in the last head at this shape) vs the oracle
    h, n0 = divmod(r0, 75600)
    rng = np.random.default_rng(1005)
    rows = np.unique(np.concatenate([[n0, 75599], rng.integers(n0, 75600, 62)])).astype(np.int64)
    Oref, Lref = oracle.attention_rows(f64(qb[:, h:h + 1]), f64(kb[:, h:h + 1]),
                                       f64(vb[:, h:h + 1]), rows)
    ri = torch.from_numpy(rows).cuda()
    assert_bf16_close(to_f64(O[:, h:h + 1, ri]), to_f64(L[:, h:h + 1, ri]), Oref, Lref,
                      "balanced long video tail")


def test_balanced_score_jump_in_a_split_chunk():
    """A late key scoring ~100 (base 2) above the first step's max of its
    chunk: the chunk's pass must take the exact-max path, and the merge must
    still give the oracle's row (dominated by that key's value)."""
    say("balanced score jump: 4 tiles on 3 slots, the last tile split in key chunks")
    rng = np.random.default_rng(92)
    q = rng.standard_normal((1, 2, 300, 128)).astype(np.float32)
    k = rng.standard_normal((1, 2, 4100, 128)).astype(np.float32)
    v = rng.standard_normal((1, 2, 4100, 128)).astype(np.float32)
    k[0, 0, 700] = 6.0 * q[0, 0, 5]          # head 0, a whole tile
    k[0, 1, 4097] = 6.0 * q[0, 1, 260]       # head 1, tail tile, last chunk's partial key tile
    qb, kb, vb = (datagen.bf16_bits(x) for x in (q, k, v))
    O, L = _run(*(bits_to_torch_bf16(x) for x in (qb, kb, vb)), torch.float32, 3)
    Oref, Lref = oracle.attention(f64(qb), f64(kb), f64(vb))
    assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "balanced score jump")
    assert abs(to_f64(O)[0, 1, 260] - f64(vb)[0, 1, 4097]).max() < 2e-2
    assert abs(to_f64(O)[0, 0, 5] - f64(vb)[0, 0, 700]).max() < 2e-2
