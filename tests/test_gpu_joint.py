"""GPU parity of joint text + image attention with RoPE, and of cross
attention, against the fp64 oracle.

* dit_rope_pack: the image and text parts land in place; V-style parts
  without tables are copied bit for bit; turned elements are the fp64
  rotation faithfully rounded to bf16 (within one bf16 unit in the last
  place of the exact value: the kernel turns in float32, then rounds to
  nearest).
* dit_attn_fwd_joint: O and LSE against oracle.joint_attention with the
  turned q and k rounded to bf16 (the reading that they enter attention in
  the model's type, as the library does), at the bf16 attention tolerances
  (O max-abs 2e-2, rel-RMS 1e-2; LSE max-abs 1e-3); O also against the
  unrounded fp64 definition at the same O tolerances.  (The unrounded LSE
  differs by up to the score error of that rounding, about 1.6e-3 * |q||k|
  * scale per score on N(0,1) inputs, which is why the LSE bar is taken
  against the rounded reading.)
* Cross attention (image queries over text keys) is dit_attn_fwd_block with
  Nkv = the text length.
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


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def f64(bits):
    return datagen.bf16_to_f32(bits).astype(np.float64)


def _image_tables(Ni, D, cols=64):
    rows = -(-Ni // cols)
    c, s = datagen.rope_tables_image(rows, cols, D)
    return np.ascontiguousarray(c[:Ni]), np.ascontiguousarray(s[:Ni])


def _case(B, H, Ht, Nt, Ni, D, seed, text_tables=True, image_tables=True):
    txt, img = datagen.joint_bf16(B, Ht, Nt, H, Ni, D, seed)
    ci, si = _image_tables(Ni, D) if image_tables else (None, None)
    ct, st = datagen.rope_tables_text(Nt, 64, 64, D) if text_tables else (None, None)
    return txt, img, (ct, st, ci, si)


def _dev_tables(tabs):
    return [None if t is None else torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in tabs]


def _faithful(got, ref):
    """Every bf16 result lies within one unit in the last place of the exact
    value (so it is one of the two bf16 numbers around it)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    nz = ref != 0
    ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(ref[nz]))).astype(np.int64) - 7)
    ok = np.all(np.abs(got[nz] - ref[nz]) < ulp) and np.all(got[~nz] == 0)
    exact = np.mean(got == f64(datagen.bf16_bits(ref.astype(np.float32))))
    return ok, exact


@pytest.mark.parametrize("B,H,Ht,h0,Nt,Ni,D", [
    (1, 2, 2, 0, 7, 100, 128),
    (2, 3, 6, 3, 77, 300, 64),     # head group 3..5 of a replicated 6-head text
    (1, 4, 4, 0, 0, 130, 32),      # image only
    (1, 2, 5, 1, 65, 0, 128),      # text only
])
def test_rope_pack(B, H, Ht, h0, Nt, Ni, D):
    say("rope_pack", B, H, Ht, h0, Nt, Ni, D)
    txt, img, tabs = _case(B, H, Ht, Nt, Ni, D, seed=Nt + Ni + D)
    ct, st, ci, si = _dev_tables(tabs)
    xt, xi = bits_to_torch_bf16(txt[0]), bits_to_torch_bf16(img[0])
    out = dta.dit_rope_pack(xt, xi, ct, st, ci, si, h0=h0)
    ref = oracle.joint_sequence(f64(txt[0])[:, h0:h0 + H], f64(img[0]), *tabs)
    ok, exact = _faithful(to_f64(out), ref)
    say(f"  faithful {ok}, equal to round-to-nearest of the exact value: {exact:.6f}")
    assert ok and exact > 0.999
    # no tables: a bit-exact copy of both parts
    plain = dta.dit_rope_pack(xt, xi, h0=h0)
    want = np.concatenate([txt[0][:, h0:h0 + H], img[0]], axis=2)
    assert np.array_equal(plain.cpu().view(torch.int16).numpy().view(np.uint16), want)


def test_rope_pack_into_guarded_output():
    say("rope_pack guard bands")
    txt, img, tabs = _case(1, 2, 2, 33, 70, 128, seed=3)
    n = 2 * 103 * 128
    buf = torch.full((n + 2048,), 7.0, device="cuda", dtype=torch.bfloat16)
    out = buf[1024:1024 + n].view(1, 2, 103, 128)
    dta.dit_rope_pack(bits_to_torch_bf16(txt[1]), bits_to_torch_bf16(img[1]),
                      *_dev_tables(tabs), out=out)
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[-1024:] == 7.0)


def _check_joint(O, L, tsel, img, tabs, rows=None, what="joint"):
    img = [f64(x) for x in img]
    Or, Lr = oracle.joint_attention(*tsel, *img, *tabs, rows=rows, to_bf16=True)
    ma, rr = assert_bf16_close(O, L, Or, Lr, what + " (bf16 turned inputs)")
    Oe, _ = oracle.joint_attention(*tsel, *img, *tabs, rows=rows)
    ma2, rr2 = assert_bf16_close(O, None, Oe, None, what + " (exact turn)")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}; against the unrounded turn {ma2:.2e} / {rr2:.2e}")


def _joint_gpu(txt, img, tabs, h0=0, scale=None):
    t = [bits_to_torch_bf16(x) for x in txt]
    i = [bits_to_torch_bf16(x) for x in img]
    return dta.dit_attn_fwd_joint(*t, *i, *_dev_tables(tabs), h0=h0, scale=scale)


@pytest.mark.parametrize("B,H,Ht,h0,Nt,Ni,D,tt,it", [
    (1, 2, 2, 0, 7, 100, 128, True, True),
    (2, 3, 6, 3, 77, 300, 64, True, True),
    (1, 2, 2, 0, 64, 257, 128, False, True),   # text unturned
    (1, 4, 4, 0, 0, 200, 32, True, True),      # image only
    (1, 2, 3, 1, 90, 0, 128, True, True),      # text only
    (1, 1, 1, 0, 1, 1, 128, True, True),       # one token each
])
def test_joint_small(B, H, Ht, h0, Nt, Ni, D, tt, it):
    say("joint", B, H, Ht, h0, Nt, Ni, D, tt, it)
    txt, img, tabs = _case(B, H, Ht, Nt, Ni, D, seed=2 * Nt + Ni, text_tables=tt, image_tables=it)
    O, L = _joint_gpu(txt, img, tabs, h0=h0)
    _check_joint(to_f64(O), to_f64(L), [f64(x)[:, h0:h0 + H] for x in txt], img, tabs)


@pytest.mark.parametrize("H,Ht,h0,Nt,Ni,D,tt", [
    (3, 3, 0, 50, 400, 128, True),     # text not on a 64-key boundary: v packed too
    (3, 3, 0, 128, 400, 128, True),    # v read from its two parts
    (2, 6, 2, 64, 300, 64, False),     # head group of a replicated text, text unturned
    (2, 2, 0, 0, 300, 32, True),       # image only
    (2, 4, 1, 192, 0, 128, True),      # text only
])
def test_joint_equals_pack_then_attention(H, Ht, h0, Nt, Ni, D, tt):
    """The joint call (queries turned in the attention kernel, v read from its
    parts when Nt % 64 == 0) gives the bits of packing q, k, v with
    dit_rope_pack and running dit_attn_fwd on the joint sequence."""
    say("joint == rope_pack x3 + dit_attn_fwd", H, Ht, h0, Nt, Ni, D, tt)
    txt, img, tabs = _case(1, H, Ht, Nt, Ni, D, seed=21 + Nt, text_tables=tt)
    O, L = _joint_gpu(txt, img, tabs, h0=h0, scale=0.1)
    dt = _dev_tables(tabs)
    q, k, v = (dta.dit_rope_pack(bits_to_torch_bf16(a), bits_to_torch_bf16(b), *tb, h0=h0)
               for a, b, tb in zip(txt, img, (dt, dt, [None] * 4)))
    O2, L2 = dta.dit_attn_fwd(q, k, v, scale=0.1)
    assert torch.equal(O, O2) and torch.equal(L, L2)


def test_joint_image_share_full():
    """Image tokens of a 1024x1024 picture (64 x 64 patches, 24 heads of 128)
    with 512 text tokens."""
    say("joint B1 H24 text 512 + image 4096 D128, full compare")
    txt, img, tabs = _case(1, 24, 24, 512, 4096, 128, seed=31)
    O, L = _joint_gpu(txt, img, tabs)
    _check_joint(to_f64(O), to_f64(L), [f64(x) for x in txt], img, tabs, what="joint image share")


def test_joint_ulysses_share_sampled_rows():
    """One Ulysses head group (heads 10..19 of 40) of a 32768-token image with
    the 512 text tokens replicated on every rank; sampled joint rows."""
    say("joint H10 of 40, text 512 + image 32768, sampled rows")
    txt, img, tabs = _case(1, 10, 40, 512, 32768, 128, seed=41)
    O, L = _joint_gpu(txt, img, tabs, h0=10)
    rows = np.unique(np.concatenate([[0, 511, 512, 33279],
                                     datagen.sample_rows(33280, 60, 42)]))
    ri = torch.from_numpy(rows).cuda()
    _check_joint(to_f64(O[:, :, ri]), to_f64(L[:, :, ri]), [f64(x)[:, 10:20] for x in txt], img,
                 tabs, rows=rows, what="joint ulysses")
    assert torch.isfinite(O).all()


@pytest.mark.parametrize("H,Nq,Nt", [(24, 4096, 512), (2, 300, 77), (3, 129, 333), (1, 64, 1)])
def test_cross_attention(H, Nq, Nt):
    """Image queries over text keys and values (no RoPE): dit_attn_fwd_block."""
    say("cross", H, Nq, Nt)
    qb, kb, vb = datagen.small_bf16(1, H, Nq, 128, seed=H + Nq + Nt, Nkv=Nt)
    O, L = dta.dit_attn_fwd_block(*(bits_to_torch_bf16(x) for x in (qb, kb, vb)),
                                  out_dtype=torch.bfloat16)
    Oref, Lref = oracle.attention(f64(qb), f64(kb), f64(vb))
    assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "cross")


def test_cross_attention_ulysses_share_sampled_rows():
    say("cross H10 N32768 over 512 text tokens, sampled rows")
    q = datagen.workload_inputs("ulysses_share")[0][:, :10]
    _, kb, vb = datagen.small_bf16(1, 10, 1, 128, seed=51, Nkv=512)
    O, L = dta.dit_attn_fwd_block(*(bits_to_torch_bf16(x) for x in (q, kb, vb)),
                                  out_dtype=torch.bfloat16)
    rows = datagen.sample_rows(32768, 64, 52)
    Oref, Lref = oracle.attention_rows(f64(q), f64(kb), f64(vb), rows)
    ri = torch.from_numpy(rows).cuda()
    assert_bf16_close(to_f64(O[:, :, ri]), to_f64(L[:, :, ri]), Oref, Lref, "cross ulysses")
