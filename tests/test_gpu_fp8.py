"""GPU parity of the FP8 path against the fp64 oracle.

* dit_quant_fp8 is bit-exact: codes and descales equal oracle.quantize_fp8
  (amax exact, quotient and descale correctly rounded float32, E4M3 rounding
  to nearest-even with the +-448 clamp).
* dit_attn_fwd_fp8 takes codes and descales made by the oracle (never by the
  library) and is held to the bf16 attention bars against
  oracle.attention_fp8 on the same codes (O max-abs 2e-2, rel-RMS 1e-2; LSE
  max-abs 1e-3) on the N(0,1) workloads.  P and V are bf16 as in the bf16
  kernel; the scores come from v_mfma_f32_16x16x128_f8f6f4, which keeps each
  product only down to 2^-13 of the largest product of the same output
  (measured on gfx950: 2^16 + 8 exact, 2^16 + 4 and 2^16 + 1 lost), so a
  score can be off by up to scale * descales * 128 * 2^-13 * max_d |q_d k_d|
  (codes).  The LSE, a softmax average of scores, is held to 1e-3 plus that
  bound where scores are far from unit size.
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


def f32(bits):
    return datagen.bf16_to_f32(bits)


def _dev_codes(c):
    return torch.from_numpy(np.ascontiguousarray(c)).cuda()


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("B,H,N,D,spread", [
    (1, 2, 64, 128, 0.0),
    (2, 3, 37, 64, 6.0),       # values spanning 2^-8.6 .. 2^8.6: subnormal codes too
    (1, 1, 1, 32, 0.0),
    (1, 4, 300, 128, 12.0),
])
def test_quant_bit_exact(B, H, N, D, spread):
    say("quant", B, H, N, D, spread)
    r = np.random.default_rng(N + D)
    x = r.standard_normal((B, H, N, D)).astype(np.float32)
    x *= np.exp(r.uniform(-spread, spread, size=x.shape)).astype(np.float32)
    if H > 2:
        x[0, 1] = 0.0                      # an all-zero head
        x[0, 2, 0, 0] = 3.0e30             # a head whose scale is huge
    bits = datagen.bf16_bits(x)
    codes, ds = dta.dit_quant_fp8(bits_to_torch_bf16(bits))
    want_c, want_d = oracle.quantize_fp8(f32(bits))
    assert np.array_equal(ds.cpu().numpy(), want_d)
    got_c = codes.cpu().numpy()
    bad = np.count_nonzero(got_c != want_c)
    assert bad == 0, f"{bad} codes differ"


def test_quant_empty_sequence():
    say("quant N=0")
    x = torch.empty((1, 3, 0, 128), device="cuda", dtype=torch.bfloat16)
    codes, ds = dta.dit_quant_fp8(x)
    assert codes.numel() == 0 and torch.equal(ds, torch.ones_like(ds))


@pytest.mark.parametrize("B,H,Nq,Nkv,D", [(1, 3, 300, 77, 128), (2, 2, 64, 0, 64), (1, 10, 32768, 32768, 128)])
def test_quant_qk_equals_two_single_calls_and_oracle(B, H, Nq, Nkv, D):
    """dit_quant_fp8_qk (q and k in three launches) gives the bits of two
    dit_quant_fp8 calls, and the oracle's codes and descales."""
    say("quant qk", B, H, Nq, Nkv, D)
    r = np.random.default_rng(Nq + 3 * Nkv)
    xs = []
    for n in (Nq, Nkv):
        x = r.standard_normal((B, H, n, D)).astype(np.float32)
        x *= np.exp(r.uniform(-4, 4, size=x.shape)).astype(np.float32)
        if n and H > 2:
            x[0, 1] = 0.0
        xs.append(datagen.bf16_bits(x))
    tq, tk = (bits_to_torch_bf16(x) for x in xs)
    qc, kc, qd, kd = dta.dit_quant_fp8_qk(tq, tk)
    qc1, qd1 = dta.dit_quant_fp8(tq)
    kc1, kd1 = dta.dit_quant_fp8(tk)
    assert torch.equal(qc, qc1) and torch.equal(qd, qd1)
    assert torch.equal(kc, kc1) and torch.equal(kd, kd1)
    if Nq * H <= 300 * 3:
        for bits, c, d in ((xs[0], qc, qd), (xs[1], kc, kd)):
            want_c, want_d = oracle.quantize_fp8(f32(bits))
            assert np.array_equal(d.cpu().numpy(), want_d)
            assert np.array_equal(c.cpu().numpy(), want_c)
    if Nkv == 0:
        assert torch.equal(kd, torch.ones_like(kd))


def _oracle_inputs(qb, kb):
    qc, qd = oracle.quantize_fp8(f32(qb))
    kc, kd = oracle.quantize_fp8(f32(kb))
    return qc, qd, kc, kd


def _score_error_bound(qc, qd, kc, kd, scale):
    """Per query row: scale * descales * 128 * 2^-13 * max_j max_d |q_id k_jd|."""
    q = np.abs(oracle.e4m3_decode(qc))
    kmax = np.abs(oracle.e4m3_decode(kc)).max(axis=2)            # [B,H,D]
    m = (q * kmax[:, :, None, :]).max(axis=3)                    # [B,H,Nq]
    return scale * (qd * kd)[:, :, None].astype(np.float64) * 128 * 2.0 ** -13 * m


def _gpu_fp8(qc, qd, kc, kd, vb, scale=None, out_dtype=torch.bfloat16):
    return dta.dit_attn_fwd_fp8(_dev_codes(qc), _dev_codes(kc), bits_to_torch_bf16(vb), _dev_f32(qd),
                                _dev_f32(kd), scale=scale, out_dtype=out_dtype)


@pytest.mark.parametrize("B,H,Nq,Nkv", [
    (1, 2, 128, 128),
    (2, 3, 300, 200),      # ragged query and key tiles
    (1, 1, 1, 1),
    (1, 2, 64, 1000),
    (1, 1, 257, 129),
    (1, 2, 1000, 1000),
])
def test_fp8_attention_small(B, H, Nq, Nkv):
    say("fp8 attention", B, H, Nq, Nkv)
    qb, kb, vb = datagen.small_bf16(B, H, Nq, 128, seed=Nq * 3 + Nkv, Nkv=Nkv)
    qc, qd, kc, kd = _oracle_inputs(qb, kb)
    O, L = _gpu_fp8(qc, qd, kc, kd, vb)
    Oref, Lref = oracle.attention_fp8(qc, kc, f32(vb), qd, kd)
    ma, rr = assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "fp8")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}")
    O32, L32 = _gpu_fp8(qc, qd, kc, kd, vb, out_dtype=torch.float32)
    assert_bf16_close(to_f64(O32), to_f64(L32), Oref, Lref, "fp8 f32 out")


def test_fp8_large_scores_take_the_exact_max_pass():
    """Queries scaled x3 with scale 0.5: scores far above the first key tile's
    maximum, so the fixed-reference pass overflows its bound and the workgroup
    recomputes with the exact row max."""
    say("fp8 wide score range")
    qb, kb, vb = datagen.small_bf16(1, 2, 300, 128, seed=61, Nkv=700)
    q3 = datagen.bf16_bits(f32(qb) * 3.0)
    kw = f32(kb).copy()
    kw[:, :, 650:] *= 4.0
    qc, qd, kc, kd = _oracle_inputs(q3, datagen.bf16_bits(kw))
    O, L = _gpu_fp8(qc, qd, kc, kd, vb, scale=0.5)
    Oref, Lref = oracle.attention_fp8(qc, kc, f32(vb), qd, kd, 0.5)
    assert_bf16_close(to_f64(O), None, Oref, None, "fp8 wide")
    err = np.abs(to_f64(L) - Lref)
    bound = 1e-3 + _score_error_bound(qc, qd, kc, kd, 0.5)
    say(f"  LSE max-abs {err.max():.2e} (|LSE| up to {np.abs(Lref).max():.0f}); "
        f"worst err / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


def test_fp8_exact_max_pass_in_later_units():
    """The wide-score case over 2 heads x 157 query tiles (more than the
    compute units): units past a workgroup's first take the exact-max pass
    after their queries' codes were replaced by the next unit's during the
    last key tile, and must load them again."""
    say("fp8 wide score range, later persistent units")
    qb, kb, vb = datagen.small_bf16(1, 2, 40000, 128, seed=63, Nkv=700)
    q3 = datagen.bf16_bits(f32(qb) * 3.0)
    kw = f32(kb).copy()
    kw[:, :, 650:] *= 4.0
    qc, qd, kc, kd = _oracle_inputs(q3, datagen.bf16_bits(kw))
    O, L = _gpu_fp8(qc, qd, kc, kd, vb, scale=0.5)
    rows = np.unique(np.concatenate([[0, 255, 256, 39999], datagen.sample_rows(40000, 40, 64)]))
    Oref, Lref = oracle.attention_fp8(qc, kc, f32(vb), qd, kd, 0.5, rows=rows)
    ri = torch.from_numpy(rows).cuda()
    assert_bf16_close(to_f64(O[:, :, ri]), None, Oref, None, "fp8 wide, later units")
    err = np.abs(to_f64(L[:, :, ri]) - Lref)
    bound = 1e-3 + _score_error_bound(qc[:, :, rows], qd, kc, kd, 0.5)
    assert np.all(err <= bound)


def test_fp8_quant_then_attention_and_determinism():
    say("fp8 end to end on the GPU")
    qb, kb, vb = datagen.small_bf16(1, 3, 500, 128, seed=62, Nkv=400)
    qc, qd = dta.dit_quant_fp8(bits_to_torch_bf16(qb))
    kc, kd = dta.dit_quant_fp8(bits_to_torch_bf16(kb))
    v = bits_to_torch_bf16(vb)
    O1, L1 = dta.dit_attn_fwd_fp8(qc, kc, v, qd, kd)
    O2, L2 = dta.dit_attn_fwd_fp8(qc, kc, v, qd, kd)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    oqc, oqd, okc, okd = _oracle_inputs(qb, kb)
    Oref, Lref = oracle.attention_fp8(oqc, okc, f32(vb), oqd, okd)
    assert_bf16_close(to_f64(O1), to_f64(L1), Oref, Lref, "fp8 e2e")


def test_fp8_image_share_full():
    say("fp8 image share B1 H24 N4096 D128, full compare")
    qb, kb, vb = datagen.workload_inputs("image_share")
    qc, qd, kc, kd = _oracle_inputs(qb, kb)
    O, L = _gpu_fp8(qc, qd, kc, kd, vb)
    Oref, Lref = oracle.attention_fp8(qc, kc, f32(vb), qd, kd)
    ma, rr = assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "fp8 image share")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}")


def test_fp8_ulysses_share_sampled_rows():
    say("fp8 Ulysses share B1 H10 N32768 D128, sampled rows")
    qb, kb, vb = (x[:, :10] for x in datagen.workload_inputs("ulysses_share"))
    qc, qd, kc, kd = _oracle_inputs(qb, kb)
    O, L = _gpu_fp8(qc, qd, kc, kd, vb)
    rows = datagen.sample_rows(32768, 64, 71)
    Oref, Lref = oracle.attention_fp8(qc, kc, f32(vb), qd, kd, rows=rows)
    ri = torch.from_numpy(rows).cuda()
    ma, rr = assert_bf16_close(to_f64(O[:, :, ri]), to_f64(L[:, :, ri]), Oref, Lref, "fp8 ulysses")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}")
    assert torch.isfinite(O).all()
