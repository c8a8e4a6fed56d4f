"""GPU parity of the power-of-two-scaled FP8 path against the fp64 oracle.

* dit_quant_fp8_qk_mx is bit-exact: codes and descales equal
  oracle.quantize_fp8_mx (q times the float32 softmax constant, power-of-two
  descales, exact quotients, E4M3 nearest-even).
* dit_attn_fwd_fp8_mx takes codes and descales made by the oracle and is held
  to the bf16 attention bars against oracle.attention_fp8_mx on the same codes
  (O max-abs 2e-2, rel-RMS 1e-2; LSE max-abs 1e-3), as dit_attn_fwd_fp8 is:
  the same fp8 product, whose sums keep each product only down to 2^-13 of the
  largest one, so where scores are far from unit size the LSE is held to 1e-3
  plus ln 2 * descales * 128 * 2^-13 * max_d |q_d k_d| (codes; base-2 scores).
"""
import math
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


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def _gpu(qc, kc, vb, qd, kd, out_dtype=torch.bfloat16):
    return dta.dit_attn_fwd_fp8_mx(_dev(qc), _dev(kc), bits_to_torch_bf16(vb),
                                   _dev(qd.astype(np.float32)), _dev(kd.astype(np.float32)),
                                   out_dtype=out_dtype)


def _score_error_bound(qc, qd, kc, kd):
    """Per query row, natural-log units: ln 2 * descales * 128 * 2^-13 * max_j max_d |q_id k_jd|."""
    q = np.abs(oracle.e4m3_decode(qc))
    kmax = np.abs(oracle.e4m3_decode(kc)).max(axis=2)
    m = (q * kmax[:, :, None, :]).max(axis=3)
    return math.log(2.0) * (qd.astype(np.float64) * kd)[:, :, None] * 128 * 2.0 ** -13 * m


@pytest.mark.parametrize("B,H,Nq,Nkv,D,qmul,scale", [
    (1, 2, 64, 64, 128, 1.0, None),
    (2, 3, 37, 53, 64, 40.0, 0.3),     # large magnitudes, another head dim
    (1, 1, 1, 1, 32, 1.0, None),
    (1, 4, 300, 200, 128, 1e-3, 2.0),  # small magnitudes: subnormal codes
    (1, 2, 100, 0, 128, 1.0, None),    # empty key tensor: descale 1
])
def test_quant_mx_bit_exact(B, H, Nq, Nkv, D, qmul, scale):
    say("quant mx", B, H, Nq, Nkv, D, qmul, scale)
    qb, kb, _ = datagen.small_bf16(B, H, Nq, D, seed=Nq + 7 * Nkv, Nkv=max(Nkv, 1))
    qb = datagen.bf16_bits(f32(qb) * qmul)
    kb = kb[:, :, :Nkv].copy()
    if B * H > 1:  # an all-zero head of q
        qb[0, 0] = 0
    qc, kc, qd, kd = dta.dit_quant_fp8_qk_mx(bits_to_torch_bf16(qb), bits_to_torch_bf16(kb), scale)
    wqc, wkc, wqd, wkd = oracle.quantize_fp8_mx(f32(qb), f32(kb), scale)
    assert np.array_equal(qd.cpu().numpy(), wqd) and np.array_equal(kd.cpu().numpy(), wkd)
    assert np.array_equal(qc.cpu().numpy(), wqc) and np.array_equal(kc.cpu().numpy(), wkc)


@pytest.mark.parametrize("B,H,Nq,Nkv", [
    (1, 2, 128, 128),
    (2, 3, 300, 200),
    (1, 1, 1, 1),
    (1, 2, 64, 1000),
    (1, 1, 257, 129),
    (1, 2, 1000, 1000),
])
def test_fp8_mx_attention_small(B, H, Nq, Nkv):
    say("fp8 mx attention", B, H, Nq, Nkv)
    qb, kb, vb = datagen.small_bf16(B, H, Nq, 128, seed=Nq * 5 + Nkv, Nkv=Nkv)
    qc, kc, qd, kd = oracle.quantize_fp8_mx(f32(qb), f32(kb))
    O, L = _gpu(qc, kc, vb, qd, kd)
    Oref, Lref = oracle.attention_fp8_mx(qc, kc, f32(vb), qd, kd)
    ma, rr = assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "fp8 mx")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}")
    O32, L32 = _gpu(qc, kc, vb, qd, kd, out_dtype=torch.float32)
    assert_bf16_close(to_f64(O32), to_f64(L32), Oref, Lref, "fp8 mx f32 out")


@pytest.mark.parametrize("Nq", [300, 40000])
def test_fp8_mx_wide_scores_take_the_exact_max_pass(Nq):
    """Queries x3 with scale 0.5 and the last keys x4: scores far above the
    first key tile's maximum, so the fixed-reference pass overflows its bound
    and the workgroup recomputes with the exact row max (with 40000 queries,
    in units past a workgroup's first)."""
    say("fp8 mx wide score range", Nq)
    qb, kb, vb = datagen.small_bf16(1, 2, Nq, 128, seed=64 + Nq % 7, Nkv=700)
    kw = f32(kb).copy()
    kw[:, :, 650:] *= 4.0
    qc, kc, qd, kd = oracle.quantize_fp8_mx(f32(qb) * 3.0, kw, 0.5)
    O, L = _gpu(qc, kc, vb, qd, kd)
    rows = np.arange(Nq) if Nq <= 300 else np.unique(
        np.concatenate([[0, 255, 256, Nq - 1], datagen.sample_rows(Nq, 40, 65)]))
    Oref, Lref = oracle.attention_fp8_mx(qc, kc, f32(vb), qd, kd, rows=rows)
    ri = torch.from_numpy(rows).cuda()
    assert_bf16_close(to_f64(O[:, :, ri]), None, Oref, None, "fp8 mx wide")
    err = np.abs(to_f64(L[:, :, ri]) - Lref)
    bound = 1e-3 + _score_error_bound(qc[:, :, rows], qd, kc, kd)
    say(f"  LSE max-abs {err.max():.2e} (|LSE| up to {np.abs(Lref).max():.0f}); "
        f"worst err / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


def test_fp8_mx_quant_then_attention_and_determinism():
    say("fp8 mx end to end on the GPU")
    qb, kb, vb = datagen.small_bf16(1, 3, 500, 128, seed=66, Nkv=400)
    qc, kc, qd, kd = dta.dit_quant_fp8_qk_mx(bits_to_torch_bf16(qb), bits_to_torch_bf16(kb))
    v = bits_to_torch_bf16(vb)
    O1, L1 = dta.dit_attn_fwd_fp8_mx(qc, kc, v, qd, kd)
    O2, L2 = dta.dit_attn_fwd_fp8_mx(qc, kc, v, qd, kd)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    wqc, wkc, wqd, wkd = oracle.quantize_fp8_mx(f32(qb), f32(kb))
    Oref, Lref = oracle.attention_fp8_mx(wqc, wkc, f32(vb), wqd, wkd)
    assert_bf16_close(to_f64(O1), to_f64(L1), Oref, Lref, "fp8 mx e2e")


def test_fp8_mx_image_share_full():
    say("fp8 mx image share B1 H24 N4096 D128, full compare")
    qb, kb, vb = datagen.workload_inputs("image_share")
    qc, kc, qd, kd = oracle.quantize_fp8_mx(f32(qb), f32(kb))
    O, L = _gpu(qc, kc, vb, qd, kd)
    Oref, Lref = oracle.attention_fp8_mx(qc, kc, f32(vb), qd, kd)
    ma, rr = assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, "fp8 mx image share")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}")


def test_fp8_mx_ulysses_share_sampled_rows():
    say("fp8 mx Ulysses share B1 H10 N32768 D128, sampled rows")
    qb, kb, vb = (x[:, :10] for x in datagen.workload_inputs("ulysses_share"))
    qc, kc, qd, kd = dta.dit_quant_fp8_qk_mx(bits_to_torch_bf16(qb), bits_to_torch_bf16(kb))
    wqc, wkc, wqd, wkd = oracle.quantize_fp8_mx(f32(qb), f32(kb))
    assert np.array_equal(qc.cpu().numpy(), wqc) and np.array_equal(kd.cpu().numpy(), wkd)
    O, L = dta.dit_attn_fwd_fp8_mx(qc, kc, bits_to_torch_bf16(vb), qd, kd)
    rows = datagen.sample_rows(32768, 64, 72)
    Oref, Lref = oracle.attention_fp8_mx(wqc, wkc, f32(vb), wqd, wkd, rows=rows)
    ri = torch.from_numpy(rows).cuda()
    ma, rr = assert_bf16_close(to_f64(O[:, :, ri]), to_f64(L[:, :, ri]), Oref, Lref, "fp8 mx ulysses")
    say(f"  O max-abs {ma:.2e} rel-RMS {rr:.2e}")
    assert torch.isfinite(O).all()
