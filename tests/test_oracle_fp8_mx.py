"""Pins for the oracle's power-of-two-scaled FP8 path (quantize_fp8_mx,
attention_fp8_mx, pow2_descale).

The reading (oracle/ref.py): per (b, h) a power-of-two scale, the smallest
that brings the head's largest magnitude within E4M3's 448; the queries are
first multiplied in float32 by scale * log2(e), so the scaled products are the
scores in base 2.  Pinned by
* a library routine: torch's float32 -> float8_e4m3fn conversion of the
  float32 quotients, and torch's scaled_dot_product_attention in float64 on
  inputs that the quantizer keeps exact;
* closed forms: single-channel queries and keys whose base-2 scores are
  integers, so that every softmax weight and the LSE are exact fractions and
  logarithms of powers of two;
* invariants: every scale is a power of two, the smallest one that keeps the
  head within 448; an all-zero head gets scale 1; doubling a head of k
  doubles its scale and keeps its codes.
Planted mistakes in a copy (natural exponent, missing log2 e, amax/448 scale,
a scale one power too large, scores without the scales) each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _torch_codes(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _exact_inputs(seed, B=1, H=3, N=24, D=16):
    """q, k whose quantization is exact under the reading: k in E4M3's grid at
    a power-of-two scale, and q chosen so that q * c0 (c0 the float32 softmax
    constant at scale 1/log2(e) rounded) lands on the grid too (q = g / c0 with
    g on the grid and the division exact enough that float32(q * c0) == g)."""
    r = _rng(seed)
    grid = oracle.e4m3_decode(np.arange(0, 0x78, dtype=np.uint8))  # non-negative finite codes < 256
    grid = grid[(grid >= 0.25) & (grid <= 6)]
    k = (r.choice(grid, (B, H, N, D)) * r.choice([-1.0, 1.0], (B, H, N, D))).astype(np.float32)
    g = (r.choice(grid, (B, H, N, D)) * r.choice([-1.0, 1.0], (B, H, N, D))).astype(np.float32)
    return g, k


# ----------------------------------------------------------------- pins
def pin_descale_minimal_power_of_two(f):
    a = np.concatenate([np.array([0.0, 448.0, 449.0, 224.0, 1e-42, 3e38], np.float32),
                        (np.exp(_rng(1).uniform(-80, 80, 2000))).astype(np.float32)])
    d = f["pow2"](a).astype(np.float64)
    m, _ = np.frexp(d)
    a64 = a.astype(np.float64)
    pos = a64 > 0
    return (np.all(m == 0.5)                                            # powers of two
            and np.all(d[~pos] == 1.0)
            and np.all(a64[pos] <= 448.0 * d[pos])                      # within 448
            and np.all((a64[pos] > 224.0 * d[pos]) | (d[pos] == 2.0 ** -126)))  # smallest


def pin_codes_match_torch(f):
    r = _rng(2)
    q = (r.standard_normal((2, 3, 40, 32)) * np.exp(r.uniform(-3, 3, (2, 3, 1, 1)))).astype(np.float32)
    k = (r.standard_normal((2, 3, 56, 32)) * np.exp(r.uniform(-3, 3, (2, 3, 1, 1)))).astype(np.float32)
    scale = 0.2
    qc, kc, qd, kd = f["quant"](q, k, scale)
    c0 = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    wq = _torch_codes((q * c0) / qd[:, :, None, None])
    wk = _torch_codes(k / kd[:, :, None, None])
    return np.array_equal(qc, wq) and np.array_equal(kc, wk)


def pin_head_scaling_and_zero_head(f):
    r = _rng(3)
    q, k = (r.standard_normal((1, 2, 16, 8)).astype(np.float32) for _ in range(2))
    qc, kc, qd, kd = f["quant"](q, k, 0.5)
    k2 = k.copy()
    k2[:, 1] *= 2
    qc2, kc2, qd2, kd2 = f["quant"](q, k2, 0.5)
    z = np.zeros_like(k)
    qc3, kc3, qd3, kd3 = f["quant"](z, z, 0.5)
    return (np.array_equal(kc, kc2) and kd2[0, 1] == 2 * kd[0, 1] and kd2[0, 0] == kd[0, 0]
            and np.array_equal(qc, qc2) and np.all(kc3 == 0) and np.all(qc3 == 0)
            and np.all(qd3 == 1) and np.all(kd3 == 1))


def pin_closed_form_base2(f):
    # one channel: q = 1 (code 0x38), k_j = a_j (integers), scales 1: base-2
    # scores a_j, weights 2^a_j / sum, LSE = ln 2 * log2 sum 2^a_j
    a = np.array([0.0, 1.0, 3.0, -2.0, 2.0, 1.0])
    qc = np.zeros((1, 1, 1, 2), np.uint8)
    qc[..., 0] = oracle.e4m3_encode(np.array([1.0]))[0]
    kc = np.zeros((1, 1, len(a), 2), np.uint8)
    kc[0, 0, :, 0] = oracle.e4m3_encode(a)
    v = np.zeros((1, 1, len(a), 2))
    v[0, 0, :, 0] = np.arange(len(a))
    v[0, 0, :, 1] = 1.0
    one = np.ones((1, 1), np.float32)
    O, L = f["attn"](qc, kc, v, one, one)
    w = 2.0 ** a / (2.0 ** a).sum()
    return (abs(O[0, 0, 0, 0] - (w * np.arange(len(a))).sum()) < 1e-14
            and abs(O[0, 0, 0, 1] - 1.0) < 1e-14
            and abs(L[0, 0, 0] - math.log(2.0) * math.log2((2.0 ** a).sum())) < 1e-14)


def pin_descales_enter_scores(f):
    # the same codes with scales (2, 1/4) give base-2 scores halved
    r = _rng(4)
    qc = oracle.e4m3_encode(r.standard_normal((1, 2, 5, 8)))
    kc = oracle.e4m3_encode(r.standard_normal((1, 2, 7, 8)))
    v = r.standard_normal((1, 2, 7, 8))
    one = np.ones((1, 2), np.float32)
    O1, L1 = f["attn"](qc, kc, v, one * 2, one / 4)
    q = oracle.e4m3_decode(qc)
    k = oracle.e4m3_decode(kc)
    O2, L2 = oracle.attention(q, k, v, scale=math.log(2.0) / 2)
    return np.abs(O1 - O2).max() < 1e-12 and np.abs(L1 - L2).max() < 1e-12


def pin_end_to_end_exact_inputs(f):
    # inputs the quantizer keeps exact: the FP8 path is then torch's fp64 SDPA
    scale = 1.0 / float(np.float32(1.4426950408889634))
    g, k = _exact_inputs(5)
    c0 = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    q = g.astype(np.float64) / np.float64(c0)
    q32 = q.astype(np.float32)
    if not np.array_equal(q32 * c0, g):
        return False
    v = _rng(6).standard_normal(k.shape)
    qc, kc, qd, kd = f["quant"](q32, k, scale)
    O, L = f["attn"](qc, kc, v, qd, kd)
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    want = torch.nn.functional.scaled_dot_product_attention(t(q32), t(k), t(v), scale=scale).numpy()
    s = np.einsum("bhid,bhjd->bhij", q32.astype(np.float64), k.astype(np.float64)) * scale
    lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    return np.abs(O - want).max() < 1e-6 and np.abs(L - lse).max() < 1e-6


PINS = [pin_descale_minimal_power_of_two, pin_codes_match_torch, pin_head_scaling_and_zero_head,
        pin_closed_form_base2, pin_descales_enter_scores, pin_end_to_end_exact_inputs]

ORACLE = {"pow2": oracle.pow2_descale, "quant": oracle.quantize_fp8_mx, "attn": oracle.attention_fp8_mx}


@pytest.mark.parametrize("pin", PINS)
def test_fp8_mx_pin(pin):
    assert pin(ORACLE)


def test_rows_subset():
    r = _rng(7)
    q, k = (r.standard_normal((1, 2, 12, 16)).astype(np.float32) for _ in range(2))
    v = r.standard_normal((1, 2, 12, 16))
    qc, kc, qd, kd = oracle.quantize_fp8_mx(q, k)
    O, L = oracle.attention_fp8_mx(qc, kc, v, qd, kd)
    O2, L2 = oracle.attention_fp8_mx(qc, kc, v, qd, kd, rows=[0, 5, 11])
    assert np.abs(O2 - O[:, :, [0, 5, 11]]).max() == 0 and np.abs(L2 - L[:, :, [0, 5, 11]]).max() == 0


# ---------------------------------------------------- planted mistakes
def _variant(mut):
    def pow2(amax):
        if mut == "amax_scale":
            a = np.asarray(amax, np.float32)
            return np.where(a > 0, a / np.float32(448), np.float32(1)).astype(np.float32)
        d = oracle.pow2_descale(amax)
        return (d * 2).astype(np.float32) if mut == "one_power_up" else d

    def quant(q, k, scale=None):
        q32, k32 = np.asarray(q, np.float32), np.asarray(k, np.float32)
        scale = oracle.default_scale(q32.shape[-1]) if scale is None else scale
        c0 = np.float32(scale) if mut == "no_log2e" else np.float32(np.float32(scale) * oracle.LOG2E_F32)
        out = []
        for x in (q32 * c0, k32):
            d = pow2(np.abs(x).max(axis=(2, 3)))
            out.append((oracle.e4m3_encode(x.astype(np.float64) / d.astype(np.float64)[:, :, None, None]), d))
        return out[0][0], out[1][0], out[0][1], out[1][1]

    def attn(qc, kc, v, qd, kd, rows=None):
        if mut == "natural_exp":
            return oracle.attention_fp8(qc, kc, v, qd, kd, scale=1.0, rows=rows)
        if mut == "no_descales":
            one = np.ones_like(np.asarray(qd))
            return oracle.attention_fp8_mx(qc, kc, v, one, one, rows)
        return oracle.attention_fp8_mx(qc, kc, v, qd, kd, rows)
    return {"pow2": pow2, "quant": quant, "attn": attn}


MUTANTS = ["amax_scale", "one_power_up", "no_log2e", "natural_exp", "no_descales"]


def _passes(pin, impl):
    try:
        with np.errstate(all="ignore"):
            return pin(impl)
    except (ValueError, IndexError, OverflowError):
        return False


def test_unmutated_copy_passes_every_pin():
    assert all(p(_variant(None)) for p in PINS)


@pytest.mark.parametrize("mut", MUTANTS)
def test_pins_reject_planted_mistake(mut):
    caught = [p.__name__ for p in PINS if not _passes(p, _variant(mut))]
    assert caught, f"no pin rejects planted mistake {mut}"
