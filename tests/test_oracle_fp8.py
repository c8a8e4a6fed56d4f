"""Pins for the oracle's FP8 (OCP E4M3) arithmetic and FP8 attention.

The pages only say that FP8 low precision is stacked on top of the parallel
split; the format and the per-head scaling are readings.  The oracle's E4M3
functions are pinned by
* a library routine: torch's float8_e4m3fn decoding of all 256 codes, and
  its float32 -> float8_e4m3fn rounding of 10^5 in-range values (including
  the code of the float32 quotient x / descale that quantize_fp8 takes);
* special cases: every finite code round-trips; halfway values go to the
  even code, in the normal and in the subnormal range; magnitudes beyond 448
  clamp to 448;
* invariants of the per-head quantization: the largest magnitude of a head
  maps to +-448 exactly, every value is recovered within half a step,
  doubling a head doubles its scale and leaves its codes unchanged, an
  all-zero head gets scale 1 and zero codes.
attention_fp8 is attention on the decoded, rescaled values (pinned in
test_oracle.py); here: exactness of that composition and its invariance when
a factor moves between a descale and the softmax scale.
"""
import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _torch_codes(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------- pins
def pin_decode_matches_torch(f):
    c = np.arange(256, dtype=np.uint8)
    d = f["decode"](c)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.array_equal(np.isnan(d), np.isnan(t)) and np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])


def pin_codes_round_trip(f):
    c = np.arange(256, dtype=np.uint8)
    d = oracle.e4m3_decode(c)
    fin = ~np.isnan(d)
    return np.array_equal(f["encode"](d[fin]), c[fin])


def pin_round_matches_torch(f):
    r = _rng(1)
    x = (r.standard_normal(100000) * np.exp(r.uniform(-14, 7, 100000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    return np.array_equal(f["encode"](x.astype(np.float64)), _torch_codes(x))


def pin_ties_to_even(f):
    rnd = f["round"]
    cases = {1 + 1 / 16: 1.0,           # between 1 (mantissa 0) and 1.125 (1)
             1.1875: 1.25,              # between 1.125 (1) and 1.25 (2)
             2.0 ** -10: 0.0,           # half the smallest subnormal
             3 * 2.0 ** -10: 2.0 ** -8,  # between 2^-9 (1) and 2^-8 (2)
             -(1 + 1 / 16): -1.0,
             464.0: 448.0}              # between 448 and the NaN slot: clamp
    return all(rnd(np.array([k]))[0] == v for k, v in cases.items())


def pin_clamps(f):
    got = f["round"](np.array([449.0, 1e6, -500.0, 448.0, 447.0]))
    return np.array_equal(got, [448.0, 448.0, -448.0, 448.0, 448.0])


def pin_quantize_amax_and_error(f):
    x = _rng(2).standard_normal((2, 3, 50, 16)).astype(np.float32)
    codes, ds = f["quantize"](x)
    dec = oracle.e4m3_decode(codes) * ds[:, :, None, None]
    amax = np.abs(x).max(axis=(2, 3))
    at = np.abs(x) == amax[:, :, None, None]
    if not np.all(np.abs(oracle.e4m3_decode(codes[at])) == 448.0):
        return False
    # half a step: 2^-4 relative for normals, 2^-10 * descale below 2^-6 * descale
    q = np.abs(x) / ds[:, :, None, None]
    tol = np.where(q >= 2.0 ** -6, np.abs(x) * 2.0 ** -4, ds[:, :, None, None] * 2.0 ** -10)
    return np.all(np.abs(dec - x) <= tol * (1 + 1e-6))


def _halfway_quotients(d):
    """float32 x whose exact quotient x / d lies just below a halfway value M
    (between an odd code and the even code above it) while the float32
    quotient rounds onto M itself."""
    out = []
    for e in range(-3, 8):
        for m in (1, 3, 5, 7):
            M = (1 + (m + 0.5) / 8) * 2.0 ** e
            x = np.float32(M * np.float64(d))
            for _ in range(8):
                x = np.nextafter(x, np.float32(0))
            for _ in range(16):
                x = np.nextafter(x, np.float32(np.inf))
                if np.float32(x / d) == np.float32(M) and np.float64(x) / np.float64(d) < M:
                    out.append(x)
    return out


def pin_quantize_matches_torch_quotient(f):
    x = (_rng(3).standard_normal((1, 4, 64, 32)) * 3).astype(np.float32)
    # head 0: amax 6 (descale 6/448, not a power of two) and values whose
    # float32 quotient is a tie (going up to the even code) although the exact
    # one is below it, so the code depends on taking the quotient in float32
    d = np.float32(np.float32(6.0) / np.float32(448.0))
    ties = _halfway_quotients(d)[:64]
    x[0, 0] = np.clip(x[0, 0], -5.0, 5.0)
    x[0, 0, 0, 0] = 6.0
    x[0, 0, 1:3].reshape(-1)[:len(ties)] = ties
    codes, ds = f["quantize"](x)
    want = _torch_codes((torch.from_numpy(x) / torch.from_numpy(ds)[:, :, None, None]).numpy())
    return len(ties) >= 4 and np.array_equal(codes, want)


def pin_quantize_head_scaling(f):
    x = _rng(4).standard_normal((1, 2, 40, 8)).astype(np.float32)
    c1, d1 = f["quantize"](x)
    y = x.copy()
    y[:, 1] *= 2
    c2, d2 = f["quantize"](y)
    z = np.zeros_like(x)
    c3, d3 = f["quantize"](z)
    return (np.array_equal(c1, c2) and d2[0, 1] == 2 * d1[0, 1] and d2[0, 0] == d1[0, 0]
            and np.all(c3 == 0) and np.all(d3 == 1))


PINS = [pin_decode_matches_torch, pin_codes_round_trip, pin_round_matches_torch, pin_ties_to_even,
        pin_clamps, pin_quantize_amax_and_error, pin_quantize_matches_torch_quotient,
        pin_quantize_head_scaling]

ORACLE = {"decode": oracle.e4m3_decode, "round": oracle.e4m3_round, "encode": oracle.e4m3_encode,
          "quantize": oracle.quantize_fp8}


@pytest.mark.parametrize("pin", PINS)
def test_fp8_pin(pin):
    assert pin(ORACLE)


def test_attention_fp8_composition_and_scale_invariance():
    r = _rng(5)
    q, k = (r.standard_normal((1, 2, 20, 16)).astype(np.float32) for _ in range(2))
    v = r.standard_normal((1, 2, 20, 16))
    qc, qs = oracle.quantize_fp8(q)
    kc, ks = oracle.quantize_fp8(k)
    O, L = oracle.attention_fp8(qc, kc, v, qs, ks, 0.3)
    deq = lambda c, s: oracle.e4m3_decode(c) * s.astype(np.float64)[:, :, None, None]
    Or, Lr = oracle.attention(deq(qc, qs), deq(kc, ks), v, 0.3)
    assert np.abs(O - Or).max() == 0 and np.abs(L - Lr).max() == 0
    O2, L2 = oracle.attention_fp8(qc, kc, v, qs * 2, ks, 0.15)
    assert np.abs(O - O2).max() < 1e-14 and np.abs(L - L2).max() < 1e-13
    Or3, Lr3 = oracle.attention_fp8(qc, kc, v, qs, ks, 0.3, rows=[0, 7, 19])
    assert np.abs(Or3 - O[:, :, [0, 7, 19]]).max() == 0


# ---------------------------------------------------- planted mistakes
def _variant(mut):
    def rnd(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x) if mut == "no_clamp" else np.minimum(np.abs(x), 448.0)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        ulp = np.ldexp(1.0, (e - 3).astype(np.int64))
        if mut != "no_subnormals":
            ulp = np.where(a >= 2.0 ** -6, ulp, 2.0 ** -9)
        if mut == "half_away":
            r = np.floor(a / ulp + 0.5) * ulp
        else:
            r = np.round(a / ulp) * ulp
        if mut != "no_clamp":
            r = np.minimum(r, 448.0)
        return np.copysign(r, x)

    def enc(x):
        v = rnd(x)
        a = np.abs(v)
        sub = a < 2.0 ** -6
        e = np.floor(np.log2(np.where(sub, 1.0, np.where(a > 0, a, 1.0))))
        m = np.round((a / np.ldexp(1.0, e.astype(np.int64)) - 1.0) * 8.0)
        code = np.where(sub, np.round(a / 2.0 ** -9), (e + 7) * 8 + m)
        code = np.clip(code, 0, 127)
        return code.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)

    def dec(c):
        d = oracle.e4m3_decode(c)
        if mut == "decode_bias_8":
            e = (np.asarray(c, np.int64) >> 3) & 15
            d = np.where(e > 0, d / 2, d)
        return d

    def quant(x):
        x32 = np.asarray(x, dtype=np.float32)
        amax = np.abs(x32).max(axis=(2, 3))
        top = 240.0 if mut == "fnuz_max" else 448.0
        ds = np.where(amax > 0, amax / np.float32(top), np.float32(1)).astype(np.float32)
        if mut == "quotient_f64":
            quo = x32.astype(np.float64) / ds.astype(np.float64)[:, :, None, None]
        else:
            quo = (x32 / ds[:, :, None, None]).astype(np.float64)
        return enc(quo), ds
    return {"decode": dec, "round": rnd, "encode": enc, "quantize": quant}


MUTANTS = ["no_clamp", "no_subnormals", "half_away", "decode_bias_8", "fnuz_max", "quotient_f64"]


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
