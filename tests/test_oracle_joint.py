"""Pins for the oracle's rotary embedding and joint text + image attention.

The pages name the rotary tables of the image and text tokens and the joint
attention over their concatenation, but print neither the rotation nor any
value.  The oracle's rope is pinned by
* a library routine: numpy complex multiplication of the pair x[2i] + i x[2i+1]
  by cos + i sin;
* special cases: a quarter turn (cos 0, sin 1) maps (a, b) to (-b, a) exactly;
  cos 1, sin 0 is the identity;
* invariants: unit tables keep every pair's length; with angles n * w_i the
  dot product of a turned query at m and a turned key at n depends on m - n
  only.
The joint attention is pinned by brute force (pure-Python loops, the turn as
Python complex arithmetic, math.exp / math.fsum) on tiny inputs, by the empty
text case reducing to plain attention of the turned image tokens, and by key
order not mattering (image-first concatenation gives the same rows).

round_bf16 (the reading that the turned tokens enter attention as bf16) is
pinned by the halfway cases (ties go to the even neighbour) and by agreement
with datagen's integer bit-pattern rounding of float32 values.

The planted-mistake tests check that each mistake in a copy of the oracle is
rejected by at least one pin.
"""
import math

import numpy as np
import pytest

import datagen
import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_tables(N, half, seed):
    ang = _rng(seed).uniform(-math.pi, math.pi, size=(N, half))
    return np.cos(ang), np.sin(ang)


def _joint_inputs(seed, B=1, H=2, Nt=3, Ni=5, D=4):
    r = _rng(seed)
    txt = [r.standard_normal((B, H, Nt, D)) for _ in range(3)]
    img = [r.standard_normal((B, H, Ni, D)) for _ in range(3)]
    ct, st = _unit_tables(Nt, D // 2, seed + 100)
    ci, si = _unit_tables(Ni, D // 2, seed + 200)
    return txt, img, (ct, st, ci, si)


# ----------------------------------------------------------------- pins
def pin_complex_product(rope, joint):
    x = _rng(1).standard_normal((2, 3, 7, 8))
    c, s = _unit_tables(7, 4, 2)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * (c + 1j * s)
    y = rope(x, c, s)
    return (np.abs(y[..., 0::2] - z.real).max() < 1e-14 and
            np.abs(y[..., 1::2] - z.imag).max() < 1e-14)


def pin_quarter_turn(rope, joint):
    x = _rng(3).standard_normal((1, 1, 5, 6))
    y = rope(x, np.zeros((5, 3)), np.ones((5, 3)))
    return np.array_equal(y[..., 0::2], -x[..., 1::2]) and np.array_equal(y[..., 1::2], x[..., 0::2])


def pin_identity(rope, joint):
    x = _rng(4).standard_normal((2, 2, 4, 8))
    return np.array_equal(rope(x, np.ones((4, 4)), np.zeros((4, 4))), x)


def pin_pair_lengths(rope, joint):
    x = _rng(5).standard_normal((1, 3, 9, 16))
    c, s = _unit_tables(9, 8, 6)
    y = rope(x, c, s)
    n0 = np.hypot(x[..., 0::2], x[..., 1::2])
    n1 = np.hypot(y[..., 0::2], y[..., 1::2])
    return np.abs(n0 - n1).max() < 1e-13


def pin_relative_position(rope, joint):
    N, D = 11, 8
    w = 10000.0 ** (-np.arange(D // 2) / (D // 2))
    ang = np.outer(np.arange(N), w)
    r = _rng(7)
    q = r.standard_normal((1, 1, N, D))
    k = r.standard_normal((1, 1, N, D))
    qr, kr = rope(q, np.cos(ang), np.sin(ang)), rope(k, np.cos(ang), np.sin(ang))
    for m in range(N):
        for n in range(N):
            a = np.full((N, D // 2), 0.0)
            a[m] = (m - n) * w
            qd = rope(q, np.cos(a), np.sin(a))
            if abs(qr[0, 0, m] @ kr[0, 0, n] - qd[0, 0, m] @ k[0, 0, n]) > 1e-12:
                return False
    return True


def _brute_joint(txt, img, tabs, scale):
    (qt, kt, vt), (qi, ki, vi), (ct, st, ci, si) = txt, img, tabs
    B, H, Nt, D = qt.shape
    Ni = qi.shape[2]

    def turn(vec, c, s):
        out = []
        for i in range(D // 2):
            z = complex(vec[2 * i], vec[2 * i + 1]) * complex(c[i], s[i])
            out += [z.real, z.imag]
        return out

    O = np.zeros((B, H, Nt + Ni, D))
    L = np.zeros((B, H, Nt + Ni))
    for b in range(B):
        for h in range(H):
            qs = [turn(qt[b, h, n], ct[n], st[n]) for n in range(Nt)] + \
                 [turn(qi[b, h, n], ci[n], si[n]) for n in range(Ni)]
            ks = [turn(kt[b, h, n], ct[n], st[n]) for n in range(Nt)] + \
                 [turn(ki[b, h, n], ci[n], si[n]) for n in range(Ni)]
            vs = [list(vt[b, h, n]) for n in range(Nt)] + [list(vi[b, h, n]) for n in range(Ni)]
            for i, qv in enumerate(qs):
                sc = [scale * math.fsum(a * c for a, c in zip(qv, kv)) for kv in ks]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                l = math.fsum(e)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(e[j] * vs[j][d] for j in range(len(vs))) / l
                L[b, h, i] = m + math.log(l)
    return O, L


def pin_brute_force_joint(rope, joint):
    for seed, shape in [(10, dict(Nt=3, Ni=5, D=4)), (11, dict(B=2, H=1, Nt=1, Ni=4, D=6))]:
        txt, img, tabs = _joint_inputs(seed, **shape)
        O, L = joint(*txt, *img, *tabs, scale=0.7)
        Ob, Lb = _brute_joint(txt, img, tabs, 0.7)
        if np.abs(O - Ob).max() > 1e-12 or np.abs(L - Lb).max() > 1e-12:
            return False
    return True


def pin_no_text_is_plain_attention(rope, joint):
    txt, img, (ct, st, ci, si) = _joint_inputs(12, Nt=0, Ni=9, D=8)
    O, L = joint(*txt, *img, ct, st, ci, si)
    Or, Lr = oracle.attention(rope(img[0], ci, si), rope(img[1], ci, si), img[2])
    return np.abs(O - Or).max() < 1e-13 and np.abs(L - Lr).max() < 1e-13


def pin_key_order(rope, joint):
    txt, img, (ct, st, ci, si) = _joint_inputs(13, Nt=4, Ni=6, D=8)
    O, L = joint(*txt, *img, ct, st, ci, si, scale=0.4)
    q = np.concatenate([rope(img[0], ci, si), rope(txt[0], ct, st)], axis=2)
    k = np.concatenate([rope(img[1], ci, si), rope(txt[1], ct, st)], axis=2)
    v = np.concatenate([img[2], txt[2]], axis=2)
    Or, Lr = oracle.attention(q, k, v, 0.4)
    Or = np.concatenate([Or[:, :, 6:], Or[:, :, :6]], axis=2)
    Lr = np.concatenate([Lr[:, :, 6:], Lr[:, :, :6]], axis=2)
    return np.abs(O - Or).max() < 1e-13 and np.abs(L - Lr).max() < 1e-13


PINS = [pin_complex_product, pin_quarter_turn, pin_identity, pin_pair_lengths,
        pin_relative_position, pin_brute_force_joint, pin_no_text_is_plain_attention,
        pin_key_order]


@pytest.mark.parametrize("pin", PINS)
def test_joint_pin(pin):
    assert pin(oracle.rope, oracle.joint_attention)


def test_rows_subset_and_no_tables():
    txt, img, tabs = _joint_inputs(14, Nt=5, Ni=7, D=8)
    O, L = oracle.joint_attention(*txt, *img, *tabs)
    rows = [0, 4, 5, 11]
    Or, Lr = oracle.joint_attention(*txt, *img, *tabs, rows=rows)
    assert np.abs(Or - O[:, :, rows]).max() < 1e-13 and np.abs(Lr - L[:, :, rows]).max() < 1e-13
    # no tables: plain attention over the concatenation
    O2, _ = oracle.joint_attention(*txt, *img)
    cat = [np.concatenate([t, i], axis=2) for t, i in zip(txt, img)]
    assert np.abs(O2 - oracle.attention(*cat)[0]).max() < 1e-13


def test_datagen_tables_are_unit_and_axial():
    ci, si = datagen.rope_tables_image(4, 6, 16)
    ct, st = datagen.rope_tables_text(3, 4, 6, 16)
    assert ci.shape == (24, 8) and ct.shape == (3, 8) and ci.dtype == np.float32
    assert np.abs(ci.astype(np.float64) ** 2 + si.astype(np.float64) ** 2 - 1).max() < 1e-6
    # token 0 is the grid origin: no turn; the pair 0 of the row half turns by the row index
    assert np.all(ci[0] == 1) and np.all(si[0] == 0)
    assert abs(float(si[6, 0]) - math.sin(1.0)) < 1e-7 and float(si[6, 4]) == 0.0
    assert abs(float(si[1, 4]) - math.sin(1.0)) < 1e-7 and float(si[1, 0]) == 0.0
    assert abs(float(ct[0, 0]) - math.cos(6.0)) < 1e-7


def test_round_bf16_ties_to_even():
    r = oracle.round_bf16
    # bf16 spacing at 1 is 2**-7: 1 + 2**-8 is halfway to 1 + 2**-7 (odd), so it stays 1;
    # 1 + 3 * 2**-8 is halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even)
    assert r(1 + 2 ** -8) == 1.0 and r(-(1 + 2 ** -8)) == -1.0
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7     # just past halfway
    assert r(0.0) == 0.0 and r(2.0 ** -100) == 2.0 ** -100
    assert r(255.5) == 256.0 and r(254.5) == 254.0       # spacing 1 in [128, 256)


def test_round_bf16_matches_bit_pattern_rounding():
    x = (_rng(20).standard_normal(200000) * np.exp(_rng(21).uniform(-20, 20, 200000))).astype(np.float32)
    want = datagen.bf16_to_f32(datagen.bf16_bits(x)).astype(np.float64)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.round_bf16(got), got)


# ---------------------------------------------------- planted mistakes
def _rope_variant(mut):
    def rope(x, c, s):
        x, c, s = (np.asarray(a, dtype=np.float64) for a in (x, c, s))
        if mut == "cos_sin_swapped":
            c, s = s, c
        if mut == "half_split":
            h = x.shape[-1] // 2
            a, b = x[..., :h], x[..., h:]
            return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
        a, b = x[..., 0::2], x[..., 1::2]
        y = np.empty_like(x)
        if mut == "turn_back":
            y[..., 0::2], y[..., 1::2] = a * c + b * s, b * c - a * s
        else:
            y[..., 0::2], y[..., 1::2] = a * c - b * s, a * s + b * c
        return y
    return rope


def _joint_variant(mut):
    rope = _rope_variant(mut)

    def joint(qt, kt, vt, qi, ki, vi, ct=None, st=None, ci=None, si=None, scale=None, rows=None):
        Nt = np.asarray(qt).shape[2]
        if mut == "text_uses_image_table":
            ct, st = ci[:Nt], si[:Nt]
        q = np.concatenate([rope(qt, ct, st), rope(qi, ci, si)], axis=2)
        kt_ = kt if mut == "k_not_turned" else rope(kt, ct, st)
        ki_ = ki if mut == "k_not_turned" else rope(ki, ci, si)
        k = np.concatenate([kt_, ki_], axis=2)
        if mut == "v_turned":
            v = np.concatenate([rope(vt, ct, st), rope(vi, ci, si)], axis=2)
        else:
            v = np.concatenate([vt, vi], axis=2)
        if mut == "no_text_keys":
            k, v = k[:, :, Nt:], v[:, :, Nt:]
        return oracle.attention(q, k, v, scale)
    return rope, joint


MUTANTS = ["cos_sin_swapped", "half_split", "turn_back", "text_uses_image_table",
           "k_not_turned", "v_turned", "no_text_keys"]


def _passes(pin, impl):
    try:
        return pin(*impl)
    except (ValueError, IndexError):
        return False


def test_unmutated_copy_passes_every_pin():
    impl = _joint_variant(None)
    assert all(p(*impl) for p in PINS)


@pytest.mark.parametrize("mut", MUTANTS)
def test_pins_reject_planted_mistake(mut):
    impl = _joint_variant(mut)
    caught = [p.__name__ for p in PINS if not _passes(p, impl)]
    assert caught, f"no pin rejects planted mistake {mut}"
