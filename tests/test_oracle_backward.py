"""Pins for the oracle's attention backward (dq, dk, dv, delta).

The pages give no gradient values or formulas; the oracle applies the chain
rule to the forward definition.  It is pinned by
* central finite differences of sum(dO * O) through the oracle's forward
  (itself pinned by brute force in test_oracle.py), on tiny float64 inputs;
* a library routine: torch autograd through CPU scaled_dot_product_attention
  in float64 (the routine the pull request's op-level parity compares with);
* invariants: shifting every key by w leaves the softmax unchanged, so the
  key gradients sum to zero; the rows of P sum to one, so the value
  gradients sum to the sum of dO; identical keys make P independent of q,
  so dq = 0; dO = 0 gives zero gradients; delta equals sum_j P_ij dP_ij.

The planted-mistake tests check that each mistake in a copy of the backward
is rejected by at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, B, H, Nq, Nkv, D):
    r = _rng(seed)
    q = r.standard_normal((B, H, Nq, D))
    k = r.standard_normal((B, H, Nkv, D))
    v = r.standard_normal((B, H, Nkv, D))
    do = r.standard_normal((B, H, Nq, D))
    return q, k, v, do


def _oracle_bwd(q, k, v, do, scale):
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale)
    return dq, dk, dv


# ----------------------------------------------------------------- pins
def pin_finite_differences(bwd):
    q, k, v, do = _inputs(3, 1, 2, 4, 5, 3)
    scale = 0.8
    loss = lambda q_, k_, v_: float((oracle.attention(q_, k_, v_, scale)[0] * do).sum())
    dq, dk, dv = bwd(q, k, v, do, scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            if abs(fd - g[idx]) > 1e-7 * max(1.0, abs(fd)):
                return False
    return True


def pin_torch_autograd(bwd):
    for seed, (Nq, Nkv, D), scale in [(4, (9, 13, 8), 0.3), (5, (16, 7, 16), None)]:
        q, k, v, do = _inputs(seed, 2, 2, Nq, Nkv, D)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        o.backward(torch.tensor(do))
        s = 1 / math.sqrt(D) if scale is None else scale
        got = bwd(q, k, v, do, s)
        for g, t in zip(got, (tq, tk, tv)):
            if np.abs(g - t.grad.numpy()).max() > 1e-10:
                return False
    return True


def pin_key_gradients_sum_to_zero(bwd):
    q, k, v, do = _inputs(6, 1, 3, 11, 17, 6)
    _, dk, _ = bwd(q, k, v, do, 0.5)
    return np.abs(dk.sum(axis=2)).max() < 1e-12 * max(1.0, np.abs(dk).max()) * 17


def pin_value_gradients_sum_to_dout(bwd):
    q, k, v, do = _inputs(7, 2, 2, 12, 5, 4)
    _, _, dv = bwd(q, k, v, do, 0.7)
    return np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() < 1e-12 * 12


def pin_identical_keys_give_zero_dq(bwd):
    q, k, v, do = _inputs(8, 1, 2, 6, 9, 5)
    k[:] = k[:, :, :1]
    dq, _, _ = bwd(q, k, v, do, 0.9)
    return np.abs(dq).max() < 1e-12


def pin_zero_dout(bwd):
    q, k, v, do = _inputs(9, 1, 1, 5, 6, 4)
    got = bwd(q, k, v, np.zeros_like(do), 0.5)
    return all(np.abs(g).max() == 0.0 for g in got)


BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_key_gradients_sum_to_zero,
            pin_value_gradients_sum_to_dout, pin_identical_keys_give_zero_dq, pin_zero_dout]


@pytest.mark.parametrize("pin", BWD_PINS)
def test_backward_pin(pin):
    assert pin(_oracle_bwd)


def test_delta_is_sum_of_p_times_dp():
    q, k, v, do = _inputs(10, 1, 2, 7, 9, 4)
    _, _, _, delta = oracle.attention_backward(q, k, v, do, 0.6)
    P = oracle.probabilities(q, k, 0.6)
    dP = np.einsum("bhnd,bhmd->bhnm", do, v)
    assert np.abs(delta - (P * dP).sum(-1)).max() < 1e-12


def test_row_and_key_subsets_match_full():
    q, k, v, do = _inputs(11, 1, 2, 300, 270, 8)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do)
    rows, keys = np.array([0, 5, 255, 256, 299]), np.array([0, 3, 200, 269])
    dq_r, delta_r = oracle.attention_backward_rows(q, k, v, do, rows)
    assert np.abs(dq_r - dq[:, :, rows]).max() < 1e-12
    assert np.abs(delta_r - delta[:, :, rows]).max() < 1e-12
    dk_s, dv_s = oracle.attention_backward_keys(q, k, v, do, keys)
    assert np.abs(dk_s - dk[:, :, keys]).max() < 1e-12
    assert np.abs(dv_s - dv[:, :, keys]).max() < 1e-12


# ---------------------------------------------------- planted mistakes
def _bwd_variant(q, k, v, do, scale, mut):
    """A copy of the oracle's backward with one switchable planted mistake."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            O = P @ v[b, h]
            dP = do[b, h] @ v[b, h].T
            dl = (do[b, h] * O).sum(axis=1)
            if mut == "delta_from_dp":
                dl = dP.sum(axis=1)
            dS = P * (dP - dl[:, None])
            if mut == "no_delta":
                dS = P * dP
            if mut == "ds_sign":
                dS = -dS
            sq = 1.0 if mut == "dq_no_scale" else scale
            sk = 1.0 if mut == "dk_no_scale" else scale
            dq[b, h] = sq * (dS @ k[b, h])
            dk[b, h] = sk * (dS.T @ (k[b, h] if mut == "dk_uses_k" else q[b, h]))
            dv[b, h] = (E if mut == "dv_unnormalized" else P).T @ (O if mut == "dv_uses_o" else do[b, h])
    return dq, dk, dv


BWD_MUTANTS = ["delta_from_dp", "no_delta", "ds_sign", "dq_no_scale", "dk_no_scale", "dk_uses_k",
               "dv_uses_o", "dv_unnormalized"]


def _passes(pin, fn):
    try:
        return pin(fn)
    except (ValueError, FloatingPointError, IndexError):
        return False


def test_unmutated_backward_copy_matches_oracle():
    q, k, v, do = _inputs(12, 2, 2, 10, 12, 6)
    want = _oracle_bwd(q, k, v, do, 0.4)
    got = _bwd_variant(q, k, v, do, 0.4, None)
    assert all(np.abs(a - b).max() < 1e-12 for a, b in zip(want, got))
    assert all(p(lambda *a: _bwd_variant(*a, None)) for p in BWD_PINS)


@pytest.mark.parametrize("mut", BWD_MUTANTS)
def test_pins_reject_planted_backward_mistake(mut):
    with np.errstate(all="ignore"):
        bwd = lambda q, k, v, do, s: _bwd_variant(q, k, v, do, s, mut)
        caught = [p.__name__ for p in BWD_PINS if not _passes(p, bwd)]
    assert caught, f"no pin rejects planted mistake {mut}"
