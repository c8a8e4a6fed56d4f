"""Pins for the CPU oracle: what fixes its values other than itself.

The pages print no attention values, so the oracle is pinned by
* brute force on tiny inputs (pure-Python loops, math.exp / math.fsum, no
  max subtraction) -- a different evaluation order of the definition;
* closed forms (K = 0 gives LSE = ln Nkv and O = mean of the V rows);
* invariants (softmax rows sum to one; uniform V returns V; permuting keys
  with their values changes nothing; shifting every key by w shifts LSE by
  scale*q.w and leaves O unchanged; a dominant key returns its value row);
* a library routine: torch's CPU scaled_dot_product_attention in float64,
  the routine the handbook's simulation uses as its reference;
* the handbook's printed outcome of its four-card Ulysses simulation
  (tests/golden/ulysses_simulation.json), on its own seed-0 data;
* the exact split-then-merge identity of the ring paragraph.

The last test plants mistakes in a copy of the oracle's attention and merge
and checks that at least one pin rejects each of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import datagen
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.default_rng(seed)


def _brute(q, k, v, scale):
    """Attention by pure-Python loops straight from the definition."""
    B, H, Nq, D = q.shape
    Nkv, Dv = k.shape[2], v.shape[3]
    O = np.zeros((B, H, Nq, Dv))
    L = np.zeros((B, H, Nq))
    for b, h, i in itertools.product(range(B), range(H), range(Nq)):
        s = [scale * math.fsum(float(q[b, h, i, d]) * float(k[b, h, j, d]) for d in range(D))
             for j in range(Nkv)]
        e = [math.exp(x) for x in s]
        z = math.fsum(e)
        for c in range(Dv):
            O[b, h, i, c] = math.fsum(e[j] * float(v[b, h, j, c]) for j in range(Nkv)) / z
        L[b, h, i] = math.log(z)
    return O, L


# ----------------------------------------------------------------- pins
def pin_brute_force(attn):
    ok = True
    for seed, (Nq, Nkv, D), scale in [(0, (5, 7, 3), None), (1, (4, 9, 8), 0.7), (2, (6, 6, 4), 1.9)]:
        r = _rng(seed)
        q = r.standard_normal((1, 2, Nq, D))
        k = r.standard_normal((1, 2, Nkv, D))
        v = r.standard_normal((1, 2, Nkv, D + 1))
        sc = 1 / math.sqrt(D) if scale is None else scale
        O, L = attn(q, k, v, scale)
        Ob, Lb = _brute(q, k, v, sc)
        ok &= np.abs(O - Ob).max() <= 1e-12 and np.abs(L - Lb).max() <= 1e-12
    return bool(ok)


def pin_k_zero(attn):
    r = _rng(3)
    q = r.standard_normal((1, 2, 6, 8))
    k = np.zeros((1, 2, 11, 8))
    v = r.standard_normal((1, 2, 11, 8))
    O, L = attn(q, k, v, None)
    return bool(np.abs(L - math.log(11)).max() <= 1e-14
                and np.abs(O - v.mean(axis=2, keepdims=True)).max() <= 1e-14)


def pin_rows_sum_to_one(attn):
    # With V = I (D = Nkv) the output rows are the softmax rows themselves.
    r = _rng(4)
    Nkv = 12
    q = r.standard_normal((1, 1, 7, 5)) * 2
    k = r.standard_normal((1, 1, Nkv, 5)) * 2
    v = np.eye(Nkv)[None, None]
    O, _ = attn(q, k, v, None)
    return bool(np.abs(O.sum(-1) - 1).max() <= 1e-12 and O.min() >= 0)


def pin_uniform_v(attn):
    r = _rng(5)
    q = r.standard_normal((1, 2, 9, 16))
    k = r.standard_normal((1, 2, 13, 16)) * 3
    u = r.standard_normal(16)
    v = np.broadcast_to(u, (1, 2, 13, 16)).copy()
    O, _ = attn(q, k, v, None)
    return bool(np.abs(O - u).max() <= 1e-12)


def pin_kv_permutation(attn):
    r = _rng(6)
    q = r.standard_normal((1, 2, 8, 16))
    k = r.standard_normal((1, 2, 40, 16))
    v = r.standard_normal((1, 2, 40, 16))
    perm = r.permutation(40)
    O1, L1 = attn(q, k, v, None)
    O2, L2 = attn(q, k[:, :, perm], v[:, :, perm], None)
    return bool(np.abs(O1 - O2).max() <= 1e-12 and np.abs(L1 - L2).max() <= 1e-12)


def pin_key_shift(attn):
    r = _rng(7)
    D = 16
    q = r.standard_normal((1, 2, 8, D))
    k = r.standard_normal((1, 2, 30, D))
    v = r.standard_normal((1, 2, 30, D))
    w = r.standard_normal(D) * 2
    scale = 1 / math.sqrt(D)
    O1, L1 = attn(q, k, v, None)
    O2, L2 = attn(q, k + w, v, None)
    return bool(np.abs(O1 - O2).max() <= 1e-11
                and np.abs((L2 - L1) - scale * (q @ w)).max() <= 1e-11)


def pin_dominant_key(attn):
    # One key aligned with the query at a huge score: O = its value row,
    # LSE = its score, without overflow.
    # A second, ordinary query row in the same head must stay exact: the
    # stabilising max is per row, not shared.
    D, Nkv = 8, 10
    r = _rng(8)
    q = np.zeros((1, 1, 2, D)); q[0, 0, 0, 0] = 100.0
    q[0, 0, 1, 1:] = r.standard_normal(D - 1)
    k = np.zeros((1, 1, Nkv, D)); k[0, 0, 3, 0] = 100.0
    k[0, 0, :, 1:] = r.standard_normal((Nkv, D - 1))
    v = r.standard_normal((1, 1, Nkv, D))
    O, L = attn(q, k, v, 1.0)
    Ob, Lb = _brute(q[:, :, 1:], k, v, 1.0)
    return bool(np.isfinite(O).all() and np.abs(O[0, 0, 0] - v[0, 0, 3]).max() <= 1e-12
                and abs(L[0, 0, 0] - 1e4) <= 1e-9
                and np.abs(O[:, :, 1:] - Ob).max() <= 1e-12 and np.abs(L[:, :, 1:] - Lb).max() <= 1e-12)


def pin_torch_sdpa(attn):
    # The handbook's reference routine, in float64 on the CPU; N=300 spans
    # more than one 256-row block of the oracle.
    ok = True
    for seed, (B, H, N, D) in [(9, (1, 3, 300, 64)), (10, (2, 2, 77, 32))]:
        r = _rng(seed)
        q, k, v = (r.standard_normal((B, H, N, D)) for _ in range(3))
        O, _ = attn(q, k, v, None)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x) for x in (q, k, v))).numpy()
        ok &= np.abs(O - ref).max() <= 1e-10
    return bool(ok)


ATTN_PINS = [pin_brute_force, pin_k_zero, pin_rows_sum_to_one, pin_uniform_v,
             pin_kv_permutation, pin_key_shift, pin_dominant_key, pin_torch_sdpa]


def pin_merge_split_equals_unsplit(attn, merge):
    r = _rng(11)
    q = r.standard_normal((1, 2, 33, 16))
    k = r.standard_normal((1, 2, 48, 16)) * 1.5
    v = r.standard_normal((1, 2, 48, 16))
    O, L = attn(q, k, v, None)
    ok = True
    for nblk in (1, 2, 3, 4):
        parts = [attn(q, kb, vb, None) for kb, vb in oracle.split_kv(k, v, nblk)]
        Om, Lm = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        ok &= np.abs(Om - O).max() <= 1e-13 and np.abs(Lm - L).max() <= 1e-13
    return bool(ok)


def pin_merge_equal_lse(merge):
    r = _rng(12)
    o = r.standard_normal((3, 1, 2, 5, 4))
    lse = np.broadcast_to(r.standard_normal((1, 1, 2, 5)), (3, 1, 2, 5)).copy()
    Om, Lm = merge(o, lse)
    return bool(np.abs(Om - o.mean(0)).max() <= 1e-14
                and np.abs(Lm - (lse[0] + math.log(3))).max() <= 1e-14)


def pin_merge_identity_and_order(merge):
    r = _rng(13)
    o = r.standard_normal((1, 1, 2, 5, 4))
    lse = r.standard_normal((1, 1, 2, 5))
    O1, L1 = merge(o, lse)
    ok = np.array_equal(O1, o[0]) and np.array_equal(L1, lse[0])
    o4 = r.standard_normal((4, 1, 2, 5, 4))
    l4 = r.standard_normal((4, 1, 2, 5)) * 3
    Oa, La = merge(o4, l4)
    p = [2, 0, 3, 1]
    Ob, Lb = merge(o4[p], l4[p])
    ok &= np.abs(Oa - Ob).max() <= 1e-14 and np.abs(La - Lb).max() <= 1e-14
    return bool(ok)


MERGE_PINS = [pin_merge_equal_lse, pin_merge_identity_and_order]


# ----------------------------------------------------------------- tests
@pytest.mark.parametrize("pin", ATTN_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    assert pin(oracle.attention)


def test_merge_split_equals_unsplit():
    assert pin_merge_split_equals_unsplit(oracle.attention, oracle.merge)


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda f: f.__name__)
def test_merge_pin(pin):
    assert pin(oracle.merge)


def test_merge_all_minus_inf_is_zero_not_nan():
    o = np.ones((3, 1, 1, 2, 4))
    lse = np.full((3, 1, 1, 2), -np.inf)
    lse[1, 0, 0, 1] = 0.5
    O, L = oracle.merge(o, lse)
    assert np.array_equal(O[0, 0, 0], np.zeros(4)) and L[0, 0, 0] == -np.inf
    assert np.array_equal(O[0, 0, 1], np.ones(4)) and L[0, 0, 1] == 0.5


def test_ring_attention_equals_attention():
    r = _rng(14)
    q, k, v = (r.standard_normal((1, 3, 64, 32)) for _ in range(3))
    O, L = oracle.attention(q, k, v)
    Or, Lr = oracle.ring_attention(q, k, v, 4)
    assert np.abs(O - Or).max() <= 1e-13 and np.abs(L - Lr).max() <= 1e-13


def test_attention_rows_matches_full():
    r = _rng(15)
    q, k, v = (r.standard_normal((1, 2, 50, 16)) for _ in range(3))
    rows = np.array([0, 7, 49])
    O, L = oracle.attention(q, k, v)
    Os, Ls = oracle.attention_rows(q, k, v, rows)
    assert np.array_equal(O[:, :, rows], Os) and np.array_equal(L[:, :, rows], Ls)


def test_probabilities_match_attention_with_identity_v():
    r = _rng(16)
    q, k = r.standard_normal((1, 2, 5, 4)), r.standard_normal((1, 2, 6, 4))
    O, _ = oracle.attention(q, k, np.broadcast_to(np.eye(6), (1, 2, 6, 6)))
    assert np.abs(O - oracle.probabilities(q, k)).max() <= 1e-14


# ---------------------------------------------------- Ulysses permutes
def _seq2head_by_index(shards):
    """out[r][b,h',s*N/P+n,d] = in[s][b,r*H/P+h',n,d], element by element."""
    P, B, H, Ns, D = shards.shape
    g = H // P
    out = np.empty((P, B, g, Ns * P, D), dtype=shards.dtype)
    for r, s, b, hh, n in itertools.product(range(P), range(P), range(B), range(g), range(Ns)):
        out[r, b, hh, s * Ns + n] = shards[s, b, r * g + hh, n]
    return out


def _shard_by_index(x, P):
    """out[r][b,h,i,d] = x[b,h,r*N/P+i,d], element by element."""
    B, H, N, D = x.shape
    n = N // P
    out = np.empty((P, B, H, n, D), dtype=x.dtype)
    for r, b, h, i in itertools.product(range(P), range(B), range(H), range(n)):
        out[r, b, h, i] = x[b, h, r * n + i]
    return out


def _head2seq_by_index(groups):
    """out[s][b,r*H/P+h',i,d] = in[r][b,h',s*N/P+i,d], element by element."""
    P, B, g, N, D = groups.shape
    n = N // P
    out = np.empty((P, B, g * P, n, D), dtype=groups.dtype)
    for s, r, b, hh, i in itertools.product(range(P), range(P), range(B), range(g), range(n)):
        out[s, b, r * g + hh, i] = groups[r, b, hh, s * n + i]
    return out


@pytest.mark.parametrize("P,B,H,N,D", [(4, 1, 8, 16, 3), (2, 2, 6, 10, 4), (3, 1, 3, 9, 2), (1, 1, 2, 4, 2),
                                       (3, 2, 6, 12, 1)])
def test_seq2head_index_map(P, B, H, N, D):
    x = np.arange(B * H * N * D, dtype=np.int64).reshape(B, H, N, D)
    shards = oracle.shard_tokens(x, P)
    assert np.array_equal(shards, _shard_by_index(x, P))
    out = oracle.seq2head(shards)
    assert np.array_equal(out, _seq2head_by_index(shards))
    # head2seq checked on its own map (distinct values everywhere), not only
    # as the inverse of seq2head
    y = (np.arange(P * B * (H // P) * N * D, dtype=np.int64) * 7 + 3).reshape(P, B, H // P, N, D)
    assert np.array_equal(oracle.head2seq(y), _head2seq_by_index(y))
    back = oracle.head2seq(out)
    assert np.array_equal(back, shards)
    assert np.array_equal(oracle.unshard_tokens(back), x)


def test_permute_pins_reject_planted_mistakes():
    """Plausible slips in the exchanges (rank axes swapped, group and rank
    swapped in the head index, token slices joined in reverse) each fail the
    element-by-element maps."""
    P, B, H, N, D = 3, 2, 6, 12, 2
    x = np.arange(B * H * N * D, dtype=np.int64).reshape(B, H, N, D)
    shards = oracle.shard_tokens(x, P)
    g, n = H // P, N // P

    def rank_axes_swapped(sh):        # out[s] gets group s of rank r's slice at r*n
        t = sh.reshape(P, B, P, g, n, D).transpose(0, 1, 3, 2, 4, 5)
        return np.ascontiguousarray(t).reshape(P, B, g, P * n, D)

    def head_index_swapped(sh):       # head split as h'*P + r instead of r*g + h'
        t = sh.reshape(P, B, g, P, n, D).transpose(3, 1, 2, 0, 4, 5)
        return np.ascontiguousarray(t).reshape(P, B, g, P * n, D)

    def slices_reversed(sh):
        return oracle.seq2head(sh[::-1])

    want = _seq2head_by_index(shards)
    for bad in (rank_axes_swapped, head_index_swapped, slices_reversed):
        assert not np.array_equal(bad(shards), want), bad.__name__


def test_permute_divisibility_errors():
    x = np.zeros((1, 6, 10, 2))
    with pytest.raises(ValueError):
        oracle.shard_tokens(x, 4)           # N % P != 0
    with pytest.raises(ValueError):
        oracle.seq2head(oracle.shard_tokens(x, 5))  # H % P != 0


def test_handbook_simulation_outcome():
    """The handbook's four-card simulation on its own seed-0 data prints True
    (atol 1e-5 against unsharded SDPA) and about 72 KB sent per card."""
    gold = json.load(open(os.path.join(HERE, "golden", "ulysses_simulation.json")))
    s = gold["setup"]
    q, k, v = datagen.tiny_f32()
    assert q.shape == (s["B"], s["H"], s["N"], s["D"])
    full = oracle.ulysses_attention(q, k, v, s["P"])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    close = bool(np.allclose(full, ref, atol=gold["printed"]["reassembled_equals_unsharded_atol"], rtol=1e-5))
    assert close == gold["printed"]["reassembled_equals_unsharded"]
    # heads are computed independently, so the round trip is exact in the oracle
    assert np.array_equal(full, oracle.attention(q, k, v)[0])
    sent = oracle.ulysses_send_bytes_per_rank(s["B"], s["H"], s["N"], s["D"], s["P"], elem_bytes=2)
    assert round(sent / 2 ** 10) == gold["printed"]["send_kib_per_rank_rounded"]


# ---------------------------------------------------- planted mistakes
def _attention_variant(q, k, v, scale=None, mut=None):
    """A copy of the oracle's attention with one switchable planted mistake."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, Nq, D = q.shape
    scale = 1 / math.sqrt(D) if scale is None else float(scale)
    if mut == "no_scale":
        scale = 1.0
    if mut == "sqrt_missing":
        scale = 1.0 / D
    O = np.empty((B, H, Nq, v.shape[-1]))
    L = np.empty((B, H, Nq))
    rb = 256
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, rb):
                r1 = min(Nq, r0 + rb) - (1 if mut == "row_block_off_by_one" and Nq > rb else 0)
                S = scale * (q[b, h, r0:r1] @ k[b, h].T)
                m = S.max(axis=1, keepdims=True)
                if mut == "no_max_subtraction":
                    m = np.zeros_like(m)
                if mut == "max_over_queries":
                    m = S.max(axis=0, keepdims=True).max() * np.ones_like(m) - 1.0
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                if mut == "normalize_over_queries":
                    l = E.sum(axis=0, keepdims=True).sum(axis=1, keepdims=True) / E.shape[0]
                vv = k[b, h] if mut == "k_for_v" else v[b, h]
                O[b, h, r0:r1] = (E @ vv) / l
                if mut == "lse_sign":
                    L[b, h, r0:r1] = m[:, 0] - np.log(l[:, 0])
                elif mut == "lse_drops_max":
                    L[b, h, r0:r1] = np.log(l[:, 0])
                elif mut == "lse_log2":
                    L[b, h, r0:r1] = m[:, 0] + np.log2(l[:, 0])
                else:
                    L[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])
    if mut == "row_block_off_by_one":
        O = np.nan_to_num(O)
    return O, L


def _merge_variant(o_parts, lse_parts, mut=None):
    o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
    M = lse_parts.max(axis=0)
    w = np.exp(lse_parts - M[None])
    lse = M + np.log(w.sum(0))
    if mut == "weights_sign":
        w = np.exp(-(lse_parts - lse[None]))
    elif mut == "no_normalize":
        w = np.exp(lse_parts - M[None])
    elif mut == "lse_drops_max":
        lse = np.log(w.sum(0))
        w = np.exp(lse_parts - (M + lse)[None])
    else:
        w = np.exp(lse_parts - lse[None])
    if mut == "lse_mean":
        lse = lse_parts.mean(0)
    return (w[..., None] * o_parts).sum(0), lse


def _passes(pin, fn):
    """A pin passes only if it runs and holds; a crash counts as a rejection."""
    try:
        return pin(fn)
    except (ValueError, FloatingPointError, IndexError):
        return False


ATTN_MUTANTS = ["no_scale", "sqrt_missing", "row_block_off_by_one", "no_max_subtraction",
                "max_over_queries", "normalize_over_queries", "k_for_v", "lse_sign",
                "lse_drops_max", "lse_log2"]
MERGE_MUTANTS = ["weights_sign", "no_normalize", "lse_drops_max", "lse_mean"]


def test_unmutated_copies_match_oracle():
    r = _rng(17)
    q, k, v = (r.standard_normal((1, 2, 300, 16)) for _ in range(3))
    O1, L1 = oracle.attention(q, k, v)
    O2, L2 = _attention_variant(q, k, v)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert all(p(_attention_variant) for p in ATTN_PINS)
    assert pin_merge_split_equals_unsplit(oracle.attention, _merge_variant)
    assert all(p(_merge_variant) for p in MERGE_PINS)


@pytest.mark.parametrize("mut", ATTN_MUTANTS)
def test_pins_reject_planted_attention_mistake(mut):
    import warnings
    with warnings.catch_warnings(), np.errstate(all="ignore"):
        warnings.simplefilter("ignore")
        attn = lambda q, k, v, s: _attention_variant(q, k, v, s, mut)
        caught = [p.__name__ for p in ATTN_PINS if not _passes(p, attn)]
    assert caught, f"no pin rejects planted mistake {mut}"


@pytest.mark.parametrize("mut", MERGE_MUTANTS)
def test_pins_reject_planted_merge_mistake(mut):
    with np.errstate(all="ignore"):
        mg = lambda o, l: _merge_variant(o, l, mut)
        caught = [p.__name__ for p in MERGE_PINS if not _passes(p, mg)]
        if not pin_merge_split_equals_unsplit(oracle.attention, mg):
            caught.append("split_equals_unsplit")
    assert caught, f"no pin rejects planted mistake {mut}"


# ---------------------------------------------------- input generator
def test_bf16_rounding_matches_torch():
    r = _rng(18)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, 3.0e38], np.float32)])
    ours = datagen.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(datagen.bf16_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic():
    a = datagen.normal_bf16((1, 2, 40, 8), 3, row_scale=(0.5, 2.0))
    b = datagen.normal_bf16((1, 2, 40, 8), 3, row_scale=(0.5, 2.0))
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    c = datagen.normal_bf16((1, 2, 40, 8), 4, token_offset_std=0.1)
    assert not np.array_equal(a[0], c[0])
    t1, t2 = datagen.tiny_f32(), datagen.tiny_f32()
    assert all(np.array_equal(x, y) for x, y in zip(t1, t2))


def test_sample_rows_forced_members():
    rows = datagen.sample_rows(75600, 64, 1004)
    assert len(rows) == 64 and len(set(rows.tolist())) == 64
    assert rows[0] == 0 and rows[-1] == 75599
    assert any(r >= 75600 - 75600 % 128 and r < 75599 for r in rows)


def test_threaded_runner_is_the_oracle_row_by_row():
    """The worker-thread runner the full-size GPU tests use returns the
    oracle's rows (all rows, and a row sample).  Rows are independent; only
    the BLAS blocking of a different row count can move the last bits."""
    from _helpers import oracle_attention_threaded
    r = _rng(19)
    q, k, v = r.standard_normal((2, 3, 70, 8)), r.standard_normal((2, 3, 50, 8)), r.standard_normal((2, 3, 50, 8))
    O, L = oracle.attention(q, k, v, 0.4)
    O2, L2 = oracle_attention_threaded(q, k, v, 0.4, block=16)
    assert np.abs(O - O2).max() <= 1e-13 and np.abs(L - L2).max() <= 1e-13
    rows = np.array([0, 5, 33, 69])
    O3, L3 = oracle_attention_threaded(q, k, v, 0.4, rows=rows, block=3)
    assert np.abs(O3 - O[:, :, rows]).max() <= 1e-13 and np.abs(L3 - L[:, :, rows]).max() <= 1e-13
    # a wrong row mapping (rows taken in block order from the start) is caught
    O4, _ = oracle_attention_threaded(q, k, v, 0.4, rows=np.arange(4), block=3)
    assert np.abs(O4 - O[:, :, rows]).max() > 1e-3
