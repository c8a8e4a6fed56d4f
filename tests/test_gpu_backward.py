"""GPU parity of the attention backward (dit_attn_bwd) against the fp64 oracle.

The GPU backward takes the GPU forward's bf16 O and float32 LSE, as a
training step would; the oracle differentiates the exact definition on the
same bf16 input values.  Tolerances (per gradient tensor, over the whole
tensor or the sampled rows): relative RMS error <= 1e-2 -- the pages' op-level
band for bf16 gradients is 8e-3 relative -- and max-abs error <= 3e-2 of the
tensor's largest reference magnitude; delta to 1e-2 of its RMS.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
import diffusion_transformer_attention_amd as dta
from _helpers import bits_to_torch_bf16, run_threaded, to_f64

pytestmark = pytest.mark.gpu

GRAD_REL_RMS = 1e-2
GRAD_MAX_ABS_REL = 3e-2


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def f64(bits):
    return datagen.bf16_to_f32(bits).astype(np.float64)


def _check_grad(got, ref, name, what):
    err = got - ref
    rr = float(np.linalg.norm(err.ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))
    ma = float(np.abs(err).max() / max(np.abs(ref).max(), 1e-300))
    say(f"{what} {name}: rel-RMS {rr:.2e}  max-abs/max|ref| {ma:.2e}")
    assert rr <= GRAD_REL_RMS, f"{what} {name} rel-RMS {rr:.3e}"
    assert ma <= GRAD_MAX_ABS_REL, f"{what} {name} max-abs {ma:.3e}"


def _inputs(B, H, Nq, Nkv, seed, D=128):
    qb, kb, vb = datagen.small_bf16(B, H, Nq, D, seed=seed, Nkv=Nkv)
    dob = datagen.small_bf16(B, H, Nq, D, seed=seed + 1)[0]
    return qb, kb, vb, dob


def _gpu_fwd_bwd(qb, kb, vb, dob, scale=None):
    tq, tk, tv, tdo = (bits_to_torch_bf16(x) for x in (qb, kb, vb, dob))
    O, L = dta.dit_attn_fwd_block(tq, tk, tv, scale=scale, out_dtype=torch.bfloat16)
    return (tq, tk, tv, tdo, O, L), dta.dit_attn_bwd(tq, tk, tv, O, tdo, L, scale=scale)


@pytest.mark.parametrize("B,H,Nq,Nkv", [
    (1, 2, 128, 128),
    (2, 3, 300, 200),      # ragged query and key tiles
    (1, 1, 1, 1),          # one token
    (1, 2, 64, 1000),
    (1, 1, 257, 129),
    (1, 2, 1000, 1000),
])
def test_backward_small_full_compare(B, H, Nq, Nkv):
    say("bwd", B, H, Nq, Nkv)
    qb, kb, vb, dob = _inputs(B, H, Nq, Nkv, seed=Nq * 5 + Nkv)
    _, (dq, dk, dv, delta) = _gpu_fwd_bwd(qb, kb, vb, dob)
    rq, rk, rv, rd = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(dob))
    what = f"B{B} H{H} Nq{Nq} Nkv{Nkv}"
    for got, ref, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _check_grad(to_f64(got), ref, n, what)
    dd = to_f64(delta) - rd
    assert np.linalg.norm(dd) <= 1e-2 * max(np.linalg.norm(rd), 1e-12)


@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("B,H,Nq,Nkv", [
    (1, 2, 128, 128),
    (2, 3, 300, 200),      # ragged query and key tiles
    (1, 1, 1, 1),          # one token
    (1, 1, 257, 1029),     # several workgroups each way, ragged
    (1, 2, 640, 96),       # more query tiles than key tiles
])
def test_backward_head_dims(B, H, Nq, Nkv, D):
    say("bwd D", D, B, H, Nq, Nkv)
    qb, kb, vb, dob = _inputs(B, H, Nq, Nkv, seed=Nq * 7 + Nkv + D, D=D)
    ins, (dq, dk, dv, delta) = _gpu_fwd_bwd(qb, kb, vb, dob)
    rq, rk, rv, rd = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(dob))
    what = f"D{D} B{B} H{H} Nq{Nq} Nkv{Nkv}"
    for got, ref, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        assert tuple(got.shape[2:]) == ref.shape[2:]
        _check_grad(to_f64(got), ref, n, what)
    dd = to_f64(delta) - rd
    assert np.linalg.norm(dd) <= 1e-2 * max(np.linalg.norm(rd), 1e-12)
    # a second call gives the same bits
    tq, tk, tv, tdo, O, L = ins
    again = dta.dit_attn_bwd(tq, tk, tv, O, tdo, L)
    for a, b, n in zip((dq, dk, dv, delta), again, ("dq", "dk", "dv", "delta")):
        assert torch.equal(a, b), f"{what} {n} not repeatable"


def test_backward_explicit_scale_and_large_scores():
    say("bwd explicit scale, wide score range")
    qb, kb, vb, dob = _inputs(1, 2, 200, 300, seed=77)
    q3 = datagen.bf16_bits(datagen.bf16_to_f32(qb) * 3.0)
    _, (dq, dk, dv, _) = _gpu_fwd_bwd(q3, kb, vb, dob, scale=0.2)
    rq, rk, rv, _ = oracle.attention_backward(f64(q3), f64(kb), f64(vb), f64(dob), 0.2)
    for got, ref, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _check_grad(to_f64(got), ref, n, "scale 0.2, q x3")


def test_backward_deterministic_and_per_head():
    """Bitwise repeatable, and a head's gradients do not depend on the other
    heads of the call (the Ulysses split computes whole heads)."""
    say("bwd determinism / head independence")
    qb, kb, vb, dob = _inputs(1, 4, 500, 500, seed=5)
    (tq, tk, tv, tdo, O, L), g1 = _gpu_fwd_bwd(qb, kb, vb, dob)
    g2 = dta.dit_attn_bwd(tq, tk, tv, O, tdo, L)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    sl = slice(1, 3)
    sub = [t[:, sl].contiguous() for t in (tq, tk, tv, O, tdo)]
    g3 = dta.dit_attn_bwd(*sub, L[:, sl].contiguous())
    assert all(torch.equal(a[:, sl], b) for a, b in zip(g1, g3))


def test_backward_ring_blocks():
    """Per K/V block with the merged O and LSE: each block's dk, dv equal the
    full call's rows bit for bit; the dq shares sum to the full dq."""
    say("bwd ring blocks")
    qb, kb, vb, dob = _inputs(1, 2, 512, 768, seed=9)
    (tq, tk, tv, tdo, O, L), (dq, dk, dv, _) = _gpu_fwd_bwd(qb, kb, vb, dob)
    dq_sum = torch.zeros_like(dq)
    for i in range(3):
        ks = slice(256 * i, 256 * (i + 1))
        dqi, dki, dvi, _ = dta.dit_attn_bwd(tq, tk[:, :, ks].contiguous(), tv[:, :, ks].contiguous(),
                                            O, tdo, L)
        assert torch.equal(dki, dk[:, :, ks]) and torch.equal(dvi, dv[:, :, ks])
        dq_sum += dqi
    rel = (dq_sum - dq).norm() / dq.norm()
    assert rel < 1e-5, rel


def test_backward_image_share_full():
    say("bwd image share B1 H24 N4096 D128, full compare")
    qb, kb, vb = datagen.workload_inputs("image_share")
    dob = datagen.small_bf16(1, 24, 4096, 128, seed=1001)[0]
    _, (dq, dk, dv, _) = _gpu_fwd_bwd(qb, kb, vb, dob)
    rq, rk, rv, _ = oracle.attention_backward(f64(qb), f64(kb), f64(vb), f64(dob))
    for got, ref, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _check_grad(to_f64(got), ref, n, "image share")


def test_backward_ulysses_share_sampled_rows():
    say("bwd Ulysses share B1 H10 N32768 D128: sampled dq rows and dk, dv keys")
    qb, kb, vb = (x[:, :10] for x in datagen.workload_inputs("ulysses_share"))
    dob = datagen.small_bf16(1, 10, 32768, 128, seed=1002)[0]
    _, (dq, dk, dv, delta) = _gpu_fwd_bwd(qb, kb, vb, dob)
    q64, k64, v64, do64 = f64(qb), f64(kb), f64(vb), f64(dob)
    rows = datagen.sample_rows(32768, 64, 1003)
    ri = torch.from_numpy(rows).cuda()

    def rows_task(h):
        return oracle.attention_backward_rows(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1],
                                              do64[:, h:h + 1], rows)

    res = run_threaded(rows_task, range(10))
    rq = np.concatenate([r[0] for r in res], axis=1)
    rd = np.concatenate([r[1] for r in res], axis=1)
    _check_grad(to_f64(dq[:, :, ri]), rq, "dq", "ulysses share sampled rows")
    assert np.abs(to_f64(delta[:, :, ri]) - rd).max() <= 1e-2 * np.abs(rd).max()
    # dk, dv of 64 keys per head: each sums over all 32768 query rows
    keys = datagen.sample_rows(32768, 64, 1005)
    ki = torch.from_numpy(keys).cuda()

    def keys_task(h):
        return oracle.attention_backward_keys(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1],
                                              do64[:, h:h + 1], keys)

    res = run_threaded(keys_task, range(10))
    rk = np.concatenate([r[0] for r in res], axis=1)
    rv = np.concatenate([r[1] for r in res], axis=1)
    _check_grad(to_f64(dk[:, :, ki]), rk, "dk", "ulysses share sampled keys")
    _check_grad(to_f64(dv[:, :, ki]), rv, "dv", "ulysses share sampled keys")
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()


# Grids of tens to several hundred dK/dV and dQ workgroups: 12 cases drawn
# once from a fixed seed, B in {1, 2}, H up to 12, independent ragged Nq and
# Nkv up to 6000, an explicit scale half the time; dq and delta on 24 sampled
# query rows, dk and dv on 24 sampled keys, per head.
def _grid_cases():
    r = np.random.default_rng(2027)
    out = []
    for i in range(12):
        B, H = int(r.integers(1, 3)), int(r.integers(1, 13))
        Nq, Nkv = int(r.integers(1, 6001)), int(r.integers(1, 6001))
        scale = None if r.random() < 0.5 else float(r.uniform(0.03, 0.2))
        out.append((i, B, H, Nq, Nkv, scale))
    return out


@pytest.mark.parametrize("i,B,H,Nq,Nkv,scale", _grid_cases())
def test_backward_grids_sampled(i, B, H, Nq, Nkv, scale):
    say(f"bwd grid {i}: B{B} H{H} Nq{Nq} Nkv{Nkv} scale {scale}")
    qb, kb, vb, dob = _inputs(B, H, Nq, Nkv, seed=9100 + 2 * i)
    _, (dq, dk, dv, delta) = _gpu_fwd_bwd(qb, kb, vb, dob, scale)
    q64, k64, v64, do64 = f64(qb), f64(kb), f64(vb), f64(dob)
    rows = datagen.sample_rows(Nq, min(Nq, 24), 9300 + i)
    keys = datagen.sample_rows(Nkv, min(Nkv, 24), 9400 + i)
    ri, ki = torch.from_numpy(rows).cuda(), torch.from_numpy(keys).cuda()
    heads = [(b, h) for b in range(B) for h in range(H)]

    def task(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rd = oracle.attention_backward_rows(q64[sl], k64[sl], v64[sl], do64[sl], rows, scale)
        rk, rv = oracle.attention_backward_keys(q64[sl], k64[sl], v64[sl], do64[sl], keys, scale)
        return rq, rd, rk, rv

    res = run_threaded(task, heads)
    pick = lambda j: np.stack([np.stack([res[b * H + h][j][0, 0] for h in range(H)]) for b in range(B)])
    _check_grad(to_f64(dq[:, :, ri]), pick(0), "dq", f"grid {i} sampled rows")
    rd = pick(1)
    assert np.abs(to_f64(delta[:, :, ri]) - rd).max() <= 1e-2 * max(np.abs(rd).max(), 1e-30)
    _check_grad(to_f64(dk[:, :, ki]), pick(2), "dk", f"grid {i} sampled keys")
    _check_grad(to_f64(dv[:, :, ki]), pick(3), "dv", f"grid {i} sampled keys")
