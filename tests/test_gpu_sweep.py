"""A seeded sweep of ragged shapes through every forward variant and the
backward, compared in full with the oracle.

Forty shapes drawn once from a fixed seed: B in {1, 2}, H in {1, 2, 3}, query
and key counts from 1 to 700, one in five of them from 1 to 8 (so partial key
tiles, partial query tiles and single tokens meet in every combination), D in
{32, 64, 128} with half the draws at 128, an explicit softmax scale half the
time.  Each goes through the bf16 kernel with bf16 and with float32 O, the
float32-input kernel, the FP8 kernel (D = 128; codes made by the oracle), and
the merge of the bf16 kernel's float32 partials over two key blocks; sixteen
more shapes (D = 128) go through the backward.  Every output element is
compared with the fp64 oracle at the tolerances of the other parity tests.
Twelve more shapes of more query tiles than compute units (several units per
persistent workgroup, some ending in a half-height round) are compared on
sampled rows, and 96 drawn cases take every forward entry point (plain,
Ring partial in float32 and bf16, work-balanced, fused Ulysses, FP8) through
launches of one to several rounds, also on sampled rows.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
import diffusion_transformer_attention_amd as dta
from _helpers import F32_MAX_ABS, assert_bf16_close, bits_to_torch_bf16, max_abs, to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _shapes():
    r = np.random.default_rng(2024)
    out = []
    for i in range(40):
        B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
        Nq, Nkv = (int(r.integers(1, 9)) if r.random() < 0.2 else int(r.integers(1, 701))
                   for _ in range(2))
        D = int(r.choice([32, 64, 128], p=[0.25, 0.25, 0.5]))
        scale = None if r.random() < 0.5 else float(r.uniform(0.02, 0.3))
        out.append((i, B, H, Nq, Nkv, D, scale))
    return out


SHAPES = _shapes()


def _f64(bits):
    return datagen.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("i,B,H,Nq,Nkv,D,scale", SHAPES)
def test_sweep(i, B, H, Nq, Nkv, D, scale):
    say(f"sweep {i}: B{B} H{H} Nq{Nq} Nkv{Nkv} D{D} scale {scale}")
    qb, kb, vb = datagen.small_bf16(B, H, Nq, D, seed=1000 + i, Nkv=Nkv)
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    Oref, Lref = oracle.attention(_f64(qb), _f64(kb), _f64(vb), scale)

    O, L = dta.dit_attn_fwd_block(q, k, v, scale=scale, out_dtype=torch.bfloat16)
    assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, f"sweep {i} bf16 out")
    O32, L32 = dta.dit_attn_fwd_block(q, k, v, scale=scale, out_dtype=torch.float32)
    assert_bf16_close(to_f64(O32), to_f64(L32), Oref, Lref, f"sweep {i} f32 out")

    # float32 inputs (the same values), float32 kernel
    qf, kf, vf = (t.float() for t in (q, k, v))
    Of, Lf = dta.dit_attn_fwd_block(qf, kf, vf, scale=scale, out_dtype=torch.float32)
    assert max_abs(to_f64(Of), Oref) <= F32_MAX_ABS and max_abs(to_f64(Lf), Lref) <= F32_MAX_ABS

    # two key blocks merged (Ring)
    if Nkv >= 2:
        cut = Nkv // 2
        parts = [dta.dit_attn_fwd_block(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(),
                                        scale=scale, out_dtype=torch.float32)
                 for a, b in ((0, cut), (cut, Nkv))]
        Om, Lm = dta.dit_attn_merge(torch.stack([p[0] for p in parts]),
                                    torch.stack([p[1] for p in parts]), out_dtype=torch.bfloat16)
        assert_bf16_close(to_f64(Om), to_f64(Lm), Oref, Lref, f"sweep {i} merged")

    # FP8 (head dim 128): codes and descales from the oracle
    if D == 128:
        qc, qd = oracle.quantize_fp8(datagen.bf16_to_f32(qb))
        kc, kd = oracle.quantize_fp8(datagen.bf16_to_f32(kb))
        O8, L8 = dta.dit_attn_fwd_fp8(torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), v,
                                      torch.from_numpy(qd).cuda(), torch.from_numpy(kd).cuda(),
                                      scale=scale)
        O8r, L8r = oracle.attention_fp8(qc, kc, _f64(vb), qd, kd, scale)
        assert_bf16_close(to_f64(O8), to_f64(L8), O8r, L8r, f"sweep {i} fp8")


GRAD_REL_RMS, GRAD_MAX_ABS_REL = 1e-2, 3e-2  # the backward parity test's bands


def _bwd_shapes():
    r = np.random.default_rng(4048)
    out = []
    for i in range(16):
        B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
        Nq, Nkv = (int(r.integers(1, 9)) if r.random() < 0.2 else int(r.integers(1, 701))
                   for _ in range(2))
        scale = None if r.random() < 0.5 else float(r.uniform(0.02, 0.3))
        out.append((i, B, H, Nq, Nkv, scale))
    return out


@pytest.mark.parametrize("i,B,H,Nq,Nkv,scale", _bwd_shapes())
def test_sweep_backward(i, B, H, Nq, Nkv, scale):
    say(f"bwd sweep {i}: B{B} H{H} Nq{Nq} Nkv{Nkv} scale {scale}")
    qb, kb, vb = datagen.small_bf16(B, H, Nq, 128, seed=3000 + i, Nkv=Nkv)
    dob = datagen.small_bf16(B, H, Nq, 128, seed=5000 + i)[0]
    q, k, v, do = (bits_to_torch_bf16(x) for x in (qb, kb, vb, dob))
    O, L = dta.dit_attn_fwd_block(q, k, v, scale=scale, out_dtype=torch.bfloat16)
    dq, dk, dv, delta = dta.dit_attn_bwd(q, k, v, O, do, L, scale=scale)
    refs = oracle.attention_backward(_f64(qb), _f64(kb), _f64(vb), _f64(dob), scale)
    for got, ref, n in zip((dq, dk, dv, delta), refs, ("dq", "dk", "dv", "delta")):
        err = to_f64(got) - ref
        rr = float(np.linalg.norm(err.ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))
        ma = float(np.abs(err).max() / max(np.abs(ref).max(), 1e-300))
        assert rr <= GRAD_REL_RMS, f"bwd sweep {i} {n} rel-RMS {rr:.3e}"
        if n != "delta":
            assert ma <= GRAD_MAX_ABS_REL, f"bwd sweep {i} {n} max-abs {ma:.3e}"


# Launches of more query tiles than compute units: the persistent loop over
# several units per workgroup (the next unit's queries loaded during the last
# key tile), and a half-height last round when it fills at most half the
# units.  Twelve shapes drawn once from a fixed seed: B H in 2..12 heads,
# Nq from 8000 to 40000 (ragged), Nkv from 1 to 3000, D in {32, 64, 128};
# sampled query rows (first, last, tile edges, random) compared with the
# oracle, bf16 and float32 O.
def _multi_unit_shapes():
    r = np.random.default_rng(2025)
    out = []
    for i in range(12):
        B, H = int(r.integers(1, 3)), int(r.integers(1, 7))
        Nq = int(r.integers(8000, 40001))
        Nkv = int(r.integers(1, 9)) if r.random() < 0.25 else int(r.integers(9, 3001))
        D = int(r.choice([32, 64, 128]))
        out.append((i, B, H, Nq, Nkv, D))
    return out


@pytest.mark.parametrize("i,B,H,Nq,Nkv,D", _multi_unit_shapes())
def test_sweep_multi_unit(i, B, H, Nq, Nkv, D):
    tiles = B * H * ((Nq + 255) // 256)
    say(f"multi-unit {i}: B{B} H{H} Nq{Nq} Nkv{Nkv} D{D} ({tiles} tiles)")
    qb, kb, vb = datagen.small_bf16(B, H, Nq, D, seed=3000 + i, Nkv=Nkv)
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    rg = np.random.default_rng(i)
    rows = sorted(set([0, 127, 128, 255, 256, Nq - 1, Nq - 129, Nq // 2]) |
                  set(int(x) for x in rg.integers(0, Nq, 24)))
    rows = [x for x in rows if 0 <= x < Nq]
    Oref, Lref = oracle.attention_rows(_f64(qb), _f64(kb), _f64(vb), rows)
    for od in (torch.bfloat16, torch.float32):
        O, L = dta.dit_attn_fwd_block(q, k, v, out_dtype=od)
        assert_bf16_close(to_f64(O)[:, :, rows], to_f64(L)[:, :, rows], Oref, Lref,
                          f"multi-unit {i} {od}")


# Every forward entry point on launches of one to several rounds of query
# tiles: 96 cases drawn once from a fixed seed, each an entry point (plain
# bf16, Ring partial with float32 or bf16 O, work-balanced, fused Ulysses with
# P in {2, 4, 8}, FP8) on B in {1, 2}, H up to 24, N up to 9000 (keys ragged
# and independent of the queries for the Ring partials), D in {32, 64, 128},
# q scaled by 2.5 in half the bf16 cases (peaked softmax rows); 24 sampled
# query rows per head compared with the oracle at the bf16 tolerances.
def _entry_point_cases():
    r = np.random.default_rng(2026)
    kinds = ("plain", "block_f32", "block_bf16", "balanced", "ulysses", "fp8")
    out = []
    for i in range(96):
        kind = kinds[i % len(kinds)]
        B, H = int(r.integers(1, 3)), int(r.integers(1, 25))
        D = int(r.choice([32, 64, 128], p=[0.2, 0.2, 0.6]))
        Nq = int(r.integers(1, 9001))
        Nkv = int(r.integers(1, 6001)) if kind.startswith("block") else Nq
        P, qscale = 1, float(r.choice([1.0, 2.5]))
        if kind == "ulysses":
            P = int(r.choice([2, 4, 8]))
            H = P * int(r.integers(1, 7))
            Nq = Nkv = P * int(r.integers(64, 1500))  # shards of at least a key tile
        if kind == "fp8":
            D, H, Nq, qscale = 128, min(H, 6), min(Nq, 4000), 1.0
            Nkv = Nq
        out.append((i, kind, B, H, Nq, Nkv, D, P, qscale))
    return out


@pytest.mark.parametrize("i,kind,B,H,Nq,Nkv,D,P,qscale", _entry_point_cases())
def test_sweep_entry_points(i, kind, B, H, Nq, Nkv, D, P, qscale):
    say(f"entry {i}: {kind} B{B} H{H} Nq{Nq} Nkv{Nkv} D{D} P{P} q x{qscale}")
    qb, kb, vb = datagen.small_bf16(B, H, Nq, D, seed=7000 + i, Nkv=Nkv)
    if qscale != 1.0:
        qb = datagen.bf16_bits(datagen.bf16_to_f32(qb) * np.float32(qscale))
    rows = datagen.sample_rows(Nq, min(Nq, 24), 8000 + i)
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    if kind == "fp8":
        qc, qd = oracle.quantize_fp8(datagen.bf16_to_f32(qb))
        kc, kd = oracle.quantize_fp8(datagen.bf16_to_f32(kb))
        O, L = dta.dit_attn_fwd_fp8(torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), v,
                                    torch.from_numpy(qd).cuda(), torch.from_numpy(kd).cuda())
        Oref, Lref = oracle.attention_fp8(qc, kc, _f64(vb), qd, kd, rows=rows)
    else:
        Oref, Lref = oracle.attention_rows(_f64(qb), _f64(kb), _f64(vb), rows)
        if kind == "plain":
            O, L = dta.dit_attn_fwd(q, k, v)
        elif kind == "block_f32":
            O, L = dta.dit_attn_fwd_block(q, k, v, out_dtype=torch.float32)
        elif kind == "block_bf16":
            O, L = dta.dit_attn_fwd_block(q, k, v, out_dtype=torch.bfloat16)
        elif kind == "balanced":
            O, L = dta.dit_attn_fwd_balanced(q, k, v)
        else:  # token shards in, token shards out; rank r holds heads [r H/P, (r+1) H/P)
            shards = [torch.stack(t.chunk(P, dim=2)).contiguous() for t in (q, k, v)]
            out = torch.empty_like(shards[0])
            L = torch.cat([dta.dit_attn_fwd_ulysses(*shards, r, out=out)[1] for r in range(P)], dim=1)
            O = torch.cat(list(out), dim=2)
    assert_bf16_close(to_f64(O)[:, :, rows], to_f64(L)[:, :, rows], Oref, Lref, f"entry {i} {kind}")
