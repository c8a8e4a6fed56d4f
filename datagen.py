"""Seeded synthetic inputs for the DiT sequence-parallel attention workloads.

This module holds no attention, merge or permute arithmetic.  It only draws
random tensors, applies each workload's stated value structure, and rounds
float32 to bfloat16 bit patterns.  The CPU oracle tests and the GPU path both
take their inputs from here, so the two sides see the same bits.

Workload shapes come from the models the pages discuss ("Multi-GPU
parallelism: spreading one step over several cards", sections "Sequence
parallelism: Ulysses and Ring" and "Guidance parallelism"; the miles_diffusion
USP pull request, "Ring kernel selection"):

* tiny_f32      B1 H8 N256 D32 fp32 from seed 0 (torch's CPU generator), the
                numbers of the handbook's four-card Ulysses simulation.
* image_share   B1 H24 N4096 D128 bf16, FLUX 1024^2 image tokens (64x64 patch
                grid, 24 heads, head dim 128); each (tensor, b, h, token) row
                is scaled by a factor drawn from U(0.5, 2).
* ulysses_share B1 H10 N32768 D128 bf16: one rank's head group after the
                Ulysses seq->head exchange of a [1,40,32768,128] Wan-shaped
                tensor at P=4 (the pull request's benchmark shape).
* ring_merge    B1 H40 N32768 D128 bf16, K/V split in 4 contiguous blocks of
                8192 tokens; same draw as ulysses_share.
* long_video    B1 H10 N75600 D128 bf16, the 21x45x80 latent patch grid of a
                Wan 720p 81-frame video; each (tensor, b, token) gets one mean
                offset drawn from N(0, 0.1) (0.1 is the standard deviation),
                shared by every head and channel.

Random draws use numpy's PCG64 ``default_rng(seed)`` in the order q, k, v,
then the structure draws in the order q, k, v.  The tiny workload instead
draws from torch's CPU generator, which gives the handbook simulation's own
numbers, so its printed outcome can be checked on identical data.
"""
from __future__ import annotations

import numpy as np

# name -> shape/seed description.  "full_heads" is the head count before the
# Ulysses split; "P" the Ulysses degree; "nblk" the ring block count.
WORKLOADS = {
    "tiny_f32": dict(B=1, H=8, N=256, D=32, dtype="f32", seed=0, P=4),
    "image_share": dict(B=1, H=24, N=4096, D=128, dtype="bf16", seed=1),
    "ulysses_share": dict(B=1, H=10, N=32768, D=128, dtype="bf16", seed=2,
                          P=4, full_heads=40),
    "ring_merge": dict(B=1, H=40, N=32768, D=128, dtype="bf16", seed=2, nblk=4),
    "long_video": dict(B=1, H=10, N=75600, D=128, dtype="bf16", seed=4),
}


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) -> uint16 bits.

    Inputs are finite, so the NaN/Inf encodings need no special case.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    b = x32.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to the float32 values they encode."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tiny_f32():
    """The tiny float32 workload: q, k, v [1,8,256,32] ~ N(0,1) from seed 0.

    One [3,1,8,256,32] standard-normal draw of a torch CPU generator seeded
    with 0, split into q, k, v.  These are the same numbers as the
    handbook's four-card simulation draws, so its printed outcome can be
    checked on identical data.
    """
    import torch
    gen = torch.Generator(device="cpu").manual_seed(0)
    qkv = torch.randn((3, 1, 8, 256, 32), generator=gen, dtype=torch.float32).numpy()
    return tuple(np.ascontiguousarray(qkv[i]) for i in range(3))


def normal_bf16(shape, seed, row_scale=None, token_offset_std=None):
    """Draw q, k, v ~ N(0,1) float32, apply the workload structure, round to bf16.

    row_scale=(lo, hi): one factor per (tensor, b, h, n) from U(lo, hi)
    multiplies the whole row.  token_offset_std=s: one offset per
    (tensor, b, n) from N(0, s) is added to every head and channel.
    Returns three uint16 arrays of bf16 bits, shape ``shape``.
    """
    B, H, N, D = shape
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    if row_scale is not None:
        lo, hi = row_scale
        for x in xs:
            x *= rng.uniform(lo, hi, size=(B, H, N, 1)).astype(np.float32)
    if token_offset_std is not None:
        for x in xs:
            x += rng.normal(0.0, token_offset_std, size=(B, 1, N, 1)).astype(np.float32)
    return tuple(bf16_bits(x) for x in xs)


def small_bf16(B, H, N, D, seed, Nkv=None):
    """Plain N(0,1) bf16 q [B,H,N,D] and k, v [B,H,Nkv,D] for parity cases."""
    Nkv = N if Nkv is None else Nkv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Nkv, D), dtype=np.float32)
    v = rng.standard_normal((B, H, Nkv, D), dtype=np.float32)
    return bf16_bits(q), bf16_bits(k), bf16_bits(v)


def device_normal_bf16(shape, seed, device="cuda"):
    """N(0,1) bf16 tensor drawn on the device by torch's seeded generator
    (for tensors too large to draw on the host; the oracle gets the slices it
    needs copied back)."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)


def small_f32(B, H, N, D, seed, Nkv=None):
    """Plain N(0,1) float32 q [B,H,N,D] and k, v [B,H,Nkv,D]."""
    Nkv = N if Nkv is None else Nkv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Nkv, D), dtype=np.float32)
    v = rng.standard_normal((B, H, Nkv, D), dtype=np.float32)
    return q, k, v


def workload_inputs(name):
    """q, k, v for a named workload: float32 arrays (tiny_f32) or bf16 bits.

    ulysses_share and ring_merge share one [1,40,32768,128] draw from seed 2;
    ulysses_share returns that full tensor (the permutes act on all 40 heads;
    rank r's attention share is heads [10r, 10r+10)).
    """
    w = WORKLOADS[name]
    if name == "tiny_f32":
        return tiny_f32()
    if name == "image_share":
        return normal_bf16((w["B"], w["H"], w["N"], w["D"]), w["seed"], row_scale=(0.5, 2.0))
    if name in ("ulysses_share", "ring_merge"):
        return normal_bf16((1, 40, 32768, 128), 2)
    if name == "long_video":
        return normal_bf16((w["B"], w["H"], w["N"], w["D"]), w["seed"], token_offset_std=0.1)
    raise KeyError(name)


def sample_rows(N, count, seed, tile=128):
    """``count`` distinct query rows in [0, N), always holding 0, N-1 and a row
    of the last partial ``tile``-row block when N is not a multiple of tile."""
    rng = np.random.default_rng(seed)
    forced = [0, N - 1]
    rem = N % tile
    if rem:
        forced.append(N - rem + int(rng.integers(0, rem)))
    forced = sorted(set(forced))
    pool = np.setdiff1d(np.arange(N), np.array(forced))
    extra = rng.choice(pool, size=max(0, count - len(forced)), replace=False)
    return np.sort(np.concatenate([np.array(forced, dtype=np.int64), extra.astype(np.int64)]))


# --------------------------------------------------------------------------
# Joint text + image inputs.  The rotary angle schedule is the model's choice,
# so it is an input here: pairs [0, D/4) follow the token's row on the patch
# grid and pairs [D/4, D/2) its column, pair j of each half turning at
# frequency base**(-j / (D/4)).  Image token n sits at (n // cols, n % cols);
# text token t sits at (g + t, g + t) with g = max(rows, cols), on the
# diagonal past the grid.  Tables are float32 [N, D/2] (cosine, sine).
# --------------------------------------------------------------------------
def _axial_tables(pos_r, pos_c, D, base):
    quarter = D // 4
    freq = base ** (-np.arange(quarter, dtype=np.float64) / quarter)
    ang = np.concatenate([np.outer(pos_r, freq), np.outer(pos_c, freq)], axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_tables_image(rows, cols, D, base=10000.0):
    n = np.arange(rows * cols, dtype=np.float64)
    return _axial_tables(n // cols, n % cols, D, base)


def rope_tables_text(Nt, rows, cols, D, base=10000.0):
    p = max(rows, cols) + np.arange(Nt, dtype=np.float64)
    return _axial_tables(p, p, D, base)


def joint_bf16(B, Ht, Nt, H, Ni, D, seed):
    """Text q, k, v [B,Ht,Nt,D] then image q, k, v [B,H,Ni,D], N(0,1) bf16
    bits, drawn in that order from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    txt = [bf16_bits(rng.standard_normal((B, Ht, Nt, D), dtype=np.float32)) for _ in range(3)]
    img = [bf16_bits(rng.standard_normal((B, H, Ni, D), dtype=np.float32)) for _ in range(3)]
    return tuple(txt), tuple(img)
