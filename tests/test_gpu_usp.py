"""Ulysses x Ring (USP) on one GPU, composed from the library's entry points.

The pull request's op-level parity bands compare the hybrid sequence-parallel
attention with full-sequence attention at Ulysses x Ring degrees u4r1, u2r2
and u1r4 ("Feat: USP sequence parallelism ...", Validation).  Here the
u*r ranks are list entries, as in the handbook's simulation: ring group i
holds tokens [i N/r, (i+1) N/r), split into u Ulysses shards; seq2head
(P = u) inside each ring group gives Ulysses rank j the heads
[j H/u, (j+1) H/u) over that token block; each (i, j) runs the block kernel
against the K/V blocks of every ring group and merges the r float32
partials by log-sum-exp; head2seq (P = u) returns the tokens.  The result
must meet the bf16 tolerances against the fp64 oracle's full attention and
stay within the pages' ring deviation band of the single-pass kernel; with
r = 1 (pure Ulysses) it must equal the single pass bit for bit (one partial
merges to itself).
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
import diffusion_transformer_attention_amd as dta
from _helpers import assert_bf16_close, bits_to_torch_bf16, max_abs, to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def usp_forward(q, k, v, u, r):
    B, H, N, D = q.shape
    blk = N // r
    shard = lambda x, i: torch.stack(x[:, :, i * blk:(i + 1) * blk].chunk(u, dim=2)).contiguous()
    G = [[dta.ulysses_seq2head(shard(x, i)) for i in range(r)] for x in (q, k, v)]
    out_blocks, lse_blocks = [], []
    for i in range(r):
        per_rank, lse_rank = [], []
        for j in range(u):
            parts = [dta.dit_attn_fwd_block(G[0][i][j], G[1][i2][j], G[2][i2][j],
                                            out_dtype=torch.float32) for i2 in range(r)]
            Om, Lm = dta.dit_attn_merge(torch.stack([p[0] for p in parts]),
                                        torch.stack([p[1] for p in parts]),
                                        out_dtype=torch.bfloat16)
            per_rank.append(Om)
            lse_rank.append(Lm)
        back = dta.ulysses_head2seq(torch.stack(per_rank))           # [u][B,H,blk/u,D]
        out_blocks.append(torch.cat(list(back), dim=2))
        lse_blocks.append(torch.cat(lse_rank, dim=1))                 # [B,H,blk]
    return torch.cat(out_blocks, dim=2), torch.cat(lse_blocks, dim=2)


@pytest.mark.parametrize("u,r", [(4, 1), (2, 2), (1, 4), (2, 4)])
def test_usp_degrees(u, r):
    B, H, N, D = 1, 8, 2048, 128
    say(f"USP u{u}r{r}: B{B} H{H} N{N} D{D}")
    qb, kb, vb = datagen.small_bf16(B, H, N, D, seed=600 + 10 * u + r)
    q, k, v = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    O, L = usp_forward(q, k, v, u, r)
    f64 = lambda b: datagen.bf16_to_f32(b).astype(np.float64)
    Oref, Lref = oracle.attention(f64(qb), f64(kb), f64(vb))
    assert_bf16_close(to_f64(O), to_f64(L), Oref, Lref, f"u{u}r{r}")
    Os, Ls = dta.dit_attn_fwd(q, k, v)
    if r == 1:
        assert torch.equal(O, Os) and torch.equal(L, Ls)
    else:
        assert max_abs(to_f64(O), to_f64(Os)) <= 2e-2
        assert max_abs(to_f64(L), to_f64(Ls)) <= 1e-3
