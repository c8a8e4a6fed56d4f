"""dit_attn_fwd_balanced_noalloc (static device scratch, no allocation) against
dit_attn_fwd_balanced (caller workspace), through the C ABI.

Two calls in a row on one GPU share its scratch array: the long-video shape
(its key-chunk partials fill 133 MB of the array), then the smaller image
share (a different plan, written over the first call's partials).  Each is
compared with the workspace form's output, which uses the same plan and
kernels, so the results agree bit for bit; they are also held to the bf16
parity bars against it, and the second call's split rows to the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import diffusion_transformer_attention_amd as dta
from _helpers import assert_bf16_close, bits_to_torch_bf16, oracle_attention_threaded, to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _both(name, out_dtype):
    qb, kb, vb = datagen.workload_inputs(name)
    tq, tk, tv = (bits_to_torch_bf16(x) for x in (qb, kb, vb))
    B, H, Nq, D = tq.shape
    need = dta.dit_attn_fwd_balanced_workspace(B, H, Nq, tk.shape[2], D)
    assert 0 < need <= dta.DIT_SCRATCH_BYTES, need      # the plan splits and fits the scratch
    O_ws, L_ws = dta.dit_attn_fwd_balanced(tq, tk, tv, out_dtype=out_dtype)
    O_na = torch.full_like(O_ws, float("nan"))
    L_na = torch.full_like(L_ws, float("nan"))
    dta.dit_attn_fwd_balanced_noalloc(tq, tk, tv, O_na, L_na)
    torch.cuda.synchronize()
    say(f"{name}: {need / 1e6:.1f} MB of partials in the static scratch")
    return (qb, kb, vb), O_ws, L_ws, O_na, L_na


def test_noalloc_matches_workspace_form_on_two_calls():
    say("no-alloc balanced forward: long video, then image share")
    _, O_ws, L_ws, O_na, L_na = _both("long_video", torch.bfloat16)
    assert torch.equal(O_na, O_ws) and torch.equal(L_na, L_ws)
    assert_bf16_close(to_f64(O_na), to_f64(L_na), to_f64(O_ws), to_f64(L_ws), "long video no-alloc")
    del O_ws, L_ws, O_na, L_na

    (qb, kb, vb), O_ws, L_ws, O_na, L_na = _both("image_share", torch.float32)
    assert torch.equal(O_na, O_ws) and torch.equal(L_na, L_ws)
    assert_bf16_close(to_f64(O_na), to_f64(L_na), to_f64(O_ws), to_f64(L_ws), "image share no-alloc")
    # the tail rows (the split tiles of the last partial wave) against the oracle
    f64 = lambda b: datagen.bf16_to_f32(b).astype(np.float64)
    rows = np.arange(4096 - 512, 4096)
    Oref, Lref = oracle_attention_threaded(f64(qb), f64(kb), f64(vb), rows=rows)
    assert_bf16_close(to_f64(O_na[:, :, rows]), to_f64(L_na[:, :, rows]), Oref, Lref,
                      "image share no-alloc, tail rows")
