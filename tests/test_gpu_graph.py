"""The library under HIP graph capture.

The entry points enqueue kernels only (no allocation, copy or memset) on the
caller's stream, so a caller can capture a whole step once and replay it.
The step captured here: the Ulysses round trip (seq2head, attention of each
head group with LSE, head2seq), the backward of head group 0, per-head FP8
quantization followed by FP8 attention, the paired quantizer with
power-of-two scales followed by its FP8 attention, a joint text + image call and a
work-balanced call that takes its key-split path (its device query runs
under capture too).  It is
replayed three times, with unrelated eager launches and synchronizations in
between, and every replay must reproduce the eager outputs bit for bit (the
kernels are deterministic, so any difference would come from the capture).
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import diffusion_transformer_attention_amd as dta
from _helpers import bits_to_torch_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


P, B, H, N, D = 4, 1, 8, 1024, 128


def _inputs():
    g = torch.Generator().manual_seed(7)
    full = [torch.randn(B, H, N, D, generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    shards = [torch.stack(t.chunk(P, dim=2)).contiguous() for t in full]
    dout = torch.randn(B, H // P, N, D, generator=g).to(torch.bfloat16).cuda()
    txt, img = datagen.joint_bf16(B, H, 77, H, 300, D, seed=5)
    c, s = datagen.rope_tables_image(5, 64, D)
    tabs = [torch.from_numpy(np.ascontiguousarray(x[:300])).cuda() for x in (c, s)]
    ct, st = datagen.rope_tables_text(77, 5, 64, D)
    tabs = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (ct, st)] + tabs
    joint = [bits_to_torch_bf16(x) for x in txt + img]
    bal = [torch.randn(1, 2, n, D, generator=g).to(torch.bfloat16).cuda() for n in (256, 4096, 4096)]
    return shards, dout, joint + [bal], tabs


def _buffers(shards):
    return {
        "groups": [torch.empty((P, B, H // P, N, D), device="cuda", dtype=torch.bfloat16)
                   for _ in range(3)],
        "o": torch.empty((P, B, H // P, N, D), device="cuda", dtype=torch.bfloat16),
        "lse": torch.empty((P, B, H // P, N), device="cuda", dtype=torch.float32),
        "back": torch.empty_like(shards[0]),
        "dq": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.float32),
        "dk": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.float32),
        "dv": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.float32),
        "delta": torch.empty((B, H // P, N), device="cuda", dtype=torch.float32),
        "qc": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.uint8),
        "kc": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.uint8),
        "qd": torch.empty((B, H // P), device="cuda", dtype=torch.float32),
        "kd": torch.empty((B, H // P), device="cuda", dtype=torch.float32),
        "o8": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.bfloat16),
        "l8": torch.empty((B, H // P, N), device="cuda", dtype=torch.float32),
        "qcx": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.uint8),
        "kcx": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.uint8),
        "qdx": torch.empty((B, H // P), device="cuda", dtype=torch.float32),
        "kdx": torch.empty((B, H // P), device="cuda", dtype=torch.float32),
        "ox": torch.empty((B, H // P, N, D), device="cuda", dtype=torch.bfloat16),
        "lx": torch.empty((B, H // P, N), device="cuda", dtype=torch.float32),
        "oj": torch.empty((B, H, 377, D), device="cuda", dtype=torch.bfloat16),
        "lj": torch.empty((B, H, 377), device="cuda", dtype=torch.float32),
        "ws": torch.empty((3, B, H, 377, D), device="cuda", dtype=torch.bfloat16),
        "ob": torch.empty((1, 2, 256, D), device="cuda", dtype=torch.bfloat16),
        "lb": torch.empty((1, 2, 256), device="cuda", dtype=torch.float32),
        "wb": torch.empty((dta.dit_attn_fwd_balanced_workspace(1, 2, 256, 4096, D),),
                          device="cuda", dtype=torch.uint8),
    }


def _step(shards, dout, joint, tabs, b):
    for s, g in zip(shards, b["groups"]):
        dta.ulysses_seq2head(s, out=g)
    for r in range(P):
        dta.dit_attn_fwd(b["groups"][0][r], b["groups"][1][r], b["groups"][2][r], out=b["o"][r],
                         lse=b["lse"][r])
    dta.ulysses_head2seq(b["o"], out=b["back"])
    q0, k0, v0 = (g[0] for g in b["groups"])
    dta.dit_attn_bwd(q0, k0, v0, b["o"][0], dout, b["lse"][0], dq=b["dq"], dk=b["dk"], dv=b["dv"],
                     delta=b["delta"])
    dta.dit_quant_fp8(q0, codes=b["qc"], descale=b["qd"])
    dta.dit_quant_fp8(k0, codes=b["kc"], descale=b["kd"])
    dta.dit_attn_fwd_fp8(b["qc"], b["kc"], v0, b["qd"], b["kd"], out=b["o8"], lse=b["l8"])
    dta.dit_quant_fp8_qk_mx(q0, k0, q_codes=b["qcx"], k_codes=b["kcx"], q_descale=b["qdx"],
                            k_descale=b["kdx"])
    dta.dit_attn_fwd_fp8_mx(b["qcx"], b["kcx"], v0, b["qdx"], b["kdx"], out=b["ox"], lse=b["lx"])
    dta.dit_attn_fwd_joint(*joint[:6], *tabs, out=b["oj"], lse=b["lj"], workspace=b["ws"])
    dta.dit_attn_fwd_balanced(*joint[6], out=b["ob"], lse=b["lb"], workspace=b["wb"])


def _snapshot(b):
    keys = ("back", "lse", "dq", "dk", "dv", "delta", "qc", "kc", "qd", "kd", "o8", "l8", "qcx",
            "kcx", "qdx", "kdx", "ox", "lx", "oj", "lj", "ob", "lb")
    return {k: b[k].clone() for k in keys}


def test_graph_replays_match_eager():
    shards, dout, joint, tabs = _inputs()
    eager = _buffers(shards)
    say("eager step")
    _step(shards, dout, joint, tabs, eager)
    torch.cuda.synchronize()
    want = _snapshot(eager)

    b = _buffers(shards)
    say("capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream's allocator state first
        _step(shards, dout, joint, tabs, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(shards, dout, joint, tabs, b)
    torch.cuda.synchronize()

    junk = torch.randn(1, 2, 512, D, device="cuda").to(torch.bfloat16)
    for rep in range(3):
        for t in b.values():  # the replay must rewrite every output
            if isinstance(t, torch.Tensor):
                t.fill_(7)
            else:
                for u in t:
                    u.fill_(7)
        dta.dit_attn_fwd(junk, junk, junk)  # unrelated eager work between replays
        torch.cuda.synchronize()
        say(f"replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(b)
        bad = [k for k in want if not torch.equal(want[k], got[k])]
        assert not bad, f"replay {rep}: {bad} differ from the eager step"
