"""Benchmark of the DiT sequence-parallel attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-ring]
                    [--no-legs]

One step is the Ulysses round trip of one P=4 sequence-parallel attention
layer of a Wan-shaped tensor [1,40,32768,128] bf16, run on one GPU:
  1. ulysses_seq2head on q, k and v ([4][1,40,8192,128] -> [4][1,10,32768,128]);
  2. dit_attn_fwd with LSE on each of the 4 head groups, B1 H10 N32768 D128;
  3. ulysses_head2seq on the outputs.
Inputs are resident in HBM before the timed region.  `value` is the
attention FLOPs of the step (4 * 4*B*H*N^2*D) over the step's wall time.

The fused leg runs the same step as four dit_attn_fwd_ulysses calls that
read the token shards and write the token-shard output directly, with no
exchange buffers; it is reported under "legs" beside the unfused step, both
timed with events on the launch stream, four repetitions each, in six
interleaved pairs whose order alternates (medians).

The backward leg times dit_attn_bwd (dQ, dK, dV from the forward's O and
LSE) on one head group; its TFLOP/s counts the five products of the
backward, 10*B*H*N^2*D.

The joint leg times dit_attn_fwd_joint (RoPE + packing of text and image
tokens, then attention) on 512 text + 4096 image tokens, B1 H24 D128, and the
attention alone; the cross leg times dit_attn_fwd_block of the 10-head share's
32768 queries over 512 text keys.

The fp8 leg quantizes the share's q and k per head to E4M3 (dit_quant_fp8_qk)
and times dit_attn_fwd_fp8 on them (same FLOP count as the bf16 launch), then
the same with power-of-two scales and the softmax constant in the query codes
(dit_quant_fp8_qk_mx, dit_attn_fwd_fp8_mx).  Two
more bf16 forward legs: all 40 heads of the draw in one call, and the
[1,10,75600,128] long-video shape.

The ring leg (K/V in 4 blocks of 8192: four dit_attn_fwd_block calls with
float32 partials, then dit_attn_merge, B1 H40 N32768 D128) is timed after the
steps and reported under "legs"; it is not part of `value`.

The roofline object is for the dominant kernel, the attention forward: its
algorithmic FLOPs per launch over its average launch duration, measured with
events on the launch stream around every attention launch of the timed steps.
cpu_baseline times the fp64 CPU oracle on a bounded sample of the same
workload (query rows of the 10-head share against all 32768 keys).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak, B1 H10 N32768 D128 bf16"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0
B, H_FULL, N, D, P = 1, 40, 32768, 128, 4
H = H_FULL // P


def attn_flops(b, h, nq, nkv, d):
    return 4.0 * b * h * nq * nkv * d


KERNEL_SRC = os.path.join(ROOT, "diffusion_transformer_attention_amd", "csrc", "attn_bf16.hip")
COUNTERS_MD = os.path.join(ROOT, "profiles", "attn_fwd_bf16_ulysses_share.md")


def measured_traffic():
    """HBM bytes per attention launch from the committed FETCH_SIZE / WRITE_SIZE
    counters (already scaled by the copy-kernel calibration), or None when the
    kernel source has changed since they were taken."""
    import hashlib
    try:
        text = open(COUNTERS_MD).read()
        fields = dict(l.split(": ", 1) for l in text.splitlines()
                      if l.startswith(("counters-for-source-sha256:", "traffic_bytes_per_launch:")))
        src = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if fields.get("counters-for-source-sha256", "").strip() != src:
        return None
    return float(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ring", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the fused, backward, joint, cross, fp8, H40 and long-video legs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run three 1 GiB device-to-device copies (counter calibration)")
    return ap.parse_args()


def host_cpus():
    """(CPUs this process may use, CPUs in its affinity set, CPU model name).

    The usable count is the affinity set capped by the cgroup CPU quota, when
    one is set: a container given a share of a larger host sees every host
    CPU in its affinity set but may run only its quota at once."""
    affinity = len(os.sched_getaffinity(0))
    usable = affinity
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            usable = min(affinity, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return usable, affinity, model


def cpu_baseline(qb, kb, vb, target_s):
    """Time the fp64 oracle on query rows of the 10-head share (all 32768 keys)."""
    import concurrent.futures as cf

    import oracle
    import datagen
    from threadpoolctl import threadpool_limits
    cores, affinity, model = host_cpus()
    f64 = lambda b: datagen.bf16_to_f32(b).astype(np.float64)
    k64 = [f64(kb[:, h:h + 1]) for h in range(H)]
    v64 = [f64(vb[:, h:h + 1]) for h in range(H)]

    def run(rows_per_head):
        rows = np.arange(rows_per_head) * (N // rows_per_head)
        tasks = [(h, rows[i:i + 64]) for h in range(H) for i in range(0, len(rows), 64)]

        def one(task):
            h, r = task
            return oracle.attention_rows(f64(qb[:, h:h + 1]), k64[h], v64[h], r)

        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            with cf.ThreadPoolExecutor(max_workers=cores) as ex:
                list(ex.map(one, tasks))
            return time.perf_counter() - t0

    # 256 rows per head (40 tasks, enough to keep every worker busy) calibrate
    # the sample size
    probe = run(256)
    rows_per_head = int(min(N, max(256, 256 * target_s / max(probe, 1e-3))))
    rows_per_head = 64 * max(1, rows_per_head // 64)
    dt = run(rows_per_head)
    flops = attn_flops(1, H, rows_per_head, N, D)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_per_head} query rows x {H} heads against all {N} keys "
                      f"(fp64 numpy, {len(range(0, rows_per_head, 64)) * H} tasks of 64 rows "
                      f"on {cores} threads, BLAS 1 thread each), {dt:.1f} s",
            "seconds": dt, "flops": flops, "cpu_model": model, "affinity_cpus": affinity,
            "workers": cores}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(no collectives or multi-GPU sharding are built)", file=sys.stderr)
        sys.exit(2)
    import torch

    import datagen
    import diffusion_transformer_attention_amd as dta
    dta.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print("[bench] generating the seed-2 [1,40,32768,128] draw", file=sys.stderr, flush=True)
    qb, kb, vb = datagen.workload_inputs("ulysses_share")
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    full = [to_dev(x) for x in (qb, kb, vb)]
    # rank s's token slice [s*N/P, (s+1)*N/P) of every head: the input each rank holds
    shards = [torch.stack(t.chunk(P, dim=2)).contiguous() for t in full]
    groups = [torch.empty((P, B, H, N, D), device=dev, dtype=torch.bfloat16) for _ in range(3)]
    outs = torch.empty((P, B, H, N, D), device=dev, dtype=torch.bfloat16)
    lses = torch.empty((P, B, H, N), device=dev, dtype=torch.float32)
    back = torch.empty((P, B, H_FULL, N // P, D), device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    ev = []

    def step(record):
        for s, g in zip(shards, groups):
            dta.ulysses_seq2head(s, out=g)
        for r in range(P):
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            dta.dit_attn_fwd(groups[0][r], groups[1][r], groups[2][r], out=outs[r], lse=lses[r])
            if record:
                e1.record(stream)
                ev.append((e0, e1))
        dta.ulysses_head2seq(outs, out=back)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print("[bench] timed steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_avg_ms = float(np.mean(attn_ms))
    flops_launch = attn_flops(B, H, N, N, D)
    value = P * flops_launch / (ms_per_step * 1e-3) / 1e12
    achieved = flops_launch / (attn_avg_ms * 1e-3) / 1e12

    # permute legs, timed alone (bytes moved = read + write of one tensor)
    def time_it(fn, reps=10, min_ms=25.0):
        """Mean event time of back-to-back calls: after one call, warm up for
        about min_ms (a short kernel timed right after a long leg otherwise
        runs at the clock that leg left), then time at least `reps` calls and
        at least min_ms."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        n = max(1, math.ceil(min_ms / max(a.elapsed_time(b), 1e-3)))
        for _ in range(min(n, 200) - 1):
            fn()
        n = min(max(reps, n), 500)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    perm_bytes = 2.0 * B * H_FULL * N * D * 2
    s2h_ms = time_it(lambda: dta.ulysses_seq2head(shards[0], out=groups[0]))
    h2s_ms = time_it(lambda: dta.ulysses_head2seq(outs, out=back))
    legs = {"attn_fwd_ms_avg": attn_avg_ms, "attn_fwd_ms_min": float(np.min(attn_ms)),
            "seq2head_ms": s2h_ms, "seq2head_GBps": perm_bytes / (s2h_ms * 1e-3) / 1e9,
            "head2seq_ms": h2s_ms, "head2seq_GBps": perm_bytes / (h2s_ms * 1e-3) / 1e9}
    # practical ceiling of the HBM-bound kernels: a plain 1 GiB device-to-device
    # copy (2 GiB moved per copy; larger than the 256 MB Infinity Cache)
    csrc = torch.empty(1 << 30, device=dev, dtype=torch.uint8)
    cdst = torch.empty_like(csrc)
    copy_ms = time_it(lambda: cdst.copy_(csrc), reps=5)
    legs.update({"copy_1GiB_ms": copy_ms, "copy_GBps": 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9})
    del csrc, cdst

    if not args.no_legs:
        # fused leg: the same step with dit_attn_fwd_ulysses reading the shards
        # and writing the token-shard output directly (no exchange buffers)
        print("[bench] fused Ulysses leg", file=sys.stderr, flush=True)
        fused_out = torch.empty_like(back)

        def fused_step():
            for r in range(P):
                dta.dit_attn_fwd_ulysses(*shards, r, out=fused_out, lse=lses[r])

        # the same timer and repetition count for both forms, interleaved in
        # alternating order (fused first in even pairs, unfused first in odd
        # ones) so that a drift of the clock over the leg favours neither;
        # medians of six pairs
        fused_v, unfused_v = [], []
        for i in range(6):
            if i % 2 == 0:
                fused_v.append(time_it(fused_step, reps=4))
                unfused_v.append(time_it(lambda: step(False), reps=4))
            else:
                unfused_v.append(time_it(lambda: step(False), reps=4))
                fused_v.append(time_it(fused_step, reps=4))
        fused_ms, unfused_ms = float(np.median(fused_v)), float(np.median(unfused_v))
        legs.update({"fused_step_ms": fused_ms,
                     "fused_step_TFLOPs": P * flops_launch / (fused_ms * 1e-3) / 1e12,
                     "unfused_step_ms": unfused_ms,
                     "fused_vs_unfused": unfused_ms / fused_ms})

        # backward leg: dit_attn_bwd on the same head group (the forward's O and
        # LSE, a seeded dO); algorithmic FLOPs of the five products 10*B*H*N^2*D.
        print("[bench] backward leg", file=sys.stderr, flush=True)
        dout = torch.empty_like(outs[0]).normal_(generator=torch.Generator(device=dev).manual_seed(5))
        g_dq = torch.empty((B, H, N, D), device=dev, dtype=torch.float32)
        g_dk, g_dv = torch.empty_like(g_dq), torch.empty_like(g_dq)
        g_delta = torch.empty((B, H, N), device=dev, dtype=torch.float32)
        bwd_ms = time_it(lambda: dta.dit_attn_bwd(groups[0][0], groups[1][0], groups[2][0], outs[0], dout,
                                                  lses[0], dq=g_dq, dk=g_dk, dv=g_dv, delta=g_delta),
                         reps=3)
        legs.update({"bwd_ms": bwd_ms,
                     "bwd_TFLOPs": 2.5 * flops_launch / (bwd_ms * 1e-3) / 1e12,
                     "fwd_plus_bwd_ms": attn_avg_ms + bwd_ms})
        del g_dq, g_dk, g_dv, dout

        # joint leg: 512 text + 4096 image tokens (1024x1024 picture, 64x64
        # patches), 24 heads of 128, RoPE on q and k: dit_attn_fwd_joint (one
        # pack launch + the attention) and the attention alone on the packed
        # buffers; FLOPs 4*B*H*N^2*D over the N = 4608 joint tokens.
        print("[bench] joint text+image leg", file=sys.stderr, flush=True)
        jt, ji = datagen.joint_bf16(1, 24, 512, 24, 4096, D, seed=31)
        jt, ji = [to_dev(x) for x in jt], [to_dev(x) for x in ji]
        tabs = [torch.from_numpy(x).to(dev) for x in
                (*datagen.rope_tables_text(512, 64, 64, D), *datagen.rope_tables_image(64, 64, D))]
        jws = torch.empty((3, 1, 24, 4608, D), device=dev, dtype=torch.bfloat16)
        jo = torch.empty((1, 24, 4608, D), device=dev, dtype=torch.bfloat16)
        jl = torch.empty((1, 24, 4608), device=dev, dtype=torch.float32)
        joint_ms = time_it(lambda: dta.dit_attn_fwd_joint(*jt, *ji, *tabs, workspace=jws, out=jo,
                                                          lse=jl), reps=20)
        # the attention alone, on q, k, v packed (and q, k turned) by dit_rope_pack
        jq, jk, jv = (dta.dit_rope_pack(a, b, *tb) for a, b, tb in
                      zip(jt, ji, (tabs, tabs, [None] * 4)))
        jattn_ms = time_it(lambda: dta.dit_attn_fwd(jq, jk, jv, out=jo, lse=jl), reps=20)
        jflops = attn_flops(1, 24, 4608, 4608, D)
        legs.update({"joint_ms": joint_ms, "joint_TFLOPs": jflops / (joint_ms * 1e-3) / 1e12,
                     "joint_attn_only_ms": jattn_ms,
                     # the joint call over the attention alone: the k pack and the joint
                     # kernel's own per-unit query work
                     "joint_overhead_ms": joint_ms - jattn_ms})
        del jt, ji, jws, jo, jq, jk, jv

        # cross leg: the 10-head share's 32768 image queries over 512 text keys
        # and values (dit_attn_fwd_block, bf16 out).
        print("[bench] cross attention leg", file=sys.stderr, flush=True)
        _, ck, cv = (to_dev(x) for x in datagen.small_bf16(1, H, 1, D, seed=51, Nkv=512))
        co = torch.empty((B, H, N, D), device=dev, dtype=torch.bfloat16)
        cl = torch.empty((B, H, N), device=dev, dtype=torch.float32)
        cross_ms = time_it(lambda: dta.dit_attn_fwd_block(groups[0][0], ck, cv, out=co, lse=cl), reps=20)
        legs.update({"cross_ms": cross_ms,
                     "cross_TFLOPs": attn_flops(B, H, N, 512, D) / (cross_ms * 1e-3) / 1e12})
        del co, cl

        # fp8 leg: the same 10-head share with q and k quantized per head to
        # E4M3 (dit_quant_fp8, timed for both tensors) and the fp8 attention.
        print("[bench] fp8 leg", file=sys.stderr, flush=True)
        q0, k0, v0 = groups[0][0], groups[1][0], groups[2][0]
        qc, qd = dta.dit_quant_fp8(q0)
        kc, kd = dta.dit_quant_fp8(k0)
        fo, fl = torch.empty_like(outs[0]), torch.empty_like(lses[0])
        quant_ms = time_it(lambda: dta.dit_quant_fp8_qk(q0, k0, qc, kc, qd, kd), reps=10)
        fp8_ms = time_it(lambda: dta.dit_attn_fwd_fp8(qc, kc, v0, qd, kd, out=fo, lse=fl), reps=5)
        # quantizer traffic: q and k read twice (amax pass, code pass), codes written
        qbytes = 2 * (2 * 2 + 1) * B * H * N * D
        legs.update({"fp8_attn_ms": fp8_ms,
                     "fp8_attn_TFLOPs": flops_launch / (fp8_ms * 1e-3) / 1e12,
                     "fp8_quant_qk_ms": quant_ms,
                     "fp8_quant_qk_GBps": qbytes / (quant_ms * 1e-3) / 1e9})
        # power-of-two form: the quantizer folds the softmax constant into q
        mqc, mkc, mqd, mkd = dta.dit_quant_fp8_qk_mx(q0, k0, None, qc, kc, qd, kd)
        mx_quant_ms = time_it(lambda: dta.dit_quant_fp8_qk_mx(q0, k0, None, mqc, mkc, mqd, mkd),
                              reps=10)
        mx_ms = time_it(lambda: dta.dit_attn_fwd_fp8_mx(mqc, mkc, v0, mqd, mkd, out=fo, lse=fl),
                        reps=5)
        legs.update({"fp8_mx_attn_ms": mx_ms,
                     "fp8_mx_attn_TFLOPs": flops_launch / (mx_ms * 1e-3) / 1e12,
                     "fp8_mx_quant_qk_ms": mx_quant_ms})
        del qc, kc, fo, fl, mqc, mkc

        # single-pass ring-merge shape: all 40 heads of the [1,40,32768,128]
        # draw in one dit_attn_fwd (the full head count the ring blocks cover)
        print("[bench] single-pass H40 leg", file=sys.stderr, flush=True)
        so = torch.empty_like(full[0])
        sl = torch.empty((B, H_FULL, N), device=dev, dtype=torch.float32)
        sp_ms = time_it(lambda: dta.dit_attn_fwd(full[0], full[1], full[2], out=so, lse=sl), reps=3)
        legs.update({"single_pass_h40_ms": sp_ms,
                     "single_pass_h40_TFLOPs": attn_flops(B, H_FULL, N, N, D) / (sp_ms * 1e-3) / 1e12})
        del so, sl

        # long video: the 21x45x80 latent grid of a Wan 720p 81-frame clip,
        # [1,10,75600,128] (N not a multiple of the 256-row query tile)
        print("[bench] long video leg", file=sys.stderr, flush=True)
        lv = [to_dev(x) for x in datagen.workload_inputs("long_video")]
        lo = torch.empty_like(lv[0])
        ll = torch.empty(lv[0].shape[:3], device=dev, dtype=torch.float32)
        lv_ms = time_it(lambda: dta.dit_attn_fwd(lv[0], lv[1], lv[2], out=lo, lse=ll), reps=3)
        nlv = lv[0].shape[2]
        legs.update({"long_video_ms": lv_ms,
                     "long_video_TFLOPs": attn_flops(1, 10, nlv, nlv, D) / (lv_ms * 1e-3) / 1e12})
        # the same with the work-balanced entry point: 2960 query tiles are
        # 11.56 waves of 256 workgroups; the last partial wave's tiles run as
        # key chunks merged by log-sum-exp
        nws = dta.dit_attn_fwd_balanced_workspace(1, 10, nlv, nlv, D)
        lws = torch.empty((max(nws, 1),), device=dev, dtype=torch.uint8)
        lvb_ms = time_it(lambda: dta.dit_attn_fwd_balanced(lv[0], lv[1], lv[2], out=lo, lse=ll,
                                                            workspace=lws), reps=3)
        legs.update({"long_video_balanced_ms": lvb_ms,
                     "long_video_balanced_TFLOPs":
                         attn_flops(1, 10, nlv, nlv, D) / (lvb_ms * 1e-3) / 1e12,
                     "long_video_balanced_workspace_MB": nws / 1e6})
        del lv, lo, ll, lws

        # image share: FLUX 1024^2 image tokens, [1,24,4096,128] -- 384 query
        # tiles, 1.5 waves: plain and work-balanced
        print("[bench] image share leg", file=sys.stderr, flush=True)
        im = [to_dev(x) for x in datagen.workload_inputs("image_share")]
        io = torch.empty_like(im[0])
        il = torch.empty(im[0].shape[:3], device=dev, dtype=torch.float32)
        nim = im[0].shape[2]
        im_ms = time_it(lambda: dta.dit_attn_fwd(im[0], im[1], im[2], out=io, lse=il), reps=20)
        nws = dta.dit_attn_fwd_balanced_workspace(1, 24, nim, nim, D)
        iws = torch.empty((max(nws, 1),), device=dev, dtype=torch.uint8)
        imb_ms = time_it(lambda: dta.dit_attn_fwd_balanced(im[0], im[1], im[2], out=io, lse=il,
                                                            workspace=iws), reps=20)
        imf = attn_flops(1, 24, nim, nim, D)
        legs.update({"image_share_ms": im_ms, "image_share_TFLOPs": imf / (im_ms * 1e-3) / 1e12,
                     "image_share_balanced_ms": imb_ms,
                     "image_share_balanced_TFLOPs": imf / (imb_ms * 1e-3) / 1e12})
        del im, io, il, iws

    if not args.no_ring:
        print("[bench] ring leg", file=sys.stderr, flush=True)
        nblk, s = 4, N // 4
        kblk = [full[1][:, :, i * s:(i + 1) * s].contiguous() for i in range(nblk)]
        vblk = [full[2][:, :, i * s:(i + 1) * s].contiguous() for i in range(nblk)]
        o_parts = torch.empty((nblk, B, H_FULL, N, D), device=dev, dtype=torch.float32)
        l_parts = torch.empty((nblk, B, H_FULL, N), device=dev, dtype=torch.float32)
        o_m = torch.empty((B, H_FULL, N, D), device=dev, dtype=torch.bfloat16)
        l_m = torch.empty((B, H_FULL, N), device=dev, dtype=torch.float32)

        def blocks():
            for i in range(nblk):
                dta.dit_attn_fwd_block(full[0], kblk[i], vblk[i], out=o_parts[i], lse=l_parts[i])

        blk_ms = time_it(blocks, reps=3) / nblk
        mrg_ms = time_it(lambda: dta.dit_attn_merge(o_parts, l_parts, out=o_m, lse=l_m), reps=5)
        merge_bytes = nblk * (B * H_FULL * N * D * 4 + B * H_FULL * N * 4) + B * H_FULL * N * (D * 2 + 4)
        legs.update({"ring_block_fwd_ms": blk_ms,
                     "ring_block_fwd_TFLOPs": attn_flops(B, H_FULL, N, s, D) / (blk_ms * 1e-3) / 1e12,
                     "merge_ms": mrg_ms, "merge_GBps": merge_bytes / (mrg_ms * 1e-3) / 1e9})
        del o_parts, l_parts

    if args.copy_probe:
        # A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for
        # 1 GiB in and 1 GiB out calibrates the attention kernel's counters.
        src = torch.empty(1 << 30, device=dev, dtype=torch.uint8).fill_(7)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(qb[:, :H], kb[:, :H], vb[:, :H], args.cpu_seconds)

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ulysses_share: P=4 round trip of [1,40,32768,128] bf16; "
                               "attention per head group B1 H10 N32768 D128 (x4), seed 2",
                   "B": B, "H": H, "N": N, "D": D, "P": P, "heads_before_split": H_FULL},
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16_kernel<128,false,2>",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                     "flops_per_launch": flops_launch, "launches_timed": len(attn_ms)},
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
