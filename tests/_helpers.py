"""Shared test helpers: error metrics, tolerances, tensor conversion, and a
thread pool that runs the oracle over many rows at once.

Holds no attention arithmetic; the oracle lives in oracle/, the kernels in
the HIP library.
"""
import concurrent.futures as cf
import os

import numpy as np

# Tolerances for bf16 inputs (O against the fp64 oracle, over the whole
# tensor or the sampled rows) and for float32 inputs.
BF16_O_MAX_ABS = 2e-2
BF16_O_REL_RMS = 1e-2
BF16_LSE_MAX_ABS = 1e-3
F32_MAX_ABS = 1e-4


def max_abs(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def rel_rms(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))


def to_f64(t):
    """GPU or CPU torch tensor (bf16 / f32) -> float64 numpy."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits_to_torch_bf16(bits, device="cuda"):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def assert_bf16_close(O, L, Oref, Lref, what=""):
    ma, rr = max_abs(O, Oref), rel_rms(O, Oref)
    assert ma <= BF16_O_MAX_ABS, f"{what} O max-abs {ma:.3e} > {BF16_O_MAX_ABS}"
    assert rr <= BF16_O_REL_RMS, f"{what} O rel-RMS {rr:.3e} > {BF16_O_REL_RMS}"
    if L is not None:
        la = max_abs(L, Lref)
        assert la <= BF16_LSE_MAX_ABS, f"{what} LSE max-abs {la:.3e} > {BF16_LSE_MAX_ABS}"
    return ma, rr


def cpu_workers():
    """CPUs this process may use: its affinity set, capped by the cgroup CPU
    quota when one is set (a container's share of a larger host)."""
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    return n


def run_threaded(fn, tasks, workers=None):
    """fn over tasks on worker threads, BLAS held to one thread per worker
    (numpy's matmul and ufuncs release the GIL, so the workers run in
    parallel)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with cf.ThreadPoolExecutor(max_workers=workers or cpu_workers()) as ex:
            return list(ex.map(fn, tasks))


def oracle_attention_threaded(q, k, v, scale=None, rows=None, block=512):
    """oracle.attention on float64 q [B,H,Nq,D], k, v [B,H,Nkv,D], for every
    query row (or the rows ``rows`` of every head), as (b, h, row block) tasks
    on worker threads.  Rows are independent, so the result is the oracle's
    own, row by row."""
    import oracle
    B, H = q.shape[:2]
    rows = np.arange(q.shape[2]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((B, H, len(rows), v.shape[-1]))
    L = np.empty((B, H, len(rows)))

    def one(t):
        b, h, i0 = t
        sel = rows[i0:i0 + block]
        o, l = oracle.attention(q[b:b + 1, h:h + 1, sel], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale)
        O[b, h, i0:i0 + len(sel)] = o[0, 0]
        L[b, h, i0:i0 + len(sel)] = l[0, 0]

    run_threaded(one, [(b, h, i0) for b in range(B) for h in range(H) for i0 in range(0, len(rows), block)])
    return O, L
