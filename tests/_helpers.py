"""Shared test helpers: error metrics, tolerances and tensor conversion.

Holds no attention arithmetic; the oracle lives in oracle/, the kernels in
the HIP library.
"""
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
