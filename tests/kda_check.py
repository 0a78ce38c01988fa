"""Shared helpers of the GPU tests: device copies, oracle calls and the parity bars.

Parity bars (stated once, used by every GPU test):
  * fp32 path: max|gpu - oracle| / max|oracle| <= 1e-4, for o and for S;
  * bf16 path: max|gpu - oracle| <= 2e-2 * max|oracle|, for o and for S.
The oracle always reads the exact values the GPU received, upcast to float64.
"""

import numpy as np
import torch

from oracle import kda_oracle as ora

RTOL_F32 = 1e-4
ATOL_BF16 = 2e-2


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def to_dev(inp, device="cuda"):
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in inp.items()}


def bar(dtype):
    return RTOL_F32 if dtype == torch.float32 else ATOL_BF16


def max_rel(gpu, ref):
    gpu = np64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    return float(np.max(np.abs(gpu - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def assert_close(gpu, ref, dtype, what=""):
    err = max_rel(gpu, ref)
    assert np.all(np.isfinite(np64(gpu) if isinstance(gpu, torch.Tensor) else gpu)), f"{what}: non-finite"
    assert err <= bar(dtype), f"{what}: error {err:.3e} over bar {bar(dtype):.1e} ({dtype})"
    return err


def oracle_forward(inp, g_min=-5.0, flags=ora.FLAGS_DEFAULT, heads=None, T=None):
    """Oracle on the same (cast) inputs; optionally on a subset of heads/tokens."""
    q, k, v, z, br = (np64(inp[n]) for n in ("q", "k", "v", "z", "beta_raw"))
    A = np64(inp["A_log"])
    S0 = np64(inp["S0"])
    if T is not None:
        q, k, v, z, br = q[:, :T], k[:, :T], v[:, :T], z[:, :T], br[:, :T]
    if heads is not None:
        q, k, v, z, br = q[:, :, heads], k[:, :, heads], v[:, :, heads], z[:, :, heads], br[:, :, heads]
        A = A[heads]
        S0 = None if S0 is None else S0[:, heads]
    return ora.forward(q, k, v, z, br, A, S0, g_min, flags)
