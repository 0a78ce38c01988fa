"""Seeded synthetic inputs for the KDA workloads.

This module draws random tensors and casts them; it contains none of the
method's arithmetic (no normalisation, no gates, no recurrence), so both the
HIP path and the fp64 oracle can take their inputs from it.

Recipe (the pages print no datasets; the workloads are synthetic):
  * q, k, v, z, beta_raw ~ N(0, 1); A_log ~ N(0, a_std) per head (zeros when
    a_std == 0); S0 ~ N(0, s_std) in fp32 (absent when s_std == 0);
  * drawn in that fixed order from one `torch.Generator` seeded with `seed`;
  * q and k are drawn raw: the L2 normalisation named by the workloads is the
    path's own (the QK_L2NORM switch is on), done separately by the kernels
    and by the oracle;
  * the five tensors q, k, v, z, beta_raw are cast to the path dtype by
    round-to-nearest-even; A_log and S0 stay fp32.  The oracle reads the cast
    values upcast to float64, so parity measures kernel error only.
"""

from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str          # "f32" or "bf16"
    a_std: float        # std of A_log
    s_std: float        # std of S0 (0 => zero initial state)
    seed: int
    segments: int = 1   # KCP segments (long-context workload)
    steps: int = 0      # decode steps (decode workload)


WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=64, H=2, Dk=16, Dv=16, chunk=16, dtype="f32",
                     a_std=0.0, s_std=0.0, seed=1001),
    "small": Workload("small", B=2, T=1024, H=4, Dk=64, Dv=64, chunk=64, dtype="f32",
                      a_std=0.5, s_std=0.1, seed=1002),
    "layer": Workload("layer", B=4, T=4096, H=16, Dk=128, Dv=128, chunk=64, dtype="bf16",
                      a_std=0.5, s_std=0.0, seed=1003),
    "long": Workload("long", B=1, T=65536, H=32, Dk=128, Dv=128, chunk=64, dtype="bf16",
                     a_std=0.5, s_std=0.0, seed=1004, segments=8),
    "decode": Workload("decode", B=256, T=1, H=32, Dk=128, Dv=128, chunk=0, dtype="bf16",
                       a_std=0.5, s_std=0.05, seed=1005, steps=1024),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(B, T, H, Dk, Dv, dtype="f32", seed=0, a_std=0.0, s_std=0.0):
    """Draw one set of chunk-path inputs on the CPU.

    Returns a dict with q, k, z [B,T,H,Dk]; v [B,T,H,Dv]; beta_raw [B,T,H]
    (all in `dtype`), A_log [H] fp32 and S0 [B,H,Dk,Dv] fp32 or None.
    """
    gen = torch.Generator().manual_seed(int(seed))
    dt = torch_dtype(dtype)

    def normal(*shape, std=1.0):
        x = torch.randn(*shape, generator=gen, dtype=torch.float32)
        return x * std if std != 1.0 else x

    q = normal(B, T, H, Dk)
    k = normal(B, T, H, Dk)
    v = normal(B, T, H, Dv)
    z = normal(B, T, H, Dk)
    beta_raw = normal(B, T, H)
    A_log = normal(H, std=a_std) if a_std > 0 else torch.zeros(H, dtype=torch.float32)
    S0 = normal(B, H, Dk, Dv, std=s_std) if s_std > 0 else None
    return {
        "q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "z": z.to(dt),
        "beta_raw": beta_raw.to(dt), "A_log": A_log, "S0": S0,
    }


def make_workload(w: Workload, T: int | None = None, seed: int | None = None):
    """Inputs for a named workload (optionally with a shorter T for sampling)."""
    return make_inputs(w.B, w.T if T is None else T, w.H, w.Dk, w.Dv, w.dtype,
                       w.seed if seed is None else seed, w.a_std, w.s_std)


def decode_step_seed(w: Workload, s: int) -> int:
    """Seed of decode step s: base seed * 10**6 + s."""
    return w.seed * 10 ** 6 + s


def make_decode_step(w: Workload, s: int):
    """Per-step decode inputs: q, k, z [B,H,Dk]; v [B,H,Dv]; beta_raw [B,H]."""
    gen = torch.Generator().manual_seed(decode_step_seed(w, s))
    dt = torch_dtype(w.dtype)
    q = torch.randn(w.B, w.H, w.Dk, generator=gen)
    k = torch.randn(w.B, w.H, w.Dk, generator=gen)
    v = torch.randn(w.B, w.H, w.Dv, generator=gen)
    z = torch.randn(w.B, w.H, w.Dk, generator=gen)
    beta_raw = torch.randn(w.B, w.H, generator=gen)
    return {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "z": z.to(dt),
            "beta_raw": beta_raw.to(dt)}


def make_decode_state(w: Workload):
    """Initial decode state S0 ~ N(0, s_std) fp32 [B,H,Dk,Dv] and A_log [H]."""
    gen = torch.Generator().manual_seed(int(w.seed))
    A_log = torch.randn(w.H, generator=gen) * w.a_std
    S0 = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=gen) * w.s_std
    return S0, A_log
