"""A seeded sweep of chunk-call shapes against the oracle (plain and grouped entries).

Each case draws its own shape from a fixed generator: batch 1-3, 1-600
tokens (so most sequences end in a ragged chunk and some are shorter than one
chunk), 1-5 heads, key and value widths from {16, 32, 64, 128} chosen
independently, state chunk 16, 32 or 64, fp32 or bf16 inputs, and an
incoming state or none.  The bounded gate, L2 normalisation and sigmoid beta
are on (the other switches have their own tests).  Every case compares o
and the final state with the fp64 token recurrence ("Implémenter KDA", 'La
forme par blocs': the chunk form must reproduce the recurrence) at the
parity bars of the other GPU tests, and every output must be finite.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_82_amd import inputs, kda
from oracle import kda_oracle as ora
from tests.kda_check import assert_close, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    widths = [16, 32, 64, 128]
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 601))
        H = int(rng.choice([1, 2, 3, 5]))
        Dk, Dv = int(rng.choice(widths)), int(rng.choice(widths))
        C = int(rng.choice([16, 32, 64]))
        dt = "bf16" if rng.random() < 0.5 else "f32"
        s_std = 0.1 if rng.random() < 0.6 else 0.0
        out.append((i, B, T, H, Dk, Dv, C, dt, s_std))
    return out


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{1}T{2}H{3}k{4}v{5}C{6}{7}{8}".format(
    *c[:8], "S0" if c[8] else ""))
def test_sweep_matches_oracle(case):
    i, B, T, H, Dk, Dv, C, dt, s_std = case
    print(f"sweep {i}: B{B} T{T} H{H} Dk{Dk} Dv{Dv} C{C} {dt} S0={'yes' if s_std else 'no'}", flush=True)
    inp = inputs.make_inputs(B, T, H, Dk, Dv, dt, seed=7000 + i, a_std=0.5, s_std=s_std)
    d = to_dev(inp)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], d["S0"], chunk=C)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp)
    dtype = BF16 if dt == "bf16" else F32
    assert_close(o, o_ref, dtype, f"sweep {i} o")
    assert_close(S, S_ref, dtype, f"sweep {i} S")


def _grouped_cases(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    widths = [16, 32, 64, 128]
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        T = int(rng.integers(1, 401))
        H = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4]))
        Dk, Dv = int(rng.choice(widths)), int(rng.choice(widths))
        C = int(rng.choice([16, 32, 64]))
        dt = "bf16" if rng.random() < 0.5 else "f32"
        bias = bool(rng.random() < 0.7)
        out.append((i, B, T, H, G, Dk, Dv, C, dt, bias))
    return out


@pytest.mark.parametrize("case", _grouped_cases(), ids=lambda c: "B{1}T{2}H{3}G{4}k{5}v{6}C{7}{8}{9}".format(
    *c[:9], "bias" if c[9] else ""))
def test_sweep_grouped_matches_oracle(case):
    """The grouped entry: H q/k heads shared by G value heads each, with or
    without the per-channel gate bias ("KDAAttention 层", 完整数据流 and its
    parameter table)."""
    i, B, T, H, G, Dk, Dv, C, dt, bias = case
    HV = H * G
    print(f"grouped sweep {i}: B{B} T{T} H{H} HV{HV} Dk{Dk} Dv{Dv} C{C} {dt} bias={bias}", flush=True)
    gen = torch.Generator().manual_seed(8000 + i)
    cast = torch.bfloat16 if dt == "bf16" else torch.float32
    q = torch.randn(B, T, H, Dk, generator=gen).to(cast)
    k = torch.randn(B, T, H, Dk, generator=gen).to(cast)
    v = torch.randn(B, T, HV, Dv, generator=gen).to(cast)
    z = torch.randn(B, T, HV, Dk, generator=gen).to(cast)
    br = torch.randn(B, T, HV, generator=gen).to(cast)
    A = (torch.randn(HV, generator=gen) * 0.5).float()
    db = (torch.randn(HV, Dk, generator=gen) * 0.5).float() if bias else None
    S0 = (torch.randn(B, HV, Dk, Dv, generator=gen) * 0.1).float()
    o, S = kda.chunk_fwd(*(t.cuda() for t in (q, k, v, z, br, A)), S0.cuda(), chunk=C,
                         dt_bias=None if db is None else db.cuda())
    torch.cuda.synchronize()
    n64 = lambda t: None if t is None else t.to(torch.float64).numpy()
    o_ref, S_ref = ora.forward_grouped(n64(q), n64(k), n64(v), n64(z), n64(br), n64(A), n64(db), n64(S0))
    dtype = BF16 if dt == "bf16" else F32
    assert_close(o, o_ref, dtype, f"grouped sweep {i} o")
    assert_close(S, S_ref, dtype, f"grouped sweep {i} S")
