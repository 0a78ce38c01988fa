"""GPU parity of the backward (kda_chunk_bwd) against the fp64 oracle's
adjoint of the recurrence, on the same (cast) inputs, to the bars of
tests/kda_check.py per gradient tensor."""

import numpy as np
import pytest
import torch

from gated_delta_rule_82_amd import inputs, kda
from oracle import kda_oracle as ora
from tests.kda_check import assert_close, np64

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16
V1 = kda.FLAGS_DEFAULT | kda.GATE_SOFTPLUS
NAMES = ("dq", "dk", "dv", "dz", "dbeta_raw", "dA_log", "dS0")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load()
    yield
    torch.cuda.synchronize()


def case(B, T, H, Dk, Dv, dtype, seed, flags, with_S0=True, with_dST=True):
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "bf16" if dtype == BF16 else "f32", seed=seed, a_std=0.5,
                             s_std=0.3 if with_S0 else 0.0)
    rng = np.random.default_rng(seed + 1)
    if not flags & kda.GATE_IN_KERNEL:   # the caller's log-decay in the gate slot
        inp["z"] = torch.tensor(-np.abs(rng.standard_normal((B, T, H, Dk))) * 1.5, dtype=F32).to(dtype)
    if not flags & kda.BETA_SIGMOID:     # beta itself
        inp["beta_raw"] = torch.tensor(rng.uniform(0.05, 0.95, (B, T, H)), dtype=F32).to(dtype)
    if not with_S0:
        inp["S0"] = None
    do = torch.tensor(rng.standard_normal((B, T, H, Dv)), dtype=F32).to(dtype)
    dST = torch.tensor(rng.normal(0, 0.5, (B, H, Dk, Dv)), dtype=F32) if with_dST else None
    return inp, do, dST


def run_and_compare(inp, do, dST, dtype, flags, what=""):
    dev = {k_: (None if v_ is None else v_.cuda().contiguous()) for k_, v_ in inp.items()}
    g = kda.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["z"], dev["beta_raw"], dev["A_log"], do.cuda(),
                      dev["S0"], None if dST is None else dST.cuda(), flags=flags)
    torch.cuda.synchronize()
    ref = ora.backward(*(np64(inp[n]) for n in ("q", "k", "v", "z", "beta_raw", "A_log")), np64(do),
                       np64(dST), np64(inp["S0"]), flags=flags)
    for n in NAMES:
        if n == "dA_log" and not flags & kda.GATE_IN_KERNEL:
            assert torch.count_nonzero(g[n]) == 0, f"{what} {n}: the gate switch is off"
            continue
        # dA_log and dS0 are fp32 sums in either path; the rest carry the input dtype
        assert_close(g[n], ref[n], F32 if n in ("dA_log", "dS0") and dtype == F32 else dtype, f"{what} {n}")


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Dk,Dv,T", [(64, 64, 70), (128, 128, 100), (16, 16, 33), (32, 64, 64), (64, 32, 97),
                                     (16, 128, 45), (128, 16, 40)])
def test_backward_matches_oracle(dtype, Dk, Dv, T):
    inp, do, dST = case(2, T, 2, Dk, Dv, dtype, Dk + Dv + T, kda.FLAGS_DEFAULT)
    run_and_compare(inp, do, dST, dtype, kda.FLAGS_DEFAULT, f"Dk{Dk} Dv{Dv} T{T}")


@pytest.mark.parametrize("flags", [V1, 0, 3, 5, 1])
def test_backward_switches(flags):
    inp, do, dST = case(2, 50, 2, 64, 64, F32, 100 + flags, flags)
    run_and_compare(inp, do, dST, F32, flags, f"flags {flags}")


def test_backward_without_gate_needs_no_A_log():
    # the gate switch off: A_log may be NULL and every gradient is the same
    inp, do, dST = case(2, 45, 2, 64, 64, F32, 9, 3)
    d = {k_: v_.cuda().contiguous() for k_, v_ in inp.items()}
    g1 = kda.chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], do.cuda(), d["S0"], dST.cuda(),
                       flags=3)
    g2 = kda.chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], None, do.cuda(), d["S0"], dST.cuda(), flags=3)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("with_S0,with_dST", [(False, False), (True, False), (False, True)])
def test_backward_optional_states(with_S0, with_dST):
    inp, do, dST = case(1, 40, 3, 64, 64, F32, 7, kda.FLAGS_DEFAULT, with_S0, with_dST)
    run_and_compare(inp, do, dST, F32, kda.FLAGS_DEFAULT, f"S0 {with_S0} dS_T {with_dST}")


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("zscale,zshift", [(6.0, 8.0), (4.0, 4.0), (2.0, 2.0)])
def test_backward_v1_gate_strong_decay(dtype, zscale, zshift):
    # per-token decays far beyond any bounded gate: 16-token blocks wider than
    # the factored sums allow (summed element by element) on every channel,
    # on some channels only, or on none
    inp, do, dST = case(1, 70, 2, 128, 64, dtype, 11, V1)
    inp["z"] = (inp["z"].float() * zscale + zshift).to(inp["z"].dtype)
    run_and_compare(inp, do, dST, dtype, V1, f"v1 strong decay z*{zscale}+{zshift}")


@pytest.mark.parametrize("T", [1, 31, 32, 33])
def test_backward_short_and_ragged(T):
    inp, do, dST = case(2, T, 2, 32, 32, F32, 30 + T, kda.FLAGS_DEFAULT)
    run_and_compare(inp, do, dST, F32, kda.FLAGS_DEFAULT, f"T{T}")


def test_backward_empty_sequence():
    # T = 0: the state gradient is dS_T itself and every other gradient is empty / zero
    B, H, Dk, Dv = 2, 3, 64, 64
    e = lambda *s: torch.empty(*s, device="cuda")
    q = e(B, 0, H, Dk)
    dST = torch.randn(B, H, Dk, Dv, device="cuda")
    g = kda.chunk_bwd(q, q.clone(), e(B, 0, H, Dv), q.clone(), e(B, 0, H), torch.zeros(H, device="cuda"),
                      e(B, 0, H, Dv), None, dST)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dST) and torch.count_nonzero(g["dA_log"]) == 0


def test_backward_is_the_gradient_of_the_gpu_forward():
    # a directional derivative of the GPU forward (fp32, central difference)
    # matches <gradient, direction> from the GPU backward
    inp, do, dST = case(1, 48, 2, 64, 64, F32, 44, kda.FLAGS_DEFAULT)
    d = {k_: v_.cuda().contiguous() for k_, v_ in inp.items()}
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], do.cuda(), d["S0"], dST.cuda())
    rng = np.random.default_rng(45)
    dirs = {n: torch.tensor(rng.standard_normal(tuple(d[n].shape)), dtype=F32, device="cuda")
            for n in ("q", "k", "v", "z", "beta_raw")}

    def loss(eps):
        x = {n: (d[n] + eps * dirs[n] if n in dirs else d[n]) for n in d}
        o, S = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta_raw"], x["A_log"], x["S0"], chunk=32)
        return float((o.double() * do.cuda().double()).sum() + (S.double() * dST.cuda().double()).sum())

    h = 1e-2
    fd = (loss(h) - loss(-h)) / (2 * h)
    an = sum(float((g["d" + n].double() * dirs[n].double()).sum()) for n in dirs)
    torch.cuda.synchronize()
    assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (fd, an)


def test_backward_layer_workload_sampled_heads():
    # the layer workload (B4 T4096 H16 D128 bf16) in one call; the (b, h)
    # recurrences are independent, so two sampled heads are checked against
    # the oracle over the whole sequence (dA_log sums over the batch: checked
    # through the per-head gate gradient dz instead)
    w = inputs.WORKLOADS["layer"]
    inp = inputs.make_workload(w)
    rng = np.random.default_rng(77)
    do = torch.tensor(rng.standard_normal((w.B, w.T, w.H, w.Dv)), dtype=F32).to(BF16)
    d = {k_: (None if v_ is None else v_.cuda().contiguous()) for k_, v_ in inp.items()}
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], do.cuda(), d["S0"], None)
    torch.cuda.synchronize()
    for b, h in ((0, 3), (3, 14)):
        sl = lambda t: None if t is None else np64(t[b:b + 1, :, h:h + 1])
        S0 = None if inp["S0"] is None else np64(inp["S0"][b:b + 1, h:h + 1])
        ref = ora.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["z"]),
                           np64(inp["beta_raw"][b:b + 1, :, h:h + 1]), np64(inp["A_log"][h:h + 1]),
                           sl(do), None, S0)
        for n in ("dq", "dk", "dv", "dz"):
            assert_close(g[n][b:b + 1, :, h:h + 1], ref[n], BF16, f"layer b{b} h{h} {n}")
        assert_close(g["dbeta_raw"][b:b + 1, :, h:h + 1], ref["dbeta_raw"], BF16, f"layer b{b} h{h} dbeta")
        assert_close(g["dS0"][b:b + 1, h:h + 1], ref["dS0"], BF16, f"layer b{b} h{h} dS0")


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("H,HV,bias,T", [(2, 4, True, 70), (1, 4, False, 45), (2, 2, True, 33), (4, 8, True, 96)])
def test_backward_grouped_matches_oracle(dtype, H, HV, bias, T):
    # value head hv reads q/k head hv / (HV / H); dq, dk sum over the value heads;
    # the gate bias gradient sums the logit gradient over batch and tokens
    rng = np.random.default_rng(H * 100 + HV * 10 + T)
    B, Dk, Dv = 2, 64, 64
    to = lambda x: torch.tensor(x, dtype=F32).to(dtype)
    q, k = to(rng.standard_normal((B, T, H, Dk))), to(rng.standard_normal((B, T, H, Dk)))
    v = to(rng.standard_normal((B, T, HV, Dv)))
    z = to(rng.standard_normal((B, T, HV, Dk)))
    br = to(rng.standard_normal((B, T, HV)))
    A = torch.tensor(rng.normal(0, 0.5, HV), dtype=F32)
    db = torch.tensor(rng.normal(0, 0.7, (HV, Dk)), dtype=F32) if bias else None
    S0 = torch.tensor(rng.normal(0, 0.3, (B, HV, Dk, Dv)), dtype=F32)
    do = to(rng.standard_normal((B, T, HV, Dv)))
    dST = torch.tensor(rng.normal(0, 0.5, (B, HV, Dk, Dv)), dtype=F32)
    g = kda.chunk_bwd(*(t.cuda() for t in (q, k, v, z, br, A, do)), S0.cuda(), dST.cuda(),
                      dt_bias=None if db is None else db.cuda())
    torch.cuda.synchronize()
    ref = ora.backward_grouped(np64(q), np64(k), np64(v), np64(z), np64(br), np64(A), np64(do), np64(db),
                               np64(dST), np64(S0))
    names = list(NAMES) + (["ddt_bias"] if bias else [])
    for n in names:
        assert_close(g[n], ref[n], F32 if n in ("dA_log", "dS0", "ddt_bias") and dtype == F32 else dtype,
                     f"grouped H{H} HV{HV} {n}")


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_backward_strong_bounded_gate(dtype):
    """g_min = -10: the 16-token factored tile is unsafe (kda_safe_chunk_size
    returns 8); the backward takes every decay factor in one exponent and is
    accepted and exact for it."""
    flags = kda.FLAGS_DEFAULT
    inp, do, dST = case(2, 90, 2, 64, 64, dtype, 4242, flags)
    inp["z"] = (inp["z"].float() * 2.0 + 3.0).to(inp["z"].dtype)
    dev = {k_: (None if v_ is None else v_.cuda().contiguous()) for k_, v_ in inp.items()}
    g = kda.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["z"], dev["beta_raw"], dev["A_log"], do.cuda(),
                      dev["S0"], dST.cuda(), flags=flags, g_min=-10.0)
    torch.cuda.synchronize()
    ref = ora.backward(*(np64(inp[n]) for n in ("q", "k", "v", "z", "beta_raw", "A_log")), np64(do),
                       np64(dST), np64(inp["S0"]), g_min=-10.0, flags=flags)
    for n in NAMES:
        assert_close(g[n], ref[n], F32 if n in ("dA_log", "dS0") and dtype == F32 else dtype, f"g_min -10 {n}")
