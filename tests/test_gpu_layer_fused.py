"""GPU parity of the layer body with the output side fused into the core's
output stores (kda_layer_fwd): y = sigmoid(gate) * o / sqrt(mean o^2 + 1e-6)
* w per head row ("KDA 模块交互式演示" §1.7 完整层; "Implémenter KDA" 'La porte
de sortie de rang plein'), with and without the input-side convolution.

Checks per case:
  * against the unfused pipeline through the C ABI (kda_chunk_fwd or
    kda_chunk_fwd_conv, then kda_output_gate): the final state bit for bit
    (the state path is the same), y to one rounding of the output type (the
    norm's partial sums are added in another order);
  * against the fp64 oracle, step by step: the core's o (of the unfused call)
    and the final state against ora.forward (after ora.conv_silu of each
    input, rounded to the input type, when the convolution is fused), and y
    against ora.output_gate of that o, each to the bars of tests/kda_check.py.
    The norm divides each row by its RMS, so a row's error in y is its error
    in o scaled by max|o| / rms(row): y is held to the bar against the output
    side of the o it was formed from, and o to the bar against the oracle.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_82_amd import inputs, kda
from oracle import kda_oracle as ora
from tests.kda_check import assert_close, np64, to_dev

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load()
    yield
    torch.cuda.synchronize()


def gate_inputs(B, T, H, Dv, dtype, seed, weight=True):
    g = torch.Generator().manual_seed(seed)
    gate = torch.randn(B, T, H, Dv, generator=g).to(dtype)
    w = (torch.rand(Dv, generator=g) + 0.5).float() if weight else None
    return gate, w


def conv_params(B, H, Dk, Dv, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    Cc = H * (2 * Dk + Dv)
    w = (torch.randn(Cc, 4, generator=g) * 0.5).float()
    b = (torch.randn(Cc, generator=g) * 0.1).float()
    st = torch.randn(B, 3, Cc, generator=g).to(dtype)
    return w, b, st


def fused(d, gate, w, chunk, conv=None, flags=7):
    cw, cb, cs = (None, None, None) if conv is None else (t.cuda() for t in conv)
    y, S = kda.layer_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], gate.cuda(),
                         None if w is None else w.cuda(), d["S0"], conv_w=cw, conv_b=cb, conv_state=cs,
                         chunk=chunk, flags=flags)
    torch.cuda.synchronize()
    return y, S


def unfused(d, gate, w, chunk, conv=None, flags=7):
    if conv is None:
        o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], d["S0"], chunk=chunk,
                             flags=flags)
    else:
        cw, cb, cs = (t.cuda() for t in conv)
        o, S = kda.chunk_fwd_conv(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], cw, cb, cs, d["S0"],
                                  chunk=chunk, flags=flags)
    y = kda.output_gate(o, gate.cuda(), None if w is None else w.cuda())
    torch.cuda.synchronize()
    return y, S, o


def oracle(inp, dtype, conv=None, flags=7, heads=None, batch=None, T=None):
    """o and S of the fp64 oracle on (b, h, token) subsets."""
    B, Tt, H, Dk = inp["q"].shape
    Dv = inp["v"].shape[-1]
    q, k, v = (np64(inp[n]) for n in ("q", "k", "v"))
    if conv is not None:
        cw, cb, cs = conv
        o1, o2 = H * Dk, 2 * H * Dk
        parts = ((q, slice(0, o1)), (k, slice(o1, o2)), (v, slice(o2, None)))
        conv_out = []
        for x, sl in parts:
            D = x.shape[-1]
            y, _ = ora.conv_silu(x.reshape(B, Tt, H * D), np64(cw[sl]), np64(cb[sl]), np64(cs[:, :, sl]))
            conv_out.append(torch.tensor(y).to(dtype).double().numpy().reshape(B, Tt, H, D))
        q, k, v = conv_out
    z, br, A, S0 = np64(inp["z"]), np64(inp["beta_raw"]), np64(inp["A_log"]), np64(inp["S0"])
    if T is not None:
        q, k, v, z, br = q[:, :T], k[:, :T], v[:, :T], z[:, :T], br[:, :T]
    if batch is not None:
        q, k, v, z, br = q[batch], k[batch], v[batch], z[batch], br[batch]
        S0 = None if S0 is None else S0[batch]
    if heads is not None:
        q, k, v, z, br = (x[:, :, heads] for x in (q, k, v, z, br))
        A = A[heads]
        S0 = None if S0 is None else S0[:, heads]
    return ora.forward(q, k, v, z, br, A, S0, -5.0, flags)


def check_against_oracle(y_f, o_u, S_f, gate, w, o_ref, S_ref, dtype, what, sel=(slice(None),) * 3):
    """o (of the unfused call) and S against the oracle's core; y against the
    oracle's output side of that o.  sel picks (batch, tokens, heads)."""
    bb, tt, hh = sel
    o_sel = o_u[bb, tt, hh]
    assert_close(o_sel, o_ref, dtype, f"{what} o")
    y_ref = ora.output_gate(np64(o_sel), np64(gate[bb, tt, hh]), np64(w))
    assert_close(y_f[bb, tt, hh], y_ref, dtype, f"{what} y")
    if S_ref is not None:
        assert_close(S_f[bb, hh], S_ref, dtype, f"{what} S")


def assert_one_rounding(y_f, y_u, dtype, what):
    """The fused and unfused y differ only by the order of the norm's sum:
    within one rounding of the output type (relative 2^-7 for bf16, 1e-5 for
    fp32) element by element."""
    a, b = y_f.double().cpu(), y_u.double().cpu()
    rel = 2.0 ** -7 if dtype == BF16 else 1e-5
    bad = (a - b).abs() > rel * b.abs() + 1e-6
    assert not bool(bad.any()), f"{what}: {int(bad.sum())} elements differ beyond one rounding"


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Dk,Dv,chunk,T,weight", [
    (128, 128, 32, 200, True), (128, 128, 64, 130, False), (64, 64, 16, 77, True),
    (16, 16, 16, 2, True), (128, 32, 32, 1, True), (64, 128, 64, 67, False),
    (32, 64, 32, 96, True), (128, 16, 64, 100, True),
])
def test_layer_fused_equals_unfused_and_oracle(dtype, Dk, Dv, chunk, T, weight):
    B, H = 2, 3
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "bf16" if dtype == BF16 else "f32", seed=T * 5 + Dk + Dv + chunk,
                             a_std=0.5, s_std=0.2)
    gate, w = gate_inputs(B, T, H, Dv, dtype, seed=T + Dv, weight=weight)
    d = to_dev(inp)
    y_f, S_f = fused(d, gate, w, chunk)
    y_u, S_u, o_u = unfused(d, gate, w, chunk)
    assert torch.equal(S_f, S_u), "fused S differs from chunk_fwd"
    assert_one_rounding(y_f, y_u, dtype, f"y Dk{Dk} Dv{Dv} C{chunk} T{T}")
    o_ref, S_ref = oracle(inp, dtype)
    check_against_oracle(y_f, o_u, S_f, gate, w, o_ref, S_ref, dtype, f"fused Dk{Dk} Dv{Dv} C{chunk} T{T}")


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Dk,Dv,chunk,T", [(128, 128, 32, 150), (64, 64, 64, 65), (32, 128, 16, 40)])
def test_layer_fused_with_convolution(dtype, Dk, Dv, chunk, T):
    B, H = 2, 2
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "bf16" if dtype == BF16 else "f32", seed=900 + T + Dk,
                             a_std=0.5, s_std=0.2)
    gate, w = gate_inputs(B, T, H, Dv, dtype, seed=T)
    conv = conv_params(B, H, Dk, Dv, dtype, seed=Dk + Dv)
    d = to_dev(inp)
    y_f, S_f = fused(d, gate, w, chunk, conv=conv)
    y_u, S_u, o_u = unfused(d, gate, w, chunk, conv=conv)
    assert torch.equal(S_f, S_u)
    assert_one_rounding(y_f, y_u, dtype, f"conv y Dk{Dk} Dv{Dv} C{chunk} T{T}")
    o_ref, S_ref = oracle(inp, dtype, conv=conv)
    check_against_oracle(y_f, o_u, S_f, gate, w, o_ref, S_ref, dtype, "fused conv")


def test_layer_fused_repeatable_and_zero_head():
    """Two calls agree bit for bit (the groups' partials are added in a fixed
    order); a head whose inputs are all zero gives y = 0 (the epsilon)."""
    B, T, H, D = 2, 100, 4, 128
    inp = inputs.make_inputs(B, T, H, D, D, "bf16", seed=77, a_std=0.5, s_std=0.0)
    inp["S0"] = None
    inp["v"][1, :, 2] = 0
    gate, w = gate_inputs(B, T, H, D, BF16, seed=78)
    d = to_dev(inp)
    y1, S1 = fused(d, gate, w, 32)
    y2, S2 = fused(d, gate, w, 32)
    assert torch.equal(y1, y2) and torch.equal(S1, S2)
    assert torch.count_nonzero(y1[1, :, 2]) == 0


def test_layer_fused_not_resident_takes_separate_output_side():
    """More (b, h) pairs than the device holds at once: the call runs the core
    into y and the output side in place; the results still match."""
    props = torch.cuda.get_device_properties(0)
    B, T, H, D = 3 * props.multi_processor_count // 16 + 1, 40, 16, 128   # > one workgroup per CU at 1 wave
    inp = inputs.make_inputs(B, T, H, D, D, "bf16", seed=31, a_std=0.5, s_std=0.2)
    gate, w = gate_inputs(B, T, H, D, BF16, seed=32)
    d = to_dev(inp)
    y_f, S_f = fused(d, gate, w, 32)
    y_u, S_u, o_u = unfused(d, gate, w, 32)
    assert torch.equal(S_f, S_u)
    assert torch.equal(y_f, y_u), "the separate output side is the unfused pipeline itself"
    for bb, h in ((0, 0), (B - 1, H - 1)):
        o_ref, S_ref = oracle(inp, BF16, heads=[h], batch=slice(bb, bb + 1))
        check_against_oracle(y_f, o_u, S_f, gate, w, o_ref, S_ref, BF16, f"not resident b{bb} h{h}",
                             (slice(bb, bb + 1), slice(None), slice(h, h + 1)))


def test_layer_fused_layer_workload():
    """B4 T4096 H16 D128 bf16 at the benchmarked chunk with the convolution:
    the unfused pipeline over the whole call, and the oracle on three (b, h)
    pairs over all tokens."""
    w_ = inputs.WORKLOADS["layer"]
    inp = inputs.make_workload(w_)
    gate, w = gate_inputs(w_.B, w_.T, w_.H, w_.Dv, BF16, seed=4243)
    conv = conv_params(w_.B, w_.H, w_.Dk, w_.Dv, BF16, seed=4242)
    d = to_dev(inp)
    y_f, S_f = fused(d, gate, w, 32, conv=conv)
    y_u, S_u, o_u = unfused(d, gate, w, 32, conv=conv)
    assert torch.equal(S_f, S_u)
    assert_one_rounding(y_f, y_u, BF16, "layer workload y")
    for bb, h in ((0, 0), (2, 9), (3, 15)):
        o_ref, S_ref = oracle(inp, BF16, conv=conv, heads=[h], batch=slice(bb, bb + 1))
        check_against_oracle(y_f, o_u, S_f, gate, w, o_ref, S_ref, BF16, f"layer b{bb} h{h}",
                             (slice(bb, bb + 1), slice(None), slice(h, h + 1)))


def test_layer_fused_long_workload_slices():
    """B1 T65536 H32 D128 bf16 (chunk 32): the chunk blocks exceed one slice,
    so the call alternates the kernels over slices, each with its own exchange
    area marks; the unfused pipeline over the whole call, the oracle on one
    head over the first 2048 tokens."""
    w_ = inputs.WORKLOADS["long"]
    inp = inputs.make_workload(w_)
    assert kda.kernel_count(w_.B, w_.T, w_.H, w_.Dk, w_.Dv, 32, BF16) > 2, "one slice: the case needs several"
    gate, w = gate_inputs(w_.B, w_.T, w_.H, w_.Dv, BF16, seed=4244)
    d = to_dev(inp)
    y_f, S_f = fused(d, gate, w, 32)
    y_u, S_u, o_u = unfused(d, gate, w, 32)
    assert torch.equal(S_f, S_u)
    assert_one_rounding(y_f, y_u, BF16, "long workload y")
    o_ref, _ = oracle(inp, BF16, heads=[5], T=2048)
    check_against_oracle(y_f, o_u, S_f, gate, w, o_ref, None, BF16, "long h5",
                         (slice(None), slice(0, 2048), slice(5, 6)))
