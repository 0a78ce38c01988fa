"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test runs the kernels of libkda.so through the ctypes binding and
compares with the oracle on the same seeded inputs, to the bars stated in
tests/kda_check.py.  Sizes are chosen so that the oracle finishes in seconds
while covering several tiles and a ragged tail; the full-size workloads are
checked on sampled heads (the heads are independent) or prefixes.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_82_amd import inputs, kda
from oracle import kda_oracle as ora
from tests.kda_check import ATOL_BF16, RTOL_F32, assert_close, max_rel, np64, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load()
    yield
    torch.cuda.synchronize()


def run_chunk(inp, chunk=64, g_min=-5.0, flags=7, **kw):
    d = to_dev(inp)
    out = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], d["S0"],
                        chunk=chunk, g_min=g_min, flags=flags, **kw)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ kda_step

@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (128, 128), (16, 128), (128, 16)])
def test_step_matches_oracle(dtype, Dk, Dv):
    inp = inputs.make_inputs(3, 1, 5, Dk, Dv, "bf16" if dtype == BF16 else "f32", seed=Dk * 7 + Dv,
                             a_std=0.5, s_std=0.3)
    d = to_dev(inp)
    S = d["S0"].clone()
    o = kda.step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(),
                 d["z"][:, 0].contiguous(), d["beta_raw"][:, 0].contiguous(), d["A_log"], S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp)
    # o is rounded to the input dtype; the state is fp32 arithmetic for either dtype
    assert_close(o, o_ref[:, 0], dtype, "step o")
    assert max_rel(S, S_ref) <= RTOL_F32


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("flags", [0, 1, 2, 4, 6])
def test_step_switches(flags, D):
    rng = np.random.default_rng(flags)
    B, H, Dk, Dv = 2, 3, D, D
    q = torch.tensor(ora.l2_normalize(rng.standard_normal((B, 1, H, Dk))), dtype=F32)
    k = torch.tensor(ora.l2_normalize(rng.standard_normal((B, 1, H, Dk))), dtype=F32)
    z = torch.tensor(rng.uniform(-4.9, -0.1, (B, 1, H, Dk)) if not flags & 4 else rng.standard_normal((B, 1, H, Dk)), dtype=F32)
    br = torch.tensor(rng.uniform(0.05, 0.95, (B, 1, H)) if not flags & 2 else rng.standard_normal((B, 1, H)), dtype=F32)
    inp = {"q": q, "k": k, "v": torch.randn(B, 1, H, Dv), "z": z, "beta_raw": br,
           "A_log": torch.tensor(rng.normal(0, 0.5, H), dtype=F32),
           "S0": torch.randn(B, H, Dk, Dv)}
    d = to_dev(inp)
    S = d["S0"].clone()
    o = kda.step(*(d[n][:, 0].contiguous() for n in ("q", "k", "v", "z", "beta_raw")), d["A_log"], S,
                 flags=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp, flags=flags)
    assert max_rel(o, o_ref[:, 0]) <= RTOL_F32 and max_rel(S, S_ref) <= RTOL_F32


# ------------------------------------------------------------ kda_chunk_fwd

def check_chunk(inp, dtype, chunk=64, flags=7, what=""):
    o, S = run_chunk(inp, chunk=chunk, flags=flags)
    o_ref, S_ref = oracle_forward(inp, flags=flags)
    e1 = assert_close(o, o_ref, dtype, f"{what} o")
    e2 = assert_close(S, S_ref, dtype, f"{what} S")
    return e1, e2


def test_tiny_workload():
    w = inputs.WORKLOADS["tiny"]
    check_chunk(inputs.make_workload(w), F32, chunk=w.chunk, what="tiny")


def test_small_workload():
    w = inputs.WORKLOADS["small"]
    check_chunk(inputs.make_workload(w), F32, chunk=w.chunk, what="small")


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Dk,Dv,chunk,T", [
    (16, 16, 16, 37), (32, 32, 32, 100), (64, 64, 64, 130), (128, 128, 64, 200),
    (128, 64, 32, 77), (64, 128, 16, 50), (32, 128, 64, 65), (128, 32, 16, 33),
    (16, 64, 64, 1), (128, 128, 16, 64),
])
def test_chunk_shapes(dtype, Dk, Dv, chunk, T):
    inp = inputs.make_inputs(2, T, 3, Dk, Dv, "bf16" if dtype == BF16 else "f32",
                             seed=Dk + 3 * Dv + chunk + T, a_std=0.5, s_std=0.2)
    check_chunk(inp, dtype, chunk=chunk, what=f"Dk{Dk} Dv{Dv} C{chunk} T{T}")


@pytest.mark.parametrize("flags", [0, 1, 2, 4, 3, 5, 6])
def test_chunk_switches(flags):
    rng = np.random.default_rng(100 + flags)
    B, T, H, Dk, Dv = 1, 90, 2, 64, 64
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if not flags & 1:
        q, k = ora.l2_normalize(q), ora.l2_normalize(k)
    z = rng.standard_normal((B, T, H, Dk)) if flags & 4 else rng.uniform(-4.99, -0.01, (B, T, H, Dk))
    br = rng.standard_normal((B, T, H)) if flags & 2 else rng.uniform(0.01, 0.99, (B, T, H))
    t = lambda x: torch.tensor(x, dtype=F32)
    inp = {"q": t(q), "k": t(k), "v": torch.randn(B, T, H, Dv), "z": t(z), "beta_raw": t(br),
           "A_log": t(rng.normal(0, 0.5, H)), "S0": torch.randn(B, H, Dk, Dv) * 0.1}
    check_chunk(inp, F32, chunk=32, flags=flags, what=f"flags {flags}")


def test_chunk_strongest_decay_is_finite():
    # worst-case gate (every token at the lower bound) exercises the e^80 factor range
    B, T, H, Dk, Dv = 1, 128, 2, 64, 64
    rng = np.random.default_rng(5)
    inp = {"q": torch.randn(B, T, H, Dk), "k": torch.randn(B, T, H, Dk), "v": torch.randn(B, T, H, Dv),
           "z": torch.full((B, T, H, Dk), -5.0 + 1e-4), "beta_raw": torch.randn(B, T, H),
           "A_log": torch.zeros(H), "S0": torch.randn(B, H, Dk, Dv)}
    check_chunk(inp, F32, chunk=64, flags=3, what="g = g_min")
    inp = {k_: (v_.to(BF16) if k_ in ("q", "k", "v", "z", "beta_raw") else v_) for k_, v_ in inp.items()}
    check_chunk(inp, BF16, chunk=64, flags=3, what="g = g_min bf16")


def test_chunk_empty_sequence_passes_state_through():
    B, H, Dk, Dv = 2, 3, 64, 32
    inp = inputs.make_inputs(B, 0, H, Dk, Dv, "f32", seed=1, s_std=0.5)
    d = to_dev(inp)
    o, S, M = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], d["S0"], want_M=True)
    torch.cuda.synchronize()
    assert torch.equal(S, d["S0"])
    assert torch.equal(M, torch.eye(Dk, device="cuda").expand(B, H, Dk, Dk))


# ------------------------------------------------------------- KCP on GPU

@pytest.mark.parametrize("dtype", [F32, BF16])
def test_segment_fragment_matches_oracle(dtype):
    # M_out is the product of per-token transitions; P_out gives o(S0) = o(0) + P S0.
    B, T, H, Dk, Dv = 2, 150, 2, 64, 32
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "bf16" if dtype == BF16 else "f32", seed=77, a_std=0.5)
    o0, St, M, P = run_chunk(inp, chunk=32, want_M=True, want_P=True)
    qh, kh, g, beta = ora.prepare(*(np64(inp[n]) for n in ("q", "k", "z", "beta_raw")), np64(inp["A_log"]))
    M_ref, St_ref = ora.segment_fragment(kh, np64(inp["v"]), g, beta)
    assert_close(M, M_ref, dtype, "M")
    assert_close(St, St_ref, dtype, "S_tilde")
    S_in = torch.randn(B, H, Dk, Dv) * 0.5
    o_ref, _ = ora.recurrent(qh, kh, np64(inp["v"]), g, beta, np64(S_in))
    o_fix = np64(o0) + np.einsum("bthk,bhkv->bthv", np64(P), np64(S_in))
    assert_close(o_fix, o_ref, dtype, "o + P S_in")
    assert_close(P, ora.readout_map(qh, kh, g, beta), dtype, "readout map P")


@pytest.mark.parametrize("n,Dk,Dv", [(5, 128, 64), (1, 128, 128), (2, 16, 32), (7, 32, 16), (4, 64, 128),
                                     (9, 128, 16)])
def test_compose_matches_oracle(n, Dk, Dv):
    rng = np.random.default_rng(3 + n + Dk + Dv)
    B, H = 2, 3
    M = torch.tensor(rng.normal(0, 0.15, (n, B, H, Dk, Dk)), dtype=F32)
    St = torch.tensor(rng.standard_normal((n, B, H, Dk, Dv)), dtype=F32)
    S_in = torch.tensor(rng.standard_normal((B, H, Dk, Dv)), dtype=F32)
    out = kda.segment_compose(M.cuda(), St.cuda(), S_in.cuda())
    torch.cuda.synchronize()
    ref = ora.compose([(np64(M[s]), np64(St[s])) for s in range(n)], np64(S_in))
    for s in range(n):
        assert max_rel(out[s], ref[s]) <= RTOL_F32
    out0 = kda.segment_compose(M.cuda(), St.cuda(), None)
    ref0 = ora.compose([(np64(M[s]), np64(St[s])) for s in range(n)], None)
    torch.cuda.synchronize()
    assert max_rel(out0[-1], ref0[-1]) <= RTOL_F32


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Dk,Dv,Tseg", [(16, 16, 7), (32, 32, 530), (64, 128, 530), (128, 64, 45),
                                        (128, 128, 530), (16, 128, 100), (128, 16, 530)])
@pytest.mark.parametrize("with_state", [False, True])
def test_fixup_matches_oracle(dtype, Dk, Dv, Tseg, with_state):
    # every strip grouping (Dv 16, 32, 64, 128), tiles of 512 tokens with a
    # ragged tail, a segment shorter than one 16-token block, with and without
    # an incoming state for the first segment
    rng = np.random.default_rng(Dk * 1000 + Dv * 10 + Tseg + with_state)
    n, B, H = 3, 2, 2
    P = torch.tensor(rng.normal(0, 0.3, (n, B, Tseg, H, Dk))).to(dtype)
    o = torch.tensor(rng.standard_normal((n, B, Tseg, H, Dv))).to(dtype)
    S_pref = torch.tensor(rng.standard_normal((n, B, H, Dk, Dv)), dtype=F32)
    S_in = torch.tensor(rng.standard_normal((B, H, Dk, Dv)), dtype=F32) if with_state else None
    ref = ora.segment_fixup(np64(o), np64(P), np64(S_pref), np64(S_in))
    out = kda.segment_fixup(P.cuda(), S_pref.cuda(), o.cuda(), None if S_in is None else S_in.cuda())
    torch.cuda.synchronize()
    assert_close(out, ref, dtype, "fixed-up o")
    if not with_state:
        assert torch.equal(out[0].cpu(), o[0]), "the first segment has no incoming state: untouched"


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_segmented_equals_full_run(dtype):
    # a B = 1 sequence cut into n equal segments is the batch [n, T/n]: fragments in
    # one call, compose, then fix up the outputs with P.
    n, Tseg, H, Dk, Dv = 4, 96, 2, 64, 64
    inp = inputs.make_inputs(1, n * Tseg, H, Dk, Dv, "bf16" if dtype == BF16 else "f32", seed=8, a_std=0.5)
    o_full, S_full = run_chunk(inp, chunk=32)
    seg = {k_: (v_.reshape(n, Tseg, *v_.shape[2:]) if k_ in ("q", "k", "v", "z", "beta_raw") else v_)
           for k_, v_ in inp.items()}
    o0, St, M, P = run_chunk(seg, chunk=32, want_M=True, want_P=True)
    S_pref = kda.segment_compose(M.unsqueeze(1).contiguous(), St.unsqueeze(1).contiguous())
    o_fix = kda.segment_fixup(P.unsqueeze(1).contiguous(), S_pref, o0.unsqueeze(1).contiguous())
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp)
    assert_close(o_fix.reshape(o_full.shape), o_ref, dtype, "segmented o")
    assert_close(S_pref[-1, 0], S_ref, dtype, "segmented S")
    assert_close(o_full, o_ref, dtype, "full o")


# ------------------------------------------------------------ cross-path

def test_step_loop_matches_chunk():
    B, T, H, Dk, Dv = 2, 70, 3, 64, 64
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "f32", seed=21, a_std=0.5, s_std=0.2)
    o_c, S_c = run_chunk(inp, chunk=32)
    d = to_dev(inp)
    S = d["S0"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.step(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "z", "beta_raw")),
                             d["A_log"], S))
    torch.cuda.synchronize()
    assert max_rel(torch.stack(outs, 1), np64(o_c)) <= RTOL_F32
    assert max_rel(S, np64(S_c)) <= RTOL_F32


def test_chunk_size_invariance_and_resume():
    B, T, H, Dk, Dv = 1, 160, 2, 128, 64
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "f32", seed=22, a_std=0.5, s_std=0.2)
    res = {c: run_chunk(inp, chunk=c) for c in (16, 32, 64)}
    for c in (16, 32):
        assert max_rel(res[c][0], np64(res[64][0])) <= RTOL_F32
        assert max_rel(res[c][1], np64(res[64][1])) <= RTOL_F32
    a = {k_: (v_[:, :70].contiguous() if k_ in ("q", "k", "v", "z", "beta_raw") else v_) for k_, v_ in inp.items()}
    oa, Sa = run_chunk(a)
    b = {k_: (v_[:, 70:].contiguous() if k_ in ("q", "k", "v", "z", "beta_raw") else v_) for k_, v_ in inp.items()}
    b["S0"] = Sa.cpu()
    ob, Sb = run_chunk(b)
    assert max_rel(torch.cat([oa, ob], 1), np64(res[64][0])) <= RTOL_F32
    assert max_rel(Sb, np64(res[64][1])) <= RTOL_F32


def test_bitwise_repeatable_and_state_aliasing():
    # no atomics anywhere: two runs agree bit for bit; S_out may alias S0.
    inp = inputs.make_inputs(2, 300, 4, 128, 128, "bf16", seed=23, a_std=0.5, s_std=0.1)
    o1, S1 = run_chunk(inp)
    o2, S2 = run_chunk(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    d = to_dev(inp)
    S = d["S0"].clone()
    kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], S, S_out=S)
    torch.cuda.synchronize()
    assert torch.equal(S, S1)


# ------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("chunk", [32, 64])
def test_layer_workload_sampled_heads(chunk):
    """B4 T4096 H16 D128 bf16, one full GPU run per state chunk (32 is the
    benchmarked launch, 64 the workload's named chunk): every one of the 64
    (b, h) pairs against the oracle over the first 512 tokens (the output is
    causal, so the full run's prefix is the prefix run), and three pairs over
    all 4096 tokens with their final state, which covers every chunk of the
    serial carry and the inter kernel's operand ring wrapping many times."""
    w = inputs.WORKLOADS["layer"]
    inp = inputs.make_workload(w)
    o, S = run_chunk(inp, chunk=chunk)
    Tp = 512
    o_ref, _ = oracle_forward(inp, T=Tp)
    assert_close(o[:, :Tp], o_ref, BF16, f"layer C{chunk} o[:, :{Tp}] all heads")
    for b, h in ((0, 0), (1, 7), (3, 15)):
        sub = {k_: (v_[b:b + 1] if v_ is not None and k_ != "A_log" else v_) for k_, v_ in inp.items()}
        o_ref, S_ref = oracle_forward(sub, heads=[h])
        assert_close(o[b:b + 1, :, h:h + 1], o_ref, BF16, f"layer C{chunk} o b{b} h{h}")
        assert_close(S[b:b + 1, h:h + 1], S_ref, BF16, f"layer C{chunk} S b{b} h{h}")


def test_decode_workload():
    """B256 H32 D128, bf16 q/k/v/z, fp32 state, all 1024 steps of the workload:
    every (b, h) against the oracle for the first 4 steps, and a fixed subset
    of 64 (b, h) pairs (outputs and, at the end, states) over all 1024 steps."""
    w = inputs.WORKLOADS["decode"]
    S0, A_log = inputs.make_decode_state(w)
    S = S0.cuda()
    A = A_log.cuda()
    rng = np.random.default_rng(0)
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, 64), rng.integers(0, w.H, 64))]
    bi = torch.tensor([b for b, _ in pairs])
    hi = torch.tensor([h for _, h in pairs])
    Sref_full = np64(S0)
    Sref_sub = np64(S0[bi, hi])[None]   # [1, 64, Dk, Dv]
    A_sub = np64(A_log[hi])
    worst = 0.0
    for s in range(w.steps):
        st = inputs.make_decode_step(w, s)
        d = to_dev(st)
        o = kda.step(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], A, S)
        if s < 4:
            o_ref, Sref_full = ora.step(Sref_full, *(np64(st[n]) for n in ("q", "k", "v", "z", "beta_raw")),
                                        np64(A_log))
            torch.cuda.synchronize()
            assert_close(o, o_ref, BF16, f"decode o step {s}")
            assert max_rel(S, Sref_full) <= RTOL_F32
        o_sub, Sref_sub = ora.step(Sref_sub, *(np64(st[n][bi, hi])[None] for n in ("q", "k", "v", "z", "beta_raw")),
                                   A_sub)
        worst = max(worst, assert_close(o.cpu()[bi, hi], o_sub[0], BF16, f"decode subset o step {s}"))
    assert max_rel(S.cpu()[bi, hi], Sref_sub[0]) <= RTOL_F32
    print(f"decode: worst subset output error over {w.steps} steps {worst:.3e}")


@pytest.mark.parametrize("chunk", [32, 64])
def test_long_workload_segmented(chunk):
    """B1 T65536 H32 D128 bf16 cut into 8 x 8192: fragments, compose and fixup
    equal the single full run; the oracle checks the first 2048 tokens on 2 heads.
    Chunk 32 is the benchmarked launch, 64 the workload's named chunk."""
    w = inputs.WORKLOADS["long"]
    inp = inputs.make_workload(w)
    n, Tseg = w.segments, w.T // w.segments
    d = to_dev(inp)
    o_full, S_full = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], None, chunk=chunk)
    seg = {k_: (v_.reshape(n, Tseg, *v_.shape[2:]) if k_ in ("q", "k", "v", "z", "beta_raw") else v_)
           for k_, v_ in d.items()}
    o0, St, M, P = kda.chunk_fwd(seg["q"], seg["k"], seg["v"], seg["z"], seg["beta_raw"], seg["A_log"], None,
                                 chunk=chunk, want_M=True, want_P=True)
    S_pref = kda.segment_compose(M.unsqueeze(1).contiguous(), St.unsqueeze(1).contiguous())
    o_seg = kda.segment_fixup(P.unsqueeze(1).contiguous(), S_pref, o0.unsqueeze(1).contiguous())
    torch.cuda.synchronize()
    o_seg = o_seg.reshape(o_full.shape)
    scale = float(o_full.abs().max())
    assert float((o_seg.float() - o_full.float()).abs().max()) <= ATOL_BF16 * scale
    assert max_rel(S_pref[-1, 0], np64(S_full)) <= ATOL_BF16
    del seg, o0, P, d
    for h in (0, 31):
        o_ref, _ = oracle_forward(inp, heads=[h], T=2048)
        assert_close(o_full[:, :2048, h:h + 1], o_ref, BF16, f"long prefix h{h}")


def test_sliced_sequence_matches_oracle():
    """Enough heads that the sequence is cut into slices: the state and
    transition carried between slices must match the oracle."""
    # 9000 heads: one chunk's blocks (9000 x 59 904 B) pass half the 1 GiB
    # slice budget, so each of the 3 chunks is a slice of its own
    B, T, H, Dk, Dv = 1, 130, 9000, 128, 128
    assert kda.kernel_count(B, T, H, Dk, Dv, 64, BF16) == 6   # 3 slices x (intra, inter)
    inp = inputs.make_inputs(B, T, H, Dk, Dv, "bf16", seed=31, a_std=0.5, s_std=0.2)
    o, S, M, P = run_chunk(inp, chunk=64, want_M=True, want_P=True)
    for b, h in ((0, 0), (0, H - 1)):
        sub = {k_: (v_[b:b + 1] if v_ is not None and k_ != "A_log" else v_) for k_, v_ in inp.items()}
        o_ref, S_ref = oracle_forward(sub, heads=[h])
        assert_close(o[b:b + 1, :, h:h + 1], o_ref, BF16, f"sliced o b{b} h{h}")
        assert_close(S[b:b + 1, h:h + 1], S_ref, BF16, f"sliced S b{b} h{h}")
        qh, kh, g, beta = ora.prepare(*(np64(sub[n][:, :, [h]]) for n in ("q", "k", "z", "beta_raw")),
                                      np64(inp["A_log"])[[h]])
        M_ref, _ = ora.segment_fragment(kh, np64(sub["v"][:, :, [h]]), g, beta)
        assert_close(M[b:b + 1, h:h + 1], M_ref, BF16, f"sliced M b{b} h{h}")


@pytest.mark.parametrize("dtype,B,H,want,Dk", [
    (BF16, 2, 20, False, 128), (BF16, 2, 48, False, 128), (BF16, 1, 24, True, 128), (BF16, 3, 16, True, 128),
    (F32, 2, 20, False, 128), (F32, 2, 48, True, 128), (BF16, 4, 48, True, 16), (F32, 4, 48, True, 16),
    (BF16, 4, 64, False, 128), (BF16, 2, 64, True, 128), (BF16, 8, 64, True, 128),
])
def test_inter_wave_counts(dtype, B, H, want, Dk):
    """Head counts spread over the inter kernel's 1, 2, 4 and 8 compute waves
    per workgroup (the launch takes the fewest waves whose grid is resident at
    once: on 256 CUs with one workgroup each, 8 value strips per head give 1
    wave up to 32 heads, 2 up to 64, 4 up to 128, then 8 for bf16 up to 256;
    the transition strips double the strip count; a grid that is not resident
    takes the most waves), each against the oracle on every head.  With Dk = 16 the one
    transition strip shares a workgroup's output rows with value strips; its
    transition M decays to about 1e-4 of the identity over the 45 tokens, so in
    bf16 (operands rounded to 2^-8 of entries that start near 1) M is held to
    the bar only in the fp32 case, while o and o(0) + P S0 check the rows."""
    inp = inputs.make_inputs(B, 45, H, Dk, 128, "bf16" if dtype == BF16 else "f32", seed=B * H + want,
                             a_std=0.5, s_std=0.2)
    o, S, *MP = run_chunk(inp, chunk=32, want_M=want, want_P=want)
    o_ref, S_ref = oracle_forward(inp)
    assert_close(o, o_ref, dtype, f"waves B{B} H{H} o")
    assert_close(S, S_ref, dtype, f"waves B{B} H{H} S")
    if want:
        M, P = MP
        qh, kh, g, beta = ora.prepare(*(np64(inp[n]) for n in ("q", "k", "z", "beta_raw")), np64(inp["A_log"]))
        M_ref, _ = ora.segment_fragment(kh, np64(inp["v"]), g, beta)
        if not (dtype == BF16 and Dk == 16):
            assert_close(M, M_ref, dtype, f"waves B{B} H{H} M")
        o_zero, _ = ora.recurrent(qh, kh, np64(inp["v"]), g, beta, None)
        o_fix = o_zero + np.einsum("bthk,bhkv->bthv", np64(P), np64(inp["S0"]))
        assert_close(o_fix, o_ref, dtype, f"waves B{B} H{H} o(0) + P S0")


# ------------------------------------------------------ grouped value heads

def grouped_case(B, T, H, HV, Dk, Dv, dtype, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    cast = (lambda x: x.to(dtype))
    q = cast(torch.randn(B, T, H, Dk, generator=g))
    k = cast(torch.randn(B, T, H, Dk, generator=g))
    v = cast(torch.randn(B, T, HV, Dv, generator=g))
    z = cast(torch.randn(B, T, HV, Dk, generator=g))
    br = cast(torch.randn(B, T, HV, generator=g))
    A = (torch.randn(HV, generator=g) * 0.5).float()
    db = (torch.randn(HV, Dk, generator=g) * 0.5).float() if bias else None
    S0 = (torch.randn(B, HV, Dk, Dv, generator=g) * 0.2).float()
    return q, k, v, z, br, A, db, S0


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("B,T,H,HV,Dk,Dv,bias", [
    (2, 77, 2, 6, 64, 64, True), (1, 130, 1, 4, 128, 128, True), (2, 45, 3, 3, 32, 64, True),
    (1, 33, 2, 8, 128, 64, False),
])
def test_grouped_chunk_matches_oracle(dtype, B, T, H, HV, Dk, Dv, bias):
    q, k, v, z, br, A, db, S0 = grouped_case(B, T, H, HV, Dk, Dv, dtype, seed=T + 10 * HV + Dk)
    if not bias:
        db = None
    o, S = kda.chunk_fwd(*(t.cuda() for t in (q, k, v, z, br, A)), S0.cuda(), chunk=32,
                         dt_bias=None if db is None else db.cuda())
    torch.cuda.synchronize()
    o_ref, S_ref = ora.forward_grouped(np64(q), np64(k), np64(v), np64(z), np64(br), np64(A), np64(db), np64(S0))
    assert_close(o, o_ref, dtype, f"grouped o H{H} HV{HV}")
    assert_close(S, S_ref, dtype, f"grouped S H{H} HV{HV}")


def test_grouped_with_equal_heads_and_no_bias_is_the_plain_call():
    q, k, v, z, br, A, _, S0 = grouped_case(2, 70, 3, 3, 64, 64, BF16, seed=3, bias=False)
    args = [t.cuda() for t in (q, k, v, z, br, A)]
    o1, S1 = kda.chunk_fwd(*args, S0.cuda(), chunk=32)
    zero = torch.zeros(3, 64, device="cuda")
    o2, S2 = kda.chunk_fwd(*args, S0.cuda(), chunk=32, dt_bias=zero)   # grouped entry, zero bias
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_grouped_step_matches_oracle(dtype):
    B, H, HV, Dk, Dv = 3, 2, 8, 128, 128
    q, k, v, z, br, A, db, S0 = grouped_case(B, 1, H, HV, Dk, Dv, dtype, seed=17)
    S = S0.cuda().clone()
    o = kda.step(q[:, 0].cuda().contiguous(), k[:, 0].cuda().contiguous(), v[:, 0].cuda().contiguous(),
                 z[:, 0].cuda().contiguous(), br[:, 0].cuda().contiguous(), A.cuda(), S, dt_bias=db.cuda())
    torch.cuda.synchronize()
    o_ref, S_ref = ora.step_grouped(np64(S0), np64(q[:, 0]), np64(k[:, 0]), np64(v[:, 0]), np64(z[:, 0]),
                                    np64(br[:, 0]), np64(A), np64(db))
    assert_close(o, o_ref, dtype, "grouped step o")
    assert_close(S, S_ref, F32, "grouped step S")   # the state is fp32 in both paths


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("B,H,HV", [(7, 45, 45), (5, 120, 120), (40, 2, 8)])
def test_step_heads_beyond_one_round(dtype, B, H, HV):
    """Dk = Dv = 128 decode with more (b, h) heads than one resident round of
    workgroups (315, 600 and 320 heads), so that workgroups carry two or three
    heads each in uneven numbers: three steps in a row, every head against
    the oracle (grouped heads with a gate bias in the last case)."""
    q, k, v, z, br, A, db, S0 = grouped_case(B, 3, H, HV, 128, 128, dtype, seed=B * 1000 + HV, bias=HV != H)
    print(f"step: B{B} H{H} HV{HV} D128 {dtype}", flush=True)
    S = S0.cuda().clone()
    S_ref = np64(S0)
    for t in range(3):
        args = [x[:, t].cuda().contiguous() for x in (q, k, v, z, br)]
        o = kda.step(*args, A.cuda(), S, dt_bias=None if db is None else db.cuda())
        torch.cuda.synchronize()
        o_ref, S_ref = ora.step_grouped(S_ref, *(np64(x[:, t]) for x in (q, k, v, z, br)), np64(A),
                                        None if db is None else np64(db))
        assert_close(o, o_ref, dtype, f"step {t} o")
    assert_close(S, S_ref, F32, "state after three steps")
