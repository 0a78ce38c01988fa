"""HIP graph capture of the C-ABI calls a serving loop captures: the
allocation-free chunk call, the chunk call on a caller workspace, the layer
call with the fused output side and the decode step.  The library launches kernels on the caller's stream and never
allocates, synchronises or clears memory with a memset, so a call records
into a graph as it is.  Each graph is replayed three times on new inputs
copied into its static tensors, with eager work and synchronisations between
the replays; every replay must equal the eager call on the same inputs bit
for bit."""

import pytest
import torch

from gated_delta_rule_82_amd import inputs, kda
from tests.kda_check import to_dev

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "z", "beta_raw", "A_log", "S0")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load()
    yield
    torch.cuda.synchronize()


def capture(fn):
    """Warm fn up eagerly on a side stream, then record it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("entry", ["noalloc", "workspace"])
def test_chunk_call_replays_equal_eager(entry):
    B, T, H, D, C = 2, 300, 4, 128, 32
    sets = [to_dev(inputs.make_inputs(B, T, H, D, D, "bf16", seed=900 + i, a_std=0.5, s_std=0.1))
            for i in range(3)]
    st = {n: sets[0][n].clone() for n in NAMES}
    o = torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda")
    S = torch.empty(B, H, D, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(B, T, H, D, D, C, torch.bfloat16), dtype=torch.uint8, device="cuda")

    def call():
        args = tuple(st[n] for n in NAMES)
        if entry == "noalloc":
            kda.chunk_fwd_noalloc(*args, chunk=C, o=o, S_out=S)
        else:
            kda.chunk_fwd(*args, chunk=C, o=o, S_out=S, workspace=ws)

    print(f"graph: chunk call ({entry}) B{B} T{T} H{H} D{D} bf16 chunk {C}", flush=True)
    g = capture(call)
    for i, inp in enumerate(sets):
        for n in NAMES:
            st[n].copy_(inp[n])
        g.replay()
        torch.cuda.synchronize()
        o_g, S_g = o.clone(), S.clone()
        o_e, S_e = kda.chunk_fwd(*(inp[n] for n in NAMES), chunk=C)  # eager, its own outputs and workspace
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {i}: o differs from the eager call"
        assert torch.equal(S_g, S_e), f"replay {i}: S differs from the eager call"


def test_layer_call_replays_equal_eager():
    """kda_layer_fwd: its intra kernel marks the output side's exchange area
    unwritten on every call, so every replay of the graph (and the eager call
    on another workspace between replays) exchanges afresh."""
    B, T, H, D, C = 2, 300, 4, 128, 32
    sets = [to_dev(inputs.make_inputs(B, T, H, D, D, "bf16", seed=950 + i, a_std=0.5, s_std=0.1))
            for i in range(3)]
    g_gen = torch.Generator().manual_seed(951)
    gates = [torch.randn(B, T, H, D, generator=g_gen).to(torch.bfloat16).cuda() for _ in range(3)]
    gw = (torch.rand(D, generator=g_gen) + 0.5).float().cuda()
    st = {n: sets[0][n].clone() for n in NAMES}
    gate = gates[0].clone()
    y = torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda")
    S = torch.empty(B, H, D, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.layer_workspace_bytes(B, T, H, D, D, C, torch.bfloat16), dtype=torch.uint8, device="cuda")

    def call():
        kda.layer_fwd(*(st[n] for n in NAMES[:6]), gate, gw, st["S0"], chunk=C, y=y, S_out=S, workspace=ws)

    print(f"graph: layer call B{B} T{T} H{H} D{D} bf16 chunk {C}", flush=True)
    g = capture(call)
    for i, inp in enumerate(sets):
        for n in NAMES:
            st[n].copy_(inp[n])
        gate.copy_(gates[i])
        g.replay()
        torch.cuda.synchronize()
        y_g, S_g = y.clone(), S.clone()
        y_e, S_e = kda.layer_fwd(*(inp[n] for n in NAMES[:6]), gates[i], gw, inp["S0"], chunk=C)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {i}: y differs from the eager call"
        assert torch.equal(S_g, S_e), f"replay {i}: S differs from the eager call"


def test_decode_step_replays_equal_eager():
    w = inputs.WORKLOADS["decode"]
    B, H = 16, w.H
    S0, A_log = inputs.make_decode_state(w)
    S_graph = S0[:B].contiguous().cuda()
    S_eager = S_graph.clone()
    A = A_log.cuda()
    steps = [to_dev({n: t[:B] for n, t in inputs.make_decode_step(w, s).items()}) for s in range(3)]
    names = ("q", "k", "v", "z", "beta_raw")
    st = {n: steps[0][n].clone() for n in names}
    o = torch.empty(B, H, w.Dv, dtype=torch.bfloat16, device="cuda")
    S_warm = S_graph.clone()
    state = {"S": S_warm}  # the warm-up updates a throwaway copy of the state

    def call():
        kda.step(*(st[n] for n in names), A, state["S"], o=o)

    print(f"graph: decode step B{B} H{H} D{w.Dk} bf16", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    state["S"] = S_graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i, inp in enumerate(steps):
        for n in names:
            st[n].copy_(inp[n])
        g.replay()
        torch.cuda.synchronize()
        o_g = o.clone()
        o_e = kda.step(*(inp[n] for n in names), A, S_eager)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {i}: o differs from the eager step"
        assert torch.equal(S_graph, S_eager), f"replay {i}: the state differs from the eager steps"
