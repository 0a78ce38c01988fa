"""kda_chunk_fwd_noalloc (the allocation-free entry point) against
kda_chunk_fwd on the same inputs, through the C ABI: two calls in a row on
the built-in scratch, the second smaller than the first, each equal to the
workspace call bit for bit (slicing the sequence carries the fp32 state
exactly), and a size beyond the scratch rejected before any launch."""

import pytest
import torch

from gated_delta_rule_82_amd import inputs, kda
from tests.kda_check import assert_close, oracle_forward, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load()
    yield
    torch.cuda.synchronize()


def both(inp, chunk, want):
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["z"], d["beta_raw"], d["A_log"], d["S0"])
    ref = kda.chunk_fwd(*args, chunk=chunk, want_M=want, want_P=want)
    got = kda.chunk_fwd_noalloc(*args, chunk=chunk, want_M=want, want_P=want)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_workspace_call_twice():
    # 1) the layer workload at the benchmarked chunk: 231 MB of blocks, so the
    #    64 MiB scratch cuts the sequence into slices
    w = inputs.WORKLOADS["layer"]
    print("noalloc: layer workload B4 T4096 H16 D128 bf16 chunk 32", flush=True)
    ref, got = both(inputs.make_workload(w), 32, False)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    # 2) a smaller call on the same scratch right after: fp32, incoming state,
    #    transition and correction rows (augmented state), ragged tail
    print("noalloc: B2 T333 H3 Dk64 Dv32 f32 chunk 64 with S0, M, P", flush=True)
    inp = inputs.make_inputs(2, 333, 3, 64, 32, "f32", seed=77, a_std=0.5, s_std=0.2)
    ref, got = both(inp, 64, True)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    o_ref, S_ref = oracle_forward(inp)
    assert_close(got[0], o_ref, torch.float32, "noalloc o")
    assert_close(got[1], S_ref, torch.float32, "noalloc S")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # B*H = 422 heads of Dk = Dv = 128 need more than the 64 MiB scratch:
    # refused with KDA_ERR_SCRATCH before anything is enqueued
    dev = torch.device("cuda")
    B, T, D = 1, 32, 128

    def zeros(H):
        x = torch.zeros(B, T, H, D, dtype=torch.bfloat16, device=dev)
        return x, torch.zeros(B, T, H, dtype=torch.bfloat16, device=dev), torch.zeros(H, device=dev)

    x, br, A = zeros(422)
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd_noalloc(x, x, x, x, br, A, chunk=32)
    assert e.value.status == 8
    # the largest head count that fits: accepted and computed
    x, br, A = zeros(421)
    o, S = kda.chunk_fwd_noalloc(x, x, x, x, br, A, chunk=32)
    torch.cuda.synchronize()
    assert float(o.float().abs().max()) == 0.0 and float(S.abs().max()) == 0.0
