"""The entry points enqueue only kernels on the caller's stream, so a call can
be captured into a HIP graph: every replay must give the eager call's bytes
(replays interleaved with unrelated eager work and synchronisations)."""
import pytest
import torch

from decode_attention_kv_06_amd import harness
from decode_attention_kv_06_amd.workloads import IfaSpec, make_ifa, make_sfa, small_variant, workloads
from gpu_util import say

pytestmark = pytest.mark.gpu

CASES = {
    "dense_gqa": lambda: make_ifa(small_variant("dense_gqa_bf16_bsh")),
    "paged_masked": lambda: make_ifa(small_variant("paged_bf16_bs128")),
    "int8_leftpad": lambda: make_ifa(small_variant("int8_leftpad_f16")),
    "bias_int8_out": lambda: make_ifa(IfaSpec("graph_q", 710, "bf16", "bf16", B=3, N=16, Nkv=4, D=128, layout="BSH",
                                              S=700, len_range=(1, 700), pse=True, out_int8="per_channel",
                                              qs_range=(5.0, 25.0))),
    "sparse": lambda: make_sfa(small_variant("sfa_mla_bf16")),
    "tiny_row_mode": lambda: make_ifa(workloads()["tiny_dense_f16"]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_captured_call_replays_give_the_eager_bytes(name):
    inp = CASES[name]()
    say("GPU step: graph capture of %s" % name)
    dev = harness.to_device(inp)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    eager = harness.alloc_out(dev)
    harness.call(dev, eager, workspace=ws)
    torch.cuda.synchronize()
    out = harness.alloc_out(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        harness.call(dev, out, workspace=ws)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        out.zero_()
        junk.mul_(1.5)                       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.uint8), eager.view(torch.uint8))
        say("  replay %d identical: %s" % (rep, same))
        assert same
