"""Row mode: small decodes run as one launch, one workgroup per (batch, KV
head, head group) row, whose four waves each take a quarter of the window and
merge their states in LDS before writing the normalised output.

The planner takes it when every window is at most four tiles long and the
rows fit in the resident waves, for 16-bit caches and outputs; the call then
needs no workspace, which is how the tests see which mode ran.  Each case is
checked against the fp64 oracle."""
from dataclasses import replace

import pytest
import torch

from decode_attention_kv_06_amd import harness
from decode_attention_kv_06_amd.workloads import IfaSpec, make_ifa, workloads
from gpu_util import compare, say

pytestmark = pytest.mark.gpu


def tile(D, G):
    return (4 if G >= 8 else 8) * 512 // D


def run_mode(inp):
    """(output, workspace bytes the call needed)."""
    say("GPU step: row-mode candidate %s B=%d N=%d Nkv=%d D=%d" % (inp["spec"].name, inp["spec"].B, inp["spec"].N,
                                                                  inp["spec"].nkv, inp["spec"].D))
    dev = harness.to_device(inp)
    out = harness.alloc_out(dev)
    out.fill_(float("nan"))
    n = harness.call(dev, out)
    torch.cuda.synchronize()
    return out, n


def test_tiny_dense_workload_is_one_launch():
    inp = make_ifa(workloads()["tiny_dense_f16"])
    out, n = run_mode(inp)
    assert n == 0
    compare(inp, out)


@pytest.mark.parametrize("layout", ["BSH", "BNSD", "BSND"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_layouts_dtypes_head_dims(layout, dt, D):
    G = 4                       # N = 6 over N_kv = 2: groups of 3 heads padded to 4
    spec = IfaSpec("rowmode", 600 + D, dt, dt, B=4, N=6, Nkv=2, D=D, layout=layout, S=4 * tile(D, G),
                   len_range=(1, 4 * tile(D, G)))
    inp = make_ifa(spec)
    out, n = run_mode(inp)
    assert n == 0
    compare(inp, out)


@pytest.mark.parametrize("extra", ["mask", "pse", "both"])
@pytest.mark.parametrize("paged", [False, True])
def test_masks_biases_and_paged_caches(extra, paged):
    D, G = 128, 4
    S = 4 * tile(D, G)
    kw = dict(mask="u8" if extra in ("mask", "both") else None, mask_p=0.3, mask_heads=8,
              pse=extra in ("pse", "both"))
    if paged:
        kw.update(paged=True, block_size=16, num_blocks=64, max_blocks=S // 16)
    spec = IfaSpec("rowmode_x", 620, "bf16", "bf16", B=3, N=8, Nkv=2, D=D, layout="BNSD", S=S,
                   lengths=[S, 0, 37], **kw)
    inp = make_ifa(spec)
    if inp["mask"] is not None:
        inp["mask"][2, 5, 0, :] = 1            # batch 2, head 5: every position masked
    out, n = run_mode(inp)
    assert n == 0
    o = out.float().cpu().reshape(3, 8, D)
    assert (o[1] == 0).all()                   # the empty window
    if inp["mask"] is not None:
        assert (o[2, 5] == 0).all()
    compare(inp, out)


def group(g):
    G = 1
    while G < g and G < 8:
        G *= 2
    return G


@pytest.mark.parametrize("N,Nkv,D", [(4, 4, 128), (8, 4, 256), (16, 2, 512), (24, 2, 64), (12, 1, 128)])
def test_head_group_sizes(N, Nkv, D):
    # groups of 1, 2, 8 (the largest LDS merge: 4 waves x 8 heads x 512 floats), and 12 or
    # 24 heads per KV head split into padded groups of 8
    G = group(N // Nkv)
    S = 4 * tile(D, G)
    spec = IfaSpec("rowmode_g", 630 + N + D, "bf16", "bf16", B=3, N=N, Nkv=Nkv, D=D, layout="BSND", S=S,
                   lengths=[S, 1, 4 * tile(D, G) // 3 + 5])
    inp = make_ifa(spec)
    out, n = run_mode(inp)
    assert n == 0
    compare(inp, out)


def test_every_batch_empty():
    spec = IfaSpec("rowmode_empty", 621, "f16", "f16", B=3, N=4, Nkv=4, D=64, layout="BNSD", S=100,
                   lengths=[0, 0, 0])
    inp = make_ifa(spec)
    out, n = run_mode(inp)
    assert n == 0
    assert (out == 0).all()


def test_longer_rows_and_int8_paths_keep_the_split():
    D, G = 128, 4
    spec = IfaSpec("rowmode_long", 622, "bf16", "bf16", B=2, N=8, Nkv=2, D=D, layout="BSH",
                   S=4 * tile(D, G) + 1, lengths=[4 * tile(D, G) + 1, 3])
    inp = make_ifa(spec)
    out, n = run_mode(inp)
    assert n > 0                               # one window past four tiles: split and combine
    compare(inp, out)
    aq = replace(spec, name="rowmode_i8", cfg_id=623, q_dtype="f16", kv_dtype="i8", antiquant="per_channel",
                 S=64, lengths=[64, 10])
    inp = make_ifa(aq)
    out, n = run_mode(inp)
    assert n > 0                               # the antiquant epilogue lives in the combine
    compare(inp, out)


@pytest.mark.parametrize("B,row_mode", [(64, True), (65, False)])
def test_row_table_limit(B, row_mode):
    # 8 KV heads x one group of 8 heads: 8 rows a batch.  64 batches fill the
    # 512-row window table of the kernel arguments exactly (one launch); 65
    # batches are past it and take the split and the combine.
    S = 4 * tile(128, 8)
    spec = IfaSpec("row_table", 830 + B, "bf16", "bf16", B=B, N=64, Nkv=8, D=128, layout="BSH", S=S,
                   len_range=(0, S))
    inp = make_ifa(spec)
    out, n = run_mode(inp)
    assert (n == 0) == row_mode
    compare(inp, out)
