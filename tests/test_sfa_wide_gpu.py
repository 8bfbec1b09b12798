"""The all-heads sparse kernel: one workgroup takes every query head of a
chunk.  The planner picks it when there are more than 64 heads and the
workgroups of 64 heads would not all fit on the compute units at once.  These
cases force that with enough query rows or a forced chunk count, check through
sfa_decode_mla_plan that it was chosen, and compare with the fp64 oracle: head
counts that leave a wave or a head group of a wave empty, both dtypes, the
three cache layouts and the TND query, several causal query rows with padding
rows, block-wise selection, a value tensor that aliases the key, the one-chunk
direct output, softmax_max / softmax_sum, and scores spread far enough that
the running maximum is raised after the first tile (the accumulator
rescale)."""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_kv_06_amd import binding, harness
from decode_attention_kv_06_amd.workloads import make_sfa
from gpu_util import compare, run_gpu, say
from test_sfa_breadth_gpu import run_lse, small

pytestmark = pytest.mark.gpu


def plan_of(dev, out, split):
    return binding.sfa_decode_mla_plan(dev["q"], dev["q_rope"], dev["key"], dev["key_rope"], dev["value"],
                                       dev["sparse_indices"], dev["block_table"], dev["actual_seq_lengths_kv"], out,
                                       **harness.sfa_options(dev, split))


def run_wide(inp, split):
    """Run a case that must take the all-heads kernel."""
    dev = harness.to_device(inp)
    out = harness.alloc_out(dev)
    out.fill_(float("nan"))
    pl = plan_of(dev, out, split)
    say("GPU step: all-heads plan %s" % pl)
    assert pl["all_heads"], pl
    out, _ = run_gpu(inp, split=split, dev=dev, out=out)
    return out, pl


# 20 query rows x 7 chunks x 2 blocks of 64 heads = 288 workgroups > 256 CUs
ROWS20 = dict(B=20, lkv_range=(300, 3000), sparse_size=600, tail_range=(0, 40))


@pytest.mark.parametrize("QN,dt", [(65, "bf16"), (80, "f16"), (100, "bf16"), (128, "f16"), (128, "bf16")])
def test_head_counts(QN, dt):
    # 65: waves 0-2 active, wave 3 without heads; 80, 100: a head group of the last active wave past the count
    inp = make_sfa(small(QN=QN, dtype=dt, cfg_id=900 + QN, **ROWS20))
    out, pl = run_wide(inp, split=8)
    assert pl["chunks"] == 7
    compare(inp, out)


@pytest.mark.parametrize("layout_q,layout_kv", [("BSND", "BSND"), ("BSND", "TND"), ("TND", "PA_BSND"),
                                                ("TND", "TND")])
def test_layouts(layout_q, layout_kv):
    kw = dict(ROWS20, QN=96, layout_q=layout_q, layout_kv=layout_kv, cfg_id=910)
    if layout_q == "TND":
        kw["lq"] = [1] * 20
    if layout_kv == "BSND":
        kw["kv_seq"] = 3000
    inp = make_sfa(small(**kw))
    out, _ = run_wide(inp, split=8)
    compare(inp, out)


@pytest.mark.parametrize("sbs", [1, 4])
def test_causal_query_rows_with_padding(sbs):
    # 10 batches x 4 query rows (some padding) = 40 rows x 4 chunks x 2 blocks = 320 workgroups
    inp = make_sfa(small(B=10, QN=128, QS=4, lq=[4, 2, 0, 3, 4, 1, 4, 4, 2, 3], sparse_mode=3, past_limit=True,
                         sparse_block_size=sbs, sparse_size=600 // sbs, lkv_range=(200, 4000),
                         tail_range=(0, 10), cfg_id=920 + sbs))
    out, _ = run_wide(inp, split=4)
    compare(inp, out)


def test_value_aliases_key_and_sorted_indices():
    inp = make_sfa(small(QN=128, value_aliases_key=True, sorted_indices=True, cfg_id=930, **ROWS20))
    out, _ = run_wide(inp, split=8)
    compare(inp, out)


def test_one_chunk_writes_the_output_and_softmax_statistics_directly():
    # 3 batches x 48 query rows = 144 rows x 1 chunk x 2 blocks = 288 workgroups
    import oracle
    inp = make_sfa(small(B=3, QN=72, QS=48, sparse_size=64, tail_range=(0, 20), layout_kv="BSND",
                         lkv=[500, 64, 2000], kv_seq=2000, cfg_id=940))
    dev = harness.to_device(inp)
    out = harness.alloc_out(dev)
    pl = plan_of(dev, out, 1)
    assert pl["all_heads"] and pl["chunks"] == 1, pl
    out, mx, sm = run_lse(inp, 1)
    compare(inp, out)
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    empty = rsm == 0
    assert (mx[empty] == -np.inf).all() and (sm[empty] == 0).all()
    np.testing.assert_allclose(mx[~empty], rmx[~empty], rtol=0, atol=1e-3)
    np.testing.assert_allclose(sm[~empty], rsm[~empty], rtol=2e-3, atol=0)


@pytest.mark.parametrize("layout_kv", ["PA_BSND", "TND"])
def test_raised_maximum_rescales_the_accumulators(layout_kv):
    """Scores spread over hundreds of log2 units: the running max of a head
    group is raised on later tiles, and the group's accumulators are rescaled
    before that tile's P.V.  Checked on the output and, for the TND cache, on
    softmax_max / softmax_sum through the chunk merge."""
    import oracle
    kw = dict(ROWS20, QN=128, scale=4.0, layout_kv=layout_kv, cfg_id=950)
    inp = make_sfa(small(**kw))
    if layout_kv == "PA_BSND":
        out, _ = run_wide(inp, split=8)
        assert np.isfinite(out.float().cpu().numpy()).all()
        compare(inp, out)
        return
    dev = harness.to_device(inp)
    assert plan_of(dev, harness.alloc_out(dev), 8)["all_heads"]
    out, mx, sm = run_lse(inp, 8)
    compare(inp, out)
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    np.testing.assert_allclose(mx, rmx, rtol=0, atol=1e-3)
    np.testing.assert_allclose(sm, rsm, rtol=2e-3, atol=0)


def shape_args(**kw):
    """Arguments with placeholder pointers: enough for the planner, never launched."""
    fake = ctypes.c_void_p(0x1000)
    a = binding.SfaMlaArgs()
    a.struct_size = ctypes.sizeof(binding.SfaMlaArgs)
    a.query = a.query_rope = a.key = a.key_rope = a.value = a.sparse_indices = a.block_table = fake
    a.actual_seq_lengths_kv = a.attention_out = fake
    a.dtype = binding._DT[torch.bfloat16]
    a.batch, a.q_seq, a.q_heads, a.kv_heads, a.head_dim, a.rope_dim = 32, 1, 128, 1, 512, 64
    a.sparse_size, a.block_size, a.num_blocks, a.max_blocks = 2048, 64, 32768, 1024
    a.scale_value = 0.04
    a.sparse_block_size, a.sparse_mode, a.attention_mode = 1, 0, 2
    a.layout_query, a.layout_kv = b"BSND", b"PA_BSND"
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def plan_of_shape(**kw):
    pl = binding.SfaMlaPlan()
    assert binding.lib().sfa_decode_mla_plan(ctypes.byref(shape_args(**kw)), ctypes.byref(pl)) == 0
    return pl.chunks, pl.chunk_entries, pl.workgroups, pl.all_heads


def test_planner_choice_on_the_benchmark_shapes():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # 32 query rows: 4 chunks of 512 x 2 head blocks fill the CUs once; the 64-head kernel stays
    ch, ce, wg, allh = plan_of_shape()
    if cus == 256:
        assert (ch, ce, wg, allh) == (4, 512, 256, 0)
    # two causal query rows per batch (64 rows): 512 workgroups of 64 heads would take two rounds
    ch, ce, wg, allh = plan_of_shape(q_seq=2, sparse_mode=3)
    if cus == 256:
        assert (ch, ce, wg, allh) == (4, 512, 256, 1)
    # at most 64 heads there is one head block, so nothing to halve
    assert plan_of_shape(q_seq=2, sparse_mode=3, q_heads=64)[3] == 0


N_RANDOM = 48


def draw_all_heads(i: int):
    """A seeded configuration on which the planner must take the all-heads
    kernel: more than 64 heads, and query rows x chunks past 128 so that the
    64-head grid overflows 256 compute units."""
    from decode_attention_kv_06_amd.workloads import SfaSpec
    r = np.random.default_rng(9500 + i)
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    split = pick([8, 12, 16])
    B = int(r.integers(9, 17))
    layout_q = pick(["BSND", "BSND", "TND"])
    layout_kv = pick(["PA_BSND", "PA_BSND", "BSND", "TND"])
    kw = dict(dtype=pick(["bf16", "f16"]), B=B, QN=int(r.integers(65, 129)), layout_q=layout_q,
              layout_kv=layout_kv, sparse_mode=pick([0, 3]))
    if layout_q == "BSND":
        kw["QS"] = QS = int(r.integers(2, 4))
        if r.random() < 0.5:
            kw["lq"] = [int(r.integers(0, QS + 1)) for _ in range(B)]
    else:
        kw["lq"] = [int(r.integers(1, 4)) for _ in range(B)]
    rows = sum(kw["lq"]) if layout_q == "TND" else B * kw["QS"]
    while rows * split <= 128:
        split += 4
    lkv = [int(r.integers(64, 3000)) for _ in range(B)]
    kw["lkv"] = lkv
    sbs = pick([1, 1, 2, 4])
    if layout_kv == "PA_BSND":
        bs = pick([64, 128, 256])
        max_blocks = -(-max(lkv) // bs)
        kw.update(block_size=bs, max_blocks=max_blocks, num_blocks=B * max_blocks)
    elif layout_kv == "BSND":
        kw["kv_seq"] = max(lkv)
    kw["sparse_block_size"] = sbs
    gran = max(1, 32 // sbs)
    kw["sparse_size"] = split * gran * int(r.integers(1, 4))       # splits into exactly `split` chunks
    kw["tail_range"] = (0, min(kw["sparse_size"] - 1, 30))
    kw["past_limit"] = bool(r.random() < 0.3) and kw["sparse_mode"] == 3
    kw["value_aliases_key"] = bool(r.random() < 0.2)
    lse = layout_kv != "PA_BSND" and r.random() < 0.5
    return SfaSpec("sfa_all_heads_%d" % i, 9500 + i, **kw), split, lse


@pytest.mark.parametrize("i", range(N_RANDOM))
def test_random_all_heads_configuration(i):
    import oracle
    spec, split, lse = draw_all_heads(i)
    say("GPU step: random all-heads case %d: %s split=%d lse=%s" % (i, spec, split, lse))
    inp = make_sfa(spec)
    dev = harness.to_device(inp)
    pl = plan_of(dev, harness.alloc_out(dev), split)
    assert pl["all_heads"] and pl["chunks"] == split, pl
    if not lse:
        out, _ = run_gpu(inp, split=split, dev=dev)
        compare(inp, out)
        return
    out, mx, sm = run_lse(inp, split)
    compare(inp, out)
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    empty = rsm == 0
    assert (mx[empty] == -np.inf).all() and (sm[empty] == 0).all()
    np.testing.assert_allclose(mx[~empty], rmx[~empty], rtol=0, atol=1e-3)
    np.testing.assert_allclose(sm[~empty], rsm[~empty], rtol=2e-3, atol=0)
