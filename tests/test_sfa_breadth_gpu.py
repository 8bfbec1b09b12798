"""SparseFlashAttention breadth on the GPU against the fp64 oracle: several
query rows per batch (rightDownCausal), block-wise selection, BSND and TND
query and cache layouts (SparseFlashAttention README, parameter table)."""
import pytest

from decode_attention_kv_06_amd.workloads import SfaSpec, make_sfa, workloads
from gpu_util import compare, run_gpu

pytestmark = pytest.mark.gpu


def small(cfg_id=500, **kw):
    d = dict(B=3, QN=16, num_blocks=128, max_blocks=64, block_size=64, lkv_range=(300, 4096), sparse_size=300,
             tail_range=(1, 40))
    d.update(kw)
    return SfaSpec("sfa_breadth", cfg_id, **d)


@pytest.mark.parametrize("mode", [0, 3])
@pytest.mark.parametrize("QN", [16, 128])
def test_query_rows_per_batch(mode, QN):
    inp = make_sfa(small(QS=4, lq=[4, 2, 0], sparse_mode=mode, QN=QN, cfg_id=501 + QN))
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_causal_limit_filters_indices_past_it():
    # every row also selects positions past its causal limit: the kernel must leave them out
    inp = make_sfa(small(QS=3, sparse_mode=3, past_limit=True, lkv=[40, 300, 2000], sparse_size=256,
                         tail_range=(0, 8), cfg_id=510))
    out, _ = run_gpu(inp)
    compare(inp, out)


@pytest.mark.parametrize("sbs", [2, 16, 64])
@pytest.mark.parametrize("split", [0, 3])
def test_block_wise_selection(sbs, split):
    inp = make_sfa(small(QS=2, sparse_mode=3, sparse_block_size=sbs, sparse_size=max(8, 600 // sbs),
                         tail_range=(0, 4), past_limit=True, cfg_id=520 + sbs))
    out, _ = run_gpu(inp, split=split)
    compare(inp, out)


def test_block_wise_128_on_1024_blocks():
    inp = make_sfa(small(sparse_block_size=128, block_size=1024, num_blocks=16, max_blocks=4,
                         lkv_range=(1000, 4096), sparse_size=12, tail_range=(0, 3), cfg_id=530))
    out, _ = run_gpu(inp)
    compare(inp, out)


@pytest.mark.parametrize("given", [True, False])
def test_bsnd_cache(given):
    lkv = [700, 1200, 64] if given else [1200, 1200, 1200]
    spec = small(layout_kv="BSND", lkv=lkv, kv_seq=1200, QS=2, sparse_mode=3, cfg_id=540)
    inp = make_sfa(spec)
    if not given:
        inp["actual_seq_lengths_kv"] = None          # KV_S for every batch
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_tnd_cache():
    inp = make_sfa(small(layout_kv="TND", lkv=[700, 33, 1500], QS=2, sparse_mode=0, cfg_id=541))
    out, _ = run_gpu(inp)
    compare(inp, out)


@pytest.mark.parametrize("layout_kv", ["PA_BSND", "TND"])
def test_tnd_query(layout_kv):
    inp = make_sfa(small(B=4, layout_q="TND", lq=[3, 0, 1, 4], layout_kv=layout_kv, lkv=[500, 900, 40, 3000],
                         sparse_mode=3, cfg_id=542))
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_tnd_query_split_chunks():
    inp = make_sfa(small(B=2, layout_q="TND", lq=[2, 3], sparse_mode=3, sparse_size=900, lkv=[1000, 4000],
                         cfg_id=543))
    out, _ = run_gpu(inp, split=4)
    compare(inp, out)


def test_multi_token_full_size_sampled_rows():
    inp = make_sfa(workloads()["sfa_mtp_bf16"])
    out, _ = run_gpu(inp)
    n = inp["q_rows"] * inp["spec"].QN
    rows = sorted(set([0, 1, n // 2, n - 1] + list(range(5, n, max(1, n // 97)))))
    compare(inp, out, rows=rows)


# ------------------------------------------------------- softmax_max / softmax_sum
def run_lse(inp, split):
    """Output plus softmax_max / softmax_sum from one call (return_softmax_lse)."""
    import torch
    from decode_attention_kv_06_amd import binding, harness
    from gpu_util import say
    dev = harness.to_device(inp)
    out = harness.alloc_out(dev)
    n = inp["q_rows"] * inp["spec"].QN
    mx = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    sm = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    say("GPU step: sfa_decode_mla with return_softmax_lse, %s/%s split=%d" % (
        inp["spec"].layout_q, inp["spec"].layout_kv, split))
    binding.sfa_decode_mla(dev["q"], dev["q_rope"], dev["key"], dev["key_rope"], dev["value"],
                           dev["sparse_indices"], dev["block_table"], dev["actual_seq_lengths_kv"], out,
                           softmax_max_out=mx, softmax_sum_out=sm, **harness.sfa_options(dev, split))
    torch.cuda.synchronize()
    return out, mx.cpu().double().numpy(), sm.cpu().double().numpy()


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("layout_kv", ["BSND", "TND"])
def test_softmax_max_and_sum(layout_kv, split):
    import numpy as np
    import oracle
    kw = dict(layout_kv=layout_kv, lkv=[700, 1200, 64], QS=2, lq=[2, 1, 2], sparse_mode=3, QN=32,
              sparse_size=600, cfg_id=550)
    if layout_kv == "BSND":
        kw["kv_seq"] = 1200
    inp = make_sfa(small(**kw))
    out, mx, sm = run_lse(inp, split)
    compare(inp, out)                                     # the output is the same call's
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    empty = rsm == 0
    assert empty.any() and (~empty).any()                 # batch 1's second query row attends nothing
    assert (mx[empty] == -np.inf).all() and (sm[empty] == 0).all()
    np.testing.assert_allclose(mx[~empty], rmx[~empty], rtol=0, atol=1e-3)
    np.testing.assert_allclose(sm[~empty], rsm[~empty], rtol=2e-3, atol=0)


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("layout_kv", ["PA_BSND", "BSND"])
def test_peaked_scores(layout_kv, split):
    """Scores spread over hundreds of log2 units, so that a running max taken
    from part of a tile (or raised late) overflows exp2 and poisons the row.
    The softmax is then nearly one-hot, and a row's largest score sits in any
    of the four lane groups of its head."""
    import numpy as np
    import oracle
    kw = dict(layout_kv=layout_kv, QS=2, lq=[2, 2, 1], sparse_mode=3, sparse_size=500, scale=4.0, cfg_id=560)
    if layout_kv == "BSND":
        kw.update(lkv=[900, 1500, 300], kv_seq=1500)
    inp = make_sfa(small(**kw))
    if layout_kv == "PA_BSND":
        out, _ = run_gpu(inp, split=split)
        assert torch_isfinite(out)
        compare(inp, out)
        return
    out, mx, sm = run_lse(inp, split)
    assert torch_isfinite(out)
    compare(inp, out)
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    live = rsm > 0
    assert np.abs(rmx[live]).max() > 100                  # the scores really are that spread
    np.testing.assert_allclose(mx[live], rmx[live], rtol=1e-5, atol=1e-3)
    np.testing.assert_allclose(sm[live], rsm[live], rtol=2e-3, atol=0)


def torch_isfinite(t):
    import torch
    return bool(torch.isfinite(t.float()).all())



@pytest.mark.parametrize("layout_kv,sparse_size", [("TND", 3000), ("PA_BSND", 4096)])
def test_more_than_64_chunks(layout_kv, sparse_size):
    """One query row with a long index list: the planner cuts it into about
    one chunk per compute unit (well past 64), where the merge reads the
    chunks' (max, sum) pairs 64 at a time and requests the outputs of only
    the first 8 up front; the trailing -1 entries leave the last chunks
    empty (sum 0, weight 0).  The TND case checks softmax_max / softmax_sum
    too."""
    import numpy as np
    import oracle
    from decode_attention_kv_06_amd import binding, harness
    inp = make_sfa(small(B=1, QN=16, lkv=[sparse_size + 500], sparse_size=sparse_size, tail_range=(0, 90),
                         layout_kv=layout_kv, max_blocks=80, cfg_id=560 + sparse_size % 97))
    dev = harness.to_device(inp)
    pl = binding.sfa_decode_mla_plan(dev["q"], dev["q_rope"], dev["key"], dev["key_rope"], dev["value"],
                                     dev["sparse_indices"], dev["block_table"], dev["actual_seq_lengths_kv"],
                                     harness.alloc_out(dev), **harness.sfa_options(dev, 0))
    assert pl["chunks"] > 64 and not pl["all_heads"], pl
    if layout_kv == "PA_BSND":
        out, _ = run_gpu(inp, split=0, dev=dev)
        compare(inp, out)
        return
    out, mx, sm = run_lse(inp, 0)
    compare(inp, out)
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    np.testing.assert_allclose(mx, rmx, rtol=0, atol=1e-3)
    np.testing.assert_allclose(sm, rsm, rtol=2e-3, atol=0)
