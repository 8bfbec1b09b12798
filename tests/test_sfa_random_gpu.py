"""Seeded random SparseFlashAttention configurations against the fp64 oracle.

Crosses the sparse path's options in one parametrised test: fp16 and bf16,
query head counts from 1 to 128, BSND queries with several rows per batch
(some of them padding) and TND queries, paged (block sizes 16-1024), BSND
and TND caches, index lists of 1-900 entries with invalid tails, entries
past the causal limit, block-wise selection, sparse_mode 0 and 3, sorted
indices and a value tensor that aliases the key, forced chunk counts, and
the softmax_max / softmax_sum outputs on the caches that have them.  Every
case is drawn from its own seed."""
import numpy as np
import pytest

from decode_attention_kv_06_amd.workloads import SfaSpec, make_sfa
from gpu_util import compare, run_gpu, say
from test_sfa_breadth_gpu import run_lse

pytestmark = pytest.mark.gpu

N_CASES = 200


def draw(i: int):
    """(spec, forced chunk count, with softmax statistics) of case i."""
    r = np.random.default_rng(9000 + i)
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    B = int(r.integers(1, 5))
    layout_q = pick(["BSND", "BSND", "TND"])
    layout_kv = pick(["PA_BSND", "PA_BSND", "BSND", "TND"])
    kw = dict(dtype=pick(["bf16", "f16"]), B=B, QN=pick([1, 5, 16, 48, 64, 100, 128]),
              layout_q=layout_q, layout_kv=layout_kv, sparse_mode=pick([0, 3]))
    if layout_q == "BSND":
        QS = int(r.integers(1, 4))
        kw["QS"] = QS
        if r.random() < 0.5:
            kw["lq"] = [int(r.integers(0, QS + 1)) for _ in range(B)]
    else:
        kw["lq"] = [int(r.integers(0, 4)) for _ in range(B)]
        if sum(kw["lq"]) == 0:
            kw["lq"][0] = 1
    lkv = [int(r.integers(1, 4000)) for _ in range(B)]
    kw["lkv"] = lkv
    bs = pick([16, 64, 128, 256, 1024])
    sbs = pick([1, 1, 1, 2, 4, 16, 64])
    if layout_kv == "PA_BSND":
        while bs % sbs:
            sbs //= 2
        max_blocks = -(-max(lkv) // bs)
        kw.update(block_size=bs, max_blocks=max_blocks, num_blocks=B * max_blocks + int(r.integers(0, 3)))
    elif layout_kv == "BSND":
        kw["kv_seq"] = max(lkv) + int(r.integers(0, 50))
    kw["sparse_block_size"] = sbs
    kw["sparse_size"] = int(r.integers(1, 900 // sbs + 2))
    kw["tail_range"] = (0, max(0, min(kw["sparse_size"] - 1, int(r.integers(0, 60)))))
    kw["past_limit"] = bool(r.random() < 0.3) and kw["sparse_mode"] == 3
    kw["sorted_indices"] = bool(r.random() < 0.2)
    kw["value_aliases_key"] = bool(r.random() < 0.2)
    split = pick([0, 0, 1, 2, 3, 8])
    lse = layout_kv != "PA_BSND" and r.random() < 0.5
    return SfaSpec("sfa_random_%d" % i, 9000 + i, **kw), split, lse


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_sparse_configuration(i):
    spec, split, lse = draw(i)
    say("GPU step: random sparse case %d: %s split=%d lse=%s" % (i, spec, split, lse))
    inp = make_sfa(spec)
    if not lse:
        out, _ = run_gpu(inp, split=split)
        compare(inp, out)
        return
    import oracle
    out, mx, sm = run_lse(inp, split)
    compare(inp, out)
    _, rmx, rsm = oracle.sfa(inp, lse=True)
    rmx, rsm = rmx.reshape(-1), rsm.reshape(-1)
    empty = rsm == 0
    assert (mx[empty] == -np.inf).all() and (sm[empty] == 0).all()
    np.testing.assert_allclose(mx[~empty], rmx[~empty], rtol=1e-5, atol=1e-3)
    np.testing.assert_allclose(sm[~empty], rsm[~empty], rtol=2e-3, atol=0)
