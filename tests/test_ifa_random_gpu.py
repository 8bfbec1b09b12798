"""Seeded random IFA configurations against the fp64 oracle.

The feature tests check one thing at a time; these cases cross them: query
and cache dtypes (int8 caches with per-tensor or per-channel antiquant),
every query layout, dense, paged (both cache layouts, block sizes 16-512)
and tensor-list caches, head dims from 8 to 512, GQA groups from 1 to 16,
lengths that include empty and full windows, left padding, masks (shared,
per head, per batch or broadcast), the positional bias, int8 output, and
the planner's choices (row mode, the cost split, forced work-item sizes).
Every case is drawn from its own seed, so a failure names a reproducible
configuration."""
import numpy as np
import pytest

from decode_attention_kv_06_amd.workloads import IfaSpec, make_ifa
from gpu_util import compare, compare_int8, run_gpu, say

pytestmark = pytest.mark.gpu

N_CASES = 600


def draw(i: int):
    """(spec, forced work-item size) of case i."""
    r = np.random.default_rng(5000 + i)
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    q_dtype = pick(["f16", "bf16"])
    kv_dtype = pick([q_dtype, q_dtype, "i8"])
    Nkv = pick([1, 2, 4])
    g = pick([1, 2, 3, 4, 5, 8, 16])
    N = min(Nkv * g, 256)
    D = pick([8, 16, 24, 40, 64, 72, 96, 128, 136, 192, 256, 320, 512])
    B = int(r.integers(1, 6))
    storage = pick(["dense", "dense", "paged", "lists"])
    layout = pick(["BSH", "BNSD", "BSND"])
    S = int(r.integers(16, 600))
    kw = {}
    if storage == "paged":
        cache_layout = pick([0, 1])
        if cache_layout == 0:
            layout = "BNSD"           # the (blocknum, KV_N, bs, D) cache pairs with a BNSD query
        bs = pick([32, 64, 128, 256, 512] if kv_dtype == "i8" else [16, 48, 64, 128, 512])
        max_blocks = -(-S // bs)
        kw.update(paged=True, block_size=bs, cache_layout=cache_layout, max_blocks=max_blocks,
                  num_blocks=B * max_blocks + int(r.integers(0, 4)))
    elif storage == "lists":
        kw.update(kv_list=True, list_slack=int(r.integers(0, 20)))
    lengths = [int(r.integers(0, S + 1)) for _ in range(B)]
    if r.random() < 0.3:
        lengths[int(r.integers(B))] = S
    if r.random() < 0.2:
        lengths[int(r.integers(B))] = 0
    kw["lengths"] = lengths
    if storage == "dense" and r.random() < 0.3:
        kw["pad_off"] = (0, int(r.integers(0, 30)))
    if r.random() < 0.4:
        kw.update(mask=pick(["bool", "i8", "u8"]), mask_p=float(r.uniform(0.0, 0.5)),
                  mask_heads=pick([1, N]), mask_batch=pick([0, 1]))
    if r.random() < 0.3:
        kw.update(pse=True, pse_batch=pick([0, 1]), pse_scale=float(r.uniform(0.5, 3.0)))
    if kv_dtype == "i8":
        kw["antiquant"] = pick(["per_tensor", "per_channel"])
    if r.random() < 0.15:
        kw.update(out_int8=pick(["per_tensor", "per_channel"]),
                  qs_range=(50.0, 200.0) if q_dtype == "f16" else (5.0, 25.0))
    split = pick([0, 0, 0, 16, 48, 256])
    spec = IfaSpec("random_%d" % i, 6000 + i, q_dtype, kv_dtype, B=B, N=N, Nkv=Nkv, D=D, layout=layout, S=S, **kw)
    return spec, split


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    spec, split = draw(i)
    say("GPU step: random case %d: %s split=%d" % (i, spec, split))
    inp = make_ifa(spec)
    out, _ = run_gpu(inp, split=split)
    if spec.out_int8:
        compare_int8(inp, out, min_clear=0.0)      # a drawn call may have a constant output
    else:
        compare(inp, out)
