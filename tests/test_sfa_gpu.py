"""SparseFlashAttention (MLA-absorb) on the GPU against the fp64 oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from decode_attention_kv_06_amd import binding, harness
from decode_attention_kv_06_amd.workloads import SfaSpec, make_sfa, small_variant, workloads
from gpu_util import compare, run_gpu, say

pytestmark = pytest.mark.gpu


def small(cfg_id=400, **kw):
    d = dict(B=3, QN=16, num_blocks=128, max_blocks=64, block_size=64, lkv_range=(300, 4096), sparse_size=300,
             tail_range=(1, 40))
    d.update(kw)
    return SfaSpec("sfa_small", cfg_id, **d)


def test_small_variant_matches_oracle():
    inp = make_sfa(small_variant("sfa_mla_bf16"))
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_full_size_workload_matches_oracle():
    inp = make_sfa(workloads()["sfa_mla_bf16"])
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_full_size_value_is_key_sampled_rows():
    # the value tensor is the key tensor (one device buffer): the pipeline that
    # copies each gathered row once
    inp = make_sfa(workloads()["sfa_mla_alias_bf16"])
    out, dev = run_gpu(inp)
    assert dev["value"].data_ptr() == dev["key"].data_ptr()
    n = inp["q_rows"] * inp["spec"].QN
    rows = sorted(set([0, 1, n // 2, n - 1] + list(range(3, n, max(1, n // 131)))))
    compare(inp, out, rows=rows)


@pytest.mark.parametrize("QN", [1, 16, 20, 64, 100, 128])
def test_head_counts(QN):
    inp = make_sfa(small(QN=QN, cfg_id=401))
    out, _ = run_gpu(inp)
    compare(inp, out)


@pytest.mark.parametrize("split", [1, 2, 3, 8])
def test_forced_chunk_counts_agree(split):
    inp = make_sfa(small(QN=32, sparse_size=700, cfg_id=402))
    out, _ = run_gpu(inp, split=split)
    compare(inp, out)


@pytest.mark.parametrize("bs", [16, 48, 64, 80, 1024])
def test_block_sizes(bs):
    nb = max(8, (4096 + bs - 1) // bs * 3)
    inp = make_sfa(small(block_size=bs, num_blocks=nb, max_blocks=(4096 + bs - 1) // bs, cfg_id=403))
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_fp16():
    inp = make_sfa(small(dtype="f16", QN=24, cfg_id=404))
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_value_aliasing_key_and_sorted_indices():
    inp = make_sfa(small(value_aliases_key=True, sorted_indices=True, cfg_id=405))
    out, _ = run_gpu(inp)
    compare(inp, out)


def test_one_valid_index_returns_value_row_bit_exact():
    inp = make_sfa(small(QN=20, cfg_id=406))
    idx = torch.full_like(inp["sparse_indices"], -1)
    picks = [0, 117, 299]
    for b, t in enumerate(picks):
        idx[b, 0, 0, 5 + b] = t                 # not at the front: every valid entry counts
    inp["sparse_indices"] = idx
    out, _ = run_gpu(inp, split=2)
    bt = inp["block_table"]
    for b, t in enumerate(picks):
        row = int(bt[b, t // 64]) * 64 + t % 64
        ref = inp["value"].view(-1, 512)[row]
        for h in range(20):
            assert torch.equal(out[b, 0, h].cpu(), ref)


def test_no_valid_index_gives_zero_rows():
    inp = make_sfa(small(cfg_id=407))
    idx = inp["sparse_indices"].clone()
    idx[1] = -1
    idx[2, 0, 0, :] = 10 ** 7                  # out of range: invalid
    inp["sparse_indices"] = idx
    out, _ = run_gpu(inp)
    o = out.float().cpu()
    assert (o[1] == 0).all() and (o[2] == 0).all()
    compare(inp, out)


def test_invalid_entries_in_the_middle_and_duplicates():
    inp = make_sfa(small(QN=16, cfg_id=408))
    idx = inp["sparse_indices"].clone()
    idx[0, 0, 0, 10:20] = -1
    idx[0, 0, 0, 30:40] = idx[0, 0, 0, 50:60]   # duplicates count once per occurrence
    inp["sparse_indices"] = idx
    out, _ = run_gpu(inp, split=2)
    compare(inp, out)


def test_sparse_mode_three_equals_mode_zero():
    inp = make_sfa(small(cfg_id=409))
    out0, dev = run_gpu(inp)
    inp3 = dict(inp)
    inp3["spec"] = replace(inp["spec"], sparse_mode=3)
    dev3 = dict(dev)
    dev3["spec"] = inp3["spec"]
    out3, _ = run_gpu(inp3, dev=dev3)
    assert torch.equal(out0, out3)


def test_query_length_zero_gives_zero_row():
    inp = make_sfa(small(cfg_id=410))
    dev = harness.to_device(inp)
    out = harness.alloc_out(dev)
    lq = torch.tensor([1, 0, 1], dtype=torch.int32, device="cuda")
    s = inp["spec"]
    say("GPU step: sfa_decode_mla with actual_seq_lengths_query=[1,0,1]")
    binding.sfa_decode_mla(dev["q"], dev["q_rope"], dev["key"], dev["key_rope"], dev["value"],
                           dev["sparse_indices"], dev["block_table"], dev["actual_seq_lengths_kv"], out,
                           scale_value=s.scale_value, actual_seq_lengths_query=lq)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert (o[1] == 0).all()
    ref = __import__("oracle").sfa(inp)
    err = np.abs(o.double().numpy().reshape(3, 16, 512)[[0, 2]] - ref[[0, 2]]).max()
    assert err <= 2e-2


def test_repeated_calls_are_bitwise_identical():
    inp = make_sfa(small(QN=64, cfg_id=411))
    out1, dev = run_gpu(inp)
    out2, _ = run_gpu(inp, dev=dev)
    assert torch.equal(out1, out2)


def test_index_past_block_table_reach_is_left_out():
    # actual_seq_lengths_kv larger than the table's reach: indices beyond it are
    # never looked up and count as invalid
    inp = make_sfa(small(QN=16, cfg_id=412, lkv=[4000, 4000, 4000]))
    reach = 64 * 64
    idx = inp["sparse_indices"].clone()
    idx[0, 0, 0, :5] = reach + 7
    inp["sparse_indices"] = idx
    lkv_big = torch.tensor([reach + 100, 4000, 4000], dtype=torch.int32)
    inp_gpu = dict(inp)
    inp_gpu["actual_seq_lengths_kv"] = lkv_big
    out, _ = run_gpu(inp_gpu)
    compare(inp, out)           # the oracle sees the in-range length, so those entries are invalid there too
