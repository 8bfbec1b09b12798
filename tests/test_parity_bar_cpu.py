"""The float parity bar discriminates at full size (CPU only).

On the dense GQA workload (bf16, 64 batches, 32 query heads over 8 KV heads,
head dim 128, lengths 1024..8192) softmax rows are long and nearly uniform,
so every output element is small and a systematic error can hide under the
2e-2 max-abs bar.  Here the oracle's own output, rounded to bf16 as the
kernel's is, passes the bar, and the same output computed with the score
scale off by 3 % fails it (IncreFlashAttention README, Formula: the scores
are q.K^T times the scale)."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_06_amd.workloads import make_ifa, workloads
from gpu_util import RMS_TOL, TOL, check_close


@pytest.fixture(scope="module")
def dense_full():
    return make_ifa(workloads()["dense_gqa_bf16_bsh"])


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).double().numpy()


def test_scale_error_of_three_percent_fails_the_bar(dense_full):
    inp = dense_full
    s = inp["spec"]
    rows = np.arange(0, s.B * s.N, 7)                      # a spread sample over every batch and head
    ref = oracle.ifa(inp, rows=rows)
    check_close(_bf16(ref), ref, TOL[torch.bfloat16], RMS_TOL[torch.bfloat16])
    for factor in (0.97, 1.03):
        off = oracle.ifa(inp, rows=rows, scale=s.scale_value * factor)
        got = _bf16(off)
        # the max-abs bar alone lets it through ...
        assert np.abs(got - ref).max() <= TOL[torch.bfloat16]
        # ... the rms bar does not
        with pytest.raises(AssertionError, match="rms error"):
            check_close(got, ref, TOL[torch.bfloat16], RMS_TOL[torch.bfloat16])
