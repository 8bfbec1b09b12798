"""ifa_decode_noalloc: the dense decode on the library's built-in scratch.

Through the C ABI, against ifa_decode with a caller workspace (same kernels
and plan, so the bytes must agree exactly) and against the fp64 oracle, on two
calls in a row, the second on a smaller input; then a call too large for the
scratch is refused and leaves the output untouched."""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_kv_06_amd import binding, harness
from decode_attention_kv_06_amd.workloads import IfaSpec, make_ifa, small_variant, workloads
from gpu_util import compare, say


def _noalloc(dev, out):
    s = dev["spec"]
    binding.ifa_decode_noalloc(dev["q"], dev["k"], dev["v"], out, num_heads=s.N, num_key_value_heads=s.Nkv,
                               input_layout=s.layout, scale_value=s.scale_value,
                               actual_seq_lengths=dev["actual_seq_lengths"], kv_padding_size=dev["kv_padding_size"],
                               atten_mask=dev["mask"], pse_shift=dev.get("pse"), antiquant_scale=dev["aq_scale"],
                               antiquant_offset=dev["aq_offset"], antiquant_mode=dev["aq_mode"])


def _case(inp):
    dev = harness.to_device(inp)
    ref_out = harness.alloc_out(dev)
    harness.call(dev, ref_out)                       # ifa_decode, binding-allocated workspace
    out = harness.alloc_out(dev)
    out.fill_(float("nan"))
    _noalloc(dev, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "ifa_decode_noalloc differs from ifa_decode"
    compare(inp, out)


@pytest.mark.gpu
def test_noalloc_matches_ifa_decode_on_two_calls_second_smaller():
    first = make_ifa(small_variant("int8_leftpad_f16"))          # int8 cache, left padding, head groups of 8
    say("GPU step: ifa_decode_noalloc, " + first["spec"].name)
    _case(first)
    second = make_ifa(workloads()["tiny_dense_f16"])
    say("GPU step: ifa_decode_noalloc, " + second["spec"].name + " (smaller)")
    _case(second)


@pytest.mark.gpu
def test_noalloc_full_size_dense_and_masked():
    inp = make_ifa(workloads()["dense_gqa_bf16_bsh"])
    say("GPU step: ifa_decode_noalloc, full-size " + inp["spec"].name)
    dev = harness.to_device(inp)
    ref_out = harness.alloc_out(dev)
    harness.call(dev, ref_out)
    out = torch.full_like(ref_out, float("nan"))
    _noalloc(dev, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    rows = np.random.default_rng(5).choice(inp["spec"].B * inp["spec"].N, 96, replace=False)
    compare(inp, out, rows=rows)
    del dev
    spec = IfaSpec("noalloc_mask", 990, "bf16", "bf16", B=5, N=16, Nkv=4, D=256, layout="BNSD", S=900,
                   len_range=(1, 900), mask="u8", mask_p=0.2, pse=True)
    inp = make_ifa(spec)
    say("GPU step: ifa_decode_noalloc, masked + bias " + spec.name)
    _case(inp)


@pytest.mark.gpu
def test_noalloc_refuses_a_call_larger_than_its_scratch():
    # a forced split of 16 positions on 2 x 65536 positions needs about 34 MB of partial states
    spec = IfaSpec("noalloc_big", 991, "bf16", "bf16", B=2, N=8, Nkv=2, D=128, layout="BSH", S=1 << 16,
                   len_range=(1 << 16, 1 << 16))
    inp = make_ifa(spec)
    dev = harness.to_device(inp)
    out = harness.alloc_out(dev)
    out.fill_(3.0)
    a = binding.ifa_decode_args(dev["q"], dev["k"], dev["v"], out, num_heads=8, num_key_value_heads=2,
                                input_layout="BSH", scale_value=spec.scale_value, split_tokens=16)
    n = ctypes.c_size_t(0)
    assert binding.lib().ifa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > binding.NOALLOC_SCRATCH_BYTES
    say("GPU step: ifa_decode_noalloc refusing a %d-byte call" % n.value)
    rc = binding.lib().ifa_decode_noalloc(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == binding.IFA_ERR_PARAM_INVALID
    assert (out == 3.0).all()


def test_noalloc_size_limit_is_checked_before_any_device_work():
    # the same oversize call with dummy pointers: refused by validation alone,
    # so this runs on a machine without a GPU as well
    a = binding.IfaDecodeArgs()
    a.struct_size = ctypes.sizeof(binding.IfaDecodeArgs)
    a.query = a.key = a.value = a.attention_out = ctypes.c_void_p(0x1000)
    a.dtype_q = a.dtype_kv = a.dtype_out = binding.DT_BF16
    a.input_layout = b"BSH"
    a.batch, a.num_heads, a.num_key_value_heads, a.head_dim, a.kv_seq_len = 2, 8, 2, 128, 1 << 16
    a.scale_value = 0.1
    a.split_tokens = 16
    n = ctypes.c_size_t(0)
    assert binding.lib().ifa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > binding.NOALLOC_SCRATCH_BYTES
    assert binding.lib().ifa_decode_noalloc(ctypes.byref(a), None) == binding.IFA_ERR_PARAM_INVALID
    a.kv_seq_len = 64                         # small enough: the call goes on to the device
    assert binding.lib().ifa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value <= binding.NOALLOC_SCRATCH_BYTES


def test_scratch_size_in_header_matches_binding():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                            "ifa_decode.h")).read()
    m = re.search(r"#define IFA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES
