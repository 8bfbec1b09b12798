"""Moves a generated workload to the GPU and calls the matching entry point.

Marshalling only (device copies, output allocation, argument selection); the
attention itself runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import binding
from .workloads import IfaSpec, SfaSpec


def to_device(inp: dict, device: str = "cuda") -> dict:
    """Device copies of the host inputs.  A host tensor that appears under
    several names (a value tensor that is the key tensor) gets one device copy,
    so the call sees the same pointer for both."""
    out = {}
    copies: dict = {}
    for key, val in inp.items():
        if isinstance(val, torch.Tensor):
            if id(val) not in copies:
                copies[id(val)] = val.to(device)
            out[key] = copies[id(val)]
        elif isinstance(val, list) and val and isinstance(val[0], torch.Tensor):
            out[key] = [t.to(device) for t in val]
        else:
            out[key] = val
    return out


def alloc_out(inp: dict) -> torch.Tensor:
    if inp.get("quant_scale2") is not None:
        return torch.empty(inp["q"].shape, dtype=torch.int8, device=inp["q"].device)
    return torch.empty_like(inp["q"])


def sfa_options(dev: dict, split: int = 0) -> dict:
    """Keyword arguments of an SFA call beyond its tensors."""
    s = dev["spec"]
    return dict(scale_value=s.scale_value, sparse_mode=s.sparse_mode, sparse_block_size=s.sparse_block_size,
                actual_seq_lengths_query=dev.get("actual_seq_lengths_query"), layout_query=s.layout_q,
                layout_kv=s.layout_kv, split_hint=split)


def call(dev: dict, out: torch.Tensor, split: int = 0, workspace=None, stream=None) -> int:
    """Run the entry point that `dev["spec"]` describes; returns workspace bytes."""
    s = dev["spec"]
    if isinstance(s, SfaSpec):
        return binding.sfa_decode_mla(dev["q"], dev["q_rope"], dev["key"], dev["key_rope"], dev["value"],
                                      dev["sparse_indices"], dev["block_table"], dev["actual_seq_lengths_kv"], out,
                                      workspace=workspace, stream=stream, **sfa_options(dev, split))
    assert isinstance(s, IfaSpec)
    common = dict(num_heads=s.N, num_key_value_heads=s.Nkv, input_layout=s.layout, scale_value=s.scale_value,
                  actual_seq_lengths=dev["actual_seq_lengths"], atten_mask=dev["mask"], pse_shift=dev.get("pse"),
                  antiquant_scale=dev["aq_scale"], antiquant_offset=dev["aq_offset"], antiquant_mode=dev["aq_mode"],
                  quant_scale2=dev.get("quant_scale2"), quant_offset2=dev.get("quant_offset2"),
                  split_tokens=split, workspace=workspace, stream=stream)
    if s.paged:
        return binding.ifa_decode_paged(dev["q"], dev["k"], dev["v"], out, dev["block_table"],
                                        kv_cache_layout=s.cache_layout, **common)
    if dev.get("k_list") is not None:
        return binding.ifa_decode(dev["q"], None, None, out, kv_padding_size=dev["kv_padding_size"],
                                  key_list=dev["k_list"], value_list=dev["v_list"], **common)
    return binding.ifa_decode(dev["q"], dev["k"], dev["v"], out, kv_padding_size=dev["kv_padding_size"], **common)
