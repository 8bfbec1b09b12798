"""fp64 CPU oracle for decode attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it, and it shares no code with them.

``ifa(inputs)`` and ``sfa(inputs)`` take the host tensors produced by
``decode_attention_kv_06_amd.workloads`` and return the exact attention
output, unrounded, as a float64 numpy array.  The arithmetic lives in
``oracle.c``; see its header for the passages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

DT = {torch.float16: 1, torch.bfloat16: 2, torch.int8: 3, torch.float32: 6}
LAYOUT = {"BSH": 0, "BNSD": 1, "BSND": 2}


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def bind(path: str) -> ctypes.CDLL:
    """Load an oracle shared object and declare its signatures."""
    lb = ctypes.CDLL(path)
    P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lb.oracle_ifa.argtypes = [P, I, P, P, I, I, I64, I64, I64, I64, I64, D, P, P, P, I64, I64, I64,
                                    P, I64, I64, I64, I, P, P, I, P, I64, P, P, I64, I64, P, P, P]
    lb.oracle_ifa.restype = I
    lb.oracle_quant_int8.argtypes = [P, I64, I64, P, P, I, P, P]
    lb.oracle_quant_int8.restype = I
    lb.oracle_sfa.argtypes = [P, P, P, P, P, I, P, P, P, P, I, I, I64, I64, I64, I64, I64, I64, I64, I64, I64, I64,
                              I64, I, I64, D, P, I64, P, P, P]
    lb.oracle_sfa.restype = I
    lb.oracle_set_threads.argtypes = [I]
    lb.oracle_set_threads.restype = I
    lb.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lb.oracle_f16_to_f64.restype = D
    lb.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lb.oracle_bf16_to_f64.restype = D
    return lb


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = bind(build())
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        assert t.is_contiguous() and t.device.type == "cpu"
        return ctypes.c_void_p(t.data_ptr())
    assert isinstance(t, np.ndarray) and t.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(t.ctypes.data)


def ifa(inp: dict, rows=None, scale=None, use=None) -> np.ndarray:
    """Exact IFA output [B, N, D] (or [len(rows), D]) in float64."""
    s = inp["spec"]
    B, N, D = s.B, s.N, s.D
    q, k, v = inp["q"].contiguous(), inp["k"].contiguous(), inp["v"].contiguous()
    actual = inp["actual_seq_lengths"]
    actual = None if actual is None else np.ascontiguousarray(actual, dtype=np.int64)
    pad = inp["kv_padding_size"]
    if pad is not None:
        pad = np.ascontiguousarray(np.broadcast_to(np.asarray(pad, dtype=np.int64), (B,)))
    mask = inp["mask"]
    mB = mN = mS = 0
    if mask is not None:
        mB, mN, mS = mask.shape[0], mask.shape[1], mask.shape[3]
        mask = mask.contiguous().view(torch.uint8) if mask.dtype == torch.bool else mask.contiguous().view(torch.uint8)
    bt = inp.get("block_table")
    bt = None if bt is None or not s.paged else bt.contiguous()
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = B * N if rows is None else len(rows_a)
    out = np.empty((n, D), dtype=np.float64)
    aqs = inp["aq_scale"].contiguous() if inp["aq_scale"] is not None else None
    aqo = inp["aq_offset"].contiguous() if inp["aq_offset"] is not None else None
    k_list = inp.get("k_list")
    kl = vl = seq = None
    if k_list is not None:
        keep = [t.contiguous() for t in k_list] + [t.contiguous() for t in inp["v_list"]]
        kl = (ctypes.c_void_p * B)(*[t.data_ptr() for t in keep[:B]])
        vl = (ctypes.c_void_p * B)(*[t.data_ptr() for t in keep[B:]])
        seq = np.ascontiguousarray(inp["list_seq"], dtype=np.int64)
    pse = inp.get("pse")
    pB = pS = 0
    if pse is not None:
        pB, pS = pse.shape[0], pse.shape[3]
        pse = pse.contiguous()
    rc = (use or lib()).oracle_ifa(
        _ptr(q), DT[q.dtype], _ptr(k), _ptr(v), DT[k.dtype], LAYOUT[s.layout], B, N, s.nkv, D, inp["S"],
        float(s.scale_value if scale is None else scale), _ptr(actual), _ptr(pad), _ptr(mask), mB, mN, mS,
        _ptr(bt), inp.get("max_blocks", 0) if bt is not None else 0, s.block_size if bt is not None else 0,
        inp.get("num_blocks", 0) if bt is not None else 0, s.cache_layout,
        _ptr(aqs), _ptr(aqo), int(inp["aq_mode"]), _ptr(rows_a), n, _ptr(out), _ptr(pse), pB, pS,
        None if kl is None else ctypes.cast(kl, ctypes.c_void_p), None if vl is None else ctypes.cast(vl, ctypes.c_void_p),
        _ptr(seq))
    if rc != 0:
        raise ValueError("oracle_ifa rejected its input (code %d)" % rc)
    return out.reshape(B, N, D) if rows is None else out


def sfa(inp: dict, rows=None, use=None, lse: bool = False):
    """Exact SFA output [query rows, QN, D] (or [len(rows), D]) in float64;
    rows are (query row) * QN + head.  With lse=True also the softmax_max and
    softmax_sum outputs ([query rows, QN], or [len(rows)]): returns
    (out, softmax_max, softmax_sum)."""
    s = inp["spec"]
    key = inp["key"].contiguous()
    value = inp["value"].contiguous()
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = inp["q_rows"]
    n = R * s.QN if rows is None else len(rows_a)
    out = np.empty((n, s.D), dtype=np.float64)
    lmax = np.empty(n, dtype=np.float64) if lse else None
    lsum = np.empty(n, dtype=np.float64) if lse else None
    bt = inp["block_table"]
    lq = inp["actual_seq_lengths_query"]
    lkv = inp["actual_seq_lengths_kv"]
    lay_q = {"BSND": 0, "TND": 1}[s.layout_q]
    lay_kv = {"PA_BSND": 0, "BSND": 1, "TND": 2}[s.layout_kv]
    rc = (use or lib()).oracle_sfa(
        _ptr(inp["q"].contiguous()), _ptr(inp["q_rope"].contiguous()), _ptr(key),
        _ptr(inp["key_rope"].contiguous()), _ptr(value), DT[key.dtype],
        _ptr(inp["sparse_indices"].contiguous()), _ptr(None if bt is None else bt.contiguous()),
        _ptr(None if lkv is None else lkv.contiguous()), _ptr(None if lq is None else lq.contiguous()),
        lay_q, lay_kv, s.B, s.QS, R, s.QN, s.D, s.DR, inp["sparse_indices"].shape[-1], s.block_size,
        key.shape[0] if lay_kv == 0 else 0, bt.shape[1] if bt is not None else 0, inp.get("kv_seq", 0),
        int(s.sparse_mode), int(s.sparse_block_size), float(s.scale_value), _ptr(rows_a), n, _ptr(out),
        _ptr(lmax), _ptr(lsum))
    if rc != 0:
        raise ValueError("oracle_sfa rejected its input (code %d)" % rc)
    if rows is None:
        out = out.reshape(R, s.QN, s.D)
        if lse:
            lmax, lsum = lmax.reshape(R, s.QN), lsum.reshape(R, s.QN)
    return (out, lmax, lsum) if lse else out


def quant_int8(o: np.ndarray, scale: torch.Tensor, offset=None, use=None):
    """int8 codes of the exact output `o` ([..., N*D] order) under quantScale2 /
    quantOffset2 (1 or N*D values, fp32 or bf16); returns (codes, value before rounding)."""
    o = np.ascontiguousarray(o, dtype=np.float64)
    sc = scale.contiguous().reshape(-1)
    off = None if offset is None else offset.contiguous().reshape(-1)
    codes = np.empty(o.shape, dtype=np.int8)
    pre = np.empty(o.shape, dtype=np.float64)
    rc = (use or lib()).oracle_quant_int8(_ptr(o), o.size, sc.numel(), _ptr(sc), _ptr(off), DT[sc.dtype],
                                          _ptr(codes), _ptr(pre))
    if rc != 0:
        raise ValueError("oracle_quant_int8 rejected its input (code %d)" % rc)
    return codes, pre


def set_threads(n: int) -> int:
    """Threads the oracle's row loops use from now on; returns the count in effect."""
    return lib().oracle_set_threads(int(n))


def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(bits)
