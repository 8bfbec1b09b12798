"""ctypes binding of libifadecode (include/ifa_decode.h).

Argument marshalling only: shapes and dtypes are read off torch tensors, the
argument structs are filled, and the C entry points are called on the current
HIP stream.  Every computation happens in the library's HIP kernels; there is
no fallback path, and a missing library is an error.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libifadecode.so")

IFA_OK = 0
IFA_ERR_PARAM_NULLPTR = 161001
IFA_ERR_PARAM_INVALID = 161002
IFA_ERR_RUNTIME = 361001
NOALLOC_SCRATCH_BYTES = 32 << 20      # IFA_NOALLOC_SCRATCH_BYTES of ifa_decode.h

DT_F16, DT_BF16, DT_I8, DT_U8, DT_BOOL, DT_F32 = 1, 2, 3, 4, 5, 6
_DT = {torch.float16: DT_F16, torch.bfloat16: DT_BF16, torch.int8: DT_I8, torch.uint8: DT_U8, torch.bool: DT_BOOL,
       torch.float32: DT_F32}

P = ctypes.c_void_p
I32, I64, U32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32


class IfaDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", U32), ("query", P), ("key", P), ("value", P), ("attention_out", P),
        ("dtype_q", I32), ("dtype_kv", I32), ("dtype_out", I32), ("input_layout", ctypes.c_char_p),
        ("batch", I64), ("num_heads", I64), ("num_key_value_heads", I64), ("head_dim", I64), ("kv_seq_len", I64),
        ("scale_value", ctypes.c_double), ("actual_seq_lengths", P), ("kv_padding_size", P),
        ("kv_padding_size_count", I64), ("atten_mask", P), ("dtype_mask", I32), ("mask_batch", I64),
        ("mask_heads", I64), ("mask_seq", I64), ("pse_shift", P), ("antiquant_scale", P), ("antiquant_offset", P),
        ("antiquant_mode", I32), ("split_tokens", I64), ("profile_event_begin", P), ("profile_event_end", P),
        ("pse_batch", I64), ("pse_seq", I64), ("key_list", P), ("value_list", P), ("kv_list_seq_len", P),
        ("quant_scale2", P), ("quant_offset2", P), ("quant_count", I64), ("dtype_quant", I32)]


class IfaPagedArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", U32), ("query", P), ("key_cache", P), ("value_cache", P), ("attention_out", P),
        ("dtype_q", I32), ("dtype_kv", I32), ("dtype_out", I32), ("input_layout", ctypes.c_char_p),
        ("batch", I64), ("num_heads", I64), ("num_key_value_heads", I64), ("head_dim", I64),
        ("scale_value", ctypes.c_double), ("actual_seq_lengths", P), ("atten_mask", P), ("dtype_mask", I32),
        ("mask_batch", I64), ("mask_heads", I64), ("mask_seq", I64), ("pse_shift", P), ("antiquant_scale", P),
        ("antiquant_offset", P), ("antiquant_mode", I32), ("block_table", P), ("max_blocks_per_seq", I64),
        ("block_size", I64), ("num_blocks", I64), ("kv_cache_layout", I32), ("split_tokens", I64),
        ("profile_event_begin", P), ("profile_event_end", P), ("pse_batch", I64), ("pse_seq", I64),
        ("quant_scale2", P), ("quant_offset2", P), ("quant_count", I64), ("dtype_quant", I32)]


class SfaMlaArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", U32), ("query", P), ("query_rope", P), ("key", P), ("key_rope", P), ("value", P),
        ("sparse_indices", P), ("block_table", P), ("actual_seq_lengths_query", P), ("actual_seq_lengths_kv", P),
        ("attention_out", P), ("dtype", I32), ("batch", I64), ("q_seq", I64), ("q_heads", I64), ("kv_heads", I64),
        ("head_dim", I64), ("rope_dim", I64), ("sparse_size", I64), ("block_size", I64), ("num_blocks", I64),
        ("max_blocks", I64), ("scale_value", ctypes.c_float), ("sparse_block_size", I64), ("sparse_mode", I64),
        ("attention_mode", I64), ("layout_query", ctypes.c_char_p), ("layout_kv", ctypes.c_char_p),
        ("split_hint", I64), ("profile_event_begin", P), ("profile_event_end", P), ("q_tokens", I64),
        ("kv_tokens", I64), ("kv_seq", I64), ("softmax_max_out", P), ("softmax_sum_out", P),
        ("return_softmax_lse", I32)]


class SfaMlaPlan(ctypes.Structure):
    _fields_ = [("chunks", ctypes.c_int32), ("chunk_entries", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("all_heads", ctypes.c_int32)]


class IfaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s returned %d (%s)" % (what, status, status_string(status)))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        size_t_p = ctypes.POINTER(ctypes.c_size_t)
        for name, st in (("ifa_decode", IfaDecodeArgs), ("ifa_decode_paged", IfaPagedArgs),
                         ("sfa_decode_mla", SfaMlaArgs)):
            ws = getattr(L, name + "_workspace_size")
            ws.argtypes = [ctypes.POINTER(st), size_t_p]
            ws.restype = ctypes.c_int
            run = getattr(L, name)
            run.argtypes = [ctypes.POINTER(st), P, ctypes.c_size_t, P]
            run.restype = ctypes.c_int
        L.sfa_decode_mla_plan.argtypes = [ctypes.POINTER(SfaMlaArgs), ctypes.POINTER(SfaMlaPlan)]
        L.sfa_decode_mla_plan.restype = ctypes.c_int
        L.ifa_decode_noalloc.argtypes = [ctypes.POINTER(IfaDecodeArgs), P]
        L.ifa_decode_noalloc.restype = ctypes.c_int
        L.ifa_status_string.argtypes = [ctypes.c_int]
        L.ifa_status_string.restype = ctypes.c_char_p
        L.ifa_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ifa_status_string(status).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _host_i64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        a = a.cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).reshape(-1))


def _on_stream(stream):
    """Context that makes `stream` (None: the current stream; a torch stream;
    or a raw HIP stream handle) current while a call allocates its workspace,
    copies its pointer arrays and launches: those allocations then belong to
    the launch stream, so torch's caching allocator hands their memory to
    other work only after the call's kernels on that stream."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _check_operands(q: torch.Tensor, operands: dict, int32: tuple = ()) -> None:
    """Reject operands the kernels cannot read as the C ABI describes them:
    every tensor must be a contiguous GPU tensor on the query's device (a CPU
    tensor would hand a host address to a kernel, a strided view would be
    read as if it were dense), and index / length tensors must be int32."""
    for name in int32:
        t = operands.get(name)
        if t is not None and t.dtype != torch.int32:
            raise ValueError("%s must be torch.int32, got %s" % (name, t.dtype))
    for name, t in operands.items():
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous (an expanded or strided view is read as dense)" % name)
    if not q.is_cuda:
        raise ValueError("query must be a GPU tensor, got one on %s" % q.device)
    for name, t in operands.items():
        if t is not None and t.device != q.device:
            raise ValueError("%s must be on the query's device %s, got %s" % (name, q.device, t.device))


def _run(name: str, args, workspace: Optional[torch.Tensor], device) -> int:
    """Size the workspace, allocate one when none (or too small a one) is
    given, and call the entry point on the current stream."""
    L = lib()
    nbytes = ctypes.c_size_t(0)
    rc = getattr(L, name + "_workspace_size")(ctypes.byref(args), ctypes.byref(nbytes))
    if rc != IFA_OK:
        raise IfaError(rc, name + "_workspace_size")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=device)
    rc = getattr(L, name)(ctypes.byref(args), ctypes.c_void_p(workspace.data_ptr()),
                          ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != IFA_OK:
        raise IfaError(rc, name)
    return int(nbytes.value)


def _mask_fields(mask):
    if mask is None:
        return None, 0, 0, 0, 0
    if mask.dim() != 4 or mask.shape[2] != 1:
        raise ValueError("atten_mask must be (B|1, N|1, 1, S)")
    return mask, _DT[mask.dtype], mask.shape[0], mask.shape[1], mask.shape[3]


def _pse_fields(pse, q, num_heads):
    """(pointer, pse_batch, pse_seq) of a pseShift tensor (pse_batch, N, 1, pse_seq) in the query dtype."""
    if pse is None:
        return None, 0, 0
    if pse.dim() != 4 or pse.shape[1] != num_heads or pse.shape[2] != 1:
        raise ValueError("pse_shift must be (B|1, N, 1, S_pse)")
    if pse.dtype != q.dtype or not pse.is_contiguous():
        raise ValueError("pse_shift must be contiguous, in the query dtype")
    return pse, pse.shape[0], pse.shape[3]


def _kv_lists(key_list, value_list, input_layout, device):
    """Device pointer arrays and host lengths of per-batch K/V tensors (batch 1 each)."""
    if len(key_list) != len(value_list):
        raise ValueError("key and value lists differ in length")
    for t in list(key_list) + list(value_list):
        if not t.is_contiguous() or t.shape[0] != 1:
            raise ValueError("list tensors must be contiguous, of batch 1")
    seq_axis = 2 if input_layout == "BNSD" else 1
    kp = torch.tensor([t.data_ptr() for t in key_list], dtype=torch.int64, device=device)
    vp = torch.tensor([t.data_ptr() for t in value_list], dtype=torch.int64, device=device)
    seq = np.ascontiguousarray([t.shape[seq_axis] for t in key_list], dtype=np.int64)
    return kp, vp, seq


def _set_quant(a, quant_scale2, quant_offset2):
    """int8 output: quantScale2 (required) and quantOffset2 (optional), 1 or N*D values, fp32 or bf16."""
    if quant_scale2 is None:
        if quant_offset2 is not None:
            raise ValueError("quant_offset2 without quant_scale2")
        return
    if quant_offset2 is not None and (quant_offset2.dtype != quant_scale2.dtype or
                                      quant_offset2.numel() != quant_scale2.numel()):
        raise ValueError("quant_offset2 must match quant_scale2 in dtype and size")
    a.quant_scale2, a.quant_offset2 = _ptr(quant_scale2), _ptr(quant_offset2)
    a.quant_count, a.dtype_quant = quant_scale2.numel(), _DT[quant_scale2.dtype]


def ifa_decode_args(q, k, v, out, *, num_heads, num_key_value_heads=0, input_layout="BSH", scale_value,
                    actual_seq_lengths=None, kv_padding_size=None, atten_mask=None, pse_shift=None,
                    antiquant_scale=None, antiquant_offset=None, antiquant_mode=0, split_tokens=0, keep=None,
                    key_list=None, value_list=None, quant_scale2=None, quant_offset2=None):
    """Fill an IfaDecodeArgs from tensors; `keep` collects arrays that must outlive the call.
    With key_list / value_list (per-batch tensors of batch 1), k and v must be None.
    scale_value is required: the scale is an argument of the operator, not
    something this marshalling layer derives."""
    _check_operands(q, dict(query=q, key=k, value=v, attention_out=out, atten_mask=atten_mask, pse_shift=pse_shift,
                            antiquant_scale=antiquant_scale, antiquant_offset=antiquant_offset,
                            quant_scale2=quant_scale2, quant_offset2=quant_offset2))
    for t in list(key_list or []) + list(value_list or []):
        _check_operands(q, {"key_list/value_list entry": t})
    N = int(num_heads)
    kref = k if key_list is None else key_list[0]
    if input_layout == "BSH":
        B, H, S = q.shape[0], q.shape[2], kref.shape[1]
        D = H // N
    elif input_layout == "BNSD":
        B, D, S = q.shape[0], q.shape[3], kref.shape[2]
    elif input_layout == "BSND":
        B, D, S = q.shape[0], q.shape[3], kref.shape[1]
    else:
        B, D, S = q.shape[0], 0, 0
    lists = None
    if key_list is not None:
        lists = _kv_lists(key_list, value_list, input_layout, q.device)
        S = 0
    lens = _host_i64(actual_seq_lengths)
    pads = _host_i64(kv_padding_size)
    mask, dmask, mB, mN, mS = _mask_fields(atten_mask)
    pse, pB, pS = _pse_fields(pse_shift, q, N)
    if keep is not None:
        keep.extend([lens, pads, input_layout.encode(), lists])
    a = IfaDecodeArgs()
    a.struct_size = ctypes.sizeof(IfaDecodeArgs)
    a.query, a.key, a.value, a.attention_out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.dtype_q, a.dtype_kv, a.dtype_out = _DT[q.dtype], _DT[kref.dtype], _DT[out.dtype]
    if lists is not None:
        a.key_list, a.value_list = lists[0].data_ptr(), lists[1].data_ptr()
        a.kv_list_seq_len = lists[2].ctypes.data
    _set_quant(a, quant_scale2, quant_offset2)
    a.input_layout = input_layout.encode()
    a.batch, a.num_heads, a.num_key_value_heads, a.head_dim, a.kv_seq_len = B, N, int(num_key_value_heads), D, S
    a.scale_value = float(scale_value)
    a.actual_seq_lengths = None if lens is None else lens.ctypes.data
    a.kv_padding_size = None if pads is None else pads.ctypes.data
    a.kv_padding_size_count = 0 if pads is None else len(pads)
    a.atten_mask, a.dtype_mask, a.mask_batch, a.mask_heads, a.mask_seq = _ptr(mask), dmask, mB, mN, mS
    a.pse_shift, a.pse_batch, a.pse_seq = _ptr(pse), pB, pS
    a.antiquant_scale, a.antiquant_offset = _ptr(antiquant_scale), _ptr(antiquant_offset)
    a.antiquant_mode = int(antiquant_mode)
    a.split_tokens = int(split_tokens)
    return a


def ifa_decode(q, k, v, out, *, workspace=None, stream=None, **kw) -> int:
    """IncreFlashAttention over a dense padded cache; writes `out`, returns workspace bytes used."""
    keep: list = []
    with _on_stream(stream):     # the list pointer arrays and the workspace belong to the launch stream
        a = ifa_decode_args(q, k, v, out, keep=keep, **kw)
        return _run("ifa_decode", a, workspace, q.device)


def ifa_decode_noalloc(q, k, v, out, *, stream=None, **kw) -> None:
    """ifa_decode on the library's built-in scratch (no workspace, nothing
    allocated by the library); raises IfaError(161002) when the call needs more
    scratch than the library holds.  With key_list / value_list this wrapper
    builds the two device pointer arrays itself, which allocates: a caller
    that cannot allocate passes its own arrays to the C entry point."""
    keep: list = []
    with _on_stream(stream):
        a = ifa_decode_args(q, k, v, out, keep=keep, **kw)
        rc = lib().ifa_decode_noalloc(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != IFA_OK:
        raise IfaError(rc, "ifa_decode_noalloc")


def ifa_paged_args(q, key_cache, value_cache, out, block_table, *, num_heads, num_key_value_heads=0,
                   input_layout="BNSD", scale_value, actual_seq_lengths=None, atten_mask=None,
                   pse_shift=None, antiquant_scale=None, antiquant_offset=None, antiquant_mode=0, kv_cache_layout=0,
                   split_tokens=0, keep=None, quant_scale2=None, quant_offset2=None):
    """Fill an IfaPagedArgs from tensors; block_table is a device int32 tensor."""
    _check_operands(q, dict(query=q, key_cache=key_cache, value_cache=value_cache, attention_out=out,
                            block_table=block_table, atten_mask=atten_mask, pse_shift=pse_shift,
                            antiquant_scale=antiquant_scale, antiquant_offset=antiquant_offset,
                            quant_scale2=quant_scale2, quant_offset2=quant_offset2), int32=("block_table",))
    N = int(num_heads)
    nkv = int(num_key_value_heads) or N
    if kv_cache_layout == 0:
        nblk, bs, D = key_cache.shape[0], key_cache.shape[2], key_cache.shape[3]
    else:
        nblk, bs = key_cache.shape[0], key_cache.shape[1]
        D = key_cache.shape[2] // nkv
    lens = _host_i64(actual_seq_lengths)
    mask, dmask, mB, mN, mS = _mask_fields(atten_mask)
    pse, pB, pS = _pse_fields(pse_shift, q, N)
    if keep is not None:
        keep.extend([lens, input_layout.encode()])
    a = IfaPagedArgs()
    a.struct_size = ctypes.sizeof(IfaPagedArgs)
    a.query, a.key_cache, a.value_cache, a.attention_out = _ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(out)
    a.dtype_q, a.dtype_kv, a.dtype_out = _DT[q.dtype], _DT[key_cache.dtype], _DT[out.dtype]
    a.input_layout = input_layout.encode()
    a.batch, a.num_heads, a.num_key_value_heads, a.head_dim = q.shape[0], N, int(num_key_value_heads), D
    a.scale_value = float(scale_value)
    a.actual_seq_lengths = None if lens is None else lens.ctypes.data
    a.atten_mask, a.dtype_mask, a.mask_batch, a.mask_heads, a.mask_seq = _ptr(mask), dmask, mB, mN, mS
    a.pse_shift, a.pse_batch, a.pse_seq = _ptr(pse), pB, pS
    a.antiquant_scale, a.antiquant_offset = _ptr(antiquant_scale), _ptr(antiquant_offset)
    a.antiquant_mode = int(antiquant_mode)
    a.block_table = _ptr(block_table)
    a.max_blocks_per_seq = block_table.shape[1]
    a.block_size, a.num_blocks, a.kv_cache_layout = bs, nblk, int(kv_cache_layout)
    a.split_tokens = int(split_tokens)
    _set_quant(a, quant_scale2, quant_offset2)
    return a


def ifa_decode_paged(q, key_cache, value_cache, out, block_table, *, workspace=None, stream=None, **kw) -> int:
    """IncreFlashAttention over a paged cache; writes `out`, returns workspace bytes used."""
    keep: list = []
    with _on_stream(stream):
        a = ifa_paged_args(q, key_cache, value_cache, out, block_table, keep=keep, **kw)
        return _run("ifa_decode_paged", a, workspace, q.device)


def sfa_args(query, query_rope, key, key_rope, value, sparse_indices, block_table, actual_seq_lengths_kv, out, *,
             scale_value, actual_seq_lengths_query=None, sparse_mode=0, sparse_block_size=1,
             attention_mode=2, layout_query="BSND", layout_kv="PA_BSND", split_hint=0, keep=None,
             softmax_max_out=None, softmax_sum_out=None):
    """Fill an SfaMlaArgs.  query BSND [B, Q_S, Q_N, D] or TND [Q_T, Q_N, D] (B = the length of
    actual_seq_lengths_query); key PA_BSND [blocks, block_size, 1, D], BSND [B, KV_S, 1, D] or
    TND [KV_T, 1, D].  Index, table and length tensors are device int32.  softmax_max_out /
    softmax_sum_out (both or neither): fp32 tensors of (query rows) x Q_N elements, which turn on
    return_softmax_lse."""
    if (softmax_max_out is None) != (softmax_sum_out is None):
        raise ValueError("softmax_max_out and softmax_sum_out go together")
    for t in (softmax_max_out, softmax_sum_out):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("softmax_max_out / softmax_sum_out must be torch.float32")
    _check_operands(query, dict(query=query, query_rope=query_rope, key=key, key_rope=key_rope, value=value,
                                sparse_indices=sparse_indices, block_table=block_table,
                                actual_seq_lengths_kv=actual_seq_lengths_kv,
                                actual_seq_lengths_query=actual_seq_lengths_query, attention_out=out,
                                softmax_max_out=softmax_max_out, softmax_sum_out=softmax_sum_out),
                    int32=("sparse_indices", "block_table", "actual_seq_lengths_kv", "actual_seq_lengths_query"))
    if layout_query == "TND":
        QT, QN, D = query.shape
        if actual_seq_lengths_query is None:
            raise ValueError("a TND query needs actual_seq_lengths_query (prefix sums)")
        B, QS = actual_seq_lengths_query.shape[0], 1
    else:
        B, QS, QN, D = query.shape
        QT = 0
    DR = query_rope.shape[-1]
    a = SfaMlaArgs()
    a.struct_size = ctypes.sizeof(SfaMlaArgs)
    a.query, a.query_rope, a.key, a.key_rope, a.value = (_ptr(query), _ptr(query_rope), _ptr(key),
                                                         _ptr(key_rope), _ptr(value))
    a.sparse_indices, a.block_table = _ptr(sparse_indices), _ptr(block_table)
    a.actual_seq_lengths_query = _ptr(actual_seq_lengths_query)
    a.actual_seq_lengths_kv = _ptr(actual_seq_lengths_kv)
    a.attention_out = _ptr(out)
    a.dtype = _DT[query.dtype]
    a.batch, a.q_seq, a.q_heads, a.kv_heads = B, QS, QN, key.shape[-2]
    a.head_dim, a.rope_dim = D, DR
    a.sparse_size = sparse_indices.shape[-1]
    if layout_kv == "PA_BSND":
        a.block_size, a.num_blocks = key.shape[1], key.shape[0]
        a.max_blocks = block_table.shape[1]
    elif layout_kv == "BSND":
        a.kv_seq = key.shape[1]
    else:
        a.kv_tokens = key.shape[0]
    a.q_tokens = QT
    a.scale_value = float(scale_value)
    a.sparse_block_size, a.sparse_mode, a.attention_mode = sparse_block_size, sparse_mode, attention_mode
    lq, lk = layout_query.encode(), layout_kv.encode()
    if keep is not None:
        keep.extend([lq, lk])
    a.layout_query, a.layout_kv = lq, lk
    a.split_hint = int(split_hint)
    if softmax_max_out is not None:
        a.softmax_max_out, a.softmax_sum_out = _ptr(softmax_max_out), _ptr(softmax_sum_out)
        a.return_softmax_lse = 1
    return a


def sfa_decode_mla_plan(query, query_rope, key, key_rope, value, sparse_indices, block_table,
                        actual_seq_lengths_kv, out, **kw) -> dict:
    """The launch sfa_decode_mla would make for these arguments (sfa_decode_mla_plan):
    chunks per query row, entries per chunk, workgroups, and whether one workgroup
    takes every head of a chunk."""
    keep: list = []
    a = sfa_args(query, query_rope, key, key_rope, value, sparse_indices, block_table, actual_seq_lengths_kv, out,
                 keep=keep, **kw)
    pl = SfaMlaPlan()
    rc = lib().sfa_decode_mla_plan(ctypes.byref(a), ctypes.byref(pl))
    if rc != 0:
        raise IfaError(rc, "sfa_decode_mla_plan")
    return dict(chunks=pl.chunks, chunk_entries=pl.chunk_entries, workgroups=pl.workgroups,
                all_heads=bool(pl.all_heads))


def sfa_decode_mla(query, query_rope, key, key_rope, value, sparse_indices, block_table, actual_seq_lengths_kv,
                   out, *, workspace=None, stream=None, **kw) -> int:
    """SparseFlashAttention (MLA-absorb); writes `out`, returns workspace bytes used."""
    keep: list = []
    with _on_stream(stream):
        a = sfa_args(query, query_rope, key, key_rope, value, sparse_indices, block_table, actual_seq_lengths_kv,
                     out, keep=keep, **kw)
        return _run("sfa_decode_mla", a, workspace, query.device)
