"""Seeded synthetic inputs for the decode-attention workloads.

This module only draws random numbers and lays them out in the tensor shapes
the operator pages describe.  It holds none of the attention arithmetic, so the
oracle (test infrastructure) and the HIP library can both be fed from it
without sharing any computation.

Every tensor ``t`` of workload ``k`` is drawn from
``numpy.random.default_rng([6, k, t])`` so that draws do not depend on the
order in which tensors are made.  Tensor ids:

    0 lengths  1 q  2 k  3 v  4 mask  5 block permutation  6 padding offsets
    7 antiquant scale  8 antiquant offset  9 q_rope  10 k_rope
    11 sparse valid counts  12 sparse indices  13 positional bias (pseShift)
    14 per-batch cache lengths of tensor lists  15 output quant scale  16 output quant offset

Normals are float32 ``standard_normal`` draws rounded to nearest-even into
fp16/bf16; integers are uniform and inclusive.  Whole buffers are filled,
including positions past each sequence's length and blocks no sequence uses,
so a kernel that reads out of range changes its answer.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

TID_LEN, TID_Q, TID_K, TID_V, TID_MASK, TID_PERM, TID_PAD = 0, 1, 2, 3, 4, 5, 6
TID_AQ_SCALE, TID_AQ_OFFSET, TID_QROPE, TID_KROPE, TID_NVALID, TID_IDX = 7, 8, 9, 10, 11, 12
TID_PSE = 13
TID_LIST = 14
TID_QSCALE2, TID_QOFFSET2 = 15, 16

_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8, "f32": torch.float32}
_CHUNK = 1 << 24


def rng_for(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([6, int(cfg_id), int(tensor_id)])


def normal_tensor(rng: np.random.Generator, shape: Sequence[int], dtype: str) -> torch.Tensor:
    """float32 N(0,1) draws rounded RNE to ``dtype`` (fp16 or bf16)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=_TORCH_DT[dtype])
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = torch.from_numpy(rng.standard_normal(e - s, dtype=np.float32)).to(out.dtype)
    return out.view(*shape)


def int8_tensor(rng: np.random.Generator, shape: Sequence[int], lo: int = -127, hi: int = 127) -> torch.Tensor:
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.int8)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = torch.from_numpy(rng.integers(lo, hi, size=e - s, endpoint=True, dtype=np.int8))
    return out.view(*shape)


def uniform_tensor(rng: np.random.Generator, shape: Sequence[int], lo: float, hi: float, dtype: str) -> torch.Tensor:
    a = rng.uniform(lo, hi, size=int(np.prod(shape))).astype(np.float32)
    return torch.from_numpy(a).to(_TORCH_DT[dtype]).view(*shape)


# --------------------------------------------------------------------------
# IncreFlashAttention workloads (dense padded cache or paged cache)
# --------------------------------------------------------------------------
@dataclass
class IfaSpec:
    name: str
    cfg_id: int
    q_dtype: str                 # "f16" | "bf16"
    kv_dtype: str                # "f16" | "bf16" | "i8"
    B: int
    N: int
    Nkv: int                     # 0 means Nkv == N
    D: int
    layout: str = "BNSD"         # query layout; dense KV uses the same layout
    S: int = 0                   # Smax of the padded cache (dense); mask length (paged)
    scale: float = 0.0           # 0 -> 1/sqrt(D)
    lengths: Optional[Sequence[int]] = None       # explicit per-batch lengths
    len_range: Optional[tuple] = None              # (lo, hi) inclusive uniform draw
    no_lengths: bool = False     # pass actualSeqLengths = NULL
    # left padding: pad_b = S - L_b - offset_b, offset_b ~ U{pad_off}
    pad_off: Optional[tuple] = None
    pads: Optional[Sequence[int]] = None           # explicit kvPaddingSize values
    # mask
    mask: Optional[str] = None   # None | "bool" | "i8" | "u8"
    mask_p: float = 0.0          # Bernoulli rate on valid positions
    mask_heads: int = 1          # 1 or N
    mask_batch: int = 0          # 0 -> B, else 1
    # paged cache
    paged: bool = False
    block_size: int = 128
    num_blocks: int = 0          # 0 -> exactly the blocks needed (rounded up)
    max_blocks: int = 0          # 0 -> ceil(S / block_size)
    cache_layout: int = 0        # 0: (blocknum, KV_N, bs, D)  1: (blocknum, bs, H)
    # int8 antiquant
    antiquant: Optional[str] = None  # None | "per_channel" | "per_tensor"
    aq_scale: tuple = (0.005, 0.02)
    aq_offset: tuple = (-2.0, 2.0)
    q_mult: float = 1.0          # multiplies q after rounding (a "peaky" variant), re-rounded
    # positional bias (pseShift): (pse_batch, N, 1, S_pse), query dtype, N(0,1) * pse_scale
    pse: bool = False
    pse_batch: int = 0           # 0 -> B, else 1
    pse_scale: float = 1.0
    # per-batch K/V tensors (tensor lists): batch b gets its own cache of
    # S_b = L_b + U{0..list_slack} positions (at most S), cut from the padded one
    kv_list: bool = False
    list_slack: int = 16
    # int8 output (post-quantisation): quantScale2 ~ U[qs_range], quantOffset2 ~ U[qo_range]
    out_int8: Optional[str] = None       # None | "per_tensor" | "per_channel"
    quant_dtype: str = "f32"             # "f32" | "bf16"
    quant_offset: bool = True
    qs_range: tuple = (100.0, 400.0)
    qo_range: tuple = (-8.0, 8.0)

    @property
    def nkv(self) -> int:
        return self.N if self.Nkv == 0 else self.Nkv

    @property
    def scale_value(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.D)


def _draw_lengths(spec: IfaSpec, smax: int) -> np.ndarray:
    if spec.lengths is not None:
        return np.asarray(spec.lengths, dtype=np.int64)
    lo, hi = spec.len_range if spec.len_range else (smax, smax)
    return rng_for(spec.cfg_id, TID_LEN).integers(lo, hi, size=spec.B, endpoint=True).astype(np.int64)


def make_ifa(spec: IfaSpec) -> dict:
    """Host tensors (torch CPU) for one IFA call described by ``spec``."""
    B, N, nkv, D = spec.B, spec.N, spec.nkv, spec.D
    k_id = spec.cfg_id
    out: dict = {"spec": spec}
    q = normal_tensor(rng_for(k_id, TID_Q), (B * N * D,), spec.q_dtype)
    if spec.q_mult != 1.0:
        q = (q.float() * spec.q_mult).to(q.dtype)
    if spec.layout == "BSH":
        q = q.view(B, 1, N * D)
    elif spec.layout == "BSND":
        q = q.view(B, 1, N, D)
    else:
        q = q.view(B, N, 1, D)
    out["q"] = q

    if spec.paged:
        bs = spec.block_size
        smax = spec.S if spec.S else (spec.max_blocks * bs if spec.max_blocks else 8192)
        lengths = _draw_lengths(spec, smax)
        max_blocks = spec.max_blocks or max(1, math.ceil(smax / bs))
        need = int(sum(math.ceil(int(L) / bs) for L in lengths))
        nblk = spec.num_blocks or max(1, B * max_blocks)
        if nblk < need:
            raise ValueError("num_blocks too small for the drawn lengths")
        perm = rng_for(k_id, TID_PERM).permutation(nblk)
        if nblk >= B * max_blocks:
            bt = perm[: B * max_blocks].reshape(B, max_blocks)
        else:  # fewer physical blocks than table slots: hand out used slots first, pad with valid ids
            bt = np.zeros((B, max_blocks), dtype=np.int64)
            pos = 0
            for b in range(B):
                nb = math.ceil(int(lengths[b]) / bs)
                bt[b, :nb] = perm[pos:pos + nb]
                pos += nb
                bt[b, nb:] = perm[(np.arange(max_blocks - nb) + pos) % nblk]
        out["block_table"] = torch.from_numpy(np.ascontiguousarray(bt.astype(np.int32)))
        if spec.cache_layout == 0:
            kv_shape = (nblk, nkv, bs, D)
        else:
            kv_shape = (nblk, bs, nkv * D)
        out["S"] = smax
        out["num_blocks"] = nblk
        out["max_blocks"] = max_blocks
    else:
        smax = spec.S
        lengths = _draw_lengths(spec, smax)
        if spec.layout == "BSH":
            kv_shape = (B, smax, nkv * D)
        elif spec.layout == "BSND":
            kv_shape = (B, smax, nkv, D)
        else:
            kv_shape = (B, nkv, smax, D)
        out["S"] = smax

    if spec.kv_dtype == "i8":
        out["k"] = int8_tensor(rng_for(k_id, TID_K), kv_shape)
        out["v"] = int8_tensor(rng_for(k_id, TID_V), kv_shape)
    else:
        out["k"] = normal_tensor(rng_for(k_id, TID_K), kv_shape, spec.kv_dtype)
        out["v"] = normal_tensor(rng_for(k_id, TID_V), kv_shape, spec.kv_dtype)

    out["actual_seq_lengths"] = None if spec.no_lengths else lengths
    out["lengths_drawn"] = lengths

    pads = None
    if spec.pads is not None:
        pads = np.asarray(spec.pads, dtype=np.int64)
    elif spec.pad_off is not None:
        offs = rng_for(k_id, TID_PAD).integers(spec.pad_off[0], spec.pad_off[1], size=B, endpoint=True)
        pads = (smax - lengths - offs).astype(np.int64)
    out["kv_padding_size"] = pads

    if spec.mask is not None:
        mb = 1 if spec.mask_batch == 1 else B
        mh = spec.mask_heads
        ms = smax
        r = rng_for(k_id, TID_MASK).random((mb, mh, ms))
        m = r < spec.mask_p
        # The bits outside each batch's valid window are set to 0 ("attend"),
        # so a kernel that ignores the lengths reads them and is caught.
        for bi in range(mb):
            L = int(lengths[bi]) if mb == B else int(lengths.max())
            if spec.paged or pads is None:
                m[bi, :, L:] = False
            else:
                p = max(0, int(pads[bi]))
                lo_, hi_ = smax - p - L, smax - p
                m[bi, :, :max(lo_, 0)] = False
                m[bi, :, max(hi_, 0):] = False
        m = m.reshape(mb, mh, 1, ms)
        if spec.mask == "bool":
            out["mask"] = torch.from_numpy(m)
        elif spec.mask == "i8":
            out["mask"] = torch.from_numpy(m.astype(np.int8))
        else:
            out["mask"] = torch.from_numpy(m.astype(np.uint8))
    else:
        out["mask"] = None

    if spec.pse:
        pb = 1 if spec.pse_batch == 1 else B
        ps = out["max_blocks"] * spec.block_size if spec.paged else smax
        bias = normal_tensor(rng_for(k_id, TID_PSE), (pb * N * ps,), spec.q_dtype)
        if spec.pse_scale != 1.0:
            bias = (bias.float() * spec.pse_scale).to(bias.dtype)
        out["pse"] = bias.view(pb, N, 1, ps)
    else:
        out["pse"] = None

    if spec.kv_list:
        if spec.paged or pads is not None:
            raise ValueError("tensor lists are dense and take no left padding")
        extra = rng_for(k_id, TID_LIST).integers(0, spec.list_slack, size=B, endpoint=True)
        seq = np.minimum(lengths + extra, smax).astype(np.int64)
        seq = np.maximum(seq, 1)
        cut = (lambda t, b, n: t[b:b + 1, :, :n]) if spec.layout == "BNSD" else (lambda t, b, n: t[b:b + 1, :n])
        out["k_list"] = [cut(out["k"], b, int(seq[b])).contiguous() for b in range(B)]
        out["v_list"] = [cut(out["v"], b, int(seq[b])).contiguous() for b in range(B)]
        out["list_seq"] = seq

    if spec.out_int8 is not None:
        n = 1 if spec.out_int8 == "per_tensor" else N * D
        qdt = "f32" if spec.quant_dtype == "f32" else "bf16"
        out["quant_scale2"] = uniform_tensor(rng_for(k_id, TID_QSCALE2), (n,), *spec.qs_range, qdt)
        out["quant_offset2"] = (uniform_tensor(rng_for(k_id, TID_QOFFSET2), (n,), *spec.qo_range, qdt)
                                if spec.quant_offset else None)
    else:
        out["quant_scale2"] = out["quant_offset2"] = None

    if spec.antiquant is not None:
        shp = (2,) if spec.antiquant == "per_tensor" else (2, nkv, 1, D)
        out["aq_scale"] = uniform_tensor(rng_for(k_id, TID_AQ_SCALE), shp, *spec.aq_scale, spec.q_dtype)
        out["aq_offset"] = uniform_tensor(rng_for(k_id, TID_AQ_OFFSET), shp, *spec.aq_offset, spec.q_dtype)
        out["aq_mode"] = 1 if spec.antiquant == "per_tensor" else 2
    else:
        out["aq_scale"] = out["aq_offset"] = None
        out["aq_mode"] = 0
    return out


# --------------------------------------------------------------------------
# SparseFlashAttention (MLA-absorb, PA_BSND cache) workloads
# --------------------------------------------------------------------------
@dataclass
class SfaSpec:
    name: str
    cfg_id: int
    dtype: str = "bf16"
    B: int = 32
    QN: int = 128
    D: int = 512
    DR: int = 64
    block_size: int = 64
    num_blocks: int = 32768
    max_blocks: int = 1024
    lkv_range: tuple = (8192, 65536)
    lkv: Optional[Sequence[int]] = None
    sparse_size: int = 2048
    tail_range: tuple = (1, 256)          # number of trailing -1 entries per row
    n_valid: Optional[Sequence[int]] = None
    sorted_indices: bool = False
    value_aliases_key: bool = False
    scale: float = 0.0                    # 0 -> float32(1/sqrt(D + DR))
    sparse_mode: int = 0
    # breadth beyond one query row over a paged cache
    QS: int = 1                           # query rows per batch (BSND query)
    lq: Optional[Sequence[int]] = None    # valid query rows per batch (None: QS each)
    pass_lq: bool = False                 # hand actual_seq_lengths_query over even when it is all QS
    layout_q: str = "BSND"                # "BSND" | "TND" (rows packed, lq as prefix sums)
    layout_kv: str = "PA_BSND"            # "PA_BSND" | "BSND" | "TND"
    kv_seq: int = 0                       # KV_S of a BSND cache (0: the largest length)
    sparse_block_size: int = 1            # positions named by one index
    past_limit: bool = False              # also select positions past the causal limit

    @property
    def scale_value(self) -> float:
        s = self.scale if self.scale else 1.0 / math.sqrt(self.D + self.DR)
        return float(np.float32(s))


def make_sfa(spec: SfaSpec) -> dict:
    """Host tensors for one SFA call.  Query rows are enumerated batch by batch
    (BSND: QS per batch, padding rows included; TND: the valid rows only);
    each row draws its own index list: distinct blocks of sparse_block_size
    positions, from below the row's causal limit under sparse_mode 3 (below
    the kv length with ``past_limit``), valid ones first, then -1."""
    B, QN, D, DR, bs = spec.B, spec.QN, spec.D, spec.DR, spec.block_size
    sbs = spec.sparse_block_size
    k_id = spec.cfg_id
    out: dict = {"spec": spec}
    if spec.lkv is not None:
        lkv = np.asarray(spec.lkv, dtype=np.int64)
    else:
        lkv = rng_for(k_id, TID_LEN).integers(spec.lkv_range[0], spec.lkv_range[1], size=B, endpoint=True)
    lq = np.asarray(spec.lq if spec.lq is not None else [spec.QS] * B, dtype=np.int64)
    if (lq < 0).any() or (spec.layout_q == "BSND" and (lq > spec.QS).any()):
        raise ValueError("query lengths outside [0, QS]")
    # query row -> (batch, position in the batch's query)
    if spec.layout_q == "TND":
        rows_b = np.repeat(np.arange(B), lq)
        rows_s = np.concatenate([np.arange(n) for n in lq]) if B else np.zeros(0, np.int64)
    else:
        rows_b = np.repeat(np.arange(B), spec.QS)
        rows_s = np.tile(np.arange(spec.QS), B)
    R = len(rows_b)
    qshape = (R, QN) if spec.layout_q == "TND" else (B, spec.QS, QN)
    out["q"] = normal_tensor(rng_for(k_id, TID_Q), qshape + (D,), spec.dtype)
    out["q_rope"] = normal_tensor(rng_for(k_id, TID_QROPE), qshape + (DR,), spec.dtype)

    if spec.layout_kv == "PA_BSND":
        if int(lkv.max(initial=0)) > spec.max_blocks * bs:
            raise ValueError("lkv exceeds the block table's reach")
        kshape = (spec.num_blocks, bs, 1)
    elif spec.layout_kv == "BSND":
        kv_seq = spec.kv_seq or int(lkv.max(initial=1))
        if int(lkv.max(initial=0)) > kv_seq:
            raise ValueError("lkv exceeds KV_S")
        kshape = (B, kv_seq, 1)
        out["kv_seq"] = kv_seq
    else:
        kshape = (max(1, int(lkv.sum())), 1)
    out["key"] = normal_tensor(rng_for(k_id, TID_K), kshape + (D,), spec.dtype)
    out["key_rope"] = normal_tensor(rng_for(k_id, TID_KROPE), kshape + (DR,), spec.dtype)
    out["value"] = out["key"] if spec.value_aliases_key else normal_tensor(
        rng_for(k_id, TID_V), kshape + (D,), spec.dtype)
    if spec.layout_kv == "PA_BSND":
        perm = rng_for(k_id, TID_PERM).permutation(spec.num_blocks)
        if spec.num_blocks >= B * spec.max_blocks:
            bt = perm[: B * spec.max_blocks].reshape(B, spec.max_blocks)
        else:
            bt = perm[np.arange(B * spec.max_blocks) % spec.num_blocks].reshape(B, spec.max_blocks)
        out["block_table"] = torch.from_numpy(np.ascontiguousarray(bt.astype(np.int32)))
    else:
        out["block_table"] = None

    # per query row: the domain of positions it selects from and how many blocks it takes
    limit = lkv[rows_b].copy()
    if spec.sparse_mode == 3 and not spec.past_limit:
        limit = np.minimum(limit, lkv[rows_b] - lq[rows_b] + rows_s + 1)
    limit = np.maximum(limit, 0)
    nblk_dom = (limit + sbs - 1) // sbs
    if spec.n_valid is not None:
        nval = np.asarray(spec.n_valid, dtype=np.int64)
        nval = np.resize(nval, R) if len(nval) != R else nval
    else:
        tails = rng_for(k_id, TID_NVALID).integers(spec.tail_range[0], spec.tail_range[1], size=R, endpoint=True)
        nval = spec.sparse_size - tails
    nval = np.minimum(np.maximum(nval, 0), np.minimum(spec.sparse_size, nblk_dom))
    idx = np.full((R, spec.sparse_size), -1, dtype=np.int32)
    r = rng_for(k_id, TID_IDX)
    for i in range(R):
        n = int(nval[i])
        if n:
            sel = r.choice(int(nblk_dom[i]), size=n, replace=False)
            if spec.sorted_indices:
                sel = np.sort(sel)
            idx[i, :n] = sel
    if spec.layout_q == "TND":
        out["sparse_indices"] = torch.from_numpy(idx.reshape(R, 1, spec.sparse_size))
    else:
        out["sparse_indices"] = torch.from_numpy(idx.reshape(B, spec.QS, 1, spec.sparse_size))
    if spec.layout_kv == "TND":
        out["actual_seq_lengths_kv"] = torch.from_numpy(np.cumsum(lkv).astype(np.int32))
    else:
        out["actual_seq_lengths_kv"] = torch.from_numpy(lkv.astype(np.int32))
    if spec.layout_q == "TND":
        out["actual_seq_lengths_query"] = torch.from_numpy(np.cumsum(lq).astype(np.int32))
    elif spec.lq is not None or spec.pass_lq:
        out["actual_seq_lengths_query"] = torch.from_numpy(lq.astype(np.int32))
    else:
        out["actual_seq_lengths_query"] = None
    out["lkv_counts"] = lkv
    out["lq_counts"] = lq
    out["row_batch"], out["row_pos"] = rows_b, rows_s
    out["q_rows"] = R
    out["n_valid"] = nval
    return out


# --------------------------------------------------------------------------
# Named workloads: the five shapes the decode path is measured on, and small
# variants of them that an fp64 CPU reference finishes in seconds.
# --------------------------------------------------------------------------
def workloads() -> dict:
    s128 = 1.0 / math.sqrt(128)
    return {
        "tiny_dense_f16": IfaSpec("tiny_dense_f16", 1, "f16", "f16", B=2, N=4, Nkv=2, D=64, layout="BNSD",
                                  S=256, lengths=[200, 256], scale=1.0 / 8),
        "dense_gqa_bf16_bsh": IfaSpec("dense_gqa_bf16_bsh", 2, "bf16", "bf16", B=64, N=32, Nkv=8, D=128,
                                      layout="BSH", S=8192, len_range=(1024, 8192), scale=s128),
        "paged_bf16_bs128": IfaSpec("paged_bf16_bs128", 3, "bf16", "bf16", B=64, N=32, Nkv=8, D=128,
                                    layout="BNSD", S=8192, len_range=(512, 8192), scale=s128, paged=True,
                                    block_size=128, num_blocks=4096, max_blocks=64, mask="bool", mask_p=0.05),
        "int8_leftpad_f16": IfaSpec("int8_leftpad_f16", 4, "f16", "i8", B=32, N=64, Nkv=8, D=128, layout="BNSD",
                                    S=32768, len_range=(4096, 32768), pad_off=(0, 64), antiquant="per_channel",
                                    scale=s128),
        "sfa_mla_bf16": SfaSpec("sfa_mla_bf16", 5),
        # multi-token decode: C5's shapes with two query rows per batch under rightDownCausal
        "sfa_mtp_bf16": SfaSpec("sfa_mtp_bf16", 7, QS=2, sparse_mode=3),
        # C5's shapes with the value tensor being the key tensor (the latent rows serve as both)
        "sfa_mla_alias_bf16": SfaSpec("sfa_mla_alias_bf16", 8, value_aliases_key=True),
        # the dense GQA workload with a per-batch positional bias (pseShift) of N(0, 4)
        "dense_pse_bf16_bsh": IfaSpec("dense_pse_bf16_bsh", 6, "bf16", "bf16", B=64, N=32, Nkv=8, D=128,
                                      layout="BSH", S=8192, len_range=(1024, 8192), scale=s128, pse=True,
                                      pse_scale=2.0),
    }


def small_variant(name: str) -> object:
    """A shrunken copy of a named workload (same structure, a few tiles per row)."""
    w = workloads()[name]
    if isinstance(w, SfaSpec):
        return replace(w, name=name + "_small", cfg_id=w.cfg_id + 100, B=3, QN=16, num_blocks=256,
                       max_blocks=64, lkv_range=(600, 4096), sparse_size=300, tail_range=(1, 40))
    if w.paged:
        return replace(w, name=name + "_small", cfg_id=w.cfg_id + 100, B=3, N=8, Nkv=2, S=1024,
                       len_range=(100, 1024), num_blocks=32, max_blocks=8)
    if w.kv_dtype == "i8":
        return replace(w, name=name + "_small", cfg_id=w.cfg_id + 100, B=3, N=16, Nkv=2, S=2048,
                       len_range=(300, 2048), pad_off=(0, 64))
    if w.B <= 2:
        return w
    return replace(w, name=name + "_small", cfg_id=w.cfg_id + 100, B=3, N=8, Nkv=2, S=1500,
                   len_range=(200, 1500))
