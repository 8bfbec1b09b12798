"""The benchmark's algorithmic byte counts (the numerator of its GB/s and of
roofline.achieved), checked against a position-by-position count on small
seeded workloads.

What a call must move, as the operator pages define the computation:
  * IncreFlashAttention: the K and V rows of every (position, KV head) in the
    batch's window that some query head of the head's group attends (a row
    that every head of the group masks out is never read), the mask bytes
    over the window, one block-table entry per cache block of the window,
    the antiquant parameters, the positional bias over the window, q and the
    output;
  * SparseFlashAttention: the key, rope and value row of every selected
    position below its query row's limit (the kv length, or the causal bound
    under sparse_mode 3; a value that is the key tensor moves once), the
    index lists, the device length arrays passed, one block-table entry per
    selected block with an attended position, q, q_rope and the output.
The counts below walk positions one at a time in plain loops, so an indexing
slip in the vectorised count (a window edge, the group of a per-head mask, a
partly attended block) shows up as a difference."""
import math

import numpy as np
import pytest

import bench
from decode_attention_kv_06_amd.workloads import IfaSpec, SfaSpec, make_ifa, make_sfa


def ifa_bytes_by_position(inp) -> int:
    s = inp["spec"]
    B, N, nkv, D = s.B, s.N, s.nkv, s.D
    g = N // nkv
    eb = 1 if s.kv_dtype == "i8" else 2
    S = inp["S"]
    m = inp["mask"]
    pads = inp["kv_padding_size"]
    total = 2 * B * N * D * 2                      # q in, output out (16-bit)
    his = []
    for b in range(B):
        L = int(inp["lengths_drawn"][b])
        lo, hi = 0, L
        if pads is not None and inp["actual_seq_lengths"] is not None:
            p = max(int(np.broadcast_to(np.asarray(pads), (B,))[b]), 0)
            lo, hi = S - p - L, S - p
            if lo < 0 or hi < 0:                   # the window leaves the cache: nothing is read
                lo = hi = 0
        his.append(hi)
        for t in range(lo, hi):
            for j in range(nkv):
                need = True
                if m is not None:
                    mb = b if m.shape[0] == B else 0
                    heads = range(j * g, (j + 1) * g) if m.shape[1] == N else [0]
                    need = any(not bool(m[mb, h, 0, t]) for h in heads)
                if need:
                    total += 2 * D * eb            # its K row and its V row
            if m is not None:
                total += m.shape[1]                # one mask byte per mask head
        if s.paged:
            total += math.ceil((hi - lo) / s.block_size) * 4
        if inp.get("pse") is not None and inp["pse"].shape[0] == B:
            total += (hi - lo) * N * 2
    if inp.get("pse") is not None and inp["pse"].shape[0] != B:
        total += max(his, default=0) * N * 2       # one bias shared by every batch
    if inp["aq_scale"] is not None:
        total += 2 * inp["aq_scale"].numel() * 2   # scale and offset, K and V
    return total


def sfa_bytes_by_position(inp) -> int:
    s = inp["spec"]
    R = inp["q_rows"]
    idx = inp["sparse_indices"].numpy().reshape(R, -1)
    lkv, lq = inp["lkv_counts"], inp["lq_counts"]
    row_bytes = (s.D + s.DR + (0 if s.value_aliases_key else s.D)) * 2
    total = R * s.QN * (s.D + s.DR) * 2 + R * s.QN * s.D * 2      # q, q_rope; output
    total += idx.size * 4
    for name in ("actual_seq_lengths_kv", "actual_seq_lengths_query"):
        if inp[name] is not None:
            total += inp[name].numel() * 4
    for r in range(R):
        b, pos_in_batch = int(inp["row_batch"][r]), int(inp["row_pos"][r])
        limit = int(lkv[b])
        if s.sparse_mode == 3:
            limit = min(limit, int(lkv[b]) - int(lq[b]) + pos_in_batch + 1)
        if pos_in_batch >= int(lq[b]):
            limit = 0                              # a padding query row attends nothing
        for e in range(idx.shape[1]):
            first = int(idx[r, e])
            if first < 0:
                continue
            n = sum(1 for u in range(s.sparse_block_size) if first * s.sparse_block_size + u < limit)
            total += n * row_bytes
            if n and s.layout_kv == "PA_BSND":
                total += 4
    return total


IFA_CASES = {
    # per-head mask over a group of 4 heads, left padding with one window pushed off the cache
    "mask_per_head_left_pad": IfaSpec("bytes_mask", 9701, "bf16", "bf16", B=4, N=8, Nkv=2, D=64, layout="BNSD",
                                      S=96, lengths=[40, 96, 7, 60], pads=[10, 0, 95, 20], mask="bool",
                                      mask_p=0.6, mask_heads=8),
    # one mask head shared by every batch
    "mask_shared": IfaSpec("bytes_mask1", 9702, "f16", "f16", B=3, N=4, Nkv=4, D=32, layout="BSH", S=80,
                           lengths=[80, 1, 33], mask="u8", mask_p=0.5, mask_heads=1, mask_batch=1),
    # paged, int8 with per-channel antiquant
    "paged_int8": IfaSpec("bytes_paged", 9703, "f16", "i8", B=3, N=8, Nkv=2, D=64, layout="BNSD", S=300,
                          lengths=[1, 129, 300], paged=True, block_size=32, antiquant="per_channel"),
    # a per-batch positional bias and a shared one
    "bias_per_batch": IfaSpec("bytes_pse", 9704, "bf16", "bf16", B=3, N=4, Nkv=2, D=64, layout="BNSD", S=70,
                              lengths=[70, 5, 0], pse=True),
    "bias_shared": IfaSpec("bytes_pse1", 9705, "bf16", "bf16", B=3, N=4, Nkv=2, D=64, layout="BNSD", S=70,
                           lengths=[12, 50, 3], pse=True, pse_batch=1),
}


@pytest.mark.parametrize("case", sorted(IFA_CASES))
def test_ifa_bytes_match_a_position_by_position_count(case):
    inp = make_ifa(IFA_CASES[case])
    got = bench.algorithmic_bytes(inp)
    assert got["total"] == ifa_bytes_by_position(inp)
    assert got["kv"] <= got["total"] <= got["streamed"]


def small_sfa(cfg_id, **kw):
    d = dict(B=3, QN=16, num_blocks=96, max_blocks=32, block_size=64, lkv_range=(100, 2000), sparse_size=96,
             tail_range=(1, 20))
    d.update(kw)
    return SfaSpec("bytes_sfa", cfg_id, **d)


SFA_CASES = {
    "one_row_per_batch": small_sfa(9711),
    # causal query rows with a padding row, and block-wise entries whose block crosses the causal limit
    "causal_block_wise": small_sfa(9712, QS=3, lq=[3, 1, 2], sparse_mode=3, past_limit=True,
                                   sparse_block_size=8, sparse_size=24),
    "value_is_key_tnd": small_sfa(9713, layout_q="TND", layout_kv="TND", lq=[2, 1, 3], sparse_mode=3,
                                  value_aliases_key=True),
    "bsnd_cache_all_rows": small_sfa(9714, layout_kv="BSND", kv_seq=2000, sparse_block_size=4, sparse_size=40),
}


@pytest.mark.parametrize("case", sorted(SFA_CASES))
def test_sfa_bytes_match_a_position_by_position_count(case):
    inp = make_sfa(SFA_CASES[case])
    got = bench.algorithmic_bytes(inp)
    assert got["total"] == sfa_bytes_by_position(inp)


def test_sfa_count_sees_partly_attended_blocks():
    """The block-wise causal case above holds blocks cut by the limit, so a
    count of whole blocks (rows / sparse_block_size) would differ."""
    inp = make_sfa(SFA_CASES["causal_block_wise"])
    rows, blocks = bench.sfa_attended(inp)
    assert rows % inp["spec"].sparse_block_size != 0 or blocks * inp["spec"].sparse_block_size != rows
