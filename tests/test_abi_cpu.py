"""The C ABI without a GPU: symbols, status strings and argument validation.

Validation runs before any HIP call, so every rejected call below returns its
status code on a machine without a GPU.  Pointers are non-null dummies that
the library must never dereference on these paths.
"""
import ctypes
import os
import re

import pytest

from decode_attention_kv_06_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)


def header_functions():
    """Every function declared by the headers under include/."""
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*\**\s*(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"ifa_decode", "ifa_decode_paged", "sfa_decode_mla", "ifa_decode_workspace_size",
            "ifa_decode_paged_workspace_size", "sfa_decode_mla_workspace_size", "ifa_status_string",
            "ifa_abi_version", "ifa_read_probe", "sfa_decode_mla_plan"} <= set(names)
    L = bd.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert bd.lib().ifa_abi_version() >= 1
    for code in (0, 161001, 161002, 361001):
        assert bd.status_string(code).startswith("IFA_")
    assert bd.status_string(42) == "unknown status"


def test_struct_sizes_match_the_c_compiler(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include "ifa_decode.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu\\n", sizeof(ifa_decode_args), sizeof(ifa_paged_args),'
                   ' sizeof(sfa_mla_args)); return 0;}\n')
    exe = tmp_path / "sz"
    import subprocess
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    a, b, c = map(int, subprocess.check_output([str(exe)]).split())
    assert (a, b, c) == (ctypes.sizeof(bd.IfaDecodeArgs), ctypes.sizeof(bd.IfaPagedArgs),
                         ctypes.sizeof(bd.SfaMlaArgs))


# ---------------------------------------------------------------- dense IFA
def dense_args(**kw):
    a = bd.IfaDecodeArgs()
    a.struct_size = ctypes.sizeof(bd.IfaDecodeArgs)
    a.query = a.key = a.value = a.attention_out = FAKE
    a.dtype_q = a.dtype_kv = a.dtype_out = bd.DT_BF16
    a.input_layout = b"BSH"
    a.batch, a.num_heads, a.num_key_value_heads, a.head_dim, a.kv_seq_len = 2, 8, 2, 128, 64
    a.scale_value = 0.1
    a.split_tokens = 64          # forced split: the size query needs no device
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def ws_size(fn, a):
    n = ctypes.c_size_t(0)
    return getattr(bd.lib(), fn)(ctypes.byref(a), ctypes.byref(n)), n.value


def test_dense_valid_call_sizes_workspace_without_a_device():
    rc, n = ws_size("ifa_decode_workspace_size", dense_args())
    assert rc == 0
    # g = 4 -> one head group of G = 4; 2 rows (KV heads) per batch of 64 positions and
    # pieces of 64 -> a row meets at most 2 pieces: 2 batches x 2 rows x 2 slots = 8 slots,
    # each G x D floats of sums plus G x 2 floats of (max, sum), both rounded up to 256 B
    assert n == 8 * 4 * 128 * 4 + 256


@pytest.mark.parametrize("D,Dc", [(8, 64), (40, 64), (96, 128), (136, 256), (200, 256), (264, 512), (504, 512)])
def test_head_dims_below_a_compiled_size_run_on_it(D, Dc):
    # any head dim up to 512 in whole 16-byte lanes is accepted; its partial
    # states take the compiled size's row length, so the workspace matches it
    rc, n = ws_size("ifa_decode_workspace_size", dense_args(head_dim=D))
    rc_c, n_c = ws_size("ifa_decode_workspace_size", dense_args(head_dim=Dc))
    assert rc == 0 and rc_c == 0
    assert n == n_c


LENS = (ctypes.c_int64 * 2)(10, 64)
BAD_LENS = (ctypes.c_int64 * 2)(10, 65)
PADS1 = (ctypes.c_int64 * 1)(3)


@pytest.mark.parametrize("kw,code", [
    (dict(query=None), 161001),
    (dict(key=None), 161001),
    (dict(value=None), 161001),
    (dict(attention_out=None), 161001),
    (dict(dtype_q=bd.DT_I8), 161002),
    (dict(dtype_out=bd.DT_F16), 161002),
    (dict(dtype_kv=bd.DT_F16), 161002),
    (dict(input_layout=b"BNS"), 161002),
    (dict(batch=0), 161002),
    (dict(batch=65537), 161002),
    (dict(num_heads=257), 161002),
    (dict(num_key_value_heads=3), 161002),
    (dict(num_key_value_heads=9), 161002),
    (dict(head_dim=100), 161002),                  # not whole 16-byte lanes
    (dict(head_dim=520), 161002),
    (dict(head_dim=4), 161002),
    (dict(head_dim=0), 161002),
    (dict(kv_seq_len=0), 161002),
    (dict(scale_value=float("nan")), 161002),
    (dict(actual_seq_lengths=ctypes.cast(BAD_LENS, ctypes.c_void_p)), 161002),
    (dict(kv_padding_size=ctypes.cast(PADS1, ctypes.c_void_p), kv_padding_size_count=3), 161002),
    (dict(pse_shift=FAKE), 161002),                               # pse_batch 0
    (dict(pse_shift=FAKE, pse_batch=3, pse_seq=64), 161002),      # pse_batch not in {1, B}
    (dict(pse_shift=FAKE, pse_batch=2, pse_seq=63), 161002),      # shorter than the attended range
    (dict(pse_shift=FAKE, pse_batch=1, pse_seq=64, struct_size=bd.IfaDecodeArgs.pse_batch.offset), 161002),
    (dict(atten_mask=FAKE, dtype_mask=bd.DT_F16, mask_batch=2, mask_heads=1, mask_seq=64), 161002),
    (dict(atten_mask=FAKE, dtype_mask=bd.DT_BOOL, mask_batch=3, mask_heads=1, mask_seq=64), 161002),
    (dict(atten_mask=FAKE, dtype_mask=bd.DT_BOOL, mask_batch=2, mask_heads=4, mask_seq=64), 161002),
    (dict(atten_mask=FAKE, dtype_mask=bd.DT_BOOL, mask_batch=2, mask_heads=1, mask_seq=63), 161002),
    (dict(antiquant_scale=FAKE, antiquant_offset=FAKE, antiquant_mode=2), 161002),
    (dict(dtype_kv=bd.DT_I8, antiquant_mode=0), 161002),
    (dict(dtype_kv=bd.DT_I8, antiquant_mode=2), 161001),
    (dict(split_tokens=24), 161002),
    (dict(struct_size=8), 161002),
])
def test_dense_rejections(kw, code):
    assert ws_size("ifa_decode_workspace_size", dense_args(**kw))[0] == code
    # the run call validates identically and launches nothing
    assert bd.lib().ifa_decode(ctypes.byref(dense_args(**kw)), None, 0, None) == code


def test_dense_null_args_and_size_pointer():
    assert bd.lib().ifa_decode_workspace_size(None, None) == 161001
    n = ctypes.c_size_t()
    assert bd.lib().ifa_decode_workspace_size(None, ctypes.byref(n)) == 161001


def test_dense_left_padding_window_rules_accept():
    a = dense_args(actual_seq_lengths=ctypes.cast(LENS, ctypes.c_void_p),
                   kv_padding_size=ctypes.cast(PADS1, ctypes.c_void_p), kv_padding_size_count=1)
    # batch 1: start = 64 - 3 - 64 < 0 -> zero row, no slots; batch 0: [51, 61) -> 2 rows x 2 slots
    rc, n = ws_size("ifa_decode_workspace_size", a)
    assert rc == 0 and n == 4 * 4 * 128 * 4 + 256


def test_dense_workspace_too_small_is_rejected():
    a = dense_args()
    assert bd.lib().ifa_decode(ctypes.byref(a), FAKE, 16, None) == 161002


# ---------------------------------------------------------------- paged IFA
PLENS = (ctypes.c_int64 * 2)(100, 64)


def paged_args(**kw):
    a = bd.IfaPagedArgs()
    a.struct_size = ctypes.sizeof(bd.IfaPagedArgs)
    a.query = a.key_cache = a.value_cache = a.attention_out = a.block_table = FAKE
    a.dtype_q = a.dtype_kv = a.dtype_out = bd.DT_F16
    a.input_layout = b"BNSD"
    a.batch, a.num_heads, a.num_key_value_heads, a.head_dim = 2, 4, 2, 64
    a.scale_value = 0.125
    a.actual_seq_lengths = ctypes.cast(PLENS, ctypes.c_void_p)
    a.max_blocks_per_seq, a.block_size, a.num_blocks, a.kv_cache_layout = 4, 32, 8, 0
    a.split_tokens = 32
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_paged_valid_call_sizes_workspace():
    rc, n = ws_size("ifa_decode_paged_workspace_size", paged_args())
    assert rc == 0
    # g = 2 -> G = 2; lengths 100 and 64 with pieces of 32 -> 5 and 3 slots per row, 2 rows each
    assert n == (2 * 5 + 2 * 3) * 2 * 64 * 4 + 256


@pytest.mark.parametrize("kw,code", [
    (dict(block_table=None), 161001),
    (dict(actual_seq_lengths=None), 161001),
    (dict(key_cache=None), 161001),
    (dict(block_size=8), 161002),
    (dict(block_size=24), 161002),
    (dict(block_size=528), 161002),
    (dict(dtype_kv=bd.DT_I8, antiquant_scale=FAKE, antiquant_offset=FAKE, antiquant_mode=1, block_size=48), 161002),
    (dict(max_blocks_per_seq=3), 161002),          # 100 positions need 4 blocks of 32
    (dict(num_blocks=5), 161002),                  # 4 + 2 blocks needed
    (dict(kv_cache_layout=2), 161002),
    (dict(input_layout=b"BSH"), 161002),           # BSH pairs only with (blocknum, blocksize, H)
])
def test_paged_rejections(kw, code):
    assert ws_size("ifa_decode_paged_workspace_size", paged_args(**kw))[0] == code


def test_paged_bsh_with_hidden_layout_is_accepted():
    assert ws_size("ifa_decode_paged_workspace_size", paged_args(input_layout=b"BSH", kv_cache_layout=1))[0] == 0


def test_paged_int8_with_32_aligned_blocks_is_accepted():
    a = paged_args(dtype_kv=bd.DT_I8, antiquant_scale=FAKE, antiquant_offset=FAKE, antiquant_mode=2, block_size=64,
                   max_blocks_per_seq=2, num_blocks=4)
    assert ws_size("ifa_decode_paged_workspace_size", a)[0] == 0


# ---------------------------------------------------------------- SFA
def sfa_args(**kw):
    a = bd.SfaMlaArgs()
    a.struct_size = ctypes.sizeof(bd.SfaMlaArgs)
    a.query = a.query_rope = a.key = a.key_rope = a.value = a.sparse_indices = a.block_table = FAKE
    a.actual_seq_lengths_kv = a.attention_out = FAKE
    a.dtype = bd.DT_BF16
    a.batch, a.q_seq, a.q_heads, a.kv_heads, a.head_dim, a.rope_dim = 2, 1, 16, 1, 512, 64
    a.sparse_size, a.block_size, a.num_blocks, a.max_blocks = 100, 64, 10, 5
    a.scale_value = 0.04
    a.sparse_block_size, a.sparse_mode, a.attention_mode = 1, 0, 2
    a.layout_query, a.layout_kv = b"BSND", b"PA_BSND"
    a.split_hint = 2
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_sfa_valid_size_query():
    assert ws_size("sfa_decode_mla_workspace_size", sfa_args())[0] == 0


@pytest.mark.parametrize("kw,code", [
    (dict(query=None), 161001),
    (dict(query_rope=None), 161001),
    (dict(key_rope=None), 161001),
    (dict(sparse_indices=None), 161001),
    (dict(block_table=None), 161001),
    (dict(actual_seq_lengths_kv=None), 161001),
    (dict(attention_out=None), 161001),
    (dict(dtype=bd.DT_I8), 161002),
    (dict(kv_heads=2), 161002),
    (dict(head_dim=256), 161002),
    (dict(rope_dim=32), 161002),
    (dict(q_heads=129), 161002),
    (dict(q_heads=0), 161002),
    (dict(q_seq=0), 161002),
    (dict(q_seq=65537), 161002),
    (dict(sparse_size=0), 161002),
    (dict(block_size=24), 161002),
    (dict(block_size=1040), 161002),
    (dict(sparse_block_size=3), 161002),
    (dict(sparse_block_size=256), 161002),
    (dict(sparse_block_size=128), 161002),                 # does not divide block_size 64
    (dict(sparse_mode=1), 161002),
    (dict(attention_mode=1), 161002),
    (dict(layout_query=b"TND"), 161001),                   # needs the query prefix sums
    (dict(layout_query=b"TND", actual_seq_lengths_query=FAKE, q_tokens=0), 161002),
    (dict(layout_query=b"BNSD"), 161002),
    (dict(layout_kv=b"BSND"), 161002),                     # kv_seq 0
    (dict(layout_kv=b"TND", kv_tokens=0), 161002),
    (dict(layout_kv=b"TND", kv_tokens=10, actual_seq_lengths_kv=None), 161001),
    (dict(layout_kv=b"PA_BNSD"), 161002),
    (dict(layout_kv=b"BSND", kv_seq=100, struct_size=bd.SfaMlaArgs.q_tokens.offset), 161002),
    (dict(struct_size=bd.SfaMlaArgs.q_tokens.offset - 8), 161002),
    # return_softmax_lse (README: not with a PA_BSND cache; both outputs required; none without the flag)
    (dict(return_softmax_lse=1, softmax_max_out=FAKE, softmax_sum_out=FAKE), 161002),
    (dict(layout_kv=b"BSND", kv_seq=100, return_softmax_lse=1, softmax_max_out=FAKE), 161001),
    (dict(layout_kv=b"BSND", kv_seq=100, softmax_max_out=FAKE, softmax_sum_out=FAKE), 161002),
    (dict(layout_kv=b"BSND", kv_seq=100, return_softmax_lse=2, softmax_max_out=FAKE, softmax_sum_out=FAKE), 161002),
    (dict(scale_value=float("inf")), 161002),
])
def test_sfa_rejections(kw, code):
    assert ws_size("sfa_decode_mla_workspace_size", sfa_args(**kw))[0] == code


def test_sfa_mode_three_is_accepted():
    assert ws_size("sfa_decode_mla_workspace_size", sfa_args(sparse_mode=3))[0] == 0


def test_sfa_workspace_holds_chunk_outputs_in_input_dtype():
    # sparse_size 100 in 2 chunks of 64 entries: 2 batches x 2 chunks x 16 heads rows,
    # 512 two-byte values each, then (m, l) as two floats per row
    rc, n = ws_size("sfa_decode_mla_workspace_size", sfa_args(split_hint=2))
    assert rc == 0 and n == 2 * 2 * 16 * 512 * 2 + 2 * 2 * 16 * 2 * 4
    rc, n = ws_size("sfa_decode_mla_workspace_size", sfa_args(split_hint=1))
    assert rc == 0 and n == 0


@pytest.mark.parametrize("kw", [
    dict(pse_shift=FAKE, pse_batch=2, pse_seq=64),
    dict(pse_shift=FAKE, pse_batch=1, pse_seq=100),
    dict(pse_shift=FAKE, pse_batch=1, pse_seq=64, actual_seq_lengths=ctypes.cast(LENS, ctypes.c_void_p)),
    dict(struct_size=bd.IfaDecodeArgs.pse_batch.offset),           # a struct without the pse dims
    dict(pse_shift=FAKE, pse_batch=2, pse_seq=64, struct_size=bd.IfaDecodeArgs.key_list.offset),  # no lists
])
def test_dense_positional_bias_accepted(kw):
    assert ws_size("ifa_decode_workspace_size", dense_args(**kw))[0] == 0


def test_paged_positional_bias_checks():
    assert ws_size("ifa_decode_paged_workspace_size", paged_args(pse_shift=FAKE, pse_batch=2, pse_seq=100))[0] == 0
    # lengths (100, 64): logical positions up to 99 need a bias
    assert ws_size("ifa_decode_paged_workspace_size", paged_args(pse_shift=FAKE, pse_batch=2, pse_seq=99))[0] \
        == 161002
    assert ws_size("ifa_decode_paged_workspace_size", paged_args(pse_shift=FAKE, pse_batch=4, pse_seq=100))[0] \
        == 161002


@pytest.mark.parametrize("kw", [
    dict(q_seq=4, sparse_mode=3),
    dict(q_seq=4, sparse_mode=3, actual_seq_lengths_query=FAKE),
    dict(sparse_block_size=64),
    dict(layout_kv=b"BSND", kv_seq=100, block_table=None, actual_seq_lengths_kv=None),
    dict(layout_kv=b"TND", kv_tokens=1000, block_table=None),
    dict(layout_query=b"TND", actual_seq_lengths_query=FAKE, q_tokens=7),
    dict(struct_size=bd.SfaMlaArgs.q_tokens.offset),                  # a struct without the breadth fields
    dict(layout_kv=b"BSND", kv_seq=100, block_table=None, actual_seq_lengths_kv=None, return_softmax_lse=1,
         softmax_max_out=FAKE, softmax_sum_out=FAKE),                   # softmax max / sum outputs
    dict(struct_size=bd.SfaMlaArgs.softmax_max_out.offset, softmax_max_out=FAKE),   # fields invisible: ignored
])
def test_sfa_breadth_accepted(kw):
    assert ws_size("sfa_decode_mla_workspace_size", sfa_args(**kw))[0] == 0


def sfa_plan(a):
    pl = bd.SfaMlaPlan()
    rc = bd.lib().sfa_decode_mla_plan(ctypes.byref(a), ctypes.byref(pl))
    return rc, pl


def test_sfa_plan_reports_the_forced_split():
    # 100 entries in 2 chunks: 50 rounded up to the 32-row tile = 64 entries, so still 2 chunks;
    # 2 query rows x 2 chunks = 4 groups, rounded up to one round of 8 (XCDs) x 1 head block
    rc, pl = sfa_plan(sfa_args(split_hint=2))
    assert rc == 0 and (pl.chunks, pl.chunk_entries, pl.workgroups, pl.all_heads) == (2, 64, 8, 0)
    # 64 heads, 3 chunks asked: 34 entries rounded up to the tile = 64, so 2 chunks
    rc, pl = sfa_plan(sfa_args(split_hint=3, q_heads=64))
    assert rc == 0 and (pl.chunks, pl.chunk_entries, pl.workgroups, pl.all_heads) == (2, 64, 8, 0)
    # block-wise entries: 64 positions each, at most 512 rows = 8 entries a chunk
    rc, pl = sfa_plan(sfa_args(split_hint=2, sparse_block_size=64))
    assert rc == 0 and (pl.chunks, pl.chunk_entries) == (13, 8)


def test_sfa_plan_validates_like_the_size_query():
    assert sfa_plan(sfa_args(query=None))[0] == 161001
    assert sfa_plan(sfa_args(head_dim=256))[0] == 161002
    assert bd.lib().sfa_decode_mla_plan(ctypes.byref(sfa_args()), None) == 161001
    assert ctypes.sizeof(bd.SfaMlaPlan) == 16


def test_sfa_plan_needs_the_device_for_more_than_64_heads():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this case needs a machine without one")
    # the choice between 64-head and all-head workgroups reads the CU count
    assert sfa_plan(sfa_args(split_hint=2, q_heads=128))[0] == 361001
    assert sfa_plan(sfa_args(split_hint=0))[0] == 361001


def test_sfa_workspace_counts_query_rows_and_block_wise_chunks():
    # 2 batches x 3 query rows = 6 rows, 2 chunks each
    rc, n = ws_size("sfa_decode_mla_workspace_size", sfa_args(q_seq=3, split_hint=2))
    assert rc == 0 and n == 6 * 2 * 16 * 512 * 2 + 6 * 2 * 16 * 2 * 4
    # blocks of 64 positions: a chunk gathers at most 512 rows = 8 entries, so 100 entries take 13 chunks
    rc, n = ws_size("sfa_decode_mla_workspace_size", sfa_args(sparse_block_size=64, split_hint=2))
    assert rc == 0 and n == 2 * 13 * 16 * 512 * 2 + 2 * 13 * 16 * 2 * 4


SEQ2 = (ctypes.c_int64 * 2)(64, 40)
SEQ_SHORT = (ctypes.c_int64 * 2)(9, 64)


def list_args(**kw):
    base = dict(key=None, value=None, key_list=FAKE, value_list=FAKE,
                kv_list_seq_len=ctypes.cast(SEQ2, ctypes.c_void_p), kv_seq_len=0)
    base.update(kw)
    return dense_args(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(actual_seq_lengths=ctypes.cast(LENS, ctypes.c_void_p), kv_list_seq_len=ctypes.cast(SEQ_SHORT,
                                                                                             ctypes.c_void_p)), 161002),
    (dict(value_list=None), 161001),
    (dict(kv_list_seq_len=None), 161001),
    (dict(key=FAKE), 161002),                                   # a contiguous key beside the lists
    (dict(kv_padding_size=ctypes.cast(PADS1, ctypes.c_void_p), kv_padding_size_count=1), 161002),
    (dict(struct_size=bd.IfaDecodeArgs.key_list.offset), 161001),  # lists invisible: key is NULL
])
def test_dense_kv_lists_validation(kw, code):
    assert ws_size("ifa_decode_workspace_size", list_args(**kw))[0] == code


def test_dense_kv_lists_batch_limit():
    seq = (ctypes.c_int64 * 257)(*([64] * 257))
    a = list_args(batch=257, kv_list_seq_len=ctypes.cast(seq, ctypes.c_void_p))
    assert ws_size("ifa_decode_workspace_size", a)[0] == 161002


# ---------------------------------------------------------------- int8 output
@pytest.mark.parametrize("kw,code", [
    (dict(dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_count=1, dtype_quant=bd.DT_F32), 0),
    (dict(dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_offset2=FAKE, quant_count=8 * 128, dtype_quant=bd.DT_BF16), 0),
    (dict(dtype_out=bd.DT_I8), 161001),                                             # quantScale2 required
    (dict(dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_count=2 * 128, dtype_quant=bd.DT_F32), 161002),
    (dict(dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_count=1, dtype_quant=bd.DT_F16), 161002),
    (dict(dtype_q=bd.DT_F16, dtype_kv=bd.DT_F16, dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_count=1,
          dtype_quant=bd.DT_BF16), 161002),                                         # bf16 only with bf16 inputs
    (dict(quant_scale2=FAKE, quant_count=1, dtype_quant=bd.DT_F32), 161002),        # float output takes none
    (dict(dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_count=1, dtype_quant=bd.DT_F32,
          struct_size=bd.IfaDecodeArgs.quant_scale2.offset), 161001),               # fields invisible
])
def test_dense_int8_output_validation(kw, code):
    assert ws_size("ifa_decode_workspace_size", dense_args(**kw))[0] == code


def test_paged_int8_output_validation():
    ok = paged_args(dtype_out=bd.DT_I8, quant_scale2=FAKE, quant_count=4 * 64, dtype_quant=bd.DT_F32)
    assert ws_size("ifa_decode_paged_workspace_size", ok)[0] == 0
    assert ws_size("ifa_decode_paged_workspace_size", paged_args(dtype_out=bd.DT_I8))[0] == 161001


# ---------------------------------------------------------------- runtime failure
def test_run_without_a_device_returns_the_runtime_code():
    """V2 page, Return Value: a failure of the runtime underneath is 361001.
    On a machine with no GPU a valid call reaches the HIP runtime and fails
    there; with the planner choosing the split it stops at the device query,
    before any launch, and with a forced split at the launch itself."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this case needs a machine without one")
    L = bd.lib()
    ws = ctypes.c_void_p(0x2000)
    for split in (0, 64):
        assert L.ifa_decode(ctypes.byref(dense_args(split_tokens=split)), ws, 1 << 20, None) == 361001
        assert L.ifa_decode_paged(ctypes.byref(paged_args(split_tokens=split)), ws, 1 << 20, None) == 361001
    for split in (0, 2):
        assert L.sfa_decode_mla(ctypes.byref(sfa_args(split_hint=split)), ws, 1 << 26, None) == 361001


# ---------------------------------------------------------------- Python binding
def _cpu_ifa_tensors():
    import torch
    q = torch.zeros(2, 1, 8 * 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 64, 2 * 128, dtype=torch.bfloat16)
    return q, k, k.clone(), torch.empty_like(q)


def test_binding_rejects_host_tensors_before_calling_the_library():
    q, k, v, out = _cpu_ifa_tensors()
    with pytest.raises(ValueError, match="GPU tensor"):
        bd.ifa_decode_args(q, k, v, out, num_heads=8, num_key_value_heads=2, input_layout="BSH", scale_value=0.1)


def test_binding_rejects_strided_views_and_wide_index_tensors():
    import torch
    q, k, v, out = _cpu_ifa_tensors()
    mask = torch.zeros(1, 1, 1, 64, dtype=torch.bool).expand(2, 8, 1, 64)     # stride-0 view
    with pytest.raises(ValueError, match="contiguous"):
        bd.ifa_decode_args(q, k, v, out, num_heads=8, num_key_value_heads=2, input_layout="BSH", scale_value=0.1,
                           atten_mask=mask)
    with pytest.raises(ValueError, match="contiguous"):
        bd.ifa_decode_args(q, k[:, ::2], v[:, ::2], out, num_heads=8, num_key_value_heads=2, input_layout="BSH",
                           scale_value=0.1)
    qp = torch.zeros(2, 8, 1, 128, dtype=torch.bfloat16)
    cache = torch.zeros(4, 2, 32, 128, dtype=torch.bfloat16)
    bt64 = torch.zeros(2, 2, dtype=torch.int64)             # torch's default integer dtype
    with pytest.raises(ValueError, match="int32"):
        bd.ifa_paged_args(qp, cache, cache, torch.empty_like(qp), bt64, num_heads=8, num_key_value_heads=2,
                          scale_value=0.1, actual_seq_lengths=[10, 20])
    q5 = torch.zeros(1, 1, 4, 512, dtype=torch.bfloat16)
    qr = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    kc = torch.zeros(2, 16, 1, 512, dtype=torch.bfloat16)
    kr = torch.zeros(2, 16, 1, 64, dtype=torch.bfloat16)
    idx = torch.zeros(1, 1, 1, 8, dtype=torch.int32)
    bt = torch.zeros(1, 2, dtype=torch.int32)
    lkv = torch.full((1,), 20, dtype=torch.int32)
    for bad in ("sparse_indices", "block_table", "actual_seq_lengths_kv"):
        t = dict(sparse_indices=idx, block_table=bt, actual_seq_lengths_kv=lkv)
        t[bad] = t[bad].long()
        with pytest.raises(ValueError, match="int32"):
            bd.sfa_args(q5, qr, kc, kr, kc, t["sparse_indices"], t["block_table"], t["actual_seq_lengths_kv"],
                        torch.empty_like(q5), scale_value=0.04)


def test_binding_requires_the_scale():
    q, k, v, out = _cpu_ifa_tensors()
    with pytest.raises(TypeError):
        bd.ifa_decode_args(q, k, v, out, num_heads=8, num_key_value_heads=2, input_layout="BSH")


def test_read_probe_rejects_bad_arguments_without_a_device():
    L = bd.lib()
    L.ifa_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert L.ifa_read_probe(None, 1024, FAKE, None) == 161001
    assert L.ifa_read_probe(FAKE, 1024, None, None) == 161001
    assert L.ifa_read_probe(FAKE, 1000, FAKE, None) == 161002          # not a multiple of 16
    assert L.ifa_read_probe(FAKE, 0, FAKE, None) == 161002
    assert L.ifa_read_probe(ctypes.c_void_p(0x1008), 1024, FAKE, None) == 161002   # misaligned
