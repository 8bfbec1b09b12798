"""Pins for the fp64 oracle, each against something other than the oracle.

- exhaustive decoding of every fp16 / bf16 bit pattern against numpy / torch;
- torch's scaled_dot_product_attention in float64 (a library routine) on tiny
  inputs, with the operator's mask polarity inverted into SDPA's
  "True = attend" convention, GQA through SDPA's own enable_gqa, and the
  positional bias as SDPA's float attn_mask (added to the scaled scores);
- closed forms: constant V, a single valid position, scale 0, the zero rule
  of left padding, the V-offset shift of antiquant;
- the one worked call on the aclnnIncreFlashAttentionV2 page ("Example").
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from decode_attention_kv_06_amd.workloads import IfaSpec, SfaSpec, make_ifa, make_sfa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def to64(t):
    return t.to(torch.float64)


def dense_kv_bnsd(inp):
    """K, V of a dense-layout input as float64 [B, Nkv, S, D]."""
    s = inp["spec"]
    B, nkv, D, S = s.B, s.nkv, s.D, inp["S"]
    k, v = to64(inp["k"]), to64(inp["v"])
    if s.layout == "BNSD":
        return k.view(B, nkv, S, D), v.view(B, nkv, S, D)
    return (k.view(B, S, nkv, D).permute(0, 2, 1, 3).contiguous(),
            v.view(B, S, nkv, D).permute(0, 2, 1, 3).contiguous())


def attend_mask(inp):
    """bool [B, N, 1, S]: True where the operator attends to position s."""
    s = inp["spec"]
    B, N, S = s.B, s.N, inp["S"]
    m = torch.zeros(B, N, 1, S, dtype=torch.bool)
    L = inp["actual_seq_lengths"]
    pad = inp["kv_padding_size"]
    for b in range(B):
        Lb = S if L is None else int(L[b])
        lo, hi = 0, Lb
        if pad is not None and L is not None:
            p = max(0, int(pad[b]))
            lo, hi = S - p - Lb, S - p
            if lo < 0 or hi < 0:
                continue
        m[b, :, 0, lo:hi] = True
    if inp["mask"] is not None:
        mk = inp["mask"].to(torch.bool)
        m &= ~mk.expand(B, N, 1, mk.shape[-1])[..., :S]
    return m


def sdpa_ref(inp, k64=None, v64=None, scale=None):
    s = inp["spec"]
    q = to64(inp["q"]).reshape(s.B, s.N, 1, s.D)
    if k64 is None:
        k64, v64 = dense_kv_bnsd(inp)
    m = attend_mask(inp)
    attn = m
    if inp.get("pse") is not None:
        # SDPA adds a float attn_mask to the scaled scores: the bias, with
        # -inf where the operator does not attend
        S = m.shape[-1]
        attn = to64(inp["pse"]).expand(s.B, s.N, 1, inp["pse"].shape[-1])[..., :S].clone()
        attn[~m] = float("-inf")
    out = F.scaled_dot_product_attention(q, k64, v64, attn_mask=attn, scale=s.scale_value if scale is None else scale,
                                         enable_gqa=True)
    out = out.reshape(s.B, s.N, s.D)
    empty = ~m.any(dim=-1).reshape(s.B, s.N)
    out[empty] = 0.0
    return out.numpy()


# ------------------------------------------------------------ decoding ----
def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_decode_exhaustive():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(b) & 0xFFFF) for b in bits.tolist()])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------------ the page sample ----
def test_v2_page_sample_constant_value():
    g = json.load(open(os.path.join(GOLDEN, "ifa_v2_sample.json")))
    spec = IfaSpec("v2_sample", 900, "f16", "f16", B=g["B"], N=g["N"], Nkv=g["Nkv"], D=g["D"], layout=g["layout"],
                   S=g["S"], lengths=g["actual_seq_lengths"], scale=g["scale"], mask="i8", mask_p=0.0)
    inp = make_ifa(spec)
    inp["q"].fill_(g["q_value"])
    inp["k"].fill_(g["k_value"])
    inp["v"].fill_(g["v_value"])
    inp["mask"].fill_(g["mask_value"])
    out = oracle.ifa(inp)
    assert out.shape == (1, 2, 16)
    assert (out == g["expected_out_value"]).all()
    # The same call with the mask polarity flipped would see no position and
    # give the empty-set zero row, so this fixture also fixes the polarity.
    inp["mask"].fill_(1)
    assert (oracle.ifa(inp) == 0.0).all()


# ------------------------------------------------- library routine pins ----
@pytest.mark.parametrize("layout", ["BNSD", "BSH", "BSND"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,Nkv", [(4, 4), (6, 2), (8, 1), (4, 0)])
def test_ifa_matches_sdpa(layout, dtype, N, Nkv):
    spec = IfaSpec("pin", 901, dtype, dtype, B=3, N=N, Nkv=Nkv, D=16, layout=layout, S=37,
                   len_range=(1, 37), mask="u8", mask_p=0.3)
    inp = make_ifa(spec)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp), rtol=0, atol=1e-12)


@pytest.mark.parametrize("heads", [1, "N"])
def test_ifa_per_head_mask_and_shared_batch(heads):
    spec = IfaSpec("pin", 902, "bf16", "bf16", B=2, N=4, Nkv=2, D=8, layout="BNSD", S=20, len_range=(5, 20),
                   mask="bool", mask_p=0.4, mask_heads=4 if heads == "N" else 1, mask_batch=1)
    inp = make_ifa(spec)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp), rtol=0, atol=1e-12)


def test_ifa_no_lengths_means_full_cache():
    spec = IfaSpec("pin", 903, "f16", "f16", B=2, N=2, Nkv=1, D=8, S=11, no_lengths=True)
    inp = make_ifa(spec)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp), rtol=0, atol=1e-12)


def test_ifa_scale_and_peaky_query():
    spec = IfaSpec("pin", 904, "bf16", "bf16", B=2, N=4, Nkv=2, D=32, S=50, len_range=(10, 50), q_mult=8.0)
    inp = make_ifa(spec)
    for sc in (0.02, 1.0 / math.sqrt(32), 0.7):
        np.testing.assert_allclose(oracle.ifa(inp, scale=sc), sdpa_ref(inp, scale=sc), rtol=0, atol=1e-12)


# ------------------------------------------------------- closed forms ----
def test_single_valid_position_returns_that_row():
    spec = IfaSpec("pin", 905, "bf16", "bf16", B=2, N=2, Nkv=1, D=16, S=30, lengths=[30, 30], mask="bool")
    inp = make_ifa(spec)
    inp["mask"].fill_(True)
    keep = [7, 22]
    for b, s_ in enumerate(keep):
        inp["mask"][b, 0, 0, s_] = False
    out = oracle.ifa(inp)
    v = to64(inp["v"]).view(2, 1, 30, 16)
    for b, s_ in enumerate(keep):
        for h in range(2):
            assert (out[b, h] == v[b, 0, s_].numpy()).all()


def test_scale_zero_gives_mean_of_valid_rows():
    spec = IfaSpec("pin", 906, "f16", "f16", B=2, N=3, Nkv=3, D=8, S=25, lengths=[9, 25])
    inp = make_ifa(spec)
    out = oracle.ifa(inp, scale=0.0)
    v = to64(inp["v"]).view(2, 3, 25, 8)
    for b, L in enumerate([9, 25]):
        np.testing.assert_allclose(out[b], v[b, :, :L].mean(dim=1).numpy(), rtol=0, atol=1e-13)


def test_empty_length_gives_zero_row():
    spec = IfaSpec("pin", 907, "f16", "f16", B=2, N=2, Nkv=2, D=8, S=10, lengths=[0, 10])
    inp = make_ifa(spec)
    out = oracle.ifa(inp)
    assert (out[0] == 0).all() and np.abs(out[1]).sum() > 0


# ------------------------------------------------------- left padding ----
def test_left_padding_window_and_zero_rule():
    S = 40
    spec = IfaSpec("pin", 908, "bf16", "bf16", B=4, N=2, Nkv=1, D=8, S=S, lengths=[10, 30, 35, 20],
                   pads=[5, -3, 10, 25])
    inp = make_ifa(spec)
    out = oracle.ifa(inp)
    # batch 0: [25, 35); batch 1: pad<0 -> 0 -> [10, 40); batch 2: start = 40-10-35 < 0 -> zeros;
    # batch 3: start = 40-25-20 < 0 -> zeros.
    assert (out[2] == 0).all() and (out[3] == 0).all()
    np.testing.assert_allclose(out, sdpa_ref(inp), rtol=0, atol=1e-12)
    # A right-padded call on the window's slice gives the same rows.
    k64, v64 = dense_kv_bnsd(inp)
    for b, (lo, hi) in enumerate([(25, 35), (10, 40)]):
        q = to64(inp["q"]).view(4, 2, 1, 8)[b:b + 1]
        ref = F.scaled_dot_product_attention(q, k64[b:b + 1, :, lo:hi], v64[b:b + 1, :, lo:hi],
                                             scale=spec.scale_value, enable_gqa=True)
        np.testing.assert_allclose(out[b], ref.view(2, 8).numpy(), rtol=0, atol=1e-12)


def test_negative_padding_equals_zero_padding():
    base = dict(B=2, N=2, Nkv=2, D=8, S=16, lengths=[16, 7])
    a = make_ifa(IfaSpec("pin", 909, "f16", "f16", pads=[-5, -1], **base))
    b = make_ifa(IfaSpec("pin", 909, "f16", "f16", pads=[0, 0], **base))
    assert (oracle.ifa(a) == oracle.ifa(b)).all()


def test_padding_without_lengths_is_right_padding():
    a = make_ifa(IfaSpec("pin", 910, "f16", "f16", B=2, N=2, Nkv=2, D=8, S=16, no_lengths=True, pads=[4, 9]))
    b = make_ifa(IfaSpec("pin", 910, "f16", "f16", B=2, N=2, Nkv=2, D=8, S=16, no_lengths=True))
    assert (oracle.ifa(a) == oracle.ifa(b)).all()


# ------------------------------------------------------------- paging ----
@pytest.mark.parametrize("cache_layout", [0, 1])
@pytest.mark.parametrize("bs", [16, 48])
def test_paged_equals_dense_on_depaged_cache(cache_layout, bs):
    spec = IfaSpec("pin", 911, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, S=6 * bs, len_range=(1, 6 * bs),
                   paged=True, block_size=bs, max_blocks=6, num_blocks=20, cache_layout=cache_layout,
                   mask="bool", mask_p=0.2)
    inp = make_ifa(spec)
    B, nkv, D, mb = 3, 2, 16, 6
    bt = inp["block_table"].long()
    k, v = to64(inp["k"]), to64(inp["v"])
    if cache_layout == 1:
        k = k.view(-1, bs, nkv, D).permute(0, 2, 1, 3)
        v = v.view(-1, bs, nkv, D).permute(0, 2, 1, 3)
    # De-page: logical position s of batch b -> cache block bt[b, s // bs], row s % bs.
    kd = k[bt].permute(0, 2, 1, 3, 4).reshape(B, nkv, mb * bs, D)
    vd = v[bt].permute(0, 2, 1, 3, 4).reshape(B, nkv, mb * bs, D)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp, kd, vd), rtol=0, atol=1e-12)


def test_paged_block_permutation_invariance():
    spec = IfaSpec("pin", 912, "f16", "f16", B=2, N=2, Nkv=1, D=8, S=64, len_range=(20, 64), paged=True,
                   block_size=16, max_blocks=4, num_blocks=10)
    inp = make_ifa(spec)
    ref = oracle.ifa(inp)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(10))
    inv = torch.argsort(perm)
    inp2 = dict(inp)
    inp2["k"] = inp["k"][perm].contiguous()      # new block i holds old block perm[i]
    inp2["v"] = inp["v"][perm].contiguous()
    inp2["block_table"] = inv[inp["block_table"].long()].to(torch.int32).contiguous()
    assert (oracle.ifa(inp2) == ref).all()


# ----------------------------------------------------------- antiquant ----
@pytest.mark.parametrize("mode", ["per_channel", "per_tensor"])
@pytest.mark.parametrize("qdt", ["f16", "bf16"])
def test_antiquant_equals_float_attention_on_dequantised_cache(mode, qdt):
    spec = IfaSpec("pin", 913, qdt, "i8", B=2, N=4, Nkv=2, D=16, S=30, len_range=(5, 30), antiquant=mode)
    inp = make_ifa(spec)
    k64, v64 = dense_kv_bnsd(inp)
    sc, of = to64(inp["aq_scale"]), to64(inp["aq_offset"])
    if mode == "per_channel":
        ks, ko = sc[0].view(1, 2, 1, 16), of[0].view(1, 2, 1, 16)
        vs, vo = sc[1].view(1, 2, 1, 16), of[1].view(1, 2, 1, 16)
    else:
        ks, ko, vs, vo = sc[0], of[0], sc[1], of[1]
    kd, vd = (k64 + ko) * ks, (v64 + vo) * vs
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp, kd, vd), rtol=0, atol=1e-12)


def test_antiquant_value_offset_shift_and_key_offset_invariance():
    spec = IfaSpec("pin", 914, "f16", "i8", B=2, N=4, Nkv=2, D=16, S=30, len_range=(5, 30),
                   antiquant="per_channel")
    inp = make_ifa(spec)
    base = oracle.ifa(inp)
    inp0 = dict(inp)
    off0 = inp["aq_offset"].clone()
    off0[1] = 0                                   # V offset removed
    inp0["aq_offset"] = off0
    shifted = oracle.ifa(inp0)
    sV = to64(inp["aq_scale"][1]).view(2, 16)
    oV = to64(inp["aq_offset"][1]).view(2, 16)
    expect = (sV * oV).repeat_interleave(2, dim=0).numpy()   # heads 2j, 2j+1 read KV head j
    np.testing.assert_allclose(base - shifted, np.broadcast_to(expect, base.shape), rtol=0, atol=1e-12)
    inpk = dict(inp)
    offk = inp["aq_offset"].clone()
    offk[0] = 0                                   # K offset removed: a per-row constant in the scores
    inpk["aq_offset"] = offk
    np.testing.assert_allclose(oracle.ifa(inpk), base, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- SFA ----
def _sfa_small(**kw):
    d = dict(B=2, QN=4, D=32, DR=8, block_size=16, num_blocks=40, max_blocks=20, lkv=[200, 317],
             sparse_size=50, n_valid=[40, 50])
    d.update(kw)
    return SfaSpec("pin", 915, **d)


def _sfa_gather_ref(inp):
    """SDPA over the gathered rows (576-style concatenated score dims)."""
    s = inp["spec"]
    out = np.zeros((s.B, s.QN, s.D))
    bt = inp["block_table"].long()
    key = to64(inp["key"]).view(-1, s.D)
    kr = to64(inp["key_rope"]).view(-1, s.DR)
    val = to64(inp["value"]).view(-1, s.D)
    for b in range(s.B):
        idx = inp["sparse_indices"][b, 0, 0].long()
        idx = idx[(idx >= 0) & (idx < int(inp["actual_seq_lengths_kv"][b]))]
        if len(idx) == 0:
            continue
        rows = bt[b, idx // s.block_size] * s.block_size + idx % s.block_size
        kk = torch.cat([key[rows], kr[rows]], dim=1)[None, None]
        vv = val[rows][None, None]
        qq = torch.cat([to64(inp["q"][b, 0]), to64(inp["q_rope"][b, 0])], dim=1)[None, :, None]
        o = F.scaled_dot_product_attention(qq, kk.expand(1, s.QN, -1, -1), vv.expand(1, s.QN, -1, -1),
                                           scale=s.scale_value)
        out[b] = o.view(s.QN, s.D).numpy()
    return out


def test_sfa_matches_sdpa_on_gathered_rows():
    inp = make_sfa(_sfa_small())
    np.testing.assert_allclose(oracle.sfa(inp), _sfa_gather_ref(inp), rtol=0, atol=1e-12)


def test_sfa_arange_indices_equal_dense_mqa_on_prefix():
    spec = _sfa_small(n_valid=[30, 30])
    inp = make_sfa(spec)
    for b in range(2):
        inp["sparse_indices"][b, 0, 0, :30] = torch.arange(30, dtype=torch.int32)
    out = oracle.sfa(inp)
    bt = inp["block_table"].long()
    for b in range(2):
        pos = torch.arange(30)
        rows = bt[b, pos // 16] * 16 + pos % 16
        kk = torch.cat([to64(inp["key"]).view(-1, 32)[rows], to64(inp["key_rope"]).view(-1, 8)[rows]], 1)
        vv = to64(inp["value"]).view(-1, 32)[rows]
        qq = torch.cat([to64(inp["q"][b, 0]), to64(inp["q_rope"][b, 0])], 1)
        ref = F.scaled_dot_product_attention(qq[None, :, None], kk[None, None].expand(1, 4, -1, -1),
                                             vv[None, None].expand(1, 4, -1, -1), scale=spec.scale_value)
        np.testing.assert_allclose(out[b], ref.view(4, 32).numpy(), rtol=0, atol=1e-12)


def test_sfa_permuting_valid_indices_and_single_and_empty():
    inp = make_sfa(_sfa_small())
    ref = oracle.sfa(inp)
    inp2 = dict(inp)
    idx = inp["sparse_indices"].clone()
    idx[0, 0, 0, :40] = idx[0, 0, 0, :40][torch.from_numpy(np.random.default_rng(1).permutation(40))]
    inp2["sparse_indices"] = idx
    np.testing.assert_allclose(oracle.sfa(inp2), ref, rtol=0, atol=1e-13)
    # one valid index -> that value row exactly; none valid -> zero row
    idx = torch.full_like(inp["sparse_indices"], -1)
    idx[0, 0, 0, 0] = 123
    inp2["sparse_indices"] = idx
    out = oracle.sfa(inp2)
    row = int(inp["block_table"][0, 123 // 16]) * 16 + 123 % 16
    assert (out[0] == to64(inp["value"]).view(-1, 32)[row].numpy()[None]).all()
    assert (out[1] == 0).all()


def test_sfa_out_of_range_entries_are_ignored():
    inp = make_sfa(_sfa_small(n_valid=[40, 50]))
    ref = oracle.sfa(inp)
    inp2 = dict(inp)
    idx = inp["sparse_indices"].clone()
    idx[0, 0, 0, 40:] = 200          # == lkv[0]: out of range, so invalid
    idx[0, 0, 0, 45] = 10 ** 6
    inp2["sparse_indices"] = idx
    np.testing.assert_allclose(oracle.sfa(inp2), ref, rtol=0, atol=0)


# ------------------------------------------------------- positional bias ----
@pytest.mark.parametrize("layout", ["BNSD", "BSH"])
@pytest.mark.parametrize("pse_batch", [0, 1])
def test_pse_matches_sdpa_float_bias(layout, pse_batch):
    spec = IfaSpec("pin", 930, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, layout=layout, S=40, len_range=(1, 40),
                   mask="u8", mask_p=0.2, pse=True, pse_batch=pse_batch, pse_scale=2.0)
    inp = make_ifa(spec)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp), rtol=0, atol=1e-12)


def test_pse_with_left_padding_uses_physical_positions():
    spec = IfaSpec("pin", 931, "f16", "f16", B=3, N=2, Nkv=1, D=8, layout="BNSD", S=48, len_range=(4, 30),
                   pad_off=(0, 10), pse=True)
    inp = make_ifa(spec)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp), rtol=0, atol=1e-12)


def test_pse_zero_and_per_row_constant_change_nothing():
    spec = IfaSpec("pin", 932, "bf16", "bf16", B=2, N=4, Nkv=2, D=16, S=33, len_range=(3, 33), pse=True)
    inp = make_ifa(spec)
    base = dict(inp)
    base["pse"] = None
    ref = oracle.ifa(base)
    zero = dict(inp)
    zero["pse"] = torch.zeros_like(inp["pse"])
    assert (oracle.ifa(zero) == ref).all()
    const = dict(inp)
    c = torch.arange(inp["pse"].shape[0] * inp["pse"].shape[1], dtype=torch.float64).reshape(
        inp["pse"].shape[0], inp["pse"].shape[1], 1, 1) * 0.75 - 3.0     # exact in bf16
    const["pse"] = c.expand_as(inp["pse"]).to(inp["pse"].dtype).contiguous()
    np.testing.assert_allclose(oracle.ifa(const), ref, rtol=0, atol=1e-12)


def test_pse_minus_infinity_equals_masking():
    spec = IfaSpec("pin", 933, "f16", "f16", B=2, N=2, Nkv=2, D=8, S=30, len_range=(10, 30), mask="bool",
                   mask_p=0.3, mask_heads=2, pse=True)
    inp = make_ifa(spec)
    m = inp["mask"].to(torch.bool)                    # (B, N, 1, S): True = excluded
    as_bias = dict(inp)
    as_bias["mask"] = None
    as_bias["pse"] = torch.where(m, torch.tensor(float("-inf"), dtype=inp["pse"].dtype), inp["pse"]).contiguous()
    np.testing.assert_allclose(oracle.ifa(as_bias), oracle.ifa(inp), rtol=0, atol=1e-12)


@pytest.mark.parametrize("cache_layout", [0, 1])
def test_paged_pse_uses_logical_positions(cache_layout):
    bs = 16
    spec = IfaSpec("pin", 934, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, S=6 * bs, len_range=(1, 6 * bs),
                   paged=True, block_size=bs, max_blocks=6, num_blocks=20, cache_layout=cache_layout, pse=True)
    inp = make_ifa(spec)
    B, nkv, D, mb = 3, 2, 16, 6
    bt = inp["block_table"].long()
    k, v = to64(inp["k"]), to64(inp["v"])
    if cache_layout == 1:
        k = k.view(-1, bs, nkv, D).permute(0, 2, 1, 3)
        v = v.view(-1, bs, nkv, D).permute(0, 2, 1, 3)
    kd = k[bt].permute(0, 2, 1, 3, 4).reshape(B, nkv, mb * bs, D)
    vd = v[bt].permute(0, 2, 1, 3, 4).reshape(B, nkv, mb * bs, D)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp, kd, vd), rtol=0, atol=1e-12)


def test_pse_shorter_than_attended_range_is_rejected():
    spec = IfaSpec("pin", 936, "bf16", "bf16", B=2, N=2, Nkv=2, D=8, S=24, len_range=(24, 24), pse=True)
    inp = make_ifa(spec)
    short = dict(inp)
    short["pse"] = inp["pse"][..., :20].contiguous()
    with pytest.raises(ValueError):
        oracle.ifa(short)


def test_mask_shorter_than_the_window_is_rejected():
    # the mask must cover every attended position (V2 page, attenMask); a
    # shorter one is an input error, never a read past its end
    spec = IfaSpec("pin", 938, "bf16", "bf16", B=2, N=2, Nkv=1, D=8, S=24, len_range=(24, 24), mask="u8",
                   mask_p=0.1)
    inp = make_ifa(spec)
    short = dict(inp)
    short["mask"] = inp["mask"][..., :20].contiguous()
    with pytest.raises(ValueError):
        oracle.ifa(short)
    # a mask that stops exactly at the window's end is fine
    lens = dict(inp)
    lens["actual_seq_lengths"] = np.asarray([20, 13], dtype=np.int64)
    lens["mask"] = short["mask"]
    assert np.isfinite(oracle.ifa(lens)).all()


def test_negative_length_and_length_past_the_block_table_are_rejected():
    # V2 page, actualSeqLengths: a length lies in [0, S]; README page
    # attention: the block table covers every attended position
    spec = IfaSpec("pin", 939, "f16", "f16", B=2, N=2, Nkv=1, D=8, S=30, len_range=(5, 20))
    inp = make_ifa(spec)
    neg = dict(inp)
    neg["actual_seq_lengths"] = np.asarray([-1, 5], dtype=np.int64)
    with pytest.raises(ValueError):
        oracle.ifa(neg)
    spec = IfaSpec("pin", 939, "bf16", "bf16", B=2, N=2, Nkv=1, D=8, S=64, len_range=(10, 40), paged=True,
                   block_size=16, max_blocks=3, num_blocks=8)
    inp = make_ifa(spec)
    far = dict(inp)
    far["actual_seq_lengths"] = np.asarray([49, 10], dtype=np.int64)     # 3 blocks of 16 reach 48
    with pytest.raises(ValueError):
        oracle.ifa(far)


def test_bias_of_minus_infinity_everywhere_is_an_empty_set():
    spec = IfaSpec("pin", 937, "f16", "f16", B=2, N=2, Nkv=1, D=8, S=20, len_range=(5, 20), pse=True)
    inp = make_ifa(spec)
    allinf = dict(inp)
    p = inp["pse"].clone()
    p[0] = float("-inf")
    allinf["pse"] = p
    out = oracle.ifa(allinf)
    assert (out[0] == 0).all() and np.isfinite(out).all()
    np.testing.assert_allclose(out[1], oracle.ifa(inp)[1], rtol=0, atol=0)


# ------------------------------------------------------- per-batch lists ----
@pytest.mark.parametrize("layout", ["BSH", "BNSD", "BSND"])
def test_kv_lists_equal_the_padded_cache(layout):
    spec = IfaSpec("pin", 940, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, layout=layout, S=50, len_range=(1, 40),
                   kv_list=True, mask="u8", mask_p=0.2, pse=True)
    inp = make_ifa(spec)
    assert [t.shape[1 if layout != "BNSD" else 2] for t in inp["k_list"]] == list(inp["list_seq"])
    padded = dict(inp)
    padded["k_list"] = None
    np.testing.assert_allclose(oracle.ifa(inp), oracle.ifa(padded), rtol=0, atol=0)
    np.testing.assert_allclose(oracle.ifa(inp), sdpa_ref(inp), rtol=0, atol=1e-12)


def test_kv_lists_without_lengths_use_each_tensors_length():
    spec = IfaSpec("pin", 941, "f16", "f16", B=3, N=2, Nkv=1, D=8, layout="BNSD", S=30, len_range=(5, 20),
                   kv_list=True, list_slack=6)
    inp = make_ifa(spec)
    nolen = dict(inp)
    nolen["actual_seq_lengths"] = None
    withseq = dict(inp)
    withseq["actual_seq_lengths"] = np.asarray(inp["list_seq"], dtype=np.int64)
    np.testing.assert_allclose(oracle.ifa(nolen), oracle.ifa(withseq), rtol=0, atol=0)
    # and differs from the lengths-only answer whenever some tensor is longer than its length
    assert (inp["list_seq"] > inp["lengths_drawn"]).any()
    assert not np.allclose(oracle.ifa(nolen), oracle.ifa(inp))


def test_kv_lists_with_left_padding_or_too_long_lengths_are_rejected():
    spec = IfaSpec("pin", 942, "f16", "f16", B=2, N=2, Nkv=1, D=8, layout="BNSD", S=30, len_range=(5, 20),
                   kv_list=True)
    inp = make_ifa(spec)
    bad = dict(inp)
    bad["actual_seq_lengths"] = np.asarray(inp["list_seq"], dtype=np.int64) + 1
    with pytest.raises(ValueError):
        oracle.ifa(bad)
    padded = dict(inp)
    padded["kv_padding_size"] = np.asarray([1, 1], dtype=np.int64)
    with pytest.raises(ValueError):
        oracle.ifa(padded)


# ------------------------------------------------------- output int8 ----
def test_quant_ties_go_to_even_and_codes_saturate():
    o = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.49999999, 126.5, 127.6, -128.5, -1000.0, 1000.0, 0.0])
    codes, pre = oracle.quant_int8(o, torch.tensor([1.0], dtype=torch.float32))
    assert codes.tolist() == [0, 2, 2, 0, -2, -2, 0, 126, 127, -128, -128, 127, 0]
    assert (pre == o).all()


def test_quant_scale_then_offset():
    o = np.array([0.25, -0.75, 0.1])
    codes, pre = oracle.quant_int8(o, torch.tensor([4.0]), torch.tensor([0.5]))
    # 0.25*4+0.5 = 1.5 -> 2; -0.75*4+0.5 = -2.5 -> -2; 0.1*4+0.5 = 0.9 -> 1
    assert codes.tolist() == [2, -2, 1]
    np.testing.assert_allclose(pre, [1.5, -2.5, 0.9], rtol=0, atol=1e-15)


def test_quant_per_channel_indexes_the_output_channel():
    N, D = 3, 4
    o = np.ones((2, N * D))
    sc = torch.zeros(N * D, dtype=torch.bfloat16)
    sc[1 * D + 2] = 7.0                  # head 1, column 2
    off = torch.zeros(N * D, dtype=torch.bfloat16)
    off[2 * D + 0] = -3.0                # head 2, column 0
    codes, _ = oracle.quant_int8(o, sc, off)
    want = np.zeros((2, N * D), dtype=np.int8)
    want[:, 1 * D + 2] = 7
    want[:, 2 * D + 0] = -3
    assert (codes == want).all()
