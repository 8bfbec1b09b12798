"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of ``oracle/oracle.c`` (on the
CPU, in a temporary directory), builds it, and checks that at least one pin
comparison now fails.  The unmodified oracle passes the same battery.
"""
import math
import subprocess

import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_06_amd.workloads import IfaSpec, SfaSpec, make_ifa, make_sfa
from dataclasses import replace

from test_oracle_pins import _sfa_gather_ref, _sfa_small, dense_kv_bnsd, sdpa_ref, to64
from test_oracle_sfa_breadth import _bsnd_from_paged, paged_rows, scores_rows, sdpa_rows
from test_oracle_sfa_breadth import small as _sfa_breadth

MUTANTS = {
    "gqa_mapping_modulo": ("j = h / g;", "j = h % Nkv;"),
    "scale_dropped": ("x[cnt] = scale * dot;\n            if (pse)", "x[cnt] = dot;\n            if (pse)"),
    "pse_before_scale": ("x[cnt] += elem(pse,", "x[cnt] += scale * elem(pse,"),
    "pse_batch_not_broadcast": ("((pB == 1 ? 0 : b) * N + h) * pS + s", "(b * N + h) * pS + s"),
    "pse_indexed_by_kv_head": ("((pB == 1 ? 0 : b) * N + h) * pS + s", "((pB == 1 ? 0 : b) * N + j) * pS + s"),
    "mask_polarity": ("if (mask[mi]) continue;", "if (!mask[mi]) continue;"),
    "bnsd_read_as_bsh": ("off = ((b * Nkv + j) * S + s) * D;", "off = (b * S + s) * Nkv * D + j * D;"),
    "padding_not_clamped": ("int64_t p = pad[b] < 0 ? 0 : pad[b];", "int64_t p = pad[b];"),
    "zero_rule_as_clamp": ("if (lo < 0 || hi < 0) {", "if (lo < 0) lo = 0;\n            if (hi < 0) {"),
    "paged_cache_dims_swapped": ("off = ((blk * Nkv + j) * block_size + s % block_size) * D;",
                                 "off = ((j * num_blocks + blk) * block_size + s % block_size) * D;"),
    "value_dequant_affine_other_way": ("v = (v + of) * sc;", "v = v * sc + of;"),
    "query_head_uses_kv_head": ("dot += elem(q, q_dtype, (b * N + h) * D + d) * kv;",
                                "dot += elem(q, q_dtype, (b * N + j) * D + d) * kv;"),
    "list_uses_first_tensor": ("*kb = k_list ? k_list[b] : k, *vb = k_list ? v_list[b] : v;",
                               "*kb = k_list ? k_list[0] : k, *vb = k_list ? v_list[0] : v;"),
    "list_bnsd_stride_of_padded_cache": ("off = layout == O_BNSD ? (j * Sb + s) * D", "off = layout == O_BNSD ? (j * S + s) * D"),
    "quant_ties_away_from_zero": ("double r = nearbyint(y);", "double r = round(y);"),
    "quant_symmetric_clamp": ("if (r < -128.0) r = -128.0;", "if (r < -127.0) r = -127.0;"),
    "quant_offset_before_scale": ("double y = o[i] * elem(qs, q_dtype, c);\n        if (qo) y += elem(qo, q_dtype, c);",
                                  "double y = o[i];\n        if (qo) y += elem(qo, q_dtype, c);\n        y *= elem(qs, q_dtype, c);"),
    "quant_one_channel": ("const int64_t c = i % C;", "const int64_t c = 0;"),
    "sfa_rope_dropped": ("dot += elem(q_rope, dtype, (qr * QN + h) * DR + d) * elem(key_rope, dtype, row * DR + d);",
                         "(void)0;"),
    "sfa_block_table_skipped": ("row = blk * block_size + t % block_size;", "row = t;"),
    "sfa_length_bound_inclusive": ("if (t >= limit) continue;", "if (t > limit) continue;"),
    "sfa_causal_off_by_one": ("if (sparse_mode == 3 && Lkv - Lq + s + 1 < limit) limit = Lkv - Lq + s + 1;",
                              "if (sparse_mode == 3 && Lkv - Lq + s < limit) limit = Lkv - Lq + s;"),
    "sfa_causal_top_left": ("if (sparse_mode == 3 && Lkv - Lq + s + 1 < limit) limit = Lkv - Lq + s + 1;",
                            "if (sparse_mode == 3 && s + 1 < limit) limit = s + 1;"),
    "sfa_padding_rows_attend": ("if (s >= Lq) limit = 0;", "(void)0;"),
    "sfa_block_index_not_scaled": ("const int64_t t = idx * sparse_block_size + u;", "const int64_t t = idx + u;"),
    "sfa_tnd_query_start_ignored": ("s = qr - start;", "s = qr;"),
    "sfa_tnd_cache_start_ignored": ("kv0 = b > 0 ? lkv[b - 1] : 0;", "kv0 = 0;"),
    "sfa_bsnd_cache_batch_stride": ("kv0 = b * kv_seq;", "kv0 = b;"),
    "lse_sum_not_shifted": ("if (z_out) *z_out = z;", "if (z_out) *z_out = z * exp(m);"),
    "lse_max_of_first_score": ("if (m_out) *m_out = m;", "if (m_out) *m_out = n ? x[0] : m;"),
}


def _battery(lib):
    """(name, passed) for each pin comparison, evaluated with ``lib``."""
    res = []

    def close(a, b):
        return bool(np.allclose(a, b, rtol=0, atol=1e-10))

    for layout in ("BNSD", "BSH"):
        inp = make_ifa(IfaSpec("m", 931, "bf16", "bf16", B=3, N=6, Nkv=2, D=16, layout=layout, S=37,
                               len_range=(1, 37), mask="u8", mask_p=0.3))
        res.append(("sdpa_" + layout, close(oracle.ifa(inp, use=lib), sdpa_ref(inp))))
    inp = make_ifa(IfaSpec("m", 932, "f16", "f16", B=4, N=2, Nkv=1, D=8, S=40, lengths=[10, 30, 35, 20],
                           pads=[5, -3, 10, 25]))
    try:
        res.append(("left_pad", close(oracle.ifa(inp, use=lib), sdpa_ref(inp))))
    except ValueError:
        res.append(("left_pad", False))
    inp = make_ifa(IfaSpec("m", 933, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, S=96, len_range=(1, 96), paged=True,
                           block_size=16, max_blocks=6, num_blocks=20))
    bt = inp["block_table"].long()
    kd = to64(inp["k"])[bt].permute(0, 2, 1, 3, 4).reshape(3, 2, 96, 16)
    vd = to64(inp["v"])[bt].permute(0, 2, 1, 3, 4).reshape(3, 2, 96, 16)
    try:
        res.append(("paged", close(oracle.ifa(inp, use=lib), sdpa_ref(inp, kd, vd))))
    except ValueError:
        res.append(("paged", False))
    inp = make_ifa(IfaSpec("m", 934, "f16", "i8", B=2, N=4, Nkv=2, D=16, S=30, len_range=(5, 30),
                           antiquant="per_channel"))
    k64, v64 = dense_kv_bnsd(inp)
    sc, of = to64(inp["aq_scale"]), to64(inp["aq_offset"])
    kdq = (k64 + of[0].view(1, 2, 1, 16)) * sc[0].view(1, 2, 1, 16)
    vdq = (v64 + of[1].view(1, 2, 1, 16)) * sc[1].view(1, 2, 1, 16)
    res.append(("antiquant", close(oracle.ifa(inp, use=lib), sdpa_ref(inp, kdq, vdq))))
    for pb in (0, 1):
        inp = make_ifa(IfaSpec("m", 935, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, S=40, len_range=(1, 40),
                               pse=True, pse_batch=pb, pse_scale=2.0))
        res.append(("pse_batch%d" % pb, close(oracle.ifa(inp, use=lib), sdpa_ref(inp))))
    for layout in ("BNSD", "BSH"):
        inp = make_ifa(IfaSpec("m", 938, "bf16", "bf16", B=3, N=4, Nkv=2, D=16, layout=layout, S=50,
                               len_range=(1, 40), kv_list=True))
        try:
            res.append(("kv_list_" + layout, close(oracle.ifa(inp, use=lib), sdpa_ref(inp))))
        except ValueError:
            res.append(("kv_list_" + layout, False))
    inp = make_sfa(_sfa_small())
    res.append(("sfa", close(oracle.sfa(inp, use=lib), _sfa_gather_ref(inp))))
    inp = make_sfa(_sfa_small(n_valid=[40, 50]))
    idx = inp["sparse_indices"].clone()
    idx[0, 0, 0, 40:] = 200                      # == lkv[0]: must be ignored
    inp["sparse_indices"] = idx
    res.append(("sfa_bound", close(oracle.sfa(inp, use=lib), _sfa_gather_ref(inp))))
    res.append(("quant", _quant_checks(lib)))
    for name, fn in (("sfa_causal", _sfa_causal), ("sfa_block_wise", _sfa_block_wise), ("sfa_tnd_q", _sfa_tnd_q),
                     ("sfa_tnd_kv", _sfa_tnd_kv), ("sfa_bsnd_kv", _sfa_bsnd_kv), ("sfa_lse", _sfa_lse)):
        try:
            res.append((name, fn(lib, close)))
        except ValueError:
            res.append((name, False))
    return res


def _quant_checks(lib):
    o = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.6, -128.5, -1000.0, 1000.0, 0.0])
    codes, _ = oracle.quant_int8(o, torch.tensor([1.0]), use=lib)
    ok = codes.tolist() == [0, 2, 2, 0, -2, -2, 126, 127, -128, -128, 127, 0]
    codes, _ = oracle.quant_int8(np.array([0.25, -0.75, 0.1]), torch.tensor([4.0]), torch.tensor([0.5]), use=lib)
    ok &= codes.tolist() == [2, -2, 1]
    sc = torch.zeros(12)
    sc[6] = 7.0
    codes, _ = oracle.quant_int8(np.ones((2, 12)), sc, use=lib)
    want = np.zeros((2, 12), dtype=np.int8)
    want[:, 6] = 7
    return ok and bool((codes == want).all())


def _sfa_causal(lib, close):
    lq = [4, 2]
    spec = _sfa_breadth(QS=4, lq=lq, sparse_mode=3, sparse_size=320, past_limit=True, lkv=[37, 300])
    inp = make_sfa(spec)
    idx = inp["sparse_indices"]
    idx.fill_(-1)
    for b, L in enumerate(spec.lkv):
        idx[b, :, 0, :L] = torch.arange(L, dtype=torch.int32)
    out = oracle.sfa(inp, use=lib)
    ok = True
    for b, L in enumerate(spec.lkv):
        mask = torch.ones(lq[b], L, dtype=torch.bool).tril(diagonal=L - lq[b])
        ref = sdpa_rows(inp, [b * 4 + s for s in range(lq[b])], paged_rows(inp, b, torch.arange(L)), mask)
        ok &= close(out[b * 4:b * 4 + lq[b]], ref) and bool((out[b * 4 + lq[b]:b * 4 + 4] == 0).all())
    return ok


def _sfa_block_wise(lib, close):
    sbs = 4
    spec = _sfa_breadth(QS=2, lq=[2, 1], sparse_mode=3, sparse_block_size=sbs, sparse_size=24, lkv=[197, 317],
                        past_limit=True)
    inp = make_sfa(spec)
    tok = dict(inp)
    tok["spec"] = replace(spec, sparse_block_size=1, sparse_size=24 * sbs)
    blk = inp["sparse_indices"].long()
    exp = (blk[..., :, None] * sbs + torch.arange(sbs)).reshape(*blk.shape[:-1], -1)
    exp[(blk < 0)[..., :, None].expand(*blk.shape, sbs).reshape(exp.shape)] = -1
    tok["sparse_indices"] = exp.to(torch.int32).contiguous()
    return close(oracle.sfa(inp, use=lib), oracle.sfa(tok, use=lib))


def _sfa_tnd_q(lib, close):
    lq = [3, 1, 0, 2]
    spec = _sfa_breadth(B=4, QS=3, lq=lq, sparse_mode=3, lkv=[50, 60, 70, 80], num_blocks=40, max_blocks=10)
    bsnd = make_sfa(spec)
    ref = oracle.sfa(bsnd, use=lib)
    valid = [b * 3 + s for b in range(4) for s in range(lq[b])]
    tnd = dict(bsnd)
    tnd["spec"] = replace(spec, layout_q="TND")
    tnd["q"] = bsnd["q"].reshape(-1, spec.QN, spec.D)[valid].contiguous()
    tnd["q_rope"] = bsnd["q_rope"].reshape(-1, spec.QN, spec.DR)[valid].contiguous()
    tnd["sparse_indices"] = bsnd["sparse_indices"].reshape(-1, 1, spec.sparse_size)[valid].contiguous()
    tnd["actual_seq_lengths_query"] = torch.tensor(np.cumsum(lq), dtype=torch.int32)
    tnd["q_rows"] = len(valid)
    return close(oracle.sfa(tnd, use=lib), ref[valid])


def _sfa_tnd_kv(lib, close):
    bsnd = _bsnd_from_paged(make_sfa(_sfa_breadth(QS=2, sparse_mode=0, lkv=[200, 317])))
    s = bsnd["spec"]
    tnd = dict(bsnd)
    tnd["spec"] = replace(s, layout_kv="TND")
    for name in ("key", "key_rope", "value"):
        tnd[name] = torch.cat([bsnd[name][b, :s.lkv[b]] for b in range(s.B)], dim=0).contiguous()
    tnd["actual_seq_lengths_kv"] = torch.tensor(np.cumsum(s.lkv), dtype=torch.int32)
    return close(oracle.sfa(tnd, use=lib), _sfa_gather_ref_rows(bsnd))


def _sfa_gather_ref_rows(bsnd):
    """SDPA per query row over its valid positions of a BSND cache (mode 0)."""
    s = bsnd["spec"]
    out = np.zeros((s.B * s.QS, s.QN, s.D))
    for b in range(s.B):
        for q in range(s.QS):
            idx = bsnd["sparse_indices"][b, q, 0].long()
            idx = idx[(idx >= 0) & (idx < s.lkv[b])]
            out[b * s.QS + q] = sdpa_rows(bsnd, [b * s.QS + q], b * s.kv_seq + idx)[0]
    return out


def _sfa_bsnd_kv(lib, close):
    inp = make_sfa(_sfa_breadth(QS=2, sparse_mode=0, lkv=[200, 317]))
    return close(oracle.sfa(_bsnd_from_paged(inp), use=lib), _sfa_gather_ref_rows(_bsnd_from_paged(inp)))


def _sfa_lse(lib, close):
    """softmax_max / softmax_sum against torch's max and logsumexp of the gathered scores."""
    bsnd = _bsnd_from_paged(make_sfa(_sfa_breadth(QS=1, sparse_mode=0, sparse_size=120, lkv=[200, 317])))
    s = bsnd["spec"]
    _, mx, sm = oracle.sfa(bsnd, use=lib, lse=True)
    ok = True
    for b in range(s.B):
        idx = bsnd["sparse_indices"][b, 0, 0].long()
        idx = idx[(idx >= 0) & (idx < s.lkv[b])]
        x = scores_rows(bsnd, b, b * s.kv_seq + idx)
        ok &= close(mx[b], torch.amax(x, dim=1).numpy())
        ok &= close(np.log(sm[b]) + mx[b], torch.logsumexp(x, dim=1).numpy())
    return ok


def _build(src, path):
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c11", src, "-o", path, "-lm"])
    return oracle.bind(path)


def test_unmodified_oracle_passes_battery():
    assert all(ok for _, ok in _battery(oracle.lib()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = _build(str(mpath), str(tmp_path / "libmutant.so"))
    results = _battery(lib)
    assert not all(ok for _, ok in results), "mistake %s passed every pin: %s" % (name, results)
