"""Shared helpers of the GPU parity tests: run a case through the C ABI and
compare it with the fp64 oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import oracle
from decode_attention_kv_06_amd import harness
from decode_attention_kv_06_amd.workloads import SfaSpec

# max-abs tolerances on the output dtype (fp32 accumulation on the GPU)
TOL = {torch.float16: 5e-3, torch.bfloat16: 2e-2}
# bounds on rms(error) / rms(output): rounding the output and P to the
# 16-bit dtype (unit roundoff 2^-9 bf16, 2^-12 fp16) keeps the ratio near
# 0.2 % for bf16 and a few 0.01 % for fp16; a 3 % error in the score scale
# puts it at a few percent
RMS_TOL = {torch.float16: 3e-3, torch.bfloat16: 1e-2}
# bound on the fp32 result's error before an int8 output is rounded: P enters
# P.V rounded to the KV dtype, which dominates (bf16 about 8x fp16)
TOL_BEFORE_QUANT = {torch.float16: 1e-3, torch.bfloat16: 1e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def describe(inp) -> str:
    s = inp["spec"]
    if isinstance(s, SfaSpec):
        return "sfa_decode_mla %s B=%d rows=%d QN=%d sparse=%d sbs=%d mode=%d %s/%s bs=%d seed=%d" % (
            s.name, s.B, inp["q_rows"], s.QN, inp["sparse_indices"].shape[-1], s.sparse_block_size, s.sparse_mode,
            s.layout_q, s.layout_kv, s.block_size, s.cfg_id)
    entry = "ifa_decode_paged" if s.paged else "ifa_decode"
    return "%s %s %s/%s %s B=%d N=%d Nkv=%d D=%d S=%d seed=%d" % (entry, s.name, s.q_dtype, s.kv_dtype, s.layout,
                                                                 s.B, s.N, s.nkv, s.D, inp["S"], s.cfg_id)


def run_gpu(inp, split=0, dev=None, out=None):
    """Run one case on cuda:0; returns (output tensor on GPU, device inputs)."""
    say("GPU step: " + describe(inp) + " split=%d" % split)
    if dev is None:
        dev = harness.to_device(inp)
    if out is None:
        out = harness.alloc_out(dev)
        out.fill_(float("nan") if out.is_floating_point() else -77)
    harness.call(dev, out, split=split)
    torch.cuda.synchronize()
    return out, dev


def oracle_of(inp, rows=None):
    return oracle.sfa(inp, rows=rows) if isinstance(inp["spec"], SfaSpec) else oracle.ifa(inp, rows=rows)


def compare_int8(inp, out, tol=None, min_clear=0.4):
    """int8 output codes against the oracle's codes of the exact output.

    The kernel decides each code from its fp32 result, the oracle from the
    exact one; the two can only differ where the scaled value lies within the
    float result's error of a rounding boundary.  Codes must agree wherever
    the oracle's value before rounding is farther than that margin from a
    boundary (k + 1/2), and differ by at most 1 elsewhere.  ``min_clear`` is the
    share of codes that must be decided away from a boundary for the check to
    mean something (0 for drawn cases whose output can be constant, such as
    an all-empty call with one per-tensor offset)."""
    s = inp["spec"]
    ref = oracle_of(inp).reshape(-1, s.N * s.D)
    codes, pre = oracle.quant_int8(ref, inp["quant_scale2"], inp["quant_offset2"])
    got = out.detach().cpu().numpy().reshape(codes.shape).astype(np.int32)
    tol = TOL_BEFORE_QUANT[inp["q"].dtype] if tol is None else tol
    qs = inp["quant_scale2"].double().reshape(1, -1).numpy()
    margin = np.abs(qs) * tol + 1e-6
    dist = np.abs(pre - (np.floor(pre) + 0.5))
    clear = (dist > margin) | (pre > 127.5 + margin) | (pre < -128.5 - margin)
    diff = np.abs(got - codes.astype(np.int32))
    say("  int8 codes: %d of %d differ, max diff %d; %d codes decided away from a boundary" % (
        int((diff > 0).sum()), diff.size, int(diff.max(initial=0)), int(clear.sum())))
    assert clear.mean() >= min_clear, "the decision margin leaves too few codes to check exactly"
    assert (diff[clear] == 0).all(), "int8 codes differ away from a rounding boundary"
    assert diff.max(initial=0) <= 1
    return int((diff > 0).sum())


def check_close(got: np.ndarray, ref: np.ndarray, tol: float, rms_tol: float):
    """The two parity bars on float outputs: max-abs error within `tol` (the
    output dtype's bound), and the RMS of the error within `rms_tol` of the
    reference's RMS.  The second catches a systematic error (a slightly wrong
    scale, a dropped term) that stays under the max-abs bar on long, nearly
    uniform softmax rows, where every output element is small."""
    assert np.isfinite(got).all(), "non-finite output"
    err = np.abs(got - ref)
    mx, rms, rref = float(err.max(initial=0)), float(np.sqrt((err ** 2).mean())), float(np.sqrt((ref ** 2).mean()))
    say("  max_abs_err=%.3e rms_err=%.3e rms_out=%.3e rms_rel=%.2e (tol %.1e, rms tol %.1e)" % (
        mx, rms, rref, rms / rref if rref > 0 else 0.0, tol, rms_tol))
    assert mx <= tol, "max abs error %.3e > %.1e" % (mx, tol)
    assert rms <= rms_tol * rref or rms <= 1e-12, "rms error %.3e > %.1e x rms output %.3e" % (rms, rms_tol, rref)
    return mx, rms, rref


def compare(inp, out, rows=None, tol=None, rms_tol=None):
    """Parity against the oracle (check_close); returns (max_err, rms_err, rms_ref)."""
    got = out.detach().to(torch.float64).cpu().numpy().reshape(-1, inp["spec"].D)
    if rows is not None:
        got = got[np.asarray(rows)]
    ref = oracle_of(inp, rows=rows).reshape(got.shape)
    return check_close(got, ref, TOL[out.dtype] if tol is None else tol,
                       RMS_TOL[out.dtype] if rms_tol is None else rms_tol)
