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
        out.fill_(float("nan"))
    harness.call(dev, out, split=split)
    torch.cuda.synchronize()
    return out, dev


def oracle_of(inp, rows=None):
    return oracle.sfa(inp, rows=rows) if isinstance(inp["spec"], SfaSpec) else oracle.ifa(inp, rows=rows)


def compare(inp, out, rows=None, tol=None):
    """max-abs check against the oracle; returns (max_err, rms_err, rms_ref)."""
    got = out.detach().to(torch.float64).cpu().numpy().reshape(-1, inp["spec"].D)
    if rows is not None:
        got = got[np.asarray(rows)]
    ref = oracle_of(inp, rows=rows).reshape(got.shape)
    tol = TOL[out.dtype] if tol is None else tol
    assert np.isfinite(got).all(), "non-finite output"
    err = np.abs(got - ref)
    mx, rms, rref = float(err.max(initial=0)), float(np.sqrt((err ** 2).mean())), float(np.sqrt((ref ** 2).mean()))
    say("  max_abs_err=%.3e rms_err=%.3e rms_out=%.3e (tol %.1e)" % (mx, rms, rref, tol))
    assert mx <= tol, "max abs error %.3e > %.1e" % (mx, tol)
    return mx, rms, rref
