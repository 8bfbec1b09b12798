#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Times the library's decode call on a seeded synthetic workload resident in
HBM and prints one JSON line: µs per call, achieved HBM GB/s over the
algorithmic bytes, the dominant kernel's roofline fraction (timed live with
HIP events that the library records around that kernel on the call's
stream), and the fp64 CPU oracle timed on the host cores as a baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--flush]

Algorithmic bytes count what the method must move: the K/V rows of the
attended window (unmasked rows only when a mask is given), the mask bytes of
the window, block-table entries used, antiquant parameters, the positional
bias of the window, q and the output;
for the sparse path the selected rows (512 + 64 + 512 elements), the indices,
the block-table entries used, q, q_rope and the output.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention µs/call + achieved HBM GB/s (% of MI355X peak) at 1 GPU"
HBM_PEAK_GBS = 8000.0
CPU_BASELINE_S = 10.0      # seconds of oracle time the CPU baseline is measured over
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")


def sources_sha() -> str:
    """Hash of the library's kernel sources and build flags; counter-based
    traffic figures are only reported for the sources they were taken on."""
    import hashlib
    pkg = os.path.join(ROOT, "decode_attention_kv_06_amd")
    h = hashlib.sha256()
    files = sorted(os.path.join("csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))) + ["build.py"]
    for rel in files:
        h.update(rel.encode())
        with open(os.path.join(pkg, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel, from the
    FETCH_SIZE / WRITE_SIZE counter summary (already scaled by the copy-kernel
    calibration), or None when absent or taken on other sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = sources_sha()
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 4 and not line.startswith("#") and parts[0] == workload and parts[-1] == sha:
                return int(parts[-2])
    return None


def algorithmic_bytes(inp) -> dict:
    import numpy as np
    from decode_attention_kv_06_amd.workloads import SfaSpec
    s = inp["spec"]
    if isinstance(s, SfaSpec):
        rows = sfa_attended_rows(inp)
        eb = 2
        R = inp["q_rows"]
        kv = rows * (s.D + s.DR + s.D) * eb
        extra = R * inp["sparse_indices"].shape[-1] * 4 + s.B * 4 * (2 if s.layout_q == "TND" else 1)
        if s.layout_kv == "PA_BSND":
            extra += rows // s.sparse_block_size * 4       # one block-table entry per selected block
        qo = R * s.QN * (s.D + s.DR) * eb + R * s.QN * s.D * eb
        return {"total": kv + extra + qo, "kv": kv, "streamed": kv + extra + qo}
    B, N, nkv, D = s.B, s.N, s.nkv, s.D
    eb = 1 if s.kv_dtype == "i8" else 2
    S = inp["S"]
    L = np.asarray(inp["lengths_drawn"], dtype=np.int64)
    pads = inp["kv_padding_size"]
    lo = np.zeros(B, dtype=np.int64)
    hi = L.copy()
    if pads is not None and inp["actual_seq_lengths"] is not None:
        p = np.maximum(np.broadcast_to(np.asarray(pads, dtype=np.int64), (B,)), 0)
        lo, hi = S - p - L, S - p
        bad = (lo < 0) | (hi < 0)
        lo[bad] = hi[bad] = 0
    n_win = (hi - lo).astype(np.int64)
    attended = n_win.copy()
    mask_bytes = 0
    m = inp["mask"]
    if m is not None:
        mm = m.numpy().astype(bool)
        for b in range(B):
            row = mm[b if mm.shape[0] == B else 0, :, 0, lo[b]:hi[b]]
            attended[b] = int((~row).all(axis=0).sum()) if mm.shape[1] > 1 else int((~row[0]).sum())
            mask_bytes += row.size
    row_bytes = nkv * D * eb * 2
    kv = int(attended.sum()) * row_bytes
    streamed = int(n_win.sum()) * row_bytes
    qo = 2 * B * N * D * 2
    extra = mask_bytes
    if s.paged:
        extra += int(sum(math.ceil(int(x) / s.block_size) for x in n_win)) * 4
    if inp["aq_scale"] is not None:
        extra += 2 * inp["aq_scale"].numel() * 2
    if inp.get("pse") is not None:
        # per-batch bias: every window position of every head; a shared one once
        extra += (int(n_win.sum()) if inp["pse"].shape[0] == B else int(hi.max(initial=0))) * N * 2
    return {"total": kv + extra + qo, "kv": kv, "streamed": streamed + extra + qo}


def sfa_attended_rows(inp) -> int:
    """Cache rows the sparse call gathers: every selected position below its
    query row's limit (the kv length, or the causal bound under mode 3)."""
    import numpy as np
    s = inp["spec"]
    lkv, lq = inp["lkv_counts"], inp["lq_counts"]
    rb, rs = inp["row_batch"], inp["row_pos"]
    limit = lkv[rb].astype(np.int64)
    if s.sparse_mode == 3:
        limit = np.minimum(limit, lkv[rb] - lq[rb] + rs + 1)
    limit[rs >= lq[rb]] = 0
    idx = inp["sparse_indices"].numpy().reshape(len(rb), -1).astype(np.int64)
    sbs = s.sparse_block_size
    pos = idx[:, :, None] * sbs + np.arange(sbs)
    ok = (idx[:, :, None] >= 0) & (pos < limit[:, None, None])
    return int(ok.sum())


def describe_config(inp) -> dict:
    from decode_attention_kv_06_amd.workloads import SfaSpec
    s = inp["spec"]
    if isinstance(s, SfaSpec):
        c = {"workload": s.name, "B": s.B, "Q_S": s.QS, "Q_N": s.QN, "KV_N": 1, "D": s.D, "Dr": s.DR,
             "block_size": s.block_size, "sparse_size": int(inp["sparse_indices"].shape[-1]),
             "lkv": "U[%d,%d]" % s.lkv_range, "layout": "%s / %s" % (s.layout_q, s.layout_kv), "dtype": s.dtype}
        if s.sparse_mode:
            c["sparse_mode"] = s.sparse_mode
        if s.sparse_block_size > 1:
            c["sparse_block_size"] = s.sparse_block_size
        return c
    c = {"workload": s.name, "B": s.B, "N": s.N, "N_kv": s.nkv, "D": s.D, "Smax": inp["S"], "layout": s.layout,
         "dtype_q": s.q_dtype, "dtype_kv": s.kv_dtype}
    if s.len_range:
        c["lengths"] = "U[%d,%d]" % s.len_range
    if s.paged:
        c.update(block_size=s.block_size, num_blocks=inp["num_blocks"], cache_layout=s.cache_layout)
    if s.mask:
        c["mask"] = "%s p=%.2f" % (s.mask, s.mask_p)
    if s.pse:
        c["pse_shift"] = "shared" if s.pse_batch == 1 else "per batch"
    if s.antiquant:
        c["antiquant"] = s.antiquant
    if s.pad_off:
        c["left_padding_offset"] = "U{%d..%d}" % s.pad_off
    return c


def cpu_baseline(inp, alg_bytes: int) -> dict:
    import oracle
    from decode_attention_kv_06_amd.workloads import SfaSpec
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    # whole-workload oracle runs, repeated until about 10 s of CPU time have
    # been timed (a single run when one already takes that long)
    run = oracle.sfa if isinstance(inp["spec"], SfaSpec) else oracle.ifa
    t0 = time.perf_counter()
    n = 0
    while True:
        run(inp)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_S or dt / n * (n + 1) > 3 * CPU_BASELINE_S:
            break
    return {"value": round(n * alg_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the whole workload (every output row), %d fp64 oracle run(s) in %.1f s" % (n, dt)}



def build_args(d: dict, o, split: int, keep: list):
    """Entry-point name and its argument struct for the workload on device."""
    from decode_attention_kv_06_amd import binding
    from decode_attention_kv_06_amd.workloads import SfaSpec
    s = d["spec"]
    if isinstance(s, SfaSpec):
        from decode_attention_kv_06_amd import harness
        a = binding.sfa_args(d["q"], d["q_rope"], d["key"], d["key_rope"], d["value"], d["sparse_indices"],
                             d["block_table"], d["actual_seq_lengths_kv"], o, keep=keep,
                             **harness.sfa_options(d, split))
        return "sfa_decode_mla", a
    if s.paged:
        a = binding.ifa_paged_args(d["q"], d["k"], d["v"], o, d["block_table"], num_heads=s.N,
                                   num_key_value_heads=s.Nkv, input_layout=s.layout, scale_value=s.scale_value,
                                   actual_seq_lengths=d["actual_seq_lengths"], atten_mask=d["mask"],
                                   pse_shift=d.get("pse"),
                                   antiquant_scale=d["aq_scale"], antiquant_offset=d["aq_offset"],
                                   antiquant_mode=d["aq_mode"], kv_cache_layout=s.cache_layout,
                                   split_tokens=split, keep=keep, quant_scale2=d.get("quant_scale2"),
                                   quant_offset2=d.get("quant_offset2"))
        return "ifa_decode_paged", a
    lists = d.get("k_list") is not None
    a = binding.ifa_decode_args(d["q"], None if lists else d["k"], None if lists else d["v"], o, num_heads=s.N,
                                num_key_value_heads=s.Nkv, key_list=d.get("k_list"), value_list=d.get("v_list"),
                                input_layout=s.layout, scale_value=s.scale_value,
                                actual_seq_lengths=d["actual_seq_lengths"],
                                kv_padding_size=d["kv_padding_size"], atten_mask=d["mask"],
                                pse_shift=d.get("pse"),
                                antiquant_scale=d["aq_scale"], antiquant_offset=d["aq_offset"],
                                antiquant_mode=d["aq_mode"], split_tokens=split, keep=keep,
                                quant_scale2=d.get("quant_scale2"), quant_offset2=d.get("quant_offset2"))
    return "ifa_decode", a

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50, help="untimed calls first (at least this many)")
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="...and at least this long: the GPU takes tens of milliseconds of calls to reach steady clocks")
    ap.add_argument("--workload", default="dense_gqa_bf16_bsh")
    ap.add_argument("--flush", action="store_true", help="evict caches between calls (outside the timed events)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", type=int, default=0, help="force the work-item size (0 = planner)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this decode-attention library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from decode_attention_kv_06_amd import binding, harness
    from decode_attention_kv_06_amd.workloads import SfaSpec, make_ifa, make_sfa, workloads

    spec = workloads()[args.workload]
    print("bench: generating %s" % args.workload, file=sys.stderr, flush=True)
    inp = make_sfa(spec) if isinstance(spec, SfaSpec) else make_ifa(spec)
    dev = harness.to_device(inp, "cuda:0")
    out = harness.alloc_out(dev)
    alg = algorithmic_bytes(inp)
    stream = torch.cuda.current_stream()

    # workspace sized once, outside the timed region
    nbytes = harness.call(dev, out, split=args.split)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0")
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0") if args.flush else None

    def make_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)      # creates the underlying hipEvent
        return evs

    # arguments are marshalled once: the timed loop only calls into the library
    keep: list = []
    name, a = build_args(dev, out, args.split, keep)
    fn = getattr(binding.lib(), name)
    a_ref = ctypes.byref(a)
    ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())
    s_ptr = ctypes.c_void_p(stream.cuda_stream)

    def one_call(kb=None, ke=None):
        a.profile_event_begin = kb.cuda_event if kb is not None else None
        a.profile_event_end = ke.cuda_event if ke is not None else None
        rc = fn(a_ref, ws_ptr, ws_len, s_ptr)
        if rc != 0:
            raise binding.IfaError(rc, name)

    # warm-up: at least W calls and at least --warmup-ms of them (short calls
    # need hundreds before the clocks settle)
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
        if flush_buf is not None:
            flush_buf.zero_()
        one_call()
        n_warm += 1
        if n_warm % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    # Timed region 1 (the throughput `value`): K back-to-back calls bracketed
    # by a synchronize and two events, nothing recorded per call.  With
    # --flush every call is preceded by a cache flush and bracketed by its own
    # events instead, and the flush stays outside them.
    cb, ce = make_events(K), make_events(K)
    e0, e1 = make_events(1)[0], make_events(1)[0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        if flush_buf is not None:
            flush_buf.zero_()
            cb[i].record(stream)
        one_call()
        if flush_buf is not None:
            ce[i].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    gpu_ms_step = e0.elapsed_time(e1) / K

    # Timed region 2 (the roofline): the same K calls, with the events the
    # library records on the call's stream around its dominant kernel.
    kb, ke = make_events(K), make_events(K)
    torch.cuda.synchronize()
    for i in range(K):
        if flush_buf is not None:
            flush_buf.zero_()
        one_call(kb[i], ke[i])
    torch.cuda.synchronize()

    kern_ms = sorted(kb[i].elapsed_time(ke[i]) for i in range(K))
    kern_mean = sum(kern_ms) / K
    if flush_buf is not None:
        call_ms = sorted(cb[i].elapsed_time(ce[i]) for i in range(K))
        call_mean = sum(call_ms) / K
        call_med = call_ms[K // 2]
    else:
        call_mean = call_med = gpu_ms_step
    per_call_s = (call_mean if args.flush else ms_step) / 1e3
    value = alg["total"] / per_call_s / 1e9
    achieved = alg["total"] / (kern_mean / 1e3) / 1e9
    s = inp["spec"]
    dtype = s.dtype if isinstance(s, SfaSpec) else s.q_dtype
    kernel_name = "sfa gather kernel" if isinstance(s, SfaSpec) else "split_kernel (split-KV decode)"
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_calls_run": n_warm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded, generated on the host; see decode_attention_kv_06_amd/workloads.py)",
        "config": describe_config(inp),
        "us_per_call": round(per_call_s * 1e6, 2),
        "us_per_call_gpu_events": round(call_med * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "algorithmic_bytes": alg["total"],
        "streamed_bytes": alg["streamed"],
        "flush_between_calls": bool(args.flush),
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload), "kernel_us_mean": round(kern_mean * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, alg["total"])
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
