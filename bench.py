#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Times the library's decode calls on seeded synthetic workloads resident in
HBM and prints one JSON line.  The headline is the dense GQA decode (bf16,
BSH, 64 batches, 32 query heads over 8 KV heads, head dim 128, lengths
U[1024, 8192]); the same line carries a record for each other workload:
the tiny fp16 decode, the paged decode with a mask, the int8-cache decode
with left padding, the sparse MLA decode, the dense decode with a
positional bias and the sparse decode with two causal query rows a batch.

Protocol, per workload:
  * inputs, output and workspace are allocated once, outside every timed region;
  * warm-up: at least --warmup calls and at least --warmup-ms of them (the
    clocks need tens of milliseconds of work to settle);
  * timed, flushed (the headline): --steps iterations of [evict the caches:
    write (zero) a 512 MiB buffer, twice the 256 MiB last-level cache, then
    read it back with the read probe so that the flush's own dirty lines are
    written back before the call rather than during it; event; call; event],
    the flush outside the event pair;
  * timed, flushed, instrumented: the same loop again with the library
    recording two events on the call's stream around its dominant kernel,
    which give that kernel's duration for the roofline.  It is a loop of its
    own because those events put a timestamp and a cache release between the
    call's launches, adding 8-10 us to each call;
  * timed, warm (secondary, labelled): --steps back-to-back calls between two
    events, nothing in between, plus the host wall time of that loop;
  * median, p10 and p90 of the flushed call times; GB/s = algorithmic bytes /
    median, as a fraction of the 8 TB/s HBM peak and of the read ceiling the
    library's read probe measures on this device under the same flush.

Algorithmic bytes count what the method must move: the K/V rows of the
attended window (for a mask, the rows some query head of the KV head
attends), the mask bytes of the window, block-table entries used, antiquant
parameters, the positional bias of the window, q and the output; for the
sparse path the selected rows (512 + 64 + 512 elements; 512 + 64 when the
value tensor is the key tensor), the indices, the
block-table entries used, q, q_rope and the output.

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--flush write-read|write|read|none]
    python bench.py --read-ceiling            # only the read probe
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
FLUSH_BYTES = 512 << 20
CEILING_BYTES = 1 << 30                  # read-probe buffer: about one dense decode's K/V bytes
CPU_BASELINE_S = 10.0                    # seconds of oracle time per CPU-baseline leg
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
HEADLINE = "dense_gqa_bf16_bsh"
OTHERS = ["tiny_dense_f16", "paged_bf16_bs128", "int8_leftpad_f16", "sfa_mla_bf16", "dense_pse_bf16_bsh",
          "sfa_mtp_bf16"]


def log(msg: str) -> None:
    print("bench: " + msg, file=sys.stderr, flush=True)


def sources_sha() -> str:
    """Hash of the library's sources (kernels, the public headers they
    include) and build flags; counter-based traffic figures are only reported
    for the sources they were taken on."""
    import hashlib
    pkg = os.path.join(ROOT, "decode_attention_kv_06_amd")
    h = hashlib.sha256()
    files = sorted(os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc")))
    files += sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")))
    files.append(os.path.join(pkg, "build.py"))
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
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


# ------------------------------------------------------------------ bytes
def algorithmic_bytes(inp) -> dict:
    import numpy as np
    from decode_attention_kv_06_amd.workloads import SfaSpec
    s = inp["spec"]
    if isinstance(s, SfaSpec):
        rows, blocks = sfa_attended(inp)
        eb = 2
        R = inp["q_rows"]
        kv = rows * (s.D + s.DR + (0 if s.value_aliases_key else s.D)) * eb   # value rows that are key rows move once
        extra = R * inp["sparse_indices"].shape[-1] * 4
        for name in ("actual_seq_lengths_kv", "actual_seq_lengths_query"):   # device length arrays, when passed
            if inp[name] is not None:
                extra += inp[name].numel() * 4
        if s.layout_kv == "PA_BSND":
            extra += blocks * 4        # one block-table entry per selected block with an attended position
        qo = R * s.QN * (s.D + s.DR) * eb + R * s.QN * s.D * eb
        return {"total": kv + extra + qo, "kv": kv, "streamed": kv + extra + qo}
    B, N, nkv, D = s.B, s.N, s.nkv, s.D
    g = N // nkv
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
    head_rows = n_win * nkv                  # (position, KV head) rows of each window
    mask_bytes = 0
    m = inp["mask"]
    if m is not None:
        mm = m.numpy().astype(bool)
        for b in range(B):
            row = mm[b if mm.shape[0] == B else 0, :, 0, lo[b]:hi[b]]      # [1 | N, window]
            if mm.shape[1] == 1:
                head_rows[b] = int((~row[0]).sum()) * nkv
            else:   # a KV head's row is needed when any query head of its group attends it
                head_rows[b] = sum(int((~row[j * g:(j + 1) * g]).any(axis=0).sum()) for j in range(nkv))
            mask_bytes += row.size
    row_bytes = D * eb * 2                   # one K row and one V row of one KV head
    kv = int(head_rows.sum()) * row_bytes
    streamed = int(n_win.sum()) * nkv * row_bytes
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


def sfa_attended(inp) -> tuple:
    """(rows, blocks) of the sparse call: the cache rows it gathers (every
    selected position below its query row's limit: the kv length, or the
    causal bound under mode 3) and the selected blocks holding at least one
    of them (each costs one block-table entry)."""
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
    return int(ok.sum()), int(ok.any(axis=2).sum())


def sfa_flops(inp) -> int:
    s = inp["spec"]
    return sfa_attended(inp)[0] * s.QN * 2 * (s.D + s.DR + s.D)


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


# ------------------------------------------------------------------ CPU baseline
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(inp, alg_bytes: int, threads: int) -> dict:
    """The fp64 oracle as it stands, at `threads` threads, on a bounded sample:
    output rows spread over the whole workload (every batch and head), as
    many as take about CPU_BASELINE_S seconds, repeated whole when one pass
    over every row takes less.  GB/s = the sample's share of the
    algorithmic bytes / time."""
    import numpy as np
    import oracle
    from decode_attention_kv_06_amd.workloads import SfaSpec
    s = inp["spec"]
    sparse = isinstance(s, SfaSpec)
    run = oracle.sfa if sparse else oracle.ifa
    total_rows = inp["q_rows"] * s.QN if sparse else s.B * s.N
    used = oracle.set_threads(threads)
    probe = np.arange(0, total_rows, max(1, total_rows // (4 * used)))    # a few rows per thread
    t0 = time.perf_counter()
    run(inp, rows=probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    n_rows = int(min(total_rows, max(len(probe), CPU_BASELINE_S / max(per_row, 1e-9))))
    rows = np.unique(np.linspace(0, total_rows - 1, n_rows).astype(np.int64))
    t0 = time.perf_counter()
    passes = 0
    while True:
        run(inp, rows=None if len(rows) == total_rows else rows)
        passes += 1
        dt = time.perf_counter() - t0
        if len(rows) < total_rows or dt >= CPU_BASELINE_S or dt / passes * (passes + 1) > 3 * CPU_BASELINE_S:
            break
    share = len(rows) / total_rows
    what = ("every output row, %d pass(es)" % passes if len(rows) == total_rows else
            "%d of %d output rows, evenly spaced over all batches and heads" % (len(rows), total_rows))
    return {"value": round(passes * share * alg_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": used,
            "seconds": round(dt, 2), "sample": "%s of the %s workload, fp64 oracle, %.1f s" % (what, s.name, dt)}


def cpu_baseline(inp, alg_bytes: int) -> dict:
    all_threads = len(os.sched_getaffinity(0))
    many = _oracle_rate(inp, alg_bytes, all_threads)
    one = _oracle_rate(inp, alg_bytes, 1)
    res = dict(many)
    res["kind"] = "oracle"
    res["cpu_model"] = cpu_model()
    res["single_thread"] = one
    return res


# ------------------------------------------------------------------ GPU timing
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


def pct(sorted_vals, q: float) -> float:
    """Linear-interpolated percentile of an already sorted list."""
    if len(sorted_vals) == 1:
        return sorted_vals[0]
    x = q * (len(sorted_vals) - 1)
    i = int(math.floor(x))
    j = min(i + 1, len(sorted_vals) - 1)
    return sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (x - i)


def stats_us(ms_list) -> dict:
    v = sorted(x * 1e3 for x in ms_list)
    return {"median": round(pct(v, 0.5), 2), "p10": round(pct(v, 0.1), 2), "p90": round(pct(v, 0.9), 2),
            "mean": round(sum(v) / len(v), 2)}


class Gpu:
    """Device state shared by every measurement: the stream, the flush
    buffers and the read probe."""

    def __init__(self, flush: str):
        import torch
        from decode_attention_kv_06_amd import binding
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.flush_mode = flush
        self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0") if flush != "none" else None
        if self.flush_buf is not None:
            self.flush_buf.zero_()
        self.sink = torch.zeros(64, dtype=torch.int32, device="cuda:0")
        L = binding.lib()
        L.ifa_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.ifa_read_probe.restype = ctypes.c_int
        self.lib = L
        self.s_ptr = ctypes.c_void_p(self.stream.cuda_stream)

    def events(self, n):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(self.stream)      # creates the underlying hipEvent
        return evs

    def read(self, buf) -> None:
        rc = self.lib.ifa_read_probe(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(buf.numel()),
                                     ctypes.c_void_p(self.sink.data_ptr()), self.s_ptr)
        if rc != 0:
            raise RuntimeError("ifa_read_probe returned %d" % rc)

    def flush(self) -> None:
        """Evict L2 and the last-level cache before a timed call, outside the
        call's events.  Zeroing 512 MiB evicts every line the call could hit;
        reading the buffer back afterwards writes the flush's dirty lines to
        HBM before the call starts.  Zeroing alone leaves up to the whole
        last-level cache dirty, and a kernel whose loads allocate there then
        pays for writing it back (measured: the sparse gather kernel 43 -> 68
        us), which is the flush's cost, not the kernel's."""
        if self.flush_mode in ("write", "write-read"):
            self.flush_buf.zero_()
        if self.flush_mode in ("read", "write-read"):
            self.read(self.flush_buf)

    def timed(self, one_call, steps: int, warmup: int, warmup_ms: float, kernel_events: bool = True) -> dict:
        """Warm-up, then the flushed loop of plain calls (the call's own
        events only), then, when the library records them, a second flushed
        loop with its event pair around the dominant kernel, then the warm
        loop.  The kernel's events stay out of the loop that times the call:
        each one puts a timestamp and a cache release between the call's
        launches, which added 8-10 us to every flushed call."""
        torch = self.torch
        t_w = time.perf_counter()
        n_warm = 0
        while n_warm < warmup or (time.perf_counter() - t_w) * 1e3 < warmup_ms:
            self.flush()
            one_call(None, None)
            n_warm += 1
            if n_warm % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        cb, ce = self.events(steps), self.events(steps)
        torch.cuda.synchronize()
        for i in range(steps):
            self.flush()
            cb[i].record(self.stream)
            one_call(None, None)
            ce[i].record(self.stream)
        torch.cuda.synchronize()
        call_ms = [cb[i].elapsed_time(ce[i]) for i in range(steps)]
        kern_ms = instr_ms = None
        if kernel_events:
            cb, ce = self.events(steps), self.events(steps)
            kb, ke = self.events(steps), self.events(steps)
            torch.cuda.synchronize()
            for i in range(steps):
                self.flush()
                cb[i].record(self.stream)
                one_call(kb[i], ke[i])
                ce[i].record(self.stream)
            torch.cuda.synchronize()
            kern_ms = [kb[i].elapsed_time(ke[i]) for i in range(steps)]
            instr_ms = [cb[i].elapsed_time(ce[i]) for i in range(steps)]
        # warm: back to back, nothing between the calls
        e0, e1 = self.events(1)[0], self.events(1)[0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(self.stream)
        for _ in range(steps):
            one_call(None, None)
        e1.record(self.stream)
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3 / steps
        return {"call": stats_us(call_ms), "kernel": stats_us(kern_ms) if kern_ms else None,
                "call_with_kernel_events": stats_us(instr_ms) if instr_ms else None,
                "warm_us": round(e0.elapsed_time(e1) / steps * 1e3, 2), "host_us": round(host_ms * 1e3, 2),
                "warmup_calls": n_warm}

    def read_ceiling(self, steps: int, warmup: int, warmup_ms: float) -> dict:
        """GB/s of the read probe over CEILING_BYTES, under the same flush."""
        buf = self.torch.zeros(CEILING_BYTES, dtype=self.torch.uint8, device="cuda:0")
        r = self.timed(lambda kb, ke: self.read(buf), steps, warmup, warmup_ms, kernel_events=False)
        del buf
        med = r["call"]["median"]
        return {"gbs": round(CEILING_BYTES / (med * 1e-6) / 1e9, 1), "bytes": CEILING_BYTES,
                "us": r["call"], "flush": self.flush_mode,
                "what": "ifa_read_probe: 16 B per lane nontemporal loads, 8 in flight per lane, one workgroup of 4 waves per CU"}


def graph_replay_us(fn, a, a_ref, ws_ptr, ws_len, calls: int = 50, replays: int = 5) -> float:
    """Device time per call of `calls` back-to-back calls captured in one HIP
    graph and replayed (warm): what a captured serving loop pays per call,
    without the per-call host path of an eager launch.  Small calls only."""
    import torch
    from decode_attention_kv_06_amd import binding
    a.profile_event_begin = a.profile_event_end = None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(calls):
            rc = fn(a_ref, ws_ptr, ws_len, sp)
            if rc != 0:
                raise binding.IfaError(rc, "captured call")
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (calls * replays)
    del g
    return round(us, 2)


def sparse_kernel_name(dev, out, split: int) -> str:
    """The gather kernel the sparse call launches (the planner's choice)."""
    from decode_attention_kv_06_amd import binding, harness
    pl = binding.sfa_decode_mla_plan(dev["q"], dev["q_rope"], dev["key"], dev["key_rope"], dev["value"],
                                     dev["sparse_indices"], dev["block_table"], dev["actual_seq_lengths_kv"], out,
                                     **harness.sfa_options(dev, split))
    return "sfa_wide_kernel (sparse gather, every head in one workgroup)" if pl["all_heads"] \
        else "sfa_kernel (sparse gather, 64 heads a workgroup)"


def ifa_kernel_name(s) -> str:
    """The split kernel the dense / paged call launches: int8 caches with D = 128, head groups
    of 8, dense and without mask or bias take the matrix-core int8 kernel."""
    if s.kv_dtype == "i8" and s.D == 128 and s.N // s.nkv >= 8 and not s.paged and s.mask is None \
            and not getattr(s, "pse", False):
        return "split_kernel_i8m (split-KV, int8 products on the matrix cores)"
    return "split_kernel (split-KV)"


def measure(gpu: Gpu, name: str, args, ceiling_gbs=None) -> tuple:
    """Run one workload through the protocol; returns (record, host inputs)."""
    import torch
    from decode_attention_kv_06_amd import binding, harness
    from decode_attention_kv_06_amd.workloads import SfaSpec, make_ifa, make_sfa, workloads

    spec = workloads()[name]
    log("generating %s" % name)
    inp = make_sfa(spec) if isinstance(spec, SfaSpec) else make_ifa(spec)
    dev = harness.to_device(inp, "cuda:0")
    out = harness.alloc_out(dev)
    alg = algorithmic_bytes(inp)
    nbytes = harness.call(dev, out, split=args.split)          # sizes the workspace
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0")
    keep: list = []
    entry, a = build_args(dev, out, args.split, keep)
    fn = getattr(binding.lib(), entry)
    a_ref = ctypes.byref(a)
    ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())

    def one_call(kb, ke):
        a.profile_event_begin = kb.cuda_event if kb is not None else None
        a.profile_event_end = ke.cuda_event if ke is not None else None
        rc = fn(a_ref, ws_ptr, ws_len, gpu.s_ptr)
        if rc != 0:
            raise binding.IfaError(rc, entry)

    steps = args.steps * (10 if name == "tiny_dense_f16" else 1)     # the launch-bound call gets more samples
    log("timing %s (%d flushed + %d warm calls)" % (name, steps, steps))
    r = gpu.timed(one_call, steps, args.warmup, args.warmup_ms)
    torch.cuda.synchronize()
    graph_us = graph_replay_us(fn, a, a_ref, ws_ptr, ws_len) if r["warm_us"] < 100.0 else None
    med_s = r["call"]["median"] * 1e-6
    kern_mean_s = r["kernel"]["mean"] * 1e-6
    gbs = alg["total"] / med_s / 1e9
    achieved = alg["total"] / kern_mean_s / 1e9
    sparse = isinstance(spec, SfaSpec)
    rec = {
        "config": describe_config(inp),
        "entry_point": entry,
        "algorithmic_bytes": alg["total"],
        "streamed_bytes": alg["streamed"],
        "us_per_call": r["call"],
        "us_per_call_with_kernel_events": r["call_with_kernel_events"],
        "gbs": round(gbs, 1),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "pct_of_measured_ceiling": round(100.0 * gbs / ceiling_gbs, 2) if ceiling_gbs else None,
        "warm_back_to_back_us_per_call": r["warm_us"],
        "warm_gbs": round(alg["total"] / (r["warm_us"] * 1e-6) / 1e9, 1),
        "host_wall_us_per_call": r["host_us"],
        "graph_replay_us_per_call": graph_us,
        "timed_calls": steps,
        "warmup_calls_run": r["warmup_calls"],
        "roofline": {"bound": "hbm", "kernel": sparse_kernel_name(dev, out, args.split) if sparse else ifa_kernel_name(spec),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name),
                     "kernel_us": r["kernel"]},
    }
    if name == "tiny_dense_f16":
        rec["roofline"]["note"] = "launch-bound: 0.24 MB per call, 0.03 us at the HBM peak"
    if sparse:
        fl = sfa_flops(inp)
        rec["mfma"] = {"flops": fl, "tflops": round(fl / kern_mean_s / 1e12, 1),
                       "pct_of_bf16_dense_peak": round(100.0 * fl / kern_mean_s / 2.5e15, 2)}
    del dev, out, ws, keep, a
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, inp


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed calls per loop (10x for the tiny workload)")
    ap.add_argument("--warmup", type=int, default=50, help="untimed calls first (at least this many)")
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="...and at least this long: the GPU takes tens of milliseconds of calls to reach steady clocks")
    ap.add_argument("--workload", default="all",
                    help="'all' (the dense GQA headline plus a record per other workload) or one workload name")
    ap.add_argument("--flush", choices=["write-read", "write", "read", "none"], default="write-read",
                    help="cache eviction before each timed call, outside its events: zero 512 MiB and read it "
                         "back (default), zero only, read only, or none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--read-ceiling", action="store_true", help="only measure the read probe")
    ap.add_argument("--split", type=int, default=0, help="force the work-item size (0 = planner)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this decode-attention library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    gpu = Gpu(args.flush)
    log("read ceiling (%d MiB, flush=%s)" % (CEILING_BYTES >> 20, args.flush))
    ceiling = gpu.read_ceiling(args.steps, args.warmup, args.warmup_ms)
    if args.read_ceiling:
        print(json.dumps({"read_ceiling": ceiling}), flush=True)
        return 0

    headline = HEADLINE if args.workload == "all" else args.workload
    others = OTHERS if args.workload == "all" else []
    rec, inp = measure(gpu, headline, args, ceiling["gbs"])
    per_config = {}
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle (all threads, then one)")
        cpu = cpu_baseline(inp, rec["algorithmic_bytes"])
    del inp
    for name in others:
        r, inp_o = measure(gpu, name, args, ceiling["gbs"])
        del inp_o
        per_config[name] = r

    from decode_attention_kv_06_amd.workloads import SfaSpec, workloads
    s = workloads()[headline]
    med_us = rec["us_per_call"]["median"]
    res = {
        "metric": METRIC,
        "value": rec["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype if isinstance(s, SfaSpec) else s.q_dtype,
        "data": "synthetic (seeded, generated on the host; see decode_attention_kv_06_amd/workloads.py)",
        "config": rec["config"],
        "us_per_call": med_us,
        "us_per_call_p10": rec["us_per_call"]["p10"],
        "us_per_call_p90": rec["us_per_call"]["p90"],
        "pct_of_hbm_peak": rec["pct_of_hbm_peak"],
        "pct_of_measured_ceiling": rec["pct_of_measured_ceiling"],
        "flush_between_calls": args.flush != "none",
        "flush": "%s %d MiB before every timed call, outside its events" % (args.flush, FLUSH_BYTES >> 20)
                 if args.flush != "none" else "none",
        "timing": "per-call HIP events on the call's stream; median, p10 and p90 over the flushed calls; "
                  "the dominant kernel's events in a second flushed loop of their own",
        "warm_back_to_back_us_per_call": rec["warm_back_to_back_us_per_call"],
        "host_wall_us_per_call": rec["host_wall_us_per_call"],
        "algorithmic_bytes": rec["algorithmic_bytes"],
        "streamed_bytes": rec["streamed_bytes"],
        "roofline": rec["roofline"],
        "read_ceiling": ceiling,
        "headline": rec,
        "per_config": per_config,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
