#!/usr/bin/env python3
"""Decode-step benchmark of the split-KV GQA decode library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

One step is one gqa_decode_ex call -- the sweep (partial) kernel and the merge
kernel -- over the whole batch, with q, k, v and seq_lens already resident in
HBM.  The default workload is the 70B-shaped ragged batch: batch 64, h_q 64,
h_kv 8, d_head 128, per-sequence lengths uniform in [1024, 32768], bf16 in and
out, fp32 accumulation, synthetic seeded data.

Prints one JSON line:
  value          K/V bytes read once per step / step time (GB/s), whole job
  us_per_step    median step time over 5 repetitions that together make the K
                 timed steps (HIP events around each), with min and max
  roofline       the sweep kernel: algorithmic K+V bytes per launch / its mean
                 duration (HIP events recorded by the library around that kernel
                 on the launch stream), against MI355X's 8 TB/s HBM peak;
                 traffic = HBM bytes per launch from the committed rocprofv3
                 counter summary if it was taken on the current kernel source
  cpu_baseline   the fp64 CPU oracle on the same inputs, on the host cores
  decode_variants  the same batch with fp16 q/k/v, with two, four or eight query
                 tokens per sequence (t_q = 2, 4, 8) and with 64 query heads per kv
                 head (h_q 512): step time, GB/s and the sweep kernel's roofline
  other_workloads  the same step on every other named workload (tiny fp32,
                 8B-shaped, single KV group, long-context stress) at its automatic
                 plan: median step time and spread, GB/s, % of the HBM peak, the
                 kernel time by events, and the traced kernel times and HBM traffic
                 ratio of its committed rocprofv3 summary (profiles/decode_*.md)
  prefill        the causal prefill row at its own workload (one KV group, 32768
                 tokens, h_q 8, d_head 128, bf16): ms per call and TFLOP/s of
                 the algorithmic causal work against the bf16 matrix-core peak,
                 in both P V precision modes, with the oracle's rate on a sample
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16 matrix-core peak of one MI355X
METRIC = "µs/decode step + K/V HBM GB/s (% of peak), GQA h_q=64 h_kv=8 d=128 @32K"
# Sources that define the sweep kernel's code and its launch plan (num_chunks,
# min_chunk and the workspace layout set the traffic per launch), so its counter
# data is tied to them.
KERNEL_SRCS = [os.path.join(ROOT, "gqa_split_kv_amd", "csrc", f)
               for f in ("sweep_kernel.hip", "merge_kernel.hip", "device_common.h", "kernels.h", "host.h", "plan.cpp",
                         "api.cpp")] + [os.path.join(ROOT, "gqa_split_kv_amd", "build.py")]   # with the compile flags
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sweep_kernel_70b_ragged_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the timing needs (events), through ctypes."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError("%s failed (%d)" % (what, rc))

    def event(self):
        e = ctypes.c_void_p()
        self._ok(self.lib.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e.value

    def record(self, ev, stream):
        self._ok(self.lib.hipEventRecord(ev, stream), "hipEventRecord")

    def sync(self, ev):
        self._ok(self.lib.hipEventSynchronize(ev), "hipEventSynchronize")

    def ms(self, a, b):
        t = ctypes.c_float()
        self._ok(self.lib.hipEventElapsedTime(ctypes.byref(t), a, b), "hipEventElapsedTime")
        return float(t.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic():
    """(bytes per launch, note) from the committed counter summary, or (None, why)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary committed"
    text = open(TRAFFIC_FILE).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t:
        return None, "counter summary unreadable"
    if h.group(1) != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return float(t.group(1)), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-kernel scaled"


REPS = 5   # the timed steps are split into this many repetitions: median and spread


def split_reps(steps: int, reps: int = REPS):
    """Sizes of the repetitions that together make exactly `steps` timed steps."""
    reps = max(1, min(reps, steps))
    base, extra = divmod(steps, reps)
    return [base + (1 if i < extra else 0) for i in range(reps)]


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def profile_fields(path: str):
    """Numbers a committed profile summary records for the current kernel sources:
    {"kernel_us": ..., "traffic_ratio": ..., ...} from its `name: value` lines, or
    (None, why) when it is missing or was taken on other sources."""
    if not os.path.exists(path):
        return None, "no profile summary committed"
    text = open(path).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not h:
        return None, "profile summary unreadable"
    if h.group(1) != kernel_source_hash():
        return None, "kernel changed since the profile was taken"
    out = {}
    for key in ("kernel_us", "merge_kernel_us", "traffic_bytes_per_launch", "traffic_ratio", "step_gap_us"):
        m = re.search(r"^%s:\s*([0-9.eE+-]+)\s*$" % key, text, flags=re.M)
        if m:
            out[key] = float(m.group(1))
    return out, os.path.relpath(path, ROOT)


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, w, budget_s: float):
    """Times the fp64 oracle on the host over whole sequences of the same inputs."""
    import numpy as np
    import oracle
    from gqa_split_kv_amd.inputs import to_host_bits
    sl = d.seq_lens_host
    # Sample: the first n sequences whose estimated oracle time fits the budget
    # (rate measured on the first sequence).
    log("cpu baseline: copying inputs to the host")
    qh, kh, vh = to_host_bits(d.q), to_host_bits(d.k), to_host_bits(d.v)
    rows0 = int(sl[0])
    t = time.perf_counter()
    oracle.gqa_decode_f64(qh[:1], kh[:rows0], vh[:rows0], sl[:1], d.scale)
    rate = rows0 / max(time.perf_counter() - t, 1e-6)            # rows (all kv heads) per second
    n = 1
    rows = rows0
    while n < len(sl) and (rows + int(sl[n])) / rate < budget_s:
        rows += int(sl[n])
        n += 1
    log("cpu baseline: oracle over %d of %d sequences (%d keys)" % (n, len(sl), rows))
    t = time.perf_counter()
    oracle.gqa_decode_f64(qh[:n], kh[:rows], vh[:rows], sl[:n], d.scale)
    dt = time.perf_counter() - t
    nbytes = rows * w.h_kv * w.d * 2 * 2
    return {
        "value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
        "cpu": cpu_model(), "seconds": dt,
        "sample": "first %d of %d sequences (%d keys, %.3g GB of K+V), same seeded inputs, "
                  "fp64 direct softmax(qK^T*scale)V per head, OpenMP over (sequence, kv head)"
                  % (n, len(sl), rows, nbytes / 1e9),
    }


def decode_variants(hip, stream, w, d, kv_bytes: int, steps: int):
    """The decode path's other input forms on the same batch and K/V bytes:
    fp16 q/k/v (gqa_decode_f16's kernels, fp16 out); two, four or eight query
    tokens per sequence (bf16, t_q = 2: every sequence's last two tokens, causal
    between them, G * t_q = 16 rows per kv head; t_q = 4: 32 rows, two 16-row
    tiles per wavefront over one load of the keys; t_q = 8: 64 rows, four tiles);
    and one token on 64 query heads per kv head (h_q 512, 64 rows).  Each is
    timed like the headline step, with the sweep kernel's own HIP events."""
    import torch
    import gqa_split_kv_amd as gqa
    from gqa_split_kv_amd.inputs import device_queries
    rows = {}
    forms = [
        ("f16", lambda: (d.q.to(torch.float16), d.k.to(torch.float16), d.v.to(torch.float16)),
         gqa.GQA_DTYPE_F16, 0),
        ("bf16_t_q2", lambda: (device_queries(w.batch, 2, w.h_q, w.d, "bf16", seed=w.seed + 7), d.k, d.v),
         gqa.GQA_DTYPE_BF16, 2),
        ("bf16_t_q4", lambda: (device_queries(w.batch, 4, w.h_q, w.d, "bf16", seed=w.seed + 9), d.k, d.v),
         gqa.GQA_DTYPE_BF16, 4),
        # 64 rows per kv head, the most the library takes: eight tokens on the same
        # grouping, and one token with G = 64 query heads per kv head (h_q 512).
        ("bf16_t_q8", lambda: (device_queries(w.batch, 8, w.h_q, w.d, "bf16", seed=w.seed + 11), d.k, d.v),
         gqa.GQA_DTYPE_BF16, 8),
        ("bf16_G64", lambda: (device_queries(w.batch, 1, 64 * w.h_kv, w.d, "bf16", seed=w.seed + 13)[:, 0]
                              .contiguous(), d.k, d.v), gqa.GQA_DTYPE_BF16, 0),
    ]
    for name, make, code, t_q in forms:
        log("decode variant %s" % name)
        q, k, v = make()
        h_q = q.shape[-2]
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        probe = gqa.make_args(q, k, v, out, d.seq_lens, w.batch, h_q, w.h_kv, w.d, d.scale, code, code,
                              stream=stream, t_q=t_q)
        ws_bytes = gqa.gqa_decode_workspace_bytes(probe)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        ev_steps = [(hip.event(), hip.event()) for _ in range(steps)]
        timed = [gqa.make_args(q, k, v, out, d.seq_lens, w.batch, h_q, w.h_kv, w.d, d.scale, code, code,
                               0, 0, ws, ws_bytes, stream, sweep_events=e, t_q=t_q) for e in ev_steps]
        warm = gqa.make_args(q, k, v, out, d.seq_lens, w.batch, h_q, w.h_kv, w.d, d.scale, code, code,
                             0, 0, ws, ws_bytes, stream, t_q=t_q)
        for _ in range(3):
            gqa.gqa_decode_ex(warm)
        torch.cuda.synchronize()
        ev = (hip.event(), hip.event())
        hip.record(ev[0], stream)
        for a in timed:
            gqa.gqa_decode_ex(a)
        hip.record(ev[1], stream)
        hip.sync(ev[1])
        ms = hip.ms(*ev) / steps
        sweep_ms = sum(hip.ms(a, b) for a, b in ev_steps) / steps
        achieved = kv_bytes / (sweep_ms / 1e3) / 1e9
        rows[name] = {"t_q": max(t_q, 1), "h_q": h_q, "rows_per_kv_head": h_q // w.h_kv * max(t_q, 1),
                      "dtype": "f16" if code == gqa.GQA_DTYPE_F16 else "bf16",
                      "us_per_step": round(ms * 1e3, 2),
                      "gb_s": round(kv_bytes / (ms / 1e3) / 1e9, 2),
                      "roofline": {"kernel": "split_kernel (key sweep)", "bound": "hbm",
                                   "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(achieved / HBM_PEAK_GBS, 4),
                                   "kernel_us": round(sweep_ms * 1e3, 2)}}
        for e in ev_steps + [ev]:
            hip.destroy(e[0])
            hip.destroy(e[1])
        # The blocks stay in torch's cache for the next form: handing them back to
        # the driver and allocating afresh measured ~4% slower sweeps on this machine.
        del q, k, v, out, ws, timed, warm
    return rows


def profile_path(workload_name: str) -> str:
    """The committed rocprofv3 summary (kernel trace and traffic) of one workload."""
    return os.path.join(ROOT, "profiles", "decode_%s.md" % workload_name)


def other_workloads(hip, stream, skip: int, steps: int):
    """The decode step on every other named workload at its automatic plan (with
    the longest length as the max_seq_len hint): median step time over REPS
    repetitions of back-to-back calls (HIP events around each repetition only),
    K/V GB/s and its fraction of the HBM peak; the kernel's own time from a second
    pass with events around each sweep launch (each event record costs the GPU
    ~3 us between kernels, which would swamp a ~10 us step, so the step loop has
    none); and, from the committed rocprofv3 summary of the workload when it was
    taken on the current kernel sources, the traced kernel times and the HBM
    traffic ratio.  Workloads whose K and V fit in the caches cycle through copies
    of their inputs totalling about 1 GiB, so every step reads its K and V from HBM."""
    import torch
    import gqa_split_kv_amd as gqa
    from gqa_split_kv_amd.inputs import WORKLOADS, device_workload
    rows = {}
    for cfg, w in sorted(WORKLOADS.items()):
        if cfg == skip:
            continue
        log("workload %d (%s)" % (cfg, w.name))
        kv_bytes = w.kv_bytes()
        rotate = 1 if kv_bytes >= (1 << 30) else min(64, -(-(1 << 30) // max(kv_bytes, 1)))
        d = device_workload(w)
        sets = [d] + [type(d)(d.q.clone(), d.k.clone(), d.v.clone(), d.seq_lens.clone(), d.seq_lens_host,
                              d.scale, d.dtype) for _ in range(rotate - 1)]
        kv_bytes = w.kv_bytes(d.seq_lens_host)
        max_len = int(d.seq_lens_host.max())
        code = gqa.GQA_DTYPE_BF16 if w.dtype == "bf16" else gqa.GQA_DTYPE_F32
        out = torch.empty((w.batch, w.h_q, w.d), dtype=d.q.dtype, device="cuda")
        probe = gqa.make_args(d.q, d.k, d.v, out, d.seq_lens, w.batch, w.h_q, w.h_kv, w.d, d.scale, code, code,
                              stream=stream, max_seq_len=max_len)
        ws_bytes = gqa.gqa_decode_workspace_bytes(probe)
        st, plan = gqa.gqa_decode_make_plan(probe, 256, 4)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        ev_steps = [(hip.event(), hip.event()) for _ in range(steps)]

        def args_for(i, events=None):
            c = sets[i % rotate]
            return gqa.make_args(c.q, c.k, c.v, out, c.seq_lens, w.batch, w.h_q, w.h_kv, w.d, c.scale, code,
                                 code, 0, 0, ws, ws_bytes, stream, sweep_events=events, max_seq_len=max_len)
        warm = [args_for(i) for i in range(rotate)]
        marked = [args_for(i, ev_steps[i]) for i in range(steps)]
        for i in range(max(rotate, 3)):
            gqa.gqa_decode_ex(warm[i % rotate])
        torch.cuda.synchronize()
        rep_ms = []
        i0 = 0
        for n in split_reps(steps):
            ev = (hip.event(), hip.event())
            hip.record(ev[0], stream)
            for i in range(i0, i0 + n):
                gqa.gqa_decode_ex(warm[i % rotate])
            hip.record(ev[1], stream)
            hip.sync(ev[1])
            rep_ms.append(hip.ms(*ev) / n)
            hip.destroy(ev[0])
            hip.destroy(ev[1])
            i0 += n
        ms = median(rep_ms)
        for a in marked:
            gqa.gqa_decode_ex(a)
        torch.cuda.synchronize()
        sweep_ms = sum(hip.ms(a, b) for a, b in ev_steps) / steps
        gbs = kv_bytes / (ms / 1e3) / 1e9
        row = {"dtype": w.dtype, "kv_bytes_per_step": kv_bytes, "rotate": rotate,
               "merge": "fused (one kernel)" if plan.fused else "merge kernel",
               "us_per_step": round(ms * 1e3, 2), "us_per_step_min": round(min(rep_ms) * 1e3, 2),
               "us_per_step_max": round(max(rep_ms) * 1e3, 2), "reps": len(rep_ms),
               "gb_s": round(gbs, 2), "pct_of_peak_hbm": round(100.0 * gbs / HBM_PEAK_GBS, 2),
               "first_kernel_us_events": round(sweep_ms * 1e3, 2),
               "us_at_hbm_peak": round(kv_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 3)}
        prof, note = profile_fields(profile_path(w.name))
        row["profile"] = note
        if prof:
            if "kernel_us" in prof:
                row["kernel_us_traced"] = prof["kernel_us"]
                row["roofline"] = {"bound": "hbm", "achieved": round(kv_bytes / prof["kernel_us"] / 1e3, 2),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(kv_bytes / prof["kernel_us"] / 1e3 / HBM_PEAK_GBS, 4)}
            for key in ("merge_kernel_us", "traffic_ratio", "step_gap_us"):
                if key in prof:
                    row[key + ("_traced" if key.endswith("_us") else "")] = prof[key]
        rows[w.name] = row
        for e in ev_steps:
            hip.destroy(e[0])
            hip.destroy(e[1])
        del d, sets, out, ws, warm, marked
    return rows


def prefill_flops(seq_lens, h_q: int, d: int) -> float:
    """Algorithmic causal-prefill work: token t of a sequence meets t + 1 keys, each
    costing 2d flops for q.k and 2d for the weighted V sum, per query head."""
    return float(sum(4.0 * d * h_q * S * (S + 1) / 2 for S in seq_lens))


def prefill_row(hip, stream, steps: int, with_oracle: bool, warmup: int = 10, group_sizes=(16, 32, 64)):
    """Times gqa_prefill_ex on the 32K-token single-KV-group workload: `warmup`
    untimed calls per mode first (the matrix-core clocks ramp up over the first
    few milliseconds of sustained work), then `steps` timed calls in REPS
    repetitions (median and spread of the per-call time).  Then the default mode
    at 16, 32 and 64 query heads per kv head on the same length (3 timed calls
    each, after 2 untimed)."""
    import torch
    import gqa_split_kv_amd as gqa
    from gqa_split_kv_amd.inputs import PREFILL_32K, device_prefill_case
    w = PREFILL_32K
    log("prefill: generating %s" % w.name)
    c = device_prefill_case(w.batch, w.h_q, w.h_kv, w.d, w.seq_lens(), w.dtype, seed=w.seed)
    out = torch.empty_like(c.q)
    flops = prefill_flops(c.seq_lens_host, w.h_q, w.d)
    row = {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "d_head": w.d,
           "seq_len": int(c.seq_lens_host[0]), "dtype": "bf16", "causal": True,
           "algorithmic_flops_per_call": flops}
    for split in (0, 1):
        a = gqa.make_prefill_args(c.q, c.k, c.v, out, c.seq_lens, w.batch, w.h_q, w.h_kv, w.d, c.scale,
                                  gqa.GQA_DTYPE_BF16, gqa.GQA_DTYPE_BF16, 0, stream, split,
                                  total_tokens=c.q.shape[0])
        for _ in range(warmup):
            gqa.gqa_prefill_ex(a)
        torch.cuda.synchronize()
        rep_ms = []
        for n in split_reps(steps):
            ev = (hip.event(), hip.event())
            hip.record(ev[0], stream)
            for _ in range(n):
                gqa.gqa_prefill_ex(a)
            hip.record(ev[1], stream)
            hip.sync(ev[1])
            rep_ms.append(hip.ms(*ev) / n)
            hip.destroy(ev[0])
            hip.destroy(ev[1])
        ms = median(rep_ms)
        tf = flops / (ms / 1e3) / 1e12
        key = "split_pv" if split else "default"
        row[key] = {"ms_per_call": round(ms, 4), "ms_min": round(min(rep_ms), 4), "ms_max": round(max(rep_ms), 4),
                    "reps": len(rep_ms), "tflops": round(tf, 1)}
        if not split:
            row["ms_per_call"] = round(ms, 4)
            row["roofline"] = {"kernel": "prefill_kernel", "bound": "mfma", "achieved": round(tf, 1),
                               "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "kernel_us": round(ms * 1e3, 1)}
    del c, out
    # Wider groups on the same sequence length (one kv head): 256 / G tokens per
    # 256-row tile, so more tiles, each sweeping its own key prefix.
    row["group_sizes"] = []
    for G in group_sizes:
        cg = device_prefill_case(1, G, 1, w.d, [w.seq_len], w.dtype, seed=w.seed + G)
        og = torch.empty_like(cg.q)
        fg = prefill_flops(cg.seq_lens_host, G, w.d)
        a = gqa.make_prefill_args(cg.q, cg.k, cg.v, og, cg.seq_lens, 1, G, 1, w.d, cg.scale,
                                  gqa.GQA_DTYPE_BF16, gqa.GQA_DTYPE_BF16, 0, stream, 0,
                                  total_tokens=cg.q.shape[0])
        for _ in range(2):
            gqa.gqa_prefill_ex(a)
        torch.cuda.synchronize()
        ev = (hip.event(), hip.event())
        hip.record(ev[0], stream)
        for _ in range(3):
            gqa.gqa_prefill_ex(a)
        hip.record(ev[1], stream)
        hip.sync(ev[1])
        ms = hip.ms(*ev) / 3
        hip.destroy(ev[0])
        hip.destroy(ev[1])
        tf = fg / (ms / 1e3) / 1e12
        row["group_sizes"].append({"G": G, "h_q": G, "h_kv": 1, "seq_len": w.seq_len, "tokens_per_tile": 256 // G,
                                   "ms_per_call": round(ms, 4), "tflops": round(tf, 1),
                                   "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        log("prefill G %d: %.3f ms per call, %.1f TFLOP/s" % (G, ms, tf))
        del cg, og
    if with_oracle:
        import numpy as np
        import oracle
        c = device_prefill_case(w.batch, w.h_q, w.h_kv, w.d, w.seq_lens(), w.dtype, seed=w.seed)
        from gqa_split_kv_amd.inputs import to_host_bits
        qh, kh, vh = to_host_bits(c.q), to_host_bits(c.k), to_host_bits(c.v)
        S = int(c.seq_lens_host[0])
        toks = list(range(S - 8, S))            # the 8 longest rows
        t = time.perf_counter()
        oracle.gqa_prefill_rows_f64(qh, kh, vh, c.seq_lens_host, c.scale, toks)
        dt = time.perf_counter() - t
        sample_flops = sum(4.0 * w.d * w.h_q * (tk + 1) for tk in toks)
        row["cpu_baseline"] = {"value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
                               "seconds": round(dt, 3),
                               "sample": "the last 8 of 32768 tokens (all 8 heads), fp64, one token at a time"}
    return row


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4, help="workload number 1..5 (default 4)")
    ap.add_argument("--num-chunks", type=int, default=0)
    ap.add_argument("--min-chunk", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=0,
                    help="independent copies of q/k/v cycled through (defeats the 256 MiB "
                         "last-level cache on small workloads); 0 = enough copies for 1 GiB "
                         "of K+V, at most 64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="timed calls of the causal prefill row (0 skips it)")
    ap.add_argument("--variant-steps", type=int, default=20,
                    help="timed steps of each other decode form (fp16, t_q = 2) on the same batch; 0 skips")
    ap.add_argument("--workload-steps", type=int, default=50,
                    help="timed steps of the decode on each other named workload; 0 skips")
    ap.add_argument("--no-step-events", action="store_true",
                    help="record no HIP events around each sweep launch in the timed loop (for kernel traces, "
                         "whose gaps between kernels the event records would lengthen); the roofline's kernel "
                         "time is then not measured")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (profiler calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X and has no "
              "multi-GPU mode (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_split_kv_amd as gqa
    from gqa_split_kv_amd.inputs import WORKLOADS, device_workload

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    hip = Hip()
    log("generating workload %d (%s)" % (w.cfg, w.name))
    kv_bytes = w.kv_bytes()
    if args.rotate <= 0:
        args.rotate = 1 if kv_bytes >= (1 << 30) else min(64, -(-(1 << 30) // max(kv_bytes, 1)))
    sets = [device_workload(w) if r == 0 else None for r in range(args.rotate)]
    d = sets[0]
    for r in range(1, args.rotate):
        sets[r] = type(d)(d.q.clone(), d.k.clone(), d.v.clone(), d.seq_lens.clone(), d.seq_lens_host,
                          d.scale, d.dtype)
    torch.cuda.synchronize()
    kv_bytes = w.kv_bytes(d.seq_lens_host)
    out = torch.empty((w.batch, w.h_q, w.d), dtype=d.q.dtype, device="cuda")
    stream = int(torch.cuda.current_stream().cuda_stream)
    dt_code = gqa.GQA_DTYPE_BF16 if w.dtype == "bf16" else gqa.GQA_DTYPE_F32
    max_len = int(d.seq_lens_host.max())     # the plan's max_seq_len hint
    probe = gqa.make_args(d.q, d.k, d.v, out, d.seq_lens, w.batch, w.h_q, w.h_kv, w.d, d.scale,
                          dt_code, dt_code, args.num_chunks, args.min_chunk, stream=stream, max_seq_len=max_len)
    ws_bytes = gqa.gqa_decode_workspace_bytes(probe)
    _, plan = gqa.gqa_decode_make_plan(probe, 256, 4)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    ev_steps = [(hip.event(), hip.event()) for _ in range(args.steps)]
    reps = split_reps(args.steps)
    ev_reps = [(hip.event(), hip.event()) for _ in reps]

    def step_args(i, events=None):
        s = sets[i % args.rotate]
        return gqa.make_args(s.q, s.k, s.v, out, s.seq_lens, w.batch, w.h_q, w.h_kv, w.d, s.scale,
                             dt_code, dt_code, args.num_chunks, args.min_chunk, ws, ws_bytes, stream,
                             sweep_events=events, max_seq_len=max_len)

    # Argument blocks are built before the timed region, so the loop issues only
    # the library calls (at a few microseconds per step the Python that fills a
    # block would otherwise be what is measured).
    warm_args = [step_args(i) for i in range(args.rotate)]
    timed_args = [step_args(i, None if args.no_step_events else ev_steps[i]) for i in range(args.steps)]
    log("warmup %d steps" % args.warmup)
    for i in range(args.warmup):
        gqa.gqa_decode_ex(warm_args[i % args.rotate])
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    decode_ex = gqa.gqa_decode_ex
    # The K timed steps run as REPS back-to-back repetitions, each bracketed by its
    # own pair of events; the step time is the median of the repetitions' means.
    t0 = time.perf_counter()
    i0 = 0
    for (e0, e1), n in zip(ev_reps, reps):
        hip.record(e0, stream)
        for a in timed_args[i0:i0 + n]:
            decode_ex(a)
        hip.record(e1, stream)
        i0 += n
    submit = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rep_ms = [hip.ms(e0, e1) / n for (e0, e1), n in zip(ev_reps, reps)]
    sweep_each = [hip.ms(a, b) for a, b in ev_steps] if not args.no_step_events else [float("nan")]
    sweep_ms = median(sweep_each)
    ms_per_step = median(rep_ms)
    value = kv_bytes / (ms_per_step / 1e3) / 1e9
    achieved = kv_bytes / (sweep_ms / 1e3) / 1e9
    traffic, traffic_note = committed_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_min": round(min(rep_ms) * 1e3, 2),
        "us_per_step_max": round(max(rep_ms) * 1e3, 2),
        "reps": len(reps),
        "timing": "median of %d repetitions of back-to-back steps (%s steps each), HIP events" % (
            len(reps), "/".join(str(n) for n in reps)),
        "pct_of_peak_hbm": round(100.0 * value / HBM_PEAK_GBS, 2),
        "wall_s_timed_region": round(wall, 4),
        "host_us_per_call": round(submit / args.steps * 1e6, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "accumulate": "fp32",
        "data": "synthetic (seeded N(0,1), rounded to bf16)",
        "config": {
            "workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "d_head": w.d,
            "seq_lens": ("uniform [%d, %d] seed %d, sum %d" % (w.ragged[0], w.ragged[1], w.seed,
                         int(d.seq_lens_host.sum()))) if w.ragged else "%d each" % w.seq_len,
            "kv_bytes_per_step": kv_bytes, "rotate": args.rotate,
            "num_chunks": args.num_chunks or "auto", "min_chunk": args.min_chunk or "auto",
            "workspace_bytes": ws_bytes,
        },
        "roofline": {
            "kernel": "fused_kernel (key sweep and merge)" if plan.fused else "split_kernel (key sweep)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
            "kernel_us": round(sweep_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": None,
    }
    # Achievable read bandwidth on this machine: the plain read probe over the
    # same K and V bytes, timed the same way.
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")     # GQA_PROBE_SINK_WORDS words
    probe_reps = 10
    for i in range(2):
        gqa.gqa_probe_read(d.k, d.k.numel() * d.k.element_size(), sink, stream)
    ev_p = (hip.event(), hip.event())
    hip.record(ev_p[0], stream)
    for i in range(probe_reps):
        gqa.gqa_probe_read(d.k, d.k.numel() * d.k.element_size(), sink, stream)
        gqa.gqa_probe_read(d.v, d.v.numel() * d.v.element_size(), sink, stream)
    hip.record(ev_p[1], stream)
    hip.sync(ev_p[1])
    probe_gbs = kv_bytes * probe_reps / (hip.ms(*ev_p) / 1e3) / 1e9
    result["roofline"]["probe_read_gbs"] = round(probe_gbs, 1)
    result["roofline"]["frac_of_probe_read"] = round(achieved / probe_gbs, 4)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        gqa.gqa_probe_copy(src, dst, n, stream)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = n
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, w, args.cpu_budget)
    if args.variant_steps > 0:
        result["decode_variants"] = decode_variants(hip, stream, w, d, kv_bytes, args.variant_steps)
    if args.workload_steps > 0:
        result["other_workloads"] = other_workloads(hip, stream, args.workload, args.workload_steps)
    if args.prefill_steps > 0:
        result["prefill"] = prefill_row(hip, stream, args.prefill_steps, not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
