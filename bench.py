"""Benchmark: chunked GLA prefill forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_16k]

A step is one gla_fwd call over the whole workload (every stage of the path:
segment end states, their scan, and the fused cumsum / intra-chunk / output /
state pass), inputs resident in HBM.  Two independent input sets alternate
between steps so that the 256 MB Infinity Cache cannot serve a whole step
from the previous one.  K steps are timed between two synchronisations with
one pair of HIP events (the headline).  The same K steps are then run again
with per-step events and the library's per-launch event tracing, which times
the dominant kernel (the output pass) on its own launch stream and gives the
latency percentiles; those events sit between kernels, so that second
region's step time is reported apart from the headline.

Prints one JSON line.  ``value`` is prefill tokens/s = B*T / step time.
``roofline`` prices the output pass against HBM bandwidth with the
algorithmic bytes of the workload (bf16 q, k, v, o + fp32 g per token-head,
plus the fp32 final state); ``cpu_baseline`` is the fp64 oracle timed on the
host cores over a bounded sample of the same workload.

Other forward configurations (separate lines): --workload prefill_4k,
batch16_4k or long_128k (bf16), and tiny_f32 (B=1, H=2, T=256, D=64), which
runs the fp32 path (gla_fwd_f32; 4-byte q, k, v, o in the algorithmic bytes,
the MFMA fraction against the fp32 peak).

Scalar gate (a separate line, not the headline):
    python bench.py --workload prefill_16k_scalar
the same step through gla_fwd_scalar (g [B,H,T]); its algorithmic bytes
per token-head are 1028 at D=128 (bf16 q, k, v, o + one fp32 gate).

Backward (a separate line, not the headline):
    python bench.py --workload prefill_16k --backward
A step is one gla_bwd call: the forward's chunk-start states recomputed,
the reverse segment pass and scan, and the backward chunk pass writing dq,
dk, dv, dg.  ``value`` is B*T / step time; ``roofline`` prices the backward
chunk pass against HBM bandwidth with its algorithmic bytes (bf16 q, k, v,
do read and dq, dk, dv written, fp32 g read and dg written, and the fp32
chunk-start state read once per chunk).

Gated delta rule (a separate line, not the headline):
    python bench.py --workload gdn_b16_4k
A step is one gla_gdn_fwd call over the workload; ``value`` is B*T / step
time; ``roofline`` prices the kernel against HBM bandwidth with its
algorithmic bytes (bf16 q, k, v, o and fp32 g, beta per token-head, plus the
fp32 final state) and also reports its bf16 MFMA rate.

Decode (a separate line, not the headline):
    python bench.py --workload decode_b256 [--steps K] [--warmup W]
A step is one gla_decode call: one token for each of B sequences x H heads
against a carried fp32 state, updated in place.  ``value`` is decode
tokens/s = B / step time; ``roofline`` prices the decode kernel against HBM
bandwidth with its algorithmic bytes (fp32 state read + written, bf16 q, k,
v, o and fp32 g per (batch, head) row).

Helpers for the counter runs (used under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE):
    --copy-calibration  also runs a plain device copy of known size, so
                        FETCH_SIZE / WRITE_SIZE can be scaled to bytes
    --summarize-counters DIR  parses rocprofv3 counter CSVs under DIR and
                        writes profiles/counters_<workload>.json
    --summarize-mfma DIR [DIR ...]  prints per-pass MFMA instruction counts, busy
                        fraction and bf16 / fp32 MFMA rates from rocprofv3
                        counter CSVs under the DIRs
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, TFLOP/s
METRIC = "prefill tokens/s, chunk GLA fwd H=16 D=128 bf16; % MFMA peak / HBM BW"
SCALAR_METRIC = "prefill tokens/s, chunk scalar-gate linear attention fwd H=16 D=128 bf16; % HBM BW"
F32_METRIC = "prefill tokens/s, chunk GLA fwd fp32 q/k/v/o; % fp32 MFMA peak / HBM BW"
BWD_METRIC = ("backward tokens/s, chunk GLA bwd H=16 D=128 bf16 (forward states recomputed); "
              "% HBM BW")
GDN_METRIC = "prefill tokens/s, chunk gated delta rule fwd H=16 D=128 bf16; % HBM BW"
DECODE_METRIC = "decode tokens/s, GLA decode step H=16 D=128 bf16 q/k/v/o, fp32 state; % HBM BW"
# The pages' number for this workload (FLA chunk_gla, RTX 4090, bf16, H=16,
# D=128, B=1, T=16K: 2.17 ms) as tokens/s: another machine, context only.
PAGES_TOKENS_PER_S = {"prefill_16k": 1 * 16384 / 2.17e-3, "prefill_4k": 1 * 4096 / 0.47e-3}
KERNEL_SOURCES = [os.path.join(ROOT, "chunked_state_recurrence_amd", "csrc", f)
                  for f in ("gla_kernels.hip", "gla_bwd.hip", "gla_gdn.hip", "gla_api.hip",
                            "gla_internal.h", "gla_device.h")]
COPY_BYTES = 1 << 30


def host_threads() -> int:
    """Every CPU this process may run on (what `nproc` reports)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def hsa_gpu_info():
    """The first GPU agent's board name (HSA_AMD_AGENT_INFO_PRODUCT_NAME,
    0xA009, 64 chars; the runtime fills it from the KFD node's marketing name
    and falls back to a generic one where libdrm's ID table is missing) and
    its maximum engine clock in MHz (HSA_AMD_AGENT_INFO_MAX_CLOCK_FREQUENCY,
    0xA003), asked of the HSA runtime in this process (hsa_init is reference
    counted); (None, None) where there is none.  No child process is started:
    a GPU process must not exec another program."""
    import ctypes
    try:
        hsa = ctypes.CDLL("libhsa-runtime64.so.1")
    except OSError:
        return None, None
    if hsa.hsa_init() != 0:
        return None, None
    found = []
    cb_t = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p)

    def visit(agent, _data):
        dev = ctypes.c_uint32(0)
        if hsa.hsa_agent_get_info(ctypes.c_uint64(agent), 17, ctypes.byref(dev)) == 0 and dev.value == 1:
            buf = ctypes.create_string_buffer(64)
            clk = ctypes.c_uint32(0)
            name = (buf.value.decode(errors="replace").strip()
                    if hsa.hsa_agent_get_info(ctypes.c_uint64(agent), 0xA009, buf) == 0 else None)
            mhz = clk.value if hsa.hsa_agent_get_info(ctypes.c_uint64(agent), 0xA003, ctypes.byref(clk)) == 0 else None
            found.append((name or None, mhz or None))
        return 0   # HSA_STATUS_SUCCESS: keep iterating

    try:
        hsa.hsa_iterate_agents(cb_t(visit), None)
    finally:
        hsa.hsa_shut_down()
    return found[0] if found else (None, None)


def gpu_label(arch, cus, mhz, board):
    """The product: gfx950 with 256 CUs is MI355X at a 2400 MHz peak engine
    clock and MI350X below it (labelled as inferred); else the board name."""
    if arch and arch.startswith("gfx950") and cus == 256 and mhz:
        return f"AMD Instinct {'MI355X' if mhz >= 2400 else 'MI350X'} (inferred: gfx950, 256 CUs, {mhz} MHz)"
    return board


def environment() -> dict:
    """GPU, ROCm and host CPU the numbers were measured on."""
    env = {"nproc": host_threads(), "os_cpu_count": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    env["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
            env["cgroup_cpus"] = None if quota == "max" else int(quota) / int(period)
    except (OSError, ValueError):
        pass
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                env["rocm"] = f.read().strip()
                break
        except OSError:
            pass
    try:
        import torch
        env["torch"] = torch.__version__
        env["torch_hip"] = torch.version.hip
        if torch.cuda.is_available():
            prop = torch.cuda.get_device_properties(0)
            board, mhz = hsa_gpu_info()
            env["gpu_arch"] = getattr(prop, "gcnArchName", None)
            env["gpu_cus"] = prop.multi_processor_count
            env["gpu_mem_gib"] = round(prop.total_memory / 2 ** 30, 1)
            env["gpu_max_clock_mhz"] = mhz
            env["gpu_board_name"] = prop.name or board
            env["gpu"] = gpu_label(env["gpu_arch"], env["gpu_cus"], mhz, env["gpu_board_name"])
    except Exception as e:   # noqa: BLE001 - informational only
        env["torch_error"] = str(e)
    return env


def algorithmic_bytes(wl) -> int:
    """q, k, v, o (2 B each in bf16, 4 B in fp32) + fp32 g (4 B; one per token
    for the scalar gate) per token-head element row, plus the fp32 h0 read and h_final write
    when present."""
    th = wl.B * wl.H * wl.T
    es = 2 if wl.dtype == "bf16" else 4
    gate = 4 if wl.scalar_gate else wl.D * 4
    per_token_head = wl.D * 4 * es + gate         # 1536 B at D=128, bf16 (scalar gate: 1028)
    state = wl.B * wl.H * wl.D * wl.D * 4
    return th * per_token_head + (state if wl.want_final else 0) + (state if wl.h0_std else 0)


KIND_NAMES = {"output": "output pass (chunk_kernel, MODE_OUT)", "segment": "state pass (state_kernel)",
              "scan": "segment-state scan (scan_kernel)",
              "states": "states-only forward pass of the backward (chunk_kernel, MODE_STATES)"}


def pass_bytes(wl, kind: str):
    """Algorithmic bytes of one launch of a forward pass: the output pass
    reads q, k, v, g and writes o for every token-head (plus h0 / h_final), so
    its unit is the workload's; other passes are not priced on their own."""
    return algorithmic_bytes(wl) if kind == "output" else None


def backward_bytes(wl, chunk: int) -> int:
    """Backward chunk pass, per token-head: bf16 q, k, v, do read and dq, dk,
    dv written (2 B each), fp32 g read and dg written, plus one fp32 D x D
    chunk-start state read per chunk."""
    th = wl.B * wl.H * wl.T
    es = 2 if wl.dtype == "bf16" else 4
    n_chunks = wl.B * wl.H * ((wl.T + chunk - 1) // chunk)
    return th * wl.D * (7 * es + 8) + n_chunks * wl.D * wl.D * 4


def gdn_bytes(wl) -> int:
    """Per token-head: bf16 q, k, v, o (2 B each) and fp32 g, beta; plus the
    fp32 final state per head."""
    return wl.B * wl.H * (wl.T * (wl.D * 8 + 8) + wl.D * wl.D * 4)


GDN_RECORD_BYTES = {128: 119808, 64: 62464}   # per chunk and head, gdn_record_bytes() in the library


def gdn_prep_bytes(wl, chunk: int = 64) -> int:
    """Two-launch form, prep launch: bf16 q, k, v and fp32 g, beta read per
    token-head; one record plus gamma_C written per chunk and head."""
    n = -(-wl.T // chunk)
    return wl.B * wl.H * (wl.T * (wl.D * 6 + 8) + n * (GDN_RECORD_BYTES[wl.D] + 4))


def gdn_walk_bytes(wl, chunk: int = 64) -> int:
    """Two-launch form, walk launch: every record (and gamma_C) read once per
    chunk and head, bf16 o written per token-head, the fp32 final state."""
    n = -(-wl.T // chunk)
    return wl.B * wl.H * (n * (GDN_RECORD_BYTES[wl.D] + 4) + wl.T * wl.D * 2 + wl.D * wl.D * 4)


def gdn_flops(wl, chunk: int = 64) -> int:
    """Matrix products per token-head of the chunk form: k k^T, q k^T, W and
    U~ (chunk-deep), W S, q S and the state update (D-deep), P U."""
    th = wl.B * wl.H * wl.T
    return th * (2 * chunk * wl.D * 5 + 2 * wl.D * wl.D * 3)


def decode_bytes(wl) -> int:
    """Per (batch, head) row: the fp32 D x D state read and written, bf16 q, k,
    v, o (2 B each) and fp32 g (4 B) of D elements."""
    return wl.B * wl.H * (2 * wl.D * wl.D * 4 + wl.D * (4 * 2 + 4))


def algorithmic_flops(wl, chunk: int) -> int:
    """Per token-head: scores (C+1)K, A.V (C+1)V, q.S 2KV, K^T V 2KV (the dense
    T^2 work the chunk form avoids is not counted)."""
    th = wl.B * wl.H * wl.T
    return th * (4 * wl.D * wl.D + (chunk + 1) * 2 * wl.D)


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that a change to a
    comment keeps the counters taken before it."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """Digest of the kernel sources' code (comments and spacing ignored)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def cpu_baseline(wl, x, budget_s: float = 20.0, min_s: float = 10.0):
    """Time the fp64 oracle on the host: whole heads of the workload, as many
    as fit the time budget (at least one), extrapolated to tokens/s of the
    full workload.  When that sample takes less than min_s it is repeated
    until min_s has passed, and the mean is used."""
    import numpy as np
    import oracle
    from chunked_state_recurrence_amd.workloads import to_f64_numpy

    threads = host_threads()
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]

    def run(sel):
        f = {n: (None if x[n] is None else
                 np.stack([to_f64_numpy(x[n][b, h]) for (b, h) in sel])[None])
             for n in ("q", "k", "v", "g", "h0")}
        t0 = time.perf_counter()
        if wl.scalar_gate:
            oracle.scalar_gate_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], wl.scale,
                                          threads=threads)
        else:
            oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], wl.scale,
                                    threads=threads)
        return time.perf_counter() - t0

    t1 = run(pairs[:1])
    n = max(1, min(len(pairs), int(budget_s / max(t1, 1e-6))))
    n = max(n, min(len(pairs), threads))  # keep every thread busy when it is cheap
    times = [run(pairs[:n]) if n > 1 else t1]
    while sum(times) < min_s:
        times.append(run(pairs[:n]))
    t = statistics.mean(times)
    full = t * len(pairs) / n
    return {"value": wl.B * wl.T / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {wl.B * wl.H} (batch, head) sequences, full T={wl.T}, fp64 "
                      f"token recurrence, {len(times)} passes of {t:.2f} s; scaled to all heads",
            "seconds": round(sum(times), 3)}


def cpu_baseline_decode(wl, x, min_s: float = 10.0):
    """Time the fp64 oracle for one decode step (the recurrence over T = 1
    from the carried state) on the host over the first sequences' rows,
    repeated until min_s has passed; scaled to decode tokens/s of all rows."""
    import numpy as np
    import oracle
    from chunked_state_recurrence_amd.workloads import to_f64_numpy

    threads = host_threads()
    nb = min(wl.B, 64)
    f = {n: np.ascontiguousarray(to_f64_numpy(x[n][:nb])) for n in ("q", "k", "v", "g", "h0")}
    times = []
    while sum(times) < min_s:
        t0 = time.perf_counter()
        oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], wl.scale, threads=threads)
        times.append(time.perf_counter() - t0)
    t = statistics.mean(times) * wl.B / nb
    return {"value": wl.B / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nb * wl.H} of {wl.B * wl.H} (batch, head) rows, one fp64 decode step "
                      f"each, {len(times)} passes of {statistics.mean(times) * 1e3:.1f} ms; "
                      "scaled to all rows",
            "seconds": round(sum(times), 3)}


def emit(res: dict):
    """Print the one JSON line, with the machine it was measured on."""
    res.setdefault("env", environment())
    if isinstance(res.get("cpu_baseline"), dict):
        res["cpu_baseline"].setdefault("cpu_model", res["env"].get("cpu_model"))
    print(json.dumps(res), flush=True)


def copy_calibration(dev):
    """A plain device copy of COPY_BYTES, three times, for counter scaling."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def bench_decode(args, wl):
    import torch

    import chunked_state_recurrence_amd as gla
    from chunked_state_recurrence_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    host = make_inputs(wl)
    sets = []
    for s in range(2):  # two independent sets (2 x 256 MiB of state) alternate
        d = {n: host[n][:, :, 0].contiguous().to(dev) for n in ("q", "k", "v", "g")}
        d["state"] = host["h0"].to(dev)
        d["o"] = torch.empty(wl.B, wl.H, wl.D, dtype=torch.bfloat16, device=dev)
        sets.append(d)
    stream = torch.cuda.current_stream()

    def step(i):
        d = sets[i & 1]
        gla.gla_decode(d["q"], d["k"], d["v"], d["g"], d["state"], scale=wl.scale, o=d["o"],
                       stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps

    gla.profile_start(args.steps + 8)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kms = [t for kind, t in gla.profile_stop() if kind == "decode"]
    k_ms = statistics.mean(kms)
    per_launch = decode_bytes(wl)
    achieved = per_launch / (k_ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(dev)
    traffic = None
    c = read_counters(wl.name)
    if c and "fetch_factor" in c:
        m = c["median_per_dispatch_KiB"]
        f, w = m.get("decode:FETCH_SIZE"), m.get("decode:WRITE_SIZE")
        if f is not None and w is not None:
            traffic = int(f * 1024 * c["fetch_factor"] + w * 1024 * c["write_factor"])
    res = {
        "metric": DECODE_METRIC,
        "value": wl.B / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "K": wl.D, "V": wl.D,
                   "state": "fp32, updated in place", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_kernel<BF16,128>", "kernel_ms": k_ms,
                     "algorithmic_bytes_per_launch": per_launch},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_decode(wl, host)
    emit(res)


def cpu_baseline_backward(wl, x, gr, min_s: float = 10.0):
    """Time the fp64 oracle backward on the host over whole heads of the
    workload (as many as fit about min_s, at least one), repeated until min_s
    has passed; scaled to tokens/s of all heads."""
    import numpy as np
    import oracle
    from chunked_state_recurrence_amd.workloads import to_f64_numpy

    threads = host_threads()
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    src = dict(x)
    src["do"], src["dhf"] = gr["do"], gr["dh_final"]

    def run(sel):
        f = {n: (None if src[n] is None else
                 np.stack([to_f64_numpy(src[n][b, h]) for (b, h) in sel])[None])
             for n in ("q", "k", "v", "g", "h0", "do", "dhf")}
        t0 = time.perf_counter()
        oracle.token_recurrence_backward(f["q"], f["k"], f["v"], f["g"], f["h0"], f["do"],
                                         f["dhf"], wl.scale, threads=threads)
        return time.perf_counter() - t0

    n = min(len(pairs), threads)
    times = [run(pairs[:n])]
    while sum(times) < min_s:
        times.append(run(pairs[:n]))
    t = statistics.mean(times) * len(pairs) / n
    return {"value": wl.B * wl.T / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {len(pairs)} (batch, head) sequences, full T={wl.T}, fp64 token "
                      f"backward, {len(times)} passes of {statistics.mean(times):.2f} s; "
                      "scaled to all heads",
            "seconds": round(sum(times), 3)}


def cpu_baseline_gdn(wl, x, min_s: float = 10.0):
    """The fp64 gated-delta-rule oracle on the host over whole heads (as many
    as there are threads), repeated until min_s has passed; scaled to all heads."""
    import numpy as np
    import oracle
    from chunked_state_recurrence_amd.workloads import to_f64_numpy

    threads = host_threads()
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)][:threads]
    f = {n: (None if x[n] is None else np.stack([to_f64_numpy(x[n][b, h]) for (b, h) in pairs])[None])
         for n in ("q", "k", "v", "g", "beta", "h0")}
    times = []
    while sum(times) < min_s:
        t0 = time.perf_counter()
        oracle.gdn_recurrence(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"], wl.scale,
                              threads=threads)
        times.append(time.perf_counter() - t0)
    t = statistics.mean(times) * wl.B * wl.H / len(pairs)
    return {"value": wl.B * wl.T / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.B * wl.H} (batch, head) sequences, full T={wl.T}, fp64 "
                      f"token recurrence, {len(times)} passes of {statistics.mean(times):.2f} s; "
                      "scaled to all heads",
            "seconds": round(sum(times), 3)}


def bench_gdn(args, wl):
    import torch

    import chunked_state_recurrence_amd as gla
    from chunked_state_recurrence_amd.workloads import make_gdn_inputs

    dev = torch.device("cuda:0")
    host = make_gdn_inputs(wl)
    sets = []
    for s in range(2):   # two independent input sets alternate
        d = {n: (None if host[n] is None else host[n].to(dev))
             for n in ("q", "k", "v", "g", "beta", "h0")}
        if s == 1:
            d = {n: (None if t is None else t.clone()) for n, t in d.items()}
        d["o"] = torch.empty(wl.B, wl.H, wl.T, wl.D, dtype=torch.bfloat16, device=dev)
        d["hf"] = torch.empty(wl.B, wl.H, wl.D, wl.D, dtype=torch.float32, device=dev)
        sets.append(d)
    stream = torch.cuda.current_stream()

    def step(i):
        d = sets[i & 1]
        gla.gla_gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=wl.scale,
                        o=d["o"], h_final=d["hf"], want_final=True, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    gla.profile_start(4 * args.steps + 8)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    by = {}
    for kind, t in gla.profile_stop():
        by.setdefault(kind, []).append(t)
    if args.copy_calibration:
        copy_calibration(dev)
    # the one-launch form, or the larger of the two launches of the other form
    names = {"gdn": ("gdn_kernel<128,64,false>", gdn_bytes(wl)),
             "gdn_prep": ("gdn_kernel<128,64,true> (prep)", gdn_prep_bytes(wl)),
             "gdn_walk": ("gdn_walk_kernel<128,64>", gdn_walk_bytes(wl))}
    kinds = [k for k in names if k in by]
    dom = max(kinds, key=lambda k: sum(by[k]))
    k_ms = statistics.mean(by[dom])
    kname, per_launch = names[dom]
    achieved = per_launch / (k_ms * 1e-3) / 1e9
    flops = gdn_flops(wl)
    path_ms = sum(sum(by[k]) for k in kinds) / args.steps
    traffic = None
    c = read_counters(wl.name)
    if c and "fetch_factor" in c:
        m = c["median_per_dispatch_KiB"]
        f, w = m.get(f"{dom}:FETCH_SIZE"), m.get(f"{dom}:WRITE_SIZE")
        if f is not None and w is not None:
            traffic = int(f * 1024 * c["fetch_factor"] + w * 1024 * c["write_factor"])
    res = {
        "metric": GDN_METRIC,
        "value": wl.B * wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "K": wl.D, "V": wl.D,
                   "chunk": 64, "h_final": True, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "kernel_ms": k_ms,
                     "algorithmic_bytes_per_launch": per_launch},
        "whole_path": {"launches": {k: statistics.mean(by[k]) for k in kinds},
                       "kernels_ms_per_step": path_ms,
                       "algorithmic_bytes": gdn_bytes(wl),
                       "hbm_frac": gdn_bytes(wl) / (path_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "mfma_tflops": flops / (path_ms * 1e-3) / 1e12,
                       "mfma_frac": flops / (path_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_gdn(wl, host)
    emit(res)


def bench_backward(args, wl):
    import torch

    import chunked_state_recurrence_amd as gla
    from chunked_state_recurrence_amd.workloads import make_grad_inputs, make_inputs

    dev = torch.device("cuda:0")
    chunk = args.chunk or 64
    host = make_inputs(wl)
    gr = make_grad_inputs(wl)
    sets = []
    for s in range(2):   # two independent input sets alternate
        d = {n: (None if host[n] is None else host[n].to(dev)) for n in ("q", "k", "v", "g", "h0")}
        d["do"] = gr["do"].to(dev)
        d["dhf"] = None if gr["dh_final"] is None else gr["dh_final"].to(dev)
        if s == 1:
            d = {n: (None if t is None else t.clone()) for n, t in d.items()}
        shp = (wl.B, wl.H, wl.T, wl.D)
        d["out"] = {"dq": torch.empty(shp, dtype=torch.bfloat16, device=dev),
                    "dk": torch.empty(shp, dtype=torch.bfloat16, device=dev),
                    "dv": torch.empty(shp, dtype=torch.bfloat16, device=dev),
                    "dg": torch.empty(shp, dtype=torch.float32, device=dev),
                    "dh0": torch.empty((wl.B, wl.H, wl.D, wl.D), dtype=torch.float32, device=dev)}
        sets.append(d)
    stream = torch.cuda.current_stream()

    def step(i):
        d = sets[i & 1]
        gla.gla_bwd(d["q"], d["k"], d["v"], d["g"], d["h0"], d["do"], d["dhf"], chunk=chunk,
                    scale=wl.scale, out=d["out"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps

    gla.profile_start(16 * args.steps + 16)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    by_kind = {}
    for kind, kms in gla.profile_stop():
        by_kind.setdefault(kind, []).append(kms)
    if args.copy_calibration:
        copy_calibration(dev)
    k_ms = statistics.mean(by_kind["bwd"])
    per_launch = backward_bytes(wl, chunk)
    achieved = per_launch / (k_ms * 1e-3) / 1e9
    traffic = None
    c = read_counters(wl.name + "_bwd")
    if c and "fetch_factor" in c:
        m = c["median_per_dispatch_KiB"]
        f, w = m.get("bwd:FETCH_SIZE"), m.get("bwd:WRITE_SIZE")
        if f is not None and w is not None:
            traffic = int(f * 1024 * c["fetch_factor"] + w * 1024 * c["write_factor"])
    res = {
        "metric": BWD_METRIC,
        "value": wl.B * wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + " backward", "B": wl.B, "H": wl.H, "T": wl.T, "K": wl.D,
                   "V": wl.D, "chunk": chunk, "h0": wl.h0_std is not None, "dh_final": True,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "backward chunk pass (bwd_kernel<BF16,128,64,BM_FULL>)",
                     "kernel_ms": k_ms, "algorithmic_bytes_per_launch": per_launch},
        "kernels_ms": {k: statistics.mean(v) for k, v in by_kind.items()},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_backward(wl, host, gr)
    emit(res)


def read_counters(wl_name: str):
    path = os.path.join(ROOT, "profiles", f"counters_{wl_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_digest") != source_digest():
        return None  # the kernel changed since the counters were taken
    return c


def kernel_kind(name: str):
    """The pass a kernel name in a rocprofv3 trace belongs to (None: not ours)."""
    if "chunk_kernel" in name:
        return {"0": "output", "1": "segment", "4": "states"}.get(name.split(",")[3].strip(" >")[:1])
    if "state_kernel" in name:   # 4th template argument: the backward's segment pass
        return "bwd_segment" if name.split(",")[3].strip(" >)(").startswith("true") else "segment"
    if "scan_kernel" in name:
        return "scan"
    if "decode_kernel" in name:
        return "decode"
    if "gdn_walk_kernel" in name:
        return "gdn_walk"
    if "gdn_kernel" in name:
        return "gdn_prep" if "true" in name else "gdn"
    if "bwd_kernel" in name:
        return "bwd" if name.split(",")[3].strip(" >)(")[:1] == "1" else "bwd_segment"
    return None


def summarize_counters(outdir: str, wl_name: str):
    """Parse rocprofv3 counter-collection CSVs (one pass for FETCH_SIZE, one
    for WRITE_SIZE, each run with --copy-calibration) and write
    profiles/counters_<workload>.json.  The calibration copies are the device
    copies dispatched after the last chunk kernel."""
    import csv
    per_counter = {}
    for p in glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            rows = list(csv.DictReader(f))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        last_chunk = max((int(r["Dispatch_Id"]) for r in rows
                          if any(s in r["Kernel_Name"]
                                 for s in ("chunk_kernel", "state_kernel", "decode_kernel",
                                           "bwd_kernel", "gdn_kernel", "gdn_walk_kernel"))),
                         default=-1)
        for r in rows:
            name, ctr, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            kind = kernel_kind(name)
            if kind is None and "copyBuffer" in name and int(r["Dispatch_Id"]) > last_chunk:
                kind = "copy"
            if kind:
                per_counter.setdefault((kind, ctr), []).append(val)
    if not per_counter:
        raise SystemExit(f"no counter rows under {outdir}")
    # medians over a kernel's dispatches; for the copies the largest one, the
    # calibration copy of COPY_BYTES (a parity check later in the run copies
    # smaller buffers)
    summary = {k[0] + ":" + k[1]: (max(v) if k[0] == "copy" else statistics.median(v))
               for k, v in per_counter.items()}
    out = {"workload": wl_name, "source_digest": source_digest(),
           "median_per_dispatch_KiB": summary, "copy_bytes": COPY_BYTES}
    cf, cw = summary.get("copy:FETCH_SIZE"), summary.get("copy:WRITE_SIZE")
    if cf and cw:
        out["fetch_factor"] = COPY_BYTES / (cf * 1024.0)
        out["write_factor"] = COPY_BYTES / (cw * 1024.0)
    path = os.path.join(ROOT, "profiles", f"counters_{wl_name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


# dense MFMA peaks of MI355X (TFLOP/s) and its SIMD count
MFMA_PEAK = {"bf16": 2500.0, "fp32": 157.3}
SIMDS = 1024


def summarize_mfma(outdirs):
    """Per-kernel MFMA figures from rocprofv3 counter CSVs under DIR (medians
    over dispatches), printed as a markdown table.  Expects a pass with
    SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE and a pass with
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 (one MOPS unit
    is 512 flops).  MFMA busy = busy cycles summed over SIMDs / (SIMDs x GPU
    active cycles, GRBM_GUI_ACTIVE summed over the 8 XCDs / 8); rates use
    each dispatch's own duration under counter collection."""
    import csv
    vals, durs = {}, {}
    paths = [p for d in outdirs
             for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)]
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                kind = kernel_kind(r["Kernel_Name"])
                if kind is None:
                    continue
                vals.setdefault((kind, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                durs.setdefault(kind, {})[(p, r["Dispatch_Id"])] = d
    if not vals:
        raise SystemExit(f"no counter rows under {outdirs}")
    med = {k: statistics.median(v) for k, v in vals.items()}
    print("| pass | dispatch us | MFMA instructions | busy cycles each | MFMA busy | "
          "bf16 TFLOP/s (of 2500) | fp32 TFLOP/s (of 157.3) |")
    print("|---|---|---|---|---|---|---|")
    out = {}
    for kind in sorted(durs):
        d = statistics.median(durs[kind].values())
        g = lambda c: med.get((kind, c))
        ins, busy, gui = g("SQ_INSTS_MFMA"), g("SQ_VALU_MFMA_BUSY_CYCLES"), g("GRBM_GUI_ACTIVE")
        util = busy / (SIMDS * gui / 8) if busy is not None and gui else None
        rate = {}
        for dt, c in (("bf16", "SQ_INSTS_VALU_MFMA_MOPS_BF16"), ("fp32", "SQ_INSTS_VALU_MFMA_MOPS_F32")):
            if g(c) is not None:
                rate[dt] = g(c) * 512 / d / 1e12
        out[kind] = {"dispatch_us": d * 1e6, "insts": ins, "busy": busy, "util": util, **rate}
        f = lambda x, s: "—" if x is None else s.format(x)
        fr = lambda dt: "—" if dt not in rate else f"{rate[dt]:.1f} ({rate[dt] / MFMA_PEAK[dt]:.3f})"
        print(f"| {kind} | {d * 1e6:.1f} | {f(ins, '{:.0f}')} | "
              f"{f(busy / ins if busy is not None and ins else None, '{:.1f}')} | "
              f"{f(util, '{:.3f}')} | {fr('bf16')} | {fr('fp32')} |")
    return out


SWEEPS = {
    # sequence-length doubling at B = 1, H = 16 (the evaluation page's short
    # vs long T comparison)
    "t_doubling": [(1, t) for t in (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)],
    # batch against length at equal total tokens (B * T = 65536, H = 16)
    "equal_tokens": [(1, 65536), (4, 16384), (16, 4096), (64, 1024), (256, 256)],
}


def bench_sweep(args):
    """Scaling curves ("面向长序列大模型的线性注意力算子性能评测方法与优化实践", section
    六.2: throughput as T doubles, and batch against length at equal total
    tokens): the prefill_4k distributions at each (B, T), H = 16, D = 128, one
    gla_fwd per step, two input sets alternating.  Prints one JSON object
    with a point per shape."""
    import dataclasses

    import torch

    import chunked_state_recurrence_amd as gla
    from chunked_state_recurrence_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    gla.set_tuning(0, 0)
    base = WORKLOADS["prefill_4k"]
    points = []
    for B, T in SWEEPS[args.sweep]:
        wl = dataclasses.replace(base, name=f"B{B}_T{T}", B=B, T=T)
        host = make_inputs(wl)
        sets = []
        for s_ in range(2):
            d = {n: host[n].to(dev) for n in ("q", "k", "v", "g")}
            if s_ == 1:
                d = {n: t.clone() for n, t in d.items()}
            d["o"] = torch.empty(B, wl.H, T, wl.D, dtype=torch.bfloat16, device=dev)
            sets.append(d)
        stream = torch.cuda.current_stream()

        def step(i):
            d = sets[i & 1]
            gla.gla_fwd(d["q"], d["k"], d["v"], d["g"], None, o=d["o"], stream=stream)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        gla.profile_start(8 * args.steps + 8)
        for i in range(args.steps):
            step(i)
        kern = {}
        for kind, kms in gla.profile_stop():
            kern[kind] = kern.get(kind, 0.0) + kms / args.steps
        nbytes = algorithmic_bytes(wl)
        points.append({"B": B, "H": wl.H, "T": T, "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
                       "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "kernels_ms_per_step": kern})
        print(f"B={B} T={T}: {ms * 1e3:.1f} us, {B * T / (ms * 1e-3):.3e} tok/s, "
              f"HBM frac {points[-1]['hbm_frac']:.3f}, " +
              ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in kern.items()), file=sys.stderr, flush=True)
        del sets, host
        torch.cuda.empty_cache()
    emit({"sweep": args.sweep, "metric": METRIC, "unit": "tokens/s", "dtype": "bf16",
          "data": "synthetic", "steps": args.steps, "warmup": args.warmup, "points": points})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_16k")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--target-wgs", type=int, default=0)
    ap.add_argument("--head-group", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-parity", action="store_true", help="skip the one-sequence parity check")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--summarize-mfma", metavar="DIR", nargs="+")
    ap.add_argument("--backward", action="store_true", help="time gla_bwd on the workload")
    ap.add_argument("--sweep", choices=sorted(SWEEPS), help="scaling curve instead of one workload")
    args = ap.parse_args()

    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters,
                           args.workload + ("_bwd" if args.backward else ""))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode: heads would shard across GPUs with no "
              "communication, a sequence split would exchange one segment state per GPU)",
              file=sys.stderr)
        sys.exit(2)

    if not (args.no_cpu and args.no_parity):
        # the oracle (CPU baseline, parity sample) is compiled here if it is
        # missing, before anything touches the GPU
        from oracle.reference import ensure_built
        ensure_built()

    if args.sweep:
        bench_sweep(args)
        return

    import torch

    import chunked_state_recurrence_amd as gla
    from chunked_state_recurrence_amd.workloads import (DECODE_WORKLOADS, GDN_WORKLOADS,
                                                        SCALAR_WORKLOADS, WORKLOADS, make_inputs)

    if args.workload in DECODE_WORKLOADS:
        bench_decode(args, DECODE_WORKLOADS[args.workload])
        return
    if args.workload in GDN_WORKLOADS:
        bench_gdn(args, GDN_WORKLOADS[args.workload])
        return
    wl = {**WORKLOADS, **SCALAR_WORKLOADS}[args.workload]
    if args.backward:
        if wl.scalar_gate or wl.dtype != "bf16":
            raise SystemExit("--backward measures the bf16 per-key-dim workloads")
        bench_backward(args, wl)
        return
    fp32 = wl.dtype == "f32"
    fwd = gla.gla_fwd_scalar if wl.scalar_gate else gla.gla_fwd_f32 if fp32 else gla.gla_fwd
    dev = torch.device("cuda:0")
    gla.set_tuning(args.target_wgs, args.head_group)
    chunk = args.chunk or 64

    host = make_inputs(wl)
    sets = []
    for s in range(2):
        d = {n: (None if host[n] is None else host[n].to(dev)) for n in ("q", "k", "v", "g", "h0")}
        if s == 1:  # a second, independent copy of the same inputs
            d = {n: (None if t is None else t.clone()) for n, t in d.items()}
        d["o"] = torch.empty(wl.B, wl.H, wl.T, wl.D, dtype=torch.float32 if fp32 else torch.bfloat16,
                             device=dev)
        d["hf"] = (torch.empty(wl.B, wl.H, wl.D, wl.D, dtype=torch.float32, device=dev)
                   if wl.want_final else None)
        sets.append(d)
    stream = torch.cuda.current_stream()

    def step(i):
        d = sets[i & 1]
        fwd(d["q"], d["k"], d["v"], d["g"], d["h0"], chunk=chunk, scale=wl.scale,
            o=d["o"], h_final=d["hf"], want_final=wl.want_final, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1 (the headline): K steps between two synchronisations,
    # bracketed by one pair of HIP events and nothing else in between
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps

    # timed region 2: the same K steps with one event between steps (no
    # library tracing) for the latency percentiles
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))

    # timed region 3: the library's per-launch HIP-event tracing on its launch
    # stream (kernel durations); those events sit between kernels, so this
    # region's step time is reported apart from the headline
    gla.profile_start(8 * args.steps + 8)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    kernels = gla.profile_stop()
    traced_wall_ms = (time.perf_counter() - t3) * 1e3 / args.steps

    if args.copy_calibration:
        copy_calibration(dev)

    by_kind = {}
    for kind, kms in kernels:
        by_kind.setdefault(kind, []).append(kms)
    kernels_ms = {k: statistics.mean(v) for k, v in by_kind.items()}
    kernels_ms_per_step = {k: sum(v) / args.steps for k, v in by_kind.items()}
    # the dominant kernel: the one with the most device time per step
    dom = max(kernels_ms_per_step, key=kernels_ms_per_step.get)
    dom_launches = len(by_kind[dom]) / args.steps
    dom_ms = kernels_ms_per_step[dom]
    bytes_alg = algorithmic_bytes(wl)
    flops = algorithmic_flops(wl, chunk)
    achieved_call = bytes_alg / (ms * 1e-3) / 1e9
    dom_bytes = pass_bytes(wl, dom)
    traffic_call, traffic_dom = None, None
    c = read_counters(args.workload)
    if c and "fetch_factor" in c:   # counters are per dispatch: one launch per pass and step
        m = c["median_per_dispatch_KiB"]
        tot, ok = 0.0, True
        for k in kernels_ms_per_step:
            f, w = m.get(f"{k}:FETCH_SIZE"), m.get(f"{k}:WRITE_SIZE")
            if f is None or w is None or len(by_kind[k]) != args.steps:
                ok = False
                break
            b_k = f * 1024 * c["fetch_factor"] + w * 1024 * c["write_factor"]
            tot += b_k
            if k == dom:
                traffic_dom = int(b_k)
        traffic_call = int(tot) if ok else None

    # parity of this run: one (batch, head) sequence of the last output of
    # input set 0 against the oracle
    parity = None
    if not args.no_parity:
        import numpy as np
        import oracle
        from chunked_state_recurrence_amd.workloads import to_f64_numpy
        sel = {n: (None if host[n] is None else to_f64_numpy(host[n][:1, :1])) for n in
               ("q", "k", "v", "g", "h0")}
        if wl.scalar_gate:
            ro, rh, *_ = (*oracle.scalar_gate_recurrence(sel["q"], sel["k"], sel["v"], sel["g"],
                                                         sel["h0"], wl.scale),)
        else:
            ro, rh, _ = oracle.token_recurrence(sel["q"], sel["k"], sel["v"], sel["g"], sel["h0"],
                                                wl.scale)
        got = sets[0]["o"][:1, :1].float().cpu().numpy()
        err = float(np.max(np.abs(got - ro)) / max(float(np.max(np.abs(ro))), 1e-30))
        parity = {"max_norm_err": err, "tolerance": 1e-3 if fp32 else 1e-2,
                  "sample": "(batch 0, head 0), whole sequence, against the fp64 oracle"}
        if wl.want_final:
            gh = sets[0]["hf"][:1, :1].cpu().numpy()
            parity["h_final_max_norm_err"] = float(np.max(np.abs(gh - rh)) /
                                                   max(float(np.max(np.abs(rh))), 1e-30))

    io_bytes = sum(t.numel() * t.element_size() for t in sets[0].values() if t is not None)
    res = {
        "metric": SCALAR_METRIC if wl.scalar_gate else F32_METRIC if fp32 else METRIC,
        "value": wl.B * wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "K": wl.D, "V": wl.D,
                   "chunk": chunk, "h_final": wl.want_final, "h0": wl.h0_std is not None,
                   "gate": "scalar [B,H,T]" if wl.scalar_gate else "per key dim [B,H,T,K]",
                   "parallelism": "single GPU"},
        # the whole gla_fwd call (every launch of the path) priced against HBM
        # bandwidth with the workload's algorithmic bytes; the dominant
        # kernel's own figure follows under "dominant_kernel"
        "roofline": {"bound": "hbm", "achieved": achieved_call, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_call / HBM_PEAK_GBS, "traffic": traffic_call,
                     "scope": "whole gla_fwd call (ms_per_step)",
                     "algorithmic_bytes_per_call": bytes_alg,
                     "dominant_kernel": {
                         "kind": dom, "kernel": KIND_NAMES.get(dom, dom),
                         "launches_per_step": dom_launches, "kernel_ms": dom_ms,
                         "algorithmic_bytes_per_launch": dom_bytes,
                         "achieved": (dom_bytes / (dom_ms * 1e-3) / 1e9) if dom_bytes else None,
                         "frac": (dom_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if dom_bytes else None,
                         "traffic": traffic_dom}},
        "whole_path": {"hbm_frac": bytes_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "mfma_tflops": flops / (ms * 1e-3) / 1e12,
                       "mfma_frac": flops / (ms * 1e-3) / 1e12 / (MFMA_F32_PEAK_TFLOPS if fp32
                                                                  else MFMA_BF16_PEAK_TFLOPS),
                       "algorithmic_bytes": bytes_alg, "algorithmic_flops": flops},
        "kernels_ms": kernels_ms,
        "kernels_ms_per_step": kernels_ms_per_step,
        "traced_step_ms": traced_wall_ms,
        "latency_ms": {"source": "untraced steps with one event between steps",
                       "mean": statistics.mean(per_step), "p50": statistics.median(per_step),
                       "p95": per_step[min(len(per_step) - 1, int(0.95 * len(per_step)))],
                       "p99": per_step[min(len(per_step) - 1, int(0.99 * len(per_step)))]},
        "memory": {"io_bytes_per_call": io_bytes, "library_workspace_bytes": gla.workspace_bytes(),
                   "torch_peak_bytes": torch.cuda.max_memory_allocated(dev),
                   "note": "io: q, k, v, g, h0, o, h_final of one input set; the bench holds two sets"},
        "parity": parity,
        "env": environment(),
    }
    if wl.name in PAGES_TOKENS_PER_S:
        res["vs_baseline"] = res["value"] / PAGES_TOKENS_PER_S[wl.name]
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, host)
    emit(res)


if __name__ == "__main__":
    main()
