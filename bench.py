#!/usr/bin/env python3
"""Benchmark of the VLA forward recurrence on one MI355X.

One step = one ``vla_forward`` over the whole batch of the d_h = 64, T = 4096
workload (B = 8, H = 16, bf16 q/k/v/u, fp32 state), writing o and the final
S, A and zkey.  Inputs are resident in HBM before the timed region.

Warm-up: the --warmup steps, extended until the forward has run for at least
SETTLE_S seconds (the device clocks take some tens of milliseconds to settle).

Prints ONE JSON line with the throughput in tokens*heads/s, the percentage of
the MI355X FP32 peak, a roofline record for the forward (algorithmic FLOP /
average time of its launches from HIP events on the launch stream; the kernels
do their d x d products on fp32 matrix cores, whose dense peak equals the FP32
vector peak), the same for each of its two passes (penalty: Grams, segment
inverses and the penalty chain; memory: the memory chain and readout), and the
fp64 CPU oracle timed on the host cores over a bounded sample of heads.
Beside it (key ``workloads``): the forward time and fraction of peak of every
other workload (single head d_h = 16; 32 heads d_h = 64 T = 1024; the
MQAR-shaped 128 heads d_h = 96 T = 16384; 64 heads d_h = 128 T = 65536 bf16)
and the long-context workload's 4096-step ``vla_step`` continuation from its
forward's final state, in microseconds per step and GB/s of state traffic.
Also (key ``baselines``) the pages' comparison models on the headline inputs:
cumulative-sum linear attention and DeltaNet, their time against the forward's,
and the state-norm contrast |S_T|_F of the three on the recall-shaped recipe.

``--backward`` prints the same kind of line for ``vla_backward`` (gradients of
q, k, v, u and the initial state for a synthetic dL/do) on the same workload,
``--scan`` for ``vla_forward_scan`` (the memory chain as a scan over chunks, a
comparison); neither is part of the default run.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VLA fwd tokens·heads/sec (fp32 state) + % of MI355X FP32 vector peak"
UNIT = "tokens*heads/s"
SETTLE_S = 0.25                         # minimum warm-up time of the timed kernel
FP32_VECTOR_PEAK_TFLOPS = 157.3          # MI355X published FP32 vector (and dense fp32 matrix) peak
WORKLOAD = 3                              # B=8, H=16, d_h=64, T=4096, bf16 inputs
KERNEL_SOURCES = ["long_context_sequence_amd/csrc/vla_twopass.hip",
                  "long_context_sequence_amd/csrc/vla_chunk_parts.h",
                  "long_context_sequence_amd/csrc/vla_dpp_blocks.h",
                  "long_context_sequence_amd/csrc/vla_common.h",
                  "long_context_sequence_amd/csrc/vla_record.h",
                  "long_context_sequence_amd/csrc/vla_sweep.h"]
TRAFFIC_SUMMARY = "profiles/vla_forward_b8h16_d64_t4096_bf16.txt"
# the backward call: the two-pass forward keeping the per-token records, then the
# reverse sweep (vla_bwd_sync_init, vla_bwd_sweep)
BWD_KERNEL_SOURCES = KERNEL_SOURCES + ["long_context_sequence_amd/csrc/vla_bwd.hip",
                                       "long_context_sequence_amd/csrc/vla_bwd_split.hip",
                                       "long_context_sequence_amd/csrc/vla_bwd.h",
                                       "long_context_sequence_amd/csrc/vla_reduce.h"]
BWD_TRAFFIC_SUMMARY = "profiles/vla_backward_b8h16_d64_t4096_bf16.txt"
COPY_BYTES = 1 << 30                      # plain copy used to scale the HBM counters


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(summary=TRAFFIC_SUMMARY, sources=None):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by a plain copy of known size), or
    None if there is none or the kernel source changed since."""
    path = os.path.join(ROOT, summary)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"^kernel_source_sha256:\s*([0-9a-f]+)", txt, re.M)
    m_traf = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_hash or not m_traf or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_traf.group(1))


def device_peak_tflops():
    """FP32 peak recomputed from the device: compute units x clock x 256 FLOP per
    clock per CU (the figure behind the published 157.3 TFLOP/s), or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    # hipDeviceAttributeMultiprocessorCount = 63, hipDeviceAttributeClockRate = 5 (kHz)
    if hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, 0) != 0:
        return None
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) != 0:
        return None
    return {"cus": cus.value, "clock_mhz": khz.value / 1e3,
            "tflops": cus.value * khz.value * 1e3 * 256 / 1e12}


def attainable_peak_tflops():
    """Attainable fp32 throughput measured on this device by the probe library
    (libvla_peak.so): the fp32 MFMA the kernels use and the plain (unpacked)
    fp32 vector FMA, each one launch filling every compute unit, or None."""
    import ctypes
    path = os.path.join(ROOT, "long_context_sequence_amd", "libvla_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.vla_peak_probe.restype = ctypes.c_int
    lib.vla_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    out = {}
    for kind, name, iters in ((0, "mfma_f32_16x16x4", 4000), (1, "valu_fma_f32_unpacked", 8000)):
        v = ctypes.c_double(0.0)
        out[name] = v.value if lib.vla_peak_probe(kind, iters, ctypes.byref(v)) == 0 else None
    return out


def flops_per_token_head(d: int) -> int:
    """Algorithmic work of one token of one head: the matrix-vector products
    A u^, A k^, S k^ and S phi(q) (2 d^2 each) and the rank-1 updates of A and
    S (2 d^2 each); O(d) terms are not counted."""
    return 12 * d * d


def backward_flops_per_token_head(d: int) -> int:
    """Algorithmic work of the reverse mode per token of one head: the forward it
    must recompute (12 d^2) and the reverse products: dS updates from the
    readout and from e (2 d^2 each), dS alpha^, dS'e, S_t'g, S_{t-1}'ge, the
    updates of dA by gy k^' and gz u^', A_t gy, (dA + dA')z counted as two
    products, and A_{t-1} gz (2 d^2 each): 36 d^2 in all."""
    return 36 * d * d


def tok_heads_total(cfg) -> int:
    return cfg.B * cfg.H * cfg.T


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (e.g. under a profiler)")
    p.add_argument("--headline-only", action="store_true",
                   help="time only the headline workload (skip the other workloads and the "
                        "decode continuation)")
    p.add_argument("--cpu-heads", type=int, default=0,
                   help="heads in the CPU-baseline sample (0 = every head of the workload)")
    p.add_argument("--scan", action="store_true",
                   help="time vla_forward_scan (memory chain as a scan over chunks) instead")
    p.add_argument("--scan-crossover", action="store_true",
                   help="time vla_forward against vla_forward_scan on the d_h = 128, T = 65536 "
                        "head shape for the head counts in --scan-heads")
    p.add_argument("--scan-heads", default="1,2,4,8,16,64")
    p.add_argument("--scan-reps", type=int, default=5)
    p.add_argument("--backward", action="store_true",
                   help="time vla_backward (gradients) on the same workload instead")
    p.add_argument("--decode", action="store_true",
                   help="only the long-context workload's decode continuation (its forward "
                        "once for the state, then the vla_step tokens), its own JSON line")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    return p.parse_args()


def calibrate_copy(reps: int = 3):
    """A plain device-to-device copy of COPY_BYTES, for scaling FETCH_SIZE /
    WRITE_SIZE counter readings to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "reps": reps}), flush=True)


def cpu_baseline(cfg, n_heads_req: int):
    """fp64 oracle on the host cores over a bounded sample of whole heads of the
    same workload (each head is an independent T-token sequence)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import gen
    import oracle

    cores = oracle.default_workers()
    n_heads = min(n_heads_req or cfg.B * cfg.H, cfg.B * cfg.H)
    heads = [divmod(i, cfg.H) for i in range(n_heads)]
    inputs = []
    for b, h in heads:
        hi = gen.head_inputs(cfg, b, h)
        inputs.append([hi[n].astype(np.float64) for n in "qkvu"])
    used = min(cores, n_heads)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=used) as ex:
        list(ex.map(lambda a: oracle.forward_head(*a, cfg.lambda0, cfg.eps), inputs))
    wall = time.perf_counter() - t0
    return {"value": n_heads * cfg.T / wall, "unit": UNIT, "cores": used, "kind": "oracle",
            "sample": f"{n_heads} of {cfg.B * cfg.H} heads, T={cfg.T}, d_h={cfg.d}, fp64, "
                      f"wall {wall:.2f} s"}


def cpu_baseline_backward(cfg, n_heads: int, dO):
    """fp64 oracle of the gradients over a bounded sample of whole heads."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import gen
    import oracle

    cores = oracle.default_workers()
    heads = [divmod(i, cfg.H) for i in range(n_heads)]
    args = []
    for b, h in heads:
        hi = gen.head_inputs(cfg, b, h)
        args.append([hi[n].astype(np.float64) for n in "qkvu"] + [dO[b, h].astype(np.float64)])
    used = min(cores, n_heads)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=used) as ex:
        list(ex.map(lambda a: oracle.backward_head(*a, cfg.lambda0, cfg.eps), args))
    wall = time.perf_counter() - t0
    return {"value": n_heads * cfg.T / wall, "unit": UNIT, "cores": used, "kind": "oracle",
            "sample": f"{n_heads} of {cfg.B * cfg.H} heads, T={cfg.T}, d_h={cfg.d}, fp64 "
                      f"reverse mode, wall {wall:.2f} s"}


def backward_bench(args):
    """One step = one vla_backward over the whole batch of the same workload:
    dL/do given (synthetic), gradients of q, k, v, u and of the initial state
    written; the forward is recomputed inside."""
    import numpy as np
    import torch

    import gen
    import long_context_sequence_amd as vla

    cfg = gen.config(WORKLOAD)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    dev = torch.device("cuda:0")
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).view(torch.bfloat16) for n in "qkvu"}
    dO_host = np.random.default_rng(WORKLOAD).standard_normal((B, H, T, d)).astype(np.float32)
    dO = torch.from_numpy(dO_host).to(dev)
    ws = torch.empty(vla.backward_workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        vla.vla_backward(t["q"], t["k"], t["v"], t["u"], dO, cfg.lambda0, cfg.eps,
                         workspace=ws, stream=stream)

    t_w, n_w = time.perf_counter(), 0
    while n_w < args.warmup or time.perf_counter() - t_w < SETTLE_S:
        step()
        n_w += 1
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s0, e0 in ev:
        s0.record(stream)
        step()
        e0.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s0.elapsed_time(e0) for s0, e0 in ev]
    kern_ms = float(np.mean(launch_ms))
    ms_per_step = wall * 1e3 / args.steps
    tok_heads = B * H * T
    flop = backward_flops_per_token_head(d) * tok_heads
    achieved = flop / (kern_ms / 1e3) / 1e12
    res = {
        "metric": "VLA backward tokens·heads/sec (gradients of q, k, v, u and the initial "
                  "state; fp32 state)",
        "value": tok_heads / (ms_per_step / 1e3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_run": n_w,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + " backward", "B": B, "H": H, "d_h": d, "T": T,
                   "input_dtype": cfg.dtype, "state_dtype": "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if d == 64 else "alu", "achieved": achieved,
                     "peak": FP32_VECTOR_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": measured_traffic(BWD_TRAFFIC_SUMMARY, BWD_KERNEL_SOURCES),
                     "kernel": "vla_backward call: vla_gram, vla_seginv, vla_pen, vla_mem "
                               "(keeping the per-token records), vla_bwd_sync_init, "
                               "vla_bwd_sweep (the two adjoint chains side by side)",
                     "kernel_ms": kern_ms,
                     "kernel_ms_median": float(np.median(launch_ms)), "flop_per_launch": flop,
                     "dtype": "fp32"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(cfg, args.cpu_heads or 32, dO_host)
    print(json.dumps(res), flush=True)


def scan_bench(args):
    """One step = one vla_forward_scan over the whole batch of the forward's
    workload (penalty pass, per-chunk maps, up- and down-sweep of the scan,
    chunk-local readout), for comparison with vla_forward."""
    import numpy as np
    import torch

    import gen
    import long_context_sequence_amd as vla

    cfg = gen.config(WORKLOAD)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    dev = torch.device("cuda:0")
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).view(torch.bfloat16) for n in "qkvu"}
    o = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    ws = torch.empty(vla.scan_workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        vla.vla_forward_scan(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, o=o,
                             workspace=ws, stream=stream)

    t_w, n_w = time.perf_counter(), 0
    while n_w < args.warmup or time.perf_counter() - t_w < SETTLE_S:
        step()
        n_w += 1
        if n_w % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s0, e0 in ev:
        s0.record(stream)
        step()
        e0.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = float(np.mean([s0.elapsed_time(e0) for s0, e0 in ev]))
    ms_per_step = wall * 1e3 / args.steps
    tok_heads = B * H * T
    flop = flops_per_token_head(d) * tok_heads
    nc = (T + 15) // 16
    n = 2
    while n < nc:
        n *= 2
    combine_flop = B * H * 2 * (n - 1) * 4 * d ** 3
    achieved = flop / (kern_ms / 1e3) / 1e12
    res = {
        "metric": "VLA fwd tokens·heads/sec with the memory chain as a scan over chunks "
                  "(fp32 state), for comparison with vla_forward",
        "value": tok_heads / (ms_per_step / 1e3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_run": n_w,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + " scan form", "B": B, "H": H, "d_h": d, "T": T,
                   "input_dtype": cfg.dtype, "state_dtype": "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": None, "kernel": "vla_forward_scan (penalty pass + scan kernels)",
                     "kernel_ms": kern_ms, "flop_per_launch": flop, "dtype": "fp32",
                     "scan_combine_flop_per_launch": combine_flop,
                     "scan_combine_tflops": combine_flop / (kern_ms / 1e3) / 1e12},
    }
    print(json.dumps(res), flush=True)


def scan_crossover(args):
    """The scan form where the pages expect it to pay: the long-context head
    shape (d_h = 128, T = 65536, bf16; the recipe of that workload) with few
    heads.  For each head count, vla_forward and vla_forward_scan are timed on
    the same inputs (HIP events on the launch stream, median of the repeats
    after a warm-up); one JSON line holds the table."""
    import numpy as np
    import torch

    import gen
    import long_context_sequence_amd as vla

    base = gen.config(5)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    for h in [int(v) for v in args.scan_heads.split(",")]:
        cfg = base.with_sizes(B=1, H=h, decode=0)
        B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
        x = gen.make_inputs(cfg)
        t = {n: torch.from_numpy(x[n]).to(dev).view(torch.bfloat16) for n in "qkvu"}
        del x
        o = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
        ws_f = torch.empty(vla.workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
        ws_s = torch.empty(vla.scan_workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)

        def fwd():
            vla.vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, o=o,
                            workspace=ws_f, stream=stream)

        def scan():
            vla.vla_forward_scan(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, o=o,
                                 workspace=ws_s, stream=stream)

        def timed(step):
            t_w, n_w = time.perf_counter(), 0
            while n_w < 2 or time.perf_counter() - t_w < 1.0:
                step()
                n_w += 1
                torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.scan_reps)]
            for e0, e1 in ev:
                e0.record(stream)
                step()
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

        f_ms, s_ms = timed(fwd), timed(scan)
        nc = (T + 15) // 16
        n = 2
        while n < nc:
            n *= 2
        comb = B * H * 2 * (n - 1) * 4 * d ** 3
        rows.append({"heads": B * H, "forward_ms": f_ms, "scan_ms": s_ms,
                     "scan_over_forward": s_ms / f_ms,
                     "forward_tokens_heads_per_s": B * H * T / (f_ms / 1e3),
                     "scan_tokens_heads_per_s": B * H * T / (s_ms / 1e3),
                     "scan_combine_flop": comb,
                     "scan_combine_tflops_if_all_time": comb / (s_ms / 1e3) / 1e12})
        print(json.dumps({"progress": rows[-1]}), flush=True)
        del t, o, ws_f, ws_s
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "VLA forward ms, chained memory pass against the scan over chunks (Eq. (12), "
                  "right-multiplication combine), few heads of the long-context shape",
        "config": {"workload": base.name + " head shape, B = 1, H = heads, no decode",
                   "d_h": base.d, "T": base.T, "input_dtype": base.dtype},
        "data": "synthetic", "rows": rows}), flush=True)


def _time_forward(vla, torch, cfg, x, reps):
    """Median and mean time of one vla_forward over the workload (events on the
    launch stream, after a warm-up of at least SETTLE_S seconds); returns them
    with the final state for a decode continuation."""
    import numpy as np
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(x[n]).to(dev) for n in "qkvu"}
    if cfg.dtype == "bf16":
        t = {n: a.view(torch.bfloat16) for n, a in t.items()}
    o = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    A = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    zk = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(vla.workspace_size(B, H, T, d), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        vla.vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, o=o, S_out=S,
                        A_out=A, zkey_out=zk, stream=stream, workspace=ws)
    t_w, n_w = time.perf_counter(), 0
    while n_w < 3 or time.perf_counter() - t_w < SETTLE_S:
        step()
        n_w += 1
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    del t, o, ws
    return float(np.median(ms)), float(np.mean(ms)), (S, A, zk)


def _fwd_record(cfg, ms):
    tok_heads = tok_heads_total(cfg)
    tf = flops_per_token_head(cfg.d) * tok_heads / (ms / 1e3) / 1e12
    return {"B": cfg.B, "H": cfg.H, "d_h": cfg.d, "T": cfg.T, "input_dtype": cfg.dtype,
            "ms": ms, "tokens_heads_per_s": tok_heads / (ms / 1e3), "achieved_tflops": tf,
            "frac": tf / FP32_VECTOR_PEAK_TFLOPS}


def decode_continuation(vla, torch, cfg, x, state):
    """cfg.decode single-token steps (vla_step) continuing from the forward's
    final state, on the workload's decode tokens.  Each step reads and writes
    the fp32 state (S, A: d^2 each, zkey: d) of every head and reads its four
    input vectors; the state traffic is reported against the HBM peak.

    Timed two ways over the same steps: captured once in a HIP graph (one kernel
    node per token, as a serving loop launches them; us_per_step) and launched
    one Python call per token (us_per_step_eager, bound by the host's launch
    rate).  The state is reset to the forward's final state before each."""
    B, H, d, n = cfg.B, cfg.H, cfg.d, cfg.decode
    dev = torch.device("cuda:0")
    S, A, zk = (a.clone() for a in state)
    dec = {}
    for nm in "qkvu":
        a = torch.from_numpy(x[nm + "_dec"]).to(dev)
        a = a.view(torch.bfloat16) if cfg.dtype == "bf16" else a
        dec[nm] = a.permute(2, 0, 1, 3).contiguous()   # [steps, B, H, d]
    o = torch.empty((n, B, H, d), dtype=torch.float32, device=dev)

    def reset():
        for dst, src in zip((S, A, zk), state):
            dst.copy_(src)
        torch.cuda.synchronize()

    def run(i):
        vla.vla_step(dec["q"][i], dec["k"][i], dec["v"][i], dec["u"][i], S, A, zk, cfg.eps,
                     o=o[i], stream=torch.cuda.current_stream())

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(8):   # warm-up
        run(i)
    reset()
    e0.record()
    for i in range(n):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) * 1e3 / n
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(n):
                run(i)
    reset()
    graph.replay()   # warm-up replay
    reset()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    del graph
    s_in = 2 if cfg.dtype == "bf16" else 4
    state_bytes = B * H * (2 * (2 * d * d + d) * 4 + 4 * d * s_in + d * 4)
    gbps = state_bytes / (us * 1e-6) / 1e9
    return {"steps": n, "from": f"the forward's final state after T={cfg.T}",
            "us_per_step": us, "launch": "HIP graph, one node per token",
            "us_per_step_eager": us_eager, "tokens_heads_per_s": B * H / (us * 1e-6),
            "bytes_per_step": state_bytes, "GBps": gbps, "hbm_frac": gbps / 8000.0}


def baselines(vla, torch, vla_ms):
    """The pages' comparison models on the headline workload's inputs: the
    cumulative-sum linear attention and DeltaNet (gate 1 on the unit key), each
    one vla_baseline_forward call (per-chunk records, then the forward's memory
    pass), timed like the forward; VLA's time over theirs; and the state-norm
    contrast of section 4.1 on the recall-shaped recipe: |S_T|_F (mean over
    heads) after T tokens for the three layers."""
    import numpy as np
    import gen
    cfg = gen.config(WORKLOAD)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    dev = torch.device("cuda:0")
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).view(torch.bfloat16) for n in "qkv"}
    o = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    zk = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = torch.empty(vla.baseline_workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    out = {"workload": cfg.name, "vla_ms": vla_ms}
    for kind, per_tok in (("linear", 4), ("delta", 6)):
        def step():
            vla.vla_baseline(kind, t["q"], t["k"], t["v"], 1.0, cfg.eps, o=o, S_out=S,
                             zkey_out=zk, workspace=ws, stream=stream)
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < SETTLE_S:
            step()
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(20)]
        for e0, e1 in ev:
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
        out[kind] = {"ms": ms, "tokens_heads_per_s": B * H * T / (ms / 1e3),
                     "vla_time_ratio": vla_ms / ms,
                     "flop_per_token_head": per_tok * d * d,
                     "vla_flop_ratio": 12 / per_tok}
    del t, o, ws
    rc = gen.config(4).with_sizes(B=1, H=8, T=4096)
    xr = gen.make_inputs(rc)
    tr = {n: torch.from_numpy(xr[n]).to(dev) for n in "qkvu"}
    norms = {"workload": f"recall-shaped, B=1, H=8, d_h={rc.d}", "T": [], "linear": [],
             "delta": [], "vla": []}
    for Tn in (256, 1024, 4096):
        sl = {n: tr[n][:, :, :Tn].contiguous() for n in "qkvu"}
        _, s_la, _ = vla.vla_baseline("linear", sl["q"], sl["k"], sl["v"], return_state=True)
        _, s_dn, _ = vla.vla_baseline("delta", sl["q"], sl["k"], sl["v"], return_state=True)
        _, s_v, _, _ = vla.vla_forward(sl["q"], sl["k"], sl["v"], sl["u"], return_state=True)
        torch.cuda.synchronize()
        norms["T"].append(Tn)
        for key, sv in (("linear", s_la), ("delta", s_dn), ("vla", s_v)):
            norms[key].append(float(sv.norm(dim=(-2, -1)).mean()))
    out["state_norm"] = norms
    return out


def decode_bench():
    """The long-context workload's forward once (for the state), then its
    decode tokens as in decode_continuation; one JSON line."""
    import torch

    import gen
    import long_context_sequence_amd as vla
    cfg = gen.config(5)
    x = gen.make_inputs(cfg)
    _, _, state = _time_forward(vla, torch, cfg, x, 1)
    dec = decode_continuation(vla, torch, cfg, x, state)
    print(json.dumps({
        "metric": "VLA decode step, µs per token for all heads (fp32 state)",
        "value": dec["us_per_step"], "unit": "us", "n_gpus": 1, "higher_is_better": False,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + " decode", "B": cfg.B, "H": cfg.H, "d_h": cfg.d,
                   "input_dtype": cfg.dtype, "state_dtype": "f32"},
        "decode": dec}), flush=True)


def other_workloads(vla, torch):
    """Forward time of each workload other than the headline one (parity
    cases, reported beside it), and the long-context workload's decode
    continuation."""
    import gen
    out = {}
    for cid, reps in ((1, 20), (2, 20), (4, 5), (5, 5)):
        cfg = gen.config(cid)
        x = gen.make_inputs(cfg)
        med, _, state = _time_forward(vla, torch, cfg, x, reps)
        rec = _fwd_record(cfg, med)
        if cfg.decode:
            rec["decode"] = decode_continuation(vla, torch, cfg, x, state)
        out[cfg.name] = rec
        del x, state
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the heads would shard across GPUs with no communication between them.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.backward:
        backward_bench(args)
        return
    if args.scan_crossover:
        scan_crossover(args)
        return
    if args.scan:
        scan_bench(args)
        return
    if args.decode:
        decode_bench()
        return

    import numpy as np
    import torch

    import gen
    import long_context_sequence_amd as vla

    cfg = gen.config(WORKLOAD)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    dev = torch.device("cuda:0")
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).view(torch.bfloat16) for n in "qkvu"}
    o = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    A = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    zk = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = torch.empty(vla.workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        vla.vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps,
                        o=o, S_out=S, A_out=A, zkey_out=zk, stream=stream, workspace=ws)

    # warm-up: the W steps asked for, continued until the device has run this
    # work for SETTLE_S seconds (its clocks take some tens of milliseconds to
    # settle after an idle period)
    t_w = time.perf_counter()
    n_w = 0
    while n_w < args.warmup or time.perf_counter() - t_w < SETTLE_S:
        step()
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    launch_ms = [s.elapsed_time(e) for s, e in ev]
    kern_ms = float(np.mean(launch_ms))

    # the two passes, timed apart on the same stream
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e0, e1, e2 in pev:
        e0.record(stream)
        vla.vla_forward_penalty(t["q"], t["k"], t["u"], cfg.lambda0, cfg.eps, workspace=ws,
                                A_out=A, zkey_out=zk, stream=stream)
        e1.record(stream)
        vla.vla_forward_memory(t["v"], workspace=ws, o=o, S_out=S, stream=stream)
        e2.record(stream)
    torch.cuda.synchronize()
    pen_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in pev]))
    mem_ms = float(np.mean([b.elapsed_time(c) for _, b, c in pev]))
    half = flops_per_token_head(d) // 2 * tok_heads_total(cfg)

    def phase(ms):
        tf = half / (ms / 1e3) / 1e12
        return {"ms": ms, "achieved": tf, "frac": tf / FP32_VECTOR_PEAK_TFLOPS,
                "flop_per_launch": half}
    ms_per_step = wall * 1e3 / args.steps
    tok_heads = B * H * T
    value = tok_heads / (ms_per_step / 1e3)
    flop = flops_per_token_head(d) * tok_heads
    achieved_tflops = flop / (kern_ms / 1e3) / 1e12
    pct_peak = 100.0 * (flop / (ms_per_step / 1e3) / 1e12) / FP32_VECTOR_PEAK_TFLOPS

    res = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": n_w,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "H": H, "d_h": d, "T": T,
                   "input_dtype": cfg.dtype, "state_dtype": "f32",
                   "lambda0": cfg.lambda0, "eps": cfg.eps, "parallelism": "single GPU"},
        "pct_fp32_vector_peak": pct_peak,
        "roofline": {"bound": "mfma", "achieved": achieved_tflops,
                     "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_tflops / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": measured_traffic(),
                     "kernel": "vla_forward: vla_gram, vla_seginv, vla_pen, vla_mem launches",
                     "kernel_ms": kern_ms, "kernel_ms_median": float(np.median(launch_ms)),
                     "flop_per_launch": flop, "dtype": "fp32",
                     "phases": {"penalty (vla_gram+vla_seginv+vla_pen; A u^, A k^, A update)":
                                phase(pen_ms),
                                "memory (vla_mem; S k^, S phi(q), S update)": phase(mem_ms)}},
        "device_peak": device_peak_tflops(),
        "attainable_peak_tflops": attainable_peak_tflops(),
    }
    if not args.headline_only:
        res["baselines"] = baselines(vla, torch, kern_ms)
        res["workloads"] = other_workloads(vla, torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_heads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
