#!/usr/bin/env python3
"""Attention forward+backward throughput on one MI355X, reported as one JSON line.

A step is one pass of the whole path over one batch: ``fa_fwd`` (O and lse)
then ``fa_bwd`` (D pre-pass, dK/dV, dQ), on inputs already resident in device
memory. The default workload is the long-context causal case the headline
metric is quoted on: B=1, H=32, N=16384, d=128, bf16, causal, synthetic N(0, 1/2)
inputs. Work is counted as dense attention FLOPs: 4*B*H*N^2*d forward, halved
for causal, and 2.5x that for backward.

Besides the step rate the line carries:
  * ``kernels``: each kernel timed alone with HIP events on the launch stream
    (average over --kernel-reps launches) against its algorithmic work, and
    the HBM rate its algorithmic bytes imply (every input read once, every
    output written once), the figure that matters for short sequences
    (``--workload gpt2m``);
  * ``roofline``: the kernel that takes longest per step, against the MI355X
    dense bf16 MFMA peak (or HBM bandwidth for the memory-bound pre-pass), with
    HBM traffic from the committed rocprofv3 counter summary when that summary
    was taken on the current kernel sources (else null);
  * ``cpu_baseline``: the fp64 CPU oracle timed on this host on the first
    heads of the same workload (forward + backward, about ten seconds);
  * ``memory``: device bytes the step allocates versus a materialised-score
    baseline that stores S and P;
  * ``env``: ROCm, compiler and torch versions, and the power and clock
    readings of amd-smi (or rocm-smi) taken while steps keep the GPU busy.
Per kernel, ``ms`` is the average over --kernel-reps back-to-back launches
(the figure the roofline uses, comparable with a rocprofv3 trace average);
``median_ms`` and ``min_ms`` come from as many launches timed one by one.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s, bf16 causal d=128, and % of MI355X MFMA peak"


def metric_label(w, has_bwd: bool) -> str:
    """The headline metric for the long causal workload; for any other workload a
    label of the same form that names what that line measures."""
    if w.name == "long_causal":
        return METRIC
    mask = ("causal" if w.causal else "non-causal") + (" ALiBi" if w.alibi else "")
    packed = ", packed sequences" if w.varlen else ""
    gqa = f", GQA {w.H}/{w.Hkv} heads" if w.Hkv != w.H else ""
    return (f"attention {'fwd/bwd' if has_bwd else 'fwd'} TFLOP/s, {w.dtype} {mask} d={w.d}{packed}{gqa} "
            f"({w.name}), and % of MI355X MFMA peak")
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2  # 256 CU x 8192 dense fp8 FLOP/clk x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "exact_io_aware_43_amd", "csrc")
KERNEL_SOURCES = {  # what each kernel's machine code depends on (the build flags included)
    "fwd": ["fa_fwd.hip", "fa_device.hpp", "fa_internal.hpp", "../build.py"],
    "bwd_dsum": ["fa_bwd.hip", "fa_device.hpp", "fa_internal.hpp", "../build.py"],
    "bwd_dkdv": ["fa_bwd_dkdv.hip", "fa_device.hpp", "fa_internal.hpp", "../build.py"],
    "bwd_dq": ["fa_bwd.hip", "fa_device.hpp", "fa_internal.hpp", "../build.py"],
}
# rocprofv3 kernel-name fragments of the four kernels
KERNEL_SYMBOLS = {"fwd": "fwd_mfma_kernel", "bwd_dsum": "bwd_dsum_kernel", "bwd_dkdv": "bwd_dkdv_kernel",
                  "bwd_dq": "bwd_dq_kernel"}
# plain elementwise copy used to calibrate the HBM byte counters: fp32 negation
# of COPY_BYTES into a second buffer reads and writes COPY_BYTES once each
COPY_BYTES = 1 << 30
COPY_SYMBOL = "neg_kernel"


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.normpath(os.path.join(CSRC, f)), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_causal")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the amd-smi reading under load (profiling runs: keeps the trace to the timed work)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="drop probability of the fused dropout (fa_fwd_dropout / fa_bwd_dropout); 0 = none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement run a plain 1 GiB fp32 copy (negation) for counter calibration")
    ap.add_argument("--counters-from", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs of this script (any counters, one or more directories) as "
                         "a per-kernel Markdown table (mean per dispatch) and exit; needs no GPU")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, both "
                         "with --copy-calibration) into profiles/traffic.json and exit; needs no GPU")
    return ap.parse_args()


def main():
    args = parse()
    if args.counters_from:
        print(summarise_counters(args.counters_from))
        return
    if args.traffic_from:
        summarise_traffic(args.workload, *args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention kernels run on a single device and this "
              "build has no multi-GPU path (no collectives, no sharding); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_43_amd as fa
    from exact_io_aware_43_amd.workloads import WORKLOADS, flops, make_inputs, seq_lengths

    if args.workload == "decode":
        bench_decode(args)
        return
    if args.workload.startswith("fp8"):
        bench_fp8(args)
        return
    w = WORKLOADS[args.workload]
    if w.dtype == "fp32":
        raise SystemExit(f"workload {w.name} is the fp32 latency case (one or two workgroups); it is a parity "
                         "case, not a throughput workload")
    has_bwd = bool(w.backward)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {w}", file=sys.stderr, flush=True)

    inp = make_inputs(w, args.seed, with_grad=True)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    if not has_bwd:
        do = None
    cu = inp["cu_seqlens"].to(dev) if inp["cu_seqlens"] is not None else None
    slopes = inp["alibi_slopes"].to(dev) if inp["alibi_slopes"] is not None else None
    lens = seq_lengths(inp, w)
    B, H, Hkv, N, d = w.B, w.H, w.Hkv, inp["max_seqlen"], w.d
    dt = {"bf16": fa.FA_BF16, "fp16": fa.FA_FP16}[w.dtype]
    scale = inp["scale"]
    causal = int(w.causal)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if has_bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = fa.fa_bwd_workspace_size(B, H, Hkv, N, d, causal, int(cu is not None), dt)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731

    drop = args.dropout
    fargs = lambda: (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d,  # noqa
                     scale, causal, P(slopes), P(cu), dt)

    def fwd():
        if drop:
            st = fa.fa_fwd_dropout(*fargs(), drop, args.seed + 1, 0, sh)
        else:
            st = fa.fa_fwd(*fargs(), sh)
        if st:
            raise fa.FaError(st)

    def bwd(stages=fa.FA_BWD_ALL):
        a_ = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
              dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, scale, causal, P(slopes), P(cu), dt)
        if drop:  # the dropout backward runs its three launches as one call
            st = fa.fa_bwd_dropout(*a_, drop, args.seed + 1, 0, ws.data_ptr(), ws_bytes, sh)
        else:
            st = fa.fa_bwd_stages(*a_, ws.data_ptr(), ws_bytes, stages, sh)
        if st:
            raise fa.FaError(st)

    def step():
        fwd()
        if has_bwd:
            bwd()

    step()
    torch.cuda.synchronize()
    lib_bytes = torch.cuda.max_memory_allocated() - mem0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s)", file=sys.stderr, flush=True)

    f_fwd = flops(w, lens)
    f_bwd = flops(w, lens, backward=True) if has_bwd else 0.0
    value = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12

    # ---- each kernel alone, HIP events on the launch stream
    launch_stats = {}

    def time_launches(fn, name):
        """Average over back-to-back launches (one event pair around all of them),
        then median and minimum of the same number of launches timed one by one."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.kernel_reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.kernel_reps)]
        for a_, b_ in evs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        one = sorted(a_.elapsed_time(b_) for a_, b_ in evs)
        launch_stats[name] = (one[len(one) // 2], one[0])
        return e0.elapsed_time(e1) / args.kernel_reps

    row_bytes = 2 if w.dtype in ("bf16", "fp16") else 4
    T = sum(lens)
    # algorithmic HBM bytes per launch: every input read once, every output
    # written once (q-side rows T*H*d, kv-side rows T*Hkv*d, fp32 row vectors T*H)
    qb, kvb, vec = T * H * d * row_bytes, T * Hkv * d * row_bytes, 4 * T * H
    dsum_bytes = 2 * qb + 3 * vec
    alg_bytes = {
        "fwd": 2 * qb + 2 * kvb + vec,                # Q, K, V in; O, lse out
        "bwd_dsum": dsum_bytes,                       # O, dO, lse in; D and L*log2(e) out
        "bwd_dkdv": 2 * qb + 4 * kvb + 2 * vec,       # Q, dO, K, V, D, L in; dK, dV out
        "bwd_dq": 3 * qb + 2 * kvb + 2 * vec,         # Q, dO, K, V, D, L in; dQ out
    }
    alg_bytes["bwd"] = alg_bytes["bwd_dsum"] + alg_bytes["bwd_dkdv"] + alg_bytes["bwd_dq"]  # the three launches
    kernels = {"fwd": dict(ms=time_launches(fwd, "fwd"), work=f_fwd, bound="mfma")}
    if has_bwd and drop:
        kernels["bwd"] = dict(ms=time_launches(bwd, "bwd"), work=2.5 * f_fwd, bound="mfma")
    elif has_bwd:
        kernels.update({
            "bwd_dsum": dict(ms=time_launches(lambda: bwd(fa.FA_BWD_PREP), "bwd_dsum"), work=dsum_bytes,
                             bound="hbm"),
            "bwd_dkdv": dict(ms=time_launches(lambda: bwd(fa.FA_BWD_DKDV), "bwd_dkdv"), work=2.0 * f_fwd,
                             bound="mfma"),
            "bwd_dq": dict(ms=time_launches(lambda: bwd(fa.FA_BWD_DQ), "bwd_dq"), work=0.5 * f_fwd, bound="mfma"),
        })
    for name, kr in kernels.items():
        if kr["bound"] == "mfma":
            kr["achieved"] = kr["work"] / (kr["ms"] * 1e-3) / 1e12
            kr["unit"] = "TFLOP/s"
            kr["frac"] = kr["achieved"] / PEAK_BF16_TFLOPS
        else:
            kr["achieved"] = kr["work"] / (kr["ms"] * 1e-3) / 1e9
            kr["unit"] = "GB/s"
            kr["frac"] = kr["achieved"] / PEAK_HBM_GBS
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    kd = kernels[dom]

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f).get(w.name, {}).get(dom)
        if tr and tr.get("source_hash") == source_hash(dom):
            traffic = tr["bytes_per_launch"]

    roofline = {
        "kernel": dom,
        "bound": kd["bound"],
        "achieved": round(kd["achieved"], 2),
        "peak": PEAK_BF16_TFLOPS if kd["bound"] == "mfma" else PEAK_HBM_GBS,
        "unit": kd["unit"],
        "frac": round(kd["frac"], 4),
        "traffic": traffic,
        "avg_launch_ms": round(kd["ms"], 4),
        "work_per_launch": kd["work"],
    }

    # ---- memory versus a materialised-score baseline (S and P stored in the input type)
    nn = sum(float(n) * n for n in lens) * H
    memory = {
        "libfa_step_bytes": int(lib_bytes),
        "materialised_sp_bytes": int(2 * nn * row_bytes),
        "ratio": round(2 * nn * row_bytes / max(lib_bytes, 1), 1),
    }

    # clock and power under load: the query runs on another thread while this
    # one keeps the launch queue full for six seconds of wall time
    import threading

    tel = {}
    if not args.no_telemetry:
        th = threading.Thread(target=lambda: tel.update(r=gpu_telemetry()))
        th.start()
        t_end = time.perf_counter() + 6.0
        while time.perf_counter() < t_end or th.is_alive():
            step()
            if time.perf_counter() > t_end + 30.0:
                break
        th.join()
        torch.cuda.synchronize()
    telemetry = tel.get("r")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, lens)

    out = {
        "metric": metric_label(w, has_bwd),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "causal": bool(w.causal),
                   "alibi": bool(w.alibi), "pass": "forward+backward" if has_bwd else "forward",
                   **({"sequences": len(lens), "tokens": int(T)} if cu is not None else {}),
                   **({"dropout": drop} if drop else {})},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(f_fwd / (kernels["fwd"]["ms"] * 1e-3) / 1e12, 2),
        "bwd_tflops": (round(f_bwd / (sum(kr["ms"] for n, kr in kernels.items() if n.startswith("bwd")) * 1e-3)
                             / 1e12, 2) if has_bwd else None),
        "kernels": {n: {"ms": round(kr["ms"], 4), "achieved": round(kr["achieved"], 2), "unit": kr["unit"],
                        "frac": round(kr["frac"], 4),
                        "median_ms": round(launch_stats[n][0], 4), "min_ms": round(launch_stats[n][1], 4),
                        "hbm_alg_bytes": int(alg_bytes[n]),
                        "hbm_alg_gbs": round(alg_bytes[n] / (kr["ms"] * 1e-3) / 1e9, 1)}
                    for n, kr in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "memory": memory,
        "env": {"rocm": _read_first("/opt/rocm/.info/version"), "hipcc": _hipcc_version(), "torch": torch.__version__,
                "gpu": torch.cuda.get_device_properties(0).gcnArchName, "telemetry_under_load": telemetry},
    }
    out["fwd_frac_of_peak"] = round(out["fwd_tflops"] / PEAK_BF16_TFLOPS, 4)
    out["bwd_frac_of_peak"] = round(out["bwd_tflops"] / PEAK_BF16_TFLOPS, 4) if has_bwd else None
    print(json.dumps(out), flush=True)

    if args.copy_calibration:
        x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: neg of {COPY_BYTES} bytes", file=sys.stderr, flush=True)


def bench_decode(args):
    """Decode over a key/value cache (fa_fwd_kvcache): one new query per sequence
    against long caches. Bound by HBM: every cached key and value is read once
    per kv head, so the roofline is the algorithmic bytes (valid K and V rows,
    Q, O, lse) over the launch time against 8 TB/s; TFLOP/s (4 H Nq L d per
    sequence) is reported beside it."""
    import torch

    import exact_io_aware_43_amd as fa
    from exact_io_aware_43_amd.workloads import DECODE, make_decode_inputs

    w, Nq, lengths = DECODE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_decode_inputs(w, Nq, lengths, seed=args.seed)
    q, kc, vc, cl = (inp[x].to(dev) for x in ("q", "k_cache", "v_cache", "cache_seqlens"))
    lens = inp["cache_seqlens"].tolist()
    B, H, Hkv, Nk, d = w.B, w.H, w.Hkv, w.N, w.d
    print(f"[bench] decode {w} Nq={Nq} lengths={lens}", file=sys.stderr, flush=True)
    ws_bytes = fa.fa_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step():
        st = fa.fa_fwd_kvcache(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               cl.data_ptr(), B, H, Hkv, Nq, Nk, d, inp["scale"], 1, None, fa.FA_BF16, 0,
                               ws.data_ptr(), ws_bytes, sh)
        if st:
            raise fa.FaError(st)

    for _ in range(args.warmup + 1):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    keys = sum(lens)
    flop = 4.0 * H * Nq * keys * d
    alg_bytes = 2 * keys * Hkv * d * 2 + 2 * B * Nq * H * d * 2 + 4 * B * H * Nq
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    # partial states per query row: the key ranges per kv head (balanced over
    # the caches laid end to end whenever the automatic choice uses several)
    ranges = ws_bytes // (B * H * Nq * (d + 1) * 4) if ws_bytes else 1
    out = {
        "metric": "decode attention HBM GB/s (every cached K/V byte read once, queries and output once), "
                  "bf16 d=128, and % of MI355X HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": "decode", "B": B, "H": H, "Hkv": Hkv, "Nq": Nq, "cache_capacity": Nk,
                   "cache_lengths": lens, "d": d, "causal": True, "pass": "forward (decode)"},
        "roofline": {"kernel": "decode_split+merge", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(ms, 4), "work_per_launch": int(alg_bytes)},
        "key_ranges_per_kv_head": int(ranges), "balanced_ranges": bool(ws_bytes),
    }
    print(json.dumps(out), flush=True)


def bench_fp8(args):
    """The FP8 forward (fa_quantize_fp8_qk for Q and K with the Hadamard rotation,
    fa_quantize_fp8_v, fa_fwd_fp8) on the shape of the long causal workload
    (``--workload fp8``) or of another named one (``--workload fp8:gqa``). A step
    quantizes the 16-bit Q, K, V resident in device memory and runs the
    attention; ``value`` counts the attention FLOPs of the step (4 B H N^2 d,
    halved for causal) over the whole step. The roofline is the attention
    kernel alone against the dense fp8 MFMA peak; the quantizers are HBM-bound
    and listed with their byte rate; the 16-bit forward on the same inputs is
    timed beside it."""
    import torch

    import exact_io_aware_43_amd as fa
    from exact_io_aware_43_amd.workloads import WORKLOADS, flops, hadamard_signs, make_inputs

    base = args.workload.split(":", 1)[1] if ":" in args.workload else "long_causal"
    w = WORKLOADS[base]
    if w.varlen is not None or w.alibi or w.d not in (64, 128):
        raise SystemExit(f"the fp8 path takes dense inputs without ALiBi and d in (64, 128); {base} is not")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w, args.seed, with_grad=False)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    B, H, Hkv, N, d = w.B, w.H, w.Hkv, w.N, w.d
    dt = {"bf16": fa.FA_BF16, "fp16": fa.FA_FP16}[w.dtype]
    causal = int(w.causal)
    print(f"[bench] fp8 forward on {w}", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    words = fa.hadamard_sign_words(hadamard_signs(d, args.seed + 5), d)
    import ctypes
    sp = ctypes.addressof(words)
    nb = (N + 127) // 128
    npad = fa.fa_fp8_v_keys(N)
    qc = torch.empty((B, N, H, d), dtype=torch.uint8, device=dev)
    kc = torch.empty((B, N, Hkv, d), dtype=torch.uint8, device=dev)
    vc = torch.empty((B, Hkv, d, npad), dtype=torch.uint8, device=dev)
    qs = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
    ks = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev)
    vs = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    def check(st):
        if st:
            raise fa.FaError(st)

    def quant():
        check(fa.fa_quantize_fp8_qk(q.data_ptr(), qc.data_ptr(), qs.data_ptr(), B, N, H, d, sp, dt, sh))
        check(fa.fa_quantize_fp8_qk(k.data_ptr(), kc.data_ptr(), ks.data_ptr(), B, N, Hkv, d, sp, dt, sh))
        check(fa.fa_quantize_fp8_v(v.data_ptr(), vc.data_ptr(), vs.data_ptr(), B, N, Hkv, d, dt, sh))

    def attn():
        check(fa.fa_fwd_fp8(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), qs.data_ptr(), ks.data_ptr(),
                            vs.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d, inp["scale"], causal, 1,
                            dt, sh))

    def fwd16():
        check(fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d,
                        inp["scale"], causal, None, None, dt, sh))

    def timed(fn, reps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    for _ in range(args.warmup + 1):
        quant()
        attn()
        fwd16()
    torch.cuda.synchronize()
    step_ms = timed(lambda: (quant(), attn()), args.steps)
    print(f"[bench] {args.steps} steps: {step_ms:.4f} ms/step", file=sys.stderr, flush=True)
    quant_ms = timed(quant, args.kernel_reps)
    attn_ms = timed(attn, args.kernel_reps)
    fwd16_ms = timed(fwd16, args.kernel_reps)
    flop = flops(w)
    tf = lambda ms: flop / (ms * 1e-3) / 1e12  # noqa: E731
    qbytes = (B * N * (H + 2 * Hkv) * d) * 3 + 4 * (B * (H + Hkv) * nb + B * Hkv * d)
    out = {
        "metric": "attention fwd TFLOP/s, fp8 e4m3 with block scales and Hadamard rotation, causal d=128, "
                  "and % of MI355X fp8 MFMA peak",
        "value": round(tf(step_ms), 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": f"fp8:{base}", "B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "causal": bool(causal),
                   "input_dtype": w.dtype, "pass": "quantize Q, K (rotated), V + forward"},
        "kernels": {
            "quantize_qkv": {"ms": round(quant_ms, 4), "hbm_gbs": round(qbytes / (quant_ms * 1e-3) / 1e9, 1),
                             "bytes": int(qbytes)},
            "fwd_fp8": {"ms": round(attn_ms, 4), "tflops": round(tf(attn_ms), 1)},
            "fwd_bf16_same_inputs": {"ms": round(fwd16_ms, 4), "tflops": round(tf(fwd16_ms), 1)},
        },
        "roofline": {"kernel": "fwd_fp8_kernel", "bound": "mfma", "achieved": round(tf(attn_ms), 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tf(attn_ms) / PEAK_FP8_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(attn_ms, 4), "work_per_launch": flop},
    }
    print(json.dumps(out), flush=True)


def _cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _read_first(path):
    try:
        with open(path) as f:
            return f.readline().strip()
    except OSError:
        return None


def _hipcc_version():
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    return next((ln.strip() for ln in r.stdout.splitlines() if "HIP version" in ln), None)


def gpu_telemetry():
    """Power and clock readings of GPU 0 from amd-smi (else rocm-smi), as flat key/value pairs; read-only queries."""
    cmds = (["/opt/rocm/bin/amd-smi", "metric", "-g", "0", "-p", "-c", "--json"],
            ["/opt/rocm/bin/rocm-smi", "-d", "0", "--showpower", "--showclocks", "--json"])
    for cmd in cmds:
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            data = json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip() else None
        except (OSError, subprocess.SubprocessError, ValueError):
            data = None
        if data is None:
            continue
        flat = {}

        def walk(x, key):
            if isinstance(x, dict):
                for k2, v2 in x.items():
                    walk(v2, f"{key}.{k2}" if key else str(k2))
            elif isinstance(x, list):
                for i, v2 in enumerate(x):
                    walk(v2, f"{key}[{i}]")
            elif any(t in key.lower() for t in ("power", "clk", "clock")) and len(flat) < 200:
                flat[key] = x

        walk(data, "")
        # amd-smi: socket power and the current gfx clock of each XCD; other tools: the raw entries
        power = [v for k, v in flat.items() if k.endswith("socket_power.value")]
        clks = [v for k, v in flat.items() if ".clock.gfx_" in k and k.endswith(".clk.value")]
        if power or clks:
            return {"tool": os.path.basename(cmd[0]), "socket_power_w": power[0] if power else None,
                    "gfx_clk_mhz": clks}
        return {"tool": os.path.basename(cmd[0]), "readings": flat}
    return {"tool": None, "readings": "unavailable"}


def _counter_rows(d):
    """(kernel name, dispatch id, counter, value) from a rocprofv3 --output-format csv directory."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                yield r["Kernel_Name"], (fn, r["Dispatch_Id"]), r["Counter_Name"], float(r["Counter_Value"])


def summarise_counters(dirs):
    """Per-kernel mean of every counter over its dispatches, from rocprofv3 --pmc
    CSV directories, as a Markdown table (kernels by the symbols bench.py
    launches; rows without a known symbol are skipped)."""
    acc = {}
    for d in dirs:
        for name, disp, cname, val in _counter_rows(d):
            key = next((k for k, sym in KERNEL_SYMBOLS.items() if sym in name), None)
            if key is None:
                continue
            acc.setdefault(key, {}).setdefault(cname, {}).setdefault(disp, 0.0)
            acc[key][cname][disp] += val
    counters = sorted({c for k in acc.values() for c in k})
    lines = ["| kernel | dispatches | " + " | ".join(counters) + " |", "|" + "---|" * (len(counters) + 2)]
    for k in KERNEL_SYMBOLS:
        if k not in acc:
            continue
        n = max(len(v) for v in acc[k].values())
        cells = []
        for c in counters:
            vals = acc[k].get(c)
            cells.append("—" if not vals else f"{sum(vals.values()) / len(vals):.4g}")
        lines.append(f"| {k} | {n} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def _per_dispatch(d, counter):
    """Mean counter value (KiB) per dispatch for each kernel of interest and the copy kernel."""
    acc = {}
    for name, disp, cname, val in _counter_rows(d):
        if cname != counter:
            continue
        key = next((k for k, sym in KERNEL_SYMBOLS.items() if sym in name), None)
        if key is None and COPY_SYMBOL in name:
            key = "copy"
        if key is None:
            continue
        acc.setdefault(key, {}).setdefault(disp, 0.0)
        acc[key][disp] += val
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in acc.items()}


def summarise_traffic(workload, fetch_dir, write_dir):
    """HBM bytes per launch of each kernel from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB copy."""
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the counter runs hold no copy-calibration dispatch (run bench.py with --copy-calibration)")
    f_fetch = COPY_BYTES / (fetch["copy"][0] * 1024.0)
    f_write = COPY_BYTES / (write["copy"][0] * 1024.0)
    res = {}
    for k in KERNEL_SYMBOLS:
        if k in fetch and k in write:
            fb = fetch[k][0] * 1024.0 * f_fetch
            wb = write[k][0] * 1024.0 * f_write
            res[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                      "fetch_kib_raw": fetch[k][0], "write_kib_raw": write[k][0],
                      "dispatches": [fetch[k][1], write[k][1]], "source_hash": source_hash(k)}
    allw = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            allw = json.load(f)
    allw[workload] = res
    allw.setdefault("_calibration", {})[workload] = {
        "copy_bytes": COPY_BYTES, "copy_fetch_kib": fetch["copy"][0], "copy_write_kib": write["copy"][0],
        "fetch_factor": f_fetch, "write_factor": f_write}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allw, f, indent=1, sort_keys=True)
    print(json.dumps({workload: res, "fetch_factor": f_fetch, "write_factor": f_write}, indent=1))


CPU_SAMPLE_SECONDS = 10.0  # heads are added to the sample until this much CPU time is spent
CPU_SAMPLE_MAX_HEADS = 8


def cpu_baseline(w, inp, lens):
    """The fp64 oracle, as it is, on the first heads of sequence 0: forward + backward,
    one head at a time, until CPU_SAMPLE_SECONDS have passed (at most
    CPU_SAMPLE_MAX_HEADS heads)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.attention as OA
    from exact_io_aware_43_amd.workloads import flops

    n = lens[0]
    G = w.H // w.Hkv
    sl = (0, slice(0, n)) if inp["cu_seqlens"] is None else (slice(0, n),)
    print(f"[bench] cpu baseline: oracle fwd+bwd per head, n={n}", file=sys.stderr, flush=True)
    t = 0.0
    heads = 0
    while heads < min(w.H, CPU_SAMPLE_MAX_HEADS) and t < CPU_SAMPLE_SECONDS:
        h = heads
        q = OA._f64(inp["q"][sl][:, h])
        k = OA._f64(inp["k"][sl][:, h // G])
        v = OA._f64(inp["v"][sl][:, h // G])
        slope = None if inp["alibi_slopes"] is None else float(inp["alibi_slopes"][h])
        t0 = time.perf_counter()
        OA.head_fwd(q, k, v, inp["scale"], w.causal, slope)
        if w.backward:
            OA.head_bwd(q, k, v, OA._f64(inp["do"][sl][:, h]), inp["scale"], w.causal, slope)
        t += time.perf_counter() - t0
        heads += 1
    one = w.with_(B=1, H=1, Hkv=1)
    work = heads * (flops(one, [n]) + (flops(one, [n], backward=True) if w.backward else 0.0))
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return {
        "value": round(work / t / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(max(blas) if blas else 1),
        "kind": "oracle",
        "sample": f"heads 0..{heads - 1} of sequence 0 of {w.name}: N={n}, d={w.d}, causal={w.causal}; "
                  f"fp64 numpy forward{' + backward' if w.backward else ''}, {t:.1f} s",
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "seconds": round(t, 2),
    }


if __name__ == "__main__":
    main()
