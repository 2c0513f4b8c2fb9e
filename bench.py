"""Benchmark of the fused-dequant prefill linear layer on one MI355X.

Default workload: one Qwen3-8B-shaped dense layer's seven linears at M = 658
prompt tokens, fp16 activations (q/k/v/o/gate/up in Q4_K, down in Q6_K).  A
step is one pass over the seven linears with inputs already resident in HBM;
projections that read the same input run as one GEMM over their weights
concatenated along N (q/k/v as qkv, gate/up as gate_up; --no-merge runs all
seven separately).
By default the GEMMs read fragment-major activations: the step makes that
copy of each distinct input once (qgemm_x_to_xf: q/k/v share one input,
gate/up another, o and down one each) and the copies are timed inside the
step; --x-layout row runs the same GEMMs on the row-major inputs instead.

Prints ONE JSON line: whole-step throughput in TFLOP/s (2*M*N*K summed over
the seven linears / step time), the linear-only prefill rate, per-kernel
times from HIP events, the roofline of the dominant kernel and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--steps 20] [--warmup 5] [--workload NAME] [--no-cpu-baseline]

Profiling helpers (same JSON line, restricted work):
    --only LABEL        run only that GEMM of the workload
    --pool-mb MB        every GEMM rotates through copies of its packed weights
                        totalling >= MB (default 640), so the 256 MB Infinity
                        Cache cannot serve them (0: one copy)
    --rung R            force rung R instead of the M-ladder's choice
    --x-layout xf|row   activation layout the GEMMs read (default xf; row for
                        the mixture-of-experts FFN, where the two steps tie:
                        the grouped GEMMs gain about what the copies cost)
    --no-merge          seven separate GEMMs instead of qkv, o, gate_up, down
                        (for the mixture-of-experts FFN: gate and up as two
                        grouped launches instead of one over both)
    --copy-calibration BYTES
                        run a plain device-to-device copy of BYTES bytes three
                        times and exit (reference for HBM byte counters)
    --no-ceiling        skip the MFMA rate probe (`mfma_ceiling`: what the
                        chip sustains on random operands under its power
                        limit, for reading `roofline.frac` against)
    --no-int8           skip the int8-activation arm (`int8_arm`: the same
                        step with per-row int8 activations quantized inside the
                        step and the weights requantized to int8 inside the
                        GEMM, on the same rotating weight copies)
"""
from __future__ import annotations

import argparse
import ctypes
import functools
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import quantized_weight_prefill_amd as qg  # noqa: E402
from quantized_weight_prefill_amd import probe, synth  # noqa: E402

METRIC = "fused Q4_K GEMM TFLOP/s + prefill tok/s (Qwen3-8B shapes, M=658); % roofline"
PEAK_TFLOPS = {qg.F16: 2500.0, qg.BF16: 2500.0}  # dense MFMA, fp16 / bf16
PEAK_HBM_GBPS = 8000.0
PEAK_INT8_TOPS = 5000.0  # dense int8 MFMA
BYTES_PER_WEIGHT = {"q4k": 144 / 256, "q6k": 210 / 256}
PROFILE_STEPS = 10  # steps of the per-launch profiling pass


def weight_bytes(fmt: str, N: int, K: int, group: int, sym: bool) -> float:
    if fmt in BYTES_PER_WEIGHT:
        return BYTES_PER_WEIGHT[fmt] * N * K
    return N * K / 2 + (K // group) * N * 2 + (0 if sym else (K // group) * N / 2)


def source_hash() -> str:
    """Digest of the library's sources (every file under csrc/ but the probe
    library's), the key that ties a committed counter summary to the
    kernels it was taken on."""
    h = hashlib.sha256()
    base = os.path.join(ROOT, "quantized_weight_prefill_amd", "csrc")
    for f in sorted(os.listdir(base)):
        path = os.path.join(base, f)
        if os.path.isfile(path):
            h.update(f.encode())
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


class HipTimer:
    """HIP events for timing only, made with hipEventDisableSystemFence: when
    such an event is recorded the runtime skips the system-scope fence (an L2
    writeback and invalidate) that an ordinary event adds between two
    kernels.  They come from the HIP runtime already loaded in the process
    (the one PyTorch uses, so streams are shared)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
        rt = ctypes.CDLL(path)
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt, self.events = rt, []

    def pair(self):
        evs = []
        for _ in range(2):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e)
        self.events += evs
        return evs

    def record(self, ev, stream):
        if self.rt.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, e0, e1) -> float:
        v = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(v), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(v.value)

    def close(self):
        for e in self.events:
            self.rt.hipEventDestroy(e)
        self.events = []


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=70)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_layer_m658",
                    choices=sorted(synth.WORKLOADS) + sorted(synth.MOE_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--only", default=None, help="run only the GEMM with this label")
    ap.add_argument("--rung", type=int, default=-1, help="force a rung (-1: M-ladder)")
    ap.add_argument("--no-merge", action="store_true",
                    help="run the projections that share an input (q/k/v, gate/up) as separate GEMMs")
    ap.add_argument("--x-layout", choices=["xf", "row"], default=None,
                    help="xf: fragment-major copies made inside the step (default of the dense layers); row: row-major "
                         "X (default of the mixture-of-experts FFN, whose routed rows arrive row-major)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA rate probe")
    ap.add_argument("--no-staged", action="store_true", help="skip the staged-arm comparison")
    ap.add_argument("--no-gpu-state", action="store_true",
                    help="skip the clock/temperature window (~2400 extra steps; for profiler runs)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the comparison with the vendor dense GEMM on the unpacked weights")
    ap.add_argument("--no-int8", action="store_true", help="skip the int8-activation arm")
    ap.add_argument("--pool-mb", type=float, default=640.0,
                    help="every GEMM rotates through copies of its weights totalling at least this many MB, so the "
                         "256 MB Infinity Cache cannot hold them (0: no rotation)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by N or K across GPUs, which is not implemented)", file=sys.stderr)
        return 2

    if args.x_layout is None:
        args.x_layout = "row" if args.workload in synth.MOE_WORKLOADS else "xf"

    import torch

    torch.cuda.init()
    if args.workload in synth.MOE_WORKLOADS:
        return run_grouped(args)
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    lib = qg.lib()
    # every launch of the step goes to one stream created here (the null
    # stream carries the runtime's implicit synchronisation with other streams)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    sp = ctypes.c_void_p(stream.cuda_stream)
    timer = HipTimer()

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr())

    xf_layout = args.x_layout == "xf"
    inputs = {}  # GEMM index whose activations are read -> its device copies
    gemms = []
    for sg in synth.step_gemms(args.workload, merge=not args.no_merge):
        label, fmt, M, K, N = sg["label"], sg["fmt"], sg["M"], sg["K"], sg["N"]
        dt, group, sym = sg["dt"], sg["group"], sg["sym"]
        if args.only is not None and label != args.only:
            continue
        X, enc = synth.step_inputs(args.workload, sg["members"])
        packed = qg.pack(fmt, enc, N, K)
        tdt = torch.float16 if dt == qg.F16 else torch.bfloat16
        src = synth.x_source(args.workload, sg["members"][0])
        prep = None
        if src not in inputs:
            x = torch.from_numpy(X.view(np.int16)).view(tdt).to(dev)
            xf = torch.empty((qg.xf_bytes(M, K) // 2,), dtype=tdt, device=dev) if xf_layout else None
            inputs[src] = (x, xf)
            if xf_layout:  # the first GEMM reading this input makes its fragment-major copy
                prep = dict(label=f"x_to_xf({wl['gemms'][src][0]})", M=M, K=K,
                            call=functools.partial(lib.qgemm_x_to_xf, ptr(x), ptr(xf), M, K, sp),
                            bytes=2.0 * M * K + qg.xf_bytes(M, K))
        x, xf = inputs[src]
        wp = torch.from_numpy(packed).to(dev)
        y = torch.empty((M, N), dtype=tdt, device=dev)
        if args.rung >= 0:
            info = qg.rung_info(args.rung, fmt, M, N, K, dt)
        else:
            info = (qg.select_rung_xf if xf_layout else qg.select_rung)(fmt, M, N, K, dt)
        wbytes = weight_bytes(fmt, N, K, group or 128, sym)
        intensity = 2.0 * M * N * K / (wbytes + 2 * M * K + 2 * M * N)
        below_ridge = intensity < PEAK_TFLOPS[dt] * 1e12 / (PEAK_HBM_GBPS * 1e9)
        # every GEMM rotates through copies of its packed weights (>= --pool-mb
        # MB), so each launch reads weights the 256 MB Infinity Cache does not
        # hold, as in a model whose layers' weights far exceed it
        ncopy = max(1, int(np.ceil(args.pool_mb * 1e6 / packed.nbytes))) if args.pool_mb > 0 else 1
        pool = [wp] + [wp.clone() for _ in range(ncopy - 1)]
        # pre-marshalled C calls (one per weight copy): the GEMM entry point
        # for the layout, rung -1 being the layout's M-ladder
        grp, zp = (group if fmt == "w4a16" else 0), int(not sym)
        # the split rungs' partial sums live in a workspace the caller owns
        nws = qg.workspace_bytes(fmt, args.rung, M, N, K, dt, qg.X_FRAG if xf_layout else qg.X_ROW)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        if xf_layout:
            calls = [functools.partial(lib.qgemm_gemm_xf, qg.FORMATS[fmt], args.rung, ptr(xf), ptr(w), ptr(y), M, N, K,
                                       grp, zp, dt, ptr(ws), nws, sp) for w in pool]
        else:
            calls = [functools.partial(lib.qgemm_gemm_rung, qg.FORMATS[fmt], args.rung, ptr(x), ptr(w), ptr(y), M, N,
                                       K, grp, zp, dt, ptr(ws), nws, sp) for w in pool]
        gemms.append(dict(label=label, fmt=fmt, M=M, K=K, N=N, dt=dt, group=group, sym=sym, x=x, wp=wp, y=y,
                          X=X, enc=enc, rung=info["name"], flops=2.0 * M * N * K, wbytes=wbytes, pool=pool, turn=0,
                          calls=calls, prep=prep, src=src, ws=ws,
                          members=[wl["gemms"][i][0] for i in sg["members"]], below_ridge=below_ridge))
        print(f"[bench] {label}: {fmt} M={M} K={K} N={N} x={args.x_layout} rung={info['name']}", file=sys.stderr,
              flush=True)

    if not gemms:
        print(f"bench.py: no GEMM labelled {args.only!r} in {args.workload}", file=sys.stderr)
        return 2

    def call(g):
        st = g["calls"][g["turn"] % len(g["calls"])]()
        g["turn"] += 1
        if st != 0:
            raise qg.QGemmError(f"{g['label']} GEMM", st)

    def call_prep(p):
        st = p["call"]()
        if st != 0:
            raise qg.QGemmError(p["label"], st)

    for _ in range(args.warmup):
        for g in gemms:
            if g["prep"] is not None:
                call_prep(g["prep"])
            call(g)
    torch.cuda.synchronize()

    # Per-launch times: a pass of PROFILE_STEPS steps, untimed, with HIP events
    # around every launch on the launch stream (an event between two kernels
    # costs the queue a few microseconds, so the timed steps below carry
    # events around the dominant GEMM only).
    preps = [g["prep"] for g in gemms if g["prep"] is not None]
    nprof = max(3, min(args.steps, PROFILE_STEPS))
    ev = [[timer.pair() for _ in gemms] for _ in range(nprof)]
    evp = [[timer.pair() for _ in preps] for _ in range(nprof)]
    for s in range(nprof):
        i = 0
        for j, g in enumerate(gemms):
            if g["prep"] is not None:
                timer.record(evp[s][i][0], sp)
                call_prep(g["prep"])
                timer.record(evp[s][i][1], sp)
                i += 1
            timer.record(ev[s][j][0], sp)
            call(g)
            timer.record(ev[s][j][1], sp)
    torch.cuda.synchronize()
    per = []
    for i, p in enumerate(preps):
        ms = float(np.mean([timer.ms(*evp[s][i]) for s in range(nprof)]))
        per.append(dict(label=p["label"], M=p["M"], K=p["K"], rung="x_to_xf", ms=round(ms, 5),
                        gbps=round(p["bytes"] / ms / 1e6, 1)))
    per_prep = len(per)
    gemm_ms = [float(np.mean([timer.ms(*ev[s][j]) for s in range(nprof)])) for j in range(len(gemms))]
    jd = int(np.argmax(gemm_ms))  # the dominant GEMM: largest share of the step

    # timed region: K steps back to back, in (up to) ten samples of
    # consecutive steps; fence-less HIP events on the launch stream mark the
    # samples' ends and bracket every launch of the dominant GEMM
    nsamp = min(10, args.steps)
    bounds = [round(i * args.steps / nsamp) for i in range(nsamp + 1)]
    evs = [timer.pair() for _ in range(nsamp)]
    evd = [timer.pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(nsamp):
        timer.record(evs[i][0], sp)
        for s in range(bounds[i], bounds[i + 1]):
            for j, g in enumerate(gemms):
                if g["prep"] is not None:
                    call_prep(g["prep"])
                if j == jd:
                    timer.record(evd[s][0], sp)
                    call(g)
                    timer.record(evd[s][1], sp)
                else:
                    call(g)
        timer.record(evs[i][1], sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gemm_ms[jd] = float(np.mean([timer.ms(e0, e1) for e0, e1 in evd]))
    sample_ms = [timer.ms(*evs[i]) / (bounds[i + 1] - bounds[i]) for i in range(nsamp)]
    launches_per_step = len(gemms) + len(preps)

    def run_step():
        for g in gemms:
            if g["prep"] is not None:
                call_prep(g["prep"])
            call(g)
    state = None if args.no_gpu_state else gpu_state(run_step)

    for j, g in enumerate(gemms):
        ms = gemm_ms[j]
        per.append(dict(label=g["label"], fmt=g["fmt"], M=g["M"], K=g["K"], N=g["N"], rung=g["rung"],
                        ms=round(ms, 5), tflops=round(g["flops"] / ms / 1e9, 2),
                        weight_gbps=round(g["wbytes"] / ms / 1e6, 1),
                        weight_frac_hbm=round(g["wbytes"] / ms / 1e6 / PEAK_HBM_GBPS, 4),
                        weight_copies=len(g["pool"])))
    # Weight-bound GEMMs are short: per-launch events add a fixed cost, so they
    # are also timed back to back (50 launches a sample, median of 5, weights
    # rotating) next to a plain streaming read of the same bytes.
    for g, p in zip(gemms, per[per_prep:]):
        if g["below_ridge"] and len(g["pool"]) > 1:
            samples = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(50):
                    call(g)
                e1.record(stream)
                torch.cuda.synchronize()
                samples.append(e0.elapsed_time(e1) / 50)
            b2b = float(np.median(samples))
            p["ms_back_to_back"] = round(b2b, 5)
            p["weight_gbps_back_to_back"] = round(g["wbytes"] / b2b / 1e6, 1)
            p["read_probe_gbps"] = read_ceiling(g["pool"])
            p["weight_frac_of_read_probe"] = round(p["weight_gbps_back_to_back"] / p["read_probe_gbps"], 4)
    flops_step = sum(g["flops"] for g in gemms)
    kernel_ms_step = sum(p["ms"] for p in per)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # dominant kernel and its roofline (its time is the timed region's mean)
    gd, pd = gemms[jd], per[per_prep + jd]
    pd["timed_in_step"] = True
    intensity = gd["flops"] / (gd["wbytes"] + 2 * gd["M"] * gd["K"] + 2 * gd["M"] * gd["N"])
    ridge = PEAK_TFLOPS[gd["dt"]] * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": pd["tflops"], "peak": PEAK_TFLOPS[gd["dt"]], "unit": "TFLOP/s",
                "frac": round(pd["tflops"] / PEAK_TFLOPS[gd["dt"]], 4)}
    else:
        gbps = (gd["wbytes"] + 2 * gd["M"] * gd["K"] + 2 * gd["M"] * gd["N"]) / (pd["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    roof["kernel"] = f"{gd['label']} ({gd['fmt']} M={gd['M']} K={gd['K']} N={gd['N']}, rung {gd['rung']})"
    roof["traffic"] = measured_traffic(f"{args.workload}/{gd['label']}")
    staged = None if args.no_staged else staged_arm(gd, call)
    dense = None if args.no_dense else dense_reference(gemms, call)
    int8 = None if args.no_int8 else int8_arm(gemms, wl, lib, sp, timer, args)
    ceiling = None if args.no_ceiling else mfma_ceiling(gd["dt"])
    if ceiling is not None and roof["bound"] == "mfma":
        roof["frac_of_sustained"] = round(pd["tflops"] / ceiling["value"], 4)
    if roof["bound"] == "hbm" and "read_probe_gbps" in pd:
        roof["frac_of_sustained"] = round(pd["weight_gbps_back_to_back"] / pd["read_probe_gbps"], 4)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(float(np.median(sample_ms)), 5),
        "ms_per_step_samples": [round(v, 5) for v in sample_ms],
        "timing": f"{args.steps} steps in {nsamp} samples of consecutive steps ({launches_per_step} launches a step, "
                  f"{min(b - a for a, b in zip(bounds, bounds[1:])) * launches_per_step}+ a sample); ms_per_step is "
                  "the wall clock over all of them between synchronisations, ms_per_step_median the median of the "
                  "samples' HIP-event times",
        "gpu_state": state,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if all(g["dt"] == qg.F16 for g in gemms) else "bf16" if all(g["dt"] == qg.BF16 for g in gemms) else "f16+bf16",
        "data": "synthetic (seeded; shapes and value distributions of the workload, random weights)",
        "config": {"workload": args.workload, "gemms": [f"{g['label']}:{g['fmt']}:{g['M']}x{g['K']}x{g['N']}"
                                                       for g in gemms],
                   "x_layout": "fragment-major (copies made inside the step)" if xf_layout else "row-major",
                   "merged": {g["label"]: g["members"] for g in gemms if len(g["members"]) > 1}},
        "kernel_ms_per_step": round(kernel_ms_step, 5),
        "per_kernel_timing": "HIP events (hipEventDisableSystemFence) on the launch stream around every launch in a "
                             "separate profiling pass; the dominant GEMM's time is the mean of such events around "
                             "its launches inside the timed region",
        "per_kernel": per,
        "roofline": roof,
    }
    if ceiling is not None:
        out["mfma_ceiling"] = ceiling
    if staged is not None:
        out["staged_arm"] = staged
    if dense is not None:
        out["dense_reference"] = dense
    if int8 is not None:
        out["int8_arm"] = int8
    if args.only is not None or args.rung >= 0:
        out["config"]["only"] = args.only
        out["config"]["rung"] = args.rung
    if args.workload == "qwen3_8b_layer_m658" and args.only is None:
        # linear layers only: 36 layers x the seven projections of one layer
        out["prefill_tok_s_linear_only"] = round(synth.QWEN3_8B_PROMPT / (synth.QWEN3_8B_LAYERS * ms_per_step * 1e-3), 1)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(gemms, args.cpu_seconds, xf_layout)
    print(json.dumps(out), flush=True)
    return 0


def gpu_state(run_step, steps: int = 2400, every: int = 80) -> dict:
    """Shader clock, memory clock and temperatures while the step runs: the
    step is queued `every` steps at a time and the GPU's metrics table is read
    between the batches (the GPU is busy with the queued work meanwhile), over
    `steps` steps after the timed region (about a second of the layer step:
    the metrics table refreshes on its own period, so a window of a few
    milliseconds would repeat one reading).  Read through amdsmi; on a host
    without it the reason is recorded instead."""
    import torch

    try:
        import amdsmi

        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        h = handles[0]
        try:  # the GPU torch runs on, by PCI address, when several are listed
            props = torch.cuda.get_device_properties(0)
            want = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}"
            for cand in handles:
                if amdsmi.amdsmi_get_gpu_device_bdf(cand).lower().startswith(want):
                    h = cand
                    break
        except Exception:
            pass
    except Exception as e:  # pragma: no cover - depends on the host
        return {"error": f"amdsmi unavailable: {e}"}

    def valid(v):
        vals = v if isinstance(v, (list, tuple)) else [v]
        return [float(x) for x in vals if isinstance(x, (int, float)) and 0 < x < 0xFFFF]

    keys = {"sclk_mhz": ("current_gfxclk", "current_gfxclks"), "mclk_mhz": ("current_uclk",),
            "temp_hotspot_c": ("temperature_hotspot",), "temp_mem_c": ("temperature_mem",),
            "power_w": ("current_socket_power",), "gfx_activity_pct": ("average_gfx_activity",)}
    got = {k: [] for k in keys}
    err = None
    t0 = time.perf_counter()
    for i in range(steps // every):
        for _ in range(every):
            run_step()
        if i < 2:
            continue  # let the queue fill first
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        except Exception as e:  # pragma: no cover
            err = str(e)
            break
        for k, names in keys.items():
            for n in names:
                if n in m and valid(m[n]):
                    got[k].append(float(np.mean(valid(m[n]))))
                    break
    torch.cuda.synchronize()
    window_ms = (time.perf_counter() - t0) * 1e3
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    out = {k: ([round(min(v), 1), round(float(np.mean(v)), 1), round(max(v), 1)] if v else None)
           for k, v in got.items()}
    out["format"] = "[min, mean, max] over the samples read while the step ran (amdsmi gpu_metrics; sclk averaged over XCDs)"
    out["samples"] = max((len(v) for v in got.values()), default=0)
    out["window_ms"] = round(window_ms, 1)
    if err:
        out["error"] = err
    return out


def mfma_ceiling(dt) -> dict:
    """What the chip sustains on dense MFMA work: the rate probe (four waves
    per SIMD, four independent 32x32x16 accumulators per wave) on seeded
    uniform random operands, timed with HIP events on the launch stream.  The
    clock drops under this load by an amount that depends on the operand
    bits, so this sits below the spec peak (which assumes the full clock)."""
    import torch

    rng = np.random.default_rng(7)
    tdt = torch.float16 if dt == qg.F16 else torch.bfloat16
    blocks, iters, reps = 1024, 4000, 5
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flops = 2.0 * 32 * 32 * 16 * 4 * iters * 4 * blocks

    def rate(ops):
        for _ in range(2):
            probe.mfma(ops, out, blocks, iters, dt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            probe.mfma(ops, out, blocks, iters, dt)
        e1.record(stream)
        torch.cuda.synchronize()
        return round(flops / (e0.elapsed_time(e1) / reps) / 1e9, 1)

    random_ops = torch.from_numpy(rng.uniform(-1.0, 1.0, 256 * 8 * 8).astype(np.float32)).to(tdt).cuda()
    zero_ops = torch.zeros(256 * 8 * 8, dtype=tdt, device="cuda")
    return {"value": rate(random_ops), "unit": "TFLOP/s", "dtype": "f16" if dt == qg.F16 else "bf16",
            "operands": "uniform random in [-1, 1], seeded", "zero_operands": rate(zero_ops),
            "probe": "32x32x16 MFMA, 4 waves/SIMD, 4 chains/wave"}


def run_grouped(args) -> int:
    """A mixture-of-experts FFN at prompt size: each GEMM is one grouped launch
    over the routed rows (already grouped by expert), by default on those
    row-major rows; --x-layout xf runs them on the rows' fragment-major copy
    made inside the step (one copy for gate and up, which read the same rows,
    one for down).  Gate and up run as one grouped GEMM over each expert's
    gate and up columns side by side (--no-merge: two launches).  Beside it: the two layouts' steps and GEMMs interleaved,
    and the same work issued as one launch per expert.  Weight-bound, so the
    experts' weights rotate through copies totalling >= --pool-mb, and the
    streaming-read probe of the same bytes sits beside each GEMM.  Launches
    are pre-marshalled C calls on one stream, timed as the layer step is."""
    import torch

    name = args.workload
    w = synth.MOE_WORKLOADS[name]
    E = w["experts"]
    counts = synth.moe_counts(name)
    offs_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offs_h[-1])
    lib = qg.lib()
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    sp = ctypes.c_void_p(stream.cuda_stream)
    timer = HipTimer()

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr())

    offs = torch.from_numpy(offs_h).cuda()
    xf_layout = args.x_layout == "xf"
    gemms, inputs = [], {}
    for sg in synth.moe_step_gemms(name, merge=not args.no_merge):
        label, fmt, K, N = sg["label"], sg["fmt"], sg["K"], sg["N"]
        if args.only is not None and label != args.only:
            continue
        X, enc = synth.moe_step_inputs(name, sg["members"])
        per = [qg.pack(fmt, enc[e * N:(e + 1) * N], N, K) for e in range(E)]
        stride = per[0].nbytes
        wp = torch.from_numpy(np.concatenate(per)).cuda()
        del per, enc
        ncopy = max(1, int(np.ceil(args.pool_mb * 1e6 / wp.numel()))) if args.pool_mb > 0 else 1
        pool = [wp] + [wp.clone() for _ in range(ncopy - 1)]
        src = sg["input"]
        if src not in inputs:
            x = torch.from_numpy(X.view(np.int16)).view(torch.float16).cuda()
            xf = torch.empty(qg.xf_bytes(T, K) // 2, dtype=torch.float16, device="cuda")
            inputs[src] = dict(label=f"x_to_xf({w['gemms'][src][0]})", x=x, xf=xf, K=K,
                               call=functools.partial(lib.qgemm_x_to_xf, ptr(x), ptr(xf), T, K, sp))
        inp = inputs[src]
        y = torch.empty((T, N), dtype=torch.float16, device="cuda")
        F = qg.FORMATS[fmt]
        calls = {"xf": [functools.partial(lib.qgemm_grouped_xf, F, ptr(inp["xf"]), ptr(wq), ptr(y), ptr(offs), E, T, N,
                                          K, 0, 0, qg.F16, sp) for wq in pool],
                 "row": [functools.partial(lib.qgemm_grouped, F, ptr(inp["x"]), ptr(wq), ptr(y), ptr(offs), E, T, N, K,
                                           0, 0, qg.F16, sp) for wq in pool]}
        used = int((counts > 0).sum())
        gemms.append(dict(label=label, fmt=fmt, K=K, N=N, inp=inp, y=y, pool=pool, turn=0, stride=stride, calls=calls,
                          flops=2.0 * T * N * K, wbytes=float(used * stride)))
        print(f"[bench] {label}: grouped {fmt} T={T} K={K} N={N} E={E} ({used} with rows), rows of "
              f"{w['gemms'][src][0]}, x={args.x_layout}", file=sys.stderr, flush=True)
    if not gemms:
        print(f"bench.py: no GEMM labelled {args.only!r} in {name}", file=sys.stderr)
        return 2

    def call(g, layout):
        st = g["calls"][layout][g["turn"] % len(g["pool"])]()
        g["turn"] += 1
        if st != 0:
            raise qg.QGemmError(f"{g['label']} grouped GEMM", st)

    def copy(inp):
        st = inp["call"]()
        if st != 0:
            raise qg.QGemmError(inp["label"], st)

    def step(layout):
        if layout == "xf":
            for inp in inputs.values():
                copy(inp)
        for g in gemms:
            call(g, layout)

    lay = "xf" if xf_layout else "row"
    for _ in range(args.warmup):
        step(lay)
    torch.cuda.synchronize()

    # per-launch times: an untimed pass with events around every launch
    nprof = max(3, min(args.steps, PROFILE_STEPS))
    inps = list(inputs.values()) if xf_layout else []
    evc = [[timer.pair() for _ in inps] for _ in range(nprof)]
    ev = [[timer.pair() for _ in gemms] for _ in range(nprof)]
    for s_ in range(nprof):
        for i, inp in enumerate(inps):
            timer.record(evc[s_][i][0], sp)
            copy(inp)
            timer.record(evc[s_][i][1], sp)
        for j, g in enumerate(gemms):
            timer.record(ev[s_][j][0], sp)
            call(g, lay)
            timer.record(ev[s_][j][1], sp)
    torch.cuda.synchronize()

    # timed region: K steps in (up to) ten samples of consecutive steps,
    # events only at the samples' ends
    nsamp = min(10, args.steps)
    bounds = [round(i * args.steps / nsamp) for i in range(nsamp + 1)]
    evs = [timer.pair() for _ in range(nsamp)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(nsamp):
        timer.record(evs[i][0], sp)
        for s_ in range(bounds[i], bounds[i + 1]):
            step(lay)
        timer.record(evs[i][1], sp)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    sample_ms = [timer.ms(*evs[i]) / (bounds[i + 1] - bounds[i]) for i in range(nsamp)]

    steps_cmp = interleaved({"fragment_major_with_copies": lambda: step("xf"), "row_major": lambda: step("row")},
                            reps=10)
    out_k = []
    for i, inp in enumerate(inps):
        ms = float(np.mean([timer.ms(*evc[s_][i]) for s_ in range(nprof)]))
        out_k.append(dict(label=inp["label"], T=T, K=inp["K"], ms=round(ms, 5),
                          gbps=round(4.0 * T * inp["K"] / ms / 1e6, 1)))
    for j, g in enumerate(gemms):
        ms = float(np.mean([timer.ms(*ev[s_][j]) for s_ in range(nprof)]))
        b2b = interleaved({"xf": lambda: call(g, "xf"), "row": lambda: call(g, "row")})

        def per_expert():
            wp = g["pool"][0]
            for e in range(E):
                if counts[e]:
                    a, b = int(offs_h[e]), int(offs_h[e + 1])
                    qg.gemm_rung(g["fmt"], -1, g["inp"]["x"][a:b], wp[e * g["stride"]:(e + 1) * g["stride"]], g["N"],
                                 out=g["y"][a:b])
        loop = interleaved({"loop": per_expert}, reps=3, rounds=3)["loop"]
        rd = read_ceiling(g["pool"])
        out_k.append(dict(label=g["label"], fmt=g["fmt"], T=T, K=g["K"], N=g["N"], experts=E, ms=round(ms, 5),
                          tflops=round(g["flops"] / ms / 1e9, 2), weight_gbps=round(g["wbytes"] / ms / 1e6, 1),
                          read_probe_gbps=rd, weight_frac_of_read_probe=round(g["wbytes"] / ms / 1e6 / rd, 4),
                          back_to_back_ms_by_layout={k: round(v, 5) for k, v in b2b.items()},
                          per_expert_launches_ms=round(loop, 5), weight_copies=len(g["pool"])))
    timer.close()
    flops_step = sum(g["flops"] for g in gemms)
    gk = [p for p in out_k if "fmt" in p]
    jd = int(np.argmax([p["ms"] for p in gk]))
    gd, pd = gemms[jd], gk[jd]
    gbps = (gd["wbytes"] + 2.0 * T * gd["K"] + 2.0 * T * gd["N"]) / (pd["ms"] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "kernel": f"{gd['label']} (grouped {gd['fmt']} T={T} K={gd['K']} N={gd['N']} E={E})",
            "traffic": measured_traffic(f"{name}/{gd['label']}") if not xf_layout else None,
            "frac_of_sustained": pd["weight_frac_of_read_probe"]}
    print(json.dumps({
        "metric": METRIC, "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(float(np.median(sample_ms)), 5),
        "ms_per_step_samples": [round(v, 5) for v in sample_ms],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded; routed row counts drawn from a Zipf-like expert popularity, random weights)",
        "config": {"workload": name, "tokens": w["tokens"], "top_k": w["top_k"], "experts": E, "rows": T,
                   "rows_per_expert_min_mean_max": [int(counts.min()), round(float(counts.mean()), 1), int(counts.max())],
                   "x_layout": "fragment-major (copies of the routed rows made inside the step: one for gate and up, one "
                               "for down)" if xf_layout else "row-major"},
        "steps_interleaved_ms": {k: round(v, 5) for k, v in steps_cmp.items()},
        "per_kernel": out_k, "roofline": roof}), flush=True)
    return 0


def interleaved(arms: dict, reps: int = 20, rounds: int = 5) -> dict:
    """Median ms per launch of each arm, the arms interleaved (one sample of
    `reps` back-to-back launches of each arm in turn, `rounds` times), so
    that clock and thermal drift hit every arm alike.  HIP events on the
    launch stream around each sample."""
    import torch

    stream = torch.cuda.current_stream()
    for fn in arms.values():
        fn()
    samples = {k: [] for k in arms}
    for _ in range(rounds):
        for k, fn in arms.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            samples[k].append(e0.elapsed_time(e1) / reps)
    return {k: float(np.median(v)) for k, v in samples.items()}


def staged_arm(g, call, reps: int = 20) -> dict:
    """The dominant GEMM fused (its rung in the step, on the step's activation
    layout, and the 128x128 rung on row-major activations, the tile the staged
    GEMM shares) against the staged arm: unpack into a 2-byte scratch, then
    the same 128x128 streaming kernel on it, on row-major activations.  The
    arms are interleaved: five rounds of 20 back-to-back launches each, the
    median sample per arm."""
    import torch

    rung128 = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-128x128"][0]
    grp = g["group"] if g["fmt"] == "w4a16" else 0
    scratch = torch.empty(qg.staged_scratch_bytes(g["N"], g["K"]), dtype=torch.uint8, device="cuda")
    x0 = g["x"][:0]
    y0 = g["y"][:0]
    # every arm rotates through the same weight copies as the step
    turn = [0]

    def wp():
        turn[0] += 1
        return g["pool"][turn[0] % len(g["pool"])]

    t = interleaved({
        "fused": lambda: call(g),
        "same_tile": lambda: qg.gemm_rung(g["fmt"], rung128, g["x"], wp(), g["N"], group=grp, has_zp=not g["sym"],
                                          out=g["y"]),
        "staged": lambda: qg.staged(g["fmt"], g["x"], wp(), g["N"], scratch=scratch, group=grp, has_zp=not g["sym"],
                                    out=g["y"]),
        "unpack": lambda: qg.staged(g["fmt"], x0, wp(), g["N"], scratch=scratch, group=grp, has_zp=not g["sym"],
                                    out=y0)}, reps)
    fused, same_tile, staged, unpack = t["fused"], t["same_tile"], t["staged"], t["unpack"]
    wq = g["wbytes"]
    w16 = 2.0 * g["K"] * (-(-g["N"] // 16) * 16)
    return {"gemm": g["label"], "fused_rung": g["rung"], "fused_ms": round(fused, 5),
            "fused_same_tile_ms": round(same_tile, 5),
            "staged_ms": round(staged, 5), "unpack_ms": round(unpack, 5),
            "staged_gemm_ms": round(staged - unpack, 5), "staged_over_fused_same_tile": round(staged / same_tile, 3),
            "weight_bytes_fused": round(wq), "weight_bytes_staged": round(wq + 2 * w16),
            "timing": "arms interleaved, 5 rounds of 20 launches each, median",
            "note": "staged = unpack pass (reads packed W, writes 2 B/weight) + the same 128x128 kernel reading "
                    "2 B/weight; its Y equals the fused 128x128 rung's Y bit for bit"}


def dense_reference(gemms, call, reps: int = 20) -> dict:
    """Each GEMM of the step fused (its rung and activation layout as in the
    step) against the vendor library's dense GEMM on the same shape: W
    unpacked once by the library's own dequant to fp16/bf16, then
    torch.matmul (hipBLASLt) of row-major X by it, its dense copies rotating
    through >= 640 MB as the packed ones do.  Arms interleaved, five rounds
    of 20 launches, medians.  A calibration of what the chip reaches on these
    shapes without any unpacking, not a path of the library."""
    import torch

    rows = []
    for g in gemms:
        grp = g["group"] if g["fmt"] == "w4a16" else 0
        w = qg.dequant(g["fmt"], g["pool"][0], g["N"], g["K"], g["dt"], group=grp, has_zp=not g["sym"])
        copies = max(1, -(-int(640e6) // (w.numel() * w.element_size())))
        pool = [w] + [w.clone() for _ in range(copies - 1)]
        y = torch.empty((g["M"], g["N"]), dtype=w.dtype, device="cuda")
        turn = [0]

        def dense(g=g, pool=pool, y=y):
            turn[0] += 1
            torch.matmul(g["x"], pool[turn[0] % len(pool)], out=y)

        t = interleaved({"fused": lambda g=g: call(g), "dense": dense}, reps)
        flops = 2.0 * g["M"] * g["N"] * g["K"]
        rows.append({"gemm": g["label"], "shape": f"{g['fmt']} M={g['M']} K={g['K']} N={g['N']}",
                     "fused_rung": g["rung"], "fused_ms": round(t["fused"], 5), "dense_ms": round(t["dense"], 5),
                     "fused_tflops": round(flops / t["fused"] / 1e9, 1), "dense_tflops": round(flops / t["dense"] / 1e9, 1),
                     "dense_over_fused_time": round(t["dense"] / t["fused"], 3)})
        del pool, w, y
        torch.cuda.empty_cache()
    return {"what": "vendor dense GEMM (torch.matmul / hipBLASLt) on the unpacked weights, same shapes, "
                    "weights rotating, interleaved with the fused launches: a calibration, not a library path",
            "per_gemm": rows}


def int8_arm(gemms, wl, lib, sp, timer, args) -> dict:
    """The same step on the int8-activation path: each distinct input is
    quantized per row (qgemm_i8_quantize, inside the step, replacing the
    fragment-major copy), each GEMM unpacks its packed weights straight to
    int8 (per-column factors from qgemm_i8_colscale, computed once here as at
    load) on the same rotating weight copies.  Per-launch times from HIP
    events in a profiling pass, the step time from the wall clock over
    --steps steps between synchronisations, the dominant GEMM's time from
    events around it inside that region (as for the main line)."""
    import torch

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr())

    dev = gemms[0]["y"].device
    quant, arm = {}, []
    for g in gemms:
        M, N, K, dt = g["M"], g["N"], g["K"], g["dt"]
        grp, zp, f = (g["group"] if g["fmt"] == "w4a16" else 0), int(not g["sym"]), qg.FORMATS[g["fmt"]]
        rw = torch.empty(N, dtype=torch.float32, device=dev)
        sw = torch.empty(N, dtype=torch.float32, device=dev)
        st = lib.qgemm_i8_colscale(f, ptr(g["wp"]), ptr(rw), ptr(sw), N, K, grp, zp, sp)
        if st != 0:
            raise qg.QGemmError("qgemm_i8_colscale", st)
        prep = None
        if g["src"] not in quant:
            xq = torch.empty(qg.i8_xq_bytes(M, K), dtype=torch.int8, device=dev)
            sx = torch.empty(M, dtype=torch.float32, device=dev)
            quant[g["src"]] = (xq, sx)
            prep = dict(label=f"i8_quantize({wl['gemms'][g['src']][0]})", M=M, K=K,
                        call=functools.partial(lib.qgemm_i8_quantize, ptr(g["x"]), ptr(xq), ptr(sx), M, K, dt, sp),
                        bytes=2.0 * M * K + qg.i8_xq_bytes(M, K) + 4.0 * M)
        xq, sx = quant[g["src"]]
        nws = qg.i8_workspace_bytes(g["fmt"], -1, M, N, K)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        # rw and sw are the same for every copy of the weights
        calls = [functools.partial(lib.qgemm_i8_gemm, f, -1, ptr(xq), ptr(sx), ptr(w), ptr(rw), ptr(sw), ptr(g["y"]),
                                   M, N, K, grp, zp, dt, ptr(ws), nws, sp) for w in g["pool"]]
        arm.append(dict(g=g, prep=prep, calls=calls, turn=0, rw=rw, sw=sw, ws=ws,
                        rung=qg.i8_select_rung(g["fmt"], M, N, K)["name"]))

    def run(a, which):
        if which == "prep":
            st = a["prep"]["call"]()
        else:
            st = a["calls"][a["turn"] % len(a["calls"])]()
            a["turn"] += 1
        if st != 0:
            raise qg.QGemmError(f"int8 {a['g']['label']} {which}", st)

    for _ in range(max(1, args.warmup)):
        for a in arm:
            if a["prep"] is not None:
                run(a, "prep")
            run(a, "gemm")
    torch.cuda.synchronize()
    nprof = max(3, min(args.steps, PROFILE_STEPS))
    evg = [[timer.pair() for _ in arm] for _ in range(nprof)]
    evp = [[timer.pair() for _ in arm] for _ in range(nprof)]
    for s in range(nprof):
        for j, a in enumerate(arm):
            if a["prep"] is not None:
                timer.record(evp[s][j][0], sp)
                run(a, "prep")
                timer.record(evp[s][j][1], sp)
            timer.record(evg[s][j][0], sp)
            run(a, "gemm")
            timer.record(evg[s][j][1], sp)
    torch.cuda.synchronize()
    gemm_ms = [float(np.mean([timer.ms(*evg[s][j]) for s in range(nprof)])) for j in range(len(arm))]
    jd = int(np.argmax(gemm_ms))
    evd = [timer.pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for j, a in enumerate(arm):
            if a["prep"] is not None:
                run(a, "prep")
            if j == jd:
                timer.record(evd[s][0], sp)
                run(a, "gemm")
                timer.record(evd[s][1], sp)
            else:
                run(a, "gemm")
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    gemm_ms[jd] = float(np.mean([timer.ms(e0, e1) for e0, e1 in evd]))
    per = []
    for j, a in enumerate(arm):
        if a["prep"] is not None:
            p = a["prep"]
            ms = float(np.mean([timer.ms(*evp[s][j]) for s in range(nprof)]))
            per.append(dict(label=p["label"], M=p["M"], K=p["K"], rung="i8_quantize", ms=round(ms, 5),
                            gbps=round(p["bytes"] / ms / 1e6, 1)))
        g = a["g"]
        per.append(dict(label=g["label"], fmt=g["fmt"], M=g["M"], K=g["K"], N=g["N"], rung=a["rung"],
                        ms=round(gemm_ms[j], 5), tops=round(g["flops"] / gemm_ms[j] / 1e9, 2),
                        weight_copies=len(g["pool"])))
    ops = sum(a["g"]["flops"] for a in arm)
    gd = arm[jd]["g"]
    dom = next(p for p in per if p.get("fmt") and p["label"] == gd["label"])
    dom["timed_in_step"] = True
    out = {"what": "the same step with per-row int8 activations (quantized inside the step) and weights unpacked to "
                   "int8 inside the GEMM (per-column scales computed once at load): bit-exact to its own definition, "
                   "an approximation of the fp16 path's result",
           "ms_per_step": round(ms_step, 5), "tops": round(ops / (ms_step * 1e-3) / 1e12, 3), "unit": "TOP/s",
           "per_kernel": per,
           "roofline": {"bound": "mfma", "achieved": dom["tops"], "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                        "frac": round(dom["tops"] / PEAK_INT8_TOPS, 4),
                        "kernel": f"{gd['label']} ({gd['fmt']} M={gd['M']} K={gd['K']} N={gd['N']}, rung "
                                  f"{arm[jd]['rung']})"}}
    if args.workload == "qwen3_8b_layer_m658" and args.only is None:
        out["prefill_tok_s_linear_only"] = round(synth.QWEN3_8B_PROMPT / (synth.QWEN3_8B_LAYERS * ms_step * 1e-3), 1)
    return out


def read_ceiling(pool, reps: int = 30) -> float:
    """GB/s of the streaming-read probe over the same rotating weight copies
    (best of three grid sizes), timed like the GEMMs: HIP events on the launch
    stream around back-to-back launches."""
    import torch

    stream = torch.cuda.current_stream()
    best = 0.0
    for blocks in (1024, 2048, 4096):
        out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        for i in range(3):
            probe.read(pool[i % len(pool)], out, blocks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            probe.read(pool[i % len(pool)], out, blocks)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, pool[0].numel() * pool[0].element_size() / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9)
    return round(best, 1)


def copy_calibration(nbytes: int) -> int:
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read
    for it gives the scale of those counters."""
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 3}), flush=True)
    return 0


def _oracle_leg(items, rows_cap, target_s):
    """Time the oracle on `items` (dicts with fmt, enc, N, K, M, dt, X): the
    full dequant of every weight, then the fp64 GEMM of the first r and 2r
    rows of each (r grown by 4x until r >= 8 and the 2r run takes about
    target_s / 4, or 2r reaches all rows).  Rows are independent and cost the same, so the
    GEMM time is linear in the rows plus a fixed part (the oracle's
    transposed copy of W): the two runs give both, and the GEMM time of all
    rows follows.  Returns (unpack seconds, GEMM seconds for all rows, r)."""
    import oracle

    t0 = time.perf_counter()
    Ws = [oracle.dequant(g["fmt"], g["enc"], g["N"], g["K"], g["dt"]) for g in items]
    t_unpack = time.perf_counter() - t0

    def run(rows):
        t0 = time.perf_counter()
        for g, W in zip(items, Ws):
            oracle.gemm(g["X"][:min(rows, g["M"])], W, g["dt"], want_bound=False)
        return time.perf_counter() - t0

    Mmin = min(g["M"] for g in items)
    r = 1
    while True:
        t2 = run(min(2 * r, Mmin))
        if 2 * r >= min(Mmin, rows_cap) or (t2 >= target_s / 4 and r >= 8):
            break
        r *= 4
    if 2 * r >= Mmin and all(g["M"] == Mmin for g in items):
        return t_unpack, run(Mmin), Mmin  # every row timed
    t1 = run(r)
    per_row = max(t2 - t1, 0.0) / r
    fixed = max(t1 - per_row * r, 0.0)
    # (items share a row count or the smallest bounds it; each item's rows beyond it cost per_row / len(items) on average)
    total = fixed + sum(per_row / len(items) * g["M"] for g in items)
    return t_unpack, total, r


def cpu_baseline(gemms, target_s: float, xf_layout: bool = False) -> dict:
    """The oracle as it stands, on the host's cores: the step's weights
    unpacked in full and the fp64 GEMM of a row sample extrapolated to all
    rows (reported in the metric's unit, unpack and GEMM also apart), and the
    single Q4_K GEMM workloads (16x1024x512 and the FFN up projection at
    M = 512) on all cores and on one."""
    import oracle

    cores = oracle.num_threads()
    flops = sum(g["flops"] for g in gemms)
    t_copy = 0.0
    if xf_layout:
        t0 = time.perf_counter()
        for g in gemms:
            if g["prep"] is not None:
                oracle.fragment_major(g["X"])
        t_copy = time.perf_counter() - t0
    unpack, gemm_s, rows = _oracle_leg(gemms, 10 ** 9, target_s)
    full = unpack + gemm_s + t_copy
    out = {"value": round(flops / full / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "nproc": os.cpu_count(),
           "unpack_s": round(unpack, 3), "gemm_s_extrapolated": round(gemm_s, 3), "layout_copy_s": round(t_copy, 3),
           "sample": f"full dequant of all {len(gemms)} weights ({unpack:.2f} s) + fp64 GEMM of the first {rows} rows "
                     f"of each linear, extrapolated linearly to all rows ({gemm_s:.1f} s)"
                     f"{' + the oracle layout copies of the inputs' if xf_layout else ''}; {cores} OpenMP threads"}
    try:
        configs = {}
        for name in ("q4k_small", "q4k_ffn_up_m512"):
            X, _fields, enc = synth.workload_inputs(name, 0)
            _, fmt, M, K, N, dt, _, _ = synth.WORKLOADS[name]["gemms"][0]
            item = dict(fmt=fmt, enc=enc, N=N, K=K, M=M, dt=dt, X=X)
            leg = {}
            for threads in (cores, 1):
                oracle.set_num_threads(threads)
                u, gs, r = _oracle_leg([item], M, target_s / 6)
                leg["all_cores" if threads == cores else "one_core"] = {
                    "unpack_s": round(u, 4), "gemm_s_extrapolated": round(gs, 4), "rows_timed": r,
                    "gemm_gflops": round(2.0 * M * N * K / gs / 1e9, 3)}
            configs[name] = dict(shape=f"{fmt} M={M} K={K} N={N}", **leg)
        out["configs"] = configs
    finally:
        oracle.set_num_threads(cores)
    return out


if __name__ == "__main__":
    sys.exit(main())
