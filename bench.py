"""Benchmark of the INT4 quantize -> unpack -> dequantizing-matmul path on one MI355X.

Workload: the 7B-class linear layers [4096,4096], [11008,4096] and [4096,11008]
(weights ~N(0, 0.02) float32 with 0.1% entries x20, group 128; activations
fp16 ~N(0,1); all seeded and synthetic, see workloads.py). One step runs the
whole hot path on the three matrices:
  1. int4_quantize of each fp32 weight matrix (fresh output buffers),
  2. int4_unpack of each packed matrix,
  3. a decode pass at M = 1: int4_matmul over a pool of R copies of the three
     packed matrices (R * 55 MB >= 1 GiB, four times the 256 MB last-level
     cache, so every launch streams its weights from HBM),
  4. a prefill pass at M = 2048: int4_matmul on each matrix.
Inputs are resident in HBM before the timed region. Per-phase durations are
measured with HIP events recorded on the stream the kernels run on.

The headline value is the packed-weight bandwidth of phase 3 (algorithmic
bytes N*ceil(K/2) + 2*N*G per launch over the launch's average duration); the
M = 2048 rate (2*M*N*K flops over the phase's time) is reported beside it,
each as a fraction of the MI355X peak (HBM 8 TB/s; dense fp16 MFMA
2.5 PFLOP/s).

After the timed steps the fused matmul is compared, per shape and outside
the step, with the unfused baseline the engine page measures it against:
int4_dequantize to a float16 w_hat, then a library fp16 GEMM (torch's
F.linear, hipBLASLt) on it ("unfused_baseline"; --no-unfused skips it).

Also after the timed steps, "gated_cases" times each case the path is
measured against on its own: M = 1 on the three shapes and on the
[28672, 8192] FFN matrix (gate: 70% of HBM peak on packed weights + scales),
M = 2048 on the three shapes (gate: 50% of the dense fp16 MFMA peak), and
M = 4096 on the FFN matrix (reported). --no-gates skips it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-probe]

--copy-probe adds, after the timed region, three plain device-to-device
copies of 512 MiB: under rocprofv3 --pmc they give the FETCH_SIZE and
WRITE_SIZE readings of a kernel whose HBM traffic is known, which calibrates
the same counters on the path's kernels.

python bench.py --summarize-pmc FETCH_CSV WRITE_CSV OUT_JSON turns the
counter_collection.csv files of two such runs (one counter each) into
per-launch HBM traffic per phase, scaled by the copy calibration, and records
the sha256 of the kernel sources it was measured on. A later bench run fills
each roofline's "traffic" from that file only while those sources are
unchanged (else it reports null).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
SHAPES = [("q_proj", 4096, 4096), ("up_proj", 11008, 4096), ("down_proj", 4096, 11008)]
GROUP = 128
M_DECODE, M_PREFILL = 1, 2048
POOL_BYTES = 1 << 30
COPY_PROBE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c4.json")
CSRC = os.path.join(ROOT, "dequantizing_gemm_amd", "csrc")
# kernel-name fragment -> bench phase
PHASE_KERNELS = {"quantize": "quantize_vec_kernel", "unpack": "unpack_flat_kernel",
                 "decode_m1": "matmul_gemv", "prefill_m2048": "matmul_tiled_kernel"}


def csrc_digest():
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def summarize_pmc(fetch_csv, write_csv, out_json, command=""):
    """Per-phase HBM bytes per launch from two rocprofv3 --pmc runs of
    `bench.py --copy-probe` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by (512 MiB / its largest reading on the runtime's
    copy kernel), i.e. by what it reads for the probe copy of known size.
    Every phase launches the three shapes in the order of SHAPES, so within a
    kernel family the shape of a dispatch is its position mod 3."""
    import csv
    import statistics

    out = {"source_sha256": csrc_digest(), "command": command, "phases": {}, "shapes": {}}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        copy_max = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        factor = COPY_PROBE_BYTES / 1024 / copy_max
        out[label + "_factor"] = round(factor, 4)
        for phase, frag in PHASE_KERNELS.items():
            vals = [float(r["Counter_Value"]) for r in rows if frag in r["Kernel_Name"]]
            if not vals or len(vals) % len(SHAPES):
                continue
            per_shape = [statistics.median(vals[i::len(SHAPES)]) * 1024 * factor for i in range(len(SHAPES))]
            out["shapes"].setdefault(phase, {})[label + "_bytes"] = {
                name: round(b) for (name, _, _), b in zip(SHAPES, per_shape)}
            out["phases"].setdefault(phase, {})[label + "_bytes_per_launch"] = round(sum(per_shape) / len(SHAPES))
    for ph in out["phases"].values():
        ph["traffic_bytes_per_launch"] = ph.get("fetch_bytes_per_launch", 0) + ph.get("write_bytes_per_launch", 0)
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def measured_traffic():
    """Per-phase traffic from the committed counter summary, or {} if the
    kernel sources have changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("source_sha256") != csrc_digest():
        return {}
    return {k: v["traffic_bytes_per_launch"] for k, v in t.get("phases", {}).items()}


def unfused_comparison(mats, pool, reps=20):
    """Fused int4_matmul against dequantize-to-fp16 + library GEMM, per shape,
    at M = 1 (weights from the HBM rotation pool) and M = 2048. Each variant is
    captured in a HIP graph of `reps` calls and replayed; the best of three
    replays counts. Returns microseconds per call and the HBM bytes each
    variant moves for the weights."""
    import torch
    import torch.nn.functional as F
    import dequantizing_gemm_amd as dq

    L = dq.lib

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) * 1e3 / reps)
        return best

    out = {}
    for M_, key in ((M_DECODE, "m1"), (M_PREFILL, "m2048")):
        tot = {"fused_us": 0.0, "dequant_us": 0.0, "gemm_us": 0.0}
        per = {}
        for i, m in enumerate(mats):
            N, K = m["N"], m["K"]
            x = m["x1"] if M_ == M_DECODE else m["xp"]
            y = m["y1"] if M_ == M_DECODE else m["yp"]
            what = torch.empty((N, K), dtype=torch.float16, device=x.device)
            copies = [pool[r][i] for r in range(len(pool))] if M_ == M_DECODE else [(m["packed"], m["scales"])]
            it = {"k": 0}

            def nxt():
                p, s_ = copies[it["k"] % len(copies)]
                it["k"] += 1
                return p, s_

            def fused():
                p, s_ = nxt()
                assert L.int4_matmul(x.data_ptr(), 1, M_, p.data_ptr(), s_.data_ptr(), N, K, GROUP,
                                     y.data_ptr(), cur()) == 0

            def dequant():
                p, s_ = nxt()
                assert L.int4_dequantize(p.data_ptr(), s_.data_ptr(), N, K, GROUP, 1, what.data_ptr(),
                                         cur()) == 0

            def gemm():
                F.linear(x, what)

            bias = torch.randn(N, device=x.device)

            def fused_bias_relu():
                p, s_ = nxt()
                assert L.int4_matmul_ex(x.data_ptr(), 1, M_, p.data_ptr(), s_.data_ptr(), N, K, GROUP,
                                        bias.data_ptr(), 1, y.data_ptr(), cur()) == 0

            t_f, t_d, t_g = timed(fused), timed(dequant), timed(gemm)
            t_e = timed(fused_bias_relu)
            per[m["name"]] = {"fused_us": round(t_f, 3), "dequant_us": round(t_d, 3),
                              "gemm_us": round(t_g, 3), "fused_bias_relu_us": round(t_e, 3)}
            tot["fused_us"] += t_f
            tot["dequant_us"] += t_d
            tot["gemm_us"] += t_g
            tot["fused_bias_relu_us"] = tot.get("fused_bias_relu_us", 0.0) + t_e
            del what
        unf = tot["dequant_us"] + tot["gemm_us"]
        w_bytes = sum(packed_weight_bytes(m["N"], m["K"]) for m in mats)
        fp16_bytes = sum(2 * m["N"] * m["K"] for m in mats)
        out[key] = {"M": M_, "fused_us": round(tot["fused_us"], 3),
                    "unfused_us": round(unf, 3), "dequant_us": round(tot["dequant_us"], 3),
                    "gemm_us": round(tot["gemm_us"], 3),
                    "fused_bias_relu_us": round(tot["fused_bias_relu_us"], 3),
                    "fused_speedup": round(unf / tot["fused_us"], 3),
                    "weight_bytes_fused": w_bytes,
                    "weight_bytes_unfused": w_bytes + 2 * fp16_bytes,
                    "per_shape": per}
    out["note"] = ("three c4 shapes summed; unfused = int4_dequantize to fp16 w_hat (written to HBM) "
                   "+ F.linear(x, w_hat) (hipBLASLt fp16 GEMM, fp16 output); fused = int4_matmul "
                   "(fp32 output); fused_bias_relu = int4_matmul_ex with a bias and ReLU; "
                   "weights from the HBM rotation pool at M = 1")
    return out


def _graph_time_us(fn, reps):
    """Best of three replays of a HIP graph of `reps` calls, microseconds per call."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e3 / reps)
    return best


# The measurement gates of the hot path: M = 1 at >= 70% of HBM peak on the
# packed weights + scales, M = 2048 at >= 50% of the dense fp16 MFMA peak
# (256 CUs x 4096 flop/clk x 2.4 GHz = 2516.6 TFLOP/s).
GATE_HBM_FRAC, GATE_MFMA_FRAC, MFMA_PEAK_GATE_TFLOPS = 0.70, 0.50, 2516.6


def gated_cases(mats, pool, dev):
    """Each gated case of the path timed on its own (graph replays, best of
    three): the three 7B-class shapes at M = 1 (weights rotating through the
    >= 1 GiB pool) and M = 2048, and the [28672, 8192] FFN matrix at M = 1
    (its own >= 1 GiB pool of quantized N(0, 0.02) weights) and M = 4096
    (reported, not gated)."""
    import torch
    import dequantizing_gemm_amd as dq

    L = dq.lib
    out = []

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def decode_case(name, N, K, copies, x, y):
        it = {"k": 0}

        def call():
            p, s_ = copies[it["k"] % len(copies)]
            it["k"] += 1
            assert L.int4_matmul(x.data_ptr(), 1, 1, p.data_ptr(), s_.data_ptr(), N, K, GROUP,
                                 y.data_ptr(), cur()) == 0
        us = _graph_time_us(call, len(copies))
        gbs = packed_weight_bytes(N, K) / us / 1e3
        gate = GATE_HBM_FRAC * HBM_PEAK_GBS
        out.append({"case": f"{name} [{N},{K}] M=1", "time_us": round(us, 3), "achieved": round(gbs, 1),
                    "unit": "GB/s", "gate": gate, "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                    "pass": gbs >= gate})

    def prefill_case(name, N, K, M_, p, s_, x, y, gated=True):
        def call():
            assert L.int4_matmul(x.data_ptr(), 1, M_, p.data_ptr(), s_.data_ptr(), N, K, GROUP,
                                 y.data_ptr(), cur()) == 0
        us = _graph_time_us(call, 10)
        tf = 2 * M_ * N * K / us / 1e6
        gate = GATE_MFMA_FRAC * MFMA_PEAK_GATE_TFLOPS
        rec = {"case": f"{name} [{N},{K}] M={M_}", "time_us": round(us, 3), "achieved": round(tf, 1),
               "unit": "TFLOP/s", "frac_of_peak": round(tf / MFMA_PEAK_GATE_TFLOPS, 4)}
        if gated:
            rec.update(gate=gate, **{"pass": tf >= gate})
        out.append(rec)

    for i, m in enumerate(mats):
        decode_case(m["name"], m["N"], m["K"], [pool[r][i] for r in range(len(pool))], m["x1"], m["y1"])
    for m in mats:
        prefill_case(m["name"], m["N"], m["K"], M_PREFILL, m["packed"], m["scales"], m["xp"], m["yp"])

    N, K = 28672, 8192
    gen = torch.Generator(device=dev).manual_seed(0)
    w = torch.randn((N, K), generator=gen, device=dev) * 0.02
    p0, s0, _ = dq.quantize_int4(w, GROUP)
    del w
    copies = [(p0, s0)] + [(p0.clone(), s0.clone())
                           for _ in range(max(1, -(-POOL_BYTES // packed_weight_bytes(N, K)) - 1))]
    x1 = torch.randn((1, K), generator=gen, device=dev).half()
    y1 = torch.empty((1, N), device=dev)
    decode_case("ffn", N, K, copies, x1, y1)
    del copies
    x4 = torch.randn((4096, K), generator=gen, device=dev).half()
    y4 = torch.empty((4096, N), device=dev)
    prefill_case("ffn", N, K, 4096, p0, s0, x4, y4, gated=False)
    del x4, y4, p0, s0
    torch.cuda.empty_cache()
    return out


def packed_weight_bytes(N, K, g=GROUP):
    return N * ((K + 1) // 2) + 2 * N * ((K + g - 1) // g)


def cpu_baseline(min_seconds: float = 10.0):
    """The oracle (scalar C, single thread) on a bounded sample of the same
    workload: repeated M = 1 passes over the three matrices until at least
    `min_seconds` of CPU time, in the headline unit (packed-weight GB/s)."""
    import numpy as np
    import oracle
    import workloads
    data = []
    for name, N, K in SHAPES:
        case = workloads.Case(name, N, K, GROUP, 0.02, True)
        p, s, _ = oracle.quantize_int4(workloads.weights(case), GROUP)
        data.append((p, s, K, workloads.activations(M_DECODE, K)))
    passes, t_total = 0, 0.0
    while t_total < min_seconds:
        t0 = time.perf_counter()
        for (p, s, K, x) in data:
            oracle.int4_matmul(x, p, s, K, GROUP)
        t_total += time.perf_counter() - t0
        passes += 1
    nbytes = passes * sum(packed_weight_bytes(N, K) for _, N, K in SHAPES)
    # the same oracle at M = 2048 on a 4-row sample of x, as flops/s
    p, s, K, _ = data[0]
    x4 = workloads.activations(4, K)
    t0 = time.perf_counter()
    oracle.int4_matmul(x4, p, s, K, GROUP)
    t_mm = time.perf_counter() - t0
    return {
        "value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{passes} M=1 passes of the scalar C oracle over the three matrices "
                  f"({t_total:.1f} s, 1 thread of os.cpu_count()={os.cpu_count()}, "
                  f"affinity={len(os.sched_getaffinity(0))})",
        "m2048_tflops_from_4_rows": round(2 * 4 * 4096 * 4096 / t_mm / 1e12, 6),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-gates", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"))
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, command=os.environ.get("PMC_COMMAND", ""))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path has no "
              "multi-GPU leg; a sharded layout is described in the design notes.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import dequantizing_gemm_amd as dq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating inputs", file=sys.stderr, flush=True)

    mats = []
    for name, N, K in SHAPES:
        case = workloads.Case(name, N, K, GROUP, 0.02, True)
        w = torch.from_numpy(workloads.weights(case)).to(dev)
        x1 = torch.from_numpy(workloads.activations(M_DECODE, K)).to(dev)
        xp = torch.from_numpy(workloads.activations(M_PREFILL, K)).to(dev)
        packed, scales, _ = dq.quantize_int4(w, GROUP)
        mats.append(dict(name=name, N=N, K=K, w=w, x1=x1, xp=xp, packed=packed, scales=scales,
                         q_out=torch.empty_like(packed), s_out=torch.empty_like(scales),
                         u_out=torch.empty((N, K), dtype=torch.int8, device=dev),
                         y1=torch.empty((M_DECODE, N), dtype=torch.float32, device=dev),
                         yp=torch.empty((M_PREFILL, N), dtype=torch.float32, device=dev)))
    set_bytes = sum(packed_weight_bytes(m["N"], m["K"]) for m in mats)
    R = max(2, -(-POOL_BYTES // set_bytes))
    pool = [[(m["packed"].clone(), m["scales"].clone()) for m in mats] for _ in range(R)]
    torch.cuda.synchronize()

    L = dq.lib

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def launch_quantize():
        for m in mats:
            rc = L.int4_quantize(m["w"].data_ptr(), m["N"], m["K"], GROUP, m["q_out"].data_ptr(),
                                 m["s_out"].data_ptr(), cur())
            assert rc == 0

    def launch_unpack():
        for m in mats:
            assert L.int4_unpack(m["q_out"].data_ptr(), m["N"], m["K"], m["u_out"].data_ptr(), cur()) == 0

    def launch_decode():
        for r in range(R):
            for m, (p, s) in zip(mats, pool[r]):
                assert L.int4_matmul(m["x1"].data_ptr(), 1, M_DECODE, p.data_ptr(), s.data_ptr(),
                                     m["N"], m["K"], GROUP, m["y1"].data_ptr(), cur()) == 0

    def launch_prefill():
        for m in mats:
            assert L.int4_matmul(m["xp"].data_ptr(), 1, M_PREFILL, m["packed"].data_ptr(),
                                 m["scales"].data_ptr(), m["N"], m["K"], GROUP, m["yp"].data_ptr(),
                                 cur()) == 0

    # The decode pass is 3*R short launches: replay it as one HIP graph so that
    # per-launch host overhead (ctypes + hipLaunchKernel) does not gate the GPU.
    for _ in range(2):
        launch_decode()
    torch.cuda.synchronize()
    eager_y1 = [m["y1"].clone() for m in mats]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_decode()
    torch.cuda.synchronize()
    for m in mats:
        m["y1"].zero_()
    for rep in range(3):                 # every replay must reproduce the eager result
        graph.replay()
        torch.cuda.synchronize()
        for m, ref in zip(mats, eager_y1):
            assert torch.equal(m["y1"], ref), f"graph replay {rep} differs for {m['name']}"

    phases = [("quantize", launch_quantize), ("unpack", launch_unpack), ("decode_m1", graph.replay),
              ("prefill_m2048", launch_prefill)]

    def step(events=None):
        for i, (_, fn) in enumerate(phases):
            if events is not None:
                events[i].record()
            fn()
        if events is not None:
            events[len(phases)].record()

    print(f"bench: warmup {args.warmup} steps (pool of {R} weight copies, "
          f"{R * set_bytes / 1e9:.2f} GB)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phase_ms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, (name, _) in enumerate(phases)}
    print(f"bench: timed {args.steps} steps in {wall:.3f} s; per-phase ms {phase_ms}",
          file=sys.stderr, flush=True)

    # algorithmic work per phase and per launch
    q_bytes = sum(m["N"] * m["K"] * 4 + packed_weight_bytes(m["N"], m["K"]) for m in mats)
    u_bytes = sum(m["N"] * ((m["K"] + 1) // 2) + m["N"] * m["K"] for m in mats)
    d_bytes = R * set_bytes
    p_flops = sum(2 * M_PREFILL * m["N"] * m["K"] for m in mats)
    per_launch = {"quantize": 3, "unpack": 3, "decode_m1": 3 * R, "prefill_m2048": 3}

    traffic = measured_traffic()

    def roof(name, bound, work, unit, peak):
        t = phase_ms[name] * 1e-3
        achieved = work / t / (1e9 if unit == "GB/s" else 1e12)
        return {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic.get(name),
                "algorithmic_per_launch": round(work / per_launch[name]),
                "avg_launch_us": round(phase_ms[name] * 1e3 / per_launch[name], 3),
                "launches_per_step": per_launch[name]}

    roofs = [roof("quantize", "hbm", q_bytes, "GB/s", HBM_PEAK_GBS),
             roof("unpack", "hbm", u_bytes, "GB/s", HBM_PEAK_GBS),
             roof("decode_m1", "hbm", d_bytes, "GB/s", HBM_PEAK_GBS),
             roof("prefill_m2048", "mfma", p_flops, "TFLOP/s", FP16_MFMA_PEAK_TFLOPS)]
    dominant = max(roofs, key=lambda r: phase_ms[r["kernel"]])
    decode = roofs[2]
    ms_per_step = wall * 1e3 / args.steps
    line = {
        "metric": "int4_matmul packed-weight HBM GB/s @M=1 + TFLOP/s @M=2048, % of roofline",
        "value": decode["achieved"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4 weights x fp16 activations -> fp32",
        "data": "synthetic",
        "config": {"workload": "7B-class linears [4096,4096],[11008,4096],[4096,11008], "
                               "N(0,0.02) + 0.1% x20 outliers, group 128; x fp16 N(0,1); "
                               f"step = quantize+unpack of all three, M=1 over {R} pooled copies, "
                               "M=2048 on each", "group": GROUP, "m_decode": M_DECODE,
                   "m_prefill": M_PREFILL, "pool_copies": R},
        "m1_frac_of_hbm_peak": decode["frac"],
        "m2048_tflops": roofs[3]["achieved"], "m2048_frac_of_fp16_peak": roofs[3]["frac"],
        "roofline": dominant,
        "rooflines": roofs,
        "phase_ms": {k: round(v, 4) for k, v in phase_ms.items()},
    }
    if not args.no_unfused:
        print("bench: fused vs dequantize-then-GEMM", file=sys.stderr, flush=True)
        line["unfused_baseline"] = unfused_comparison(mats, pool)
        # Context for the prefill fraction: the library's plain fp16 GEMM on
        # the same three shapes at M = 2048 (fp16 weights, fp16 output), timed
        # in the same run; the fused kernel's rate as a fraction of it.
        flops = sum(2.0 * M_PREFILL * m["N"] * m["K"] for m in mats)
        lib_tf = flops / line["unfused_baseline"]["m2048"]["gemm_us"] / 1e6
        line["library_fp16_gemm_m2048"] = {
            "tflops": round(lib_tf, 1), "frac_of_peak": round(lib_tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "fused_frac_of_library": round(roofs[3]["achieved"] / lib_tf, 4),
            "note": "F.linear (hipBLASLt) on the same three shapes, fp16 weights and output"}
    if not args.no_gates:
        print("bench: gated cases", file=sys.stderr, flush=True)
        line["gated_cases"] = gated_cases(mats, pool, dev)
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = COPY_PROBE_BYTES
        del src, dst
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
