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

Also after the timed steps, "cases" times every (configuration, matrix, M)
of the workloads on its own (the small-transformer linears at M = 1, 4, 16
with groups 64 and 32; the 7B-class linears at M = 1, 16, 512, 2048; the
[28672, 8192] FFN matrix at M = 1, 8, 256, 4096, and its full-W quantize):
median of five replays of a HIP graph of at least 100 back-to-back calls,
each against its roofline min(HBM, MFMA) from
its algorithmic bytes and flops, M = 1 also against a measured streaming-read
ceiling of the same weight pool, MFMA-bound cases also against a measured
matrix-core ceiling (an MFMA-only probe kernel; the prefill roofline carries
the same fraction); the gated cases (M = 1 at >= 70% of HBM
peak on packed weights + scales for the 7B-class and FFN matrices, M = 2048
at >= 50% of the fp16 MFMA peak) report pass or fail. --no-report skips it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-probe]
       [--no-unfused] [--no-report]

--copy-probe adds, after the timed region, three plain device-to-device
copies of 512 MiB: under rocprofv3 --pmc they give the FETCH_SIZE and
WRITE_SIZE readings of a kernel whose HBM traffic is known, which calibrates
the same counters on the path's kernels.

--decode-traffic runs, instead of the benchmark, three eager int4_linear_ws
calls on each matrix of DECODE_TRAFFIC_CASES (the 5-16 row kernel and the
M = 1 kernels it is compared with) and then the copy probe, for the same two
counter runs; python bench.py --summarize-decode-pmc FETCH_CSV WRITE_CSV
OUT_TXT writes their per-call HBM bytes beside the algorithmic bytes.

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
    """sha256 of the kernel sources (.hip files and their device headers; the
    host-side C ABI in api.cpp launches them but moves no bytes)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h"))):
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


# (configuration, matrix, N, K, M) of the decode traffic check, in launch order
DECODE_TRAFFIC_CASES = [("c4", "q_proj", 4096, 4096, 1), ("c4", "q_proj", 4096, 4096, 16),
                        ("c4", "up_proj", 11008, 4096, 1), ("c4", "up_proj", 11008, 4096, 16),
                        ("c4", "down_proj", 4096, 11008, 1), ("c4", "down_proj", 4096, 11008, 16),
                        ("c5", "ffn", 28672, 8192, 1), ("c5", "ffn", 28672, 8192, 8),
                        ("c5", "ffn", 28672, 8192, 16)]
DECODE_TRAFFIC_CALLS = 3


def decode_traffic(dev):
    """Three eager int4_linear_ws calls per case of DECODE_TRAFFIC_CASES (fp16 x,
    fp32 y, the workspace the shape asks for), then the copy probe."""
    import torch
    import dequantizing_gemm_amd as dq
    import workloads
    L = dq.lib
    st = torch.cuda.current_stream().cuda_stream
    for cfg, name, N, K, M in DECODE_TRAFFIC_CASES:
        gen = torch.Generator(device=dev).manual_seed(N + K)
        w = torch.randn((N, K), generator=gen, device=dev) * 0.02
        p, sc, _ = dq.quantize_int4(w, GROUP)
        del w
        x = torch.from_numpy(workloads.activations(M, K)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = dq.linear_workspace(M, N, K, GROUP, device=dev)
        for _ in range(DECODE_TRAFFIC_CALLS):
            assert L.int4_linear_ws(x.data_ptr(), 1, M, p.data_ptr(), sc.data_ptr(), None, N, K, GROUP, None,
                                    0, y.data_ptr(), 0, ws.data_ptr() if ws.numel() else None, ws.numel(),
                                    st) == 0
        torch.cuda.synchronize()
        print(f"bench: decode traffic {cfg} {name} [{N},{K}] M={M} ({dq.matmul_select(x, p, sc, K, GROUP)})",
              file=sys.stderr, flush=True)
        del p, sc, x, y, ws
        torch.cuda.empty_cache()
    copy_probe(dev)


def copy_probe(dev):
    """Three plain device-to-device copies of COPY_PROBE_BYTES (the counters'
    calibration)."""
    import torch
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def summarize_decode_pmc(fetch_csv, write_csv, out_txt, command=""):
    """Per-call HBM bytes of the int4_linear_ws calls of `bench.py
    --decode-traffic` from its two counter runs (FETCH_SIZE, WRITE_SIZE),
    scaled by the copy calibration like summarize_pmc; the matmul dispatches
    come DECODE_TRAFFIC_CALLS per case in the order of DECODE_TRAFFIC_CASES."""
    import csv
    import statistics
    per = {}
    factors = {}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        copy_max = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        factors[label] = COPY_PROBE_BYTES / 1024 / copy_max
        mm = [r for r in rows if "matmul" in r["Kernel_Name"]]
        if len(mm) != DECODE_TRAFFIC_CALLS * len(DECODE_TRAFFIC_CASES):
            raise SystemExit(f"{path}: {len(mm)} matmul dispatches, expected "
                             f"{DECODE_TRAFFIC_CALLS * len(DECODE_TRAFFIC_CASES)}")
        for i, case in enumerate(DECODE_TRAFFIC_CASES):
            grp = mm[i * DECODE_TRAFFIC_CALLS:(i + 1) * DECODE_TRAFFIC_CALLS]
            per.setdefault(case, {})[label] = statistics.median(float(r["Counter_Value"]) for r in grp) \
                * 1024 * factors[label]
            per[case]["kernel"] = grp[0]["Kernel_Name"].split("(")[0].replace("void ", "")[:60]
    lines = ["HBM traffic of int4_linear_ws on the decode shapes (median of "
             f"{DECODE_TRAFFIC_CALLS} eager calls each; FETCH_SIZE and WRITE_SIZE scaled by",
             f"the copy calibration: fetch x{factors['fetch']:.4f}, write x{factors['write']:.4f}); "
             "algorithmic = packed codes + scales + x (fp16) + y (fp32)",
             f"kernel sources sha256 {csrc_digest()}",
             f"command: {command}", ""]
    for case in DECODE_TRAFFIC_CASES:
        cfg, name, N, K, M = case
        alg, _ = algorithmic(N, K, GROUP, M)
        f, w = per[case]["fetch"], per[case]["write"]
        lines.append(f"{cfg} {name:9s} [{N},{K}] M={M:<2d} {per[case]['kernel']:60s} fetch {f / 1e6:9.3f} MB  "
                     f"write {w / 1e6:7.3f} MB  algorithmic {alg / 1e6:9.3f} MB  traffic/algorithmic "
                     f"{(f + w) / alg:.3f}")
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_csv, steps, out_txt, command=""):
    """Per-shape kernel durations of the timed steps from a rocprofv3
    --kernel-trace CSV of `bench.py --steps STEPS --no-unfused --no-report
    --no-cpu-baseline`: in each phase's kernel family the last STEPS x
    (launches per step) dispatches are the timed ones (nothing launches after
    them in that run), and within a phase the shape of a dispatch is its
    position mod 3 (every phase launches the shapes in the order of SHAPES)."""
    import csv
    import statistics

    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    per_step = {"quantize": 3, "unpack": 3, "prefill_m2048": 3}
    out = [f"rocprofv3 kernel trace of the timed steps, per shape (median, mean, min, max of the",
           f"dispatch durations; timed steps only)", f"command: {command}", ""]
    work = {}
    for name, N, K in SHAPES:
        work[name] = {"quantize": N * K * 4 + packed_weight_bytes(N, K),
                      "unpack": N * ((K + 1) // 2) + N * K,
                      "decode_m1": packed_weight_bytes(N, K),
                      "prefill_m2048": 2 * M_PREFILL * N * K}
    for phase, frag in PHASE_KERNELS.items():
        d = [r for r in rows if frag in r["Kernel_Name"]]
        if not d:
            continue
        count = per_step.get(phase)
        if count is None:                      # decode: 3 shapes x R copies per step
            R = max(2, -(-POOL_BYTES // sum(packed_weight_bytes(N, K) for _, N, K in SHAPES)))
            count = 3 * R
        timed = d[-steps * count:]
        out.append(f"{phase} ({frag}), {len(timed)} dispatches")
        unit, peak = ("GB/s", HBM_PEAK_GBS) if phase != "prefill_m2048" else ("TFLOP/s", FP16_MFMA_PEAK_TFLOPS)
        for i, (name, N, K) in enumerate(SHAPES):
            us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed[i::3]]
            med = statistics.median(us)
            rate = work[name][phase] / med / (1e3 if unit == "GB/s" else 1e6)
            out.append(f"  {name:10s} [{N},{K}]  median {med:8.3f} us  mean {statistics.mean(us):8.3f}  "
                       f"min {min(us):8.3f}  max {max(us):8.3f}  -> {rate:8.1f} {unit} "
                       f"({rate / peak:.4f} of peak)")
        allus = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
        tot = sum(work[n][phase] for n, _, _ in SHAPES)
        rate = tot * len(allus) / 3 / sum(allus) / (1e3 if unit == "GB/s" else 1e6)
        out.append(f"  all three: mean {statistics.mean(allus):.3f} us per launch -> {rate:.1f} {unit} "
                   f"({rate / peak:.4f} of peak)")
        out.append("")
    text = "\n".join(out)
    with open(out_txt, "w") as f:
        f.write(text + "\n")
    print(text)


def summarize_counters(out_txt, csvs, command=""):
    """Per-shape medians of the tiled kernel's counters from rocprofv3 --pmc
    runs of `bench.py --steps 2 --warmup 1 --no-unfused --no-report
    --no-cpu-baseline` (one CSV per pass): the prefill phase launches the
    three shapes in the order of SHAPES, so a dispatch's shape is its
    position mod 3 among the tiled kernel's dispatches. Adds the kernel
    clock, the matrix-pipe busy share (the profiler's MfmaUtil expression),
    MFMA flops against 2MNK and each wave-cycle counter as a share of
    SQ_WAVE_CYCLES."""
    import csv
    import statistics

    per = {name: {} for name, _, _ in SHAPES}
    for path in csvs:
        rows = [r for r in csv.DictReader(open(path)) if PHASE_KERNELS["prefill_m2048"] in r["Kernel_Name"]]
        disp = {}
        for r in rows:
            d = disp.setdefault(int(r["Dispatch_Id"]), {"dur_us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
        ids = sorted(disp)
        for i, (name, _, _) in enumerate(SHAPES):
            for k in ids[i::3]:
                for c, v in disp[k].items():
                    per[name].setdefault(c, []).append(v)
    out = ["Counters of the tiled kernel (matmul_tiled_kernel) in the bench's prefill phase, per shape",
           "(medians over the dispatches of all passes; M = 2048, group 128, fp16 x, fp32 y)",
           f"command: {command}", ""]
    for name, N, K in SHAPES:
        m = {c: statistics.median(v) for c, v in per[name].items()}
        out.append(f"{name} [{N},{K}] M={M_PREFILL}: dispatch {m['dur_us']:.1f} us")
        for c in sorted(k for k in m if k != "dur_us"):
            out.append(f"  {c:34s} {m[c]:.6g}")
        if "GRBM_GUI_ACTIVE" in m:
            gui = m["GRBM_GUI_ACTIVE"] / 8                 # the CSV sums the 8 XCDs
            out.append(f"  kernel clock {gui / m['dur_us'] / 1e3:.2f} GHz (GRBM_GUI_ACTIVE / 8 / duration)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                out.append(f"  MfmaUtil {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * 1024):.1f}% "
                           "(MFMA busy cycles / (GUI-active cycles x 1024 SIMDs))")
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in m:
            out.append(f"  MFMA flops / 2MNK = {m['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512 / (2 * M_PREFILL * N * K):.4f}")
        if "SQ_WAVE_CYCLES" in m:
            wc = m["SQ_WAVE_CYCLES"]
            shares = [c for c in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                                  "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC", "SQ_WAIT_INST_ANY",
                                  "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS") if c in m]
            out.append("  share of wave cycles: " + ", ".join(f"{c[3:]} {m[c] / wc:.2f}" for c in shares))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            out.append(f"  VALU co-issued in {m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.2f} "
                       "of the matrix pipe's busy cycles")
        if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m:
            out.append(f"  VALU instructions per MFMA: {(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_INSTS_MFMA']:.2f}")
        out.append("")
    text = "\n".join(out)
    with open(out_txt, "w") as f:
        f.write(text + "\n")
    print(text)


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
    captured in a HIP graph of `reps` calls and replayed; the median of five
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
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / reps)
        return sorted(ts)[2]

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


def _graph_times_us(fn, reps, trials=5):
    """Per-call times (microseconds) of `trials` replays of a HIP graph of
    `reps` calls of fn, after one warm replay."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e3 / reps)
    return out


def _reps(period, at_least=100):
    """Calls per timed replay: at least `at_least` back-to-back launches, a
    whole number of turns of a rotation pool of `period` copies."""
    return -(-at_least // period) * period


def _graph_time_us(fn, reps):
    """Median of five graph replays, microseconds per call."""
    import statistics
    return statistics.median(_graph_times_us(fn, reps))


# The measurement gates of the hot path: M = 1 at >= 70% of HBM peak on the
# packed weights + scales, M = 2048 at >= 50% of the dense fp16 MFMA peak.
GATE_HBM_FRAC, GATE_MFMA_FRAC = 0.70, 0.50

# Every (configuration, matrix, M) of the workloads, as the report lists them.
C3_SHAPES = [("c_attn", 2304, 768), ("attn_c_proj", 768, 768), ("c_fc", 3072, 768),
             ("mlp_c_proj", 768, 3072)]


def report_cases():
    cases = []
    for g in (64, 32):
        for name, N, K in C3_SHAPES:
            for M in (1, 4, 16):
                cases.append(("c3", f"{name}_g{g}", N, K, g, M))
    for name, N, K in SHAPES:
        for M in (1, 16, 512, 2048):
            cases.append(("c4", name, N, K, GROUP, M))
    for M in (1, 8, 256, 4096):
        cases.append(("c5", "ffn", 28672, 8192, GROUP, M))
    return cases


def algorithmic(N, K, g, M):
    """(bytes, flops) one int4_matmul call must move and compute: packed
    weights, scales, x (fp16) and y (fp32); 2 M N K."""
    return packed_weight_bytes(N, K, g) + 2 * M * K + 4 * M * N, 2 * M * N * K


_probe = None


def _probe_lib():
    """The measurement probes (dequantizing_gemm_amd/probe), loaded by path."""
    global _probe
    if _probe is None:
        import ctypes
        path = os.path.join(ROOT, "dequantizing_gemm_amd", "probe", "libint4dq_probe.so")
        lib = ctypes.CDLL(path)
        lib.int4dq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                 ctypes.c_int, ctypes.c_void_p]
        lib.int4dq_probe_stream_read.restype = ctypes.c_int
        lib.int4dq_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.int4dq_probe_mfma.restype = ctypes.c_int
        _probe = lib
    return _probe


def mfma_ceiling():
    """Measured dense binary16 matrix-core rate (TFLOP/s): the probe kernel
    (eight independent chains of v_mfma_f32_32x32x16_f16 per wavefront, four
    wavefronts per SIMD, nonzero operands, no memory traffic), median of five
    launches of about 2 ms after three warm ones (the first launches after an
    idle spell run at a lower clock). The ceiling MFMA-bound cases are
    compared with beside the nominal peak."""
    import statistics
    import torch
    lib = _probe_lib()
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    blocks, iters = 1024, 4096
    flops = blocks * 4 * iters * 8 * 32768

    def launch():
        assert lib.int4dq_probe_mfma(blocks, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    return flops / statistics.median(ts) / 1e12


def stream_read_ceiling(copies):
    """Measured streaming-read rate (GB/s) over a rotation pool, timed like the
    matmul (graph replays, median of five): a plain read of each copy's packed
    bytes (the probe kernel: 1 KB per wavefront load, four loads in flight per
    lane, 8 blocks of 4 wavefronts per CU), the bytes int4_matmul streams at
    M = 1 less the 1.5% of scales; the faster of 512 and 2048 blocks, the
    better launch shape for large and for small pools)."""
    import torch
    lib = _probe_lib()
    sink = torch.zeros(1, dtype=torch.int32, device=copies[0][0].device)
    best = float("inf")
    for blocks in (512, 2048):                 # the faster of two launch shapes
        it = {"k": 0}

        def call():
            p = copies[it["k"] % len(copies)][0]
            it["k"] += 1
            assert lib.int4dq_probe_stream_read(p.data_ptr(), p.numel(), sink.data_ptr(), blocks,
                                                torch.cuda.current_stream().cuda_stream) == 0
        best = min(best, _graph_time_us(call, _reps(len(copies))))
    return copies[0][0].numel() / best / 1e3


def case_report(dev, mfma_ceil=None):
    """Every case of the report timed on its own (int4_linear_ws, binary32 y, with
    the workspace its shape asks for): HIP graphs of at least 100 calls,
    median of five replays (min and max beside it); for M <= 16 the weights
    rotate through a >= 1 GiB pool of copies so every launch streams them from
    HBM. Each case gets its roofline min(HBM, MFMA) from its algorithmic bytes
    and flops; M = 1 cases also get the streaming-read ceiling of the same pool
    and their fraction of it, cases of 2 to 16 rows their time over the same
    matrix's M = 1 time; MFMA-bound cases their fraction of the measured
    matrix-core ceiling `mfma_ceil` (TFLOP/s) when given; the gated cases (M = 1
    on the 7B-class and FFN matrices, M = 2048 on the 7B-class matrices) report
    pass or fail."""
    import statistics
    import numpy as np
    import torch
    import dequantizing_gemm_amd as dq
    import workloads

    L = dq.lib
    out = []

    def cur():
        return torch.cuda.current_stream().cuda_stream

    by_matrix = {}
    for c in report_cases():
        by_matrix.setdefault(c[:5], []).append(c[5])
    for (cfg, name, N, K, g), Ms in by_matrix.items():
        print(f"bench: report {cfg} {name} [{N},{K}] g={g}", file=sys.stderr, flush=True)
        if cfg == "c5":
            gen = torch.Generator(device=dev).manual_seed(0)
            w = torch.randn((N, K), generator=gen, device=dev) * 0.02
        else:
            case = workloads.Case(name, N, K, g, 0.02, cfg == "c4")
            w = torch.from_numpy(workloads.weights(case)).to(dev)
        p0, s0, _ = dq.quantize_int4(w, g)
        if cfg == "c5":
            # full-W quantize: fp32 read, packed codes and scales written
            qb = N * K * 4 + packed_weight_bytes(N, K, g)
            pq, sq = torch.empty_like(p0), torch.empty_like(s0)

            def qcall():
                assert L.int4_quantize(w.data_ptr(), N, K, g, pq.data_ptr(), sq.data_ptr(), cur()) == 0
            ts = _graph_times_us(qcall, _reps(1))
            us = statistics.median(ts)
            out.append({"case": f"c5 int4_quantize [{N},{K}] g={g} (full W)", "time_us": round(us, 3),
                        "min_us": round(min(ts), 3), "max_us": round(max(ts), 3),
                        "achieved": round(qb / us / 1e3, 1), "unit": "GB/s", "bound": "hbm",
                        "frac_of_peak": round(qb / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": qb})
            del pq, sq
        del w
        wb = packed_weight_bytes(N, K, g)
        copies = [(p0, s0)]
        if min(Ms) <= 16:
            copies += [(p0.clone(), s0.clone()) for _ in range(max(1, -(-POOL_BYTES // wb) - 1))]
        ceiling = stream_read_ceiling(copies) if 1 in Ms else None
        t_m1 = None
        for M in Ms:
            x = torch.from_numpy(workloads.activations(M, K)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            pool = copies if M <= 16 else copies[:1]
            ws = dq.linear_workspace(M, N, K, g, device=dev)      # split of K where it helps
            wptr = ws.data_ptr() if ws.numel() else None
            it = {"k": 0}

            def call():
                p, s_ = pool[it["k"] % len(pool)]
                it["k"] += 1
                assert L.int4_linear_ws(x.data_ptr(), 1, M, p.data_ptr(), s_.data_ptr(), None, N, K, g,
                                        None, 0, y.data_ptr(), 0, wptr, ws.numel(), cur()) == 0
            ts = _graph_times_us(call, _reps(len(pool)))
            us = statistics.median(ts)
            nbytes, flops = algorithmic(N, K, g, M)
            t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e3), flops / (FP16_MFMA_PEAK_TFLOPS * 1e6)
            bound = "hbm" if t_hbm >= t_mfma else "mfma"
            rec = {"case": f"{cfg} {name} [{N},{K}] g={g} M={M}",
                   "kernel": dq.matmul_select(x, p0, s0, K, g) + (" split of K" if ws.numel() else ""),
                   "time_us": round(us, 3), "min_us": round(min(ts), 3), "max_us": round(max(ts), 3),
                   "bound": bound, "roofline_us": round(max(t_hbm, t_mfma), 3),
                   "frac_of_roofline": round(max(t_hbm, t_mfma) / us, 4),
                   "gbs": round(nbytes / us / 1e3, 1), "tflops": round(flops / us / 1e6, 2)}
            if M == 1:
                t_m1 = us
            elif M <= 16 and t_m1:
                rec["time_vs_m1"] = round(us / t_m1, 3)
            if M == 1:
                rec["weight_gbs"] = round(wb / us / 1e3, 1)
                rec["weight_frac_of_peak"] = round(wb / us / 1e3 / HBM_PEAK_GBS, 4)
                rec["stream_read_ceiling_gbs"] = round(ceiling, 1)
                rec["frac_of_measured_ceiling"] = round(wb / us / 1e3 / ceiling, 4)
                if cfg in ("c4", "c5"):
                    rec["gate"] = f">= {GATE_HBM_FRAC} of HBM peak on packed weights + scales"
                    rec["pass"] = rec["weight_frac_of_peak"] >= GATE_HBM_FRAC
            if bound == "mfma" and mfma_ceil:
                rec["mfma_ceiling_tflops"] = round(mfma_ceil, 1)
                rec["frac_of_measured_ceiling"] = round(flops / us / 1e6 / mfma_ceil, 4)
            if M == 2048 and cfg == "c4":
                rec["gate"] = f">= {GATE_MFMA_FRAC} of the fp16 MFMA peak"
                rec["pass"] = flops / us / 1e6 / FP16_MFMA_PEAK_TFLOPS >= GATE_MFMA_FRAC
            out.append(rec)
            del x, y, ws
        del copies, p0, s0
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
    ap.add_argument("--no-report", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"))
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_CSV", "STEPS", "OUT_TXT"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="OUT_TXT CSV")
    ap.add_argument("--decode-traffic", action="store_true")
    ap.add_argument("--summarize-decode-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_TXT"))
    args = ap.parse_args()
    if args.summarize_decode_pmc:
        summarize_decode_pmc(*args.summarize_decode_pmc, command=os.environ.get("PMC_COMMAND", ""))
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, command=os.environ.get("PMC_COMMAND", ""))
        return
    if args.summarize_counters:
        out_txt, *csvs = args.summarize_counters
        summarize_counters(out_txt, csvs, command=os.environ.get("PMC_COMMAND", ""))
        return
    if args.summarize_trace:
        csv_path, steps, out_txt = args.summarize_trace
        summarize_trace(csv_path, int(steps), out_txt, command=os.environ.get("TRACE_COMMAND", ""))
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
    if args.decode_traffic:
        decode_traffic(dev)
        return
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
    if not args.no_report:
        print("bench: measured MFMA ceiling", file=sys.stderr, flush=True)
        ceil_tf = mfma_ceiling()
        line["mfma_ceiling_tflops"] = round(ceil_tf, 1)
        for r in roofs:
            if r["bound"] == "mfma":
                r["measured_ceiling"] = round(ceil_tf, 1)
                r["frac_of_measured_ceiling"] = round(r["achieved"] / ceil_tf, 4)
        print("bench: per-case report", file=sys.stderr, flush=True)
        line["cases"] = case_report(dev, ceil_tf)
        gated = [c for c in line["cases"] if "pass" in c]
        line["gates_passed"] = f"{sum(c['pass'] for c in gated)} of {len(gated)}"
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
