"""Benchmark of the blockwise-FP8 MoE FFN forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3_decode|v3_prefill|v3_skew|dense_ffn|tiny]

A step is one moe_ffn_forward (all stages: x quantisation, router GEMM +
sigmoid, group-limited top-k, permutation, gate/up grouped GEMM with fused
SwiGLU + requantisation, down grouped GEMM, combine/cast) over one batch of
seeded synthetic tokens already resident in HBM, with random-init weights of
the DeepSeek-V3 layer shapes (weights are drawn on the device and quantised
with the library's own 128x128 block quantiser before timing).  The default
workload is the V3-shape decode step (T=64).

Prints one JSON line.  ``roofline`` describes the dominant kernel (the gate/up
grouped GEMM) from HIP events that the library records on the launch stream
around it in every timed step (the only events in the timed steps: each record
costs the stream a few microseconds); ``stages_ms`` for the other stages comes
from the same steps run again with every stage event; ``cpu_baseline`` times the CPU oracle on a bounded token
sample of the same workload.  ``roofline.traffic`` is the HBM traffic per launch
of that kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE counters, stored in
profiles/<workload>_gate_up_traffic.md together with a hash of the GEMM sources;
it is reported only while the sources still match (else null).  With the default (decode)
workload the line also carries sub-records timed the same way: ``v3_prefill`` (T = 4096),
``dense_ffn``, ``v3_skew`` (T = 16384, load-skewed), ``v3_prefill_ue8m0`` (power-of-two scales)
and ``v3_prefill_backward`` (the routed experts' FP8 dgrad and wgrad).

Helpers for the counter runs:
  --calibrate-copy MIB     a plain copy of MIB MiB (the library's row gather with the identity
                           permutation): the counters' scale factor.
  --traffic-summary DIR    turns the four counter runs under DIR (fetch/, write/, copy_fetch/,
                           copy_write/; commands in the written file) into
                           profiles/<workload>_gate_up_traffic.md.
  --mfma-summary DIR       turns the MFMA counter run under DIR (mfma/) and a bench line
                           (DIR/bench.json) into profiles/<workload>_mfma_utilization.md.
  --trace-summary DIR      turns a rocprofv3 --kernel-trace --stats run under DIR (ktrace/) and
                           its bench line (DIR/bench.json) into profiles/<workload>_kernel_trace.md.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (no sparsity)
METRIC = "MoE-layer tokens/s + FP8 TFLOP/s (% MFMA peak / % HBM peak) at V3 shapes"


class HipEvents:
    """hipEvent_t handles through the HIP runtime (events are recorded by the library itself)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> ctypes.c_void_p:
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream) -> None:
        assert self.rt.hipEventRecord(e, stream) == 0

    def sync(self, e) -> None:
        assert self.rt.hipEventSynchronize(e) == 0

    def ms(self, a, b) -> float:
        f = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return float(f.value)

    def destroy(self, e) -> None:
        self.rt.hipEventDestroy(e)


def build_layer(shape, dev, ue8m0: bool = False, rmsnorm: bool = False):
    """Device weights of the layer: fp32 draws quantised by fp8_quant_128x128 (power-of-two scales with
    ue8m0), then packed into the GEMMs' fragment order (moe_pack_weights), expert by expert; with rmsnorm
    an RMSNorm weight (bf16, seeded uniform in [0.5, 1.5]) goes in front."""
    import torch

    import sparse_moe_ffn_sigmoid_amd as moe
    import synth
    E, d = shape.n_experts, shape.hidden
    kw = {}
    if E:
        W = shape.inter
        kw["w13_q"] = torch.empty((E, 2 * W, d), dtype=torch.uint8, device=dev)
        kw["w13_s"] = torch.empty((E, 2 * W // 128, d // 128), dtype=torch.float32, device=dev)
        kw["w2_q"] = torch.empty((E, d, W), dtype=torch.uint8, device=dev)
        kw["w2_s"] = torch.empty((E, d // 128, W // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            moe.quantize_pack_128x128(synth.torch_expert_weight(shape, e, "w13", dev), q=kw["w13_q"][e], s=kw["w13_s"][e],
                                      ue8m0=ue8m0)
            moe.quantize_pack_128x128(synth.torch_expert_weight(shape, e, "w2", dev), q=kw["w2_q"][e], s=kw["w2_s"][e],
                                      ue8m0=ue8m0)
        wr = synth.gen_router_w(shape)
        import numpy as np
        kw["w_router"] = torch.from_numpy(wr.view(np.int16)).to(dev).view(torch.bfloat16)
        if shape.skewed:
            kw["bias"] = torch.from_numpy(synth.skew_bias()).to(dev)
    if shape.n_shared:
        a, b = moe.quantize_pack_128x128(synth.torch_expert_weight(shape, E, "w13", dev), ue8m0=ue8m0)
        c, e_ = moe.quantize_pack_128x128(synth.torch_expert_weight(shape, E, "w2", dev), ue8m0=ue8m0)
        kw.update(sh_w13_q=a, sh_w13_s=b, sh_w2_q=c, sh_w2_s=e_)
    if rmsnorm:
        kw["norm_w"] = norm_weight(shape, dev)
    torch.cuda.synchronize()
    return moe.MoeWeights(**kw)


COPY_MIB = 2048
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/common.h", "csrc/launch.h")


def gemm_source_hash() -> str:
    """SHA-256 of the GEMM sources with comments and blank space removed, so that a comment
    edit keeps the stored counters while any change to the code drops them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_moe_ffn_sigmoid_amd", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def gate_up_kernel(shape, ue8m0: bool = False) -> str:
    """Name of the kernel the library runs for the gate/up GEMM of this shape (the library picks
    the weight-streaming kernel when groups average at most 10 rows, its 32-row variant up to 18,
    else the MFMA tile kernel with 64-row tiles up to 56 rows per group on average (64 for a single
    group) and 128-row tiles beyond; the template argument after the epilogue says whether the
    scales are powers of two)."""
    groups = shape.n_experts if shape.n_experts else 1
    rows = shape.tokens * (shape.top_k if shape.n_experts else 1) // groups
    scaled = "true" if ue8m0 else "false"
    if rows <= 10:
        return f"stream_gemm_kernel<2, 2, 6, 2, {scaled}, true>"
    if rows <= 18:
        return f"stream_gemm2_kernel<2, 2, 3, 2, {scaled}, true>"
    mt = 2 if rows <= (56 if groups > 1 else 64) else 4
    return f"mfma_gemm_kernel<2, 4, {mt}, 2, {scaled}>"


def traffic_file(shape) -> str:
    return os.path.join(ROOT, "profiles", f"{shape.name}_gate_up_traffic.md")


def stored_traffic(shape):
    """HBM bytes per launch of the gate/up kernel from the stored counter summary, or None when
    there is none or the GEMM sources changed since the counters were taken."""
    try:
        text = open(traffic_file(shape)).read()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in text.splitlines() if l.startswith(("traffic_bytes_per_launch: ",
                                                                           "source_sha256: ")))
    if kv.get("source_sha256") != gemm_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def calibrate_copy(mib: int) -> None:
    """A plain copy of known size: moe_permute with one expert and k = 1 gathers rows by the
    identity permutation, so its gather kernel (one 16-byte chunk per lane, consecutive lanes on
    consecutive chunks) reads mib MiB of rows (+ 4 bytes of index per row) and writes mib MiB."""
    import torch

    import sparse_moe_ffn_sigmoid_amd as moe
    rows = torch.ones((mib, 1 << 20), dtype=torch.uint8, device="cuda")
    idx = torch.zeros((mib, 1), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        out = moe.moe_permute(idx, 1, rows)[3]
        del out
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": mib << 20, "dispatches": 3}))


def _counter_means(d: str, counter: str, substr: str):
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {substr!r} under {d}")
    return sum(vals) / len(vals), len(vals)


def _gemm_flops(shape):
    """Algorithmic FLOPs of the gate/up and the down grouped GEMM of one layer call."""
    cols = shape.top_k * shape.inter if shape.n_experts else 0
    cols += shape.n_shared * shape.inter_shared
    gu = 2.0 * shape.tokens * shape.hidden * 2 * cols
    return gu, gu / 2


def mfma_summary(d: str, shape) -> None:
    """MFMA utilisation of the two grouped GEMMs from one rocprofv3 counter run: busy fraction of
    the MFMA pipes (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles of the dispatch; GRBM_GUI_ACTIVE
    counts the dispatch's cycles once per XCD, so it is divided by the 8 XCDs), pipe cycles per
    MFMA instruction, the clock the counters imply, and the kernels' FLOP rate at the live
    durations of the bench line in DIR/bench.json."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(d, "mfma", "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            if "gemm_kernel" not in k:
                continue
            e = per.setdefault(k.split("(")[0].replace("void ", "").replace("moefp8::", ""), {})
            e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            e.setdefault("_ns", {})[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        raise SystemExit(f"no GEMM rows under {d}/mfma")
    live = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    gu, dn = _gemm_flops(shape)
    cmd = f"python3 $R/bench.py --workload {shape.name} --steps 3 --warmup 1 --no-cpu-baseline"
    lines = [
        f"# MFMA utilisation of the grouped GEMMs, {shape.name}", "",
        "Commands (R = repository root, OUT = the directory the runs write to; the counter run from `cd /tmp && export TMPDIR=/tmp`):", "", "```",
        f"timeout -s KILL 120 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_BUSY_CYCLES GRBM_GUI_ACTIVE "
        f"-f csv -d $OUT/mfma -o mfma -- {cmd}",
        f"python3 $R/bench.py --workload {shape.name} --steps 20 --no-cpu-baseline > $OUT/bench.json",
        f"python3 bench.py --workload {shape.name} --mfma-summary $OUT", "```", "",
        "busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs): the fraction of SIMD-cycles",
        "in which the MFMA pipe works. The exact gate/up path runs bf16 16x16x32 MFMAs (16 pipe cycles,",
        "1024 FLOP per cycle and SIMD: its own peak is half the FP8 one); the down GEMM FP8 16x16x128",
        "(32 cycles, 2048 FLOP per cycle). Durations under the profiler run longer than live ones; the",
        "FLOP rates use the live stage times of the bench line (HIP events on the launch stream).", "",
        "| kernel | dispatches | busy | cycles/MFMA | clock GHz (counters) | live ms | TFLOP/s | % FP8 peak |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for name, e in sorted(per.items()):
        n = len(e["SQ_INSTS_MFMA"])
        busy = sum(e["SQ_VALU_MFMA_BUSY_CYCLES"]) / n
        inst = sum(e["SQ_INSTS_MFMA"]) / n
        grbm = sum(e["GRBM_GUI_ACTIVE"]) / n
        ns = sum(e["_ns"].values()) / len(e["_ns"])
        frac = busy / (grbm / 8 * 1024)
        is_gu = name.split("<")[1].split(",")[-2].strip() == "2"     # the epilogue argument: SwiGLU
        ms = live["stages_ms"]["gate_up_gemm" if is_gu else "down_gemm"]
        fl = gu if is_gu else dn
        tf = fl / (ms * 1e-3) / 1e12
        lines.append(f"| `{name}` ({'gate/up' if is_gu else 'down'}) | {n} | {100 * frac:.1f}% | {busy / inst:.1f} | "
                     f"{grbm / 8 / ns:.2f} | {ms:.3f} | {tf:.0f} | {100 * tf / FP8_PEAK_TFLOPS:.1f} |")
    out = os.path.join(ROOT, "profiles", f"{shape.name}_mfma_utilization.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def traffic_summary(d: str, shape) -> None:
    kern = gate_up_kernel(shape)
    f_k, n_f = _counter_means(os.path.join(d, "fetch"), "FETCH_SIZE", kern)
    w_k, n_w = _counter_means(os.path.join(d, "write"), "WRITE_SIZE", kern)
    f_c, _ = _counter_means(os.path.join(d, "copy_fetch"), "FETCH_SIZE", "perm_gather_kernel")
    w_c, _ = _counter_means(os.path.join(d, "copy_write"), "WRITE_SIZE", "perm_gather_kernel")
    n = COPY_MIB << 20
    ff, fw = (n + 4 * COPY_MIB) / (f_c * 1024), n / (w_c * 1024)
    traffic = f_k * 1024 * ff + w_k * 1024 * fw
    bench = f"python3 $R/bench.py --workload {shape.name} --steps 3 --warmup 1 --no-cpu-baseline"
    run = "timeout -s KILL 90 rocprofv3 --pmc {c} -f csv -d $OUT/traffic/{o} -o {o} -- {cmd}"
    lines = [
        f"# HBM traffic of the gate/up GEMM kernel, {shape.name}",
        "",
        "Counter runs (one counter per run, R = repository root, OUT = the directory the runs write to, from `cd /tmp && export TMPDIR=/tmp`):",
        "",
        "```",
        run.format(c="FETCH_SIZE", o="fetch", cmd=bench),
        run.format(c="WRITE_SIZE", o="write", cmd=bench),
        run.format(c="FETCH_SIZE", o="copy_fetch", cmd=f"python3 $R/bench.py --calibrate-copy {COPY_MIB}"),
        run.format(c="WRITE_SIZE", o="copy_write", cmd=f"python3 $R/bench.py --calibrate-copy {COPY_MIB}"),
        f"python3 bench.py --workload {shape.name} --traffic-summary $OUT/traffic",
        "```",
        "",
        f"Kernel: `{kern}` ({n_f} and {n_w} dispatches). Counters are KiB per dispatch.",
        "The copy kernel is the library's row gather (moe_permute with one expert and k = 1: the",
        "identity permutation of 1 MiB rows, one 16-byte chunk per lane), which reads and writes",
        f"{COPY_MIB} MiB (+ 4 bytes of index per row); the factors scale each counter to bytes.",
        "",
        "```",
        f"kernel_FETCH_SIZE_KiB: {f_k:.1f}",
        f"kernel_WRITE_SIZE_KiB: {w_k:.1f}",
        f"copy_FETCH_SIZE_KiB: {f_c:.1f}",
        f"copy_WRITE_SIZE_KiB: {w_c:.1f}",
        f"fetch_factor: {ff:.4f}",
        f"write_factor: {fw:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"source_sha256: {gemm_source_hash()}",
        "```",
        "",
    ]
    with open(traffic_file(shape), "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {traffic_file(shape)}: {traffic / 1e9:.3f} GB per launch")


def trace_summary(d: str, shape) -> None:
    """Turns a `rocprofv3 --kernel-trace --stats` run of this workload's bench (DIR/ktrace, its bench
    line in DIR/bench.json) into profiles/<workload>_kernel_trace.md."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "ktrace", "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}/ktrace")
    rows = list(csv.DictReader(open(files[0])))
    live = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    layer, prep = [], []
    prep_marks = ("at::native", "quant_128x128", "pack_kernel", "copyBuffer", "perm_gather")
    for r in rows:
        name = r["Name"].replace("void ", "").replace("moefp8::", "").split("(")[0]
        short = name if len(name) <= 60 else name[:60] + "\u2026"
        line = (f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                f"{float(r['MaxNs']) / 1e3:.1f} |")
        (prep if any(m in r["Name"] for m in prep_marks) else layer).append(line)
    steps, warm = live["steps"], live["warmup"]
    cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv -d $OUT/ktrace -o kt -- "
           f"python3 $R/bench.py --workload {shape.name} --steps {steps} --warmup {warm} --no-cpu-baseline --no-prefill "
           f"> $OUT/bench.json")
    st = live["stages_ms"]
    lines = [
        f"# Kernel trace, {shape.name} (`moe_ffn_forward`; {warm} warm-up + {steps} timed + {steps} stage-timing calls)",
        "", "Commands (R = repository root, OUT = the directory the run writes to):", "", "```", cmd,
        f"python3 $R/bench.py --workload {shape.name} --trace-summary $OUT", "```", "",
        "Per-launch durations from `kt_kernel_stats.csv` (the layer's kernels; weight preparation before the",
        "timed region is listed apart).", "",
        "| kernel | calls | average µs | min µs | max µs |", "|---|---|---|---|---|", *layer, "",
        "Weight preparation (not timed):", "", "| kernel | calls | average µs | min µs | max µs |", "|---|---|---|---|---|",
        *prep, "", "The same run's bench line (HIP events on the launch stream):", "", "```",
        f"ms_per_step: {live['ms_per_step']:.4f}",
        "stages_ms: " + ", ".join(f"{k} {v:.4f}" for k, v in st.items()),
        f"roofline kernel: {live['roofline']['kernel']}, avg_ms {live['roofline']['avg_ms']:.4f}", "```", ""]
    out = os.path.join(ROOT, "profiles", f"{shape.name}_kernel_trace.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {out}")


def norm_weight(shape, dev):
    import numpy as np
    import torch

    import synth
    g = np.random.default_rng(shape.cfg_id).uniform(0.5, 1.5, shape.hidden).astype(np.float32)
    return torch.from_numpy(synth.f32_to_bf16_bits(g).view(np.int16)).to(dev).view(torch.bfloat16)


def time_launches(hip, stream, fn, n: int = 20) -> float:
    """Average ms of fn() (which enqueues on `stream`) over n launches, HIP events on that stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = hip.create(), hip.create()
    hip.record(a, stream)
    for _ in range(n):
        fn()
    hip.record(b, stream)
    hip.sync(b)
    ms = hip.ms(a, b) / n
    hip.destroy(a)
    hip.destroy(b)
    return ms


def next_rows(shape, x, idx, hip, stream, dev) -> dict:
    """Per-launch timing of the kernels next to the layer, on this workload's tensors: the RMSNorm
    fused with the 1x128 quantisation (x [T, hidden] -> normalised bf16 rows + codes + scales) and
    the routing-bias balancing step on this step's expert choices."""
    import torch

    from sparse_moe_ffn_sigmoid_amd import _lib
    lib = _lib.load()
    T, d = x.shape
    g = norm_weight(shape, dev)
    y = torch.empty_like(x)
    q = torch.empty((T, d), dtype=torch.uint8, device=dev)
    s = torch.empty((T, d // 128), dtype=torch.float32, device=dev)
    args = [ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(g.data_ptr()), 1e-6, T, d, d, ctypes.c_void_p(y.data_ptr()),
            d, ctypes.c_void_p(q.data_ptr()), d, ctypes.c_void_p(s.data_ptr()), 0, stream]
    ms = time_launches(hip, stream, lambda: lib.fp8_rmsnorm_quant_1x128(*args))
    nbytes = T * d * (2 + 2 + 1) + T * (d // 128) * 4 + 2 * d
    res = {"rmsnorm_quant_1x128": {"us": ms * 1e3, "hbm_gbs_algorithmic": nbytes / ms / 1e6,
                                   "pct_hbm_peak": 100 * nbytes / ms / 1e6 / HBM_PEAK_GBS, "bytes": nbytes}}
    if shape.n_experts:
        bias = torch.zeros(shape.n_experts, dtype=torch.float32, device=dev)
        k = idx.shape[1]
        bargs = [ctypes.c_void_p(idx.data_ptr()), T, k, shape.n_experts, 1e-3, ctypes.c_void_p(bias.data_ptr()), None,
                 stream]
        ms = time_launches(hip, stream, lambda: lib.moe_bias_update(*bargs))
        res["bias_update"] = {"us": ms * 1e3, "assignments": T * k}
    return res


def algorithmic_bytes(shape, touched: int) -> dict:
    """Bytes the method must move (codes + scales of experts with load > 0 and the shared
    expert, router weights and bias, x in and the output, both bf16)."""
    d = shape.hidden
    routed = touched * shape.expert_bytes(shape.inter) if shape.n_experts else 0
    shared = shape.expert_bytes(shape.inter_shared) if shape.n_shared else 0
    router = shape.n_experts * d * 2 + shape.n_experts * 4
    io = 2 * shape.tokens * d * 2
    w13 = lambda width: 2 * width * d + 4 * (2 * width // 128) * (d // 128)  # noqa: E731
    gate_up = touched * w13(shape.inter) + (w13(shape.inter_shared) if shape.n_shared else 0)
    gate_up += shape.tokens * (d + 4 * d // 128)                              # x codes + scales in
    rows = shape.tokens * (shape.top_k + shape.n_shared)
    width = shape.inter if shape.n_experts else shape.inter_shared
    gate_up += rows * (width + 4 * width // 128)                              # h codes + scales out
    return {"layer": routed + shared + router + io, "gate_up": gate_up}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, x_bits, n_tokens: int, repeats: int = 3) -> dict:
    """The CPU oracle, as it stands, on the first n_tokens of the same workload: the tokens (independent
    given their routing) are split into one group per host core, each group a plain oracle call in its
    own thread with BLAS held to one thread, so the run uses exactly the cores the process may run on.
    Median wall time of `repeats` runs."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import ffn, route
    cores = len(os.sched_getaffinity(0))
    x = synth.bf16_bits_to_f32(x_bits[:n_tokens])
    wr = synth.bf16_bits_to_f32(synth.gen_router_w(shape)) if shape.n_experts else None
    bias = synth.skew_bias() if shape.skewed else None
    need = [shape.n_experts] if shape.n_shared else []
    if shape.n_experts:
        sc = route.sigmoid_scores(route.router_logits(x, wr))
        idx, _ = route.select(sc, bias, shape.n_group, shape.topk_group, shape.top_k)
        need += sorted(set(int(e) for e in np.unique(idx)))
    dev = torch.device("cuda:0")
    experts = {}
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(cores) as ex:       # oracle-side weight quantisation: preparation, not timed
        for i in range(0, len(need), 32):
            host = {e: (synth.torch_expert_weight(shape, e, "w13", dev).cpu().numpy(),
                        synth.torch_expert_weight(shape, e, "w2", dev).cpu().numpy()) for e in need[i:i + 32]}
            for e, q in ex.map(lambda e: (e, ffn.quantize_expert(*host[e])), list(host)):
                experts[e] = q
            del host
    groups = [g for g in np.array_split(np.arange(n_tokens), cores) if g.size]

    def run(rows):
        return ffn.moe_ffn(x[rows], shape.n_experts, shape.top_k, shape.n_group, shape.topk_group,
                           experts.__getitem__, w_router=wr, bias=bias, n_shared=shape.n_shared)
    times = []
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(len(groups)) as ex:
        for _ in range(repeats):
            t0 = time.perf_counter()
            list(ex.map(run, groups))
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": len(groups), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"all {n_tokens} tokens of {shape.name} (T={shape.tokens}), {len(need)} experts quantised by "
                      f"the oracle beforehand (not timed); {len(groups)} token groups in parallel threads, BLAS at "
                      f"one thread each; median of {repeats} runs: {dt:.1f} s of numpy fp64 on the host "
                      f"(runs {', '.join(f'{t:.1f}' for t in times)} s)"}


def time_workload(shape, steps: int, warmup: int, ue8m0: bool = False, rmsnorm: bool = False,
                  deterministic: bool = False, with_next_rows: bool = True):
    """Builds the layer and times `steps` calls of moe_ffn_forward after `warmup` untimed ones.
    Returns (record, x_bits): the record holds the whole-step timing and rates, the per-stage times
    and the gate/up GEMM's roofline (see the module docstring)."""
    import numpy as np
    import torch

    import sparse_moe_ffn_sigmoid_amd as moe
    import synth
    from sparse_moe_ffn_sigmoid_amd import _lib

    dev = torch.device("cuda:0")
    print(f"[bench] {shape.name}: building weights on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    t_build = time.perf_counter()
    weights = build_layer(shape, dev, ue8m0=ue8m0, rmsnorm=rmsnorm)
    cfg = moe.MoeConfig.of(shape, ue8m0=ue8m0)
    x_bits = synth.gen_x(shape)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    T = shape.tokens
    ws = moe.alloc_workspace(T, cfg, dev)
    out = torch.empty_like(x)
    idx = torch.empty((T, max(shape.top_k, 1)), dtype=torch.int32, device=dev)
    print(f"[bench] weights ready in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)

    lib = _lib.load()
    hip = HipEvents()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    c, wc = cfg.c(), weights.c()
    flags = moe.MOE_FWD_DETERMINISTIC if deterministic else 0
    NEV = _lib.MOE_FWD_STAGE_EVENTS
    evs = [[hip.create() for _ in range(NEV)] for _ in range(steps)]
    ev_arrays = [(ctypes.c_void_p * NEV)(*[e.value for e in row]) for row in evs]
    # the timed steps record only the two events around the gate/up GEMM (the roofline kernel):
    # each event record costs the stream a few microseconds; the other stages are timed after
    GU0, GU1 = 2, 3
    ev_gu = [(ctypes.c_void_p * NEV)(*[e.value if j in (GU0, GU1) else None for j, e in enumerate(row)])
             for row in evs]

    def step(ev_arr):
        st = lib.moe_ffn_forward_stages(
            ctypes.c_void_p(x.data_ptr()), T, ctypes.byref(c), ctypes.byref(wc), ctypes.c_void_p(ws.data_ptr()),
            ws.numel(), ctypes.c_void_p(out.data_ptr()), None,
            ctypes.c_void_p(idx.data_ptr()) if shape.n_experts else None, None, flags, ev_arr,
            NEV if ev_arr is not None else 0, stream)
        if st != 0:
            raise RuntimeError(f"moe_ffn_forward_stages: {lib.moe_last_error().decode()}")

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t_a, t_b = hip.create(), hip.create()
    wall0 = time.perf_counter()
    hip.record(t_a, stream)
    for i in range(steps):
        step(ev_gu[i])
    hip.record(t_b, stream)
    hip.sync(t_b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = hip.ms(t_a, t_b) / steps
    gu_timed = float(np.mean([hip.ms(evs[i][GU0], evs[i][GU1]) for i in range(steps)]))
    # per-stage breakdown: the same steps again, untimed, with every stage event recorded
    for i in range(steps):
        step(ev_arrays[i])
    torch.cuda.synchronize()
    names = ["quant_x", "route_permute", "gate_up_gemm", "down_gemm", "combine"]
    stage = {n: float(np.mean([hip.ms(evs[i][j], evs[i][j + 1]) for i in range(steps)]))
             for j, n in enumerate(names)}
    stage["gate_up_gemm"] = gu_timed             # the roofline kernel: from the timed steps
    for row in evs:
        for e in row:
            hip.destroy(e)

    if shape.n_experts:
        loads = np.bincount(idx.cpu().numpy().reshape(-1), minlength=shape.n_experts)
        touched = int((loads > 0).sum())
    else:
        loads = np.zeros(0)
        touched = 0
    nbytes = algorithmic_bytes(shape, touched)
    flops = shape.fp8_flops()
    t_s = ms_step / 1e3
    tflops = flops / t_s / 1e12
    hbm_gbs = nbytes["layer"] / t_s / 1e9
    gate_up_flops = 2.0 * shape.tokens * (shape.top_k + shape.n_shared) * shape.hidden * 2 * (
        shape.inter if shape.n_experts else shape.inter_shared)
    t_gu = stage["gate_up_gemm"] / 1e3
    ai = gate_up_flops / nbytes["gate_up"]
    if ai < FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": nbytes["gate_up"] / t_gu / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gate_up_flops / t_gu / 1e12, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # counted on the default scale format, at the workload's own size
    counted = not (ue8m0 or rmsnorm) and shape == synth.SHAPES[shape.name]
    roof["traffic"] = stored_traffic(shape) if counted else None
    roof["kernel"] = gate_up_kernel(shape, ue8m0) + " (gate/up GEMM, SwiGLU + requantisation epilogue)"
    roof["avg_ms"] = stage["gate_up_gemm"]
    # the other bound, for the record: the gate/up GEMM's FLOP rate or its algorithmic byte rate
    roof["hbm_gbs_algorithmic"] = nbytes["gate_up"] / t_gu / 1e9
    roof["tflops"] = gate_up_flops / t_gu / 1e12
    attainable = max(flops / (FP8_PEAK_TFLOPS * 1e12), nbytes["layer"] / (HBM_PEAK_GBS * 1e9))
    rec = {
        "value": T / t_s, "unit": "tokens/s", "steps": steps, "warmup": warmup, "ms_per_step": ms_step,
        "config": {"workload": shape.name, "tokens": T, "hidden": shape.hidden, "inter": shape.inter,
                   "n_experts": shape.n_experts, "top_k": shape.top_k, "n_shared": shape.n_shared,
                   "inter_shared": shape.inter_shared, "n_group": shape.n_group, "topk_group": shape.topk_group,
                   "scales": "ue8m0" if ue8m0 else "fp32", "rmsnorm": bool(rmsnorm),
                   "parallelism": "single GPU"},
        "fp8_tflops": tflops, "pct_fp8_mfma_peak": 100 * tflops / FP8_PEAK_TFLOPS,
        "hbm_gbs_algorithmic": hbm_gbs, "pct_hbm_peak": 100 * hbm_gbs / HBM_PEAK_GBS,
        "frac_attainable_roofline": attainable / t_s, "stages_ms": stage, "wall_s_timed": wall,
        "experts_touched": touched,
        "load_max_over_mean": float(loads.max() / loads.mean()) if loads.size else None,
        "roofline": roof,
    }
    if with_next_rows:
        rec["next_rows"] = next_rows(shape, x, idx, hip, stream, dev)
    del weights, ws, out, x, idx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, x_bits


def time_backward(shape, steps: int, warmup: int) -> dict:
    """The FP8 backward of the routed experts' two grouped GEMMs at this workload's routing, timed
    as one pass: dgrad of the down projection (dH = dY . W2: dY 1x128-quantised, W2^T packed),
    its wgrad (dW2_e = dY_e^T . H_e: both 128x1-quantised per expert), dgrad of gate/up
    (dX = dGU . W13) and its wgrad (dW13_e = dGU_e^T . X_e), with every quantisation inside the
    timed region; fp32 weight gradients.  The gradients dY, dGU and the activations H, X are seeded
    synthetic rows (N(0, 1), bf16) in the routing's sorted order; the SwiGLU, combine and router
    backward steps are not part of it."""
    import numpy as np
    import torch

    import sparse_moe_ffn_sigmoid_amd as moe
    import synth
    dev = torch.device("cuda:0")
    E, d, W, k, T = shape.n_experts, shape.hidden, shape.inter, shape.top_k, shape.tokens
    cfg = moe.MoeConfig.of(shape)
    xb = torch.from_numpy(synth.gen_x(shape).view(np.int16)).to(dev).view(torch.bfloat16)
    wr = torch.from_numpy(synth.gen_router_w(shape).view(np.int16)).to(dev).view(torch.bfloat16)
    _, idx, _ = moe.moe_route(cfg, T, dev, x=xb, w_router=wr)
    offsets = moe.moe_permute(idx, E)[0]
    M = T * k
    print(f"[bench] backward {shape.name}: transposing the expert weights", file=sys.stderr, flush=True)
    w2t_q = torch.empty((E, W, d), dtype=torch.uint8, device=dev)
    w2t_s = torch.empty((E, W // 128, d // 128), dtype=torch.float32, device=dev)
    w13t_q = torch.empty((E, d, 2 * W), dtype=torch.uint8, device=dev)
    w13t_s = torch.empty((E, d // 128, 2 * W // 128), dtype=torch.float32, device=dev)
    for e in range(E):
        q2, s2 = moe.fp8_quant_128x128(synth.torch_expert_weight(shape, e, "w2", dev))
        w2t_q[e], w2t_s[e] = moe.moe_pack_weights_transposed(q2, s2)
        q13, s13 = moe.fp8_quant_128x128(synth.torch_expert_weight(shape, e, "w13", dev))
        w13t_q[e], w13t_s[e] = moe.moe_pack_weights_transposed(q13, s13)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.stream_seed(shape.cfg_id, 9))
    dy = torch.randn((M, d), generator=gen, device=dev).to(torch.bfloat16)
    h = torch.randn((M, W), generator=gen, device=dev).to(torch.bfloat16)
    dgu = torch.randn((M, 2 * W), generator=gen, device=dev).to(torch.bfloat16)
    xs = torch.randn((M, d), generator=gen, device=dev).to(torch.bfloat16)
    dw2 = torch.empty((E, d, W), dtype=torch.float32, device=dev)
    dw13 = torch.empty((E, 2 * W, d), dtype=torch.float32, device=dev)
    dh = torch.empty((M, W), dtype=torch.float32, device=dev)
    dx = torch.empty((M, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        q, s = moe.fp8_quant_1x128(dy)
        moe.fp8_grouped_gemm_blockscaled(q, s, w2t_q, w2t_s, offsets, moe.MOE_EPI_STORE_F32, m_max=M, out=dh)
        a, as_, po = moe.fp8_quant_128x1_grouped(dy, offsets)
        b, bs, _ = moe.fp8_quant_128x1_grouped(h, offsets)
        moe.fp8_grouped_gemm_wgrad(a, as_, b, bs, po, M, out=dw2)
        q, s = moe.fp8_quant_1x128(dgu)
        moe.fp8_grouped_gemm_blockscaled(q, s, w13t_q, w13t_s, offsets, moe.MOE_EPI_STORE_F32, m_max=M, out=dx)
        a, as_, po = moe.fp8_quant_128x1_grouped(dgu, offsets)
        b, bs, _ = moe.fp8_quant_128x1_grouped(xs, offsets)
        moe.fp8_grouped_gemm_wgrad(a, as_, b, bs, po, M, out=dw13)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record()
    for _ in range(steps):
        step()
    b_ev.record()
    torch.cuda.synchronize()
    ms = a_ev.elapsed_time(b_ev) / steps
    flops = 2.0 * M * d * W * 2 + 2.0 * M * d * 2 * W * 2          # dgrad + wgrad of both GEMMs
    grad_bytes = 4.0 * E * 3 * d * W                                  # the fp32 weight gradients written
    tf = flops / (ms * 1e-3) / 1e12
    rec = {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "fp8_tflops": tf,
           "pct_fp8_mfma_peak": 100 * tf / FP8_PEAK_TFLOPS,
           "weight_grad_write_gbs": grad_bytes / (ms * 1e-3) / 1e9,
           "pct_hbm_peak_weight_grads": 100 * grad_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "steps": steps, "warmup": warmup,
           "scope": "routed experts' dgrad + wgrad of gate/up and down with their 1x128 / 128x1 quantisations; "
                    "fp32 weight gradients; synthetic gradients"}
    del w2t_q, w13t_q, dw2, dw13, dh, dx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_decode")
    ap.add_argument("--tokens", type=int, help="run the workload's layer at this many tokens instead (a batch-size "
                                                "sweep; the line's config records it)")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="tokens of the workload the CPU oracle runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the V3 prefill sub-record that the default (decode) line carries")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--ue8m0", action="store_true", help="power-of-two (UE8M0) scales for weights and activations")
    ap.add_argument("--rmsnorm", action="store_true", help="the RMSNorm in front, fused with x's quantisation")
    ap.add_argument("--calibrate-copy", type=int, metavar="MIB")
    ap.add_argument("--traffic-summary", metavar="DIR")
    ap.add_argument("--mfma-summary", metavar="DIR")
    ap.add_argument("--trace-summary", metavar="DIR")
    ap.add_argument("--backward", action="store_true", help="time only the FP8 backward GEMMs of the workload")
    args = ap.parse_args()
    if args.trace_summary:
        import synth
        trace_summary(args.trace_summary, synth.SHAPES[args.workload])
        return
    if args.mfma_summary:
        import synth
        mfma_summary(args.mfma_summary, synth.SHAPES[args.workload])
        return
    if args.traffic_summary:
        import synth
        traffic_summary(args.traffic_summary, synth.SHAPES[args.workload])
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import synth
    shape = synth.SHAPES[args.workload]
    if args.tokens:
        shape = synth.with_tokens(shape, args.tokens)
    if args.backward:
        print(json.dumps({"workload": shape.name, "backward": time_backward(shape, args.steps, args.warmup)}))
        return
    rec, x_bits = time_workload(shape, args.steps, args.warmup, ue8m0=args.ue8m0, rmsnorm=args.rmsnorm,
                                deterministic=args.deterministic)
    res = {"metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)", "data": "synthetic"}
    res.update({k: v for k, v in rec.items() if k not in res and k not in ("steps", "warmup")})
    if shape == synth.V3_DECODE and not args.no_prefill:
        # the MFMA half of the metric: the V3 prefill step (T = 4096) timed the same way
        sub, _ = time_workload(synth.V3_PREFILL, max(5, args.steps // 2), max(2, args.warmup), ue8m0=args.ue8m0,
                               rmsnorm=args.rmsnorm, deterministic=args.deterministic, with_next_rows=False)
        res["v3_prefill"] = sub
        # the other MFMA-heavy configurations, timed the same way: the dense FFN layer, the
        # load-skewed prefill batch, and the V3 prefill with power-of-two (UE8M0) scales
        for key, sh, ue in (("dense_ffn", synth.DENSE_FFN, args.ue8m0), ("v3_skew", synth.V3_SKEW, args.ue8m0),
                            ("v3_prefill_ue8m0", synth.V3_PREFILL, True)):
            if key == "v3_prefill_ue8m0" and args.ue8m0:
                continue
            res[key], _ = time_workload(sh, max(5, args.steps // 2), max(2, args.warmup), ue8m0=ue,
                                        rmsnorm=args.rmsnorm, deterministic=args.deterministic, with_next_rows=False)
        res["v3_prefill_backward"] = time_backward(synth.V3_PREFILL, max(3, args.steps // 10), 1)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(shape, x_bits, min(args.cpu_tokens, shape.tokens))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
