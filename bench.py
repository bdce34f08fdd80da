#!/usr/bin/env python3
"""Benchmark of the Switch MoE layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]

A step is one whole layer forward (router, dispatch, expert FFN, combine
and loss) over one batch of seeded synthetic inputs already resident in
HBM.  The headline workload is the Mixtral-shaped layer (8192 tokens,
d_model 4096, d_ff 14336, 8 SwiGLU experts, top-2), the largest of the five.
First the GPU settles: untimed forwards run for --settle-seconds (0.3 s),
since the chip leaves its idle clocks only under load.  Then W untimed
warm-up steps, then exactly K timed steps bracketed by device
synchronisation; each step starts with the 256 MB last-level cache flushed
(512 MB of scratch written before it, outside its HIP-event interval), and
value = T K / the summed step time.  warm_tokens_per_s gives the same K
steps back to back.

The same K steps then run through moe_forward_staged, which records HIP
events at the stage boundaries on the stream the kernels run on, giving each
stage's average duration; the roofline object reports the stage that takes
the longest, with its algorithmic bytes / flops per launch (`stage_work`).
The other four workloads follow (their tokens/s and dominant-kernel roofline
under "workloads"), then the CPU baseline: the CPU oracle on the headline
workload, on this host.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import datagen  # noqa: E402

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}

METRIC = "MoE-layer fwd tokens/s (1 GPU) + grouped-GEMM MFMA % of peak + permute GB/s"


def fused_forward(cfg: dict) -> tuple[bool, bool]:
    """(gather, scatter): what the library's forward fuses for this workload.

    bf16 with tokens: the first GEMM gathers the token rows of x (no dispatch
    copy); with k = 1 also the second GEMM writes gated rows to y (no combine
    pass).  Mirrors the choice in moe_forward."""
    gather = cfg["dtype"] == "bf16" and cfg["T"] > 0
    return gather, gather and cfg["k"] == 1


def stage_work(cfg: dict, A: int) -> dict:
    """Algorithmic bytes and flops of each stage for one forward.

    A = kept (token, rank) choices.  Only real rows count: weights once, the
    activations each stage must read or write, no padding, no re-reads.
      router   x [T,d] + W_r [E,d] fp32 read, expert_idx + gate [T,k] written;
               flops 2 T d E (fp32).  With bf16 tokens and E <= 256 the router
               forms each fp32 product exactly as three bf16 MFMA products
               (W_r split into three bf16 parts), so its bound is the bf16
               MFMA peak over 3 x 2 T d E flops; otherwise fp32 vector ALU
      dispatch T k (4 + 4 + 1) (indices read, slots and drop flags written)
               + 2 A d s (x rows read, xbuf rows written), or, fused,
               + 4 A (row index written) [+ (T - A) d s, dropped rows of y cleared]
      gemm1    W1 (+W3) [E,f,d] + A d s read (the kept token rows);
               flops 2 A d f (x2 for SwiGLU)
      gemm2    W2 [E,d,f] read + A d s written (the expert output rows);
               flops 2 A f d [fused: + 8 A, the row's token and gate]
      combine  A d s read + T d s written + T k 12 (indices, slots, gates);
               nothing when the second GEMM wrote y
    The FFN's minimum bytes are the weights once plus its input and output
    rows; the hidden activations H [A, f] written by the first GEMM and read
    by the second are not part of them (a fused FFN would keep H on chip),
    so their round trip shows up only in the measured traffic.
    """
    T, d, f, E, k = cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"]
    s = 2 if cfg["dtype"] == "bf16" else 4
    m = 2 if cfg["act"] == "swiglu" else 1
    gather, scatter = fused_forward(cfg)
    mfma_router = cfg["dtype"] == "bf16" and E <= 256
    disp = T * k * 9 + (4 * A + (T - A) * d * s * scatter if gather else 2 * A * d * s)
    return {
        "router": dict(bytes=T * d * s + E * d * 4 + T * k * 8,
                       flops=(3 if mfma_router else 1) * 2 * T * d * E,
                       dtype="bf16" if mfma_router else "f32"),
        "dispatch": dict(bytes=disp, flops=0, dtype=cfg["dtype"]),
        "expert_gemm1": dict(bytes=m * E * f * d * s + A * d * s, flops=2 * m * A * d * f,
                             dtype=cfg["dtype"]),
        "expert_gemm2": dict(bytes=E * d * f * s + A * d * s + 8 * A * scatter,
                             flops=2 * A * f * d, dtype=cfg["dtype"]),
        "combine": dict(bytes=0 if scatter else A * d * s + T * d * s + T * k * 12, flops=0,
                        dtype=cfg["dtype"]),
    }


def noisy_router_work(cfg: dict) -> dict:
    """Algorithmic bytes and flops of one noisy top-k router call.

    x [T,d] + W_r and W_noise [E,d] fp32 + the draws eps [T,E] fp32 read,
    expert_idx + gate [T,k] written; flops 2 x 2 T d E (the clean and the
    noise logits).  With bf16 tokens and E <= 256 both are exact fp32 dot
    products from three bf16 MFMA products each, as in the plain router, so
    the bound is the bf16 MFMA peak over 3 x 4 T d E flops; otherwise fp32
    vector ALU.
    """
    T, d, E, k = cfg["T"], cfg["d"], cfg["E"], cfg["k"]
    s = 2 if cfg["dtype"] == "bf16" else 4
    mfma = cfg["dtype"] == "bf16" and E <= 256
    return dict(bytes=T * d * s + 2 * E * d * 4 + T * E * 4 + T * k * 8,
                flops=(3 if mfma else 1) * 4 * T * d * E, dtype="bf16" if mfma else "f32")


def roofline_of(work: dict, seconds: float) -> dict:
    """Which roofline bounds a stage, and the achieved rate against that peak."""
    peak_f = PEAK_TFLOPS[work["dtype"]]
    if work["bytes"] == 0 and work["flops"] == 0:
        return dict(bound="none", achieved=None, peak=None, unit=None, frac=None)
    t_mem = work["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_flop = work["flops"] / (peak_f * 1e12) if work["flops"] else 0.0
    if t_flop > t_mem:
        ach = work["flops"] / seconds / 1e12
        return dict(bound="mfma" if work["dtype"] == "bf16" else "alu", achieved=round(ach, 2),
                    peak=peak_f, unit="TFLOP/s", frac=round(ach / peak_f, 4))
    ach = work["bytes"] / seconds / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(ach / PEAK_HBM_GBS, 4))


CSRC = os.path.join(ROOT, "sparse_mixture_experts_argmax_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_TAG = "traffic-json: "
COPY_PROBE_BYTES = 1 << 30

# The rocprofv3 runs that the traffic summary is built from; {w} is the
# workload, {o} the output directory.  Counters are collected in runs of
# their own, one counter group per pass.
PROFILE_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d {o}/ktrace -o k -- "
    "python3 $REPO/bench.py --workload {w} --steps 10 --warmup 3 --cpu-seconds 0 --others 0 "
    "--expert-backward-calls 2",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {o}/fetch -o f -- "
    "python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --cpu-seconds 0 --others 0 "
    "--expert-backward-calls 1",
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {o}/write -o w -- "
    "python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --cpu-seconds 0 --others 0 "
    "--expert-backward-calls 1",
    "timeout -s KILL 120 rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv "
    "-d {o}/mfma -o m -- python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --cpu-seconds 0 --others 0 "
    "--expert-backward-calls 1",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {o}/copy_fetch -o c -- "
    "python3 $REPO/bench.py --copy-probe %d" % COPY_PROBE_BYTES,
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {o}/copy_write -o c -- "
    "python3 $REPO/bench.py --copy-probe %d" % COPY_PROBE_BYTES,
    "python3 $REPO/bench.py --summarize {o} --workload {w} > $REPO/profiles/kernels_{w}.md",
]


def source_digest() -> str:
    """The kernel sources' digest (comments and blank space removed): counters
    taken on other code are stale, a reworded comment changes nothing."""
    from sparse_mixture_experts_argmax_amd.source_digest import source_digest as digest
    return digest(CSRC)


_GEMM_ACT = re.compile(r"gemm_(?:bf16|f32)_kernel<(?:[^<>]*<[^<>]*>, )?(\d+),")


# the noisy router kernels: NZ (the fifth argument) 1 or 2, tokens per block after it
_NOISY = re.compile(r"router_generic_kernel<\w+, true>|router_mfma_kernel<\d+, \d+, \w+, \d+, [12](?:, \d+)?>"
                    r"|router_split_noisy_kernel|router_reduce_kernel")


def kernel_stage(name: str) -> str:
    """The forward stage a kernel belongs to, from its (demangled) name.

    The noisy router and the standalone router reduction run only in the
    noisy-router measurement (the forward sums the router's partials in its
    dispatch scan), so they form a stage of their own."""
    if "combine_backward" in name or "router_bwd" in name:
        return "gate_backward"
    if any(t in name for t in ("transpose_kernel", "act_backward", "rowsum_kernel", "fill_i32", "zero16",
                               "dispatch_backward")):
        return "expert_backward"
    if _NOISY.search(name):
        return "noisy_router"
    if "router" in name:
        return "router"
    if any(t in name for t in ("priority_list", "priority_slot", "permute_slots")):
        return "priority_dispatch"          # permute_slots also serves the re-routing dispatch
    if "reroute_" in name:
        return "reroute_dispatch"
    if any(t in name for t in ("slot_rank", "slot_scan", "slot_index", "permute_kernel", "tile_map")):
        return "dispatch"
    m = _GEMM_ACT.search(name)
    if m:
        return "expert_gemm2" if m.group(1) == "0" else "expert_gemm1"
    if "combine" in name:
        return "combine"
    return "other"


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def stages_by_dispatch(rows) -> dict:
    """Stage of every dispatch (rows with Dispatch_Id and Kernel_Name), in
    dispatch order.  The launches of an expert-side backward call, from its
    first kernel (fill_i32_kernel) to its un-permute (dispatch_backward_kernel),
    belong to the expert backward whatever their name: its products run on
    the forward's GEMM kernel."""
    names = {}
    for r in rows:
        names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    stage, inside = {}, False
    for did in sorted(names):
        nm = names[did]
        if "fill_i32_kernel" in nm:
            inside = True
        stage[did] = "expert_backward" if inside else kernel_stage(nm)
        if "dispatch_backward_kernel" in nm:
            inside = False
    return stage


def _per_stage_kib(d: str, counter: str) -> dict:
    """Mean counter value (KiB) per launch of each stage's kernels."""
    rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
    stage = stages_by_dispatch(rows)
    acc = {}
    for r in rows:
        acc.setdefault(stage[int(r["Dispatch_Id"])], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _num_xcc(d: str) -> int:
    """XCDs of the profiled GPU (GRBM_GUI_ACTIVE adds up one count per XCD)."""
    for path in glob.glob(os.path.join(d, "*agent_info.csv")):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r.get("Agent_Type") == "GPU" and r.get("Num_Xcc"):
                    return int(r["Num_Xcc"])
    raise SystemExit(f"no GPU agent under {d}")


def mfma_by_stage(d: str, peak: float = PEAK_TFLOPS["bf16"] * 1e12) -> dict:
    """Per stage, over the launches that ran bf16 MFMAs: the MFMA flops the
    counters saw (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), MfmaUtil (MFMA busy
    cycles over active cycles x SIMDs, duration-weighted), the effective
    clock (GRBM_GUI_ACTIVE per XCD over the launch's duration) and the flop
    rate as a fraction of the nominal bf16 peak (under the counters)."""
    rows = _counter_rows(d)
    stage = stages_by_dispatch(rows)
    per = {}
    for r in rows:
        did = int(r["Dispatch_Id"])
        rec = per.setdefault(did, dict(dur=int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        rec[r["Counter_Name"]] = float(r["Counter_Value"])
    xcc = _num_xcc(d)
    acc = {}
    for did, rec in per.items():
        mops = rec.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        if mops <= 0 or rec["dur"] <= 0:
            continue
        a = acc.setdefault(stage[did], dict(n=0, dur=0, mops=0.0, util_dur=0.0, cycles=0.0))
        a["n"] += 1
        a["dur"] += rec["dur"]
        a["mops"] += mops
        a["util_dur"] += rec.get("MfmaUtil", 0.0) * rec["dur"]
        a["cycles"] += rec.get("GRBM_GUI_ACTIVE", 0.0) / xcc
    out = {}
    for st, a in acc.items():
        flops = a["mops"] * 512
        out[st] = dict(launches=a["n"], flops_per_launch=flops / a["n"], avg_us=a["dur"] / a["n"] / 1e3,
                       mfma_util_pct=a["util_dur"] / a["dur"], clock_ghz=a["cycles"] / a["dur"],
                       frac_of_peak=flops / (a["dur"] * 1e-9) / peak)
    return out


def _copy_kib(d: str, counter: str) -> float:
    vals = [float(r["Counter_Value"]) for r in _counter_rows(d)
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no copy kernel under {d}")
    return sum(vals) / len(vals)


def summarize(prof_dir: str, workload: str) -> str:
    """Markdown summary of one profile set: kernel times and HBM traffic per launch."""
    trace = glob.glob(os.path.join(prof_dir, "ktrace", "*kernel_trace.csv"))
    if not trace:
        raise SystemExit(f"no kernel_trace.csv under {prof_dir}/ktrace")
    with open(trace[0]) as fh:
        trows = list(csv.DictReader(fh))
    # per (kernel, stage): calls, mean / min / max duration, share of the time
    tstage = stages_by_dispatch(trows)
    agg = {}
    for r in trows:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        key = (r["Kernel_Name"], tstage[int(r["Dispatch_Id"])])
        a = agg.setdefault(key, [0, 0, None, 0])
        a[0] += 1
        a[1] += dur
        a[2] = dur if a[2] is None else min(a[2], dur)
        a[3] = max(a[3], dur)
    total_ns = sum(a[1] for a in agg.values()) or 1
    krows = [dict(Name=nm, Stage=st, Calls=a[0], AverageNs=a[1] / a[0], MinNs=a[2], MaxNs=a[3],
                  Percentage=100.0 * a[1] / total_ns)
             for (nm, st), a in sorted(agg.items(), key=lambda kv: -kv[1][1])]
    fetch = _per_stage_kib(os.path.join(prof_dir, "fetch"), "FETCH_SIZE")
    write = _per_stage_kib(os.path.join(prof_dir, "write"), "WRITE_SIZE")
    kib = COPY_PROBE_BYTES / 1024
    f_scale = kib / _copy_kib(os.path.join(prof_dir, "copy_fetch"), "FETCH_SIZE")
    w_scale = kib / _copy_kib(os.path.join(prof_dir, "copy_write"), "WRITE_SIZE")
    lines = [f"# Kernel times and HBM traffic, workload {workload}", "",
             "Made by (REPO = the repository root, OUT = a directory for the raw rocprofv3 output, "
             "on an MI355X):", "", "```"]
    lines += [c.format(w=workload, o="$OUT/prof_" + workload) for c in PROFILE_COMMANDS]
    lines += ["```", "", "## rocprofv3 --kernel-trace --stats", "",
              "| kernel | stage | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in krows:
        nm = r["Name"]
        short = re.sub(r"\(.*$", "", nm.replace("moe::(anonymous namespace)::", ""))
        short = short.replace("void ", "")
        lines.append(f"| `{short}` | {r['Stage']} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} "
                     f"| {float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | {float(r['Percentage']):.1f} |")
    lines += ["", "## HBM traffic per launch (rocprofv3 --pmc, scaled by the copy probe)", "",
              f"Copy probe: {COPY_PROBE_BYTES} bytes copied device to device; FETCH_SIZE scale "
              f"{f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f} (bytes moved / counter KiB*1024).", "",
              "| stage | FETCH KiB (raw) | WRITE KiB (raw) | fetch bytes | write bytes | traffic bytes |",
              "|---|---|---|---|---|---|"]
    traffic = {}
    for st in sorted(set(fetch) | set(write)):
        fb = fetch.get(st, 0.0) * 1024 * f_scale
        wb = write.get(st, 0.0) * 1024 * w_scale
        traffic[st] = dict(fetch_bytes=round(fb), write_bytes=round(wb), traffic_bytes=round(fb + wb))
        lines.append(f"| {st} | {fetch.get(st, 0):.1f} | {write.get(st, 0):.1f} | {fb:.0f} | {wb:.0f} "
                     f"| {fb + wb:.0f} |")
    mdir = os.path.join(prof_dir, "mfma")
    if os.path.isdir(mdir):
        mf = mfma_by_stage(mdir)
        lines += ["", "## MFMA utilisation (rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16)", "",
                  "MfmaUtil: MFMA busy cycles over active cycles x SIMDs (at the clock the chip ran); clock: "
                  "GRBM_GUI_ACTIVE per XCD over the launch's duration (the counter's window is a few us wider "
                  "than the kernel's, so on launches shorter than about 0.5 ms it reads high, even above the "
                  "2.4 GHz ceiling; the long launches give the clock); fraction of peak: the counted MFMA flops "
                  f"over the duration against the nominal {PEAK_TFLOPS['bf16']:.0f} TFLOP/s (counters slow a launch "
                  "by a few per cent). Stages whose launches ran no bf16 MFMA are left out.", "",
                  "| stage | launches | MFMA flops per launch (counter) | avg us (under counters) | MfmaUtil % "
                  "| effective clock GHz | fraction of nominal bf16 peak |",
                  "|---|---|---|---|---|---|---|"]
        for st in sorted(mf):
            m = mf[st]
            lines.append(f"| {st} | {m['launches']} | {m['flops_per_launch']:.4g} | {m['avg_us']:.1f} "
                         f"| {m['mfma_util_pct']:.1f} | {m['clock_ghz']:.2f} | {m['frac_of_peak']:.3f} |")
    lines += ["", "Per launch means the mean over that stage's kernel launches in the profiled steps; "
              "the dispatch, noisy_router and expert_backward stages are several kernels, each counted as "
              "one launch (the expert backward's launches are those from an expert-backward call's first "
              "kernel to its un-permute, its GEMMs included).", "",
              TRAFFIC_TAG + json.dumps(dict(workload=workload, source_digest=source_digest(),
                                             fetch_scale=round(f_scale, 5), write_scale=round(w_scale, 5),
                                             stages=traffic)), ""]
    return "\n".join(lines)


def committed_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from the committed profile summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"kernels_{workload}.md")
    if not os.path.exists(path):
        return None, "no profile summary"
    with open(path) as fh:
        for line in fh:
            if line.startswith(TRAFFIC_TAG):
                rec = json.loads(line[len(TRAFFIC_TAG):])
                if rec.get("source_digest") != source_digest():
                    return None, "kernel sources changed since the counters were taken"
                st = rec["stages"].get(stage)
                return (st["traffic_bytes"] if st else None), os.path.relpath(path, ROOT)
    return None, "no traffic record"


class HipEvents:
    """HIP events through the runtime torch already loaded (same process, same runtime)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def cpu_baseline(cfg: dict, min_seconds: float) -> dict:
    """The CPU oracle on the whole workload, repeated until min_seconds have passed."""
    from threadpoolctl import threadpool_info

    from oracle import moe as O
    reps, t0 = 0, time.perf_counter()
    while True:
        O.forward_cfg(cfg)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 20:
            break
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return dict(value=round(cfg["T"] * reps / el, 1), unit="tokens/s",
                cores=int(max(blas) if blas else 1), kind="oracle",
                sample=f"whole {cfg['name']} workload ({cfg['T']} tokens) x {reps} runs, "
                       f"{el:.1f} s; NumPy oracle, fp64 experts")


class Workload:
    """One seeded workload resident on the GPU, with its forward plan."""

    def __init__(self, name: str, torch, moe, dev):
        self.cfg = cfg = datagen.make(name, seed=0)
        self.name = name
        self.dev = dev
        bf = cfg["dtype"] == "bf16"

        def todev(a, bf16=False):
            if a is None:
                return None
            t = torch.from_numpy(a.view("int16") if bf16 else a)
            return (t.view(torch.bfloat16) if bf16 else t).to(dev)

        self.todev = todev
        self.x = todev(cfg["x"], bf)
        self.W_r = todev(cfg["W_r"])
        self.b_r = todev(cfg["b_r"])
        self.W1, self.W3, self.W2 = todev(cfg["W1"], bf), todev(cfg["W3"], bf), todev(cfg["W2"], bf)
        self.b1, self.b2 = todev(cfg["b1"], bf), todev(cfg["b2"], bf)
        dt = torch.bfloat16 if bf else torch.float32
        self.plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"], dt, act=cfg["act"],
                                    capacity_factor=cfg["cf"], alpha=cfg["alpha"], device=dev)
        self.stream = torch.cuda.current_stream(dev)

    def step(self):
        return self.plan(self.x, self.W_r, self.W1, self.W2, W3=self.W3, b1=self.b1, b2=self.b2, b_r=self.b_r)

    def staged_step(self, L, events):
        from sparse_mixture_experts_argmax_amd.api import _ACT, _dtype_code, _ptr
        p, cfg = self.plan, self.cfg
        arr = (ctypes.c_void_p * len(events))(*events)
        L.check("moe_forward_staged", L.LIB.moe_forward_staged(
            _ptr(self.x), _dtype_code(self.x), _ptr(self.W_r), _ptr(self.b_r), _ptr(self.W1), _ptr(self.b1),
            _ptr(self.W3), _ptr(self.W2), _ptr(self.b2), _ACT[cfg["act"]], cfg["T"], cfg["d"], cfg["f"],
            cfg["E"], cfg["k"], p.capacity_factor, p.alpha, _ptr(p.y), _ptr(p.aux), _ptr(p.z_loss),
            _ptr(p.expert_idx), _ptr(p.gate), _ptr(p.drop_mask), _ptr(p.ws), p.ws.numel(),
            self.stream.cuda_stream, arr))


def _spread(v, T):
    q = np.percentile(np.asarray(v, dtype=np.float64), [50, 10, 90])
    return dict(median=round(float(q[0]), 4), p10=round(float(q[1]), 4), p90=round(float(q[2]), 4),
                n=len(v), tokens_per_s=round(T / (float(q[0]) / 1e3), 1))


def measure(W: Workload, torch, L, hip, steps: int, warmup: int, settle_seconds: float, flush) -> dict:
    """Settle, warm up, then the timed steps (each after a last-level-cache flush), the
    same steps through moe_forward_staged for the stage times, and warm back-to-back steps."""
    T = W.cfg["T"]
    sid = W.stream.cuda_stream
    # settle: untimed forwards in rounds of 10 until settle_seconds have passed
    n_settle, t_s = 0, time.perf_counter()
    while n_settle == 0 or time.perf_counter() - t_s < settle_seconds:
        for _ in range(10):
            W.step()
        n_settle += 10
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_s
    for _ in range(warmup):
        W.step()
    torch.cuda.synchronize()
    # the timed steps: each forward starts with the 256 MB last-level cache
    # holding none of its data (512 MB of scratch written just before it,
    # outside its event interval)
    ev = hip.create(2 * steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush.fill_(i & 0xFF)
        hip.record(ev[2 * i], sid)
        W.step()
        hip.record(ev[2 * i + 1], sid)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cold_ms = [hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(steps)]
    hip.destroy(ev)
    # stage times: the same cold steps with an event at every stage boundary
    nev = L.MOE_STAGE_EVENTS
    sev = hip.create(nev * steps)
    for i in range(steps):
        flush.fill_(i & 0xFF)
        W.staged_step(L, sev[i * nev:(i + 1) * nev])
    torch.cuda.synchronize()
    stage_ms = {name: 0.0 for name in L.STAGES}
    for i in range(steps):
        e = sev[i * nev:(i + 1) * nev]
        for j, name in enumerate(L.STAGES):
            stage_ms[name] += hip.elapsed_ms(e[j], e[j + 1]) / steps
    hip.destroy(sev)
    # warm: back-to-back forwards, caches holding whatever the last one left
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        W.step()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t1
    A = int(W.plan.intermediate("expert_count").sum().item())
    drops = int(W.plan.drop_mask.sum().item())
    return dict(cold_ms=cold_ms, wall_s=wall, stage_ms=stage_ms, warm_s=warm_s, steps=steps, A=A, drops=drops,
                settle=dict(seconds=round(settle_s, 3), forwards=n_settle),
                value=T * steps / (sum(cold_ms) / 1e3), warm_value=T * steps / warm_s)


def stage_report(W: Workload, m: dict, L) -> tuple[dict, dict]:
    """Per-stage rooflines and the roofline object of the dominant (longest) kernel."""
    work = stage_work(W.cfg, m["A"])
    stages = {}
    for name in L.STAGES:
        r = roofline_of(work[name], m["stage_ms"][name] / 1e3)
        stages[name] = dict(us=round(m["stage_ms"][name] * 1e3, 2), bytes=work[name]["bytes"],
                            flops=work[name]["flops"], **r)
    dominant = max(L.STAGES, key=lambda n: m["stage_ms"][n])
    dom = stages[dominant]
    traffic, traffic_src = committed_traffic(W.name, dominant)
    roofline = dict(bound=dom["bound"], achieved=dom["achieved"], peak=dom["peak"], unit=dom["unit"],
                    frac=dom["frac"], traffic=traffic, traffic_unit="bytes/launch",
                    traffic_source=traffic_src, kernel=dominant,
                    algorithmic_bytes=work[dominant]["bytes"], algorithmic_flops=work[dominant]["flops"],
                    avg_us=dom["us"])
    return stages, roofline


def ffn_mfma_pct(W: Workload, m: dict) -> float:
    work = stage_work(W.cfg, m["A"])
    ffn_s = (m["stage_ms"]["expert_gemm1"] + m["stage_ms"]["expert_gemm2"]) / 1e3
    ffn_flops = work["expert_gemm1"]["flops"] + work["expert_gemm2"]["flops"]
    return round(100.0 * ffn_flops / ffn_s / 1e12 / PEAK_TFLOPS[W.cfg["dtype"]], 2)


def time_calls(hip, stream_id, torch, fn, calls: int) -> float:
    """Seconds per call of fn over `calls` calls after one untimed call (HIP events)."""
    fn()
    ev = hip.create(2)
    hip.record(ev[0], stream_id)
    for _ in range(calls):
        fn()
    hip.record(ev[1], stream_id)
    torch.cuda.synchronize()
    s = hip.elapsed_ms(ev[0], ev[1]) / calls / 1e3
    hip.destroy(ev)
    return s


def measure_variants(W: Workload, torch, moe, L, hip, args) -> dict:
    """The router and dispatch variants and the gate-side backward, each timed on its own."""
    cfg, plan, x, dev, sid = W.cfg, W.plan, W.x, W.dev, W.stream.cuda_stream
    T_, d_, E_, k_ = cfg["T"], cfg["d"], cfg["E"], cfg["k"]
    s_ = 2 if cfg["dtype"] == "bf16" else 4
    variants = {}
    # the noisy top-k router: the same tokens and W_r, seeded W_noise and standard normal draws
    if args.noisy_calls > 0:
        rng = np.random.default_rng(1)
        W_n = W.todev((rng.standard_normal((E_, d_)) * np.sqrt(0.1 / d_)).astype(np.float32))
        eps = W.todev(rng.standard_normal((T_, E_)).astype(np.float32))
        rws = torch.empty(L.LIB.moe_router_workspace_bytes(T_, d_, E_, k_), dtype=torch.uint8, device=dev)
        sec = time_calls(hip, sid, torch, lambda: moe.router(x, W.W_r, k=k_, b_r=W.b_r, workspace=rws, z_loss=True,
                                                             W_noise=W_n, noise=eps), args.noisy_calls)
        nw = noisy_router_work(cfg)
        variants["noisy_router"] = dict(us=round(sec * 1e6, 2), bytes=nw["bytes"], flops=nw["flops"],
                                        calls=args.noisy_calls, **roofline_of(nw, sec))
        del W_n, eps, rws
    # priority routing: the capacity filled in descending first-gate order
    if args.priority_calls > 0:
        pr = plan.gate[:, 0].contiguous()
        pws = torch.empty(L.LIB.moe_dispatch_priority_workspace_bytes(T_, E_, k_), dtype=torch.uint8, device=dev)
        sec = time_calls(hip, sid, torch, lambda: moe.dispatch_priority(x, plan.expert_idx, pr, E_, plan.C,
                                                                        workspace=pws), args.priority_calls)
        A_pr = int(moe.dispatch_priority(x, plan.expert_idx, pr, E_, plan.C, workspace=pws)[2].sum().item())
        pw = dict(bytes=2 * A_pr * d_ * s_ + T_ * k_ * 9 + T_ * 4, flops=0, dtype=cfg["dtype"])
        variants["priority_dispatch"] = dict(us=round(sec * 1e6, 2), bytes=pw["bytes"], kept=A_pr,
                                             calls=args.priority_calls, **roofline_of(pw, sec))
        del pws
    # the gate-side backward (combine backward, then router backward through
    # the gates, the balance loss and the z-loss) on the split API's buffers
    if args.backward_calls > 0:
        idx_b, gate_b, _, rc_b, lg_b = moe.router(x, W.W_r, k=k_, b_r=W.b_r, logits=True)
        slot_b, _, cnt_b, xbuf_b = moe.dispatch(x, idx_b, E_, plan.C)
        ybuf_b = moe.expert_ffn(xbuf_b, cnt_b, W.W1, W.W2, W3=W.W3, b1=W.b1, b2=W.b2, act=cfg["act"])
        del xbuf_b
        dy_b = torch.randn((T_, d_), device=dev).to(x.dtype)
        dyb_b = torch.zeros_like(ybuf_b)
        bws = torch.empty(max(L.LIB.moe_router_backward_workspace_bytes(T_, d_, E_), 256), dtype=torch.uint8,
                          device=dev)

        def gate_backward():
            dg, _ = moe.combine_backward(dy_b, ybuf_b, idx_b, slot_b, gate_b, dybuf=dyb_b)
            moe.router_backward(x, W.W_r, lg_b, idx_b, gate_b, dg, rc_b, alpha=cfg["alpha"], z_weight=1e-3,
                                workspace=bws)
        sec = time_calls(hip, sid, torch, gate_backward, args.backward_calls)
        A_b = int(cnt_b.sum().item())
        bw = dict(bytes=3 * A_b * d_ * s_ + 16 * T_ * k_ + 8 * T_ * E_ + T_ * d_ * (s_ + 4) + 8 * E_ * d_
                  + 12 * T_ * k_, flops=4 * T_ * E_ * d_, dtype="f32")
        variants["gate_backward"] = dict(us=round(sec * 1e6, 2), bytes=bw["bytes"], flops=bw["flops"],
                                         calls=args.backward_calls, **roofline_of(bw, sec))
        del ybuf_b, dyb_b, bws
    # the expert side of the backward: expert FFN backward (pre-activations
    # recomputed, dgrad and wgrad) then the un-permute onto the router's dx
    if args.expert_backward_calls > 0:
        idx_e, gate_e, _, rc_e, lg_e = moe.router(x, W.W_r, k=k_, b_r=W.b_r, logits=True)
        slot_e, _, cnt_e, xbuf_e = moe.dispatch(x, idx_e, E_, plan.C)
        ybuf_e = moe.expert_ffn(xbuf_e, cnt_e, W.W1, W.W2, W3=W.W3, b1=W.b1, b2=W.b2, act=cfg["act"])
        dy_e = (torch.randn((T_, d_), device=dev) * 0.02).to(x.dtype)
        _, dyb_e = moe.combine_backward(dy_e, ybuf_e, idx_e, slot_e, gate_e)
        del ybuf_e
        f_ = cfg["f"]
        ews = torch.empty(L.LIB.moe_expert_ffn_backward_workspace_bytes(E_, plan.C, d_, f_, 1 if s_ == 2 else 0,
                                                                        1 if cfg["act"] == "swiglu" else 0),
                          dtype=torch.uint8, device=dev)
        dx_r = torch.zeros((T_, d_), dtype=torch.float32, device=dev)
        dx_o = torch.empty_like(dx_r)

        def expert_backward():
            outs = moe.expert_ffn_backward(xbuf_e, cnt_e, W.W1, W.W2, dyb_e, W3=W.W3, b1=W.b1, act=cfg["act"],
                                           bias_grads=W.b1 is not None, workspace=ews)
            moe.dispatch_backward(outs[0], idx_e, slot_e, T_, dx_add=dx_r, dx=dx_o)
        sec = time_calls(hip, sid, torch, expert_backward, args.expert_backward_calls)
        A_e = int(cnt_e.sum().item())
        m_ = 2 if cfg["act"] == "swiglu" else 1
        # dgrad (dH, then dX through each first-layer weight) and wgrad (dW2,
        # each first-layer weight): twice the forward's products; the
        # recomputed pre-activations are extra work on top
        ew = dict(bytes=2 * (m_ + 1) * E_ * d_ * f_ * s_ + 3 * A_e * d_ * s_ + 8 * T_ * d_,
                  flops=2 * (2 * m_ + 2) * A_e * d_ * f_, dtype=cfg["dtype"])
        variants["expert_backward"] = dict(us=round(sec * 1e6, 2), bytes=ew["bytes"], flops=ew["flops"],
                                           recompute_flops=2 * m_ * A_e * d_ * f_, calls=args.expert_backward_calls,
                                           **roofline_of(ew, sec))
        del ews, xbuf_e, dyb_e, dx_r, dx_o
    # re-routing of the overflow: the router's top min(4, E) as preferences,
    # as many stages, the even-split capacity, gates from the logits
    if args.reroute_calls > 0:
        R_ = min(4, E_)
        idx_r, _, _, _, lg_r = moe.router(x, W.W_r, k=R_, b_r=W.b_r, logits=True)
        C1 = moe.capacity(T_, E_, 1, 1.0)
        rrws = torch.empty(max(L.LIB.moe_dispatch_reroute_workspace_bytes(T_, E_), 256), dtype=torch.uint8,
                           device=dev)
        sec = time_calls(hip, sid, torch, lambda: moe.dispatch_reroute(x, idx_r, E_, C1, R_, logits=lg_r,
                                                                       workspace=rrws), args.reroute_calls)
        A_r = int(moe.dispatch_reroute(x, idx_r, E_, C1, R_, logits=lg_r, workspace=rrws)[4].sum().item())
        rw = dict(bytes=2 * A_r * d_ * s_ + T_ * (4 * R_ + 4 * E_ + 13), flops=0, dtype=cfg["dtype"])
        variants["reroute_dispatch"] = dict(us=round(sec * 1e6, 2), bytes=rw["bytes"], kept=A_r, stages=R_,
                                            capacity=C1, calls=args.reroute_calls, **roofline_of(rw, sec))
        del rrws
    return variants


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="untimed forwards before the warm-up steps, to bring the GPU to its load clocks")
    ap.add_argument("--workload", default="mixtral", choices=datagen.CONFIG_ORDER,
                    help="the workload of the headline line (default: the Mixtral-shaped layer, the largest)")
    ap.add_argument("--others", type=int, default=1,
                    help="also measure the other four workloads (tokens/s and dominant-kernel roofline "
                         "of each under 'workloads'); 0 skips them")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--noisy-calls", type=int, default=20,
                    help="noisy top-k router calls timed after the steps (0 skips them)")
    ap.add_argument("--priority-calls", type=int, default=20,
                    help="priority-routing dispatch calls timed after the steps (0 skips them)")
    ap.add_argument("--backward-calls", type=int, default=20,
                    help="gate-side backward calls (combine + router backward) timed after the steps "
                         "(0 skips them)")
    ap.add_argument("--expert-backward-calls", type=int, default=5,
                    help="expert-side backward calls (expert FFN backward + un-permute) timed after the "
                         "steps (0 skips them)")
    ap.add_argument("--reroute-calls", type=int, default=20,
                    help="re-routing dispatch calls timed after the steps (0 skips them)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the "
                         "reference kernel that scales the HBM byte counters), then exit")
    ap.add_argument("--summarize", metavar="DIR",
                    help="only print the markdown summary of the rocprofv3 output under DIR "
                         "(ktrace/, fetch/, write/, copy_fetch/, copy_write/), then exit")
    args = ap.parse_args(argv)
    if args.summarize:
        print(summarize(args.summarize, args.workload))
        return 0
    if args.copy_probe:
        import torch
        n = args.copy_probe // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the layer's multi-GPU "
              "expert-parallel path is not built", file=sys.stderr)
        return 2

    import torch
    import sparse_mixture_experts_argmax_amd as moe
    from sparse_mixture_experts_argmax_amd import _lib as L

    dev = torch.device("cuda:0")
    hip = HipEvents()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    W = Workload(args.workload, torch, moe, dev)
    cfg = W.cfg
    print(f"[bench] {cfg['name']}: {args.steps} cold-cache steps", file=sys.stderr, flush=True)
    m = measure(W, torch, L, hip, args.steps, args.warmup, args.settle_seconds, flush)
    stages, roofline = stage_report(W, m, L)
    # the standalone dispatch (slots + permutation into xbuf), timed on its
    # own: the fused forward gathers rows inside the first GEMM when it can,
    # so it has no permutation to time
    disp_s = time_calls(hip, W.stream.cuda_stream, torch,
                        lambda: moe.dispatch(W.x, W.plan.expert_idx, cfg["E"], W.plan.C), 10)
    disp_bytes = 2 * m["A"] * cfg["d"] * (2 if cfg["dtype"] == "bf16" else 4) + cfg["T"] * cfg["k"] * 9
    variants = measure_variants(W, torch, moe, L, hip, args)
    mean_ms = float(np.mean(m["cold_ms"]))
    out = {
        "metric": METRIC,
        "value": round(m["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded, LayerNorm(N(0,1)) tokens, truncated-normal sigma=sqrt(0.1/fan_in) weights)",
        "config": {"workload": cfg["name"], "T": cfg["T"], "d_model": cfg["d"], "d_ff": cfg["f"],
                   "experts": cfg["E"], "k": cfg["k"], "capacity_factor": cfg["cf"],
                   "capacity": W.plan.C, "act": cfg["act"], "router": "fp32",
                   "kept_assignments": m["A"], "dropped": m["drops"]},
        "timing": "value = T x steps / the summed HIP-event time of the steps; each step is one whole "
                  "forward on inputs resident in HBM, started with the 256 MB last-level cache flushed "
                  "(512 MB of scratch written before it, outside its interval)",
        "warm_tokens_per_s": round(m["warm_value"], 1),
        "timed_wall_s": round(m["wall_s"], 4),
        "grouped_gemm_mfma_pct": ffn_mfma_pct(W, m),
        "permute_GBps": round(disp_bytes / disp_s / 1e9, 1),
        "permute_us": round(disp_s * 1e6, 2),
        "stages": stages,
        "variants": variants,
        "settle": m["settle"],
        "step_ms": {"cold_mall": _spread(m["cold_ms"], cfg["T"])},
        "roofline": roofline,
    }
    # the other workloads: tokens/s and the dominant kernel's roofline of each
    if args.others:
        table = {cfg["name"]: dict(tokens_per_s=out["value"], warm_tokens_per_s=out["warm_tokens_per_s"],
                                   ms_per_step=out["ms_per_step"], roofline=roofline,
                                   grouped_gemm_mfma_pct=out["grouped_gemm_mfma_pct"],
                                   stages_us={k_: v["us"] for k_, v in stages.items()})}
        host_cfg = cfg
        del W
        torch.cuda.empty_cache()
        for name in datagen.CONFIG_ORDER:
            if name in table:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            Wo = Workload(name, torch, moe, dev)
            mo = measure(Wo, torch, L, hip, min(args.steps, 20), 3, args.settle_seconds, flush)
            st_o, rf_o = stage_report(Wo, mo, L)
            table[name] = dict(tokens_per_s=round(mo["value"], 1), warm_tokens_per_s=round(mo["warm_value"], 1),
                               ms_per_step=round(float(np.mean(mo["cold_ms"])), 4), roofline=rf_o,
                               grouped_gemm_mfma_pct=ffn_mfma_pct(Wo, mo),
                               stages_us={k_: v["us"] for k_, v in st_o.items()})
            del Wo
            torch.cuda.empty_cache()
        out["workloads"] = {n: table[n] for n in datagen.CONFIG_ORDER if n in table}
        cfg = host_cfg
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
