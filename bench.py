#!/usr/bin/env python3
"""Benchmark of the Switch MoE layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload switch_base]

A step is one whole layer forward (router, dispatch, expert FFN, combine
and loss) over one batch of seeded synthetic inputs already resident in
HBM.  First the GPU settles: untimed forwards run for --settle-seconds
(0.3 s), since the chip leaves its idle clocks only under load and the
first ~100 forwards after even 0.2 s of idle run up to 25 % slower.  Then W
untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation; value = tokens per second over the K steps.

After the timed steps the same K steps run again through
moe_forward_staged, which records HIP events at the stage boundaries on the
stream the kernels run on, giving each stage's average duration (the
events cost time of their own, so the timed steps run without them); the
roofline object reports the stage that takes the longest, with its
algorithmic bytes / flops per launch (see `stage_work`).  step_ms gives the
spread of single forwards, warm and with a cold last-level cache.  The CPU
baseline times the CPU oracle on the same workload, on this host.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
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
      gemm1    W1 (+W3) [E,f,d] + A d s read + A f s written;
               flops 2 A d f (x2 for SwiGLU)
      gemm2    W2 [E,d,f] + A f s read + A d s written; flops 2 A f d
               [fused: + 8 A, the row's token and gate]
      combine  A d s read + T d s written + T k 12 (indices, slots, gates);
               nothing when the second GEMM wrote y
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
        "expert_gemm1": dict(bytes=m * E * f * d * s + A * d * s + A * f * s, flops=2 * m * A * d * f,
                             dtype=cfg["dtype"]),
        "expert_gemm2": dict(bytes=E * d * f * s + A * f * s + A * d * s + 8 * A * scatter,
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
    "python3 $REPO/bench.py --workload {w} --steps 10 --warmup 3 --cpu-seconds 0",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {o}/fetch -o f -- "
    "python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --cpu-seconds 0",
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {o}/write -o w -- "
    "python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --cpu-seconds 0",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {o}/copy_fetch -o c -- "
    "python3 $REPO/bench.py --copy-probe %d" % COPY_PROBE_BYTES,
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {o}/copy_write -o c -- "
    "python3 $REPO/bench.py --copy-probe %d" % COPY_PROBE_BYTES,
    "python3 $REPO/bench.py --summarize {o} --workload {w} > $REPO/profiles/kernels_{w}.md",
]


_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


def source_digest() -> str:
    """sha256 over the kernel sources with comments and blank space removed:
    counters taken on other code are stale, a reworded comment changes nothing."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if path.endswith((".hip", ".h")):
            h.update(os.path.basename(path).encode())
            with open(path, encoding="utf-8") as fh:
                code = _COMMENT.sub(" ", fh.read())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


_GEMM_ACT = re.compile(r"gemm_(?:bf16|f32)_kernel<(?:[^<>]*<[^<>]*>, )?(\d+),")


_NOISY = re.compile(r"router_generic_kernel<\w+, true>|router_mfma_kernel<\d+, \d+, \w+, \d+, [12]>"
                    r"|router_split_noisy_kernel|router_reduce_kernel")


def kernel_stage(name: str) -> str:
    """The forward stage a kernel belongs to, from its (demangled) name.

    The noisy router and the standalone router reduction run only in the
    noisy-router measurement (the forward sums the router's partials in its
    dispatch scan), so they form a stage of their own."""
    if "combine_backward" in name or "router_bwd" in name:
        return "gate_backward"
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


def _per_stage_kib(d: str, counter: str) -> dict:
    """Mean counter value (KiB) per launch of each stage's kernels."""
    acc = {}
    for r in _counter_rows(d):
        if r["Counter_Name"] != counter:
            continue
        st = kernel_stage(r["Kernel_Name"])
        acc.setdefault(st, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _copy_kib(d: str, counter: str) -> float:
    vals = [float(r["Counter_Value"]) for r in _counter_rows(d)
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no copy kernel under {d}")
    return sum(vals) / len(vals)


def summarize(prof_dir: str, workload: str) -> str:
    """Markdown summary of one profile set: kernel times and HBM traffic per launch."""
    stats = glob.glob(os.path.join(prof_dir, "ktrace", "*kernel_stats.csv"))
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {prof_dir}/ktrace")
    with open(stats[0]) as fh:
        krows = list(csv.DictReader(fh))
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
        lines.append(f"| `{short}` | {kernel_stage(nm)} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} "
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
    lines += ["", "Per launch means the mean over that stage's kernel launches in the profiled steps; "
              "the dispatch and noisy_router stages are several kernels, each counted as one launch.", "",
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="untimed forwards before the warm-up steps, to bring the GPU to its load clocks")
    ap.add_argument("--workload", default="switch_base", choices=datagen.CONFIG_ORDER)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--noisy-calls", type=int, default=20,
                    help="noisy top-k router calls timed after the steps (0 skips them)")
    ap.add_argument("--priority-calls", type=int, default=20,
                    help="priority-routing dispatch calls timed after the steps (0 skips them)")
    ap.add_argument("--backward-calls", type=int, default=20,
                    help="gate-side backward calls (combine + router backward) timed after the steps "
                         "(0 skips them)")
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
    from sparse_mixture_experts_argmax_amd.api import _dtype_code, _ptr, _ACT

    cfg = datagen.make(args.workload, seed=0)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32

    def todev(a, bf=False):
        if a is None:
            return None
        t = torch.from_numpy(a.view("int16") if bf else a)
        return (t.view(torch.bfloat16) if bf else t).to(dev)

    bf = cfg["dtype"] == "bf16"
    x = todev(cfg["x"], bf)
    W_r = todev(cfg["W_r"])
    b_r = todev(cfg["b_r"])
    W1, W3, W2 = todev(cfg["W1"], bf), todev(cfg["W3"], bf), todev(cfg["W2"], bf)
    b1, b2 = todev(cfg["b1"], bf), todev(cfg["b2"], bf)
    plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"], dt, act=cfg["act"],
                           capacity_factor=cfg["cf"], alpha=cfg["alpha"], device=dev)
    stream = torch.cuda.current_stream(dev)
    hip = HipEvents()
    nev = L.MOE_STAGE_EVENTS
    events = hip.create(nev * args.steps)

    def step(i=None):
        if i is None:
            return plan(x, W_r, W1, W2, W3=W3, b1=b1, b2=b2, b_r=b_r)
        arr = (ctypes.c_void_p * nev)(*events[i * nev:(i + 1) * nev])
        L.check("moe_forward_staged", L.LIB.moe_forward_staged(
            _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2),
            _ptr(b2), _ACT[cfg["act"]], cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"],
            plan.capacity_factor, plan.alpha, _ptr(plan.y), _ptr(plan.aux), _ptr(plan.z_loss),
            _ptr(plan.expert_idx),
            _ptr(plan.gate), _ptr(plan.drop_mask), _ptr(plan.ws), plan.ws.numel(),
            stream.cuda_stream, arr))

    # settle: untimed forwards in rounds of 10 until settle_seconds have passed
    n_settle, t_s = 0, time.perf_counter()
    while n_settle == 0 or time.perf_counter() - t_s < args.settle_seconds:
        for _ in range(10):
            step()
        n_settle += 10
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_s
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the stage breakdown: the same steps again through moe_forward_staged,
    # which records a HIP event at every stage boundary (the events cost
    # time of their own, so the timed steps above run without them)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()

    stage_ms = {name: 0.0 for name in L.STAGES}
    for i in range(args.steps):
        ev = events[i * nev:(i + 1) * nev]
        for j, name in enumerate(L.STAGES):
            stage_ms[name] += hip.elapsed_ms(ev[j], ev[j + 1]) / args.steps
    hip.destroy(events)

    # per-step spread (warm): one HIP event between consecutive forwards, so
    # each interval holds one forward and one event record (~4.5 us)
    step_ev = hip.create(args.steps + 1)
    hip.record(step_ev[0], stream.cuda_stream)
    for i in range(args.steps):
        step()
        hip.record(step_ev[i + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    warm_ms = [hip.elapsed_ms(step_ev[i], step_ev[i + 1]) for i in range(args.steps)]
    hip.destroy(step_ev)
    # cold last-level cache: 512 MB of scratch written before each timed forward
    n_cold = min(args.steps, 10)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_ev = hip.create(2 * n_cold)
    for i in range(n_cold):
        scratch.fill_(i & 0xFF)
        hip.record(cold_ev[2 * i], stream.cuda_stream)
        step()
        hip.record(cold_ev[2 * i + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    cold_ms = [hip.elapsed_ms(cold_ev[2 * i], cold_ev[2 * i + 1]) for i in range(n_cold)]
    hip.destroy(cold_ev)
    del scratch

    def spread(v):
        q = np.percentile(np.asarray(v, dtype=np.float64), [50, 10, 90])
        return dict(median=round(float(q[0]), 4), p10=round(float(q[1]), 4), p90=round(float(q[2]), 4),
                    n=len(v), tokens_per_s=round(cfg["T"] / (float(q[0]) / 1e3), 1))

    A = int(plan.intermediate("expert_count").sum().item())
    drops = int(plan.drop_mask.sum().item())
    work = stage_work(cfg, A)
    # the standalone dispatch (slots + permutation into xbuf), timed on its
    # own outside the steps: the forward itself gathers rows inside the first
    # GEMM when it can, so it has no permutation to time
    n_disp = 10
    disp_ev = hip.create(2)
    moe.dispatch(x, plan.expert_idx, cfg["E"], plan.C)
    hip.record(disp_ev[0], stream.cuda_stream)
    for _ in range(n_disp):
        moe.dispatch(x, plan.expert_idx, cfg["E"], plan.C)
    hip.record(disp_ev[1], stream.cuda_stream)
    torch.cuda.synchronize()
    disp_s = hip.elapsed_ms(disp_ev[0], disp_ev[1]) / n_disp / 1e3
    hip.destroy(disp_ev)
    disp_bytes = 2 * A * cfg["d"] * (2 if cfg["dtype"] == "bf16" else 4) + cfg["T"] * cfg["k"] * 9
    # the noisy top-k router variant, timed on its own outside the steps:
    # the same tokens and W_r, seeded W_noise and standard normal draws
    variants = {}
    if args.noisy_calls > 0:
        rng = np.random.default_rng(1)
        W_n = todev((rng.standard_normal((cfg["E"], cfg["d"])) * np.sqrt(0.1 / cfg["d"])).astype(np.float32))
        eps = todev(rng.standard_normal((cfg["T"], cfg["E"])).astype(np.float32))
        rws = torch.empty(L.LIB.moe_router_workspace_bytes(cfg["T"], cfg["d"], cfg["E"], cfg["k"]), dtype=torch.uint8,
                          device=dev)
        moe.router(x, W_r, k=cfg["k"], b_r=b_r, workspace=rws, z_loss=True, W_noise=W_n, noise=eps)
        nz_ev = hip.create(2)
        hip.record(nz_ev[0], stream.cuda_stream)
        for _ in range(args.noisy_calls):
            moe.router(x, W_r, k=cfg["k"], b_r=b_r, workspace=rws, z_loss=True, W_noise=W_n, noise=eps)
        hip.record(nz_ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        nz_s = hip.elapsed_ms(nz_ev[0], nz_ev[1]) / args.noisy_calls / 1e3
        hip.destroy(nz_ev)
        nw = noisy_router_work(cfg)
        variants["noisy_router"] = dict(us=round(nz_s * 1e6, 2), bytes=nw["bytes"], flops=nw["flops"],
                                        calls=args.noisy_calls, **roofline_of(nw, nz_s))
        del W_n, eps, rws
    # priority routing: the plain dispatch's work with the capacity filled in
    # descending first-gate order, timed on its own like the dispatch above
    if args.priority_calls > 0:
        pr = plan.gate[:, 0].contiguous()
        pws = torch.empty(L.LIB.moe_dispatch_priority_workspace_bytes(cfg["T"], cfg["E"], cfg["k"]),
                          dtype=torch.uint8, device=dev)
        moe.dispatch_priority(x, plan.expert_idx, pr, cfg["E"], plan.C, workspace=pws)
        pr_ev = hip.create(2)
        hip.record(pr_ev[0], stream.cuda_stream)
        for _ in range(args.priority_calls):
            moe.dispatch_priority(x, plan.expert_idx, pr, cfg["E"], plan.C, workspace=pws)
        hip.record(pr_ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        pr_s = hip.elapsed_ms(pr_ev[0], pr_ev[1]) / args.priority_calls / 1e3
        hip.destroy(pr_ev)
        A_pr = int(moe.dispatch_priority(x, plan.expert_idx, pr, cfg["E"], plan.C, workspace=pws)[2].sum().item())
        pw = dict(bytes=2 * A_pr * cfg["d"] * (2 if cfg["dtype"] == "bf16" else 4) + cfg["T"] * cfg["k"] * 9
                  + cfg["T"] * 4, flops=0, dtype=cfg["dtype"])
        variants["priority_dispatch"] = dict(us=round(pr_s * 1e6, 2), bytes=pw["bytes"], kept=A_pr,
                                             calls=args.priority_calls, **roofline_of(pw, pr_s))
        del pws
    # the gate-side backward (combine backward, then router backward through
    # the gates, the balance loss and the z-loss), on the split API's forward
    # buffers, timed on its own
    if args.backward_calls > 0:
        idx_b, gate_b, _, rc_b, lg_b = moe.router(x, W_r, k=cfg["k"], b_r=b_r, logits=True)
        slot_b, _, cnt_b, xbuf_b = moe.dispatch(x, idx_b, cfg["E"], plan.C)
        ybuf_b = moe.expert_ffn(xbuf_b, cnt_b, W1, W2, W3=W3, b1=b1, b2=b2, act=cfg["act"])
        del xbuf_b
        dy_b = torch.randn((cfg["T"], cfg["d"]), device=dev).to(x.dtype)
        dyb_b = torch.zeros_like(ybuf_b)
        bws = torch.empty(max(L.LIB.moe_router_backward_workspace_bytes(cfg["T"], cfg["d"], cfg["E"]), 256),
                          dtype=torch.uint8, device=dev)

        def gate_backward():
            dg, _ = moe.combine_backward(dy_b, ybuf_b, idx_b, slot_b, gate_b, dybuf=dyb_b)
            moe.router_backward(x, W_r, lg_b, idx_b, gate_b, dg, rc_b, alpha=cfg["alpha"], z_weight=1e-3,
                                workspace=bws)
        gate_backward()
        bw_ev = hip.create(2)
        hip.record(bw_ev[0], stream.cuda_stream)
        for _ in range(args.backward_calls):
            gate_backward()
        hip.record(bw_ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        bw_s = hip.elapsed_ms(bw_ev[0], bw_ev[1]) / args.backward_calls / 1e3
        hip.destroy(bw_ev)
        A_b = int(cnt_b.sum().item())
        T_, d_, E_, k_ = cfg["T"], cfg["d"], cfg["E"], cfg["k"]
        s_ = 2 if cfg["dtype"] == "bf16" else 4
        bw = dict(bytes=3 * A_b * d_ * s_ + 16 * T_ * k_ + 8 * T_ * E_ + T_ * d_ * (s_ + 4) + 8 * E_ * d_
                  + 12 * T_ * k_, flops=4 * T_ * E_ * d_, dtype="f32")
        variants["gate_backward"] = dict(us=round(bw_s * 1e6, 2), bytes=bw["bytes"], flops=bw["flops"],
                                         calls=args.backward_calls, **roofline_of(bw, bw_s))
        del ybuf_b, dyb_b, bws
    # re-routing of the overflow: the router's top min(4, E) as preferences,
    # as many stages, the even-split capacity, gates from the logits
    if args.reroute_calls > 0:
        R_ = min(4, cfg["E"])
        idx_r, _, _, _, lg_r = moe.router(x, W_r, k=R_, b_r=b_r, logits=True)
        C1 = moe.capacity(cfg["T"], cfg["E"], 1, 1.0)
        rrws = torch.empty(max(L.LIB.moe_dispatch_reroute_workspace_bytes(cfg["T"], cfg["E"]), 256),
                           dtype=torch.uint8, device=dev)
        out_r = moe.dispatch_reroute(x, idx_r, cfg["E"], C1, R_, logits=lg_r, workspace=rrws)
        rr_ev = hip.create(2)
        hip.record(rr_ev[0], stream.cuda_stream)
        for _ in range(args.reroute_calls):
            moe.dispatch_reroute(x, idx_r, cfg["E"], C1, R_, logits=lg_r, workspace=rrws)
        hip.record(rr_ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        rr_s = hip.elapsed_ms(rr_ev[0], rr_ev[1]) / args.reroute_calls / 1e3
        hip.destroy(rr_ev)
        A_r = int(out_r[4].sum().item())
        s_ = 2 if cfg["dtype"] == "bf16" else 4
        rw = dict(bytes=2 * A_r * cfg["d"] * s_ + cfg["T"] * (4 * R_ + 4 * cfg["E"] + 13), flops=0,
                  dtype=cfg["dtype"])
        variants["reroute_dispatch"] = dict(us=round(rr_s * 1e6, 2), bytes=rw["bytes"], kept=A_r, stages=R_,
                                            capacity=C1, calls=args.reroute_calls, **roofline_of(rw, rr_s))
        del rrws, out_r
    stages = {}
    for name in L.STAGES:
        r = roofline_of(work[name], stage_ms[name] / 1e3)
        stages[name] = dict(us=round(stage_ms[name] * 1e3, 2), bytes=work[name]["bytes"],
                            flops=work[name]["flops"], **r)
    dominant = max(L.STAGES, key=lambda n: stage_ms[n])
    dom = dict(stages[dominant])
    traffic, traffic_src = committed_traffic(cfg["name"], dominant)
    roofline = dict(bound=dom["bound"], achieved=dom["achieved"], peak=dom["peak"], unit=dom["unit"],
                    frac=dom["frac"], traffic=traffic, traffic_unit="bytes/launch",
                    traffic_source=traffic_src, kernel=dominant,
                    algorithmic_bytes=work[dominant]["bytes"], algorithmic_flops=work[dominant]["flops"],
                    avg_us=dom["us"])
    ffn_s = (stage_ms["expert_gemm1"] + stage_ms["expert_gemm2"]) / 1e3
    ffn_flops = work["expert_gemm1"]["flops"] + work["expert_gemm2"]["flops"]
    peak = PEAK_TFLOPS[cfg["dtype"]]
    ms_per_step = elapsed / args.steps * 1e3
    out = {
        "metric": METRIC,
        "value": round(cfg["T"] * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded, LayerNorm(N(0,1)) tokens, truncated-normal sigma=sqrt(0.1/fan_in) weights)",
        "config": {"workload": cfg["name"], "T": cfg["T"], "d_model": cfg["d"], "d_ff": cfg["f"],
                   "experts": cfg["E"], "k": cfg["k"], "capacity_factor": cfg["cf"],
                   "capacity": plan.C, "act": cfg["act"], "router": "fp32",
                   "kept_assignments": A, "dropped": drops},
        "grouped_gemm_mfma_pct": round(100.0 * ffn_flops / ffn_s / 1e12 / peak, 2),
        "permute_GBps": round(disp_bytes / disp_s / 1e9, 1),
        "permute_us": round(disp_s * 1e6, 2),
        "stages": stages,
        "variants": variants,
        "settle": {"seconds": round(settle_s, 3), "forwards": n_settle},
        "step_ms": {"warm": spread(warm_ms), "cold_mall": spread(cold_ms),
                    "note": "per-forward HIP event intervals (each holds one event record, "
                            "about 4.5 us); cold_mall writes 512 MB of scratch before each forward"},
        "roofline": roofline,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
