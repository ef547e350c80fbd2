"""Benchmark of the quantized MoE expert layer on one MI355X.

One step = the whole hot path on one batch of synthetic tokens: moe_route (router GEMM +
top-k) -> moe_align -> moe_expert_forward (gate_up + SwiGLU, down, combine with the shared
expert).  Each step runs from a HIP graph; steps rotate over independently seeded layer
instances and token batches so that re-read weights are not served by the Infinity Cache.

Default run (no flags): the headline is the largest single-GPU workload, the
DeepSeek-V4-Flash-shaped MXFP4 layer (H=4096, 256 experts, top-8, I=2048 with a shared
expert) on one rank's slice I_local=1024 at T=256 tokens.  The JSON line's "points" add, each
with its own roofline: that layer at T=1 and T=16; the Qwen3.6-35B-A3B-shaped NVFP4 prefill
layer at T=8192 with Zipf(1.1)-skewed routing (full I, and the 256 slice), the measure of
grouped-GEMM MFMA efficiency; the fp8-block layer at T=64 and T=4096; and the NVFP4 decode
layer at T=1 and T=64.  ``--config N`` runs one configuration's own points instead (6: bf16
experts, 7: q4_0 experts among them).  Prints ONE JSON line.

Each point reports the spread of the step time (p10 / p50 / p90 over separately timed
rotations); the line reports the bandwidth of a plain 1 GiB device copy on the same GPU
beside the fractions of the 8 TB/s peak.  The CPU baseline (the fp64 oracle on the host's
physical cores, passive OpenMP waits) runs in a child process before the GPU is touched.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 GPU; decode HBM GB/s %peak; prefill MFMA %peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0}
RIDGE_FLOP_PER_BYTE = MFMA_PEAK_TFLOPS["bf16"] * 1e12 / (HBM_PEAK_GBS * 1e9)
# the sources each gate_up kernel is built from (counter summaries are keyed on their hash)
KERNEL_SOURCES = {"k_gate_up": ("expert_kernels.h", "expert_mxfp4.hip", "device_common.h", "route_align_dev.h"),
                  "k_gate_up_wide": ("expert_wide.hip", "device_common.h")}
WIDE_FORMATS = ("nvfp4", "fp8blk", "bf16")  # formats whose 128-row align blocks run the wide GEMMs

# the default run: (config id, T, slice); the first is the headline
DEFAULT_POINTS = [(5, 256, (0, 1024)), (5, 16, (0, 1024)), (5, 1, (0, 1024)),
                  (3, 8192, (0, 512)), (3, 8192, (0, 256)),
                  (4, 64, (0, 256)), (4, 4096, (0, 256)),
                  (2, 64, (0, 256)), (2, 1, (0, 256))]
# --config N: (T of the head point, slice of the head point, other (T, slice) points)
WORKLOADS = {
    2: (64, (0, 256), [(1, (0, 256)), (8, (0, 256)), (32, (0, 256)), (64, (0, 512)), (1, (0, 512))]),
    3: (8192, (0, 512), [(8192, (0, 256))]),
    4: (64, (0, 256), [(1, (0, 256)), (4096, (0, 256))]),
    5: (256, (0, 1024), [(1, (0, 1024)), (16, (0, 1024))]),
    6: (64, (0, 256), [(1, (0, 256)), (8192, (0, 512))]),
    7: (64, (0, 256), [(1, (0, 256)), (64, (0, 512))]),
}
INSTANCES = {2: 3, 3: 3, 4: 2, 5: 1, 6: 1, 7: 3}   # layer instances rotated (>= 1 GiB of banks for 2-4, 6, 7)
BATCHES = 4                            # token batches rotated


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_slice_bytes(fmt, H, Il):
    """Algorithmic bytes of one expert's slice (both projections): codes, scales and globals read once."""
    if fmt == "nvfp4":
        return 3 * Il * H * 9 // 16 + 8 * Il + 4 * H
    if fmt == "q4_0":  # 4-bit codes and an fp16 scale per 32
        return 3 * Il * H * 9 // 16
    if fmt == "fp8blk":
        return 3 * Il * H + 4 * (2 * Il * H + H * Il) // 16384
    if fmt == "bf16":
        return 3 * Il * H * 2
    return 3 * Il * H * 17 // 32


def gate_up_slice_bytes(fmt, H, Il):
    if fmt == "nvfp4":
        return 2 * Il * H * 9 // 16 + 8 * Il
    if fmt == "q4_0":
        return 2 * Il * H * 9 // 16
    if fmt == "fp8blk":
        return 2 * Il * H + 4 * (2 * Il * H) // 16384
    if fmt == "bf16":
        return 2 * Il * H * 2
    return 2 * Il * H * 17 // 32


def kernel_source_hash(kernel_name="k_gate_up"):
    """Hash of the code (comments and whitespace removed) of the sources a kernel is built from,
    and of the compiler options given to those files."""
    import re
    from quantized_moe_expert_topk_amd.build import FILE_FLAGS
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_name]:
        text = open(os.path.join(ROOT, "quantized_moe_expert_topk_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split() + FILE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_name, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(f"{kernel_name}|{workload}")
        if e and e.get("source_hash") == kernel_source_hash(kernel_name):
            return e.get("bytes_per_launch")
    except (ValueError, OSError):
        pass
    return None


def host_topology():
    """(CPU model name, logical CPUs this process may run on, physical cores among them) from
    the scheduler affinity and the kernel's CPU topology (Linux)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cpus = sorted(os.sched_getaffinity(0))
    cores = set()
    for c in cpus:
        try:
            base = f"/sys/devices/system/cpu/cpu{c}/topology/"
            cores.add((open(base + "physical_package_id").read().strip(), open(base + "core_id").read().strip()))
        except OSError:
            cores.add(("?", str(c)))
    return model, len(cpus), len(cores)


# host threads the GPU machine gives one GPU's jobs, whatever the machine shows
HOST_CPU_SHARE = 16


def cpu_baseline_child(cid, T, lo, hi, budget_s):
    """The oracle (fp64 C, OpenMP) run in this process on whole layers of the workload (route
    and expert forward) over successive token batches, until about budget_s seconds of work."""
    from oracle import oracle as O
    from synth import synth as S
    cfg = S.CONFIGS[cid]
    done_tokens, t_used, batches = 0, 0.0, 0
    base = S.layer_inputs(cfg, T, batch=0)  # instance 0, all experts
    while t_used < budget_s and batches < 64:
        x = S.tokens(cfg.seed, T, cfg.H, batch=batches)
        t0 = time.perf_counter()
        lg, ids, w, _ = O.route(x, base.router, base.bias, cfg.k, cfg.renormalize)
        O.expert_forward(base.routed, base.shared, x, ids, w, lo, hi)
        t_used += time.perf_counter() - t0
        done_tokens += T
        batches += 1
    print(json.dumps(dict(value=done_tokens / t_used, threads=O.num_threads(), batches=batches, t_used=t_used)),
          flush=True)


def cpu_baseline(cid, T, lo, hi, budget_s):
    """Runs cpu_baseline_child in a child Python process (started before this process touches
    the GPU) with one OpenMP thread per physical core of the CPUs it may use (at most the
    box's share), threads bound to cores and passive waits: spinning threads beyond the
    physical cores are what the pages measured costing a 19x slowdown (issue #62 follow-up
    comment on the OpenMP spin-wait)."""
    import subprocess
    model, logical, physical = host_topology()
    threads = max(1, min(physical, HOST_CPU_SHARE))
    env = dict(os.environ, OMP_NUM_THREADS=str(threads), OMP_WAIT_POLICY="passive", OMP_PROC_BIND="spread",
               OMP_PLACES="cores")
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", f"{cid},{T},{lo},{hi},{budget_s}"]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=max(120, 8 * budget_s))
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline child failed: {r.stderr[-2000:]}")
    d = json.loads(r.stdout.strip().splitlines()[-1])
    return dict(value=d["value"], unit="tokens/s", cores=d["threads"], kind="oracle",
                sample=f"{d['batches']} batch(es) of T={T} tokens of config {cid}, whole layer (route + expert "
                       f"forward), slice [{lo},{hi}), {d['t_used']:.1f} s of timed oracle work",
                cpu=f"{model}; {physical} physical cores / {logical} logical CPUs available, {threads} OpenMP "
                    f"threads (one per physical core, box share {HOST_CPU_SHARE}), OMP_WAIT_POLICY=passive")


# the arithmetic each kernel family computes in (per format; streaming kernels / prefill GEMMs)
DTYPES = {
    ("nvfp4", False): "bf16 x bf16 MFMA (e2m1*e4m3 weights exact in bf16), fp32 accumulate",
    ("nvfp4", True): "bf16 x bf16 MFMA (e2m1*e4m3 weights exact in bf16), fp32 accumulate",
    ("fp8blk", False): "bf16 x bf16 MFMA (e4m3 weights exact), fp32 accumulate, fp32 block scales",
    ("fp8blk", True): "bf16 x bf16 MFMA (e4m3 weights exact), fp32 accumulate, fp32 block scales",
    ("mxfp4", False): "scaled MFMA e4m3 (activation as hi+lo planes, e8m0 per 32) x e2m1 (e8m0 per 32), fp32 accumulate",
    ("bf16", False): "bf16 x bf16 MFMA, fp32 accumulate",
    ("bf16", True): "bf16 x bf16 MFMA, fp32 accumulate",
    ("q4_0", False): "bf16 x bf16 MFMA (codes as exact bf16 128+q, offset and fp16 scale in fp32), fp32 accumulate",
}


def run(args, plan):
    """Times every (config, T, slice) point of the plan; returns the list of point dicts."""
    import torch

    import quantized_moe_expert_topk_amd as qm
    from synth import synth as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def dbank(b):  # uploaded row-major, reordered once into the kernels' tile-16 layout
        return qm.moe_pack_bank(qm.DeviceBank(b.fmt, b.E, b.H, b.I, to_dev(b.gate_up), to_dev(b.gate_up_scale),
                                              to_dev(b.down), to_dev(b.down_scale), to_dev(b.gate_up_global),
                                              to_dev(b.down_global)))

    results = []
    for cid in dict.fromkeys(c for c, _, _ in plan):  # configs in plan order
        cfg = S.CONFIGS[cid]
        points = [(T, sl) for c, T, sl in plan if c == cid]
        R = args.instances or INSTANCES[cid]
        # Weight storage of a point's slice [lo, hi): "own" = the rank holds only its slice (gate
        # rows [lo, hi), up rows [I+lo, I+hi), down columns [lo, hi) as a bank with I = hi - lo,
        # run on [0, hi - lo)); "full" = the whole bank, run on [lo, hi).
        slices = sorted({sl for _, sl in points})
        t0 = time.time()
        inst = []
        for r in range(R):
            li = S.layer_inputs(cfg, 1, instance=r)
            banks = {}
            for (lo, hi) in slices:
                if args.storage == "own" and (lo, hi) != (0, cfg.I):
                    rb = S.slice_bank(li.routed, lo, hi)
                    sb = S.slice_bank(li.shared, lo, hi) if li.shared is not None else None
                else:
                    rb, sb = li.routed, li.shared
                key = (lo, hi) if rb is not li.routed else None
                if key not in banks:
                    banks[key] = (dbank(rb), dbank(sb) if sb is not None else None)
                banks[(lo, hi)] = banks[key]
            inst.append(dict(banks=banks, router=to_dev(li.router).view(torch.bfloat16), bias=to_dev(li.bias)))
            del li
        log(f"config {cid}: {R} layer instance(s) generated and uploaded in {time.time() - t0:.1f} s")
        Tmax = max(T for T, _ in points)
        xs = [to_dev(S.tokens(cfg.seed, Tmax, cfg.H, batch=b)).view(torch.bfloat16) for b in range(BATCHES)]
        for (T, (lo, hi)) in points:
            results.append(time_point(args, qm, torch, cfg, inst, xs, T, lo, hi, R))
        del inst, xs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return results


def time_point(args, qm, torch, cfg, inst, xs, T, lo, hi, R):
    Il = hi - lo
    layers, bytes_step, flops_step, gu_bytes, gu_flops = [], [], [], [], []
    for r in range(R):
        I_ = inst[r]
        for b in range(BATCHES):
            x = xs[b][:T].contiguous()
            rbank, sbank = I_["banks"][(lo, hi)]
            klo = lo if rbank.I == cfg.I else 0  # the slice inside the bank this point runs on
            L = qm.MoeLayer(rbank, sbank, I_["router"], I_["bias"], T, cfg.k, klo, klo + Il, cfg.renormalize)
            L(x)  # eager run (warms up, and fixes this graph's routing for the byte count)
            torch.cuda.synchronize()
            counts = L.align.counts.cpu().numpy()
            active = int((counts > 0).sum()) + (1 if cfg.shared else 0)
            pairs = T * cfg.k + (T if cfg.shared else 0)
            bytes_step.append(active * expert_slice_bytes(cfg.fmt, cfg.H, Il) + cfg.E * cfg.H * 2
                              + T * cfg.H * 2 + T * cfg.H * 4 + (cfg.E * 4 if I_["bias"] is not None else 0))
            flops_step.append(2 * pairs * 3 * Il * cfg.H + 2 * T * cfg.E * cfg.H)
            gu_bytes.append(active * gate_up_slice_bytes(cfg.fmt, cfg.H, Il) + T * cfg.H * 2 + pairs * Il * 2)
            gu_flops.append(2 * pairs * 2 * Il * cfg.H)
            layers.append((L, x))
    n = len(layers)

    def capture(k):  # one graph of k steps back to back, cycling through the rotation
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(k):
                L, x = layers[i % n]
                L(x)
        return g

    # exactly W warm-up steps, then exactly K timed steps, each as one graph so that graph
    # launches do not gap the steps; the rotation graph times the spread below
    g_all = capture(n)
    if args.warmup:
        capture(args.warmup).replay()
    g_timed = capture(args.steps)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # spread: rotations timed one by one (events between whole-rotation replays)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.spread_rotations + 1)]
    ev[0].record()
    for i in range(args.spread_rotations):
        g_all.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) / n for i in range(args.spread_rotations)])
    avg_bytes = sum(bytes_step[i % n] for i in range(args.steps)) / args.steps
    avg_flops = sum(flops_step[i % n] for i in range(args.steps)) / args.steps
    # dominant kernel: gate_up (+SwiGLU), launched back to back from one captured graph on the
    # stream the events are recorded on (the graph replays on torch's current stream)
    gk = torch.cuda.CUDAGraph()
    reps = max(1, min(args.steps, 64) // n) * n
    with torch.cuda.graph(gk):
        for i in range(reps):
            L, x = layers[i % n]
            qm.moe_expert_gate_up(L.routed, L.shared, x, L.k, L.align, L.lo, L.hi, L.ws)
    gk.replay()
    torch.cuda.synchronize()
    e0.record()
    gk.replay()
    e1.record()
    torch.cuda.synchronize()
    k_ms = e0.elapsed_time(e1) / reps
    k_bytes = sum(gu_bytes[i % n] for i in range(reps)) / reps
    k_flops = sum(gu_flops[i % n] for i in range(reps)) / reps
    bm = layers[0][0].block_m
    wide = bm % 128 == 0 and cfg.fmt in WIDE_FORMATS
    kname = "k_gate_up_wide" if wide else "k_gate_up"
    workload = f"{cfg.name}; T={T}; slice [{lo},{hi})"
    # roofline of the dominant kernel: bound by the point's arithmetic intensity against the
    # ridge of the bf16 MFMA and HBM peaks
    if avg_flops / avg_bytes > RIDGE_FLOP_PER_BYTE:
        ach = k_flops / (k_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=ach, peak=MFMA_PEAK_TFLOPS["bf16"], unit="TFLOP/s",
                    frac=ach / MFMA_PEAK_TFLOPS["bf16"], per_launch=k_flops)
    else:
        ach = k_bytes / (k_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS,
                    per_launch=k_bytes)
    # algorithmic bytes of the kernel either way (the counters' traffic is compared with them)
    roof.update(kernel=f"{kname} (gate_up grouped GEMM + SwiGLU)", kernel_us=k_ms * 1e3, alg_bytes_per_launch=k_bytes,
                traffic=load_traffic(kname, f"cfg{cfg.cid}_T{T}_slice{Il}"))
    pt = dict(config=cfg.cid, workload=workload, format=cfg.fmt, T=T, slice=[lo, hi], block_m=bm,
              dtype=DTYPES[(cfg.fmt, wide)], ms_per_step=ms, tokens_per_s=T / (ms * 1e-3),
              ms_per_step_p10_p50_p90=[float(np.percentile(per_step, q)) for q in (10, 50, 90)],
              layer_hbm_gbs=avg_bytes / (ms * 1e-3) / 1e9, layer_hbm_frac=avg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
              layer_tflops=avg_flops / (ms * 1e-3) / 1e12,
              layer_mfma_frac=avg_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"],
              alg_bytes_per_step=avg_bytes, alg_flops_per_step=avg_flops, roofline=roof,
              instances_rotated=R, batches_rotated=BATCHES)
    log(json.dumps(pt))
    del layers, gk, g_all, g_timed
    torch.cuda.synchronize()
    return pt


def copy_bandwidth_gbs(mib=1024, reps=5):
    """Bytes read + written per second by a plain device copy of `mib` MiB (torch copy_),
    the best of `reps` timed launches: a STREAM-style reference for the HBM fractions."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / best / 1e9


def copy_calibration(mib):
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=0, choices=[0] + sorted(WORKLOADS),
                    help="0 (default): the headline and the cross-configuration points; N: config N's own points")
    ap.add_argument("--T", type=int, default=0, help="with --config: the head point's T")
    ap.add_argument("--slice", type=str, default="", help="with --config: the head point's slice lo,hi")
    ap.add_argument("--instances", type=int, default=0)
    ap.add_argument("--no-points", action="store_true", help="only the headline point")
    ap.add_argument("--spread-rotations", type=int, default=20,
                    help="rotations timed one by one after the timed steps, for the p10/p50/p90 step time")
    ap.add_argument("--storage", choices=("own", "full"), default="full",
                    help="weights of a slice: the rank's own slice storage, or the full bank")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-child", type=str, default="", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (fp32 negate: reads and writes MIB MiB "
                         "each) three times, as the known-size kernel that HBM byte counters are scaled by")
    args = ap.parse_args()
    if args.cpu_baseline_child:
        cid, T, lo, hi, budget = args.cpu_baseline_child.split(",")
        cpu_baseline_child(int(cid), int(T), int(lo), int(hi), float(budget))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on one rank's intermediate slice, and the cross-rank "
              "all-reduce of the partials is not implemented. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.config:
        head_T, head_slice, others = WORKLOADS[args.config]
        head_T = args.T or head_T
        head_slice = tuple(int(v) for v in args.slice.split(",")) if args.slice else head_slice
        plan = [(args.config, head_T, head_slice)] + [(args.config, T, sl) for T, sl in others
                                                      if (T, sl) != (head_T, head_slice)]
    else:
        plan = list(DEFAULT_POINTS)
    if args.no_points:
        plan = plan[:1]
    cid, T, (lo, hi) = plan[0]
    cpu = None
    if not args.no_cpu_baseline:  # before anything touches the GPU
        t0 = time.time()
        cpu = cpu_baseline(cid, T, lo, hi, args.cpu_budget)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads ({time.time() - t0:.1f} s)")
    copy_gbs = copy_bandwidth_gbs()
    results = run(args, plan)
    for pt in results:
        pt["layer_hbm_frac_of_copy"] = pt["layer_hbm_gbs"] / copy_gbs
        if pt["roofline"]["bound"] == "hbm":
            pt["roofline"]["frac_of_measured_copy"] = pt["roofline"]["achieved"] / copy_gbs
    head = results[0]
    from synth import synth as S
    cfg = S.CONFIGS[head["config"]]
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
        "config": {"workload": head["workload"], "format": cfg.fmt, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "shared_expert": cfg.shared, "T": head["T"], "slice": head["slice"], "block_m": head["block_m"],
                   "instances_rotated": head["instances_rotated"], "batches_rotated": BATCHES,
                   "weight_storage": "rank's own slice" if args.storage == "own" else "full bank, sliced"},
        "layer_hbm_frac": head["layer_hbm_frac"], "layer_mfma_frac": head["layer_mfma_frac"],
        "ms_per_step_p10_p50_p90": head["ms_per_step_p10_p50_p90"], "hbm_copy_gbs": copy_gbs,
        "roofline": head["roofline"], "points": results,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
