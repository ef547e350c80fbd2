"""Benchmark of the quantized MoE expert layer on one MI355X.

One step = the whole hot path on one batch of synthetic tokens: moe_route (router GEMM +
top-k) -> moe_align -> moe_expert_forward (gate_up + SwiGLU, down, combine with the shared
expert).  Each step runs from a HIP graph; steps rotate over independently seeded layer
instances and token batches so that re-read weights are not served by the Infinity Cache.

Default workload: the Qwen3.6-35B-A3B-shaped NVFP4 decode layer (H=2048, 256 experts, top-8,
I=512, shared expert I=512) on one rank's slice I_local=256, T=64 tokens; the other decode
batch sizes and the full-I layer are reported under "points".  ``--config`` picks another
workload (3: prefill T=8192 with Zipf routing, 4: fp8-block, 5: DeepSeek-V4-Flash-shaped
MXFP4, 6: bf16 experts, 7: q4_0).  Prints ONE JSON line.

Besides the mean over the K timed steps, each point reports the spread of the step time
(p10 / p50 / p90 over separately timed rotations), and the line reports the bandwidth of a
plain 1 GiB device copy measured on the same GPU, beside the fractions of the 8 TB/s peak.
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
KERNEL_SOURCES = {"k_gate_up": ("expert.hip", "device_common.h"),
                  "k_gate_up_wide": ("expert_wide.hip", "device_common.h")}
WIDE_FORMATS = ("nvfp4", "fp8blk", "bf16")  # formats whose 128-row align blocks run the wide GEMMs

# (config id) -> (T of the headline point, slice of the headline point, other (T, slice) points)
WORKLOADS = {
    2: (64, (0, 256), [(1, (0, 256)), (8, (0, 256)), (32, (0, 256)), (64, (0, 512)), (1, (0, 512))]),
    3: (8192, (0, 512), [(8192, (0, 256))]),
    4: (64, (0, 256), [(1, (0, 256)), (4096, (0, 256))]),
    5: (16, (0, 1024), [(1, (0, 1024)), (256, (0, 1024))]),
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
    """Hash of the code (comments and whitespace removed) of the sources a kernel is built from."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_name]:
        text = open(os.path.join(ROOT, "quantized_moe_expert_topk_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
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


def cpu_baseline(cfg, T, lo, hi, budget_s):
    """The oracle (fp64 C, OpenMP) on the host cores: whole layers over token batches of the
    same workload until about budget_s seconds of work are done."""
    from oracle import oracle as O
    from synth import synth as S
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
    return dict(value=done_tokens / t_used, unit="tokens/s", cores=O.num_threads(), kind="oracle",
                sample=f"{batches} batch(es) of T={T} tokens, whole layer (route + expert forward), "
                       f"slice [{lo},{hi}), {t_used:.1f} s of timed oracle work", cpu=host_cpu())


def host_cpu():
    """The host CPU's model name and its logical CPU count (Linux /proc/cpuinfo)."""
    model, n = "unknown", 0
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    n += 1
                    model = ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return f"{model}, {n} logical CPUs"


def run(args):
    import torch

    import quantized_moe_expert_topk_amd as qm
    from synth import synth as S

    cid = args.config
    cfg = S.CONFIGS[cid]
    head_T, head_slice, others = WORKLOADS[cid]
    if args.T:
        head_T = args.T
    if args.slice:
        head_slice = tuple(int(v) for v in args.slice.split(","))
    points = [(head_T, head_slice)] + ([] if args.no_points else [p for p in others if p != (head_T, head_slice)])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = args.instances or INSTANCES[cid]

    def to_dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def dbank(b):  # uploaded row-major, reordered once into the kernels' tile-16 layout
        return qm.moe_pack_bank(qm.DeviceBank(b.fmt, b.E, b.H, b.I, to_dev(b.gate_up), to_dev(b.gate_up_scale),
                                              to_dev(b.down), to_dev(b.down_scale), to_dev(b.gate_up_global),
                                              to_dev(b.down_global)))

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
                rb, sb = S.slice_bank(li.routed, lo, hi), (S.slice_bank(li.shared, lo, hi) if li.shared is not None else None)
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

    results = []
    for (T, (lo, hi)) in points:
        Il = hi - lo
        layers, graphs, bytes_step, flops_step, gu_bytes = [], [], [], [], []
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
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    L(x)
                layers.append((L, x))
                graphs.append(g)
        n = len(graphs)
        # one graph over the whole rotation (n steps back to back) so that graph launches do
        # not gap the steps; K steps = K // n rotations, then the first K % n single steps
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for L, x in layers:
                L(x)

        def run_steps(k):
            for _ in range(k // n):
                g_all.replay()
            for i in range(k % n):
                graphs[i].replay()

        run_steps(args.warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_steps(args.steps)
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
        # dominant kernel: gate_up (+SwiGLU), launched back to back from one captured graph
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
        pt = dict(T=T, slice=[lo, hi], ms_per_step=ms, tokens_per_s=T / (ms * 1e-3), block_m=layers[0][0].block_m,
                  ms_per_step_p10_p50_p90=[float(np.percentile(per_step, q)) for q in (10, 50, 90)],
                  layer_hbm_gbs=avg_bytes / (ms * 1e-3) / 1e9, layer_hbm_frac=avg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  layer_tflops=avg_flops / (ms * 1e-3) / 1e12,
                  layer_mfma_frac=avg_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"],
                  alg_bytes_per_step=avg_bytes, alg_flops_per_step=avg_flops,
                  gate_up_us=k_ms * 1e3, gate_up_bytes=k_bytes,
                  gate_up_gbs=k_bytes / (k_ms * 1e-3) / 1e9)
        log(json.dumps(pt))
        results.append(pt)
        del layers, graphs, gk, g_all
        torch.cuda.synchronize()
    return cfg, results


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
    ap.add_argument("--config", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--T", type=int, default=0)
    ap.add_argument("--slice", type=str, default="")
    ap.add_argument("--instances", type=int, default=0)
    ap.add_argument("--no-points", action="store_true", help="only the headline point")
    ap.add_argument("--spread-rotations", type=int, default=20,
                    help="rotations timed one by one after the timed steps, for the p10/p50/p90 step time")
    ap.add_argument("--storage", choices=("own", "full"), default="full",
                    help="weights of a slice: the rank's own slice storage, or the full bank")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (fp32 negate: reads and writes MIB MiB "
                         "each) three times, as the known-size kernel that HBM byte counters are scaled by")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on one rank's intermediate slice, and the cross-rank "
              "all-reduce of the partials is not implemented. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    copy_gbs = copy_bandwidth_gbs()
    cfg, results = run(args)
    for pt in results:
        pt["layer_hbm_frac_of_copy"] = pt["layer_hbm_gbs"] / copy_gbs
    head = results[0]
    workload = f"{cfg.name}; T={head['T']}; slice [{head['slice'][0]},{head['slice'][1]})"
    # the head point's arithmetic intensity against the ridge of the bf16 MFMA and HBM peaks
    bound = "mfma" if head["alg_flops_per_step"] / head["alg_bytes_per_step"] > RIDGE_FLOP_PER_BYTE else "hbm"
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=head["gate_up_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=head["gate_up_gbs"] / HBM_PEAK_GBS, frac_of_measured_copy=head["gate_up_gbs"] / copy_gbs)
    else:
        tf = 2 * (head["T"] * cfg.k + (head["T"] if cfg.shared else 0)) * 2 * (head["slice"][1] - head["slice"][0]) * cfg.H
        ach = tf / (head["gate_up_us"] * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=ach, peak=MFMA_PEAK_TFLOPS["bf16"], unit="TFLOP/s",
                    frac=ach / MFMA_PEAK_TFLOPS["bf16"])
    gk = "k_gate_up_wide" if head["block_m"] == 128 and cfg.fmt in WIDE_FORMATS else "k_gate_up"
    roof["kernel"] = f"{gk} (gate_up grouped GEMM + SwiGLU)"
    roof["traffic"] = load_traffic(gk, f"cfg{cfg.cid}_T{head['T']}_slice{head['slice'][1] - head['slice'][0]}")
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "format": cfg.fmt, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "shared_expert": cfg.shared, "T": head["T"], "slice": head["slice"], "instances_rotated":
                   args.instances or INSTANCES[cfg.cid], "batches_rotated": BATCHES,
                   "weight_storage": "rank's own slice" if args.storage == "own" else "full bank, sliced"},
        "layer_hbm_frac": head["layer_hbm_frac"], "layer_mfma_frac": head["layer_mfma_frac"],
        "ms_per_step_p10_p50_p90": head["ms_per_step_p10_p50_p90"], "hbm_copy_gbs": copy_gbs,
        "roofline": roof, "points": results,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, head["T"], head["slice"][0], head["slice"][1], args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
