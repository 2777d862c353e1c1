"""Benchmark of the INT8-QK / BF16-PV attention forward on one MI355X.

Default workload: B1 H56 Sq4096 Sk33600 D128 bf16 with the two-sided
raised-cosine [1,1,1,K] bias (20160-key core, 6720-key skirts).

One step is one pass of the whole path over that batch, all on the GPU:
  quantize_qk (K mean, Q and centred-K int8 codes + scales, centring term)
  attn_fwd unmasked                                  (all 33600 keys)
  attn_fwd with the fp32 [1,1,1,K] bias              (all 33600 keys)
  split: attn_fwd core (LSE) + attn_fwd skirts with bias (LSE) + lse_merge
Each of the three attention computations covers the full key range, so a
step does 3 * 4*B*H*Sq*Sk*D effective flops; ``value`` is that over the
step time. Per-call medians (CUDA/HIP events on the launch stream) give the
unmasked / bias / split figures and their ratios.

Prints one JSON line. ``--gpus`` above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd ms + TFLOPS, 56h×4096q×33600k d128 (unmasked / [1,1,1,K] bias)"
# MI355X published dense peaks: int8 MFMA 5033 TOPS, bf16 MFMA 2516.6 TFLOPS, HBM3E 8 TB/s.
PEAK_I8_TOPS = 5033.2
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
# Half of the effective flops are int8 (QK), half bf16 (PV), on the same
# matrix pipe, so their times add: the blended peak is the harmonic mean.
PEAK_BLEND = 2.0 / (1.0 / PEAK_I8_TOPS + 1.0 / PEAK_BF16_TFLOPS)
# The pages' per-call times for this exact workload (RTX 5090, comfy-kitchen
# int8_attention, first of the two runs): unmasked, fp32 bias, core+skirt.
PAGE_MS = {"unmasked": 8.64, "bias_fp32": 15.28, "split_unmerged": 11.05}

ATTN_SRC = os.path.join(ROOT, "quantized_flash_attention_amd", "csrc", "attn_fwd.hip")
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_band_unmasked_pmc.json")


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profile(launch_key: str):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary, or
    None when it is missing or was taken on another version of the kernel."""
    try:
        d = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != src_hash(ATTN_SRC):
        return None
    e = d.get("launches", {}).get(launch_key)
    return None if e is None else e.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variant-iters", type=int, default=20, help="iterations of each per-call timing loop")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows of head 0 the oracle computes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE passes over "
                         "this script with --copy-calibration) into " + os.path.relpath(PMC_FILE, ROOT))
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import quantized_flash_attention_amd as qfa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    w = W.WORKLOADS["band"]
    B, H, Sq, Sk, D = w.B, w.H, w.Sq, w.Sk, w.D
    core, skirt = w.extras["core"], w.extras["skirt"]
    skirts = [(0, skirt), (core[0] + core[1], skirt)]

    t0 = time.time()
    q_np, k_np, v_np = W.make_qkv(w)
    b64 = W.band_bias(Sk, core=core, skirt=skirt)
    bias32_np, bias16_np = W.bias_tensor(b64, "fp32"), W.bias_tensor(b64, "bf16")

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = up(q_np), up(k_np), up(v_np)
    bias32, bias16 = up(bias32_np), up(bias16_np)
    gen_s = time.time() - t0

    ws = torch.empty(qfa.quantize_workspace_bytes(B, H, Sk, D), dtype=torch.uint8, device=dev)
    o_un = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=dev)
    o_bias = torch.empty_like(o_un)
    o_core = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
    o_skirt = torch.empty_like(o_core)
    o_split = torch.empty_like(o_un)
    l_core = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    l_skirt = torch.empty_like(l_core)
    l_split = torch.empty_like(l_core)
    sm = w.sm_scale
    stream = torch.cuda.current_stream(dev)

    names = ["quantize", "unmasked", "bias_fp32", "core", "skirt", "merge"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        qk = qfa.quantize_qk(q, k, workspace=ws)
        mark(1)
        qfa.attn_fwd(qk, v, sm, out=o_un)
        mark(2)
        qfa.attn_fwd(qk, v, sm, bias=bias32, out=o_bias)
        mark(3)
        qfa.attn_fwd(qk, v, sm, segments=[core], out=o_core, lse=l_core)
        mark(4)
        qfa.attn_fwd(qk, v, sm, bias=bias32, segments=skirts, out=o_skirt, lse=l_skirt)
        mark(5)
        qfa.lse_merge(o_core, l_core, o_skirt, l_skirt, out=o_split, lse_out=l_split)
        mark(6)
        return qk

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total * 1000.0 / args.steps

    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    med = {n: statistics.median(x) for n, x in per.items()}
    mean = {n: statistics.fmean(x) for n, x in per.items()}

    # bf16-bias single call: its own loop (same kernel instance as the fp32 bias call)
    qk = step()
    torch.cuda.synchronize()
    bf = []
    for _ in range(args.variant_iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        qfa.attn_fwd(qk, v, sm, bias=bias16, out=o_bias)
        e1.record(stream)
        bf.append((e0, e1))
    torch.cuda.synchronize()
    med["bias_bf16"] = statistics.median(a.elapsed_time(b) for a, b in bf)

    flops_full = 4.0 * B * H * Sq * Sk * D
    tflops = lambda fl, ms: fl / (ms * 1e-3) / 1e12
    split_ms = med["core"] + med["skirt"] + med["merge"]
    # algorithmic bytes of the quantize step: read Q and K once, write codes, scales, mean, centring term
    qbytes = (B * H * (Sq + Sk) * D * 2 + B * H * (Sq + Sk) * D + B * H * (Sq + Sk) * 4
              + B * H * D * 4 + B * H * Sq * 4)
    mbytes = B * H * Sq * (2 * D * 4 + 2 * 4 + D * 2 + 4)
    step_flops = 3 * flops_full
    value = step_flops / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel: the unmasked attention launch (one per step)
    avg_un = mean["unmasked"]
    achieved = tflops(flops_full, avg_un)
    traffic = traffic_from_profile("unmasked")
    page_step_ms = sum(PAGE_MS.values())
    page_value = step_flops / (page_step_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / page_value, 3),
        "dtype": "i8+bf16",
        "data": "synthetic",
        "config": {
            "workload": "banded cross-attention B1 H56 Sq4096 Sk33600 D128 bf16, [1,1,1,K] raised-cosine bias "
                        "(core 20160 keys, skirts 2x6720), K centred, per-token int8 Q/K",
            "B": B, "H": H, "Sq": Sq, "Sk": Sk, "D": D, "global_batch": B, "seq_len": Sq,
            "parallelism": "none (1 GPU)",
            "step": "quantize_qk + attn unmasked + attn fp32-bias + split(core LSE, skirt LSE, lse_merge)",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel<128,bf16,4 waves,dense,no bias,no LSE> (unmasked call)",
            "achieved": round(achieved, 1),
            "peak": round(PEAK_BLEND, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BLEND, 4),
            "traffic": traffic,
            "avg_launch_ms": round(avg_un, 4),
            "flops_per_launch": flops_full,
            "peak_note": "harmonic blend of int8 5033 TOPS (QK half) and bf16 2516.6 TFLOPS (PV half)",
        },
        "calls": {
            "quantize_ms": round(med["quantize"], 4),
            "quantize_GBps": round(qbytes / (med["quantize"] * 1e-3) / 1e9, 1),
            "unmasked_ms": round(med["unmasked"], 4),
            "unmasked_tflops": round(tflops(flops_full, med["unmasked"]), 1),
            "bias_fp32_ms": round(med["bias_fp32"], 4),
            "bias_fp32_tflops": round(tflops(flops_full, med["bias_fp32"]), 1),
            "bias_bf16_ms": round(med["bias_bf16"], 4),
            "bias_fp32_over_unmasked": round(med["bias_fp32"] / med["unmasked"], 3),
            "bias_bf16_over_unmasked": round(med["bias_bf16"] / med["unmasked"], 3),
            "core_ms": round(med["core"], 4),
            "skirt_ms": round(med["skirt"], 4),
            "merge_ms": round(med["merge"], 4),
            "merge_GBps": round(mbytes / (med["merge"] * 1e-3) / 1e9, 1),
            "split_ms": round(split_ms, 4),
            "split_over_single_bias": round(split_ms / med["bias_fp32"], 3),
        },
        "page_context": {"hardware": "RTX 5090 (comfy-kitchen int8_attention)", **PAGE_MS,
                         "step_tflops": round(page_value, 1)},
        "input_gen_s": round(gen_s, 1),
    }

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()

    if args.cpu_baseline == "on":
        out["cpu_baseline"] = cpu_baseline(q_np, k_np, v_np, bias32_np, w, core, skirts, args.cpu_rows)

    print(json.dumps(out))
    return 0


COPY_BYTES = 256 << 20
UNMASKED_KERNEL = "attn_fwd_kernel<128, 1, 4, false, false, false, false>"


def _counter_per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} of one rocprofv3 counter_collection.csv (values summed
    over the rows a dispatch reports, e.g. one per XCD)."""
    import collections
    import csv
    import glob

    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    per = collections.defaultdict(float)
    names = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, r["Dispatch_Id"])
            per[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("qfa::", "")
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    return out


def pmc_summary(fetch_dir: str, write_dir: str) -> int:
    """HBM bytes per unmasked attention launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a plain device copy of COPY_BYTES."""
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")

    def pick(d, needle):
        vals = [v for n, vs in d.items() if needle in n for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of {needle!r} in the counter files")
        return statistics.median(vals)

    copy_f, copy_w = pick(fetch, "copyBuffer") * 1024.0, pick(write, "copyBuffer") * 1024.0
    f_scale, w_scale = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    un_f, un_w = pick(fetch, UNMASKED_KERNEL) * 1024.0 * f_scale, pick(write, UNMASKED_KERNEL) * 1024.0 * w_scale
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 bench.py --cpu-baseline off "
           "--steps 2 --warmup 1 --variant-iters 1 --copy-calibration")
    out = {
        "what": "HBM bytes per launch of the unmasked banded attention call (B1 H56 Sq4096 Sk33600 D128 bf16)",
        "kernel": UNMASKED_KERNEL,
        "source_sha256_16": src_hash(ATTN_SRC),
        "commands": [cmd.format(c="FETCH_SIZE"), cmd.format(c="WRITE_SIZE"),
                     "python3 bench.py --pmc-summary <fetch dir> <write dir>"],
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_counter_bytes": copy_f, "write_counter_bytes": copy_w,
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "launches": {"unmasked": {"fetch_bytes": round(un_f), "write_bytes": round(un_w),
                                  "hbm_bytes_per_launch": round(un_f + un_w)}},
    }
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out["launches"]["unmasked"]))
    return 0


def cpu_baseline(q_np, k_np, v_np, bias_np, w, core, skirts, rows):
    """The oracle, as it stands, on a bounded sample: head 0, its first `rows`
    query rows against all 33600 keys, for the same step (quantize, unmasked,
    fp32 bias, core + skirt + merge)."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    q1 = np.ascontiguousarray(q_np[:, :1, :rows])
    k1 = np.ascontiguousarray(k_np[:, :1])
    v1 = np.ascontiguousarray(v_np[:, :1])
    t0 = time.perf_counter()
    ref = oracle.quantize_qk(q1, k1)
    oracle.attn(ref, v1, w.sm_scale)
    oracle.attn(ref, v1, w.sm_scale, bias=bias_np)
    oc, lc = oracle.attn(ref, v1, w.sm_scale, segments=[core])
    os_, ls = oracle.attn(ref, v1, w.sm_scale, bias=bias_np, segments=skirts)
    oracle.lse_merge(oc, lc, os_, ls)
    dt = time.perf_counter() - t0
    flops = 3 * 4.0 * rows * w.Sk * w.D
    return {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"head 0 of 56, query rows 0..{rows - 1} of 4096, all 33600 keys: K mean + int8 quantize, "
                  f"unmasked, fp32-bias, core+skirt+merge (same step); {dt:.1f} s",
        "seconds": round(dt, 2),
    }


if __name__ == "__main__":
    sys.exit(main())
