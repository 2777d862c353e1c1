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

# the attention kernel's sources: the template, its dispatch and its instance files
ATTN_SRC = sorted(os.path.join(ROOT, "quantized_flash_attention_amd", "csrc", f)
                  for f in os.listdir(os.path.join(ROOT, "quantized_flash_attention_amd", "csrc"))
                  if f.startswith("attn_fwd"))
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_band_unmasked_pmc.json")
# the bandwidth kernels' sources (quantize, LSE merge, map-to-index)
BW_SRC = [os.path.join(ROOT, "quantized_flash_attention_amd", "csrc", f)
          for f in ("quantize.hip", "lse_merge.hip", "blockmask.hip")]


def src_hash(paths) -> str:
    h = hashlib.sha256()
    for p in ([paths] if isinstance(paths, str) else paths):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


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
    ap.add_argument("--variant-iters", type=int, default=100, help="timed iterations of each per-call loop")
    ap.add_argument("--variant-warmup", type=int, default=50, help="warm-up iterations of each per-call loop")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows per head the oracle computes")
    ap.add_argument("--cpu-heads", type=int, default=3, help="heads the oracle computes (about 13 s on 16 cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the step: time the other configurations (dense 4k with LSE off/on, d64 fp16, "
                         "tile-64 block-sparse 128k) and a bf16 / int8 GEMM on the box; one JSON line each")
    ap.add_argument("--bandwidth", action="store_true",
                    help="instead of the step: the bandwidth-bound calls (quantize, LSE merge, map-to-index) over "
                         "rotated input sets larger than the MALL; one JSON line")
    ap.add_argument("--only", default=None,
                    help="with --configs or --bandwidth: comma-separated names of the lines/rows to run")
    ap.add_argument("--pmc-table", nargs="+", metavar="DIR",
                    help="print a markdown table of rocprofv3 --pmc output directories (median per kernel and grid)")
    ap.add_argument("--kernel", default=None, help="with --pmc-table: regular expression the kernel name must match")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE passes over "
                         "this script with --copy-calibration) into " + os.path.relpath(PMC_FILE, ROOT))
    args = ap.parse_args()
    if args.pmc_table:
        return pmc_table(args.pmc_table, args.kernel)
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
    if args.configs:
        return other_configs(dev, args.only)
    if args.bandwidth:
        return bandwidth(dev, args.only)
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

    # each variant in a loop of its own: warm-ups, then timed calls (median and min); the bf16-bias
    # call runs only here (same kernel instance as the fp32 bias call)
    qk = step()
    torch.cuda.synchronize()

    def loop(fn):
        for _ in range(args.variant_warmup):
            fn()
        evs = []
        for _ in range(args.variant_iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in evs]
        return {"median_ms": round(statistics.median(ts), 4), "min_ms": round(min(ts), 4)}

    def split_call():
        qfa.attn_fwd(qk, v, sm, segments=[core], out=o_core, lse=l_core)
        qfa.attn_fwd(qk, v, sm, bias=bias32, segments=skirts, out=o_skirt, lse=l_skirt)
        qfa.lse_merge(o_core, l_core, o_skirt, l_skirt, out=o_split, lse_out=l_split)

    variants = {
        "unmasked": loop(lambda: qfa.attn_fwd(qk, v, sm, out=o_un)),
        "bias_fp32": loop(lambda: qfa.attn_fwd(qk, v, sm, bias=bias32, out=o_bias)),
        "bias_bf16": loop(lambda: qfa.attn_fwd(qk, v, sm, bias=bias16, out=o_bias)),
        "split": loop(split_call),
        "quantize": loop(lambda: qfa.quantize_qk(q, k, workspace=ws)),
    }
    med["bias_bf16"] = variants["bias_bf16"]["median_ms"]

    flops_full = 4.0 * B * H * Sq * Sk * D
    tflops = lambda fl, ms: fl / (ms * 1e-3) / 1e12
    split_ms = med["core"] + med["skirt"] + med["merge"]
    # algorithmic bytes of the quantize step: read Q and K once, write codes, scales, mean,
    # centring term (820 MB); the kernel's second read of K (the mean, then the codes) is
    # implementation traffic, reported beside it
    qbytes = (B * H * (Sq + Sk) * D * 2 + B * H * (Sq + Sk) * D + B * H * (Sq + Sk) * 4
              + B * H * D * 4 + B * H * Sq * 4)
    qbytes_k2 = B * H * Sk * D * 2
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
            "quantize_model_MB": round(qbytes / 1e6, 1),
            "quantize_second_k_read_MB": round(qbytes_k2 / 1e6, 1),
            "quantize_GBps_with_second_k_read": round((qbytes + qbytes_k2) / (med["quantize"] * 1e-3) / 1e9, 1),
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
        "variant_loops": {"warmup": args.variant_warmup, "timed": args.variant_iters, **variants,
                          "bias_fp32_over_unmasked": round(variants["bias_fp32"]["median_ms"]
                                                           / variants["unmasked"]["median_ms"], 3),
                          "split_over_single_bias": round(variants["split"]["median_ms"]
                                                          / variants["bias_fp32"]["median_ms"], 3)},
        "page_context": {"hardware": "RTX 5090 (comfy-kitchen int8_attention)", **PAGE_MS,
                         "step_tflops": round(page_value, 1)},
        "input_gen_s": round(gen_s, 1),
        "device": device_info(dev),
    }

    # the on-box MFMA ceiling of the same instruction mix (after the timed steps: it runs the
    # matrix cores flat out and would heat the GPU before them)
    try:
        ceil = probe_mfma(dev, 0)
        out["roofline"]["measured_mfma_ceiling"] = ceil
        out["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceil["tflops"], 4)
        # the same MFMAs with the tile's softmax VALU work interleaved, with no memory, LDS or barrier
        ideal = probe_mfma(dev, 3)
        out["roofline"]["measured_compute_only_tile"] = ideal
        out["roofline"]["frac_of_compute_only_tile"] = round(achieved / ideal["tflops"], 4)
    except Exception as e:   # a measurement add-on: never lose the step line to it
        out["roofline"]["measured_mfma_ceiling"] = {"error": f"{type(e).__name__}: {str(e)[:200]}"}

    # the step's bandwidth-bound calls again, over rotated input sets that do not fit the MALL
    try:
        del q, k, v, o_un, o_bias, o_core, o_skirt, o_split, qk, ws
        torch.cuda.empty_cache()
        bw = {r["row"]: r for r in bandwidth_rows(dev, ["copy", "quantize_c4", "merge_c4"])}
        out["bandwidth_rotated"] = {
            "sets": "3 per call, > 256 MB in total",
            "copy_GBps": bw["copy"]["GBps"],
            "quantize_ms": bw["quantize_c4"]["ms"], "quantize_model_MB": bw["quantize_c4"]["model_MB"],
            "quantize_GBps_model": bw["quantize_c4"]["GBps_model"],
            "quantize_frac_hbm_model": bw["quantize_c4"]["frac_hbm_model"],
            "quantize_second_k_read_MB": bw["quantize_c4"]["second_k_read_MB"],
            "quantize_GBps_with_second_k_read": bw["quantize_c4"]["GBps_with_second_k_read"],
            "merge_ms": bw["merge_c4"]["ms"], "merge_GBps": bw["merge_c4"]["GBps"],
            "merge_frac_hbm": bw["merge_c4"]["frac_hbm"]}
    except Exception as e:   # a measurement add-on: never lose the step line to it
        out["bandwidth_rotated"] = {"error": f"{type(e).__name__}: {str(e)[:200]}"}

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()

    if args.cpu_baseline == "on":
        out["cpu_baseline"] = cpu_baseline(q_np, k_np, v_np, bias32_np, w, core, skirts, args.cpu_rows,
                                           args.cpu_heads, gpu_ms=med)

    print(json.dumps(out))
    return 0


COPY_BYTES = 256 << 20
UNMASKED_KERNEL = "attn_fwd_kernel<128, 1, 4, false, false, false, false, false, false, false>"
# the unmasked instance: D 128, bf16 V, 4 waves, every mode flag false
UNMASKED_RE = r"attn_fwd_kernel<128, 1, 4(, false)+>"


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
        import re
        rx = UNMASKED_RE if needle == UNMASKED_KERNEL else re.escape(needle)
        vals = [v for n, vs in d.items() if re.search(rx, n) for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of {needle!r} in the counter files")
        return statistics.median(vals)

    def pick_copy(d):
        # the calibration copy: copyBuffer dispatches that moved at least a quarter of COPY_BYTES
        # (torch's small device-to-device copies use the same kernel)
        vals = [v for n, vs in d.items() if "copyBuffer" in n for v in vs if v * 1024.0 >= COPY_BYTES / 8]
        if not vals:
            raise SystemExit("no calibration copy in the counter files (run with --copy-calibration)")
        return statistics.median(vals)

    copy_f, copy_w = pick_copy(fetch) * 1024.0, pick_copy(write) * 1024.0
    f_scale, w_scale = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    un_f, un_w = pick(fetch, UNMASKED_KERNEL) * 1024.0 * f_scale, pick(write, UNMASKED_KERNEL) * 1024.0 * w_scale
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 bench.py --cpu-baseline off "
           "--steps 2 --warmup 1 --variant-iters 1 --variant-warmup 0 --copy-calibration")
    out = {
        "what": "HBM bytes per launch of the unmasked banded attention call (B1 H56 Sq4096 Sk33600 D128 bf16), "
                "and of the step's quantize and LSE-merge kernels on the same workload",
        "kernel": UNMASKED_KERNEL,
        "source_sha256_16": src_hash(ATTN_SRC),
        "commands": [cmd.format(c="FETCH_SIZE"), cmd.format(c="WRITE_SIZE"),
                     "python3 bench.py --pmc-summary <fetch dir> <write dir>"],
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_counter_bytes": copy_f, "write_counter_bytes": copy_w,
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "launches": {"unmasked": {"fetch_bytes": round(un_f), "write_bytes": round(un_w),
                                  "hbm_bytes_per_launch": round(un_f + un_w)}},
    }
    # the step's bandwidth kernels on the same workload: the three launches of the quantize call
    # and the LSE merge (same scaling), beside their algorithmic bytes
    B, H, Sq, Sk, D = 1, 56, 4096, 33600, 128
    q_model = (B * H * (Sq + Sk) * D * 2 + B * H * (Sq + Sk) * (D + 4) + B * H * D * 4 + B * H * Sq * 4)
    m_model = B * H * Sq * (2 * D * 4 + 2 * 4 + D * 2 + 4)
    other = {}
    for key, name in (("kmean_partial", "kmean_partial_kernel<1, 128>"), ("kmean_finalize", "kmean_finalize_kernel"),
                      ("quantize", "quantize_kernel<1, 128>"), ("lse_merge", "lse_merge_kernel<128>")):
        f_b, w_b = pick(fetch, name) * 1024.0 * f_scale, pick(write, name) * 1024.0 * w_scale
        other[key] = {"kernel": name, "fetch_bytes": round(f_b), "write_bytes": round(w_b)}
    qsum = sum(other[k]["fetch_bytes"] + other[k]["write_bytes"] for k in ("kmean_partial", "kmean_finalize", "quantize"))
    out["bandwidth_kernels"] = {
        "source_sha256_16": src_hash(BW_SRC),
        "per_dispatch": other,
        "quantize_call": {"hbm_bytes": qsum, "algorithmic_bytes": q_model,
                          "second_k_read_bytes": B * H * Sk * D * 2,
                          "ratio_to_algorithmic": round(qsum / q_model, 3)},
        "lse_merge": {"hbm_bytes": other["lse_merge"]["fetch_bytes"] + other["lse_merge"]["write_bytes"],
                      "algorithmic_bytes": m_model},
    }
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out["launches"]["unmasked"]))
    return 0


def pmc_table(dirs, kernel_rx=None) -> int:
    """Markdown table of rocprofv3 --pmc output directories: per kernel (and grid size), the number
    of dispatches, their median duration and the median over dispatches of each counter (summed
    over the rows a dispatch reports). FETCH_SIZE / WRITE_SIZE are printed in KiB as counted."""
    import collections
    import csv
    import glob
    import re

    rx = re.compile(kernel_rx) if kernel_rx else None
    per = collections.defaultdict(lambda: collections.defaultdict(float))   # (dir, dispatch) -> counter -> value
    meta = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            for r in csv.DictReader(open(f)):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("qfa::", "")
                name = name.split("(")[0].replace("void ", "")
                if rx and not rx.search(name):
                    continue
                key = (f, r["Dispatch_Id"])
                per[key][r["Counter_Name"]] += float(r["Counter_Value"])
                meta[key] = (name, int(r["Grid_Size"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    groups = collections.defaultdict(list)
    for key, (name, grid, us) in meta.items():
        groups[(name, grid)].append(key)
    counters = sorted({c for v in per.values() for c in v})
    print("| kernel | grid | dispatches | median us | " + " | ".join(counters) + " |")
    print("|---|---:|---:|---:|" + "---:|" * len(counters))
    for (name, grid), keys in sorted(groups.items()):
        us = statistics.median(meta[k][2] for k in keys)
        vals = []
        for c in counters:
            xs = [per[k][c] for k in keys if c in per[k]]
            vals.append(f"{statistics.median(xs):.4g}" if xs else "")
        print(f"| `{name}` | {grid} | {len(keys)} | {us:.1f} | " + " | ".join(vals) + " |")
    return 0


PROBE_LIB = os.path.join(ROOT, "quantized_flash_attention_amd", "libqfa_probe.so")
# multiply-add pairs counted as 2 ops each: one wave-iteration of the probe is one 32-row x 64-key
# attention tile's MFMAs (8 int8 32x32x32 + 16 bf16 32x32x16)
PROBE_OPS = {0: 8 * 65536 + 16 * 32768, 1: 8 * 65536, 2: 16 * 32768, 3: 8 * 65536 + 16 * 32768, 4: 0,
             5: 16 * 32768, 6: 8 * 65536 + 16 * 32768, 7: 8 * 65536 + 16 * 32768, 8: 8 * 65536 + 16 * 32768,
             9: 8 * 65536 + 16 * 32768, 10: 8 * 65536 + 16 * 32768}
PROBE_PEAK = {0: PEAK_BLEND, 1: PEAK_I8_TOPS, 2: PEAK_BF16_TFLOPS, 3: PEAK_BLEND, 4: None, 5: PEAK_BF16_TFLOPS,
              6: PEAK_BLEND, 7: PEAK_BLEND, 8: PEAK_BLEND, 9: PEAK_BLEND, 10: PEAK_BLEND}
PROBE_MIX = ["int8 QK + bf16 PV MFMAs (attention tile)", "int8 32x32x32 only", "bf16 32x32x16 only",
             "attention tile MFMAs + its softmax VALU work (64 fma, 16 max, 32 exp2, 16 pack, 16 dot2 per lane)",
             "the softmax VALU work alone", "bf16 32x32x16 only, constant operands",
             "int8 QK + bf16 PV MFMAs, constant operands",
             "MFMA phase and VALU phase alternating between barriers, second wave group one phase behind",
             "MFMA phase and VALU phase alternating between barriers, both wave groups in step",
             "tile MFMAs + softmax VALU work, bf16 accumulators in AccVGPRs",
             "tile MFMAs + softmax VALU work, every accumulator in AccVGPRs"]


def probe_mfma(dev, mix: int = 0, iters: int = 4000, reps: int = 3) -> dict:
    """The matrix-core throughput the GPU sustains for the attention tile's MFMA mix (qfa_probe_mfma:
    random operands, the attention kernel's launch shape of two 4-wave blocks per CU), with the
    shader clock the loop ran at (s_memtime cycles over the 100 MHz s_memrealtime). Each launch runs
    a few milliseconds: much longer launches of back-to-back MFMAs were seen to slow down about 30x
    at a high reported clock, which measures a throttle, not the matrix cores."""
    import ctypes

    import torch

    L = ctypes.CDLL(PROBE_LIB)
    L.qfa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.qfa_probe_mfma.restype = ctypes.c_int
    blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    sink = torch.empty(256 * (blocks + 1), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch():
        st = L.qfa_probe_mfma(blocks, iters, mix, ctypes.c_void_p(clocks.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                              ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"qfa_probe_mfma returned {st}")

    launch()
    torch.cuda.synchronize()
    nrec = blocks if mix < 7 else (blocks + 1) // 2   # blocks that wrote a clock record
    times, clks = [], []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        c = clocks.view(-1, 2)[:nrec].double().sum(0).tolist()
        clks.append(c[0] / c[1] * 0.1)   # cycles per 10 ns tick -> GHz
    ms = statistics.median(times)
    ghz = statistics.median(clks)
    ncu = blocks // 2
    waves_per_simd = blocks * 4 / (4 * ncu)
    out = {"mix": PROBE_MIX[mix], "clock_ghz": round(ghz, 3), "ms": round(ms, 3), "blocks": blocks, "iters": iters,
           # SIMD cycles per wave-iteration: one iteration is one 32-row x 64-key tile of one wave
           "simd_cycles_per_wave_tile": round(ms * 1e-3 * ghz * 1e9 / (iters * waves_per_simd), 1)}
    if PROBE_OPS[mix]:
        tflops = blocks * 4 * iters * PROBE_OPS[mix] / (ms * 1e-3) / 1e12
        out.update(tflops=round(tflops, 1), frac_of_published_peak=round(tflops / PROBE_PEAK[mix], 4),
                   frac_of_peak_at_this_clock=round(tflops / (PROBE_PEAK[mix] * ghz / 2.4), 4))
    return out


def device_info(dev) -> dict:
    import torch

    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__}


def _time_ms(fn, iters: int, warmup: int = 3) -> float:
    """Median milliseconds of fn() over `iters` launches, HIP events on the current stream."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in evs)


def other_configs(dev, only=None) -> int:
    """One JSON line per configuration besides the step's banded workload: quantize and attention
    times, effective TFLOPS (4*B*H*Sq*Sk_eff*D; block-sparse counts the selected 64x64 tile pairs,
    causal the S(S+1)/2 attended pairs)
    and the fraction of the blended int8/bf16 MFMA peak; quantize / map-to-index bandwidth against
    HBM's 8 TB/s. Last, a bf16 and an int8 GEMM through torch as an on-box matrix-core reference."""
    import numpy as np
    import torch

    import quantized_flash_attention_amd as qfa
    import workloads as W

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def qbytes(B, H, Sq, Sk, D, esz):
        # algorithmic bytes: read Q and K once; write codes, scales, K mean, centring term (the
        # kernel's second read of K is implementation traffic). These lines re-quantize the same
        # tensors, which the 256 MB MALL may hold: the HBM figures are those of --bandwidth.
        return B * H * (Sq + Sk) * D * esz + B * H * (Sq + Sk) * (D + 4) + B * H * D * 4 + B * H * Sq * 4

    names = ("mfma_ceiling", "dense4k", "d64", "dense4k_bias_forms", "flydsl_causal_shapes", "band_shard_h7_split_k",
             "band_keep_mask", "sparse", "gemm_reference")
    want = set(only.split(",")) if only else set(names)
    if want - set(names):
        print(f"bench.py: unknown --only lines {sorted(want - set(names))}; known: {', '.join(names)}", file=sys.stderr)
        return 2

    def sel(name):
        return name in want

    info = device_info(dev)
    if sel("mfma_ceiling"):
        print(json.dumps({"config": "mfma_ceiling", "what": "qfa_probe_mfma: the attention tile's MFMA mix on random "
                          "operands, 2 blocks of 4 waves per CU, no other work",
                          "rows": [probe_mfma(dev, m) for m in range(11)], "device": info}), flush=True)

    for name in [n for n in ("dense4k", "d64") if sel(n)]:
        w = W.WORKLOADS[name]
        q_np, k_np, v_np = W.make_qkv(w)
        q, k, v = up(q_np), up(k_np), up(v_np)
        ws = torch.empty(qfa.quantize_workspace_bytes(w.B, w.H, w.Sk, w.D), dtype=torch.uint8, device=dev)
        qk = qfa.quantize_qk(q, k, workspace=ws)
        out = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
        t_q = _time_ms(lambda: qfa.quantize_qk(q, k, workspace=ws), 20)
        t_a = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, out=out), 20)
        t_l = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, out=out, lse=lse), 20)
        t_c = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, causal=True, out=out), 20)
        fl = 4.0 * w.B * w.H * w.Sq * w.Sk * w.D
        fl_c = 4.0 * w.B * w.H * w.D * (w.Sq * (w.Sq + 1) / 2)   # attended (row, key) pairs j <= i
        qb = qbytes(w.B, w.H, w.Sq, w.Sk, w.D, 2)
        print(json.dumps({
            "config": name, "shape": f"B{w.B} H{w.H} Sq{w.Sq} Sk{w.Sk} D{w.D} {w.dtype}",
            "quantize_ms": round(t_q, 4), "quantize_GBps": round(qb / (t_q * 1e-3) / 1e9, 1),
            "quantize_frac_hbm": round(qb / (t_q * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
            "attn_ms": round(t_a, 4), "attn_tflops": round(fl / (t_a * 1e-3) / 1e12, 1),
            "attn_frac_blend": round(fl / (t_a * 1e-3) / 1e12 / PEAK_BLEND, 4),
            "attn_lse_ms": round(t_l, 4), "lse_over_plain": round(t_l / t_a, 3),
            "causal_ms": round(t_c, 4), "causal_tflops": round(fl_c / (t_c * 1e-3) / 1e12, 1),
            "causal_frac_blend": round(fl_c / (t_c * 1e-3) / 1e12 / PEAK_BLEND, 4), "device": info}), flush=True)
        del q, k, v, qk, out, lse, ws
        torch.cuda.empty_cache()

    if sel("dense4k_bias_forms"):
        # dense4k with a materialised per-query bias [1,1,Q,K] (the slow path) against the shared
        # per-key bias [1,1,1,K] and no bias
        w = W.WORKLOADS["dense4k"]
        q_np, k_np, v_np = W.make_qkv(w)
        q, k, v = up(q_np), up(k_np), up(v_np)
        qk = qfa.quantize_qk(q, k)
        out = torch.empty_like(q)
        gen = torch.Generator(device=dev)
        gen.manual_seed(2)
        b_key = torch.randn((1, 1, 1, w.Sk), generator=gen, device=dev)
        b_f32 = torch.randn((1, 1, w.Sq, w.Sk), generator=gen, device=dev)
        b_bf16 = b_f32.to(torch.bfloat16)
        b_bool = b_f32 > -1.0
        line = {"config": "dense4k_bias_forms", "shape": f"B{w.B} H{w.H} Sq{w.Sq} Sk{w.Sk} D{w.D} bf16"}
        for name, b in (("none", None), ("per_key_fp32", b_key), ("per_query_fp32", b_f32),
                        ("per_query_bf16", b_bf16), ("per_query_bool", b_bool)):
            line[name + "_ms"] = round(_time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, bias=b, out=out), 20), 4)
        line["device"] = info
        print(json.dumps(line), flush=True)
        del q, k, v, qk, out, b_key, b_f32, b_bf16, b_bool
        torch.cuda.empty_cache()

    if sel("flydsl_causal_shapes"):
        # the causal shapes of ROCm/FlyDSL PR #886's timed table, (B, S, H, Hkv, D) and its FlyDSL
        # +LSE latency in us (bf16 QK on an MI350X: context, not a target); TFLOPS as that table
        # counts them, half of 4*B*H*S*S*D
        flydsl = [((2, 2048, 16, 16, 128), 51.3), ((2, 4096, 16, 16, 128), 154.7), ((1, 8192, 16, 16, 128), 262.8),
                  ((2, 2048, 16, 2, 128), 50.4), ((4, 2048, 8, 8, 64), 38.7), ((8, 1024, 16, 16, 128), 58.5)]
        gen = torch.Generator(device=dev)
        gen.manual_seed(886)
        rows = []
        for (B, S, H, Hkv, D), page_us in flydsl:
            q = torch.randn((B, H, S, D), generator=gen, device=dev).to(torch.bfloat16)
            k = torch.randn((B, Hkv, S, D), generator=gen, device=dev).to(torch.bfloat16)
            v = torch.randn((B, Hkv, S, D), generator=gen, device=dev).to(torch.bfloat16)
            ws = torch.empty(qfa.quantize_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device=dev)
            qk = qfa.quantize_qk(q, k, workspace=ws)
            out = torch.empty_like(q)
            lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
            scale = D ** -0.5
            t_q = _time_ms(lambda: qfa.quantize_qk(q, k, workspace=ws), 20)
            t_a = _time_ms(lambda: qfa.attn_fwd(qk, v, scale, causal=True, out=out, lse=lse), 20)
            t_b = _time_ms(lambda: qfa.attn_fwd_unquant(q, k, v, scale, causal=True, out=out, lse=lse), 20)
            fl = 4.0 * B * H * S * S * D / 2
            rows.append({"shape": f"B{B} S{S} H{H} Hkv{Hkv} D{D}", "quantize_us": round(t_q * 1e3, 1),
                         "attn_us": round(t_a * 1e3, 1), "attn_tflops": round(fl / (t_a * 1e-3) / 1e12, 1),
                         "attn_frac_blend": round(fl / (t_a * 1e-3) / 1e12 / PEAK_BLEND, 4),
                         "end_to_end_us": round((t_q + t_a) * 1e3, 1),
                         "bf16qk_us": round(t_b * 1e3, 1), "bf16qk_tflops": round(fl / (t_b * 1e-3) / 1e12, 1),
                         "page_flydsl_lse_us": page_us})
            del q, k, v, ws, qk, out, lse
        torch.cuda.empty_cache()
        print(json.dumps({"config": "flydsl_causal_shapes", "mode": "causal, LSE on, bf16 V; int8 QK, and bf16 QK (bf16qk_*)",
                          "rows": rows, "device": info}), flush=True)

    if sel("band_shard_h7_split_k"):
        # split-K on the banded workload's 8-GPU shard: 7 heads give 224 query blocks for 256 CUs
        w = W.WORKLOADS["band"]
        q_np, k_np, v_np = W.make_qkv(w, H=7)
        q, k, v = up(q_np), up(k_np), up(v_np)
        del q_np, k_np, v_np
        bias = up(W.bias_tensor(W.band_bias(w.Sk, core=w.extras["core"], skirt=w.extras["skirt"]), "fp32"))
        qk = qfa.quantize_qk(q, k)
        out = torch.empty_like(q)
        lse = torch.empty((1, 7, w.Sq), dtype=torch.float32, device=dev)
        ns = qfa.splits_auto(1, 7, w.Sq, w.Sk)
        ws = torch.empty(max(1, qfa.split_workspace_bytes(1, 7, w.Sq, w.D, ns)), dtype=torch.uint8, device=dev)
        line = {"config": "band_shard_h7_split_k", "shape": f"B1 H7 Sq{w.Sq} Sk{w.Sk} D{w.D} bf16, fp32 bias, LSE on",
                "auto_splits": ns}
        fl = 4.0 * 7 * w.Sq * w.Sk * w.D
        for n in sorted({1, 2, ns, 8}):
            wsn = ws if n == ns else None
            t = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, bias=bias, out=out, lse=lse, splits=n, workspace=wsn), 10)
            line[f"splits{n}_ms"] = round(t, 4)
            line[f"splits{n}_frac_blend"] = round(fl / (t * 1e-3) / 1e12 / PEAK_BLEND, 4)
        line["device"] = info
        print(json.dumps(line), flush=True)
        del q, k, v, bias, qk, out, lse, ws
        torch.cuda.empty_cache()

    if sel("band_keep_mask"):
        # the banded workload with the pages' bool [1,1,1,K] keep mask (raised-cosine weight > 1e-3)
        w = W.WORKLOADS["band"]
        q_np, k_np, v_np = W.make_qkv(w)
        q, k, v = up(q_np), up(k_np), up(v_np)
        del q_np, k_np, v_np
        weights = np.exp(W.band_bias(w.Sk, core=w.extras["core"], skirt=w.extras["skirt"]))
        keep = torch.from_numpy((weights > 1e-3).reshape(1, 1, 1, -1)).to(dev)
        ws = torch.empty(qfa.quantize_workspace_bytes(w.B, w.H, w.Sk, w.D), dtype=torch.uint8, device=dev)
        qk = qfa.quantize_qk(q, k, workspace=ws)
        out = torch.empty_like(q)
        t_u = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, out=out), 10)
        t_k = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, bias=keep, out=out), 10)
        print(json.dumps({
            "config": "band_keep_mask", "shape": f"B{w.B} H{w.H} Sq{w.Sq} Sk{w.Sk} D{w.D} {w.dtype}",
            "kept_keys": int(keep.sum().item()), "unmasked_ms": round(t_u, 4), "keep_mask_ms": round(t_k, 4),
            "keep_over_unmasked": round(t_k / t_u, 3), "device": info}), flush=True)
        del q, k, v, qk, out, keep, ws
        torch.cuda.empty_cache()

    if sel("sparse"):
        w = W.WORKLOADS["sparse"]
        T = w.Sk // 64
        mask_np = W.sparse_mask(T, w.H, w.extras["prefix"], w.extras["band"])
        vbs_np = W.sparse_vbs(T, w.extras["last_valid"])
        q_np, k_np, v_np = W.make_qkv(w)
        for x in (q_np, k_np, v_np):
            W.zero_pads(x, vbs_np)
        q, k, v = up(q_np), up(k_np), up(v_np)
        del q_np, k_np, v_np
        mask, vbs, vsc = up(mask_np.astype(np.uint8)), up(vbs_np), up(W.v_scale(w))
        ws = torch.empty(qfa.quantize_workspace_bytes(w.B, w.H, w.Sk, w.D), dtype=torch.uint8, device=dev)
        qk = qfa.quantize_qk(q, k, vbs=vbs, workspace=ws)
        idx, cnt = qfa.blockmask_to_index(mask)
        out = torch.empty_like(q)
        t_m = _time_ms(lambda: qfa.blockmask_to_index(mask), 20)
        t_q = _time_ms(lambda: qfa.quantize_qk(q, k, vbs=vbs, workspace=ws), 10)
        t_a = _time_ms(lambda: qfa.attn_fwd(qk, v, w.sm_scale, index=idx, count=cnt, vbs=vbs, v_scale=vsc, out=out), 10)
        pairs = int(mask_np.sum())
        fl = 4.0 * w.D * 64 * 64 * pairs
        mb = mask_np.size + pairs * 4 + w.B * w.H * T * 4   # mask bytes read; entries + counts written
        qb = qbytes(w.B, w.H, w.Sq, w.Sk, w.D, 2)
        print(json.dumps({
            "config": "sparse", "shape": f"B{w.B} H{w.H} S{w.Sq} D{w.D} {w.dtype}, tile-64 mask prefix 8 + band 48",
            "tile_pairs": pairs, "map_to_index_ms": round(t_m, 4), "map_to_index_GBps": round(mb / (t_m * 1e-3) / 1e9, 1),
            "quantize_ms": round(t_q, 4), "quantize_GBps": round(qb / (t_q * 1e-3) / 1e9, 1),
            "attn_ms": round(t_a, 4), "attn_tflops": round(fl / (t_a * 1e-3) / 1e12, 1),
            "attn_frac_blend": round(fl / (t_a * 1e-3) / 1e12 / PEAK_BLEND, 4),
            "end_to_end_ms": round(t_m + t_q + t_a, 4), "device": info}), flush=True)
        del q, k, v, qk, out, idx, cnt, mask, ws
        torch.cuda.empty_cache()

    if sel("gemm_reference"):
        # matrix-core reference through torch (hipBLASLt / rocBLAS): 8192^3 GEMMs
        n = 8192
        a = torch.randn(n, n, device=dev).to(torch.bfloat16)
        b = torch.randn(n, n, device=dev).to(torch.bfloat16)
        t_bf = _time_ms(lambda: torch.matmul(a, b), 10)
        gemm = {"bf16_tflops": round(2.0 * n ** 3 / (t_bf * 1e-3) / 1e12, 1)}
        try:
            a8 = torch.randint(-127, 128, (n, n), device=dev, dtype=torch.int8)
            b8 = torch.randint(-127, 128, (n, n), device=dev, dtype=torch.int8)
            t_i8 = _time_ms(lambda: torch._int_mm(a8, b8), 10)
            gemm["int8_tops"] = round(2.0 * n ** 3 / (t_i8 * 1e-3) / 1e12, 1)
        except (RuntimeError, AttributeError) as e:
            gemm["int8_tops"] = None
            gemm["int8_note"] = str(e).splitlines()[0][:120]
        print(json.dumps({"config": "gemm_reference", "m=n=k": n, **gemm,
                          "published_dense_peaks": {"bf16_tflops": PEAK_BF16_TFLOPS, "int8_tops": PEAK_I8_TOPS},
                          "device": info}), flush=True)

    return 0


def _time_rotated(dev, fns, rounds: int):
    """Median milliseconds per call of fns[0], fns[1], ... cycled `rounds` times (HIP events on
    the current stream around each call). A run of 1 GiB fills is queued first: it flushes the
    256 MB MALL and keeps the GPU busy while the host enqueues the calls, so the host's call
    overhead stays out of the events."""
    import torch

    for f in fns:
        f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    busy = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(max(8, len(fns) * rounds // 2)):
        busy.fill_(1.0)
    evs = []
    for _ in range(rounds):
        for f in fns:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            evs.append((e0, e1))
    torch.cuda.synchronize()
    del busy
    return statistics.median(a.elapsed_time(b) for a, b in evs)


BW_ROWS = ("copy", "quantize_c2", "quantize_c3", "quantize_c4", "quantize_c5", "merge_c4", "map_to_index_c5")


def bandwidth(dev, only=None) -> int:
    """One JSON line of bandwidth_rows (below)."""
    want = only.split(",") if only else list(BW_ROWS)
    bad = set(want) - set(BW_ROWS)
    if bad:
        print(f"bench.py: unknown --only rows {sorted(bad)}; known: {', '.join(BW_ROWS)}", file=sys.stderr)
        return 2
    print(json.dumps({"config": "bandwidth", "what": "bandwidth-bound calls over rotated sets (> 256 MB in total)",
                      "rows": bandwidth_rows(dev, want), "device": device_info(dev)}), flush=True)
    return 0


def bandwidth_rows(dev, want) -> list:
    """The bandwidth-bound calls (quantize on the dense 4k, d64, banded and
    block-sparse shapes; the LSE merge of the banded split; the tile-mask map-to-index of the
    block-sparse shape) timed over >= 3 rotated input/output sets totalling more than the 256 MB
    MALL, so every call streams from HBM. Quantize bytes follow the algorithmic model (read Q and
    K once; write Q8, K8, qs, ks, the K mean and the centring term); the kernel's second read of
    K (mean, then codes) is reported as a separate figure. A plain device copy, rotated the same
    way, gives the rate the machine's HBM sustains for a read+write stream. Inputs are N(0,1) drawn on
    the GPU (the dense 4k K with its per-channel offset, the block-sparse pad rows zero): the
    calls' cost does not depend on the values."""
    import numpy as np
    import torch

    import quantized_flash_attention_amd as qfa
    import workloads as W

    gen = torch.Generator(device=dev)
    gen.manual_seed(101)
    rows = []
    want = set(want)

    def nsets(set_bytes):
        return max(3, -(-(300 << 20) // set_bytes))

    def rate(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    if "copy" in want:
        n = 256 << 20
        sets = [(torch.empty(n, dtype=torch.uint8, device=dev), torch.empty(n, dtype=torch.uint8, device=dev))
                for _ in range(3)]
        ms = _time_rotated(dev, [lambda s=s: s[1].copy_(s[0]) for s in sets], 6)
        rows.append({"row": "copy", "what": "device copy of 256 MiB (read + write)", "sets": 3,
                     "bytes": 2 * n, "ms": round(ms, 4), "GBps": rate(2 * n, ms),
                     "frac_hbm": round(2 * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        del sets

    for tag, name in (("c2", "dense4k"), ("c3", "d64"), ("c4", "band"), ("c5", "sparse")):
        if f"quantize_{tag}" not in want:
            continue
        w = W.WORKLOADS[name]
        B, H, Sq, Sk, D = w.B, w.H, w.Sq, w.Sk, w.D
        Hkv = w.extras.get("hkv", H)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        in_bytes = (B * H * Sq + B * Hkv * Sk) * D * 2
        model = in_bytes + (B * H * Sq + B * Hkv * Sk) * (D + 4) + B * Hkv * D * 4 + B * H * Sq * 4
        second_k = B * Hkv * Sk * D * 2
        n = nsets(model)
        vbs = None
        if name == "sparse":
            vbs = torch.from_numpy(W.sparse_vbs(Sk // 64, w.extras["last_valid"])).to(dev)
        sets = []
        for _ in range(n):
            q = torch.randn((B, H, Sq, D), generator=gen, device=dev, dtype=torch.float32).to(dt)
            k = torch.randn((B, Hkv, Sk, D), generator=gen, device=dev, dtype=torch.float32)
            if "k_offset_std" in w.extras:
                k += torch.randn((D,), generator=gen, device=dev) * w.extras["k_offset_std"]
            k = k.to(dt)
            if vbs is not None:
                last = Sk - 64 + w.extras["last_valid"]
                q[:, :, last:] = 0
                k[:, :, last:] = 0
            out = dict(q8=torch.empty((B, H, Sq, D), dtype=torch.int8, device=dev),
                       qs=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
                       k8=torch.empty((B, Hkv, Sk, D), dtype=torch.int8, device=dev),
                       ks=torch.empty((B, Hkv, Sk), dtype=torch.float32, device=dev),
                       kmean=torch.empty((B, Hkv, D), dtype=torch.float32, device=dev),
                       qmu=torch.empty((B, H, Sq), dtype=torch.float32, device=dev))
            ws = torch.empty(qfa.quantize_workspace_bytes(B, Hkv, Sk, D), dtype=torch.uint8, device=dev)
            sets.append((q, k, out, ws))
        fns = [lambda s=s: qfa.quantize_qk(s[0], s[1], vbs=vbs, workspace=s[3], out=s[2]) for s in sets]
        ms = _time_rotated(dev, fns, max(2, 12 // n))
        rows.append({"row": f"quantize_{tag}", "shape": f"B{B} H{H} Sq{Sq} Sk{Sk} D{D} {w.dtype}", "sets": n,
                     "model_MB": round(model / 1e6, 1), "second_k_read_MB": round(second_k / 1e6, 1),
                     "ms": round(ms, 4), "GBps_model": rate(model, ms),
                     "frac_hbm_model": round(model / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                     "GBps_with_second_k_read": rate(model + second_k, ms)})
        del sets, fns
        torch.cuda.empty_cache()

    if "merge_c4" in want:
        w = W.WORKLOADS["band"]
        B, H, S, D = w.B, w.H, w.Sq, w.D
        nbytes = B * H * S * (2 * D * 4 + 2 * 4 + D * 2 + 4)
        n = nsets(nbytes)
        sets = []
        for _ in range(n):
            oa = torch.randn((B, H, S, D), generator=gen, device=dev)
            ob = torch.randn((B, H, S, D), generator=gen, device=dev)
            la = torch.randn((B, H, S), generator=gen, device=dev)
            lb = torch.randn((B, H, S), generator=gen, device=dev)
            sets.append((oa, la, ob, lb, torch.empty((B, H, S, D), dtype=torch.bfloat16, device=dev),
                         torch.empty((B, H, S), dtype=torch.float32, device=dev)))
        fns = [lambda s=s: qfa.lse_merge(s[0], s[1], s[2], s[3], out=s[4], lse_out=s[5]) for s in sets]
        ms = _time_rotated(dev, fns, 4)
        rows.append({"row": "merge_c4", "shape": f"B{B} H{H} S{S} D{D}: two fp32 partials + LSE -> bf16 + LSE",
                     "sets": n, "MB": round(nbytes / 1e6, 1), "ms": round(ms, 4), "GBps": rate(nbytes, ms),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        del sets, fns
        torch.cuda.empty_cache()

    if "map_to_index_c5" in want:
        w = W.WORKLOADS["sparse"]
        T = w.Sk // 64
        mask_np = W.sparse_mask(T, w.H, w.extras["prefix"], w.extras["band"])
        pairs = int(mask_np.sum())
        nbytes = mask_np.size + pairs * 4 + w.B * w.H * T * 4   # mask read; entries + counts written
        n = nsets(nbytes)
        m0 = torch.from_numpy(mask_np.astype(np.uint8)).to(dev)
        masks = [m0.clone() for _ in range(n)]
        del m0
        fns = [lambda m=m: qfa.blockmask_to_index(m) for m in masks]
        ms = _time_rotated(dev, fns, 4)
        rows.append({"row": "map_to_index_c5", "shape": f"mask [1,{w.H},{T},{T}] uint8, {pairs} kept tile pairs",
                     "sets": n, "MB": round(nbytes / 1e6, 1), "ms": round(ms, 4), "GBps": rate(nbytes, ms),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        del masks, fns
        torch.cuda.empty_cache()

    return rows


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# the tiny configuration (B1 H2 S256 D128, K centred, LSE) through the oracle on one thread, best of 3;
# run in a child process (OMP_NUM_THREADS=1 must be set before the OpenMP runtime starts) that
# never touches the GPU
_C1_SINGLE = """
import json, sys, time
sys.path.insert(0, %r)
import oracle, workloads as W
w = W.WORKLOADS["tiny"]
q, k, v = W.make_qkv(w)
best = None
for _ in range(3):
    t0 = time.perf_counter()
    ref = oracle.quantize_qk(q, k)
    oracle.attn(ref, v, w.sm_scale)
    dt = time.perf_counter() - t0
    best = dt if best is None else min(best, dt)
print(json.dumps({"seconds": best}))
"""


def cpu_baseline(q_np, k_np, v_np, bias_np, w, core, skirts, rows, heads=3, gpu_ms=None):
    """The oracle, as it stands, on a bounded sample: the first `heads` heads, their first `rows`
    query rows against all 33600 keys, leg by leg as the GPU step runs them (quantize, unmasked,
    fp32 bias, core + skirt + merge), with the oracle's bias/unmasked and split/single ratios beside
    the GPU's; plus the tiny configuration on one thread."""
    import subprocess

    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    q1 = np.ascontiguousarray(q_np[:, :heads, :rows])
    k1 = np.ascontiguousarray(k_np[:, :heads])
    v1 = np.ascontiguousarray(v_np[:, :heads])
    legs = {}

    def leg(name, fn):
        t0 = time.perf_counter()
        r = fn()
        legs[name] = time.perf_counter() - t0
        return r

    ref = leg("quantize", lambda: oracle.quantize_qk(q1, k1))
    leg("unmasked", lambda: oracle.attn(ref, v1, w.sm_scale))
    leg("bias_fp32", lambda: oracle.attn(ref, v1, w.sm_scale, bias=bias_np))
    oc, lc = leg("core", lambda: oracle.attn(ref, v1, w.sm_scale, segments=[core]))
    os_, ls = leg("skirt", lambda: oracle.attn(ref, v1, w.sm_scale, bias=bias_np, segments=skirts))
    leg("merge", lambda: oracle.lse_merge(oc, lc, os_, ls))
    dt = sum(legs.values())
    flops = 3 * 4.0 * heads * rows * w.Sk * w.D
    split = legs["core"] + legs["skirt"] + legs["merge"]
    out = {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"heads 0..{heads - 1} of 56, query rows 0..{rows - 1} of 4096, all 33600 keys: K mean + int8 "
                  f"quantize, unmasked, fp32-bias, core+skirt+merge (same step); {dt:.1f} s",
        "seconds": round(dt, 2),
        "leg_ms": {k: round(v * 1e3, 1) for k, v in legs.items()},
        "oracle_bias_over_unmasked": round(legs["bias_fp32"] / legs["unmasked"], 3),
        "oracle_split_over_single_bias": round(split / legs["bias_fp32"], 3),
    }
    if gpu_ms:
        out["gpu_bias_over_unmasked"] = round(gpu_ms["bias_fp32"] / gpu_ms["unmasked"], 3)
        out["gpu_split_over_single_bias"] = round((gpu_ms["core"] + gpu_ms["skirt"] + gpu_ms["merge"])
                                                  / gpu_ms["bias_fp32"], 3)
    try:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-c", _C1_SINGLE % ROOT], env=env, capture_output=True, text=True,
                           timeout=120)
        c1 = json.loads(r.stdout.strip().splitlines()[-1])["seconds"]
        out["tiny_single_thread"] = {"config": "B1 H2 S256 D128 bf16, K centred: quantize + attention, best of 3",
                                     "ms": round(c1 * 1e3, 2), "threads": 1}
    except (subprocess.SubprocessError, ValueError, IndexError) as e:
        out["tiny_single_thread"] = {"error": str(e)[:200]}
    return out


if __name__ == "__main__":
    sys.exit(main())
