"""Benchmark: quantized-KV decode attention on one MI355X.

One step is the decode hot path for one batch: rotate-quantize-append one new
token per sequence (with tail graduation), then single-query decode attention
over the whole cache, as one kvq_decode_step call (two launches: the split
kernel, which also appends the token, and the combine).  Default workload
"long": batch 8, 40 query / 8 KV heads, head_dim 128, 65536 cached tokens,
K 8-bit / V 4-bit 32-element blocks with fp16 scales, newest 1024 tokens in a
bf16 tail, Hadamard-128 rotation.

Prints one JSON line.  `value` is cache GB/s over the full step (algorithmic
cache bytes read by the attention / step time, over the timed steps).
`roofline` reports the split-K attention kernel alone, timed with HIP events
that the library records on the call's stream around that kernel during a
second run of as many steps (the event records stay out of the timed loop).
`cpu_baseline` times the CPU oracle's decode attention on (sequence, KV head)
units of the same cache, by wall time in a process pool.  Also reported:
`configs` (the tiny, small, mid and huge decode workloads, each with an oracle
baseline), `append` (bulk append of the mid workload), `prefill` (chunked
prefill at 64k) and `secondary` (kernel percentiles, the step as two calls,
rotation off, a paged cache, outlier channels).

  python bench.py [--steps K] [--warmup W] [--workload long] [--no-cpu-baseline]
                  [--no-append] [--no-prefill] [--no-other-configs] [--no-rotation-off]
                  [--no-unfused] [--no-paged] [--no-outliers]
  python bench.py --read-ceiling | --prefill-only | --append-only
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_long_traffic.json")
KERNEL_SOURCES = ("common.hpp", "kernels.hpp", "decode_kernels.hpp", "decode_inst.hip")


def kernel_source_hash():
    """sha256 over the sources the split-K decode kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_rotate_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the split-K kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, scaled by the plain-copy calibration;
    None when that summary was taken on other sources or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return int(t["hbm_bytes_per_launch"])
FILL_CHUNK = 8192


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Seconds of untimed work before a measurement: the part runs its first
# tens of milliseconds under load below its sustained clock.
SETTLE_S = 0.3


def settle(torch, fn):
    """Call fn (device work that leaves its outputs as they were) until
    SETTLE_S seconds have passed."""
    until = time.perf_counter() + SETTLE_S
    while SETTLE_S > 0 and time.perf_counter() < until:
        fn()
        torch.cuda.synchronize()


def cache_bytes_per_step(w, lens):
    """Algorithmic bytes one attention call reads: packed codes + fp16 scales
    (scale-and-min blocks: fp16 pairs) of quantized tokens, bf16 K and V rows
    of tail tokens."""
    d, T = w["d"], w["tail"]
    nb = d // 32
    scale_bytes = 2 * nb * ((2 if w.get("km") else 1) + (2 if w.get("vm") else 1))
    if w.get("outliers"):
        # outlier channels: 32 8-bit codes and one fp16 scale each for K and V
        scale_bytes += 2 * (w["outliers"] + 2)
    tot = 0
    for n in lens:
        nt = min(n, T) if T > 0 else 0
        nq = n - nt
        q_bytes = nq * (d * w["k_bits"] // 8 + d * w["v_bits"] // 8 + scale_bytes)
        tot += (q_bytes + nt * 2 * d * 2) * w["Hkv"]
    return tot


def describe(w):
    # K8 V4: absmax blocks of those widths; "_1" marks scale-and-min blocks
    fk = "%d%s" % (w["k_bits"], "_1" if w.get("km") else "")
    fv = "%d%s" % (w["v_bits"], "_1" if w.get("vm") else "")
    extra = (", %d outlier channels at 8 bits" % w["outliers"]) if w.get("outliers") else ""
    return ("%s: batch %d, %d query / %d KV heads, head_dim %d, context %d, K%s V%s, "
            "bf16 tail %d, %s inputs%s" % (w["name"], w["B"], w["Hq"], w["Hkv"], w["d"], w["n"],
                                          fk, fv, w["tail"], w["dist"], extra))


# ----------------------------------------------------------- CPU baseline
def _oracle_unit(args):
    """Time the oracle's decode attention for one (sequence, KV head) unit
    whose cache the oracle builds itself from the same generator inputs.
    Returns the wall-clock start and end of the timed attention."""
    os.environ["OMP_NUM_THREADS"] = "1"
    k, v, q, w = args
    from oracle import OracleCache, decode_reference
    from oracle.blockquant import bf16_bits_to_f32
    n, d = k.shape[0], w["d"]
    km, vm = bool(w.get("km")), bool(w.get("vm"))
    dtype = "bf16" if k.dtype == np.uint16 else "f32"   # bf16 bit patterns or float32 values
    qv = bf16_bits_to_f32(q) if dtype == "bf16" else q
    c = OracleCache(1, 1, d, w["k_bits"], w["v_bits"], w["tail"], n, k_min=km, v_min=vm)
    c.append(k[None, :, None], v[None, :, None], [0], dtype=dtype)
    planes = c.physical()
    t0 = time.time()
    decode_reference(planes, qv[None], [n], 1, d, w["k_bits"], w["v_bits"],
                     w["tail"], k_min=km, v_min=vm)
    return t0, time.time()


def _oracle_append_unit(args):
    """Time the oracle's rotate-quantize-append of one (sequence, KV head)
    unit's tokens in one call.  Returns the wall-clock start and end."""
    os.environ["OMP_NUM_THREADS"] = "1"
    k, v, w = args
    from oracle import OracleCache
    n = k.shape[0]
    c = OracleCache(1, 1, w["d"], w["k_bits"], w["v_bits"], w["tail"], n)
    t0 = time.time()
    c.append(k[None, :, None], v[None, :, None], [0], dtype="bf16")
    return t0, time.time()


# Worker processes of the oracle baseline: the host cores a one-GPU share of
# the box gives (16), or fewer where the affinity set is smaller.
CPU_WORKERS = 16


def cpu_baseline(w, units, k_dev, v_dev, q_host, torch, scaled=False):
    """Oracle decode attention over `units`, one (sequence, KV head) unit per
    task in a process pool.  The rate is the units' algorithmic cache bytes
    over the wall time of the timed attention work (first start to last end
    across workers; building each unit's oracle cache is not timed).  scaled:
    the units are a sample of the workload, and the rate stands for it."""
    import multiprocessing as mp
    cores = min(len(os.sched_getaffinity(0)), CPU_WORKERS)
    G = w["Hq"] // w["Hkv"]
    jobs = []
    for b, g in units:
        jobs.append((host_values(k_dev[b, :, g], torch), host_values(v_dev[b, :, g], torch),
                     q_host[b, g * G:(g + 1) * G], w))
    ctx = mp.get_context("spawn")
    par = min(cores, len(jobs))
    with ctx.Pool(par) as pool:
        res = pool.map(_oracle_unit, jobs)
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    busy = sum(r[1] - r[0] for r in res)
    unit_bytes = cache_bytes_per_step(dict(w, B=1, Hkv=1), [w["n"]])
    gbs = len(jobs) * unit_bytes / wall / 1e9
    total = w["B"] * w["Hkv"]
    what = ("%d of %d (sequence, KV head) units at full context %d%s" %
            (len(jobs), total, w["n"], ", a seeded sample whose rate stands for the workload"
             if scaled or len(jobs) < total else ""))
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": par, "kind": "oracle",
            "sample": "%s; float64 attention over the oracle-built cache, %.1f s wall for the timed "
                      "attention (%.1f s of CPU time over %d processes, %.3g s per unit on one core)"
                      % (what, wall, busy, par, busy / len(jobs))}


def host_values(t, torch):
    """A device tensor of inputs as the oracle takes them: bf16 bit patterns
    (uint16) or float32 values."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.float().cpu().numpy()


def unit_sample(w, count, seed=0):
    """(sequence, KV head) units the oracle baseline times: all of them, or
    a seeded sample of `count`."""
    all_units = [(b, g) for b in range(w["B"]) for g in range(w["Hkv"])]
    if count >= len(all_units):
        return all_units
    pick = np.random.default_rng(seed).choice(len(all_units), count, replace=False)
    return [all_units[i] for i in sorted(pick)]


# ------------------------------------------------------------------ main
def main():
    global SETTLE_S
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed calls before each measurement (0 for profiling runs "
                         "that count dispatches)")
    ap.add_argument("--cpu-units", type=int, default=64,
                    help="(sequence, KV head) units the CPU oracle times (all when >= batch * KV heads)")
    ap.add_argument("--no-append", action="store_true", help="skip the bulk append measurement")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the sub-results of the tiny, small, mid and huge decode workloads")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the secondary run with the append and the attention as two calls")
    ap.add_argument("--no-rotation-off", action="store_true",
                    help="skip the secondary run with rotation disabled")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-outliers", action="store_true",
                    help="skip the secondary runs with and without outlier channels (no tail)")
    ap.add_argument("--paged", action="store_true",
                    help="run the main measurement on a paged cache (64-position pages in a "
                         "shuffled order) instead of the contiguous layout")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the secondary run on a paged cache")
    ap.add_argument("--k-bits", type=int, default=0, help="override the workload's K code width")
    ap.add_argument("--v-bits", type=int, default=0, help="override the workload's V code width")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="override the workload's head_dim (64, 128, 192 or 256)")
    ap.add_argument("--k-min", action="store_true",
                    help="K in scale-and-min blocks (q4_1 / q5_1; with a 4- or 5-bit K width)")
    ap.add_argument("--v-min", action="store_true", help="V in scale-and-min blocks")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the chunked-prefill measurement (for profiling) and exit")
    ap.add_argument("--append-only", action="store_true",
                    help="only run the bulk append measurement (for profiling) and exit")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the part's read bandwidth (a linear stream, and the "
                         "split kernel's tile pattern without its arithmetic) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (a known-size "
                         "reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    SETTLE_S = args.settle_s

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library runs the decode hot path on a single "
              "device (no collectives); run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import decode_attention_rotate_amd as kvq

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return 0

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.read_ceiling:
        print(json.dumps(read_ceiling(torch, kvq, dev)), flush=True)
        return 0
    if args.prefill_only:
        print(json.dumps(prefill_bench(torch, kvq, dev)), flush=True)
        return 0
    if args.append_only:
        print(json.dumps(bulk_append(torch, kvq, dev)), flush=True)
        return 0
    w = workloads.workload(args.workload)
    if args.k_bits:
        w["k_bits"] = args.k_bits
    if args.v_bits:
        w["v_bits"] = args.v_bits
    w["km"], w["vm"] = args.k_min, args.v_min
    if args.head_dim:
        w["d"] = args.head_dim
    B, Hq, Hkv, d, n = w["B"], w["Hq"], w["Hkv"], w["d"], w["n"]
    log("workload", describe(w))

    # (sequence, KV head) units whose inputs the CPU oracle gets
    units = unit_sample(w, args.cpu_units)
    keep = None if args.no_cpu_baseline else {}

    run = decode_run(torch, kvq, w, dev, args.warmup, args.steps, True, keep, paged=args.paged)
    ms_step = run["ms_step"]
    value = run["bytes_step"] / (ms_step * 1e-3) / 1e9
    kern_ms = run["kern_ms"]
    kern_avg_ms = float(np.mean(kern_ms))
    achieved = run["bytes_kern"] / (kern_avg_ms * 1e-3) / 1e9
    log("step %.1f us, attention kernel %.1f us (median %.1f), %.0f GB/s kernel, %.0f GB/s step"
        % (ms_step * 1e3, kern_avg_ms * 1e3, float(np.median(kern_ms)) * 1e3, achieved, value))

    result = {
        "metric": "Quantized-KV decode attention cache GB/s (decode step: append 1 token + attention)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/u4 codes, fp16 scales, f32 accumulation",
        "data": "synthetic",
        "config": {"workload": describe(w) + (", paged cache" if args.paged else ""),
                   "cache_bytes_per_step": int(run["bytes_step"]),
                   "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
                   "us_per_step": round(ms_step * 1e3, 2),
                   "attention_kernel_us": round(kern_avg_ms * 1e3, 2),
                   "fill_append_mtok_s": round(run["fill_mtok_s"], 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if args.paged else measured_traffic(args.workload)},
        "secondary": {"attention_kernel_us": percentiles(kern_ms)},
    }
    q0 = run["q0"]
    del run

    if not args.no_unfused:
        # the same step as two calls: kvq_rotate_quantize_append, then
        # kvq_decode_attention (three launches instead of two)
        uf = decode_run(torch, kvq, w, dev, args.warmup, args.steps, True, None, paged=args.paged,
                        fused=False)
        result["secondary"]["unfused_step"] = {
            "us_per_step": round(uf["ms_step"] * 1e3, 2),
            "attention_kernel_us": percentiles(uf["kern_ms"]),
            "single_token_append_us": percentiles(uf["app_ms"])}
        log("append + attention as two calls: step %.1f us" % (uf["ms_step"] * 1e3))
        del uf

    if not args.no_rotation_off:
        # the same step with rotation disabled for K and V (no query rotation,
        # no inverse rotation of the output, no rotation in the append)
        off = decode_run(torch, kvq, w, dev, args.warmup, args.steps, False, None)
        result["secondary"]["rotation_off"] = {
            "us_per_step": round(off["ms_step"] * 1e3, 2),
            "attention_kernel_us": percentiles(off["kern_ms"]),
            "step_slowdown_of_rotation_pct": round(100 * (ms_step / off["ms_step"] - 1), 2)}
        log("rotation off: step %.1f us" % (off["ms_step"] * 1e3))
        del off

    if not args.no_paged and not args.paged:
        # the same step on a paged cache: 64-position pages of a shared pool,
        # assigned in a shuffled order through the page table
        pg = decode_run(torch, kvq, w, dev, args.warmup, args.steps, True, None, paged=True)
        pg_kern = float(np.mean(pg["kern_ms"]))
        result["secondary"]["paged"] = {
            "us_per_step": round(pg["ms_step"] * 1e3, 2),
            "attention_kernel_us": percentiles(pg["kern_ms"]),
            "attention_kernel_gbs": round(pg["bytes_kern"] / (pg_kern * 1e-3) / 1e9, 1)}
        log("paged: step %.1f us, kernel %.1f us" % (pg["ms_step"] * 1e3, pg_kern * 1e3))
        del pg


    if not args.no_outliers:
        # outlier channels (32 per plane and KV head at 8 bits, the rest
        # rotated and quantized) need a cache without a bf16 tail: the long
        # workload with no tail, with and without them
        res_o = {}
        for key, extra in (("no_tail", {}), ("outliers", {"outliers": 32})):
            wo = dict(w, tail=0, **extra)
            r = decode_run(torch, kvq, wo, dev, args.warmup, args.steps, True, None)
            kern = float(np.mean(r["kern_ms"]))
            res_o[key] = {"workload": describe(wo), "us_per_step": round(r["ms_step"] * 1e3, 2),
                          "step_gbs": round(r["bytes_step"] / (r["ms_step"] * 1e-3) / 1e9, 1),
                          "attention_kernel_us": percentiles(r["kern_ms"]),
                          "kernel_gbs": round(r["bytes_kern"] / (kern * 1e-3) / 1e9, 1)}
            log("%s: step %.1f us, kernel %.1f us" % (key, r["ms_step"] * 1e3, kern * 1e3))
            del r
        res_o["kernel_cost_of_outliers_pct"] = round(
            100 * (res_o["outliers"]["attention_kernel_us"]["median"]
                   / res_o["no_tail"]["attention_kernel_us"]["median"] - 1), 2)
        result["secondary"]["outlier_channels"] = res_o

    if not args.no_other_configs:
        # the other decode workloads, each with its own oracle baseline
        result["configs"] = {}
        for name, cpu_units in OTHER_CONFIGS:
            result["configs"][name] = other_config(torch, kvq, dev, name, cpu_units, args.steps,
                                                   args.warmup, not args.no_cpu_baseline)

    if not args.no_append:
        result["append"] = bulk_append(torch, kvq, dev, not args.no_cpu_baseline)
    if not args.no_prefill:
        result["prefill"] = prefill_bench(torch, kvq, dev)

    if not args.no_cpu_baseline:
        q_host = host_values(q0, torch)
        log("cpu baseline on %d units" % len(units))
        result["cpu_baseline"] = cpu_baseline(w, units, keep["k"], keep["v"], q_host, torch)
    print(json.dumps(result), flush=True)
    return 0


# Other decode workloads reported beside the main one, with the number of
# (sequence, KV head) units their oracle baseline times (mid: 32 of 128 and
# huge: 16 of 128 are seeded samples; tiny: its one unit, small: all 8).
OTHER_CONFIGS = (("tiny", 1), ("small", 8), ("mid", 32), ("huge", 16))


def other_config(torch, kvq, dev, name, cpu_units, steps, warmup, with_cpu):
    """The decode step (kvq_decode_step) of one more workload: step and split
    kernel rates, and the oracle's rate on a sample of its units."""
    w = workloads.workload(name)
    keep = {} if with_cpu else None
    run = decode_run(torch, kvq, w, dev, warmup, steps, True, keep)
    kern = float(np.mean(run["kern_ms"]))
    kgbs = run["bytes_kern"] / (kern * 1e-3) / 1e9
    sgbs = run["bytes_step"] / (run["ms_step"] * 1e-3) / 1e9
    res = {"workload": describe(w), "cache_bytes_per_step": int(run["bytes_step"]),
           "us_per_step": round(run["ms_step"] * 1e3, 2), "step_gbs": round(sgbs, 1),
           "attention_kernel_us": percentiles(run["kern_ms"]), "kernel_gbs": round(kgbs, 1),
           "pct_hbm_peak_kernel": round(100 * kgbs / HBM_PEAK_GBS, 2)}
    if run["bytes_step"] < 256e6:
        res["note"] = ("the cache fits the part's 256 MB last-level cache, so this rate is not an "
                       "HBM rate")
    log("%s: step %.1f us, kernel %.1f us, %.0f GB/s kernel" % (name, run["ms_step"] * 1e3,
                                                              kern * 1e3, kgbs))
    if with_cpu:
        q_host = host_values(run["q0"], torch)
        units = unit_sample(w, cpu_units)
        log("%s: cpu baseline on %d units" % (name, len(units)))
        res["cpu_baseline"] = cpu_baseline(w, units, keep["k"], keep["v"], q_host, torch)
    del run, keep
    return res


def percentiles(ms):
    """p10 / median / p90 of a list of durations in ms, in us."""
    p = np.percentile(np.asarray(ms) * 1e3, [10, 50, 90])
    return {"p10": round(float(p[0]), 2), "median": round(float(p[1]), 2),
            "p90": round(float(p[2]), 2)}


def decode_run(torch, kvq, w, dev, warmup, steps, rotate, keep, paged=False, fused=True):
    """Fill a cache for workload w, then run warm-up steps, `steps` timed
    steps, and as many steps again with HIP events around the split kernel
    (recorded by the library on the call's stream) and around the append
    (kept out of the timed loop: event records sit between kernels).  When
    `keep` is a dict it receives the bf16 K and V inputs for the oracle.
    paged: the cache is a pool of 64-position pages, every tile of every
    sequence on a page drawn from a seeded shuffle of the pool."""
    B, Hq, Hkv, d, n = w["B"], w["Hq"], w["Hkv"], w["d"], w["n"]
    total_steps = warmup + 2 * steps
    max_ctx = n + total_steps + 64
    table = None
    pool = 0
    if paged:
        tiles = (max_ctx + kvq.KVQ_PAGE_TOKENS - 1) // kvq.KVQ_PAGE_TOKENS
        pool = B * tiles
        perm = np.random.default_rng(12345).permutation(pool).astype(np.int32)
        table = torch.from_numpy(perm.reshape(B, tiles)).to(dev)
    outl = int(w.get("outliers", 0))
    cfg = kvq.kvq_config(B, Hkv, d, max_ctx, w["k_bits"], w["v_bits"], w["tail"],
                         rotate_k=rotate, rotate_v=rotate, k_min=w.get("km", False),
                         v_min=w.get("vm", False), page_pool=pool, outliers=outl)
    idx = torch.from_numpy(workloads.outlier_lists(w)).to(dev) if outl else None
    cache = kvq.KVCache(cfg, dev, page_table=table, outlier_idx=idx)
    if keep is not None:
        keep["k"] = torch.empty((B, n, Hkv, d), dtype=torch.bfloat16 if w["dtype"] == "bf16" else torch.float32,
                                device=dev)
        keep["v"] = torch.empty_like(keep["k"])
    lens = [0] * B
    t_fill = 0.0
    for t0 in range(0, n, FILL_CHUNK):
        t1 = min(n, t0 + FILL_CHUNK)
        k = workloads.kv_torch(w, 1, t0, t1, dev, torch)
        v = workloads.kv_torch(w, 2, t0, t1, dev, torch)
        if keep is not None:
            keep["k"][:, t0:t1].copy_(k)
            keep["v"][:, t0:t1].copy_(v)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.kvq_rotate_quantize_append(cfg, cache, k, v, lens)
        e1.record()
        torch.cuda.synchronize()
        t_fill += e0.elapsed_time(e1) * 1e-3
        lens = [x + (t1 - t0) for x in lens]
        del k, v
    fill_mtok_s = n * B / t_fill / 1e6
    log("filled %d tokens/sequence (rotation %s), append %.1f Mtok/s"
        % (n, "on" if rotate else "off", fill_mtok_s))

    # inputs of every step, generated before timing
    qs = [workloads.q_torch(w, s, dev, torch) for s in range(total_steps)]
    ks = [workloads.new_tokens_torch(w, 1, s, dev, torch) for s in range(total_steps)]
    vs = [workloads.new_tokens_torch(w, 2, s, dev, torch) for s in range(total_steps)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(cfg, Hq), dtype=torch.uint8, device=dev)

    def new_events():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [new_events() for _ in range(total_steps)]
    ev_app = [new_events() for _ in range(total_steps)]

    def step(s, events):
        if fused:
            # one call: append the token and attend (kvq_decode_step)
            if events:
                kvq.kvq_profile_decode_events(ev[s][0], ev[s][1])
            kvq.kvq_decode_step(cfg, cache, ks[s], vs[s], qs[s], lens, out=out, workspace=ws)
            for b in range(B):
                lens[b] += 1
            return
        if events:
            ev_app[s][0].record()
        kvq.kvq_rotate_quantize_append(cfg, cache, ks[s], vs[s], lens)
        if events:
            ev_app[s][1].record()
        for b in range(B):
            lens[b] += 1
        if events:
            kvq.kvq_profile_decode_events(ev[s][0], ev[s][1])
        kvq.kvq_decode_attention(cfg, cache, qs[s], lens, out=out, workspace=ws)

    # Clock settling (a 50-step loop measured 168 us per step right after 10
    # warm-up steps, and 148-154 us per step in the loops that followed it):
    # attention calls on the filled cache, which they leave unchanged.
    settle(torch, lambda: [kvq.kvq_decode_attention(cfg, cache, qs[0], lens, out=out, workspace=ws)
                           for _ in range(8)])
    step_bytes = []
    for s in range(warmup):
        step(s, False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(warmup, warmup + steps):
        step(s, False)
        step_bytes.append(cache_bytes_per_step(w, lens))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kern_bytes = []
    for s in range(warmup + steps, total_steps):
        step(s, True)
        kern_bytes.append(cache_bytes_per_step(w, lens))
    torch.cuda.synchronize()
    kvq.kvq_profile_decode_events(None, None)
    assert torch.isfinite(out).all().item(), "non-finite attention output"
    timed = range(warmup + steps, total_steps)
    res = {"ms_step": elapsed / steps * 1e3, "bytes_step": float(np.mean(step_bytes)),
           "bytes_kern": float(np.mean(kern_bytes)),
           "kern_ms": [kvq.kernel_elapsed_ms(ev[s][0], ev[s][1]) for s in timed],
           "app_ms": [] if fused else [ev_app[s][0].elapsed_time(ev_app[s][1]) for s in timed],
           "fill_mtok_s": fill_mtok_s, "q0": qs[0]}
    del cache, qs, ks, vs
    return res


def read_ceiling(torch, kvq, dev, reps=10):
    """Read bandwidth the part reaches without the decode arithmetic:
    * a linear read of a buffer the size of the 64k workload's cache, over
      workgroup counts, loads in flight per lane and non-temporal loads;
    * the split kernel's access pattern on planes of the 64k workload's
      geometry (64 units of 1024 tiles: 8 KiB of K codes, 4 KiB of V codes
      and 512 B per scale plane per tile), over splits per unit, tiles of
      loads in flight per wave, non-temporal loads, and contiguous ranges
      per workgroup against chunks of 8 tiles dealt round-robin.
    Each configuration runs `reps` times after one warm-up (the sweep after
    SETTLE_S seconds of the first stream configuration); medians by HIP
    events on the call's stream."""
    from decode_attention_rotate_amd import _capi
    import ctypes
    C = _capi.ceiling_lib()
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    w = workloads.workload("long")
    cache_bytes = cache_bytes_per_step(w, [w["n"]] * w["B"])
    nbytes = cache_bytes // 4096 * 4096
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    stream_rows = []
    # clock settling: the first configuration, repeated
    sink0 = torch.empty(C.kvq_ceiling_sink_words(512, 1), dtype=torch.int32, device=dev)
    settle(torch, lambda: C.kvq_ceiling_stream(buf.data_ptr(), nbytes, 512, 4, 1, sink0.data_ptr(), stream))
    del sink0
    for blocks in (512, 1024, 2048, 4096, 8192):
        sink = torch.empty(C.kvq_ceiling_sink_words(blocks, 1), dtype=torch.int32, device=dev)
        for unroll in (4, 8, 16):
            for nt in (0, 1):
                def run():
                    st = C.kvq_ceiling_stream(buf.data_ptr(), nbytes, blocks, unroll, nt,
                                              sink.data_ptr(), stream)
                    assert st == 0, st
                ms = timed(run)
                stream_rows.append({"blocks": blocks, "unroll": unroll, "nontemporal": nt,
                                    "us": round(ms * 1e3, 1),
                                    "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del sink
    del buf
    units, tiles = w["B"] * w["Hkv"], w["n"] // 64
    kt, vt, st_b = 64 * 128, 64 * 64, 64 * 4 * 2
    planes = [torch.ones(units * tiles * b // 4, dtype=torch.int32, device=dev) for b in (kt, vt, st_b, st_b)]
    args = _capi.KvqCeilingTilesArgs(planes[0].data_ptr(), planes[1].data_ptr(), planes[2].data_ptr(),
                                     planes[3].data_ptr(), units, tiles, kt, vt, st_b)
    tile_bytes = units * tiles * (kt + vt + 2 * st_b)
    tile_rows = []
    for splits in (2, 4, 8, 16):
        sink = torch.empty(C.kvq_ceiling_sink_words(splits, units), dtype=torch.int32, device=dev)
        for ahead in (1, 2):
            for mode in (0, 1, 2, 3):
                def run():
                    st = C.kvq_ceiling_tiles(ctypes.byref(args), splits, ahead, mode, sink.data_ptr(),
                                             stream)
                    assert st == 0, st
                ms = timed(run)
                tile_rows.append({"workgroups_per_unit": splits, "waves": splits * 8 * units,
                                  "tiles_ahead": ahead, "nontemporal": mode & 1,
                                  "chunked": (mode >> 1) & 1, "us": round(ms * 1e3, 1),
                                  "gbs": round(tile_bytes / (ms * 1e-3) / 1e9, 1)})
        del sink
    del planes
    best_s = max(stream_rows, key=lambda r: r["gbs"])
    best_t = max(tile_rows, key=lambda r: r["gbs"])
    res = {"read_ceiling": {
        "stream_bytes": nbytes, "tile_pattern_bytes": tile_bytes,
        "best_stream_gbs": best_s["gbs"], "best_stream": best_s,
        "best_tile_pattern_gbs": best_t["gbs"], "best_tile_pattern": best_t,
        "pct_of_8000": {"stream": round(100 * best_s["gbs"] / HBM_PEAK_GBS, 1),
                        "tile_pattern": round(100 * best_t["gbs"] / HBM_PEAK_GBS, 1)},
        "stream": stream_rows, "tile_pattern": tile_rows}}
    log("read ceiling: stream %.0f GB/s (%s), tile pattern %.0f GB/s (%s)"
        % (best_s["gbs"], best_s, best_t["gbs"], best_t))
    return res


MFMA_F16_PEAK_TFLOPS = 2500.0


def prefill_bench(torch, kvq, dev, n_q=512):
    """Chunked prefill at the long workload's shape with batch 1: append a
    chunk of n_q tokens after 65536 - n_q cached ones, then attend its n_q
    queries causally over the cache.  Algorithmic work: 4 * d flops per
    (query head, visible position) pair (Q.K and P.V multiply-adds)."""
    w = workloads.workload("long", B=1)
    B, Hq, Hkv, d, n = w["B"], w["Hq"], w["Hkv"], w["d"], w["n"]
    n0 = n - n_q
    cfg = kvq.kvq_config(B, Hkv, d, n, w["k_bits"], w["v_bits"], w["tail"])
    cache = kvq.KVCache(cfg, dev)
    for t0 in range(0, n0, FILL_CHUNK):
        t1 = min(n0, t0 + FILL_CHUNK)
        kvq.kvq_rotate_quantize_append(cfg, cache, workloads.kv_torch(w, 1, t0, t1, dev, torch),
                                       workloads.kv_torch(w, 2, t0, t1, dev, torch), [t0])
    k = workloads.kv_torch(w, 1, n0, n, dev, torch)
    v = workloads.kv_torch(w, 2, n0, n, dev, torch)
    q = workloads.prefill_q_torch(w, n_q, 0, dev, torch)
    out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_prefill_workspace_bytes(cfg, Hq, n_q), dtype=torch.uint8, device=dev)
    kvq.kvq_rotate_quantize_append(cfg, cache, k, v, [n0])
    settle(torch, lambda: kvq.kvq_prefill_attention(cfg, cache, q, [n], out=out, workspace=ws))
    reps = 5
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(3 * (reps + 1))]
    app_ms, att_ms, kern_ms = [], [], []
    for r in range(reps + 1):
        e = ev[3 * r: 3 * r + 3]
        e[0][0].record()
        kvq.kvq_rotate_quantize_append(cfg, cache, k, v, [n0])
        e[0][1].record()
        e[1][0].record()
        kvq.kvq_prefill_attention(cfg, cache, q, [n], out=out, workspace=ws)
        e[1][1].record()
        kvq.kvq_profile_decode_events(e[2][0], e[2][1])
        kvq.kvq_prefill_attention(cfg, cache, q, [n], out=out, workspace=ws)
        kvq.kvq_profile_decode_events(None, None)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item(), "non-finite prefill output"
    for r in range(1, reps + 1):
        e = ev[3 * r: 3 * r + 3]
        app_ms.append(e[0][0].elapsed_time(e[0][1]))
        att_ms.append(e[1][0].elapsed_time(e[1][1]))
        kern_ms.append(kvq.kernel_elapsed_ms(e[2][0], e[2][1]))
    visible = sum(n0 + i + 1 for i in range(n_q))
    flops = 4.0 * d * Hq * B * visible
    att = float(np.median(att_ms))
    kern = float(np.median(kern_ms))
    app = float(np.median(app_ms))
    res = {"workload": "prefill: batch 1, 40 query / 8 KV heads, head_dim 128, K8 V4, bf16 tail "
                       "1024, chunk of %d tokens appended after %d cached, causal attention of "
                       "its %d queries" % (n_q, n0, n_q),
           "append_us": round(app * 1e3, 1), "attention_us": round(att * 1e3, 1),
           "split_kernel_us": round(kern * 1e3, 1),
           "query_tokens_per_s": round(n_q * B / ((att + app) * 1e-3), 1),
           "algorithmic_tflops": round(flops / (kern * 1e-3) / 1e12, 2),
           "pct_f16_mfma_peak": round(100 * flops / (kern * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 2)}
    log("prefill", res)
    del cache, k, v, q, out, ws
    return res


def bulk_append(torch, kvq, dev, with_cpu=False, cpu_units=16):
    """Rotate-quantize-append of 32768 tokens per sequence in one call:
    batch 16, 8 KV heads, head_dim 128, K4 V4, no tail."""
    w = workloads.workload("mid")
    B, Hkv, d, n = w["B"], w["Hkv"], w["d"], w["n"]
    cfg = kvq.kvq_config(B, Hkv, d, n, w["k_bits"], w["v_bits"], 0)
    cache = kvq.KVCache(cfg, dev)
    k = workloads.kv_torch(w, 1, 0, n, dev, torch)
    v = workloads.kv_torch(w, 2, 0, n, dev, torch)
    # the same positions rewritten with the same values each call
    settle(torch, lambda: kvq.kvq_rotate_quantize_append(cfg, cache, k, v, [0] * B))
    reps = 5
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps + 1)]
    for r in range(reps + 1):
        evs[r][0].record()
        kvq.kvq_rotate_quantize_append(cfg, cache, k, v, [0] * B)
        evs[r][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([evs[r][0].elapsed_time(evs[r][1]) for r in range(1, reps + 1)]))
    tokens = B * n
    moved = 2 * B * n * Hkv * d * 2 + 2 * B * n * Hkv * (d * 4 // 8 + 2 * d // 32)
    res = {"workload": "mid append: batch 16, 8 KV heads, head_dim 128, 32768 new tokens "
                       "per sequence in one call, K4 V4",
           "us": round(ms * 1e3, 1), "mtok_s": round(tokens / (ms * 1e-3) / 1e6, 1),
           "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
           "pct_hbm_peak": round(100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    log("bulk append", res)
    if with_cpu:
        # the oracle's append of a sample of the same units, one per process
        import multiprocessing as mp
        units = unit_sample(w, cpu_units, seed=1)
        jobs = []
        for b, g in units:
            kk = k[b, :, g].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            vv = v[b, :, g].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            jobs.append((kk, vv, w))
        par = min(len(os.sched_getaffinity(0)), CPU_WORKERS, len(jobs))
        with mp.get_context("spawn").Pool(par) as pool:
            r = pool.map(_oracle_append_unit, jobs)
        wall = max(x[1] for x in r) - min(x[0] for x in r)
        # a unit is one KV head of one sequence: n tokens x 1 head of the
        # B x Hkv heads a token has, so tokens per second = n * units / Hkv
        tok = n * len(jobs) / Hkv
        res["cpu_baseline"] = {
            "value": round(tok / wall / 1e6, 4), "unit": "Mtok/s", "cores": par, "kind": "oracle",
            "sample": "%d of %d (sequence, KV head) units, %d tokens each, appended by the float32 "
                      "oracle in one call per unit; %.1f s wall (a token is %d KV heads, so the rate "
                      "counts units x tokens / %d)" % (len(jobs), B * Hkv, n, wall, Hkv, Hkv)}
    del k, v, cache
    return res


if __name__ == "__main__":
    sys.exit(main())
