"""Throughput of the k-bit codec hot path on one MI355X.

One step = blockwise quantize (bf16 -> NF4 bit planes + fp32 absmax,
blocksize 64) followed by the nested 4-bit dequantize of those planes back to
bf16 (per-block scales rebuilt from 8-bit codes over groups of 256 plus a
mean offset), on an 8192 x 8192 weight drawn from N(0, 0.02).  Inputs live in
HBM before timing starts.  Several buffer sets are rotated so that the
256 MB last-level cache cannot hold a step's working set.

Prints one JSON line.  ``value`` is the step's algorithmic bytes (read +
written by both kernels) divided by the measured time per step, in GB/s.
Per-kernel throughput comes from HIP events around each launch on the
stream the kernels run on.  ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload (rank 0, N = 1 only).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--sets 4]
                    [--no-cpu-baseline] [--copy-calibration]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "quantize & nested-dequantize GB/s and % of HBM peak, 8192x8192 bf16 blk64"
HBM_PEAK_GBPS = 8000.0
ROWS = COLS = 8192
BLOCK = 64
K = 4
GROUP2 = 256


def algorithmic_bytes(n):
    """Bytes each kernel must move at minimum (read + write)."""
    nb = -(-n // BLOCK)
    ng32 = -(-n // 32)
    quant = 2 * n + 4 * ng32 * K + 4 * nb
    nested = 4 * ng32 * K + nb + 4 * (-(-nb // GROUP2)) + 2 * n + 4 * 256 + 4 * 16
    return quant, nested


def parse(argv=None):
    ap = argparse.ArgumentParser(description="k-bit codec hot-path throughput (one GPU)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotated input/output buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 256 MiB device copies (to scale HBM byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-dispatch HBM bytes measured with rocprofv3 counters, if present")
    return ap.parse_args(argv)


def cpu_baseline(seconds_target):
    """Time the CPU oracle on a bounded sample of the same workload."""
    from blockwise_bit_codebook_amd import synth
    from oracle import codebooks, kbit, nested, numerics

    cb = codebooks.nf(K)
    q = codebooks.dynamic_map8()
    chunk_rows = 128                                  # 1 Mi elements per chunk
    x_all = synth.weight(ROWS, COLS, "bf16", seed=synth.SEED_WEIGHT_SHAPES)
    t0 = time.perf_counter()
    done = 0
    while True:
        r0 = (done // COLS) % ROWS
        x = x_all[r0 * COLS:(r0 + chunk_rows) * COLS]
        x32 = numerics.widen(x, "bf16")
        idx, a = kbit.quantize(x32, cb, BLOCK)
        words = kbit.pack(idx, K)
        code, a2, off = nested.encode(a, q)
        _ = nested.dequantize_packed(words, code, a2, off, q, cb, x.size, BLOCK, "bf16")
        done += x.size
        el = time.perf_counter() - t0
        if el >= seconds_target:
            break
    qb, nb = algorithmic_bytes(done)
    return {
        "value": round((qb + nb) / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} elements ({done // COLS} rows of the 8192x8192 bf16 weight) in 1 Mi-element chunks: "
                  f"quantize + pack + nested encode + nested dequantize, numpy float32, one thread; {el:.1f} s",
        "elements_per_s": round(done / el, 1),
    }


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the hot path has no "
              "cross-GPU step to measure here.", file=sys.stderr)
        return 2

    import torch
    import blockwise_bit_codebook_amd as kb
    from blockwise_bit_codebook_amd import synth

    dev = torch.device("cuda:0")
    n = ROWS * COLS
    nb = -(-n // BLOCK)
    cb = torch.from_numpy(kb.codebook_nf(K)).to(dev)
    qmap = torch.from_numpy(kb.dynamic_map8()).to(dev)

    x = synth.weight(ROWS, COLS, "bf16", seed=synth.SEED_WEIGHT_SHAPES)
    x_dev = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    code_np, a2_np, offset = synth.nested_state_synthetic(nb, seed=3)
    sets = []
    for i in range(args.sets):
        A = x_dev if i == 0 else x_dev.clone()
        sets.append({
            "A": A,
            "packed": torch.empty(kb.n_words(n, K), dtype=torch.int32, device=dev),
            "absmax": torch.empty(nb, dtype=torch.float32, device=dev),
            "code": torch.from_numpy(code_np).to(dev),
            "absmax2": torch.from_numpy(a2_np).to(dev),
            "out": torch.empty(n, dtype=torch.bfloat16, device=dev),
        })
    torch.cuda.synchronize()

    def step(s, ev=None):
        if ev is not None:
            ev[0].record()
        kb.quantize_kbit(s["A"], cb, K, BLOCK, absmax=s["absmax"], packed=s["packed"])
        if ev is not None:
            ev[1].record()
        kb.dequantize_4bit_nested(s["packed"], cb, s["code"], qmap, s["absmax2"], offset, n,
                                  torch.bfloat16, BLOCK, out=s["out"])
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(sets[i % args.sets])
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % args.sets], evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    tq = [e[0].elapsed_time(e[1]) for e in evs]      # ms
    tn = [e[1].elapsed_time(e[2]) for e in evs]
    qbytes, nbytes = algorithmic_bytes(n)
    ms_step = wall * 1e3 / args.steps
    value = (qbytes + nbytes) / (ms_step * 1e-3) / 1e9

    def kstats(ts, nbytes_):
        ts = np.array(ts)
        avg = float(ts.mean())
        gbps = nbytes_ / (avg * 1e-3) / 1e9
        return {"avg_us": round(avg * 1e3, 3), "median_us": round(float(np.median(ts)) * 1e3, 3),
                "p10_us": round(float(np.percentile(ts, 10)) * 1e3, 3),
                "p90_us": round(float(np.percentile(ts, 90)) * 1e3, 3),
                "bytes": nbytes_, "GB/s": round(gbps, 2), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "elements_per_s": round(n / (avg * 1e-3), 1)}

    kq, kn = kstats(tq, qbytes), kstats(tn, nbytes)
    dom_name, dom = ("quantize_kbit_bf16_k4", kq) if kq["avg_us"] >= kn["avg_us"] else \
        ("dequantize_4bit_nested_bf16", kn)
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                traffic = json.load(f).get(dom_name)
        except (OSError, ValueError):
            traffic = None
    roofline = {"kernel": dom_name, "bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dom["frac_of_hbm_peak"], "traffic": traffic}

    if args.copy_calibration:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "quantize then nested-dequantize an 8192x8192 bf16 N(0,0.02) weight, "
                               "NF4 (K=4) bit planes, blocksize 64, nested groups of 256",
                   "shape": [ROWS, COLS], "blocksize": BLOCK, "K": K, "codebook": "NF4 (exact zero)",
                   "buffer_sets": args.sets, "step_bytes": qbytes + nbytes},
        "quantize": kq,
        "nested_dequantize": kn,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
