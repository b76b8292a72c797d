"""Throughput of the k-bit codec hot path on one MI355X.

One step = blockwise quantize (bf16 -> NF4 bit planes + fp32 absmax,
blocksize 64) followed by the nested 4-bit dequantize of those planes back to
bf16 (per-block scales rebuilt from 8-bit codes over groups of 256 plus a
mean offset), on an 8192 x 8192 weight drawn from N(0, 0.02).  Inputs live in
HBM before timing starts.  Several buffer sets are rotated so that the
256 MB last-level cache cannot hold a step's working set.  The timed region
is exactly --steps steps (after --warmup untimed ones, which follow at least
--settle-ms of back-to-back steps), launched eagerly, with fence-free HIP
events at its two ends on the kernels' stream.

Prints one JSON line.  ``value`` is the step's algorithmic bytes (read +
written by both kernels) divided by the wall time per step, in GB/s.
Per-kernel launch durations (``quantize``, ``nested_dequantize`` and the
``roofline`` object) come from rounds of back-to-back launches of each step
kernel over the same buffer sets right after the timed steps, with an event
at each round's ends (an event after every kernel inside the timed steps
would lengthen them).  Side kernels
are timed with events around eager launches over all buffer sets, in round
robin.  The same line also reports, as side measurements, the
quantize / dequantize pair with one-byte E4M4 block scales and the plain
fp32-scale dequantize on the same tensor, the FP4 codebook, warm-cache
numbers and the W4A4 activation path (4096 x 4096 bf16).  ``cpu_baseline`` times the CPU oracle on a bounded sample of
the same workload (N = 1 only).

    python bench.py [--gpus 1] [--steps 200] [--warmup 300] [--sets 4]
                    [--no-cpu-baseline] [--copy-calibration]
    python bench.py --summarize TRACE_DIR FETCH_DIR WRITE_DIR   (no GPU)
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
KERNEL_ROUNDS_MIN = 50  # rounds of back-to-back launches per step kernel for its launch duration
ROUND_PASSES = 4        # passes over the rotated buffer sets inside one round (one event pair)


def algorithmic_bytes(n):
    """Bytes each kernel of the step must move at minimum (read + write)."""
    b = kernel_bytes(n)
    return b["quantize_kbit_bf16_k4"], b["dequantize_4bit_nested_bf16"]


def kernel_bytes(n):
    """Minimum bytes read + written per launch, by kernel: bf16 elements,
    K bit planes per 32 elements, per-block scales (4 bytes fp32, 1 byte
    E4M4 or nested code), group absmax, tables."""
    nb = -(-n // BLOCK)
    planes = 4 * (-(-n // 32)) * K
    tables = 4 * (1 << K)
    return {
        "quantize_kbit_bf16_k4": 2 * n + planes + 4 * nb + tables,
        "dequantize_4bit_nested_bf16": planes + nb + 4 * (-(-nb // GROUP2)) + 2 * n + 4 * 256 + tables,
        "quantize_kbit_e4m4_bf16_k4": 2 * n + planes + nb + tables,
        "dequantize_kbit_e4m4_bf16_k4": planes + nb + 2 * n + tables,
        "dequantize_kbit_bf16_k4": planes + 4 * nb + 2 * n + tables,
        # nested-state encoder: absmax read twice (the mean comes first),
        # codes, group absmax, offset and the map
        "quantize_nested_absmax": 8 * nb + nb + 4 * (-(-nb // GROUP2)) + 4 + 4 * 256,
        # the encoder's two launches: the absmax read for the sums (records
        # of 100 bytes per workgroup aside), then read again for the codes
        "nested_bins_kernel": 4 * nb,
        "nested_encode_kernel": 4 * nb + nb + 4 * (-(-nb // GROUP2)) + 4 + 4 * 256,
        # quantize_4bit_nested_bf16's two kernels: the quantize variant (the
        # plain kernel's bytes; its records are a few tens of KB) and the
        # encoder's second launch (absmax read once, codes, group absmax,
        # offset, map)
        "quantize_kbit_bf16_k4 (nested sums)": 2 * n + planes + 4 * nb + tables,
        "nested_encode_kernel (quantize records)": 4 * nb + nb + 4 * (-(-nb // GROUP2)) + 4 + 4 * 256,
    }


def parse(argv=None):
    ap = argparse.ArgumentParser(description="k-bit codec hot-path throughput (one GPU)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps right before the timed ones (about 18 ms at 8192^2; the GPU needs "
                         "some milliseconds of sustained load to reach its working clocks)")
    ap.add_argument("--settle-ms", type=float, default=25.0,
                    help="before each warmup, back-to-back steps for at least this long (the GPU reaches its "
                         "sustained clocks only after some milliseconds of continuous load, whatever --warmup is)")
    ap.add_argument("--sets", type=int, default=4, help="rotated input/output buffer sets")
    ap.add_argument("--rr-reps", type=int, default=0,
                    help="rounds of the per-kernel timing (default: steps / sets, at least 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-act", action="store_true", help="skip the activation-path timing")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the NF4 step and its two kernels (what the profiles cover)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle time per leg (one thread, then all cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"after timing, run {CAL_COPIES} plain device copies of {CAL_BYTES >> 20} MiB "
                         "(known bytes, to scale HBM byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-dispatch HBM bytes measured with rocprofv3 counters, if present")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarise rocprofv3 output of the profile commands into profiles/")
    ap.add_argument("--side-only", action="store_true",
                    help="run only the activation-path and fused-linear cases the side profile covers "
                         "(eager launches; prints their timings, not the bench line)")
    ap.add_argument("--side-reps", type=int, default=20, help="rounds per case with --side-only")
    ap.add_argument("--summarize-side", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarise rocprofv3 output of the side profile commands into profiles/")
    return ap.parse_args(argv)


# --------------------------------------------------------------------------
# rocprofv3 summaries (CPU only)
# --------------------------------------------------------------------------
CAL_BYTES = 192 << 20
CAL_COPIES = 3
_Q_SRC = ["blockwise_bit_codebook_amd/csrc/quantize.hip", "blockwise_bit_codebook_amd/csrc/device.h",
          "blockwise_bit_codebook_amd/csrc/threshold.h", "blockwise_bit_codebook_amd/csrc/e4m4.h",
          "blockwise_bit_codebook_amd/csrc/nested_sums.h"]
_D_SRC = ["blockwise_bit_codebook_amd/csrc/dequantize.hip", "blockwise_bit_codebook_amd/csrc/device.h",
          "blockwise_bit_codebook_amd/csrc/e4m4.h"]
_E_SRC = ["blockwise_bit_codebook_amd/csrc/nested_encode.hip", "blockwise_bit_codebook_amd/csrc/exact_mean.h",
          "blockwise_bit_codebook_amd/csrc/device.h", "blockwise_bit_codebook_amd/csrc/nested_sums.h"]
KERNELS = {
    # name used in the JSON line: (substrings that all appear in the HIP kernel's demangled name,
    # sources that define it)
    "quantize_kbit_bf16_k4": (("::quantize_kernel<kbit::Bf16,", "F32Scale, 4,", ", false>"), _Q_SRC),
    "dequantize_4bit_nested_bf16": (("::dequantize_nested_kernel<kbit::Bf16",), _D_SRC),
    "quantize_kbit_e4m4_bf16_k4": (("::quantize_kernel<kbit::Bf16,", "E4m4Scale, 4,", ", false>"), _Q_SRC),
    "dequantize_kbit_e4m4_bf16_k4": (("::dequantize_kernel<kbit::Bf16, 4,", "E4m4Scale>"), _D_SRC),
    "dequantize_kbit_bf16_k4": (("::dequantize_kernel<kbit::Bf16, 4,", "PlainScale>"), _D_SRC),
    # the nested-state encoder's two launches
    "nested_bins_kernel": (("::nested_bins_kernel",), _E_SRC),
    "nested_encode_kernel": (("::nested_encode_kernel<8, false>",), _E_SRC),
    # quantize_4bit_nested_bf16's two launches
    "quantize_kbit_bf16_k4 (nested sums)": (("::quantize_kernel<kbit::Bf16,", "F32Scale, 4,", ", true>"),
                                            _Q_SRC),
    "nested_encode_kernel (quantize records)": (("::nested_encode_kernel<8, true>",), _E_SRC),
}


def _matches(pat, name):
    return all(p in name for p in pat)
PROFILE_STEPS = 200  # --steps of the trace command below
PROFILE_SETS = 4     # its --sets (the default)
# launches of each step kernel in the rounds after its timed steps
PROFILE_ROUND_LAUNCHES = max(KERNEL_ROUNDS_MIN, PROFILE_STEPS // PROFILE_SETS) * PROFILE_SETS * ROUND_PASSES
PROFILE_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_trace -o trace -- "
    "python3 $R/bench.py --steps 200 --warmup 300 --rr-reps 5 --no-cpu-baseline --headline-only --copy-calibration",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof_fetch -o fetch -- "
    "python3 $R/bench.py --steps 8 --warmup 4 --no-cpu-baseline --headline-only --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof_write -o write -- "
    "python3 $R/bench.py --steps 8 --warmup 4 --no-cpu-baseline --headline-only --copy-calibration",
    "cd $R && python3 bench.py --summarize gpurun_out/prof_trace gpurun_out/prof_fetch gpurun_out/prof_write",
]


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def _summarize_into(table, trace_dir, fetch_dir, write_dir, header, commands, md_name, timed_last=None):
    """Per-kernel average duration (kernel trace) and HBM bytes per dispatch
    (FETCH_SIZE / WRITE_SIZE in KiB, each scaled by what the same counter
    reads for the calibration copies of known size).  table: name ->
    (substrings of the demangled kernel name, grid size in threads or None,
    sources, algorithmic bytes per launch).  The entries are merged into
    profiles/traffic.json and written as a table to profiles/<md_name>.
    timed_last: name -> number of final dispatches the bench's per-kernel times come from
    (their average is reported beside the overall one)."""
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    counters = {c: _csv_rows(d, "counter_collection.csv") for c, d in (("FETCH_SIZE", fetch_dir),
                                                                        ("WRITE_SIZE", write_dir))}

    def hit(entry, name, grid):
        pat, g = entry[0], entry[1]
        return _matches(pat, name) and (g is None or int(grid) == g)

    scale = {}
    per_kernel = {}
    for cname, rows in counters.items():
        rows = [r for r in rows if r["Counter_Name"] == cname]
        cal = sorted((r for r in rows if "copyBuffer" in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))
        cal = cal[-CAL_COPIES:]
        kib = sum(float(r["Counter_Value"]) for r in cal) / len(cal)
        scale[cname] = (CAL_BYTES / 1024.0) / kib
        for name, entry in table.items():
            vals = [float(r["Counter_Value"]) for r in rows if hit(entry, r["Kernel_Name"], r["Grid_Size"])]
            per_kernel.setdefault(name, {})[cname] = sum(vals) / len(vals) if vals else None
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    out = {"calibration": {}, "kernels": {}}
    if os.path.exists(tj):
        with open(tj) as f:
            out = json.load(f)
    cal = {"copy_bytes": CAL_BYTES, "copies": CAL_COPIES, "fetch_scale": round(scale["FETCH_SIZE"], 4),
           "write_scale": round(scale["WRITE_SIZE"], 4)}
    if "copy_bytes" in out.get("calibration", {}):  # older single-profile layout
        out["calibration"] = {}
    out.setdefault("calibration", {})[md_name] = cal
    lines = header + ["", "Commands (R = repository root; the counter runs are separate passes):", "", "```"]
    lines += commands + ["```", "",
                         f"Calibration: the last {CAL_COPIES} device copies of {CAL_BYTES >> 20} MiB each; "
                         f"FETCH_SIZE x {scale['FETCH_SIZE']:.3f}, WRITE_SIZE x {scale['WRITE_SIZE']:.3f} "
                         "give bytes.", "",
                         "| kernel | dispatches | avg us | min us | max us | HBM read MB | HBM write MB "
                         "| algorithmic MB | traffic / algorithmic | GB/s (algorithmic) |",
                         "|---|---|---|---|---|---|---|---|---|---|"]
    timed_notes = []
    for name, entry in table.items():
        srcs, ab = entry[2], entry[3]
        hits = sorted((r for r in trace if hit(entry, r["Kernel_Name"], r["Grid_Size_X"])),
                      key=lambda r: int(r["Start_Timestamp"]))
        durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in hits]
        if not durs or per_kernel[name]["FETCH_SIZE"] is None or per_kernel[name]["WRITE_SIZE"] is None:
            continue
        avg = sum(durs) / len(durs) / 1e3
        f_kib = per_kernel[name]["FETCH_SIZE"]
        w_kib = per_kernel[name]["WRITE_SIZE"]
        rd = f_kib * 1024 * scale["FETCH_SIZE"]
        wr = w_kib * 1024 * scale["WRITE_SIZE"]
        last = (timed_last or {}).get(name)
        timed_avg = sum(durs[-last:]) / min(last, len(durs)) / 1e3 if last else None
        out["kernels"][name] = {"avg_us": round(avg, 3), "dispatches": len(durs),
                                "bench_launches_avg_us": None if timed_avg is None else round(timed_avg, 3),
                                "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1),
                                "read_bytes": int(rd), "write_bytes": int(wr), "traffic": int(rd + wr),
                                "algorithmic_bytes": ab, "source_sha256_16": source_digest(srcs),
                                "profile": md_name}
        ratio = f"{(rd + wr) / ab:.3f}" if ab else "—"
        gbs = f"{ab / (avg * 1e-6) / 1e9:.0f}" if ab else "—"
        if timed_avg is not None:
            timed_notes.append(f"{name}: {timed_avg:.2f} us over its last {last} dispatches")
        lines.append(f"| {name} | {len(durs)} | {avg:.2f} | {min(durs) / 1e3:.2f} | {max(durs) / 1e3:.2f} | "
                     f"{rd / 1e6:.1f} | {wr / 1e6:.1f} | {ab / 1e6 if ab else 0:.1f} | {ratio} | {gbs} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(tj, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    if timed_notes:
        lines += ["", "Average kernel duration over the launches the bench line's per-kernel times come from "
                      "(its last dispatches: the rounds of back-to-back launches right after the timed steps; the "
                      "average above also counts the warmup, which runs before the GPU reaches its working clocks):",
                  ""] + [f"* {t}" for t in timed_notes]
    with open(os.path.join(ROOT, "profiles", md_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def summarize(trace_dir, fetch_dir, write_dir):
    alg = kernel_bytes(ROWS * COLS)
    table = {name: (pat, None, srcs, alg.get(name)) for name, (pat, srcs) in KERNELS.items()}
    header = ["# rocprofv3 summary: k-bit quantize / dequantize kernels, 8192x8192 bf16, NF4, blocksize 64", "",
              "The bench step is quantize_kbit_bf16_k4 + dequantize_4bit_nested_bf16; the E4M4-scale pair, "
              "the plain fp32-scale dequantize and the nested-state encoder (quantize_nested_absmax: "
              "nested_bins_kernel + nested_encode_kernel, 1,048,576 blocks) run on the same tensor as side measurements, "
              "and so does quantize_4bit_nested_bf16 (the quantize kernel's nested-sums variant + "
              "nested_encode_kernel over its 512 records of non-negative sums)."]
    return _summarize_into(table, trace_dir, fetch_dir, write_dir, header, PROFILE_COMMANDS,
                           "kbit_kernels_8192sq_bf16_nf4_b64.md",
                           timed_last={"quantize_kbit_bf16_k4": PROFILE_ROUND_LAUNCHES,
                                       "dequantize_4bit_nested_bf16": PROFILE_ROUND_LAUNCHES})


def summarize_side(trace_dir, fetch_dir, write_dir):
    header = ["# rocprofv3 summary: activation-path and fused-linear kernels, bf16", "",
              "Activation assignment (quantize_act_fwht_k4_bf16 / quantize_act_rpbh_k4_bf16) on 4096 rows of "
              "d = 4096 (dedicated kernel), d = 3840 (Hadamard blocks of 256) and d = 12288 (blocks of 4096), "
              "with and without a column permutation; fused 4-bit linear (linear_4bit_nested_bf16, NF4 weights "
              "[N, 4096] with a nested state, B = 64) at M x N = 8 x 4096, 32 x 4096 and 32 x 11008.  Eager "
              "launches over rotated buffer sets (12 for the activations; > 400 MB of weights for the linear)."]
    return _summarize_into(side_kernels(), trace_dir, fetch_dir, write_dir, header, SIDE_PROFILE_COMMANDS,
                           "act_linear_kernels_bf16.md")


_CPU_X = None          # the bf16 weight, shared with forked workers


def _cpu_chunks(chunk_ids, seconds_target):
    """Oracle step (quantize + pack + nested encode + nested dequantize) on
    1 Mi-element chunks (128 rows) of the weight, cycling through chunk_ids
    until seconds_target has passed: (elements, seconds)."""
    from oracle import codebooks, kbit, nested, numerics

    cb = codebooks.nf(K)
    q = codebooks.dynamic_map8()
    chunk = 128 * COLS
    t0 = time.perf_counter()
    done = 0
    i = 0
    while True:
        c = chunk_ids[i % len(chunk_ids)]
        x = _CPU_X[c * chunk:(c + 1) * chunk]
        x32 = numerics.widen(x, "bf16")
        idx, a = kbit.quantize(x32, cb, BLOCK)
        words = kbit.pack(idx, K)
        code, a2, off = nested.encode(a, q)
        _ = nested.dequantize_packed(words, code, a2, off, q, cb, x.size, BLOCK, "bf16")
        done += x.size
        i += 1
        el = time.perf_counter() - t0
        if el >= seconds_target:
            return done, el


def _cpu_worker(arg):
    w, P, seconds = arg
    return _cpu_chunks(list(range(w, ROWS // 128, P)) or [w % (ROWS // 128)], seconds)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(seconds_target):
    """Time the CPU oracle on a bounded sample of the same workload: one
    thread, then chunk-parallel over the host's cores (forked workers; call
    before any GPU work)."""
    global _CPU_X
    import multiprocessing as mp
    from blockwise_bit_codebook_amd import synth

    _CPU_X = synth.weight(ROWS, COLS, "bf16", seed=synth.SEED_WEIGHT_SHAPES)
    n1, t1 = _cpu_chunks(list(range(ROWS // 128)), seconds_target)
    affinity = len(os.sched_getaffinity(0))
    # at most 16 workers: the job's CPU share on a one-GPU host is 16 cores,
    # whatever the affinity mask shows
    P = max(1, min(16, affinity))
    with mp.get_context("fork").Pool(P) as pool:
        res = pool.map(_cpu_worker, [(w, P, seconds_target) for w in range(P)])
    nP = sum(r[0] for r in res)
    tP = max(r[1] for r in res)
    _CPU_X = None

    def gbs(done, el):
        qb, nb = algorithmic_bytes(done)
        return round((qb + nb) / el / 1e9, 4)

    return {
        "value": gbs(nP, tP),
        "unit": "GB/s",
        "cores": P,
        "kind": "oracle",
        "sample": f"{nP} elements: 1 Mi-element chunks (128 rows) of the 8192x8192 bf16 weight, chunk-parallel "
                  f"over {P} forked processes for {tP:.1f} s; each chunk quantize + pack + nested encode + nested "
                  f"dequantize, numpy float32",
        "elements_per_s": round(nP / tP, 1),
        "cpu_model": _cpu_model(),
        "host_cores": os.cpu_count(),
        "affinity_cores": affinity,
        "cores_note": "workers capped at 16, the CPU share of one GPU's job on this host",
        "single_thread": {"value": gbs(n1, t1), "elements_per_s": round(n1 / t1, 1),
                          "sample": f"{n1} elements, chunks in order, one process, {t1:.1f} s"},
    }


ACT_ROWS = ACT_D = 4096
ACT_FLOPS_PER_ELEM = 15          # 12 butterfly add/sub + square + add (norm tree) + divide
# The activation path's arithmetic is single fp32 operations (adds, compares,
# one multiply), not fused multiply-adds, and packed fp32 is not used: its
# roof is the non-packed VALU issue rate, one lane operation per lane per
# clock: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
VALU_LANE_OPS_PEAK = 256 * 4 * 16 * 2.4e9   # 39.3e12 lane operations / s


def act_bytes(rows=ACT_ROWS, d=ACT_D):
    """Algorithmic bytes of one activation-path launch: bf16 in, sign mask,
    16 centroids, 4 bit-planes per 32 and one fp32 norm per row out."""
    n = rows * d
    return 2 * n + d // 8 + 64 + (n // 32) * 4 * 4 + 4 * rows


def bench_act(torch, kb, synth, dev, reps, rows=ACT_ROWS, d=ACT_D, perm=False, sets=12, tables=False):
    """Timing of the W4A4 activation assignment on rows x d bf16 (rows
    N(0,1) x 10^U(-1,1), shared sign mask, Lloyd-Max-16 scaled by sqrt(h/d)
    for d/h Hadamard blocks; with ``perm`` a random column permutation).
    With ``tables`` the calls take the codebook's prepared tables
    (act_tables_k4, built once before timing) instead of the codebook.
    Launches go straight to the C entry point with arguments prepared per
    buffer set, so that Python stays ahead of the GPU."""
    x, signs = synth.activations_bf16(rows, d)
    h = d & -d
    cb = (kb.codebook_lloyd_max_normal(16) * np.float32(np.sqrt(h / d))).astype(np.float32)
    cbl = torch.from_numpy(cb).to(dev)
    sg = torch.from_numpy(signs.view(np.int32)).to(dev)
    pm = None
    if perm:
        pm = torch.from_numpy(np.random.default_rng(d).permutation(d).astype(np.int32)).to(dev)
    x0 = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    bufs = [(x0 if i == 0 else x0.clone(),
             torch.empty(rows, dtype=torch.float32, device=dev),
             torch.empty(kb.n_words(rows * d, 4), dtype=torch.int32, device=dev)) for i in range(sets)]
    tab = kb.act_tables_k4(cbl) if tables else None
    # one call through the wrapper per set (argument checks), then direct calls
    for b in bufs:
        kb.quantize_act_fwht_k4_bf16(b[0], sg, None if tables else cbl, row_norm=b[1], packed=b[2], perm=pm,
                                     tables=tab)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    cb_arg = (tab if tables else cbl).data_ptr()
    name = ("quantize_act_rpbh_k4_bf16" if perm else "quantize_act_fwht_k4_bf16") + ("_tables" if tables else "")
    fn = getattr(kb.lib(), name)
    if perm:
        args = [(b[0].data_ptr(), rows, d, pm.data_ptr(), sg.data_ptr(), cb_arg, b[1].data_ptr(), b[2].data_ptr(),
                 stream) for b in bufs]
    else:
        args = [(b[0].data_ptr(), rows, d, sg.data_ptr(), cb_arg, b[1].data_ptr(), b[2].data_ptr(), stream)
                for b in bufs]
    rc = 0
    for _ in range(3):
        for a in args:
            rc |= fn(*a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        for a in args:
            rc |= fn(*a)
        ev[r + 1].record()
    torch.cuda.synchronize()
    if rc:
        raise RuntimeError(f"an activation launch failed: {kb.lib().kbit_strerror(rc)}")
    ts = np.array([ev[r].elapsed_time(ev[r + 1]) / sets for r in range(reps)])
    avg = float(ts.mean())
    nbytes = act_bytes(rows, d) + (4 * d if perm else 0)
    flops = ACT_FLOPS_PER_ELEM * rows * d
    gbps = nbytes / (avg * 1e-3) / 1e9
    tflops = flops / (avg * 1e-3) / 1e12
    return {"workload": f"{rows} x {d} bf16 activations, Hadamard blocks of {h}"
                        f"{', column permutation' if perm else ''}, Lloyd-Max-16, K=4 planes, "
                        f"{sets} rotated buffer sets"
                        f"{', prepared codebook tables' if tables else ', tables built per call'}",
            "avg_us": round(avg * 1e3, 3), "median_us": round(float(np.median(ts)) * 1e3, 3),
            "bytes": nbytes, "GB/s": round(gbps, 2), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "algorithmic_flops": flops, "TFLOP/s": round(tflops, 3),
            "alu": {"bound": "alu", "achieved": round(tflops * 1e12, 1), "peak": VALU_LANE_OPS_PEAK,
                    "unit": "lane-ops/s", "frac": round(tflops * 1e12 / VALU_LANE_OPS_PEAK, 4),
                    "note": "algorithmic operations (15 per element) against the non-packed VALU issue rate"},
            "rows_per_s": round(rows / (avg * 1e-3), 1)}


NESTED_CELL_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008), (8192, 8192))


def bench_nested_cells(torch, kb, dev, reps, sets=4):
    """Nested 4-bit dequantize for NF4 and FP4 x fp16/bf16/fp32 x the four
    weight shapes (24 cells): N(0, 0.02) weight, blocksize 64, state from
    the library's own quantize and nested encode; each cell timed in rounds
    over rotated buffer sets."""
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}
    esz = {"fp16": 2, "bf16": 2, "fp32": 4}
    qmap = torch.from_numpy(kb.dynamic_map8()).to(dev)
    cells = []
    for cbname, cbv in (("nf4", kb.codebook_nf(4)), ("fp4", kb.codebook_fp4())):
        cbt = torch.from_numpy(cbv).to(dev)
        for name, dt in tdt.items():
            for rows, cols in NESTED_CELL_SHAPES:
                n = rows * cols
                nb = n // BLOCK
                g = torch.Generator(device=dev).manual_seed(rows * 7 + cols)
                states = []
                for i in range(sets):
                    A = (torch.randn(n, generator=g, device=dev) * 0.02).to(dt)
                    packed, absmax = kb.quantize_kbit(A, cbt, 4, BLOCK)
                    code, a2, off = kb.quantize_nested_absmax(absmax, qmap)
                    states.append((packed, code, a2, float(off.item()), torch.empty(n, dtype=dt, device=dev)))
                    del A, absmax

                # checked once through the binding, then timed through the
                # C entry point with prepared arguments (a small cell's
                # kernel is shorter than the binding's per-call checks)
                for i in range(sets):
                    p_, c_, a2_, o_, out_ = states[i]
                    kb.dequantize_4bit_nested(p_, cbt, c_, qmap, a2_, o_, n, dt, BLOCK, out=out_)
                fn = getattr(kb.lib(), f"dequantize_4bit_nested_{name}")
                sp = torch.cuda.current_stream(dev).cuda_stream
                dargs = [(p_.data_ptr(), cbt.data_ptr(), c_.data_ptr(), qmap.data_ptr(), a2_.data_ptr(), o_,
                          out_.data_ptr(), n, BLOCK, sp) for p_, c_, a2_, o_, out_ in states]

                def d(i):
                    if fn(*dargs[i]):
                        raise RuntimeError("nested dequantize launch failed")

                for _ in range(3):
                    for i in range(sets):
                        d(i)
                torch.cuda.synchronize()
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
                ev[0].record()
                for r in range(reps):
                    for i in range(sets):
                        d(i)
                    ev[r + 1].record()
                torch.cuda.synchronize()
                ts = np.array([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]) / sets * 1e3
                nbytes = n // 2 + nb + 4 * (-(-nb // 256)) + esz[name] * n + 4 * 256 + 4 * 16
                us = float(ts.mean())
                cells.append({"codebook": cbname, "dtype": name, "shape": [rows, cols], "avg_us": round(us, 3),
                              "median_us": round(float(np.median(ts)), 3), "bytes": nbytes,
                              "GB/s": round(nbytes / (us * 1e-6) / 1e9, 2),
                              "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
                del states
                torch.cuda.empty_cache()
    return {"workload": "nested 4-bit dequantize, N(0,0.02) weights, blocksize 64, groups of 256, dynamic map; "
                        "NF4/FP4 x fp16/bf16/fp32 x 4096^2, 11008x4096, 4096x11008, 8192^2; 4 rotated buffer sets, "
                        "state from the library's quantize + nested encode",
            "cells": cells}


def bench_sweep(torch, kb, dev, reps, sets=4):
    """Quantize and plain dequantize of the 8192 x 8192 N(0, 0.02) weight for
    every input type and K = 2..5 (NF_K codebook, blocksize 64), each pair in
    round robin over rotated buffer sets.  After one call through each
    wrapper (argument checks), the launches go straight to the C entry
    points with arguments prepared per buffer set: a wrapper call costs
    Python time of the order of a launch, which would starve the GPU."""
    n = ROWS * COLS
    nb = n // BLOCK
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
    esz = {"fp32": 4, "fp16": 2, "bf16": 2}
    res = []
    for name, dt in tdt.items():
        g = torch.Generator(device="cpu").manual_seed(7)
        base = (torch.randn(n, generator=g) * 0.02).to(dt).to(dev)
        bufs = [(base if i == 0 else base.clone(), torch.empty(nb, dtype=torch.float32, device=dev),
                 torch.empty(n, dtype=dt, device=dev)) for i in range(sets)]
        for Kk in (2, 3, 4, 5):
            cbk = torch.from_numpy(kb.codebook_nf(Kk)).to(dev)
            packed = [torch.empty(kb.n_words(n, Kk), dtype=torch.int32, device=dev) for _ in range(sets)]

            for i in range(sets):
                kb.quantize_kbit(bufs[i][0], cbk, Kk, BLOCK, absmax=bufs[i][1], packed=packed[i])
                kb.dequantize_kbit(packed[i], cbk, bufs[i][1], Kk, n, dt, BLOCK, out=bufs[i][2])
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream(dev).cuda_stream
            qf = getattr(kb.lib(), f"quantize_kbit_{name}_k{Kk}")
            df = getattr(kb.lib(), f"dequantize_kbit_{name}_k{Kk}")
            qa = [(cbk.data_ptr(), bufs[i][0].data_ptr(), bufs[i][1].data_ptr(), packed[i].data_ptr(), n, BLOCK,
                   stream) for i in range(sets)]
            da = [(packed[i].data_ptr(), cbk.data_ptr(), bufs[i][1].data_ptr(), bufs[i][2].data_ptr(), n, BLOCK,
                   stream) for i in range(sets)]
            rc = 0

            def q(i):
                nonlocal rc
                rc |= qf(*qa[i])

            def d(i):
                nonlocal rc
                rc |= df(*da[i])

            for _ in range(3):
                for i in range(sets):
                    q(i)
                for i in range(sets):
                    d(i)
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
            for r in range(reps):
                ev[r][0].record()
                for i in range(sets):
                    q(i)
                ev[r][1].record()
                for i in range(sets):
                    d(i)
                ev[r][2].record()
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"a sweep launch failed: {kb.lib().kbit_strerror(rc)}")
            tq = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / sets * 1e3
            td = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) / sets * 1e3
            bq = esz[name] * n + 4 * (n // 32) * Kk + 4 * nb + 4 * (1 << Kk)
            res.append({"dtype": name, "K": Kk, "quantize_us": round(tq, 3),
                        "quantize_frac_of_hbm_peak": round(bq / (tq * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                        "dequantize_us": round(td, 3),
                        "dequantize_frac_of_hbm_peak": round(bq / (td * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                        "bytes": bq})
            del packed
        del bufs, base
        torch.cuda.empty_cache()
    return {"workload": "8192x8192 N(0,0.02) weight, NF_K, blocksize 64, fp32 scales; quantize and plain "
                        "dequantize per input type and K, 4 rotated buffer sets",
            "cases": res}


# Block-Hadamard activation cases: (rows, d, permutation).
ACT_BLOCK_CASES = [(4096, 3840, False), (4096, 3840, True), (4096, 12288, False), (4096, 12288, True),
                   (4096, 4096, True)]


# The page's dequantize-plus-linear controls (M, N, K) and their candidate
# medians on the page's GPU (context only, another machine).
LINEAR_SHAPES = [(1, 4096, 4096, 26.735), (8, 4096, 4096, 24.748), (32, 4096, 4096, 24.752),
                 (32, 11008, 4096, 61.726)]


# The side profile: one case per (kernel, grid) so that the trace can tell
# them apart.  (rows, d, permutation) and (M, N, K).
SIDE_ACT_CASES = [(4096, 4096, False), (4096, 3840, False), (4096, 3840, True), (4096, 12288, False),
                  (4096, 12288, True)]
SIDE_LINEAR_SHAPES = [(8, 4096, 4096), (32, 4096, 4096), (32, 11008, 4096)]
_A_SRC = ["blockwise_bit_codebook_amd/csrc/act_fwht.hip", "blockwise_bit_codebook_amd/csrc/act_common.h",
          "blockwise_bit_codebook_amd/csrc/threshold.h", "blockwise_bit_codebook_amd/csrc/device.h"]
_AB_SRC = ["blockwise_bit_codebook_amd/csrc/act_block.hip", "blockwise_bit_codebook_amd/csrc/act_common.h",
           "blockwise_bit_codebook_amd/csrc/threshold.h", "blockwise_bit_codebook_amd/csrc/device.h"]
_L_SRC = ["blockwise_bit_codebook_amd/csrc/linear.hip", "blockwise_bit_codebook_amd/csrc/device.h"]
SIDE_PROFILE_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/side_trace -o trace -- "
    "python3 $R/bench.py --side-only --side-reps 20 --copy-calibration",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/side_fetch -o fetch -- "
    "python3 $R/bench.py --side-only --side-reps 1 --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/side_write -o write -- "
    "python3 $R/bench.py --side-only --side-reps 1 --copy-calibration",
    "cd $R && python3 bench.py --summarize-side gpurun_out/side_trace gpurun_out/side_fetch gpurun_out/side_write",
]


def side_kernels():
    """name -> (name substrings, grid size in threads or None, sources, algorithmic bytes per launch)."""
    t = {}
    for rows, d, perm in SIDE_ACT_CASES:
        h = d & -d
        if d == 4096 and not perm:
            t[f"act_fwht {rows}x{d}"] = (("::act_fwht_kernel<2>",), None, _A_SRC, act_bytes(rows, d))
        else:
            L = h.bit_length() - 1
            name = f"act_block {rows}x{d} h={h}" + (" perm" if perm else "")
            t[name] = ((f"::act_block_kernel<{L}, {'true' if perm else 'false'}>",), None, _AB_SRC,
                       act_bytes(rows, d) + (4 * d if perm else 0))
    for M, N, Kd in SIDE_LINEAR_SHAPES:
        mt = 1 if M <= 16 else 2 if M <= 32 else 4
        t[f"linear_4bit_nested {M}x{N}x{Kd}"] = (("::linear4_kernel<", f"LinNested, {mt}>"), (N // 16) * 1024,
                                                 _L_SRC, linear_bytes(M, N, Kd))
    return t


def linear_bytes(M, N, K):
    """Minimum bytes of one fused linear call with a nested state (B = 64):
    packed weights, codes, group absmax, map and codebook, X and out."""
    nb = N * K // BLOCK
    return N * K // 2 + nb + 4 * (-(-nb // GROUP2)) + 4 * 256 + 64 + 2 * M * K + 2 * M * N


def bench_quantize_nested(torch, kb, sets, cb, qmap, n, reps, round_robin, kstats):
    """Per-call time of quantize_4bit_nested_bf16 (two kernels) and of
    quantize_kbit_bf16_k4 followed by quantize_nested_absmax (three), in one
    round robin over the buffer sets."""
    nb = -(-n // BLOCK)

    def fused(s):
        kb.quantize_4bit_nested(s["A"], cb, qmap, BLOCK, absmax=s["absmax"], packed=s["packed"],
                                absmax_code=s["enc_code"], absmax2=s["enc_a2"], offset=s["enc_off"],
                                workspace=s["qws"])

    def chain(s):
        kb.quantize_kbit(s["A"], cb, K, BLOCK, absmax=s["absmax"], packed=s["packed"])
        kb.quantize_nested_absmax(s["absmax"], qmap, absmax_code=s["enc_code"], absmax2=s["enc_a2"],
                                  offset=s["enc_off"], workspace=s["ws"])

    r = round_robin({"quantize_4bit_nested_bf16": fused, "quantize_kbit_bf16_k4+quantize_nested_absmax": chain},
                    reps, bufs=sets)
    kbytes = kernel_bytes(n)
    enc_once = kbytes["quantize_nested_absmax"] - 4 * nb   # the absmax read once
    return {"quantize_4bit_nested_bf16": kstats(r["quantize_4bit_nested_bf16"],
                                                kbytes["quantize_kbit_bf16_k4"] + enc_once, elems=n),
            "quantize_kbit_bf16_k4+quantize_nested_absmax": kstats(
                r["quantize_kbit_bf16_k4+quantize_nested_absmax"],
                kbytes["quantize_kbit_bf16_k4"] + kbytes["quantize_nested_absmax"], elems=n)}


def bench_linear(torch, kb, synth, dev, reps=20, shapes=None, eager=False):
    """Fused 4-bit linear (nested state) at the page's shapes.  Each timed
    call uses a different weight set (rotated through > 400 MB, beyond the
    last-level cache); the launches are captured in a HIP graph so that
    Python's launch cost is not timed.  The warm figure reuses one set."""
    cb = torch.from_numpy(kb.codebook_nf(K)).to(dev)
    q = torch.from_numpy(kb.dynamic_map8()).to(dev)
    res = []
    for M, N, Kd, page_us in (LINEAR_SHAPES if shapes is None else [(*sh, None) for sh in shapes]):
        nb = N * Kd // BLOCK
        nbytes = linear_bytes(M, N, Kd)
        sets = int(min(64, max(2, -(-(400 << 20) // nbytes))))
        g = torch.Generator(device="cpu").manual_seed(M * 131 + N)
        w0 = torch.randint(-2 ** 31, 2 ** 31 - 1, (N * Kd // 8,), dtype=torch.int32, generator=g).to(dev)
        code_np, a2_np, off = synth.nested_state_synthetic(nb, seed=M + 5)
        code0 = torch.from_numpy(code_np).to(dev)
        a20 = torch.from_numpy(a2_np).to(dev)
        X = torch.from_numpy(synth.normal(M * Kd, seed=M, dtype="bf16").view(np.int16)).to(dev).view(
            torch.bfloat16).reshape(M, Kd)
        bufs = [(w0 if i == 0 else w0.clone(), code0 if i == 0 else code0.clone(), a20 if i == 0 else a20.clone(),
                 torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for i in range(sets)]
        torch.cuda.synchronize()

        def call(b):
            kb.linear_4bit(X, b[0], cb, N, BLOCK, absmax_code=b[1], qmap2=q, absmax2=b[2], offset=off, out=b[3])

        for b in bufs:
            call(b)
        torch.cuda.synchronize()

        def timed(items):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for b in items:
                    call(b)
            gr.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * len(items))

        if eager:
            # plain launches (what the side profile traces)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                for b in bufs:
                    call(b)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(bufs))
            warm = None
        else:
            us = timed(bufs)
            warm = timed([bufs[0]] * sets)
        warm = None if warm is None else round(warm, 3)
        res.append({"M": M, "N": N, "K": Kd, "avg_us": round(us, 3), "warm_avg_us": warm,
                    "bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "TFLOP/s": round(2.0 * M * N * Kd / (us * 1e-6) / 1e12, 3),
                    "weight_sets": sets, "page_candidate_us": page_us})
        del bufs
        torch.cuda.empty_cache()
    return {"workload": "linear_4bit_nested_bf16: bf16 X [M, K] x NF4 weights [N, K] with a nested state, B=64, "
                        "graph-replayed launches over rotated weight sets",
            "shapes": res,
            "note": "page_candidate_us: the page's fused dequantize + linear medians on its own GPU, context only"}


class HipEvents:
    """Timing events recorded on a HIP stream, created with
    hipEventDisableSystemFence (no system-scope cache flush per record)."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, stream):
        import ctypes
        self.ct = ctypes
        try:
            hip = ctypes.CDLL("libamdhip64.so")
        except OSError:
            hip = ctypes.CDLL(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "libamdhip64.so"))
        vp = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        hip.hipEventDestroy.argtypes = [vp]
        self.hip = hip
        self.stream = vp(stream)

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self, k):
        out = []
        for _ in range(k):
            e = self.ct.c_void_p()
            self._ok(self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.FLAGS), "hipEventCreateWithFlags")
            out.append(e)
        return out

    def record(self, e):
        self._ok(self.hip.hipEventRecord(e, self.stream), "hipEventRecord")

    def elapsed_ms(self, a, b):
        m = self.ct.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.ct.byref(m), a, b), "hipEventElapsedTime")
        return m.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def side_only(args):
    """The side profile's workload: the activation cases, then the linear
    shapes, eagerly launched; then the calibration copies if asked."""
    import torch
    import blockwise_bit_codebook_amd as kb
    from blockwise_bit_codebook_amd import synth
    dev = torch.device("cuda:0")
    out = {"act": [], "linear": None}
    for rows, d, perm in SIDE_ACT_CASES:
        r = bench_act(torch, kb, synth, dev, args.side_reps, rows=rows, d=d, perm=perm)
        out["act"].append(r)
        print(f"[side] act {rows}x{d} perm={perm}: {r['avg_us']} us", file=sys.stderr, flush=True)
    out["linear"] = bench_linear(torch, kb, synth, dev, reps=args.side_reps, shapes=SIDE_LINEAR_SHAPES, eager=True)
    print("[side] linear done", file=sys.stderr, flush=True)
    if args.copy_calibration:
        src = torch.zeros(CAL_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(CAL_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(out))
    return 0


def main(argv=None):
    args = parse(argv)
    if args.summarize:
        return summarize(*args.summarize)
    if args.summarize_side:
        return summarize_side(*args.summarize_side)
    if args.steps < 1 or args.sets < 1 or args.warmup < 0:
        print("--steps and --sets must be positive, --warmup non-negative", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the hot path has no "
              "cross-GPU step to measure here.", file=sys.stderr)
        return 2

    if args.side_only:
        return side_only(args)

    # the CPU oracle runs first: its workers are forked before any GPU work
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

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
            "code8": torch.empty(nb, dtype=torch.uint8, device=dev),
            "enc_code": torch.empty(nb, dtype=torch.uint8, device=dev),
            "enc_a2": torch.empty(-(-nb // GROUP2), dtype=torch.float32, device=dev),
            "enc_off": torch.zeros(1, dtype=torch.float32, device=dev),
            "ws": torch.empty(kb.lib().kbit_nested_workspace_bytes(nb), dtype=torch.uint8, device=dev),
            "qws": torch.empty(kb.lib().kbit_quantize_nested_workspace_bytes(), dtype=torch.uint8, device=dev),
        })
    torch.cuda.synchronize()

    def step(s):
        kb.quantize_kbit(s["A"], cb, K, BLOCK, absmax=s["absmax"], packed=s["packed"])
        kb.dequantize_4bit_nested(s["packed"], cb, s["code"], qmap, s["absmax2"], offset, n,
                                  torch.bfloat16, BLOCK, out=s["out"])

    # The side kernels through their wrappers.  Their Python cost (a few
    # microseconds) is far below every side kernel's duration.  With direct
    # calls the whole side round robin queued up at once, and the FP4
    # quantize that follows it measured 31-44 us (average 36.4) against
    # 29.7-31.0 us with the wrappers; alone, back to back or alternating
    # with the nested dequantize, FP4 quantize runs 29.9-30.3 us, as NF4.
    def quant_only(s):
        kb.quantize_kbit(s["A"], cb, K, BLOCK, absmax=s["absmax"], packed=s["packed"])

    def nested_only(s):
        kb.dequantize_4bit_nested(s["packed"], cb, s["code"], qmap, s["absmax2"], offset, n,
                                  torch.bfloat16, BLOCK, out=s["out"])

    def quant_e4m4(s):
        kb.quantize_kbit(s["A"], cb, K, BLOCK, absmax=s["code8"], packed=s["packed"], absmax_format="e4m4")

    def dequant_e4m4(s):
        kb.dequantize_kbit(s["packed"], cb, s["code8"], K, n, torch.bfloat16, BLOCK, out=s["out"])

    def dequant_plain(s):
        kb.dequantize_kbit(s["packed"], cb, s["absmax"], K, n, torch.bfloat16, BLOCK, out=s["out"])

    def encode_nested(s):
        kb.quantize_nested_absmax(s["absmax"], qmap, absmax_code=s["enc_code"], absmax2=s["enc_a2"],
                                  offset=s["enc_off"], workspace=s["ws"])

    for s_ in sets:                              # eager once per set: per-device setup happens here
        step(s_)
    torch.cuda.synchronize()

    # The two step kernels through their C entry points, with arguments
    # prepared once per buffer set: the same calls quant_only and
    # nested_only make, without the wrappers' per-call checks, so that
    # Python stays well ahead of the GPU.
    stream_ptr = torch.cuda.current_stream(dev).cuda_stream
    qfn, dfn = kb.lib().quantize_kbit_bf16_k4, kb.lib().dequantize_4bit_nested_bf16
    qargs = [(cb.data_ptr(), s_["A"].data_ptr(), s_["absmax"].data_ptr(), s_["packed"].data_ptr(), n, BLOCK,
              stream_ptr) for s_ in sets]
    dargs = [(s_["packed"].data_ptr(), cb.data_ptr(), s_["code"].data_ptr(), qmap.data_ptr(),
              s_["absmax2"].data_ptr(), float(offset), s_["out"].data_ptr(), n, BLOCK, stream_ptr) for s_ in sets]

    def settle():
        # Steps back to back for at least --settle-ms (chunks of 16 with a
        # sync after each), so that what follows starts at the GPU's
        # sustained clocks however short --warmup is.
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        i = rc_ = 0
        while True:
            for _ in range(16):
                j = i % args.sets
                rc_ |= qfn(*qargs[j])
                rc_ |= dfn(*dargs[j])
                i += 1
            torch.cuda.synchronize()
            if time.perf_counter() >= t_end:
                break
        if rc_:
            raise RuntimeError(f"a settle launch failed: {kb.lib().kbit_strerror(rc_)}")

    # Side kernels: per-kernel launch time from events on the same stream, in
    # round robin: each round launches every kernel once per buffer set, with
    # an event before and after each kernel's launches, so that all of them
    # are timed under the same clock and power state.
    def round_robin(fns, reps, warm=3, bufs=None):
        bufs = sets if bufs is None else bufs
        for _ in range(warm):
            for fn in fns.values():
                for s_ in bufs:
                    fn(s_)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps * len(fns))]
        for r in range(reps):
            for j, fn in enumerate(fns.values()):
                e = ev[r * len(fns) + j]
                e[0].record()
                for s_ in bufs:
                    fn(s_)
                e[1].record()
        torch.cuda.synchronize()
        return {name: [ev[r * len(fns) + j][0].elapsed_time(ev[r * len(fns) + j][1]) / len(bufs)
                       for r in range(reps)] for j, name in enumerate(fns)}

    # bring the GPU to its working clocks before the side measurements too
    settle()
    for i in range(args.warmup):
        step(sets[i % args.sets])
    torch.cuda.synchronize()
    reps = args.rr_reps or max(5, args.steps // args.sets)
    # quant_e4m4 before dequant_e4m4 and quant_only before dequant_plain in
    # every round: each dequantize reads scales written by its own quantize.
    rr = round_robin({"quantize_kbit_bf16_k4": quant_only, "dequantize_4bit_nested_bf16": nested_only,
                      "quantize_kbit_e4m4_bf16_k4": quant_e4m4, "dequantize_kbit_e4m4_bf16_k4": dequant_e4m4,
                      "dequantize_kbit_bf16_k4": dequant_plain, "quantize_nested_absmax": encode_nested}, reps)
    qbytes, nbytes = algorithmic_bytes(n)

    def kstats(ts, nbytes_, elems=n):
        ts = np.array(ts)
        avg = float(ts.mean())
        gbps = nbytes_ / (avg * 1e-3) / 1e9
        return {"avg_us": round(avg * 1e3, 3), "median_us": round(float(np.median(ts)) * 1e3, 3),
                "p10_us": round(float(np.percentile(ts, 10)) * 1e3, 3),
                "p90_us": round(float(np.percentile(ts, 90)) * 1e3, 3),
                "min_us": round(float(ts.min()) * 1e3, 3), "max_us": round(float(ts.max()) * 1e3, 3),
                "bytes": nbytes_, "GB/s": round(gbps, 2), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "elements_per_s": round(elems / (avg * 1e-3), 1)}

    # One-byte E4M4 scales on the same tensor, and the plain fp32-scale
    # dequantize (distinct kernels, so they do not mix into the step's
    # per-kernel profile), from the same round robin.
    kbytes = kernel_bytes(n)
    e4 = {k: kstats(rr[k], kbytes[k]) for k in ("quantize_kbit_e4m4_bf16_k4", "dequantize_kbit_e4m4_bf16_k4",
                                                "dequantize_kbit_bf16_k4")}
    e4["note"] = ("same 8192x8192 bf16 tensor and NF4 codebook; scales as one E4M4 byte per block "
                  "(the last entry: fp32 scales, for comparison)")
    enc = kstats(rr["quantize_nested_absmax"], kbytes["quantize_nested_absmax"], elems=nb)
    enc["note"] = ("nested-state encoder on the 1,048,576 fp32 block absmax of the same tensor: two launches "
                   "(exact significand sums; mean and codes); elements_per_s counts blocks")

    # Quantize straight to the nested state (quantize_4bit_nested_bf16, two
    # kernels) against quantize then quantize_nested_absmax (three), whole
    # calls in a round robin of their own.
    qnest = {"8192x8192": bench_quantize_nested(torch, kb, sets, cb, qmap, n, reps, round_robin, kstats),
             "note": ("bf16 NF4 B=64 to the nested state (codes, absmax2, offset): quantize_4bit_nested_bf16 "
                      "(two kernels; the quantize kernel also sums its block maxima exactly) against "
                      "quantize_kbit_bf16_k4 then quantize_nested_absmax (three kernels); per call, "
                      "bit-identical results")}

    # The same two kernels with the FP4 codebook, and warm numbers (one
    # buffer set over and over, so the last-level cache holds most of it).
    fp4 = warm = act = act_block = lin = sweep = cells = None
    if not args.headline_only:
        pair = {"quantize_kbit_bf16_k4": quant_only, "dequantize_4bit_nested_bf16": nested_only}
        cb_nf = cb
        cb = torch.from_numpy(kb.codebook_fp4()).to(dev)
        r4 = round_robin(pair, reps)
        fp4 = {"quantize_kbit_bf16_k4": kstats(r4["quantize_kbit_bf16_k4"], qbytes),
               "dequantize_4bit_nested_bf16": kstats(r4["dequantize_4bit_nested_bf16"], nbytes)}
        cb = cb_nf
        rw = round_robin(pair, reps, bufs=sets[:1])
        warm = {"quantize_kbit_bf16_k4": kstats(rw["quantize_kbit_bf16_k4"], qbytes),
                "dequantize_4bit_nested_bf16": kstats(rw["dequantize_4bit_nested_bf16"], nbytes),
                "note": "same buffer set every launch (warm cache); not the headline number"}
        if not args.no_act:
            act = bench_act(torch, kb, synth, dev, reps)
            act["prepared_tables"] = bench_act(torch, kb, synth, dev, reps, tables=True)
            act_block = []
            for r, dd, pp in ACT_BLOCK_CASES:
                one = bench_act(torch, kb, synth, dev, reps, rows=r, d=dd, perm=pp)
                one["prepared_tables"] = bench_act(torch, kb, synth, dev, reps, rows=r, d=dd, perm=pp, tables=True)
                act_block.append(one)
        # The same comparison on a 4096x4096 weight.
        small = synth.weight(4096, 4096, "bf16", seed=synth.SEED_WEIGHT_SHAPES)
        n_s = small.size
        nb_s = -(-n_s // BLOCK)
        x_s = torch.from_numpy(small.view(np.int16)).to(dev).view(torch.bfloat16)
        sets_s = [{"A": x_s if i == 0 else x_s.clone(),
                   "packed": torch.empty(kb.n_words(n_s, K), dtype=torch.int32, device=dev),
                   "absmax": torch.empty(nb_s, dtype=torch.float32, device=dev),
                   "enc_code": torch.empty(nb_s, dtype=torch.uint8, device=dev),
                   "enc_a2": torch.empty(-(-nb_s // GROUP2), dtype=torch.float32, device=dev),
                   "enc_off": torch.zeros(1, dtype=torch.float32, device=dev),
                   "ws": torch.empty(kb.lib().kbit_nested_workspace_bytes(nb_s), dtype=torch.uint8, device=dev),
                   "qws": torch.empty(kb.lib().kbit_quantize_nested_workspace_bytes(), dtype=torch.uint8,
                                      device=dev)} for i in range(args.sets)]
        qnest["4096x4096"] = bench_quantize_nested(torch, kb, sets_s, cb, qmap, n_s, reps, round_robin, kstats)
        del sets_s, x_s
        lin = bench_linear(torch, kb, synth, dev)
        sweep = bench_sweep(torch, kb, dev, reps)
        cells = bench_nested_cells(torch, kb, dev, max(4, reps // 2))

    # The timed region (after the side measurements, which also bring the
    # GPU to its working clocks): args.steps steps, launched eagerly (Python
    # issues a step in far less time than the GPU runs it), with HIP events
    # only at its two ends.  An event after every kernel would lengthen each
    # step by 1-2.5 us (measured), so the per-kernel launch durations of the
    # roofline come from the rounds right after the timed region: each step
    # kernel alone, back to back over the rotated buffer sets, with an event
    # at each round's ends (max(KERNEL_ROUNDS_MIN, steps / sets) rounds of
    # ROUND_PASSES passes over the sets: an event costs about 1-2.5 us of GPU
    # time inside back-to-back work, which a round of one pass, 4 launches,
    # put at about 0.8 us on each launch's figure).
    # The events are created without the system-scope fence
    # (hipEventDisableSystemFence): default events add a cache flush per
    # record.  All launches call the two C entry points directly (qfn,
    # dfn).  A settle period of back-to-back steps comes before the
    # --warmup steps.
    settle()
    for i in range(args.warmup):
        step(sets[i % args.sets])
    torch.cuda.synchronize()
    hev = HipEvents(stream_ptr)
    marks = hev.create(2)
    rc = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hev.record(marks[0])
    for i in range(args.steps):
        j = i % args.sets
        rc |= qfn(*qargs[j])
        rc |= dfn(*dargs[j])
    hev.record(marks[1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if rc:
        raise RuntimeError(f"a timed launch failed: {kb.lib().kbit_strerror(rc)}")
    gpu_ms = hev.elapsed_ms(marks[0], marks[1])
    hev.destroy(marks)
    ms_step = wall * 1e3 / args.steps
    value = (qbytes + nbytes) / (ms_step * 1e-3) / 1e9

    def launch_rounds(fn, argsets):
        rounds = max(KERNEL_ROUNDS_MIN, args.steps // len(argsets))
        rm = hev.create(rounds + 1)
        code = 0
        hev.record(rm[0])
        for r in range(rounds):
            for _ in range(ROUND_PASSES):
                for a in argsets:
                    code |= fn(*a)
            hev.record(rm[r + 1])
        torch.cuda.synchronize()
        if code:
            raise RuntimeError(f"a timed launch failed: {kb.lib().kbit_strerror(code)}")
        ts = [hev.elapsed_ms(rm[r], rm[r + 1]) / (ROUND_PASSES * len(argsets)) for r in range(rounds)]
        hev.destroy(rm)
        return ts

    tq = launch_rounds(qfn, qargs)
    tn = launch_rounds(dfn, dargs)
    kq, kn = kstats(tq, qbytes), kstats(tn, nbytes)
    kq["note"] = kn["note"] = ("average launch duration: rounds of back-to-back launches over the rotated "
                               "buffer sets right after the timed steps; per-round averages")

    dom_name, dom = ("quantize_kbit_bf16_k4", kq) if kq["avg_us"] >= kn["avg_us"] else \
        ("dequantize_4bit_nested_bf16", kn)
    traffic = None
    if os.path.exists(args.traffic_json):
        # counters taken on a different version of the kernel's source do not count
        try:
            with open(args.traffic_json) as f:
                rec = json.load(f)["kernels"].get(dom_name)
            if rec and rec["source_sha256_16"] == source_digest(KERNELS[dom_name][1]):
                traffic = rec["traffic"]
        except (OSError, ValueError, KeyError):
            traffic = None
    roofline = {"kernel": dom_name, "bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dom["frac_of_hbm_peak"], "traffic": traffic}

    if args.copy_calibration:
        src = torch.zeros(CAL_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(CAL_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()


    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 5),
        "gpu_ms_per_step": round(gpu_ms / args.steps, 5),
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
        "e4m4_scales": e4,
        "nested_state_encoder": enc,
        "quantize_to_nested_state": qnest,
        "fp4_codebook": fp4,
        "warm": warm,
        "act_fwht": act,
        "act_block_hadamard": act_block,
        "linear_4bit": lin,
        "dtype_k_sweep": sweep,
        "nested_dequant_cells": cells,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
        "arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
        "hip": torch.version.hip,
        "environment": {"torch": torch.__version__, "rocm_hip": torch.version.hip, "python": sys.version.split()[0],
                        "cpu_model": _cpu_model(), "host_cores": os.cpu_count(),
                        "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
                        "hbm_bytes": torch.cuda.get_device_properties(dev).total_memory},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
