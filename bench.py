"""Throughput of the CSA decode hot path on one MI355X (plus the prefill stages).

One step = one CSA decode step of the V4-Flash-shaped workload (batch 32, 128K
context, 32768 compressed entries per sequence, 64 indexer heads x 128 FP8, top-512,
64 query heads x 512 bf16, 128-token window, per-head sink): lightning-indexer scores with
each 4096-entry segment's top-k (keys in the 16-entry blocked layout the decode-time
compressor appends to), then the selection of each query's top-k and the sparse
attention in one call.  Inputs are resident in HBM before timing; the step rotates over
several independent input sets (together larger than the 256 MB Infinity Cache) so the
indexer keys stream from HBM.

`value` times K eagerly launched steps; `ms_per_step_graph` the same K steps replayed
from HIP graphs.  `roofline` is for the dominant kernel (the scoring pass), its duration
timed with HIP events around each of its launches inside K more steps, on its stream.
`decode_layer` adds the decode-time compressor (main KV + indexer key append for the new
token) and the inverse-RoPE epilogue: the whole CSA layer step after the dense
projections.  `cpu_baseline` is the CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--sets N] [--eager] [--no-cpu-baseline]
                    [--subs prefill,pro,hca,compressor,prefill_attention,decode_layer]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode tokens/s + HBM GB/s @128K ctx; prefill indexer TFLOPS (% roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA
ALL_SUBS = ("prefill", "pro", "hca", "compressor", "prefill_attention", "decode_layer")
ROOFLINE_KERNEL = "index_score_fp8_decode<true, true, false, false>"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=4, help="independent input sets rotated per step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--subs", default=",".join(ALL_SUBS),
                   help="comma-separated sub-benchmarks to run (empty: none): " + ",".join(ALL_SUBS))
    p.add_argument("--eager", action="store_true", help="time eager launches only (no graph replay)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one 256 MiB device copy (reference kernel for HBM byte counters)")
    p.add_argument("--summarize-mfma", nargs=2, metavar=("COUNTER_DIR", "BENCH_LOG"),
                   help="write the prefill indexer's MFMA counter summary into profiles/")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) made "
                        "with --calibrate-copy into the committed traffic summaries")
    p.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                   help="no GPU work: turn a rocprofv3 --kernel-trace --stats run of the default bench into "
                        "the committed kernel-trace summary")
    return p.parse_args()


def index_score_bytes(B, S, Nc, H_I, d_I):
    """Algorithmic HBM bytes of one indexer launch (decode: every visible key once)."""
    per_query = Nc * (d_I + 4) + 4 * Nc + H_I * (d_I + 4 + 4) + 8   # keys+scales, scores, q+scale+w, pos
    return B * S * per_query


SEGMENT = 4096   # entries per segment of the scoring pass that also selects (csa_index_score_segments)


def index_segments_bytes(B, S, Nc, H_I, d_I, k):
    """Algorithmic HBM bytes of one scoring pass that keeps its scores on chip and writes
    every segment's top-k: keys + scales, q + scale + w, position, (key, entry) pairs."""
    per_query = Nc * (d_I + 4) + H_I * (d_I + 4 + 4) + 8 + -(-Nc // SEGMENT) * k * 8
    return B * S * per_query


def decode_step_bytes(sh):
    """Compulsory bytes of one decode step (the score/index round trip between stages excluded)."""
    B = sh.B
    keys = B * sh.n_c * (sh.d_I + 4)
    gathered = B * (sh.k + sh.W) * sh.c * 2
    q_and_o = 2 * B * sh.H * sh.c * 2
    small = B * (sh.H_I * (sh.d_I + 8) + sh.k * 4 + 8) + sh.H * 4
    return keys + gathered + q_and_o + small


COPY_BYTES = 256 << 20


# Kernels whose HBM traffic the counter runs summarise: (summary name, kernel name, total
# work-items of the dispatches meant (None: every dispatch), sources compiled into it,
# algorithmic bytes per launch, what those bytes are).  The counter runs use
# COUNTER_BENCH_ARGS: the default step (Flash decode, B = 32) and the HCA sub-benchmark.
ATTN_SOURCES = ("attention.hip", "attention_common.hpp", "select.hpp", "common.hpp")


def counter_kernels():
    from synthetic import inputs as I
    f, h = I.FLASH_DECODE, I.HCA_DECODE
    fl_rows = f.B * ((f.W + f.k) * f.c * 2 + f.H * f.c * 2 + -(-f.n_c // SEGMENT) * f.k * 8)
    hca_rows = h.B * ((h.W + h.n_c) * h.c * 2 + h.H * h.c * 2)
    return [
        ("index_score_segments_flash_decode_b32", ROOFLINE_KERNEL, None, INDEXER_SOURCES,
         index_segments_bytes(f.B, 1, f.n_c, f.H_I, f.d_I, f.k),
         "keys + scales (132 B per entry), q codes + scales + w, positions, 8 x 512 candidate pairs per query"),
        ("attn_select_flash_decode_b32", "attn_bf16<2, 4, 8, 0, false>", None, ATTN_SOURCES, fl_rows,
         "candidate pairs, window + selected rows (1 KiB each), q (the split partials it writes are not counted)"),
        ("attn_merge_flash_decode_b32", "attn_merge_tiles<4>", 32 * 8 * 256, ATTN_SOURCES,
         f.B * f.H * f.c * 2, "the bf16 output (the split partials it reads are not counted)"),
        ("attn_hca_decode_b64", "attn_rows_bf16<1>", None, ATTN_SOURCES, hca_rows,
         "window + every visible entry (1 KiB each), q (the split partials it writes are not counted)"),
        ("compress_fused_prefill_chunk8192_main", COMPRESS_MAIN_KERNEL, None, COMPRESS_SOURCES,
         compress_main_bytes(), "hidden rows of the chunk + the 4 before it, w_proj, bias, pooled vectors written"),
    ]


# The fused compressor kernels of the prefill chunk (main: 256-token tiles; indexer: 64-token tiles)
COMPRESS_MAIN_KERNEL = "compress_fused<csa::FusedShape<4, 2, 4, 2, 64, 2>"
COMPRESS_IDX_KERNEL = "compress_fused<csa::FusedShape<1, 1, 4, 2, 64, 2>"
COMPRESS_SOURCES = ("compress.hip", "entry_store.hpp", "common.hpp")


def compress_main_bytes():
    """Algorithmic bytes of the main compressor's fused kernel on the prefill chunk: bf16
    hidden rows (T + m), bf16 w_proj [4c, d], the fp32 bias, the fp32 pooled vectors."""
    from synthetic import inputs as I
    sh = I.PREFILL
    return (sh.S + sh.m) * sh.d * 2 + 4 * sh.c * sh.d * 2 + 2 * sh.m * sh.c * 4 + (sh.S // sh.m) * sh.c * 4


COUNTER_BENCH_ARGS = "--steps 5 --warmup 2 --no-cpu-baseline --calibrate-copy --eager --subs hca,compressor"


def summarize_counters(fetch_dir, write_dir):
    """Writes profiles/<name>_traffic.txt for every kernel of counter_kernels() from the two
    counter runs: each counter is scaled by what it reads for the plain device copy of
    COPY_BYTES (read and written once) in the same run."""
    import csv
    import glob

    def rows_of(d, counter):
        out = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] == counter:
                    out.append(r)
        return out

    def pick(rows, key, grid=None):
        v = [float(r["Counter_Value"]) for r in rows
             if key in r["Kernel_Name"] and (grid is None or int(float(r.get("Grid_Size", -1))) == grid)]
        if not v:
            raise SystemExit(f"no dispatch of a kernel matching {key!r} (grid {grid})")
        return v

    fr, wr = rows_of(fetch_dir, "FETCH_SIZE"), rows_of(write_dir, "WRITE_SIZE")
    copy_f, copy_w = max(pick(fr, "copyBuffer")), max(pick(wr, "copyBuffer"))      # KiB, the one large copy
    f_scale, w_scale = COPY_BYTES / (copy_f * 1024.0), COPY_BYTES / (copy_w * 1024.0)
    base = "cd /tmp && rocprofv3 --pmc {} --output-format csv -d <dir> -o run -- python3 <repo>/bench.py " + \
        COUNTER_BENCH_ARGS
    for name, kern, grid, sources, alg, what in counter_kernels():
        kf, kw = pick(fr, kern, grid), pick(wr, kern, grid)
        fetch = sum(kf) / len(kf) * 1024.0 * f_scale
        write = sum(kw) / len(kw) * 1024.0 * w_scale
        out = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
        with open(out, "w") as fo:
            fo.write(f"# HBM traffic of {kern} ({name}), from rocprofv3 counters; each counter scaled by\n")
            fo.write("# its reading for a plain 256 MiB device copy in the same run.\n")
            fo.write(f"# fetch run: {base.format('FETCH_SIZE')}\n# write run: {base.format('WRITE_SIZE')}\n")
            if grid is not None:
                fo.write(f"# dispatches of {grid} work-items only\n")
            fo.write(f"copy_fetch_kib = {copy_f:.1f}\ncopy_write_kib = {copy_w:.1f}\n")
            fo.write(f"fetch_scale = {f_scale:.4f}\nwrite_scale = {w_scale:.4f}\n")
            fo.write(f"fetch_kib_per_dispatch = {sum(kf) / len(kf):.1f}  (n={len(kf)})\n")
            fo.write(f"write_kib_per_dispatch = {sum(kw) / len(kw):.1f}  (n={len(kw)})\n")
            fo.write(f"traffic_fetch_bytes = {fetch:.0f}\ntraffic_write_bytes = {write:.0f}\n")
            fo.write(f"traffic_bytes_per_launch = {fetch + write:.0f}\n")
            fo.write(f"algorithmic_bytes_per_launch = {alg}  ({what})\n")
            fo.write(f"traffic_over_algorithmic = {(fetch + write) / alg:.3f}\n")
            fo.write(f"sources = {' + '.join(sources)}\n")
            fo.write(f"sources_sha256 = {sources_sha256(sources)}\n")
        print(open(out).read())


TRACE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
             "python3 <repo>/bench.py")


def summarize_trace(trace_dir, bench_log):
    """Writes profiles/decode_flash_b32_ctx128k_kernel_stats.txt from a kernel trace of the
    default bench command: per-kernel statistics over the whole run (as --stats gives them)
    and, for the roofline kernel, its dispatches split by the phase of the run they belong
    to (the bench line's dispatch_plan), so that the bench's event-timed duration and frac
    can be checked against the trace's own durations of the same launches."""
    import csv
    import glob
    rows = []
    for fn in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    if not rows:
        raise SystemExit("no kernel_trace.csv under " + trace_dir)
    rows.sort()
    line = [ln for ln in open(bench_log).read().splitlines() if ln.startswith("{")][-1]
    res = json.loads(line)
    stats = {}
    for t0, t1, name in rows:
        short = name.split("(")[0].replace("void ", "")
        stats.setdefault(short, []).append((t1 - t0) / 1e3)
    total = sum(sum(v) for v in stats.values())
    rl = [(t1 - t0) / 1e3 for t0, t1, name in rows if ROOFLINE_KERNEL in name]
    plan = res["roofline"]["dispatch_plan"]
    out = os.path.join(ROOT, "profiles", "decode_flash_b32_ctx128k_kernel_stats.txt")
    with open(out, "w") as fo:
        fo.write("# rocprofv3 kernel trace of the default bench run on one MI355X\n")
        fo.write(f"# command: {TRACE_CMD}\n")
        fo.write("# workload: V4-Flash CSA decode step, B=32, 128K context (32768 entries), top-512, H=64 x c=512;\n")
        fo.write(f"#   the timed step = {res['timing']}\n")
        fo.write(f"# bench line of this run (under the tracer): value={res['value']:.0f} tokens/s, "
                 f"ms_per_step={res['ms_per_step']:.4f}, roofline kernel avg_launch_us={res['roofline']['avg_launch_us']:.2f} "
                 f"(in-step, events), frac={res['roofline']['frac']:.3f}\n")
        fo.write(f"\n# {ROOFLINE_KERNEL}: the trace's durations of the same launches, by phase of the run\n")
        i = 0
        for phase, n in plan:
            seg = rl[i:i + n]
            i += n
            if seg:
                fo.write(f"phase {phase:<14} dispatches {len(seg):4d}  avg_us {np.mean(seg):8.2f}  "
                         f"min_us {np.min(seg):8.2f}  max_us {np.max(seg):8.2f}\n")
        if i != len(rl):
            fo.write(f"# note: {len(rl)} dispatches in the trace, {i} in the plan\n")
        ev = dict(plan)
        j = 0
        for phase, n in plan:
            if phase == "event_pass":
                seg = rl[j:j + n]
                tr_us = float(np.mean(seg))
                fo.write(f"event_pass_trace_avg_us = {tr_us:.2f}\n")
                fo.write(f"event_pass_bench_us = {res['roofline']['avg_launch_us']:.2f}  (the bench's events around the "
                         f"same launches)\n")
                fo.write(f"bytes_per_launch = {res['roofline']['bytes_per_launch']}\n")
                fo.write(f"frac_from_trace = {res['roofline']['bytes_per_launch'] / (tr_us * 1e-6) / 1e9 / HBM_PEAK_GBS:.3f}\n")
            j += n
        fo.write("\n# every kernel of the run\n")
        fo.write(f"{'kernel':<60} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>7}\n")
        for name, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
            fo.write(f"{name[:60]:<60} {len(v):6d} {np.mean(v):10.2f} {np.min(v):10.2f} {np.max(v):10.2f} "
                     f"{100 * sum(v) / total:7.2f}\n")
    print(open(out).read())
    if "prefill_compressor" in res:
        summarize_compressor_trace(rows, res)


def summarize_compressor_trace(rows, res):
    """profiles/compress_prefill_chunk8192_kernel_stats.txt: the prefill compressor's kernels in
    the same trace, with the fraction of the bf16 peak from the trace's own durations."""
    from synthetic import inputs as I
    sh = I.PREFILL
    f_main, f_idx = 2.0 * sh.S * sh.d * 4 * sh.c, 2.0 * sh.S * sh.d * 4 * sh.d_I
    out = os.path.join(ROOT, "profiles", "compress_prefill_chunk8192_kernel_stats.txt")
    with open(out, "w") as fo:
        fo.write("# rocprofv3 kernel trace of the default bench run: the prefill compressor sub-benchmark\n")
        fo.write(f"# command: {TRACE_CMD}\n")
        fo.write(f"# workload: one prefill chunk, T = {sh.S} tokens (+{sh.m} before it), d = {sh.d}, overlap, m = {sh.m};\n")
        fo.write(f"#   main KV c = {sh.c} (bf16 rows), indexer K c = {sh.d_I} (FP8 rows + scale)\n")
        pc = res["prefill_compressor"]
        fo.write(f"# bench (events, whole csa_compress call, under the tracer): main_ms={pc['main_ms']:.4f} "
                 f"indexer_ms={pc['indexer_ms']:.4f}\n")
        fo.write("# algorithmic flops: 2 * T * d * 4c (each entry pools 2m slots of (C, Z))\n\n")
        for label, key, fl in (("main", COMPRESS_MAIN_KERNEL, f_main), ("indexer", COMPRESS_IDX_KERNEL, f_idx),
                               ("finish (both)", "compress_pool<true>", None)):
            v = [(t1 - t0) / 1e3 for t0, t1, name in rows if key in name]
            if not v:
                continue
            fo.write(f"{label:<14} {key:<52} calls {len(v):4d}  avg_us {np.mean(v):8.2f}  min_us {np.min(v):8.2f}  "
                     f"max_us {np.max(v):8.2f}\n")
            if fl is not None:
                tf = fl / (np.mean(v) * 1e-6) / 1e12
                fo.write(f"{'':<14} flops_per_launch = {fl:.4e}  tflops_from_trace_avg = {tf:.1f}  "
                         f"frac_bf16_peak = {tf / BF16_PEAK_TFLOPS:.3f}\n")
        fo.write(f"sources = {' + '.join(COMPRESS_SOURCES)}\nsources_sha256 = {sources_sha256(COMPRESS_SOURCES)}\n")
    print(open(out).read())


MFMA_CMD = ("rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
            "--kernel-include-regex index_score_fp8_prefill --output-format csv -d <dir> -o run -- "
            "python3 <repo>/bench.py --steps 2 --warmup 1 --subs prefill --no-cpu-baseline --eager")


class TimingEvents:
    """HIP events created with hipEventDisableSystemFence, recorded on a torch stream through
    the HIP runtime torch has loaded (measurement plumbing: a default event's record adds a
    system-scope release, whose cache write-back lands inside the interval it times)."""
    FLAGS = 0x20000000                       # hipEventDisableSystemFence

    def __init__(self, n):
        import ctypes
        path = None
        for ln in open("/proc/self/maps"):
            if "libamdhip64" in ln:
                path = ln.split()[-1]
                break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.FLAGS)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, stream):
        if self.hip.hipEventRecord(self.ev[i], self.ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def device_info(torch, dev):
    """The GPU the run used and a practical HBM rate: a 1 GiB device-to-device copy (read +
    write), timed with events, best of 5."""
    props = torch.cuda.get_device_properties(dev)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(5):
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del a, b
    info = {"name": props.name, "compute_units": props.multi_processor_count,
            "memory_gib": round(props.total_memory / (1 << 30), 1),
            "copy_1gib_gbs": 2 * n / (best * 1e-3) / 1e9}
    for key in ("gcnArchName", "clock_rate", "L2_cache_size"):
        if hasattr(props, key):
            info[key] = getattr(props, key)
    return info


def summarize_mfma(counter_dir, bench_log):
    """Writes profiles/index_score_prefill_chunk8192_mfma.txt: MFMA utilisation and MFMA
    flops of the prefill indexer from rocprofv3 counters (MfmaUtil = busy MFMA cycles over
    all SIMDs / (active GPU cycles x SIMDs)), beside the same run's event-timed duration."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "index_score_fp8_prefill" in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no index_score_fp8_prefill dispatch in the counter files")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    n = len(vals.get("MfmaUtil", []))
    line = [ln for ln in open(bench_log).read().splitlines() if ln.startswith("{")][-1]
    pf = json.loads(line)["prefill_indexer"]
    flops = mean["MfmaFlopsBF16"]
    out = os.path.join(ROOT, "profiles", "index_score_prefill_chunk8192_mfma.txt")
    with open(out, "w") as fo:
        fo.write("# MFMA use of index_score_fp8_prefill, CSA prefill chunk (8192 queries x 34816 entries,\n")
        fo.write("# 64 heads x 128, FP8 codes contracted on bf16 MFMA), from rocprofv3 counters; the\n")
        fo.write("# duration is the same run's event timing of the prefill sub-benchmark.\n")
        fo.write(f"# command: cd /tmp && {MFMA_CMD}\n")
        fo.write(f"dispatches = {n}\n")
        fo.write(f"mfma_util_percent = {mean['MfmaUtil']:.1f}\n")
        fo.write(f"mfma_busy_cycles_all_simds = {mean['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}\n")
        fo.write(f"grbm_gui_active = {mean['GRBM_GUI_ACTIVE']:.4g}\n")
        fo.write(f"mfma_flops_bf16_per_dispatch = {flops:.4g}\n")
        fo.write(f"algorithmic_flops_causal = {pf['causal_flops']:.4g}\n")
        fo.write(f"event_ms = {pf['ms']:.4f}\n")
        fo.write(f"counter_tflops = {flops / (pf['ms'] * 1e-3) / 1e12:.1f}  (peak bf16 {BF16_PEAK_TFLOPS:.0f})\n")
        fo.write(f"algorithmic_tflops = {pf['tflops']:.1f}\n")
    print(open(out).read())


def main():
    args = parse()
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the CSA hot path here runs on one GPU; sharding over several GPUs "
                                   "is not launched", "n_gpus": args.gpus}))
        sys.exit(2)
    subs = [x for x in args.subs.split(",") if x]
    for x in subs:
        if x not in ALL_SUBS:
            raise SystemExit(f"unknown sub-benchmark {x!r}; choose from {','.join(ALL_SUBS)}")
    import torch
    from compressed_sparse_kv_amd import binding as L
    from synthetic import inputs as I

    torch.cuda.set_device(0)
    sh = I.FLASH_DECODE
    dev = torch.device("cuda")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def up_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    t_gen = time.time()
    host_sets, sets = [], []
    for i in range(args.sets):
        a = I.decode_inputs(sh, seed=sh.seed + 100 * i).arrays
        host_sets.append(a)
        sets.append({
            "kv": up_bf16(a["kv_comp_bf16"]), "swa": up_bf16(a["swa_bf16"]), "q": up_bf16(a["q_bf16"]),
            "sink": up(a["sink"]), "pos": up(a["q_pos"]), "k8": up(a["kI_fp8"]), "ks": up(a["kI_scale"]),
            "q8": up(a["qI_fp8"]), "qs": up(a["qI_scale"]), "w": up(a["w"]),
        })
    t_gen = time.time() - t_gen

    B, Nc, k = sh.B, sh.n_c, sh.k
    scores = torch.empty(B, 1, Nc, device=dev)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=dev)
    out = torch.empty(B, 1, sh.H, sh.c, dtype=torch.bfloat16, device=dev)
    tk_ws = torch.empty(L.topk_workspace_size(B, Nc, k), dtype=torch.uint8, device=dev)
    at_ws_n = L.attn_workspace_size(B, 1, sh.H, sh.c, sh.W + k, L.CSA_BF16)
    at_ws = torch.empty(max(at_ws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    cand = torch.empty(L.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device=dev)
    # Each set's key cache in the 16-entry blocked layout.  The compressors write this layout
    # themselves: csa_compress (prefill chunks) and csa_compress_decode (one entry per block
    # boundary) with CSA_LAYOUT_B16, the same bytes as this re-layout (tested); the
    # synthetic precompressed cache here is laid out once per set before timing.
    for s in sets:
        s["k16"] = L.csa_index_keys_b16(s["k8"], torch.empty(L.index_keys_b16_size(B, Nc), dtype=torch.uint8,
                                                             device=dev))
    torch.cuda.synchronize()

    def score_segments(s):
        L.csa_index_score_segments_b16(s["q8"], s["qs"], s["w"], s["k16"], s["ks"], s["pos"], m=sh.m, k=k,
                                       cand=cand)

    def step(i):
        # scores with each 4096-entry segment's top-k, then the attention over the k best
        # of each row's candidates (selection and attention in one call)
        s = sets[i % len(sets)]
        score_segments(s)
        L.csa_topk_sparse_attn(s["q"], s["kv"], cand, s["swa"], s["sink"], k=k, W=sh.W, out=out, ws=at_ws)

    def step_separate(i):
        # the same step with the scores written out and csa_topk over them
        s = sets[i % len(sets)]
        L.csa_index_score(s["q8"], s["qs"], s["w"], s["k8"], s["ks"], s["pos"], m=sh.m, scores=scores)
        L.csa_topk(scores, k, idx, ws=tk_ws)
        L.csa_sparse_attn(s["q"], s["kv"], idx, s["swa"], s["sink"], W=sh.W, out=out, ws=at_ws)

    def stage_step(i, ev):
        # the step's calls with events between them, the same stages as three calls
        # (merge, attention over idx), then the separate-stage calls
        s = sets[i % len(sets)]
        ev[0].record(stream)
        score_segments(s)
        ev[1].record(stream)
        L.csa_topk_sparse_attn(s["q"], s["kv"], cand, s["swa"], s["sink"], k=k, W=sh.W, out=out, ws=at_ws)
        ev[2].record(stream)
        L.csa_topk_merge(cand, B, 1, Nc, k, idx)
        ev[3].record(stream)
        L.csa_sparse_attn(s["q"], s["kv"], idx, s["swa"], s["sink"], W=sh.W, out=out, ws=at_ws)
        ev[4].record(stream)
        L.csa_index_score(s["q8"], s["qs"], s["w"], s["k8"], s["ks"], s["pos"], m=sh.m, scores=scores)
        ev[5].record(stream)
        L.csa_topk(scores, k, idx, ws=tk_ws)
        ev[6].record(stream)

    plan = []                                   # launches of the roofline kernel, by phase, in order
    for i in range(args.warmup):
        step(i)
    plan.append(("warmup", args.warmup))
    torch.cuda.synchronize()
    if args.calibrate_copy:
        a_ = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        b_ = torch.empty_like(a_)
        b_.copy_(a_)
        torch.cuda.synchronize()
        del a_, b_
    # eager: exactly K steps between two synchronisations, one library call per stage
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1) / args.steps
    plan.append(("timed", args.steps))

    # the same step through csa_index_score + csa_topk (informational; not `value`)
    for i in range(args.warmup):
        step_separate(i)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step_separate(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_separate = t0.elapsed_time(t1) / args.steps

    # graph: each input set's step captured once (same calls, same buffers) and replayed;
    # again exactly K steps between two synchronisations (reported beside the eager time)
    ms_graph = None
    if not args.eager:
        graphs = []
        for i in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(len(sets)):
            graphs[i].replay()
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            graphs[i % len(sets)].replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_graph = t0.elapsed_time(t1) / args.steps
        plan.append(("graph", len(sets) + args.steps))
    ms_per_step = ms_eager

    # the dominant kernel inside the step: K more steps with a pair of timing events around
    # each of its launches, on its stream.  The events skip the system-scope fence a default
    # event adds when it is recorded (a cache write-back that would be timed with the kernel).
    hev = TimingEvents(2 * args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        s = sets[i % len(sets)]
        hev.record(2 * i, stream)
        score_segments(s)
        hev.record(2 * i + 1, stream)
        L.csa_topk_sparse_attn(s["q"], s["kv"], cand, s["swa"], s["sink"], k=k, W=sh.W, out=out, ws=at_ws)
    torch.cuda.synchronize()
    is_us = float(np.mean([hev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)])) * 1e3
    hev.destroy()
    plan.append(("event_pass", args.steps))

    # per-stage durations (separate pass with events between the stages)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        stage_step(i, evs[i])
    torch.cuda.synchronize()
    dur = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(6)] for e in evs])
    us = dur.mean(axis=0) * 1e3
    plan.append(("stage_pass", args.steps))

    # the dominant kernel alone, back to back (rotating input sets): no attention between
    # its launches, so the chip runs it at the clock a continuous stream of it allows
    n_rl = max(args.steps, 20)
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record(stream)
    for i in range(n_rl):
        score_segments(sets[i % len(sets)])
    r1.record(stream)
    torch.cuda.synchronize()
    b2b_us = r0.elapsed_time(r1) / n_rl * 1e3
    plan.append(("back_to_back", n_rl))

    isb = index_segments_bytes(B, 1, Nc, sh.H_I, sh.d_I, k)
    achieved = isb / (is_us * 1e-6) / 1e9
    step_bytes = decode_step_bytes(sh)
    result = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "timing": "eager launches: csa_index_score_segments_b16, csa_topk_sparse_attn",
        "ms_per_step_separate_stages": ms_separate,
        "ms_per_step_graph": ms_graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-storage/bf16-mfma",
        "data": "synthetic",
        "config": {"workload": sh.name, "batch": B, "context_tokens": sh.t + 1, "ratio_m": sh.m,
                   "entries": Nc, "top_k": k, "heads": sh.H, "head_dim": sh.c, "indexer_heads": sh.H_I,
                   "indexer_dim": sh.d_I, "window": sh.W, "input_sets": args.sets},
        "hbm_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_bytes": step_bytes,
        "step_frac_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stages_us": {"csa_index_score_segments": us[0], "csa_topk_sparse_attn": us[1], "csa_topk_merge": us[2],
                      "csa_sparse_attn": us[3], "csa_index_score": us[4], "csa_topk": us[5]},
        "roofline": {"kernel": ROOFLINE_KERNEL, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(INDEXER_SOURCES, "index_score_segments_flash_decode_b32"),
                     "bytes_per_launch": isb, "avg_launch_us": is_us,
                     "timing": "HIP events (no system-scope fence) around each launch inside K steps, on its stream",
                     "avg_launch_us_back_to_back": b2b_us,
                     "frac_back_to_back": isb / (b2b_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "dispatch_plan": plan},
        "input_generation_s": t_gen,
        # (not under --calibrate-copy: its copy must stay the only large one of a counter run)
        "device": None if args.calibrate_copy else device_info(torch, dev),
    }

    if "prefill" in subs:
        result["prefill_indexer"], pf_scores = bench_prefill_indexer(torch, L, I, dev)
        result["prefill_topk"] = bench_prefill_topk(torch, L, pf_scores, I.PREFILL.k)
        del pf_scores
    if "pro" in subs:
        result["pro_decode"] = bench_csa_decode(torch, L, I, dev, I.PRO_DECODE, n_sets=2)
    if "hca" in subs:
        result["hca_decode"] = bench_hca_decode(torch, L, I, dev)
    if "compressor" in subs:
        result["prefill_compressor"] = bench_prefill_compressor(torch, L, I, dev)
    if "prefill_attention" in subs:
        result["prefill_attention"] = bench_prefill_attention(torch, L, I, dev)
    if "decode_layer" in subs:
        result["decode_layer"] = bench_decode_layer(torch, L, I, dev, sets, cand, at_ws)
        plan.append(("decode_layer", 21))

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host_sets, sh)

    print(json.dumps(result))


# Sources compiled into the indexer kernel: its counter summary is valid only for them.
INDEXER_SOURCES = ("index_score.hip", "select.hpp", "common.hpp")


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "compressed_sparse_kv_amd", "csrc", n), "rb").read())
    return h.hexdigest()


def measured_traffic(sources, name):
    """HBM bytes per launch from the committed counter summary profiles/<name>_traffic.txt, or
    None when a source of the kernel has changed since the counters were taken (the summary
    records the sha256 of the sources it measured)."""
    summary = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(summary):
        return None
    fields = {}
    for line in open(summary):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            fields[k.strip()] = v.strip()
    if fields.get("sources_sha256") != sources_sha256(sources) or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def _timed(torch, fn, reps):
    fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_csa_decode(torch, L, I, dev, sh, n_sets=2, reps=20):
    """One CSA decode step (scores -> top-k -> attention) of another decode shape."""
    sets = []
    for i in range(n_sets):
        a = I.decode_inputs(sh, seed=sh.seed + 100 * i).arrays
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        upb = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        sets.append({"kv": upb(a["kv_comp_bf16"]), "swa": upb(a["swa_bf16"]), "q": upb(a["q_bf16"]),
                     "sink": up(a["sink"]), "pos": up(a["q_pos"]), "k8": up(a["kI_fp8"]), "ks": up(a["kI_scale"]),
                     "q8": up(a["qI_fp8"]), "qs": up(a["qI_scale"]), "w": up(a["w"])})
        del a
    B, Nc, k = sh.B, sh.n_c, sh.k
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=dev)
    out = torch.empty(B, 1, sh.H, sh.c, dtype=torch.bfloat16, device=dev)
    it_ws = torch.empty(max(1, L.index_topk_workspace_size(B, 1, Nc, k)), dtype=torch.uint8, device=dev)
    at_ws = torch.empty(max(1, L.attn_workspace_size(B, 1, sh.H, sh.c, sh.W + k, L.CSA_BF16)), dtype=torch.uint8,
                        device=dev)

    cand = torch.empty(L.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        L.csa_index_topk(s["q8"], s["qs"], s["w"], s["k8"], s["ks"], s["pos"], m=sh.m, k=k, idx=idx, ws=it_ws)
        L.csa_sparse_attn(s["q"], s["kv"], idx, s["swa"], s["sink"], W=sh.W, out=out, ws=at_ws)

    def step_fused(i):
        # the headline step's two calls: scores with segment top-k, then (first merge
        # level,) selection and attention in one call
        s = sets[i % len(sets)]
        L.csa_index_score_segments(s["q8"], s["qs"], s["w"], s["k8"], s["ks"], s["pos"], m=sh.m, k=k, cand=cand)
        L.csa_topk_sparse_attn(s["q"], s["kv"], cand, s["swa"], s["sink"], k=k, W=sh.W, out=out, ws=at_ws)

    ms = _timed(torch, step, reps)
    ms_fused = _timed(torch, step_fused, reps)
    byts = decode_step_bytes(sh)
    return {"workload": sh.name, "tokens_per_s": B / (ms * 1e-3), "ms_per_step": ms, "step_bytes": byts,
            "hbm_gbs": byts / (ms * 1e-3) / 1e9, "input_sets": n_sets,
            "ms_per_step_segments_then_fused_attention": ms_fused}


def bench_hca_decode(torch, L, I, dev, reps=20):
    """HCA decode: dense attention of 64 queries over 8192 compressed entries (1M context) + window."""
    sh = I.HCA_DECODE
    a = I.decode_inputs(sh, with_indexer=False).arrays
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    upb = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    kv, swa, q, sink, pos = upb(a["kv_comp_bf16"]), upb(a["swa_bf16"]), upb(a["q_bf16"]), up(a["sink"]), up(a["q_pos"])
    del a
    out = torch.empty(sh.B, 1, sh.H, sh.c, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, L.attn_workspace_size(sh.B, 1, sh.H, sh.c, sh.W + sh.n_c, L.CSA_BF16)), dtype=torch.uint8,
                     device=dev)
    ms = _timed(torch, lambda i: L.hca_dense_attn(q, kv, pos, swa, sink, m=sh.m, W=sh.W, out=out, ws=ws), reps)
    byts = sh.B * (sh.n_c + sh.W) * sh.c * 2 + 2 * sh.B * sh.H * sh.c * 2 + sh.H * 4 + sh.B * 8
    flops = 4.0 * sh.B * sh.H * (sh.n_c + sh.W) * sh.c
    return {"workload": sh.name, "tokens_per_s": sh.B / (ms * 1e-3), "ms_per_step": ms, "bytes": byts,
            "hbm_gbs": byts / (ms * 1e-3) / 1e9, "frac_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tflops": flops / (ms * 1e-3) / 1e12}


def bench_prefill_attention(torch, L, I, dev, reps=5):
    """CSA attention over one prefill chunk: 8192 queries, each its 128-token window and
    512 selected entries of the 32768 context entries (a seeded random selection)."""
    sh = I.PREFILL
    n_ctx = sh.ctx // sh.m
    Ls = sh.S + sh.W - 1
    a = I.attention_inputs(sh.seed + 7, 1, sh.S, n_ctx, Ls)
    upb = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q, kv, swa, sink = upb(a["q_bf16"]), upb(a["kv_comp_bf16"]), upb(a["swa_bf16"]), up(a["sink"])
    del a
    g = torch.Generator(device=dev)
    g.manual_seed(sh.seed + 8)
    r = torch.rand(sh.S, n_ctx, generator=g, device=dev)
    idx = r.topk(sh.k, dim=1).indices.sort(dim=1).values.to(torch.int32).view(1, sh.S, sh.k).contiguous()
    del r
    out = torch.empty(1, sh.S, sh.H, sh.c, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, L.attn_workspace_size(1, sh.S, sh.H, sh.c, sh.W + sh.k, L.CSA_BF16)), dtype=torch.uint8,
                     device=dev)
    ms = _timed(torch, lambda i: L.csa_sparse_attn(q, kv, idx, swa, sink, W=sh.W, out=out, ws=ws), reps)
    flops = 4.0 * sh.S * sh.H * (sh.W + sh.k) * sh.c          # q.k and p.v over every row
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": "csa_prefill_chunk8192_attention_k512_w128", "ms": ms, "flops": flops,
            "tflops": tflops, "frac_bf16_peak": tflops / BF16_PEAK_TFLOPS,
            "note": "P enters P.V as bf16 hi + lo: the MFMA work is 1.5x these flops"}


def bench_prefill_compressor(torch, L, I, dev, reps=20):
    """Compressor over one prefill chunk: 8192 new tokens (+4 from the previous block), d = 5120,
    main KV (c = 512, bf16 out) and indexer K (c = 128, FP8 out)."""
    sh = I.PREFILL
    a = I.prefill_inputs(sh)
    upb = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    hid, prev = upb(a["hidden_bf16"]), upb(a["hidden_prev_bf16"])
    Wm, Wi = upb(np.ascontiguousarray(a["W_main_bf16"].T)), upb(np.ascontiguousarray(a["W_idx_bf16"].T))
    Bm, Bi = up(a["B_main"]), up(a["B_idx"])
    del a
    n = sh.S // sh.m
    kv = torch.empty(1, n, sh.c, dtype=torch.bfloat16, device=dev)
    kI = torch.empty(1, n, sh.d_I, dtype=torch.uint8, device=dev)
    kIs = torch.empty(1, n, device=dev)
    kw = dict(overlap=True, m=sh.m, d_rope=sh.d_rope, rope_theta=sh.rope_theta, rms_eps=1e-6, p0=sh.ctx)
    ws = torch.empty(L.compress_workspace_size(1, sh.S, sh.m, sh.c, True, True), dtype=torch.uint8, device=dev)
    ms_m = _timed(torch, lambda i: L.csa_compress(hid, prev, Wm, Bm, c=sh.c, out=kv, ws=ws, **kw), reps)
    ms_i = _timed(torch, lambda i: L.csa_compress(hid, prev, Wi, Bi, c=sh.d_I, out=kI, out_scale=kIs, ws=ws, **kw),
                  reps)
    # each entry pools 2m slots of (C, Z): 4c projected values per token of the chunk
    f_m, f_i = 2.0 * sh.S * sh.d * 4 * sh.c, 2.0 * sh.S * sh.d * 4 * sh.d_I
    return {"workload": "csa_prefill_chunk8192_d5120_compressor", "main_ms": ms_m, "indexer_ms": ms_i,
            "main_tflops": f_m / (ms_m * 1e-3) / 1e12, "indexer_tflops": f_i / (ms_i * 1e-3) / 1e12,
            "main_frac_bf16_peak": f_m / (ms_m * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "indexer_frac_bf16_peak": f_i / (ms_i * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def bench_prefill_indexer(torch, L, I, dev, reps=10):
    """Indexer over one prefill chunk: 8192 queries (positions 131072..139263) x 34816 entries."""
    sh = I.PREFILL
    n = sh.ctx // sh.m + sh.S // sh.m
    a = I.indexer_inputs(sh.seed, 1, sh.S, n)
    pos = (sh.ctx + np.arange(sh.S, dtype=np.int64))[None]
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q8, qs, w, k8, ks, qp = up(a["qI_fp8"]), up(a["qI_scale"]), up(a["w"]), up(a["kI_fp8"]), up(a["kI_scale"]), up(pos)
    scores = torch.empty(1, sh.S, n, device=dev)
    for _ in range(2):
        L.csa_index_score(q8, qs, w, k8, ks, qp, m=sh.m, scores=scores)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.csa_index_score(q8, qs, w, k8, ks, qp, m=sh.m, scores=scores)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nvis = np.minimum(n, (pos[0] + 1) // sh.m)
    flops = float(np.sum(nvis)) * sh.H_I * sh.d_I * 2
    tflops = flops / (ms * 1e-3) / 1e12
    res = {"workload": "csa_prefill_chunk8192_ctx128k_indexer", "ms": ms, "causal_flops": flops,
           "tflops": tflops, "frac_fp8_peak": tflops / FP8_PEAK_TFLOPS,
           "frac_bf16_peak": tflops / BF16_PEAK_TFLOPS,
           "note": "contraction on bf16 MFMA (exact e4m3->bf16); FP8 MFMA accumulation misses the 1e-5 bound"}
    return res, scores


def bench_prefill_topk(torch, L, scores, k, reps=5):
    """Top-k of the prefill chunk: the indexer's 8192 x 34816 scores (causal -inf tails) ->
    8192 x 512 indices; every score is read once (the HBM bound)."""
    rows, n = scores.shape[1], scores.shape[2]
    idx = torch.empty(1, rows, k, dtype=torch.int32, device=scores.device)
    ws = torch.empty(max(1, L.topk_workspace_size(rows, n, k)), dtype=torch.uint8, device=scores.device)
    L.csa_topk(scores, k, idx, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.csa_topk(scores, k, idx, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    byts = scores.numel() * 4 + idx.numel() * 4
    return {"workload": "csa_prefill_chunk8192_topk512", "ms": ms, "rows": rows, "entries": n,
            "bytes": byts, "hbm_gbs": byts / (ms * 1e-3) / 1e9, "frac_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_decode_layer(torch, L, I, dev, sets, cand, at_ws, reps=20):
    """The whole CSA decode layer step after the dense projections (V4-Flash shapes, hidden
    d = 5120): the new token's compressor step for the main KV (bf16 rows into the KV
    cache) and for the indexer key (FP8 appended straight into the 16-entry blocked key
    cache), the scores with each segment's top-k, and the selection + sparse attention with
    the inverse-RoPE epilogue.  Position t = 131071 completes block 32767, so every step
    emits one entry into each cache (entry 32767, which the query sees)."""
    sh = I.FLASH_DECODE
    B, Nc, k, m, c, dI, W = sh.B, sh.n_c, sh.k, sh.m, sh.c, sh.d_I, sh.W
    d = I.PREFILL.d
    a = I.decode_layer_inputs(sh.seed + 900, B, d, m, c, dI)
    upb = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    hid, prime = upb(a["hidden_bf16"]), upb(a["prime_bf16"])
    Wm, Bm, Wi, Bi = upb(a["W_main_t_bf16"]), up(a["B_main"]), upb(a["W_idx_t_bf16"]), up(a["B_idx"])
    st_m = [torch.empty(L.compress_state_size(B, m, c, True), dtype=torch.uint8, device=dev) for _ in sets]
    st_i = [torch.empty(L.compress_state_size(B, m, dI, True), dtype=torch.uint8, device=dev) for _ in sets]
    ws_m = torch.empty(L.compress_decode_workspace_size(B, d, c, True), dtype=torch.uint8, device=dev)
    ws_i = torch.empty(L.compress_decode_workspace_size(B, d, dI, True), dtype=torch.uint8, device=dev)
    kw = dict(overlap=True, m=m, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    t = sh.t
    pos_t = torch.full((B,), t, dtype=torch.int64, device=dev)
    # both compressors of the layer in one call (one projection launch, one step launch)
    comps = [L.decode_compressors(B, [dict(w_proj=Wm, bias=Bm, state=st_m[si], cache=s["kv"], c=c, **kw),
                                      dict(w_proj=Wi, bias=Bi, state=st_i[si], cache=s["k16"], c=dI,
                                           cache_scale=s["ks"], layout=L.CSA_LAYOUT_B16, Nc_max=Nc, **kw)])
             for si, s in enumerate(sets)]
    ws_2 = torch.empty(L.compress_decode_many_workspace_size(B, d, L.CSA_BF16, comps[0]), dtype=torch.uint8,
                       device=dev)

    def compress(si, h, pos, emit=True):
        L.csa_compress_decode_many(h, pos, comps[si], emit=emit, ws=ws_2)

    def compress_two_calls(si, h, pos, emit=True):
        s = sets[si]
        L.csa_compress_decode(h, Wm, Bm, pos, st_m[si], s["kv"], c=c, emit=emit, ws=ws_m, **kw)
        L.csa_compress_decode(h, Wi, Bi, pos, st_i[si], s["k16"], c=dI, cache_scale=s["ks"],
                              layout=L.CSA_LAYOUT_B16, Nc_max=Nc, emit=emit, ws=ws_i, **kw)

    # each set's rings hold the previous block and the first 2m - 1 - m tokens of this one
    for si in range(len(sets)):
        for r in range(2 * m - 1):
            compress(si, prime[:, r].contiguous(), torch.full((B,), t - (2 * m - 1) + r, dtype=torch.int64,
                                                               device=dev), emit=False)
    torch.cuda.synchronize()

    out = torch.empty_like(sets[0]["q"])

    def step(i):
        si = i % len(sets)
        s = sets[si]
        compress(si, hid, pos_t)
        L.csa_index_score_segments_b16(s["q8"], s["qs"], s["w"], s["k16"], s["ks"], s["pos"], m=m, k=k, cand=cand)
        L.csa_topk_sparse_attn(s["q"], s["kv"], cand, s["swa"], s["sink"], k=k, W=W, out=out, q_pos=s["pos"],
                               inv_rope_d=64, ws=at_ws)

    ms = _timed(torch, step, reps)
    ms_c = _timed(torch, lambda i: compress(i % len(sets), hid, pos_t), reps)
    ms_c2 = _timed(torch, lambda i: compress_two_calls(i % len(sets), hid, pos_t), reps)
    w_bytes = (4 * c + 4 * dI) * d * 2
    ring = B * (2 * m * 2 * c + 2 * c + 2 * m * 2 * dI + 2 * dI) * 4     # the 2m slots read, the new one written
    comp_bytes = w_bytes + 2 * B * d * 2 + ring + B * (c * 2 + dI + 4)
    byts = decode_step_bytes(sh) + comp_bytes
    return {"workload": "v4flash_csa_decode_layer_b32_ctx128k_d5120",
            "steps": "csa_compress_decode_many (main compressor, bf16 rows + indexer compressor, FP8, blocked "
                     "layout) + csa_index_score_segments_b16 + csa_topk_sparse_attn (inverse RoPE 64)",
            "tokens_per_s": B / (ms * 1e-3), "ms_per_step": ms, "step_bytes": byts,
            "hbm_gbs": byts / (ms * 1e-3) / 1e9, "frac_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "compressor_us": ms_c * 1e3, "compressor_us_two_calls": ms_c2 * 1e3, "compressor_bytes": comp_bytes,
            "compressor_hbm_gbs": comp_bytes / (ms_c * 1e-3) / 1e9}


def cpu_baseline(host_sets, sh):
    """The CPU oracle, as it stands, on every query of the rotated input sets (all host
    cores), and on 8 of them with one thread."""
    import math
    import platform
    from oracle import csa_oracle as O

    def one(a, b):
        qI = O.dequant_rows(a["qI_fp8"][b:b + 1], a["qI_scale"][b:b + 1])
        KI = O.dequant_rows(a["kI_fp8"][b:b + 1], a["kI_scale"][b:b + 1])
        sc = O.index_scores(qI, a["w"][b:b + 1], KI, a["q_pos"][b:b + 1], sh.m)
        idx = O.topk_indices(sc, sh.k)
        O.sparse_attention(O.bf16_bits_to_f64(a["q_bf16"][b:b + 1]), O.bf16_bits_to_f64(a["kv_comp_bf16"][b:b + 1]),
                           idx, O.bf16_bits_to_f64(a["swa_bf16"][b:b + 1]), a["sink"], 1 / math.sqrt(sh.c),
                           a["q_pos"][b:b + 1], sh.W)

    threads = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
    t = time.time()
    nq = 0
    for a in host_sets:
        for b in range(sh.B):
            one(a, b)
            nq += 1
    el = time.time() - t
    res = {"value": nq / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{nq} decode queries ({len(host_sets)} input sets x batch {sh.B}): "
                     f"scores over {sh.n_c} entries, top-{sh.k}, attention over {sh.k}+{sh.W} rows; {el:.1f} s"}
    try:
        res["nproc"] = len(os.sched_getaffinity(0))
    except Exception:
        res["nproc"] = os.cpu_count()
    model = platform.processor()
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    res["cpu_model"] = model
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t = time.time()
            for b in range(8):
                one(host_sets[0], b)
            el1 = time.time() - t
        res["value_1thread"] = 8 / el1
        res["sample_1thread"] = f"8 decode queries of input set 0 with one BLAS thread: {el1:.1f} s"
    return res


if __name__ == "__main__":
    main()
