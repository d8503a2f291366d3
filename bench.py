"""Benchmark of the 4-bit paged KV cache decode path on one MI355X.

One step = one decode step of a Qwen3.8-27B-shaped attention stack ("SGLang's
4-bit KV cache: the 56% is exact, the 1.78x is untested", per-token table: 16
full-attention layers x 4 KV heads x head dim 256; 24 query heads as a stated
workload choice): for each of the 16 layers, quantize-store the new token's
K/V of every sequence into its NVFP4 cache (kvq_quantize_store), then run paged
decode attention over the whole cached context (kvq_decode_attention: split
decode kernel + log-sum-exp merge).  Each layer has its own 1.2 GB pool, so no
pool stays in the 256 MB Infinity Cache between uses.

Printed: one JSON line.  value = effective KV GB/s of the step (packed codes +
scales of every cached token attended, summed over the 16 layers, divided by
the step time); tokens/s = batch / step time (attention only: no weights).
`roofline` prices the decode-attention call (decode + merge kernels) against
the 8 TB/s HBM peak with its algorithmic bytes; `cpu_baseline` times the CPU
oracle on a sample of the same cache.  Secondary workloads (160K shuffled
pages with chunked-prefill store, 1M split-context with prefix dequant, INT4
at 220K) are reported under "secondary".

Inputs are synthetic and seeded: K, V = exp(N(0,1)) per-(head, channel)
scale x N(0,1) in bf16 (t4 / sqrt(2) for INT4), q ~ N(0,1) bf16, generated on
the GPU with torch's generator.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn effective KV GB/s & % HBM roofline; tokens/s at 32K/160K/1M ctx"

# fmt, batch, context, page size, shuffled pages, query heads, KV heads, head dim
WORKLOADS = {
    "ctx32k": dict(fmt=1, batch=32, ctx=32768, page=16, shuffled=False, kind="lognormal",
                   desc="Qwen3.8-27B-shaped NVFP4 decode step: 16 layers x 4 KV heads x D256, 24 q heads, "
                        "batch 32, context 32,768, 16-token pages"),
    "ctx160k": dict(fmt=1, batch=4, ctx=160000, page=16, shuffled=True, kind="lognormal", chunk=64,
                    desc="NVFP4, batch 4, context 160,000, shuffled page tables, plus a 64-token "
                         "chunked-prefill quantize-store per sequence"),
    "ctx1m": dict(fmt=1, batch=1, ctx=1048576, page=16, shuffled=False, kind="lognormal", prefix=True,
                  split_sweep=(32, 64, 128, 256, 512),
                  desc="NVFP4, batch 1, context 1,048,576, split-context decode; plus kvq_dequant_prefix of "
                       "the full prefix into a bf16 workspace of 1,048,576 + 4,096 rows"),
    "int4_220k": dict(fmt=2, batch=8, ctx=220000, page=1600, shuffled=False, kind="student_t", fused_extend=True,
                      desc="INT4 per-token-head, batch 8, context 220,000, 1,600-token pages (last page half "
                           "full); 16 layers assumed; plus the fused extend of a 4,096-token chunk over the "
                           "first sequence's cached prefix"),
    "rot_32k": dict(fmt=1, batch=32, ctx=32768, page=16, shuffled=False, kind="lognormal", rotated=True,
                    desc="the 32K headline shape with a Hadamard-rotated NVFP4 cache: rotated stores, R q in, "
                         "R o rotated back (the decode call here includes both rotations)"),
    "fp8_32k": dict(fmt=3, batch=32, ctx=32768, page=16, shuffled=False, kind="lognormal",
                    desc="comparator: the 32K headline shape with an FP8 E4M3 per-tensor cache (512 B per "
                         "token and head against NVFP4's 288 B)"),
    "ext32k": dict(fmt=1, batch=1, ctx=32768, page=16, shuffled=False, kind="lognormal", prefix=True,
                   desc="extend only (profiling): NVFP4, batch 1, a 32,768-token cached prefix, prefix dequant, "
                        "then a 4,096-token chunk through the workspace and the fused extend"),
    "k8v4_32k": dict(fmt=4, batch=32, ctx=32768, page=16, shuffled=False, kind="lognormal",
                     desc="split precision: the 32K headline shape with FP8 keys and NVFP4 values (400 B per "
                          "token and head)"),
}
LAYERS, HKV, HQ, D = 16, 4, 24, 256


def token_head_bytes(fmt: int) -> int:
    # packed codes + scales of one token in one KV head, K and V
    if fmt == 3:
        return 2 * D  # FP8: one byte per value, per-tensor scales
    if fmt == 4:
        return D + D // 2 + D // 16  # FP8 keys, NVFP4 values
    return 2 * (D // 2 + (D // 16 if fmt == 1 else 4))


# ------------------------------------------------------------------ profiler summaries
# The decode call's HBM traffic comes from two rocprofv3 counter passes over a
# short run of the headline workload (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by what the same counter reads for a plain 1 GiB
# device copy in the same run.  The summary records a digest of the decode
# kernel's sources; once they change, the recorded traffic no longer applies
# and the bench reports null.
REPO = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ["bit_quantized_kv_amd/csrc/kvq_decode.hip", "bit_quantized_kv_amd/csrc/kvq_device.h",
                  "bit_quantized_kv_amd/csrc/kvq_launch.h"]
PMC_RUN = ('cd /tmp && export TMPDIR=/tmp && cd "$GRAFT_REPO_ROOT" && timeout -s KILL 200 rocprofv3 --pmc {counter} '
           '--output-format csv -d gpurun_out/pmc_{tag} -o run -- python -u bench.py --workload {workload} '
           '--secondary "" --no-cpu-baseline --no-quality --steps 5 --warmup 1 --layers 2 --copy-calibration-gib 1')
CALIB_BYTES = 4 << 30  # bytes read (and written) by one kvq_stream_copy of the copy ceiling


def decode_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(REPO, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counters_path(workload: str) -> str:
    fmt = {1: "nvfp4", 2: "int4", 3: "fp8", 4: "k8v4"}[WORKLOADS[workload]["fmt"]]
    return os.path.join(REPO, "profiles", f"decode_{fmt}_{workload}_counters.md")


def load_counter_summary(workload: str):
    """The recorded traffic of the decode call, if its kernel sources are unchanged."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None, "counter summary without a json block"
    rec = json.loads(text[start + 7:text.index("```", start + 7)])
    if rec.get("decode_source_digest") != decode_source_digest():
        return None, "decode kernel changed since the counters were taken"
    return rec, os.path.relpath(path, REPO)


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str) -> str:
    """Markdown summary of the FETCH_SIZE / WRITE_SIZE passes (see PMC_RUN)."""
    per = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _csv_rows(directory, "counter_collection.csv") if r["Counter_Name"] == counter]
        def avg(pred):
            v = [float(r["Counter_Value"]) for r in rows if pred(r)]
            return (sum(v) / len(v), len(v)) if v else (None, 0)
        # the decode call of the workload's own split plan: the most frequent
        # decode grid (a split sweep adds other grids), and the merge launched with it
        grids = [int(r["Grid_Size"]) for r in rows if "decode_kernel" in r["Kernel_Name"]]
        main_grid = max(set(grids), key=grids.count)
        n_main = grids.count(main_grid)
        merges = [int(r["Grid_Size"]) for r in rows if "merge" in r["Kernel_Name"]]
        merge_grid = max(set(merges), key=merges.count) if merges else None
        per[counter] = {
            "decode_kernel": avg(lambda r: "decode_kernel" in r["Kernel_Name"] and int(r["Grid_Size"]) == main_grid),
            "merge_kernel": avg(lambda r: "merge" in r["Kernel_Name"] and int(r["Grid_Size"]) == merge_grid),
            "stream_copy": avg(lambda r: "stream_copy_kernel" in r["Kernel_Name"]),
        }
        # every other library kernel, per (name, grid): the write-side kernels
        others = {}
        for r in rows:
            name = r["Kernel_Name"]
            if "kvq::" not in name or "decode_kernel" in name or "merge" in name or "stream_" in name:
                continue
            key = (name.split("(")[0].replace("void kvq::", ""), int(r["Grid_Size"]))
            others.setdefault(key, []).append(float(r["Counter_Value"]))
        per[counter]["others"] = {k: (sum(v) / len(v), len(v)) for k, v in others.items()}
    f_fac = CALIB_BYTES / 1024 / per["FETCH_SIZE"]["stream_copy"][0]
    w_fac = CALIB_BYTES / 1024 / per["WRITE_SIZE"]["stream_copy"][0]
    fetch_kib = per["FETCH_SIZE"]["decode_kernel"][0] + per["FETCH_SIZE"]["merge_kernel"][0]
    write_kib = per["WRITE_SIZE"]["decode_kernel"][0] + per["WRITE_SIZE"]["merge_kernel"][0]
    traffic = 1024 * (f_fac * fetch_kib + w_fac * write_kib)
    w = WORKLOADS[workload]
    algo = w["batch"] * w["ctx"] * HKV * token_head_bytes(w["fmt"])
    rec = {"workload": workload, "decode_source_digest": decode_source_digest(),
           "fetch_factor": f_fac, "write_factor": w_fac,
           "fetch_kib_per_call": fetch_kib, "write_kib_per_call": write_kib,
           "traffic_bytes_per_call": traffic, "algorithmic_bytes_per_call": algo}
    lines = [f"# HBM traffic of the decode call: {workload}", "",
             "Two counter passes (run from the repository root on one MI355X):", "", "```",
             PMC_RUN.format(counter="FETCH_SIZE", tag=f"fetch_{workload}", workload=workload),
             PMC_RUN.format(counter="WRITE_SIZE", tag=f"write_{workload}", workload=workload),
             f"python bench.py --summarize-pmc gpurun_out/pmc_fetch_{workload} gpurun_out/pmc_write_{workload} "
             f"--workload {workload}",
             "```", "",
             "Per-dispatch averages (KiB as the counters report them):", "",
             "| kernel | FETCH_SIZE | dispatches | WRITE_SIZE | dispatches |", "|---|---|---|---|---|"]
    for k in ("decode_kernel", "merge_kernel", "stream_copy"):
        fv, fn = per["FETCH_SIZE"][k]
        wv, wn = per["WRITE_SIZE"][k]
        lines.append(f"| {k} | {fv:,.1f} | {fn} | {wv:,.1f} | {wn} |")
    lines += ["",
              f"Calibration: the library's plain 4 GiB copy (kvq_stream_copy in the bench's copy ceiling, "
              f"4,194,304 KiB read and written) reads {per['FETCH_SIZE']['stream_copy'][0]:,.1f} KiB of FETCH_SIZE "
              f"and {per['WRITE_SIZE']['stream_copy'][0]:,.1f} KiB of WRITE_SIZE, so the factors are "
              f"{f_fac:.4f} (fetch) and {w_fac:.4f} (write).", "",
              f"Traffic per decode call (decode + merge kernels): {traffic:,.0f} B = "
              f"{traffic / algo:.4f} x the algorithmic {algo:,} B of packed KV.", ""]
    keys = sorted(set(per["FETCH_SIZE"]["others"]) | set(per["WRITE_SIZE"]["others"]))
    if keys:
        lines += ["Other library kernels of the same run, per dispatch (MB = the counters x the calibration "
                  "factors / 1e6; stores are cache population in 65,536-token chunks and the step's new "
                  "tokens, the dequant is the whole prefix):", "",
                  "| kernel | grid (threads) | fetched MB | written MB | dispatches |", "|---|---|---|---|---|"]
        for k in keys:
            fv, fn = per["FETCH_SIZE"]["others"].get(k, (0.0, 0))
            wv, wn = per["WRITE_SIZE"]["others"].get(k, (0.0, 0))
            lines.append(f"| `{k[0]}` | {k[1]:,} | {fv * f_fac * 1024 / 1e6:,.2f} | {wv * w_fac * 1024 / 1e6:,.2f} | "
                         f"{max(fn, wn)} |")
            rec.setdefault("other_kernels", []).append(
                {"kernel": k[0], "grid": k[1], "fetch_bytes": fv * f_fac * 1024, "write_bytes": wv * w_fac * 1024})
        lines.append("")
    lines += ["```json", json.dumps(rec, indent=1), "```", ""]
    return "\n".join(lines)


def summarize_counters(dirs: list[str], kernel: str) -> str:
    """Markdown table: per kernel (name and grid) matching `kernel`, the
    per-dispatch average of every counter found in the rocprofv3 --pmc csv
    output directories `dirs` (one directory per counter pass)."""
    agg = {}
    counters = []
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if kernel not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(")[0]
            key = (name, r["Grid_Size"])
            c = r["Counter_Name"]
            if c not in counters:
                counters.append(c)
            agg.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    lines = ["| kernel | grid | " + " | ".join(counters) + " |", "|---|---|" + "---|" * len(counters)]
    for (name, grid), cs in sorted(agg.items()):
        vals = [f"{sum(cs[c]) / len(cs[c]):,.0f}" if c in cs else "" for c in counters]
        lines.append(f"| `{name}` | {grid} | " + " | ".join(vals) + " |")
    return "\n".join(lines) + "\n"


def summarize_trace(trace_dir: str, bench_json: str | None) -> str:
    """Markdown table of kernel durations (rocprofv3 --kernel-trace, csv output) per
    kernel and launch grid, plus the bench's own live figures for comparison."""
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    groups = {}
    for r in rows:
        grid = tuple(int(r.get(f"Grid_Size_{a}", 0) or 0) for a in "XYZ")
        key = (r["Kernel_Name"], grid)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | grid (x, y, z) | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    other = 0.0
    for (name, grid), v in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        if "kvq::" not in name:  # torch's input generation and copies
            other += sum(v)
            continue
        short = name.replace("(kvq::DecodeParams)", "").replace("(kvq::StoreParams)", "")
        short = short.replace("(kvq::DequantParams)", "").replace("void kvq::", "")
        lines.append(f"| `{short}` | {grid} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    lines.append(f"\nOther kernels (torch input generation, copies): {other / 1e3:.1f} ms in total.")
    if bench_json:
        with open(bench_json) as f:
            line = json.loads([l for l in f if l.startswith("{")][-1])
        rf = line["roofline"]
        lines += ["", f"The same run's JSON line: decode call {rf['avg_launch_us']:.2f} us live (HIP events on the "
                  f"launch stream), {rf['achieved']:.0f} GB/s = {100 * rf['frac']:.1f} % of {rf['peak']:.0f} GB/s."]
    return "\n".join(lines) + "\n"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ctx32k", choices=sorted(WORKLOADS))
    ap.add_argument("--secondary", default="ctx160k,ctx1m,int4_220k,fp8_32k,k8v4_32k,rot_32k",
                    help="comma-separated extra workloads to report ('' for none)")
    ap.add_argument("--cooldown", type=float, default=10.0,
                    help="idle seconds before each secondary workload (measured: a workload run right after "
                         "another ran up to 10 %% slower, the same workload after a 10 s pause did not)")
    ap.add_argument("--secondary-steps", type=int, default=0,
                    help="timed steps of each secondary workload (0 = --steps; warm-up = --warmup)")
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--num-splits", type=int, default=0, help="decode split count (0 = the library's plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true", help="skip the per-workload quality blocks")
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="target wall time of one CPU-oracle run of the headline (the median of 3 is reported)")
    ap.add_argument("--cpu-seconds-secondary", type=float, default=1.5,
                    help="the same for each secondary workload")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (profiler counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the counter summary of two rocprofv3 --pmc runs (no GPU use)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print a kernel-duration table of a rocprofv3 --kernel-trace csv run (no GPU use)")
    ap.add_argument("--bench-json", help="with --summarize-trace: the JSON line printed by the traced run")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="print per-dispatch counter averages of the kernels named by --kernel")
    ap.add_argument("--kernel", default="extend_kernel", help="with --summarize-counters: kernel name filter")
    return ap.parse_args()


class Layer:
    """One layer: its cache, the decode-step inputs and outputs."""

    def __init__(self, torch, kvq, w, layer, bt, workload_id):
        dev = "cuda"
        B, L, P = w["batch"], w["ctx"], w["page"]
        self.pages_per_seq = bt.shape[1]
        num_pages = B * self.pages_per_seq
        self.cache = kvq.Cache(w["fmt"], num_pages, P, HKV, D, device=dev, rotated=w.get("rotated", False))
        self.bt = bt
        self.lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        g = torch.Generator(device=dev)
        from bit_quantized_kv_amd import inputs
        g.manual_seed(inputs.seed_int(workload_id, layer, inputs.STREAM_Q))
        self.q = torch.randn((B, HQ, D), generator=g, device=dev).to(torch.bfloat16)
        g.manual_seed(inputs.seed_int(workload_id, layer, inputs.STREAM_K + 32))
        self.k_new = torch.randn((B, HKV, D), generator=g, device=dev).to(torch.bfloat16)
        self.v_new = torch.randn((B, HKV, D), generator=g, device=dev).to(torch.bfloat16)
        # the new token is the last cached one: position L - 1 of each sequence
        last = L - 1
        self.slots_new = (bt[:, last // P] * P + last % P).to(torch.int32).contiguous()
        self.out = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev)
        if w.get("rotated"):
            # rotated cache: R q in, R o out (fp32), rotated back into out
            self.q_rot = torch.empty_like(self.q)
            self.out_rot = torch.empty((B, HQ, D), dtype=torch.float32, device=dev)


def student_t4(torch, g, shape):
    z = torch.randn(shape, generator=g, device="cuda")
    chi2 = torch.zeros(shape, device="cuda")
    for _ in range(4):
        chi2 += torch.randn(shape, generator=g, device="cuda") ** 2
    return z / torch.sqrt(chi2 / 4.0) / math.sqrt(2.0)


def populate(torch, kvq, inputs, w, layer_obj, layer, workload_id, chunk_tokens=1 << 16):
    """Fill every cached token of every sequence: K/V generated on the GPU in
    chunks and bulk quantize-stored.  Returns (seconds, bytes read, bytes
    written) of the quantize-store launches."""
    dev = "cuda"
    B, L, P = w["batch"], w["ctx"], w["page"]
    g = torch.Generator(device=dev)
    if w["kind"] == "lognormal":
        g.manual_seed(inputs.seed_int(workload_id, layer, inputs.STREAM_KSCALE))
        kscale = torch.exp(torch.randn((HKV, D), generator=g, device=dev))
        g.manual_seed(inputs.seed_int(workload_id, layer, inputs.STREAM_VSCALE))
        vscale = torch.exp(torch.randn((HKV, D), generator=g, device=dev))
    g.manual_seed(inputs.seed_int(workload_id, layer, inputs.STREAM_K))
    tok = torch.arange(L, device=dev, dtype=torch.int64)
    nbytes_in = 0
    # event pairs around each launch, read once at the end: no host sync between
    # chunks, so the host queues ahead and no launch gap lands inside a pair
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    store_ev = []
    running = torch.zeros(2, dtype=torch.float32, device=dev)
    for b in range(B):
        for t0 in range(0, L, chunk_tokens):
            t1 = min(L, t0 + chunk_tokens)
            n = t1 - t0
            if w["kind"] == "lognormal":
                k = (torch.randn((n, HKV, D), generator=g, device=dev) * kscale).to(torch.bfloat16)
                v = (torch.randn((n, HKV, D), generator=g, device=dev) * vscale).to(torch.bfloat16)
            else:  # Student-t, nu = 4 (z / sqrt(chi2_4 / 4)), scaled to unit variance
                k = student_t4(torch, g, (n, HKV, D)).to(torch.bfloat16)
                v = student_t4(torch, g, (n, HKV, D)).to(torch.bfloat16)
            t = tok[t0:t1]
            slots = (layer_obj.bt[b, t // P].to(torch.int64) * P + t % P).to(torch.int32)
            if w["fmt"] == 1 and layer == 0:
                # global-scale calibration pass over the same rows (the cache
                # keeps gs = 1, the configuration the pages measured)
                kvq.kvq_calibrate_amax(layer_obj.cache, k, v, running)
            store_ev.append((ev(), ev()))
            store_ev[-1][0].record()
            kvq.kvq_quantize_store(layer_obj.cache, k, v, slots)
            store_ev[-1][1].record()
            nbytes_in += 2 * k.numel() * 2
    torch.cuda.synchronize()
    total_s = sum(a.elapsed_time(b) for a, b in store_ev) / 1e3
    nbytes_out = B * L * HKV * token_head_bytes(w["fmt"])
    if w["fmt"] == 1 and layer == 0:
        # the calibration kernel's rate: back-to-back passes over the last chunk
        # (resident rows; the per-chunk launches above wait on the host)
        amax = running.cpu().tolist()
        reps = 10
        a0, a1 = ev(), ev()
        a0.record()
        for _ in range(reps):
            kvq.kvq_calibrate_amax(layer_obj.cache, k, v, running)
        a1.record()
        a1.synchronize()
        us = a0.elapsed_time(a1) / reps * 1e3
        nb = 2 * k.numel() * 2
        populate.calibration = {"us_per_call": us, "tokens_per_call": int(k.shape[0]), "read_bytes_per_call": nb,
                                "gbs": nb / (us * 1e-6) / 1e9, "population_seconds": nbytes_in / nb * us * 1e-6,
                                "amax": amax, "layer": 0}
    return total_s, nbytes_in, nbytes_out


def block_tables(torch, inputs, w, workload_id):
    """Block tables with room for the context and, where the workload appends
    a chunked-prefill chunk, for that chunk's tokens after it."""
    B, L, P = w["batch"], w["ctx"], w["page"]
    pps = -(-(L + w.get("chunk", 0)) // P)
    bt = inputs.page_tables(workload_id, B, pps, B * pps, shuffled=w["shuffled"])
    return torch.from_numpy(bt).to("cuda")


def run_workload(torch, kvq, inputs, name, steps, warmup, n_layers, cpu_target=0.0, quality=False, num_splits=0,
                 store_dequant_cpu=False):
    w = WORKLOADS[name]
    wid = sorted(WORKLOADS).index(name) + 2
    B, L, P, fmt = w["batch"], w["ctx"], w["page"], w["fmt"]
    bt = block_tables(torch, inputs, w, wid)
    layers, pop_s, pop_in, pop_out = [], 0.0, 0, 0
    for l in range(n_layers):
        lay = Layer(torch, kvq, w, l, bt, wid)
        s, bi, bo = populate(torch, kvq, inputs, w, lay, l, wid)
        pop_s, pop_in, pop_out = pop_s + s, pop_in + bi, pop_out + bo
        layers.append(lay)
    splits = num_splits or kvq.kvq_decode_num_splits(layers[0].cache, B, HQ, L)
    ws = torch.empty(kvq.kvq_decode_workspace_size(layers[0].cache, B, HQ, L, splits), dtype=torch.uint8,
                     device="cuda")
    # chunked-prefill store (160K): 64 new tokens per sequence appended at
    # positions L .. L + 63, in the pages the block table holds past the context
    chunk = None
    if w.get("chunk"):
        n = w["chunk"]
        g = torch.Generator(device="cuda")
        g.manual_seed(inputs.seed_int(wid, 0, 40))
        kc = torch.randn((B * n, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
        vc = torch.randn((B * n, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
        t = torch.arange(L, L + n, device="cuda")
        slots = torch.cat([(bt[b, t // P].to(torch.int64) * P + t % P) for b in range(B)]).to(torch.int32)
        chunk = (kc, vc, slots)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def decode_only(lay):
        if w.get("rotated"):
            kvq.kvq_hadamard_rotate(lay.q, out=lay.q_rot)
            kvq.kvq_decode_attention(lay.cache, lay.q_rot, lay.bt, lay.lens, L, out=lay.out_rot, workspace=ws,
                                     num_splits=splits)
            kvq.kvq_hadamard_rotate(lay.out_rot, out=lay.out)
        else:
            kvq.kvq_decode_attention(lay.cache, lay.q, lay.bt, lay.lens, L, out=lay.out, workspace=ws,
                                     num_splits=splits)

    def step():
        for lay in layers:
            kvq.kvq_quantize_store(lay.cache, lay.k_new, lay.v_new, lay.slots_new)
            decode_only(lay)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing
    t_start, t_end = ev(), ev()
    t_start.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / steps
    # per-call timing.  Decode: back to back over the layers, one event pair per
    # pass (the host queues calls faster than the GPU runs them, so no launch
    # wait lands inside the events).  Store (a few us, shorter than its launch
    # on the host): an event pair around each store inside the normal step,
    # where the decode calls keep the GPU busy while the host queues the next.
    dec_marks = [(ev(), ev()) for _ in range(steps)]
    for a, b_ in dec_marks:
        a.record(stream)
        for lay in layers:
            decode_only(lay)
        b_.record(stream)
    st_marks = [(ev(), ev()) for _ in range(steps * len(layers))]
    it = iter(st_marks)
    for _ in range(steps):
        for lay in layers:
            a, b_ = next(it)
            a.record(stream)
            kvq.kvq_quantize_store(lay.cache, lay.k_new, lay.v_new, lay.slots_new)
            b_.record(stream)
            decode_only(lay)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b_) / len(layers) for a, b_ in dec_marks)
    decode_ms, decode_median_ms = sum(per) / len(per), per[len(per) // 2]
    store_ms = sum(a.elapsed_time(b_) for a, b_ in st_marks) / len(st_marks)
    kv_bytes_layer = B * L * HKV * token_head_bytes(fmt)
    res = {
        "workload": name, "desc": w["desc"], "format": {1: "nvfp4", 2: "int4_per_token_head", 3: "fp8_e4m3_per_tensor",
                                                 4: "fp8_keys_nvfp4_values"}[fmt],
        "batch": B, "context": L, "page_size": P, "layers": n_layers, "num_splits": splits,
        "step_ms": step_ms, "decode_call_us": decode_ms * 1e3, "decode_call_us_median": decode_median_ms * 1e3,
        "decode_call_calls_timed": steps * len(layers), "decode_call_median_over": "passes over the layers",
        "store_call_us": store_ms * 1e3,
        "kv_bytes_per_layer": kv_bytes_layer,
        "effective_kv_gbs": n_layers * kv_bytes_layer / (step_ms * 1e-3) / 1e9,
        "decode_call_gbs": kv_bytes_layer / (decode_ms * 1e-3) / 1e9,
        "tokens_per_s": B / (step_ms * 1e-3),
        "tokens_per_s_16_layers": B / (step_ms * 1e-3 * LAYERS / n_layers),
        "populate": {"seconds": pop_s, "read_bytes": pop_in, "write_bytes": pop_out,
                     "gbs": (pop_in + pop_out) / pop_s / 1e9 if pop_s > 0 else None},
    }
    if fmt == 1 and getattr(populate, "calibration", None):
        res["calibrate_amax"] = populate.calibration
        populate.calibration = None
    res["decode_call_frac_hbm"] = res["decode_call_gbs"] / HBM_PEAK_GBS
    if chunk is not None:
        kc, vc, slots = chunk
        for _ in range(3):
            kvq.kvq_quantize_store(layers[0].cache, kc, vc, slots)
        a, b_ = ev(), ev()
        a.record(stream)
        for _ in range(steps):
            kvq.kvq_quantize_store(layers[0].cache, kc, vc, slots)
        b_.record(stream)
        torch.cuda.synchronize()
        res["chunk_store_us"] = a.elapsed_time(b_) / steps * 1e3
        res["chunk_store_tokens"] = int(slots.numel())
    if w.get("split_sweep"):
        # decode call time against the split count (fixed plan per entry), layers rotated
        sweep = {}
        for ns in w["split_sweep"]:
            wsz = torch.empty(kvq.kvq_decode_workspace_size(layers[0].cache, B, HQ, L, ns), dtype=torch.uint8,
                              device="cuda")
            times = []
            for i in range(steps + 2):
                lay = layers[i % n_layers]
                a, b_ = ev(), ev()
                a.record(stream)
                kvq.kvq_decode_attention(lay.cache, lay.q, lay.bt, lay.lens, L, out=lay.out, workspace=wsz,
                                         num_splits=ns)
                b_.record(stream)
                times.append((a, b_))
            torch.cuda.synchronize()
            us = sum(a.elapsed_time(b) for a, b in times[2:]) / steps * 1e3
            sweep[str(ns)] = {"decode_call_us": us, "gbs": kv_bytes_layer / (us * 1e-6) / 1e9}
            del wsz
        res["split_sweep"] = sweep
    if w.get("prefix"):
        rows = L + 4096
        k_ws = torch.empty((rows, HKV * D), dtype=torch.bfloat16, device="cuda")
        v_ws = torch.empty((rows, HKV * D), dtype=torch.bfloat16, device="cuda")
        times = []
        for i in range(steps + 2):
            lay = layers[i % n_layers]
            a, b_ = ev(), ev()
            a.record(stream)
            kvq.kvq_dequant_prefix(lay.cache, lay.bt[0], L, k_ws, v_ws)
            b_.record(stream)
            times.append((a, b_))
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in times[2:]) / steps * 1e3
        rd = L * HKV * token_head_bytes(fmt)
        wr = 2 * L * HKV * D * 2
        res["dequant_prefix"] = {"us": us, "read_bytes": rd, "write_bytes": wr,
                                 "gbs": (rd + wr) / (us * 1e-6) / 1e9,
                                 "frac_hbm": (rd + wr) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        # extend attention of a 4,096-token chunk over [prefix | chunk] in the same
        # workspace (the chunk's K/V in its last rows), for two prefix lengths
        n = 4096
        g = torch.Generator(device="cuda")
        g.manual_seed(inputs.seed_int(wid, 0, 50))
        k_ws[L:L + n] = torch.randn((n, HKV * D), generator=g, device="cuda").to(torch.bfloat16)
        v_ws[L:L + n] = torch.randn((n, HKV * D), generator=g, device="cuda").to(torch.bfloat16)
        qc = torch.randn((n, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
        oc = torch.empty((n, HQ, D), dtype=torch.bfloat16, device="cuda")
        ext = {}
        for lp in (32768, L):
            # the chunk rows follow the prefix: use rows [L - lp, L + n) as the workspace
            kw, vw = k_ws[L - lp:], v_ws[L - lp:]
            reps = 1 if lp == L else 5
            kvq.kvq_extend_attention(qc, kw, vw, lp, out=oc)
            a, b_ = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                kvq.kvq_extend_attention(qc, kw, vw, lp, out=oc)
            b_.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b_) / reps * 1e3
            flops = 4.0 * HQ * D * (n * lp + n * (n + 1) / 2)
            ext[str(lp)] = {"prefix_len": lp, "chunk_len": n, "us": us, "flops": flops,
                            "tflops": flops / (us * 1e-6) / 1e12,
                            "frac_bf16_mfma_peak": flops / (us * 1e-6) / 2.5e15}
        res["extend_attention"] = ext
        # the fused extend: the prefix straight from the 4-bit pages, no workspace
        fused = {}
        kc_rows, vc_rows = k_ws[L:L + n], v_ws[L:L + n]
        lay = layers[0]
        for lp in (32768, L):
            reps = 1 if lp == L else 5
            kvq.kvq_extend_attention_paged(lay.cache, lay.bt[0], lp, qc, kc_rows, vc_rows, out=oc)
            a, b_ = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                kvq.kvq_extend_attention_paged(lay.cache, lay.bt[0], lp, qc, kc_rows, vc_rows, out=oc)
            b_.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b_) / reps * 1e3
            flops = 4.0 * HQ * D * (n * lp + n * (n + 1) / 2)
            fused[str(lp)] = {"prefix_len": lp, "chunk_len": n, "us": us, "flops": flops,
                              "tflops": flops / (us * 1e-6) / 1e12,
                              "frac_bf16_mfma_peak": flops / (us * 1e-6) / 2.5e15,
                              "workspace_bytes": 0}
        res["extend_attention_fused"] = fused
        del k_ws, v_ws, qc, oc, kc_rows, vc_rows
    if w.get("fused_extend"):
        # the fused extend over this format's pages: a 4,096-token bf16 chunk
        # over the first sequence's cached prefix (32,768 tokens, and all of it)
        n = 4096
        g = torch.Generator(device="cuda")
        g.manual_seed(inputs.seed_int(wid, 0, 51))
        kc_rows = torch.randn((n, HKV * D), generator=g, device="cuda").to(torch.bfloat16)
        vc_rows = torch.randn((n, HKV * D), generator=g, device="cuda").to(torch.bfloat16)
        qc = torch.randn((n, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
        oc = torch.empty((n, HQ, D), dtype=torch.bfloat16, device="cuda")
        fused = {}
        lay = layers[0]
        for lp in (32768, L):
            reps = 1 if lp == L else 5
            kvq.kvq_extend_attention_paged(lay.cache, lay.bt[0], lp, qc, kc_rows, vc_rows, out=oc)
            a, b_ = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                kvq.kvq_extend_attention_paged(lay.cache, lay.bt[0], lp, qc, kc_rows, vc_rows, out=oc)
            b_.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b_) / reps * 1e3
            flops = 4.0 * HQ * D * (n * lp + n * (n + 1) / 2)
            fused[str(lp)] = {"prefix_len": lp, "chunk_len": n, "us": us, "flops": flops,
                              "tflops": flops / (us * 1e-6) / 1e12,
                              "frac_bf16_mfma_peak": flops / (us * 1e-6) / 2.5e15,
                              "workspace_bytes": 0}
        res["extend_attention_fused"] = fused
        del qc, oc, kc_rows, vc_rows
    if cpu_target > 0:
        res["cpu_baseline"] = cpu_baseline(torch, layers[0], w, cpu_target)
        print(f"[bench] {name}: cpu oracle {res['cpu_baseline']['value']:.4f} GB/s", file=sys.stderr, flush=True)
        if store_dequant_cpu:
            res["cpu_baseline_store_dequant"] = cpu_store_dequant_baseline(torch, layers[0], w, wid, cpu_target / 2)
    if quality and not w.get("rotated"):
        res["quality"] = quality_block(torch, kvq, inputs, w, layers[0], wid, L, n_layers)
    del layers, ws, chunk
    torch.cuda.empty_cache()
    return res


def write_copy_ceilings(torch, kvq, steps):
    """Practical HBM write and copy ceilings: the library's plain streaming
    write over 8 GiB and copy of 4 GiB into 4 GiB (no pass cached), timed
    like the decode call; the bulk store (read-dominated) and the prefix
    dequantization (write-dominated) are judged against them."""
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out = {}
    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        kvq.kvq_stream_write(buf, 0x01010101)
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(steps):
        kvq.kvq_stream_write(buf, 0x01010101)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    out["write"] = {"gbs": nbytes / (us * 1e-6) / 1e9, "us": us, "bytes": nbytes,
                    "kernel": "kvq_stream_write: grid-stride 16-byte non-temporal stores, 2048 workgroups"}
    half = nbytes // 2
    src, dst = buf[:half], buf[half:]
    for _ in range(2):
        kvq.kvq_stream_copy(src, dst)
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(steps):
        kvq.kvq_stream_copy(src, dst)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    out["copy"] = {"gbs": 2 * half / (us * 1e-6) / 1e9, "us": us, "bytes_read": half, "bytes_written": half,
                   "kernel": "kvq_stream_copy: 16-byte loads (nt) and non-temporal stores, 2048 workgroups"}
    del buf, src, dst
    torch.cuda.empty_cache()
    return out


def read_ceiling(torch, kvq, steps):
    """Practical HBM read ceiling: the library's plain streaming-read kernel over
    16 GiB (64x the Infinity Cache, so no pass finds its data cached; 4 GiB
    measured 2-3 % faster), timed like the decode call."""
    nbytes = 16 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        kvq.kvq_stream_read(buf, sink)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        kvq.kvq_stream_read(buf, sink)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    del buf
    return {"gbs": nbytes / (us * 1e-6) / 1e9, "us": us, "bytes": nbytes,
            "kernel": "kvq_stream_read: grid-stride 16-byte buffer loads (sc0 nt, as decode), 2048 workgroups"}


def mfma_ceilings(torch, kvq, steps):
    """Practical matrix-core ceilings of the extend kernels' product
    (v_mfma_f32_16x16x32_f16, the fused extend's occupancy: 768-thread
    workgroups, one per compute unit): operands in registers, and each
    product's first operand read from LDS as the extend kernels read their key
    rows (QK), and the extend kernels' own mix of that and the value-row form
    (PV: two transposing reads per operand).  512 workgroups x 2,000
    iterations per call, timed like the decode call."""
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    wgs, iters = 512, 2000
    flops = 16384.0 * 16 * 12 * iters * wgs
    out = {}
    for name, lds in (("registers", 0), ("lds_operand_per_product", 1), ("lds_qk_pv_mix", 2)):
        for _ in range(2):
            kvq.kvq_mfma_rate(lds, iters, wgs, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            kvq.kvq_mfma_rate(lds, iters, wgs, sink)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        tf = flops / (us * 1e-6) / 1e12
        out[name] = {"tflops": tf, "frac_of_peak": tf / 2500.0, "us": us, "flops": flops}
    out["kernel"] = ("kvq_mfma_rate: v_mfma_f32_16x16x32_f16, 512 workgroups of 768 threads, 16 products per "
                     "wavefront and iteration into 4 accumulators; operands in registers, the first from a "
                     "16-byte LDS read per product, or products alternating between that read and two "
                     "transposing 8-byte LDS reads (the extend kernels' QK and PV operand forms)")
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((x.split(":", 1)[1].strip() for x in f if x.startswith("model name")), "")
    except OSError:
        return ""


def _oracle_pool(oracle, lay, w, nseq, ntok):
    """The first ntok cached tokens of sequences 0 .. nseq - 1 of a layer, their
    pages copied to a host oracle pool and renumbered."""
    import numpy as np
    P = w["page"]
    npg = -(-ntok // P)
    pages = lay.bt[:nseq, :npg].reshape(-1).long()
    pool = oracle.Pool(w["fmt"], nseq * npg, P, HKV, D, rotated=w.get("rotated", False))
    pool.data[:] = lay.cache.pool[pages].cpu().numpy()
    return pool, np.arange(nseq * npg, dtype=np.int32).reshape(nseq, npg)


def cpu_baseline(torch, lay, w, target_s, one_thread=True):
    """The CPU oracle (as written: fp64 attention, scalar codecs) decoding a
    bounded sample of the same cache: whole sequences of layer 0 when one
    takes less than target_s, else the first tokens of sequence 0 -- all 24
    query heads, pages copied to the host.  Median of 3 runs after a warm-up."""
    import numpy as np
    import oracle
    P, L, B = w["page"], w["ctx"], w["batch"]
    q_all = (lay.q_rot if w.get("rotated") else lay.q).float().cpu().numpy()

    def run(nseq, ntok):
        pool, bt = _oracle_pool(oracle, lay, w, nseq, ntok)
        t = time.perf_counter()
        pool.decode_attention(q_all[:nseq], bt, np.full(nseq, ntok, np.int32))
        return time.perf_counter() - t

    n0 = min(L, 32768)
    t0 = run(1, n0)  # also the warm-up
    full = t0 * L / n0
    if full <= target_s:
        nseq, ntok = int(max(1, min(B, round(target_s / full)))), L
    else:
        nseq, ntok = 1, int(max(P, min(L, target_s / t0 * n0 // P * P)))
    runs = sorted(run(nseq, ntok) for _ in range(3))
    t = runs[1]
    nbytes = nseq * ntok * HKV * token_head_bytes(w["fmt"])
    threads = oracle.num_threads()
    res = {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"1 layer, {nseq} of {B} sequences x {ntok:,} of {L:,} cached tokens, all {HQ} query heads, "
                     f"fp64 attention over the same packed pages (median of 3 runs of {t:.2f} s after a warm-up)",
           "seconds": t, "seconds_runs": runs, "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
           "tokens_per_s_16_layers_extrapolated": nseq / (t * L / ntok * LAYERS),
           "extrapolation": "one layer timed (the sampled tokens scaled to the whole context), x16 layers assumed"}
    if one_thread:
        oracle.set_num_threads(1)
        try:
            n1 = min(L, 8192)
            t1 = run(1, n1)
        finally:
            oracle.set_num_threads(threads)
        res["one_thread"] = {"value": n1 * HKV * token_head_bytes(w["fmt"]) / t1 / 1e9, "unit": "GB/s",
                             "sample": f"1 sequence x {n1:,} tokens, 1 thread ({t1:.2f} s)"}
    return res


def cpu_store_dequant_baseline(torch, lay, w, wid, target_s):
    """The CPU oracle's quantize-store and prefix dequantization on bounded
    samples of this workload's rows: the same bf16-valued K/V distribution
    (regenerated on the host), and the layer's own cached pages."""
    import numpy as np
    import oracle
    from bit_quantized_kv_amd import inputs
    P, fmt = w["page"], w["fmt"]

    def med3(fn):
        fn()
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return sorted(ts)[1]

    out = {}
    # quantize-store: n tokens x 4 heads of K and V rows (bf16 values)
    n = 2048
    gen = inputs.kv_lognormal_channels if w["kind"] == "lognormal" else inputs.kv_student_t
    k, v = gen(wid, 0, n, HKV, D)
    npg = -(-n // P)
    pool = oracle.Pool(fmt, npg, P, HKV, D)
    slots = np.arange(n, dtype=np.int32)
    t = med3(lambda: pool.quantize_store(k, v, slots))
    n = int(max(n, min(1 << 16, n * target_s / max(t, 1e-3))) // P * P)
    k, v = gen(wid, 1, n, HKV, D)
    pool = oracle.Pool(fmt, -(-n // P), P, HKV, D)
    slots = np.arange(n, dtype=np.int32)
    t = med3(lambda: pool.quantize_store(k, v, slots))
    rd, wr = 2 * n * HKV * D * 2, n * HKV * token_head_bytes(fmt)
    out["quantize_store"] = {"value": (rd + wr) / t / 1e9, "unit": "GB/s (bf16 rows read + packed bytes written)",
                             "cores": oracle.num_threads(), "kind": "oracle", "seconds": t,
                             "sample": f"{n:,} tokens x {HKV} KV heads of K and V rows, median of 3"}
    if fmt in (1, 2):
        ntok = int(min(w["ctx"], 1 << 16) // P * P)
        pool, bt = _oracle_pool(oracle, lay, w, 1, ntok)
        t = med3(lambda: pool.dequant_prefix(bt[0], ntok))
        rd, wr = ntok * HKV * token_head_bytes(fmt), 2 * ntok * HKV * D * 2
        out["dequant_prefix"] = {"value": (rd + wr) / t / 1e9,
                                 "unit": "GB/s (packed bytes read + bf16 rows written)",
                                 "cores": oracle.num_threads(), "kind": "oracle", "seconds": t,
                                 "sample": f"the first {ntok:,} cached tokens of sequence 0, median of 3"}
    return out


def quality_block(torch, kvq, inputs, w, lay, wid, L, n_layers):
    """Attention quality at this workload on sequence 0 of layer 0: the
    kernel against the oracle on the same dequantized cache (its own error),
    and kernel and oracle against fp64 attention over the unquantized K/V
    (the format's error, not the kernel's).  The unquantized rows are those
    the cache was populated from, regenerated on the GPU from the same
    generator, with the decode step's token at position L - 1."""
    import numpy as np
    import oracle
    fmt, P = w["fmt"], w["page"]
    G = HQ // HKV
    dev = "cuda"
    lay0 = lay
    # kernel outputs of the whole batch, sequence 0 kept
    out32 = torch.empty((w["batch"], HQ, D), dtype=torch.float32, device=dev)
    out16 = torch.empty((w["batch"], HQ, D), dtype=torch.bfloat16, device=dev)
    kvq.kvq_decode_attention(lay0.cache, lay0.q, lay0.bt, lay0.lens, L, out=out32)
    kvq.kvq_decode_attention(lay0.cache, lay0.q, lay0.bt, lay0.lens, L, out=out16)
    torch.cuda.synchronize()
    k32 = out32[0].double().cpu().numpy()
    k16 = out16[0].double().cpu().numpy()
    # oracle on sequence 0: 4 query heads per KV group at most (16 of 24)
    per = min(G, 4)
    heads = [g * G + i for g in range(HKV) for i in range(per)]
    pool, bt = _oracle_pool(oracle, lay0, w, 1, L)
    qh = lay0.q[0:1, heads].float().cpu().numpy()
    ref, _ = pool.decode_attention(qh, bt, np.array([L], np.int32))
    ref = ref[0]
    del pool
    # unquantized K, V of sequence 0, regenerated as populate() drew them
    g = torch.Generator(device=dev)
    if w["kind"] == "lognormal":
        g.manual_seed(inputs.seed_int(wid, 0, inputs.STREAM_KSCALE))
        kscale = torch.exp(torch.randn((HKV, D), generator=g, device=dev))
        g.manual_seed(inputs.seed_int(wid, 0, inputs.STREAM_VSCALE))
        vscale = torch.exp(torch.randn((HKV, D), generator=g, device=dev))
    g.manual_seed(inputs.seed_int(wid, 0, inputs.STREAM_K))
    ks, vs = [], []
    for t0 in range(0, L, 1 << 16):
        n = min(L, t0 + (1 << 16)) - t0
        if w["kind"] == "lognormal":
            ks.append((torch.randn((n, HKV, D), generator=g, device=dev) * kscale).to(torch.bfloat16))
            vs.append((torch.randn((n, HKV, D), generator=g, device=dev) * vscale).to(torch.bfloat16))
        else:
            ks.append(student_t4(torch, g, (n, HKV, D)).to(torch.bfloat16))
            vs.append(student_t4(torch, g, (n, HKV, D)).to(torch.bfloat16))
    K, V = torch.cat(ks), torch.cat(vs)
    del ks, vs
    K[L - 1] = lay0.k_new[0]
    V[L - 1] = lay0.v_new[0]
    full = np.zeros((HQ, D))
    q64 = lay0.q[0].double()
    for kv in range(HKV):
        Kg = K[:, kv].double().contiguous()
        Vg = V[:, kv].double().contiguous()
        s = torch.matmul(Kg, q64[kv * G:(kv + 1) * G].t().contiguous()) / math.sqrt(D)  # [L][G]
        p = torch.softmax(s, dim=0)
        full[kv * G:(kv + 1) * G] = torch.matmul(p.t().contiguous(), Vg).cpu().numpy()
        del Kg, Vg, s, p
    del K, V
    torch.cuda.empty_cache()

    def cos(a, b):
        return float(np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b)))

    ck = [cos(k32[h], full[h]) for h in range(HQ)]
    co = [cos(ref[i], full[h]) for i, h in enumerate(heads)]
    e16 = np.abs(k16[heads] - ref)
    half_ulp = np.where(np.abs(ref) > 0, 2.0 ** (np.floor(np.log2(np.where(ref != 0, np.abs(ref), 1.0))) - 8), 0.0)
    return {
        "sequence": 0, "layer": 0, "context": L, "query_heads_vs_oracle": heads,
        "kernel_bf16_max_abs_vs_oracle": float(e16.max()),
        "kernel_bf16_max_abs_vs_oracle_where_abs_o_below_0p5": float(e16[np.abs(ref) < 0.5].max())
        if (np.abs(ref) < 0.5).any() else None,
        "kernel_bf16_max_abs_minus_half_ulp_vs_oracle": float((e16 - half_ulp).max()),
        "kernel_fp32_max_abs_vs_oracle": float(np.abs(k32[heads] - ref).max()),
        "max_abs_output": float(np.abs(ref).max()),
        "cosine_vs_unquantized_fp64": {"kernel_min": min(ck), "kernel_mean": float(np.mean(ck)),
                                       "oracle_min": min(co), "oracle_mean": float(np.mean(co)),
                                       "kernel_minus_oracle_max_abs": float(np.max(np.abs(
                                           np.array([ck[h] for h in heads]) - np.array(co))))},
        "property": "format: the cosine to unquantized attention is the cache format's quantization error on "
                    "this synthetic data (the oracle on the same cache has the same cosine); the kernel's own "
                    "error is its distance to the oracle",
        "reference": "'KV cache in 4 bits: 8.8 instead of 4.7 full sessions ...', section 'How we checked "
                     "quality' (kernel against a reference of the same format)"}


def quality_tiny():
    """The tiny reference configuration (1 layer, 1 KV head, 4 query heads, D
    256, 512 tokens, 16-token pages, fp32 K/V ~ N(0,1) with 4 channels x8):
    kernel against the oracle and both against fp64 unquantized attention."""
    import numpy as np
    import torch
    import oracle
    from bit_quantized_kv_amd import inputs, kvq
    Dt, Hkv, Hq, P, L = 256, 1, 4, 16, 512
    dev = torch.device("cuda")
    k, v = inputs.kv_outlier_channels(1, 0, L, Hkv, Dt)
    q = inputs.query(1, 0, 1, Hq, Dt)
    bt = np.arange(L // P, dtype=np.int32)[None]
    slots = inputs.slots_for(bt, P, 0, 0, L)
    out = {}
    for fmt in (1, 2):
        cache = kvq.Cache(fmt, L // P, P, Hkv, Dt, device=dev)
        kvq.kvq_quantize_store(cache, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                               torch.from_numpy(slots).to(dev))
        qd = torch.from_numpy(q).to(dev).to(torch.bfloat16)
        args = (cache, qd, torch.from_numpy(bt).to(dev), torch.tensor([L], dtype=torch.int32, device=dev), L)
        o32 = kvq.kvq_decode_attention(*args, out_dtype=torch.float32).double().cpu().numpy()[0]
        o16 = kvq.kvq_decode_attention(*args, out_dtype=torch.bfloat16).double().cpu().numpy()[0]
        ref_pool = oracle.Pool(fmt, L // P, P, Hkv, Dt)
        ref_pool.quantize_store(k, v, slots)
        ref = ref_pool.decode_attention(q, bt, np.array([L], np.int32))[0][0]
        s = q[0].astype(np.float64) @ k[:, 0].astype(np.float64).T / 16.0
        p = np.exp(s - s.max(axis=1, keepdims=True))
        full = (p / p.sum(axis=1, keepdims=True)) @ v[:, 0].astype(np.float64)

        def cos(a, b):
            return float(np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b)))

        out["nvfp4" if fmt == 1 else "int4_per_token_head"] = {
            "kernel_bf16_max_abs_vs_oracle": float(np.abs(o16 - ref).max()),
            "kernel_fp32_max_abs_vs_oracle": float(np.abs(o32 - ref).max()),
            "max_abs_output": float(np.abs(ref).max()),
            "cosine_vs_unquantized_fp64": {"kernel_min": min(cos(o32[h], full[h]) for h in range(Hq)),
                                           "oracle_min": min(cos(ref[h], full[h]) for h in range(Hq))}}
    return out


def main():
    args = parse()
    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload))
        return
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace, args.bench_json))
        return
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(args.summarize_counters, args.kernel))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the split-context path is "
              f"single-GPU by design", file=sys.stderr)
        sys.exit(2)
    import torch
    from bit_quantized_kv_amd import inputs, kvq
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    kvq.lib()  # fail loudly if the HIP library is missing
    t0 = time.time()
    cpu_main = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    cpu_sec = 0.0 if args.no_cpu_baseline else args.cpu_seconds_secondary
    main_res = run_workload(torch, kvq, inputs, args.workload, args.steps, args.warmup, args.layers,
                            cpu_target=cpu_main, quality=not args.no_quality, num_splits=args.num_splits,
                            store_dequant_cpu=True)
    print(f"[bench] {args.workload}: step {main_res['step_ms']:.3f} ms, decode call {main_res['decode_call_us']:.1f} us "
          f"({main_res['decode_call_gbs']:.0f} GB/s), {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    time.sleep(args.cooldown)  # the ceilings from the same idle state as the headline
    ceiling = read_ceiling(torch, kvq, args.steps)
    wc = write_copy_ceilings(torch, kvq, args.steps)
    print(f"[bench] plain streaming read: {ceiling['gbs']:.0f} GB/s, write {wc['write']['gbs']:.0f} GB/s, "
          f"copy {wc['copy']['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    mfma = mfma_ceilings(torch, kvq, args.steps)
    print(f"[bench] f16 MFMA: {mfma['registers']['tflops']:.0f} TFLOP/s from registers, "
          f"{mfma['lds_operand_per_product']['tflops']:.0f} TFLOP/s with one LDS operand per product, "
          f"{mfma['lds_qk_pv_mix']['tflops']:.0f} TFLOP/s with the extend's QK/PV operand mix",
          file=sys.stderr, flush=True)
    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        t1 = time.time()
        # same timing protocol as the headline, from the same idle GPU state
        torch.cuda.synchronize()
        time.sleep(args.cooldown)
        r = run_workload(torch, kvq, inputs, name, args.secondary_steps or args.steps, args.warmup, args.layers,
                         cpu_target=cpu_sec, quality=not args.no_quality,
                         store_dequant_cpu=WORKLOADS[name]["fmt"] == 2)
        rec, _ = load_counter_summary(name)
        if rec is not None:  # HBM bytes per decode call from this workload's own counter passes
            r["hbm_traffic_bytes_per_call"] = rec["traffic_bytes_per_call"]
            r["hbm_traffic_over_algorithmic"] = rec["traffic_bytes_per_call"] / rec["algorithmic_bytes_per_call"]
        secondary[name] = r
        print(f"[bench] {name}: step {r['step_ms']:.3f} ms, decode call {r['decode_call_us']:.1f} us "
              f"({r['decode_call_gbs']:.0f} GB/s), {time.time() - t1:.1f} s", file=sys.stderr, flush=True)
    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = main_res.get("cpu_baseline")
    quality = {}
    if not args.no_quality:
        quality["tiny_512"] = quality_tiny()
    for name, res in [(args.workload, main_res)] + list(secondary.items()):
        if "quality" in res:
            quality[name] = res.pop("quality")
    # the write-side kernels against the measured write and copy ceilings
    for res in [main_res] + list(secondary.values()):
        pop = res["populate"]
        if pop.get("gbs"):
            pop["frac_of_copy_ceiling"] = pop["gbs"] / wc["copy"]["gbs"]
        if "dequant_prefix" in res:
            dq = res["dequant_prefix"]
            dq["frac_of_copy_ceiling"] = dq["gbs"] / wc["copy"]["gbs"]
            dq["frac_of_write_ceiling"] = dq["gbs"] / wc["write"]["gbs"]
    # the extend kernels against the measured matrix-core ceilings
    for res in [main_res] + list(secondary.values()):
        for k in ("extend_attention", "extend_attention_fused"):
            for e in res.get(k, {}).values():
                e["frac_of_register_mfma_ceiling"] = e["tflops"] / mfma["registers"]["tflops"]
                e["frac_of_lds_fed_mfma_ceiling"] = e["tflops"] / mfma["lds_operand_per_product"]["tflops"]
                e["frac_of_operand_mix_mfma_ceiling"] = e["tflops"] / mfma["lds_qk_pv_mix"]["tflops"]
    w = WORKLOADS[args.workload]
    r = main_res
    counters, counters_note = load_counter_summary(args.workload)
    line = {
        "metric": METRIC,
        "value": r["effective_kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 mfma / f32 accumulate over u8-packed e2m1+e4m3" if w["fmt"] == 1 else
                 "f16 mfma / f32 accumulate over u8-packed int4+f32",
        "data": "synthetic",
        "config": {"workload": r["desc"], "batch": r["batch"], "context": r["context"], "layers": r["layers"],
                   "kv_heads": HKV, "q_heads": HQ, "head_dim": D, "page_size": r["page_size"],
                   "num_splits": r["num_splits"]},
        "tokens_per_s": r["tokens_per_s"],
        "pct_hbm_roofline_step": 100.0 * r["effective_kv_gbs"] / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": r["decode_call_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["decode_call_frac_hbm"],
                     "traffic": counters["traffic_bytes_per_call"] if counters else None,
                     "traffic_source": counters_note,
                     "kernel": "kvq_decode_attention call (decode_kernel + merge_kernel)",
                     "algorithmic_bytes_per_launch": r["kv_bytes_per_layer"],
                     "avg_launch_us": r["decode_call_us"],
                     "median_launch_us": r["decode_call_us_median"],
                     "frac_of_measured_read_ceiling": r["decode_call_gbs"] / ceiling["gbs"]},
        "hbm_read_ceiling": ceiling,
        "hbm_write_ceiling": wc["write"],
        "hbm_copy_ceiling": wc["copy"],
        "mfma_f16_ceiling": mfma,
        "cpu_baseline": cpu,
        "cpu_baseline_per_workload": {
            name: {k: res["cpu_baseline"][k] for k in ("value", "unit", "cores", "sample")}
            | ({"one_thread": res["cpu_baseline"]["one_thread"]} if "one_thread" in res["cpu_baseline"] else {})
            for name, res in [(args.workload, main_res)] + list(secondary.items()) if "cpu_baseline" in res},
        "cpu_baseline_store_dequant": {
            name: res["cpu_baseline_store_dequant"]
            for name, res in [(args.workload, main_res)] + list(secondary.items())
            if "cpu_baseline_store_dequant" in res},
        "quality": quality,
        "store_call_us": r["store_call_us"],
        "populate": r["populate"],
        "calibrate_amax": r.get("calibrate_amax"),
        "secondary": secondary,
    }
    for k in ("chunk_store_us", "split_sweep", "dequant_prefix", "extend_attention", "extend_attention_fused"):
        if k in r:
            line[k] = r[k]
    if "fp8_32k" in secondary and args.workload == "ctx32k":
        f8 = secondary["fp8_32k"]
        line["fp8_comparator"] = {
            "nvfp4_decode_call_us": r["decode_call_us"], "fp8_decode_call_us": f8["decode_call_us"],
            "time_ratio_nvfp4_over_fp8": r["decode_call_us"] / f8["decode_call_us"],
            "byte_ratio_nvfp4_over_fp8": token_head_bytes(1) / token_head_bytes(3),
            "decode_speedup_vs_fp8": f8["decode_call_us"] / r["decode_call_us"],
            "fp8_decode_call_gbs": f8["decode_call_gbs"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
