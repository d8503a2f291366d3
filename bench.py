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
PMC_RUN = ('cd /tmp && export TMPDIR=/tmp && cd "$GRAFT_REPO_ROOT" && timeout -s KILL 150 rocprofv3 --pmc {counter} '
           '--output-format csv -d gpurun_out/pmc_{tag} -o run -- python -u bench.py --workload {workload} '
           '--secondary "" --no-cpu-baseline --steps 5 --warmup 1 --layers 2 --copy-calibration-gib 1')
CALIB_BYTES = 1 << 30


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
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max(int(r["Grid_Size"]) for r in copies)
        per[counter] = {
            "decode_kernel": avg(lambda r: "decode_kernel" in r["Kernel_Name"]),
            "merge_kernel": avg(lambda r: "merge_kernel" in r["Kernel_Name"]),
            "copy_1gib": avg(lambda r: "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) == big),
        }
    f_fac = CALIB_BYTES / 1024 / per["FETCH_SIZE"]["copy_1gib"][0]
    w_fac = CALIB_BYTES / 1024 / per["WRITE_SIZE"]["copy_1gib"][0]
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
             PMC_RUN.format(counter="FETCH_SIZE", tag="fetch", workload=workload),
             PMC_RUN.format(counter="WRITE_SIZE", tag="write", workload=workload),
             f"python bench.py --summarize-pmc gpurun_out/pmc_fetch gpurun_out/pmc_write --workload {workload}",
             "```", "",
             "Per-dispatch averages (KiB as the counters report them):", "",
             "| kernel | FETCH_SIZE | dispatches | WRITE_SIZE | dispatches |", "|---|---|---|---|---|"]
    for k in ("decode_kernel", "merge_kernel", "copy_1gib"):
        fv, fn = per["FETCH_SIZE"][k]
        wv, wn = per["WRITE_SIZE"][k]
        lines.append(f"| {k} | {fv:,.1f} | {fn} | {wv:,.1f} | {wn} |")
    lines += ["",
              f"Calibration: a 1 GiB device copy (1,048,576 KiB read and written) reads "
              f"{per['FETCH_SIZE']['copy_1gib'][0]:,.1f} KiB of FETCH_SIZE and "
              f"{per['WRITE_SIZE']['copy_1gib'][0]:,.1f} KiB of WRITE_SIZE, so the factors are "
              f"{f_fac:.4f} (fetch) and {w_fac:.4f} (write).", "",
              f"Traffic per decode call (decode + merge kernels): {traffic:,.0f} B = "
              f"{traffic / algo:.4f} x the algorithmic {algo:,} B of packed KV.", "",
              "```json", json.dumps(rec, indent=1), "```", ""]
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
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="target wall time of one CPU-oracle run (the median of 3 is reported)")
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
        self.pages_per_seq = -(-L // P)
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
    B, L, P = w["batch"], w["ctx"], w["page"]
    pps = -(-L // P)
    bt = inputs.page_tables(workload_id, B, pps, B * pps, shuffled=w["shuffled"])
    return torch.from_numpy(bt).to("cuda")


def run_workload(torch, kvq, inputs, name, steps, warmup, n_layers, keep_for_cpu=False, num_splits=0):
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
    # chunked-prefill store (160K): 64 new tokens per sequence at positions L..L+63
    chunk = None
    if w.get("chunk"):
        n = w["chunk"]
        g = torch.Generator(device="cuda")
        g.manual_seed(inputs.seed_int(wid, 0, 40))
        kc = torch.randn((B * n, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
        vc = torch.randn((B * n, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
        # write into the sequences' own last pages (rows 0..63 of spare capacity are not
        # needed: the chunk overwrites the final 64 cached positions of each sequence)
        t = torch.arange(L - n, L, device="cuda")
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
    keep = layers[0] if keep_for_cpu else None
    del layers, ws, chunk
    torch.cuda.empty_cache()
    return res, keep


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


def cpu_baseline(torch, lay, w, target_s):
    """The CPU oracle on a sample of the same cache: whole sequences of layer 0
    (their packed pages copied to the host), all 24 query heads."""
    import numpy as np
    import oracle
    P, L = w["page"], w["ctx"]
    pps = -(-L // P)

    def run(nseq):
        pages = lay.bt[:nseq].reshape(-1).long()
        pool = oracle.Pool(w["fmt"], nseq * pps, P, HKV, D)
        pool.data[:] = lay.cache.pool[pages].cpu().numpy()
        bt = np.arange(nseq * pps, dtype=np.int32).reshape(nseq, pps)
        q = lay.q[:nseq].float().cpu().numpy()
        t = time.perf_counter()
        pool.decode_attention(q, bt, np.full(nseq, L, np.int32))
        return time.perf_counter() - t

    t1 = run(1)  # also the warm-up
    n = int(max(1, min(w["batch"], round(target_s / max(t1, 1e-3)))))
    runs = sorted(run(n) for _ in range(3))
    t = runs[1]  # median of 3
    nbytes = n * L * HKV * token_head_bytes(w["fmt"])
    threads = oracle.num_threads()
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((x.split(":", 1)[1].strip() for x in f if x.startswith("model name")), "")
    except OSError:
        pass
    # the same oracle on one thread, one sequence
    oracle.set_num_threads(1)
    try:
        t_one = run(1)
    finally:
        oracle.set_num_threads(threads)
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"1 layer, {n} of {w['batch']} sequences x {L} tokens, all {HQ} query heads, fp64 attention "
                      f"over the same packed pages (median of 3 runs of {t:.1f} s after a warm-up)",
            "seconds": t, "seconds_runs": runs, "nproc": os.cpu_count(), "cpu_model": cpu_model,
            "tokens_per_s_16_layers_extrapolated": n / (t * LAYERS),
            "extrapolation": "one layer timed, x16 layers assumed for the stack",
            "one_thread": {"value": L * HKV * token_head_bytes(w["fmt"]) / t_one / 1e9, "unit": "GB/s",
                           "sample": f"1 sequence, 1 thread ({t_one:.1f} s)"}}


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
    main_res, keep = run_workload(torch, kvq, inputs, args.workload, args.steps, args.warmup, args.layers,
                                  keep_for_cpu=not args.no_cpu_baseline, num_splits=args.num_splits)
    print(f"[bench] {args.workload}: step {main_res['step_ms']:.3f} ms, decode call {main_res['decode_call_us']:.1f} us "
          f"({main_res['decode_call_gbs']:.0f} GB/s), {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    time.sleep(args.cooldown)  # the ceiling from the same idle state as the headline
    ceiling = read_ceiling(torch, kvq, args.steps)
    print(f"[bench] plain streaming read: {ceiling['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        t1 = time.time()
        # same timing protocol as the headline, from the same idle GPU state
        torch.cuda.synchronize()
        time.sleep(args.cooldown)
        r, _ = run_workload(torch, kvq, inputs, name, args.secondary_steps or args.steps, args.warmup, args.layers)
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
    cpu = None
    if keep is not None:
        cpu = cpu_baseline(torch, keep, WORKLOADS[args.workload], args.cpu_seconds)
        print(f"[bench] cpu oracle: {cpu['value']:.4f} GB/s on {cpu['cores']} threads", file=sys.stderr, flush=True)
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
        "cpu_baseline": cpu,
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
