"""Benchmark of the paged GQA attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
    python bench.py --only decode|prefill|copy|append|d256|config2|config4|config5|fp8
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR
    python bench.py --counter-summary PMC_DIR

Prints ONE JSON line.  ``value`` is paged decode throughput in GB/s of
algorithmic HBM bytes (every live K/V element once, plus Q, O and the used
page-table entries) for the decode workload with every sequence at 16,384
tokens: 16 sequences, 32 query heads, 8 KV heads, head_dim 128, BF16, one
query row, page-table stride 1,024 pages.  The prefill half of the metric
(causal attention with sinks, 16 x 8,192 tokens, 64 query / 8 KV heads,
head_dim 64, BF16) is reported in the ``prefill`` object in TFLOP/s.

Inputs are generated on the GPU with the seeded counter-based generator and
are resident in HBM before timing.  Each timed region is K calls on one
stream, bracketed by synchronisation, timed with HIP events on that stream.
The FP64 CPU oracle is timed on a bounded sample of rows of the same
workload (``cpu_baseline``).  The line also carries every other workload:
``config2`` (decode/verify at R = 1, 4, 8, mixed and uniform lengths),
``config4`` (all nine causal-prefill points), ``config5`` (block-sparse
prefill and the dense call at its shape), the 8-bit formats, fragments,
head_dim 256, the K/V append and one GPU's head-parallel shard, each with
its roofline.

``--only`` runs one workload without the CPU baseline, for profiling under
rocprofv3 (``copy`` is a 1 GiB device-to-device copy whose counter readings
calibrate HBM byte counts; ``append`` and ``d256`` print the ``kv_append`` and
``head_dim_256`` objects of the main line).  ``--pmc-summary`` turns two rocprofv3 ``--pmc``
CSV outputs (FETCH_SIZE, then WRITE_SIZE, each over the three ``--only`` runs)
into profiles/hbm_counters.json, which fills ``roofline.traffic``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode achieved HBM GB/s @16K; causal prefill attention TFLOP/s (BF16)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense)
CPU_THREADS = 16
PROFILES = os.path.join(ROOT, "profiles")


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_gqa_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(key: str, src_hash: str, launches_per_call: int = 1):
    """HBM bytes per call from committed rocprofv3 counter summaries, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, "hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(key)
    if not rec or rec.get("src_hash") != src_hash:
        return None
    return rec.get("bytes_per_call")


COPY_BYTES = 1 << 30


def _pmc_rows(directory: str):
    """(kernel name, counter, value) of every dispatch in rocprofv3 CSV output."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]),
                             (path, r.get("Dispatch_Id", ""))))   # ids restart per process
    return rows


def pmc_summary(fetch_dir: str, write_dir: str):
    """HBM bytes per call of the decode and prefill workloads from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for
    the 1 GiB copy; written to profiles/hbm_counters.json."""
    out = {}
    per = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        acc_k = {}
        for kname, cn, v, did in _pmc_rows(d):
            if cn != cname:
                continue
            key = (kname, did)
            acc_k[key] = acc_k.get(key, 0.0) + v   # counters are summed over dimensions
        per[cname] = acc_k
    def run_of(did):   # which --only run a dispatch came from (the CSV file's name)
        return os.path.basename(did[0]).split("_")[0]

    def mean(cname, run, pred):
        vals = [v for (k, did), v in per[cname].items() if run_of(did) == run and pred(k)]
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)
    # the 1 GiB copy: the largest dispatches of the copy run
    def copy_mean(cname):
        vals = [v for (k, did), v in per[cname].items() if run_of(did) == "copy"]
        big = [v for v in vals if v >= 0.9 * max(vals)]
        return sum(big) / len(big)
    f_scale = COPY_BYTES / (copy_mean("FETCH_SIZE") * 1024)
    w_scale = COPY_BYTES / (copy_mean("WRITE_SIZE") * 1024)
    groups = {
        "decode_bf16_16k": ("decode", ("decode_valu", "decode_merge"),
                            _src_hash("decode.hip", "common.h", "attn_internal.h", "api.cpp")),
        "prefill_bf16_8k_b16": ("prefill", ("prefill_mfma",), _src_hash("prefill.hip", "common.h", "attn_internal.h")),
    }
    for key, (run, kernels, h) in groups.items():
        total = 0.0
        parts = {}
        for kn in kernels:
            fm, nf = mean("FETCH_SIZE", run, lambda k, kn=kn: kn in k)
            wm, nw = mean("WRITE_SIZE", run, lambda k, kn=kn: kn in k)
            fb, wb = fm * 1024 * f_scale, wm * 1024 * w_scale
            parts[kn] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": [nf, nw]}
            total += fb + wb
        out[key] = {"src_hash": h, "bytes_per_call": round(total), "kernels": parts}
    out["calibration"] = {"copy_bytes": COPY_BYTES, "fetch_scale": round(f_scale, 4),
                          "write_scale": round(w_scale, 4)}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "hbm_counters.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def counter_summary(directory: str):
    """Mean per dispatch of every counter of this library's kernels in rocprofv3
    --pmc CSV output (counters summed over their dimensions per dispatch)."""
    per = {}
    for kname, cn, v, did in _pmc_rows(directory):
        if "pa::" not in kname:
            continue
        d = per.setdefault(kname, {}).setdefault(cn, {})
        d[did] = d.get(did, 0.0) + v
    out = {k: {cn: {"mean": sum(d.values()) / len(d), "dispatches": len(d)} for cn, d in cs.items()}
           for k, cs in per.items()}
    print(json.dumps(out, indent=1))


def time_calls(fn, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps   # ms per call


SCRUB_BYTES = 512 << 20


def per_call_stats(fn, n: int = 50):
    """Median / p10 / p90 of single calls, each after an untimed 512 MiB read that
    evicts the 256 MiB Infinity Cache and the L2s (HIP events on the current stream)."""
    import torch
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    fn()
    for i in range(n):
        scrub.sum()   # a read: evicts without leaving dirty lines to write back
        ev[i][0].record(s)
        fn()
        ev[i][1].record(s)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    q = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    return {"median": round(q(0.5), 5), "p10": round(q(0.1), 5), "p90": round(q(0.9), 5), "n": n,
            "before_each": "512 MiB scrub read"}


def read_ceiling(ctx, steps: int = 10):
    """Read-only probe rates over 1 GiB: contiguous, and 4 KiB (a bf16 K or V
    page tile at head_dim 128) or 2 KiB (8-bit) tiles in a shuffled order."""
    import torch
    import paged_gqa_attention_amd as pa
    nbytes = 1 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    g = torch.Generator().manual_seed(7)
    order = torch.randperm(nbytes // 4096, generator=g).to(torch.int32).cuda()
    order2 = torch.randperm(nbytes // 2048, generator=g).to(torch.int32).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for name, pat, o in (("contiguous", 0, None), ("paged_4k_tiles", 1, order),
                         ("paged_2k_tiles", 2, order2)):
        ms = time_calls(lambda: pa.attn_debug_read_probe(ctx, buf, pat, o, sink), steps, 2)
        out[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["unit"] = "GB/s"
    return out


def append_bench(ctx, B, n_new, Hkv, d, kv_dtype, src_dtype, steps, warmup):
    """attn_kv_append of n_new rows per sequence into a shuffled page pool whose
    sequences end exactly at the new rows; returns (ms per call, algorithmic bytes)."""
    import torch
    import paged_gqa_attention_amd as pa
    import synth
    pages_per_seq = (n_new + 15) // 16 + 1
    npages = B * pages_per_seq
    g = torch.Generator().manual_seed(11)
    pt = torch.randperm(npages, generator=g).to(torch.int32).view(B, pages_per_seq).cuda()
    lens = torch.full((B,), pages_per_seq * 16 - 5, dtype=torch.int32, device="cuda")
    kp = torch.zeros((npages, Hkv, 16, d), dtype=kv_dtype, device="cuda")
    vp = torch.zeros((npages, Hkv, d, 16), dtype=kv_dtype, device="cuda")
    k, v = synth.append_rows(12, B, n_new, Hkv, d, dtype=src_dtype, device="cuda")
    kv = pa.make_kv(kp, vp, pt, lens, 0.05 if kv_dtype == torch.float8_e4m3fn else 1.0,
                    0.05 if kv_dtype == torch.float8_e4m3fn else 1.0)
    rows = pa.make_rows(k, v)
    ms = time_calls(lambda: pa.attn_kv_append(ctx, kv, rows), steps, warmup)
    elt_src, elt_dst = k.element_size(), kp.element_size()
    nbytes = 2 * B * n_new * Hkv * d * (elt_src + elt_dst) + 4 * B * ((n_new + 15) // 16 + 1)
    return ms, nbytes


def _dev(t, dev):
    return None if t is None else t.to(dev)


def decode_setup(ctx, p, dev="cuda", num_splits=0):
    import torch
    import paged_gqa_attention_amd as pa
    q = p.q.to(dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    io = pa.make_io(q, o)
    kv = pa.make_kv(p.k_pool.to(dev), p.v_pool.to(dev), p.page_table.to(dev),
                    p.seq_lens.to(dev), p.k_scale, p.v_scale, _dev(p.k_vs, dev), _dev(p.v_vs, dev))
    op = pa.make_opts(p.softmax_scale, None if p.sinks is None else p.sinks.to(dev),
                      None, 128, num_splits)
    P, T, W = pa.attn_paged_decode_plan(ctx, io, kv, op)
    ws = torch.empty(max(W, 16), dtype=torch.uint8, device=dev)
    call = lambda: pa.attn_paged_decode(ctx, io, kv, op, ws)
    return call, (P, T), (io, kv, op, ws)


def prefill_setup(ctx, p, dev="cuda"):
    import torch
    import paged_gqa_attention_amd as pa
    q = p.q.to(dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    io = pa.make_io(q, o)
    kv = pa.make_kv(p.k_pool.to(dev), p.v_pool.to(dev), p.page_table.to(dev),
                    p.seq_lens.to(dev), p.k_scale, p.v_scale, _dev(p.k_vs, dev), _dev(p.v_vs, dev))
    mask = None if p.mask is None else p.mask.to(dev)
    op = pa.make_opts(p.softmax_scale, None if p.sinks is None else p.sinks.to(dev), mask,
                      p.mask_block)
    fn = pa.attn_prefill if mask is None else pa.attn_prefill_blocksparse
    return (lambda: fn(ctx, io, kv, op)), (io, kv, op)


def _host_cpu():
    """(CPU model, CPUs the host reports) for the CPU-baseline record."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def _cpu_record(value, unit, used, sample, single):
    model, ncpu = _host_cpu()
    return {"value": value, "unit": unit, "cores": int(used), "kind": "oracle", "sample": sample,
            "cpu_model": model, "host_cpus": ncpu,
            "threads_note": f"{CPU_THREADS} threads: the CPU share of one GPU on this host "
                            f"(it reports {ncpu} CPUs, shared by its GPUs)",
            "single_thread": single}


def cpu_baseline_decode(p, budget_s: float = 12.0):
    """Oracle on a bounded sample of rows, scaled to GB/s of the same workload."""
    import numpy as np
    import oracle
    from paged_gqa_attention_amd import accounting as acc
    op = oracle.OracleProblem(p)
    rows_all = op.all_rows()
    g = np.random.default_rng(0)
    # calibrate on a few rows, then size the sample to the time budget
    n = CPU_THREADS
    sel = rows_all[g.choice(len(rows_all), n, replace=False)]
    t0 = time.perf_counter()
    _, _, used = oracle.attend(op, sel, threads=CPU_THREADS)
    dt = time.perf_counter() - t0
    n2 = int(min(len(rows_all), max(n, n * budget_s / max(dt, 1e-3))))
    sel = rows_all[g.choice(len(rows_all), n2, replace=False)]
    t0 = time.perf_counter()
    _, _, used = oracle.attend(op, sel, threads=CPU_THREADS)
    dt = time.perf_counter() - t0
    total = acc.decode_bytes(p.seq_lens.tolist(), p.q_rows, p.num_q_heads, p.num_kv_heads,
                             p.head_dim, p.kv_dtype, p.q_dtype, p.o_dtype)
    gbs = total * (n2 / len(rows_all)) / dt / 1e9
    # one thread on a fixed subset (the first 8 rows of the sample)
    sel1 = sel[:8]
    t0 = time.perf_counter()
    oracle.attend(op, sel1, threads=1)
    dt1 = time.perf_counter() - t0
    gbs1 = total * (len(sel1) / len(rows_all)) / dt1 / 1e9
    return _cpu_record(round(gbs, 4), "GB/s", used,
                       f"{n2} of {len(rows_all)} output rows (random, seed 0), {dt:.1f} s; "
                       f"bytes scaled by the sampled fraction of rows",
                       {"value": round(gbs1, 4), "unit": "GB/s",
                        "sample": f"{len(sel1)} rows of the same sample, {dt1:.2f} s"})


def cpu_baseline_prefill(p, budget_s: float = 8.0):
    import numpy as np
    import oracle
    from paged_gqa_attention_amd import accounting as acc
    op = oracle.OracleProblem(p)
    g = np.random.default_rng(1)
    B, S, H = p.batch, p.q_rows, p.num_q_heads

    def pick(n):
        return np.stack([g.integers(0, B, n), g.integers(0, S, n), g.integers(0, H, n)],
                        axis=1).astype(np.int32)

    sel = pick(CPU_THREADS * 4)
    t0 = time.perf_counter()
    oracle.attend(op, sel, threads=CPU_THREADS)
    dt = time.perf_counter() - t0
    n2 = int(max(len(sel), len(sel) * budget_s / max(dt, 1e-3)))
    sel = pick(n2)
    t0 = time.perf_counter()
    _, _, used = oracle.attend(op, sel, threads=CPU_THREADS)
    dt = time.perf_counter() - t0
    # flops of the sampled rows: row i of a sequence of length L sees L - S + i + 1 keys
    def flops_of(rows):
        return 4 * p.head_dim * sum(int(p.seq_lens[b]) - S + int(i) + 1 for b, i, _ in rows)
    flops = flops_of(sel)
    # one thread on a fixed subset (the first 16 rows of the sample)
    sel1 = sel[:16]
    t0 = time.perf_counter()
    oracle.attend(op, sel1, threads=1)
    dt1 = time.perf_counter() - t0
    return _cpu_record(round(flops / dt / 1e12, 6), "TFLOP/s", used,
                       f"{n2} random output rows, {dt:.1f} s",
                       {"value": round(flops_of(sel1) / dt1 / 1e12, 7), "unit": "TFLOP/s",
                        "sample": f"{len(sel1)} rows of the same sample, {dt1:.2f} s"})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "copy", "append", "d256", "config2",
                                       "config4", "config5", "fp8"])
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--counter-summary", metavar="DIR")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "a sharded deployment runs one copy per GPU on its share of the heads.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_gqa_attention_amd as pa
    import synth
    from paged_gqa_attention_amd import accounting as acc

    torch.manual_seed(0)
    dev = "cuda"
    if args.only == "copy":
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        ms = time_calls(lambda: b.copy_(a), args.steps, args.warmup)
        print(json.dumps({"workload": "copy 1 GiB", "ms": round(ms, 4),
                          "GB/s": round(2 * COPY_BYTES / ms / 1e6, 1)}), flush=True)
        return
    ctx = pa.attn_open(0)
    if args.only:
        args.no_cpu = True

    # ---------------- decode @16K (the headline) ----------------
    if args.only == "prefill":
        return only_prefill(ctx, args)
    if args.only == "append":
        print(json.dumps(kv_append_summary(ctx, args)), flush=True)
        return
    if args.only == "d256":
        print(json.dumps(wide_summary(ctx, args)), flush=True)
        return
    if args.only == "fp8":
        # the FP8 long-context decode workload alone (B=4 x 65,536 keys, R=4)
        p = synth.config3(device=dev)
        call, (P, T), keep = decode_setup(ctx, p, dev)
        ms = time_calls(call, args.steps, args.warmup)
        b = acc.decode_bytes(p.seq_lens.tolist(), 4, 32, 8, 128, synth.DT_FP8, 2, 2)
        print(json.dumps({"workload": "fp8 decode B=4, 65,536 keys, R=4", "ms": round(ms, 5),
                          "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "splits": P,
                          "bytes_per_call": b}), flush=True)
        return
    if args.only in ("config2", "config4", "config5"):
        fn = {"config2": config2_summary, "config4": config4_summary,
              "config5": config5_summary}[args.only]
        print(json.dumps(fn(ctx, args)), flush=True)
        return
    t_gen = time.perf_counter()
    p = synth.config2(q_rows=1, lens=[16384] * 16, device=dev)
    call, (P, T), keep = decode_setup(ctx, p, dev)
    gen_s = time.perf_counter() - t_gen
    ms = time_calls(call, args.steps, args.warmup)
    nbytes = acc.decode_bytes(p.seq_lens.tolist(), 1, 32, 8, 128, synth.DT_BF16,
                              synth.DT_BF16, synth.DT_BF16)
    gbs = nbytes / (ms * 1e-3) / 1e9
    dec_pc = None if args.only else per_call_stats(call)
    dec_hash = _src_hash("decode.hip", "common.h", "attn_internal.h", "api.cpp")   # api.cpp: the plan
    traffic = _traffic("decode_bf16_16k", dec_hash)
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "decode_valu<bf16,bf16,128,4> + decode_merge (one attn_paged_decode call)",
            "bytes_per_call": nbytes, "per_call_ms": dec_pc}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_decode(p)   # the oracle copies the inputs to host memory
    if args.only == "decode":
        print(json.dumps({"workload": "decode", "ms": round(ms, 5), "GB/s": round(gbs, 1),
                          "splits": P, "roofline": roof}), flush=True)
        return
    del keep, call, p
    torch.cuda.empty_cache()

    # ---------------- prefill 8K x 16 ----------------
    pp = synth.config4(seq_len=8192, batch=16, device=dev)
    pcall, pkeep = prefill_setup(ctx, pp, dev)
    psteps = max(3, args.steps // 2)
    pms = time_calls(pcall, psteps, max(1, args.warmup // 2))
    pre_pc = per_call_stats(pcall, 20)
    flops = acc.attention_flops(acc.causal_pairs(8192, 8192), 64, 64, 16)
    tfs = flops / (pms * 1e-3) / 1e12
    pre_hash = _src_hash("prefill.hip", "common.h", "attn_internal.h")
    prefill = {
        "metric": "causal prefill attention TFLOP/s (BF16)", "value": round(tfs, 1),
        "unit": "TFLOP/s", "ms_per_step": round(pms, 4), "steps": psteps,
        "config": {"workload": "causal prefill + sinks, B=16, S=8192, Hq=64, Hkv=8, d=64, bf16",
                   "flops_per_call": flops},
        "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tfs / BF16_PEAK_TFLOPS, 4),
                     "traffic": _traffic("prefill_bf16_8k_b16", pre_hash),
                     "kernel": "prefill_mfma<bf16,bf16,64,2,false>", "per_call_ms": pre_pc},
    }
    if not args.no_cpu:
        prefill["cpu_baseline"] = cpu_baseline_prefill(pp)
    del pkeep, pcall, pp
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "paged decode, B=16, Hq=32, Hkv=8, d=128, 16,384 tokens each, "
                               "bf16 K/V, 1 query row, page-table stride 1024",
                   "num_splits": P, "tokens_per_split": T, "bytes_per_call": nbytes,
                   "input_gen_s": round(gen_s, 2)},
        "roofline": roof, "cpu_baseline": cpu, "prefill": prefill,
        "read_ceiling": read_ceiling(ctx),
        "kv_append": kv_append_summary(ctx, args),
        "formats": formats_summary(ctx, args),
        "fragments": fragments_summary(ctx, args),
        "head_dim_256": wide_summary(ctx, args),
        "shard": shard_summary(ctx, args),
        "config2": config2_summary(ctx, args),
        "config4": config4_summary(ctx, args),
        "config5": config5_summary(ctx, args),
    }
    print(json.dumps(line), flush=True)


def _kernel_of_decode(rows_per_kv_head, d=128):
    return "decode_valu + decode_merge" if rows_per_kv_head <= 8 else \
        ("decode_mfma + decode_merge" if d != 256 else "attn_wide (verify) + decode_merge")


def config2_summary(ctx, args):
    """Decode / verify as specified: 16 sequences, Hq 32 / Hkv 8, d 128, bf16,
    page-table stride 1,024, R = 1, 4, 8 query rows, lengths U[8192, 16384]
    (seed 202) and, for comparison, all 16,384.  HBM roofline per call."""
    import torch
    import synth
    from paged_gqa_attention_amd import accounting as acc
    out = {"workload": "decode/verify B=16, Hq=32, Hkv=8, d=128, bf16 K/V/Q/O, 16-token pages, "
                       "page-table stride 1024"}
    for tag, lens in (("mixed", None), ("uniform16k", [16384] * 16)):
        for R in (1, 4, 8):
            p = synth.config2(q_rows=R, lens=lens, device="cuda")
            call, (P, T), keep = decode_setup(ctx, p, "cuda")
            ms = time_calls(call, args.steps, args.warmup)
            b = acc.decode_bytes(p.seq_lens.tolist(), R, 32, 8, 128, 2, 2, 2)
            gbs = b / (ms * 1e-3) / 1e9
            out[f"{tag}_R{R}"] = {
                "lengths": "U[8192,16384] seed 202" if lens is None else "16384",
                "ms": round(ms, 5), "splits": P, "tokens_per_split": T,
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "bytes_per_call": b, "kernel": _kernel_of_decode(4 * R)}}
            del keep, call, p
    torch.cuda.empty_cache()
    return out


def config4_summary(ctx, args):
    """Causal prefill with sinks at all nine (S, B) points: Hq 64 / Hkv 8, d 64,
    bf16, S in {1K, 4K, 8K}, B in {1, 4, 16}.  MFMA roofline per call."""
    import torch
    import synth
    from paged_gqa_attention_amd import accounting as acc
    out = {"workload": "causal prefill + sinks, Hq=64, Hkv=8, d=64, bf16, 16-token shuffled pages",
           "kernel": "prefill_mfma<bf16,bf16,64,2,false,false>"}
    for S in (1024, 4096, 8192):
        for B in (1, 4, 16):
            p = synth.config4(seq_len=S, batch=B, device="cuda")
            call, keep = prefill_setup(ctx, p, "cuda")
            ms = time_calls(call, max(3, args.steps // 2), max(1, args.warmup // 2))
            f = acc.attention_flops(acc.causal_pairs(S, S), 64, 64, B)
            tfs = f / (ms * 1e-3) / 1e12
            out[f"S{S}_B{B}"] = {"ms": round(ms, 4),
                                 "roofline": {"bound": "mfma", "achieved": round(tfs, 1),
                                              "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                              "frac": round(tfs / BF16_PEAK_TFLOPS, 4),
                                              "flops_per_call": f}}
            del keep, call, p
            torch.cuda.empty_cache()
    return out


def config5_summary(ctx, args):
    """Block-sparse prefill: 1 x 32,768 tokens, Hq 32 / Hkv 8, d 128, bf16, 128-token
    mask blocks keeping block 0, the diagonal and a Bernoulli(0.1) draw of the
    rest (seed 505).  TFLOP/s on the kept (query, key) pairs; the dense causal
    call at the same shape for comparison."""
    import torch
    import synth
    from paged_gqa_attention_amd import accounting as acc
    p = synth.config5(device="cuda")
    call, keep = prefill_setup(ctx, p, "cuda")
    ms = time_calls(call, max(3, args.steps // 2), max(1, args.warmup // 2))
    m = p.mask[0, 0].cpu()
    rows = [m[qb].nonzero().flatten().tolist() for qb in range(m.shape[0])]
    pairs = acc.mask_pairs(rows, 32768, 128)
    f = acc.attention_flops(pairs, 32, 128, 1)
    tfs = f / (ms * 1e-3) / 1e12
    del keep, call
    p.mask = None
    dcall, dkeep = prefill_setup(ctx, p, "cuda")
    dms = time_calls(dcall, 3, 1)
    df = acc.attention_flops(acc.causal_pairs(32768, 32768), 32, 128, 1)
    dtfs = df / (dms * 1e-3) / 1e12
    del dkeep, dcall, p
    torch.cuda.empty_cache()
    return {"workload": "block-sparse prefill B=1, S=32768, Hq=32, Hkv=8, d=128, bf16, "
                        "mask block 128, keep block 0 + diagonal + Bernoulli(0.1)",
            "kernel": "prefill_mfma<bf16,bf16,128,2,true,false>",
            "ms": round(ms, 4), "kept_pairs_per_head": pairs,
            "kept_fraction_of_causal": round(pairs / acc.causal_pairs(32768, 32768), 4),
            "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tfs / BF16_PEAK_TFLOPS, 4),
                         "flops_per_call": f},
            "dense_same_shape": {"ms": round(dms, 4), "TFLOPs": round(dtfs, 1),
                                 "frac": round(dtfs / BF16_PEAK_TFLOPS, 4),
                                 "flops_per_call": df},
            "sparse_speedup_vs_dense": round(dms / ms, 3)}


def shard_summary(ctx, args):
    """One GPU's share of the headline decode under 8-way head parallelism (one KV
    head, its 4 query heads, 16 x 16,384 tokens).  Its 128 MiB of K/V fit the
    256 MiB Infinity Cache, so the figure of record is the median of single calls
    after a 512 MiB scrub read; back-to-back calls (cache-served) are context."""
    import torch
    import synth
    from paged_gqa_attention_amd import accounting as acc
    out = {"workload": "decode B=16, Hq=4, Hkv=1, d=128, 16,384 tokens, bf16 "
                       "(1/8 of the headline's heads)"}
    for R in (1, 8):
        p = synth.make_decode(202, 16, 4, 1, 128, [16384] * 16, R, kv_dtype=synth.DT_BF16,
                              stride=1024, device="cuda")
        call, (P, T), keep = decode_setup(ctx, p, "cuda")
        nb = acc.decode_bytes(p.seq_lens.tolist(), R, 4, 1, 128, 2, 2, 2)
        pc = per_call_stats(call)
        ms = time_calls(call, args.steps, args.warmup)
        out[f"R{R}"] = {"cold_median_ms": pc["median"], "cold_GBs": round(nb / pc["median"] / 1e6, 1),
                        "cold_hbm_frac": round(nb / pc["median"] / 1e6 / HBM_PEAK_GBS, 4),
                        "warm_back_to_back_GBs": round(nb / ms / 1e6, 1), "splits": P,
                        "bytes_per_call": nb}
        del keep, call, p
    torch.cuda.empty_cache()
    return out


def kv_append_summary(ctx, args):
    """K/V append of a whole prefill (16 x 8,192 rows, Hkv=8, d=64, bf16 -> bf16)
    against the HBM roofline, and one decode step's append (16 x 1 row, d=128)."""
    import torch
    ms, nbytes = append_bench(ctx, 16, 8192, 8, 64, torch.bfloat16, torch.bfloat16,
                              args.steps, args.warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    ms8, nb8 = append_bench(ctx, 16, 8192, 8, 64, torch.float8_e4m3fn, torch.bfloat16,
                            args.steps, args.warmup)
    ms1, _ = append_bench(ctx, 16, 1, 8, 128, torch.bfloat16, torch.bfloat16, args.steps, args.warmup)
    torch.cuda.empty_cache()
    return {"workload": "attn_kv_append 16 x 8192 rows, Hkv=8, d=64, bf16 -> bf16 pool",
            "ms": round(ms, 4), "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "fp8_pool_GBs": round(nb8 / (ms8 * 1e-3) / 1e9, 1),
            "decode_step_16x1_rows_d128_us": round(ms1 * 1e3, 2)}


def formats_summary(ctx, args):
    """The 8-bit cache formats on their own workloads: decode B=4 x 65,536 keys,
    R=4 (MFMA verify path, HBM roofline) and prefill 16 x 8K (MFMA roofline),
    with per-tensor e4m3fn, per-vector-scaled e4m3fn and per-vector-scaled e5m2;
    plus e4m3fn verify at R=8 over 16 x 16,384 keys."""
    import torch
    import synth
    from paged_gqa_attention_amd import accounting as acc
    out = {"decode_workload": "B=4, Hq=32, Hkv=8, d=128, 65,536 keys, R=4, bf16 Q/O",
           "prefill_workload": "B=16, S=8192, Hq=64, Hkv=8, d=64, sinks, bf16 Q/O"}
    flops = acc.attention_flops(acc.causal_pairs(8192, 8192), 64, 64, 16)
    for name, dt, vs in (("fp8", synth.DT_FP8, False), ("fp8_vs", synth.DT_FP8, True),
                         ("bf8_vs", synth.DT_BF8, True)):
        p = synth.config3(device="cuda", kv_dtype=dt, vscales=vs)
        call, (P, T), keep = decode_setup(ctx, p, "cuda")
        ms = time_calls(call, args.steps, args.warmup)
        b = acc.decode_bytes(p.seq_lens.tolist(), 4, 32, 8, 128, dt, 2, 2, per_vector_scales=vs)
        gbs = b / (ms * 1e-3) / 1e9
        del keep, call, p
        torch.cuda.empty_cache()
        pp = synth.config4(seq_len=8192, batch=16, device="cuda", kv_dtype=dt, vscales=vs)
        pcall, pkeep = prefill_setup(ctx, pp, "cuda")
        pms = time_calls(pcall, max(3, args.steps // 2), max(1, args.warmup // 2))
        tfs = flops / (pms * 1e-3) / 1e12
        del pkeep, pcall, pp
        torch.cuda.empty_cache()
        out[name] = {"decode_GBs": round(gbs, 1), "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "decode_ms": round(ms, 4), "decode_bytes": b, "splits": P,
                     "prefill_TFLOPs": round(tfs, 1),
                     "prefill_mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4),
                     "prefill_ms": round(pms, 3)}
    # 8-bit speculative verify: 16 x 16,384 keys, R = 8 (32 rows per KV head,
    # MFMA path with three page pairs in flight per wave), per-tensor e4m3fn
    p = synth.make_decode(202, 16, 32, 8, 128, [16384] * 16, 8, kv_dtype=synth.DT_FP8,
                          q_dtype=synth.DT_BF16, o_dtype=synth.DT_BF16, stride=1024, device="cuda")
    call, (P, T), keep = decode_setup(ctx, p, "cuda")
    ms = time_calls(call, args.steps, args.warmup)
    b = acc.decode_bytes(p.seq_lens.tolist(), 8, 32, 8, 128, synth.DT_FP8, 2, 2)
    gbs = b / (ms * 1e-3) / 1e9
    del keep, call, p
    torch.cuda.empty_cache()
    out["fp8_verify_r8"] = {"workload": "B=16, Hq=32, Hkv=8, d=128, 16,384 keys, R=8, e4m3fn K/V, bf16 Q/O",
                            "kernel": "decode_mfma + decode_merge",
                            "decode_GBs": round(gbs, 1), "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                            "decode_ms": round(ms, 4), "decode_bytes": b, "splits": P}
    return out


def fragments_summary(ctx, args, fragment_bytes=256 << 10, arena_bytes=256 << 20):
    """The headline decode with the K and V pools in 256 KiB fragments placed at
    shuffled slots of 256 MiB arenas and reached through fragment tables, against
    the same call over the contiguous pools (same inputs, same plan)."""
    import torch
    import paged_gqa_attention_amd as pa
    import synth
    from paged_gqa_attention_amd import accounting as acc
    p = synth.config2(q_rows=1, lens=[16384] * 16, device="cuda")
    call, (P, T), (io, kv, op, ws) = decode_setup(ctx, p, "cuda")
    ms0 = time_calls(call, args.steps, args.warmup)
    page_bytes = p.k_pool[0].numel() * p.k_pool.element_size()
    per = fragment_bytes // page_bytes                  # pages per fragment (8 at this shape)
    log2 = per.bit_length() - 1
    tables, views = [], []
    g = torch.Generator().manual_seed(21)
    for pool in (p.k_pool, p.v_pool):
        n = pool.shape[0]
        F = (n + per - 1) // per
        per_arena = arena_bytes // fragment_bytes
        arenas = -(-F // per_arena)
        slots = torch.randperm(arenas * per_arena, generator=g)[:F]
        arena = torch.empty((arenas * per_arena, per) + tuple(pool.shape[1:]), dtype=pool.dtype,
                            device="cuda")
        full = F * per
        src = pool if full == n else torch.cat([pool, pool[: full - n]])
        arena[slots.cuda()] = src.view((F, per) + tuple(pool.shape[1:]))
        tables.append(torch.tensor([arena[int(s_)].data_ptr() for s_ in slots], dtype=torch.int64,
                                   device="cuda"))
        views.append(arena)
    kvf = pa.make_kv(views[0][0], views[1][0], kv._keep[2], kv._keep[3], p.k_scale, p.v_scale,
                     k_fragments=tables[0], v_fragments=tables[1], fragment_pages_log2=log2,
                     num_pages=p.k_pool.shape[0])
    callf = lambda: pa.attn_paged_decode(ctx, io, kvf, op, ws)
    ms1 = time_calls(callf, args.steps, args.warmup)
    nbytes = acc.decode_bytes(p.seq_lens.tolist(), 1, 32, 8, 128, synth.DT_BF16, synth.DT_BF16,
                              synth.DT_BF16)
    out = {"workload": "headline decode (16 x 16,384, bf16, R=1), K/V in 256 KiB fragments of "
                       "256 MiB arenas, shuffled", "pages_per_fragment": per,
           "contiguous_ms": round(ms0, 5), "fragmented_ms": round(ms1, 5),
           "fragmented_GBs": round(nbytes / (ms1 * 1e-3) / 1e9, 1),
           "overhead_pct": round(100.0 * (ms1 / ms0 - 1.0), 2)}
    del views, tables, kvf, call, callf, p
    torch.cuda.empty_cache()
    return out


def wide_summary(ctx, args):
    """head_dim 256, the model layout of four KV heads of 256 (16 query heads):
    decode 16 x 16,384 keys at R = 1 and R = 4 (HBM roofline), causal prefill
    with sinks 4 x 8,192 (MFMA roofline); bf16."""
    import torch
    import synth
    from paged_gqa_attention_amd import accounting as acc
    out = {"decode_workload": "B=16, Hq=16, Hkv=4, d=256, 16,384 keys, bf16",
           "prefill_workload": "B=4, S=8192, Hq=16, Hkv=4, d=256, sinks, bf16"}
    for R in (1, 4):
        p = synth.make_decode(606, 16, 16, 4, 256, [16384] * 16, R, kv_dtype=synth.DT_BF16,
                              stride=1024, device="cuda")
        call, (P, T), keep = decode_setup(ctx, p, "cuda")
        ms = time_calls(call, args.steps, args.warmup)
        b = acc.decode_bytes(p.seq_lens.tolist(), R, 16, 4, 256, 2, 2, 2)
        gbs = b / (ms * 1e-3) / 1e9
        out[f"decode_R{R}"] = {"ms": round(ms, 4), "GBs": round(gbs, 1),
                               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "splits": P}
        del keep, call, p
        torch.cuda.empty_cache()
    pp = synth.make_prefill(607, 4, 16, 4, 256, 8192, sinks=True, device="cuda")
    pcall, pkeep = prefill_setup(ctx, pp, "cuda")
    pms = time_calls(pcall, max(3, args.steps // 2), max(1, args.warmup // 2))
    flops = acc.attention_flops(acc.causal_pairs(8192, 8192), 16, 256, 4)
    tfs = flops / (pms * 1e-3) / 1e12
    out["prefill"] = {"ms": round(pms, 3), "TFLOPs": round(tfs, 1),
                      "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4), "flops_per_call": flops}
    del pkeep, pcall, pp
    torch.cuda.empty_cache()
    return out


def only_prefill(ctx, args):
    import synth
    from paged_gqa_attention_amd import accounting as acc
    pp = synth.config4(seq_len=8192, batch=16, device="cuda")
    pcall, pkeep = prefill_setup(ctx, pp, "cuda")
    pms = time_calls(pcall, args.steps, args.warmup)
    flops = acc.attention_flops(acc.causal_pairs(8192, 8192), 64, 64, 16)
    print(json.dumps({"workload": "prefill", "ms": round(pms, 4),
                      "TFLOP/s": round(flops / (pms * 1e-3) / 1e12, 1)}), flush=True)


if __name__ == "__main__":
    main()
