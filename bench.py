"""Benchmark of the DSA decode hot path on one MI355X.

One step = one dsa_decode_step (lightning-indexer scan + top-2048 + sparse
absorbed-MLA split-KV decode + LSE merge) over the decode batch of 64
requests x 2 query rows (1 + MTP) at a 131072-token context, on seeded
synthetic inputs resident in HBM.  Prints one JSON line.

The step time comes from K back-to-back steps after the W warmup steps
(extended, untimed, until the GPU has been busy for 0.25 s: its clocks ramp
over the first ~40 ms of load; `warmup_run` reports how many ran); then K
more steps run with
the library recording HIP events around each stage on the stream the stage
runs on, and the roofline of the dominant kernel (the indexer scan) is its
algorithmic bytes over the average of those per-launch durations.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--extras]
  python bench.py --summarize-trace DIR            (rocprofv3 --kernel-trace --stats output)
  python bench.py --summarize-counters FETCH_DIR WRITE_DIR   (two rocprofv3 --pmc runs)
  python bench.py --summarize-mfma DIR     (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE)

The line also carries the 32-request 32K-context decode batch, the
4096-row prefill on an empty cache (the sparse step against the masked
multi-head form), and the single-request step (1 row onto 8192 tokens)
warm and cold.  --extras adds more: the prefill-chunk form (4096 query rows
on a 61440-token prefix: indexer FP8 MFMA utilisation), the two-stream
multi-layer-indexer step on a ragged 48-request batch (selection overlap of
adjacent layers, time against the one-stream step), the layer stack, the
short-context form, cache appends, index spaces and the gathered bytes
counted once per request.  --prefill-only times just the prefill form;
--short-prefill-only just the 4096-row prefill on an empty cache (the sparse
step against the masked multi-head step).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode query-tokens/s at 128K ctx (indexer+top-2048+sparse MLA), % HBM peak"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
SETTLE_S = 0.25  # least busy time before any timed region
DECODE_WORKLOAD = 2
PREFILL_WORKLOAD = 3
MLI_WORKLOAD = 4
PROFILES = os.path.join(ROOT, "profiles")
COUNTERS_SUMMARY = os.path.join(PROFILES, "counters.decode-step.decode-b64-mtp1-ctx131072.md")
# the sources that make up the indexer scan kernel: its counters describe it
# only while these are unchanged
INDEXER_SOURCES = ["sparse_attention_02_amd/csrc/indexer.hip",
                   "sparse_attention_02_amd/csrc/device_common.h",
                   "sparse_attention_02_amd/csrc/internal.h",
                   "sparse_attention_02_amd/build.py"]
# FETCH_SIZE reads half the bytes a plain copy kernel of known size moves,
# WRITE_SIZE all of them (the device copy of 2 GiB in this script: FETCH_SIZE
# 1048588 KiB, WRITE_SIZE 2097152 KiB), so the counters are scaled by these
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def indexer_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in INDEXER_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the indexer scan from the committed counter
    summary, or None if there is none or the kernel changed since."""
    try:
        text = open(COUNTERS_SUMMARY).read()
    except OSError:
        return None
    vals = dict(line.split(":", 1) for line in text.splitlines()
                if line.startswith(("source_hash:", "hbm_bytes_per_launch:")))
    if vals.get("source_hash", "").strip() != indexer_source_hash():
        return None
    return float(vals["hbm_bytes_per_launch"])


def _short(name):
    name = name.replace("dsa::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(dsa::")[0].split("(float")[0].split("(unsigned")[0][:60]


def _grid(r):
    """The dispatch's grid size (work-items) from a rocprofv3 CSV row."""
    if r.get("Grid_Size"):
        return r["Grid_Size"]
    dims = [r.get(f"Grid_Size_{a}") for a in "XYZ"]
    return "x".join(d for d in dims if d) or "?"


def summarize_trace(d):
    """Per (kernel, grid size): dispatches of the same kernel on different
    workloads (the 128K batch and the 32K batch share kernels) stay apart."""
    import collections
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(f)):
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        agg[(_short(r["Kernel_Name"]), _grid(r), r.get("Stream_Id", "?"))].append(ns)
    total = sum(sum(v) for v in agg.values())
    print("| kernel | grid (work-items) | stream | calls | avg us | min us | max us | % time |\n"
          "|---|---|---|---|---|---|---|---|")
    for (k, g, st), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {k} | {g} | {st} | {len(v)} | {sum(v) / len(v) / 1e3:.1f} | "
              f"{min(v) / 1e3:.1f} | {max(v) / 1e3:.1f} | {100 * sum(v) / total:.2f} |")


def summarize_counters(fetch_dir, write_dir):
    import collections
    import csv
    import glob
    vals = {}
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == c:
                agg[(_short(r["Kernel_Name"]), _grid(r), r.get("Queue_Id", "?"))].append(
                    float(r["Counter_Value"]))
        vals[c] = {k: (len(v), sum(v) / len(v)) for k, v in agg.items()}
    print("| kernel | grid (work-items) | queue | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | "
          "HBM bytes (scaled) |\n|---|---|---|---|---|---|---|")
    idx = None
    for (k, g, qu), (n, fk) in vals["FETCH_SIZE"].items():
        wk = vals["WRITE_SIZE"].get((k, g, qu), (0, 0.0))[1]
        hbm = 1024 * (FETCH_SCALE * fk + WRITE_SCALE * wk)
        print(f"| {k} | {g} | {qu} | {n} | {fk:.0f} | {wk:.0f} | {hbm:.4g} |")
        # the 128K batch's scan: the largest launch of the page kernel
        if k.startswith("index_score_page") and (idx is None or hbm > idx):
            idx = hbm
    print(f"\nfetch_scale: {FETCH_SCALE}\nwrite_scale: {WRITE_SCALE}")
    if idx is not None:
        print(f"hbm_bytes_per_launch: {idx:.0f}\nsource_hash: {indexer_source_hash()}")


class Step:
    """Buffers and the call of one dsa_decode_step over a batch on the GPU."""

    def __init__(self, b, d, mode=0, attend_idx=None, layer=0, mla_layer=None):
        import torch

        import sparse_attention_02_amd as dsa
        import synth
        self.dsa, self.torch = dsa, torch
        self.d, self.T, self.k = d, b.T, synth.TOPK
        mla_layer = layer if mla_layer is None else mla_layer
        self.mode, self.attend_idx = mode, attend_idx
        self.ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, self.k, 0)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.idx = torch.empty((b.T, self.k), dtype=torch.int32, device="cuda")
        self.out = torch.empty((b.T, 128, 512), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((b.T, 128), dtype=torch.float32, device="cuda")
        self.ix = dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[layer],
                       k_scale=d.k_scale[layer])
        self.ml = dict(q=d.q[mla_layer], kv_cache=d.kv[mla_layer], sm_scale=synth.SM_SCALE)
        self.aux = torch.cuda.Stream() if mode == dsa.DSA_MODE_MLI else None

    def __call__(self, events=None):
        self.dsa.dsa_decode_step(self.d.meta, self.ix, self.ml, self.k, self.mode, 0,
                                 self.attend_idx, self.idx, self.out, self.lse, self.ws,
                                 self.ws_bytes, stream_aux=self.aux, stage_events=events)


def stage_event_sets(n):
    """n sets of 2 * DSA_NUM_STAGES timing events, each created by one record."""
    import torch

    import sparse_attention_02_amd as dsa
    sets = []
    for _ in range(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * dsa.DSA_NUM_STAGES)]
        for e in evs:
            e.record()
        sets.append(evs)
    torch.cuda.synchronize()
    return sets


def timed_steps(step, steps, warmup):
    """Wall time per step over `steps` back-to-back calls, then the mean
    device time of each stage from HIP events that the library records
    around the stages inside a second run of `steps` calls.  (The event
    records cost the step time of their own, so the step time is taken from
    the run without them.)"""
    import torch

    import sparse_attention_02_amd as dsa
    # the W warmup steps, then more untimed steps until the GPU has been busy
    # for SETTLE_S: its clocks ramp over the first ~40 ms of load (0.43 ->
    # 0.37 ms per step on the 128K batch), which a short warmup would leave
    # inside the timed region
    t_w = time.perf_counter()
    n_w = 0
    while n_w < warmup or time.perf_counter() - t_w < SETTLE_S:
        step()
        n_w += 1
        if n_w % 16 == 0:
            torch.cuda.synchronize()
    timed_steps.warmup_run = n_w
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / steps
    sets = stage_event_sets(steps)
    torch.cuda.synchronize()
    for evs in sets:
        step([e.cuda_event for e in evs])
    torch.cuda.synchronize()
    stage_ms = [sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for evs in sets) / steps
                for i in range(dsa.DSA_NUM_STAGES)]
    # device time of each step: from the event before its first stage to the
    # one after its last
    timed_steps.last_step_ms = [evs[0].elapsed_time(evs[-1]) for evs in sets]
    return ms_step, stage_ms


def percentiles(xs):
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])
    return {"p10": float(p10), "p50": float(p50), "p90": float(p90), "n": len(xs)}


def wall_ms(fn, iters, warmup=2, settle_s=0.1):
    """Wall time per call over `iters` calls, after `warmup` calls and at
    least `settle_s` of untimed calls (clock ramp after idle time)."""
    import torch
    t_w = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t_w < settle_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    return 1e3 * (time.perf_counter() - t0) / iters


def copy_bandwidth(gib=2, iters=10):
    """HBM bandwidth of a plain device-to-device copy (read + write bytes)."""
    import torch
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    s.record()
    for _ in range(iters):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    gbs = 2 * n * iters / (s.elapsed_time(e) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def read_ceilings(d, iters=20):
    """HBM read rates this GPU delivers for the scan's bytes: a linear
    streaming read of the whole key pool, and a load-only pass over the key
    stream in the scan's own order (each request's pages through its page
    table, two pages in flight per wave), both from the library's
    measurement kernels (include/dsa_bench.h)."""
    import torch

    import sparse_attention_02_amd as dsa
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    k8 = d.k8[0]
    nbytes = k8.numel()
    L = d.meta.seqlens_k.cpu().numpy()
    key_bytes = int(sum((int(x) + 63) // 64 for x in L)) * 64 * 128

    def timed(fn):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / iters * 1e-3

    t_lin = timed(lambda: dsa.binding.dsa_bench_stream_read(k8, sink))
    t_key = timed(lambda: dsa.binding.dsa_bench_key_stream_read(d.meta, k8, sink))
    return {"linear_read_gbs": nbytes / t_lin / 1e9,
            "key_stream_read_gbs": key_bytes / t_key / 1e9,
            "key_stream_read_us": t_key * 1e6, "key_stream_bytes": key_bytes}


def decode_b32_measure(steps):
    """The 32-request decode batch (2 rows each, 32768-token contexts): step
    time, query-tokens/s and the step's algorithmic bytes over its time."""
    import torch

    import synth
    from sparse_attention_02_amd import accounting
    from synth.device import to_device
    b = synth.make_workload(1)
    d = to_device(b)
    # on a stream of its own (default priority), so that kernel traces keep
    # its launches apart from the 128K batch's launches of the same kernels
    with torch.cuda.stream(torch.cuda.Stream()):
        step = Step(b, d)
        ms_step, stage_ms = timed_steps(step, steps, 5)
    work = accounting.batch_work(b.seqlens_k, b.n_q)
    res = {"workload": b.name, "query_rows": b.T, "ms_per_step": ms_step,
           "query_tokens_per_s": b.T / (ms_step * 1e-3),
           "stages_ms": dict(zip(("index_score", "topk", "attention"), stage_ms)),
           "algorithmic_bytes": work["bytes"],
           "achieved_gbs": work["bytes"] / (ms_step * 1e-3) / 1e9,
           "frac": work["bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "indexer_gbs": work["indexer_bytes"] / (stage_ms[0] * 1e-3) / 1e9,
           "attention_gbs": work["attention_bytes"] / (stage_ms[2] * 1e-3) / 1e9}
    del step, d
    torch.cuda.empty_cache()
    return res


def cpu_baseline(batch, rows, threads):
    """The float64 oracle over a sample of rows: scores, top-k, attention."""
    import numpy as np

    import synth
    from oracle import oracle as O
    meta = O.Meta.of(batch)
    t0 = time.perf_counter()
    vis = [meta.visible(t) for t in rows]
    sc = O.index_score(meta, batch.q8, batch.q_scale, batch.w, batch.k8[0], batch.k_scale[0], rows,
                       ld=max(vis), threads=threads)
    sel, flags, kth, Ks = O.topk(np.nan_to_num(sc, nan=-np.inf), vis, synth.TOPK, threads=threads)
    O.sparse_mla(meta, batch.q[0], batch.kv[0], sel, rows, synth.SM_SCALE, threads=threads)
    return time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def prefill_measure(steps):
    """Prefill-chunk form: the indexer as a dense causal FP8 contraction."""
    import torch

    import synth
    from sparse_attention_02_amd import accounting
    from synth.device import to_device
    b = synth.make_workload(PREFILL_WORKLOAD)
    d = to_device(b)
    step = Step(b, d)
    ms_step, stage_ms = timed_steps(step, steps, 2)
    work = accounting.batch_work(b.seqlens_k, b.n_q)
    tflops = work["indexer_flops"] / (stage_ms[0] * 1e-3) / 1e12
    res = {"workload": b.name, "query_rows": b.T, "ms_per_step": ms_step,
           "stages_ms": dict(zip(("index_score", "topk", "attention"), stage_ms)),
           "indexer_fp8_tflops": tflops, "indexer_mfma_frac": tflops / FP8_PEAK_TFLOPS,
           "attention_bf16_tflops": work["mla_flops"] / (stage_ms[2] * 1e-3) / 1e12}
    del step, d
    torch.cuda.empty_cache()
    return res


def latency_measure(iters=50, flush_mib=512):
    """The single-request decode step (1 row onto 8192 cached tokens): warm
    (inputs in cache from the previous step) and cold (a write of flush_mib
    MiB between steps evicts them); device time per step from HIP events."""
    import torch

    import synth
    from synth.device import to_device
    b = synth.make_workload(0)
    d = to_device(b)
    step = Step(b, d)
    flush = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda")
    res = {"workload": b.name, "query_rows": b.T}
    for name, cold in (("warm", False), ("cold", True)):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        for _ in range(3):
            step()
        for a, c in evs:
            if cold:
                flush.fill_(1.0)
            a.record()
            step()
            c.record()
        torch.cuda.synchronize()
        res[name + "_us"] = percentiles([1e3 * a.elapsed_time(c) for a, c in evs])
    del step, d, flush
    torch.cuda.empty_cache()
    return res


def union_bytes(b, idx):
    """The stricter attention byte count: each request's distinct selected
    latent rows once (its query rows can share reads), instead of per row."""
    import torch
    cu = [int(x) for x in b.cu_seqlens_q]
    total = 0
    for r in range(b.B):
        sel = idx[cu[r]:cu[r + 1]].reshape(-1)
        total += int(torch.unique(sel[sel >= 0]).numel())
    return total * 1152


def summarize_mfma(d, simds=1024):
    """MFMA busy share per kernel from one rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: busy cycles summed over the
    SIMDs / (the kernel's active cycles x SIMDs), the MfmaUtil formula of
    rocprofv3's derived counters.  GRBM_GUI_ACTIVE is reported per XCD and
    summed here, so the per-XCD mean stands for its maximum."""
    import collections
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    n_xcd = 8
    for r in csv.DictReader(open(f)):
        agg[(_short(r["Kernel_Name"]), _grid(r), r.get("Queue_Id", "?"))][
            r["Counter_Name"]].append(float(r["Counter_Value"]))
    print("| kernel | grid (work-items) | queue | dispatches | MFMA busy cycles (sum over SIMDs) "
          "| active cycles per XCD | MFMA busy % |\n|---|---|---|---|---|---|---|")
    for (k, g, qu), v in agg.items():
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES")
        act = v.get("GRBM_GUI_ACTIVE")
        if not busy or not act or sum(busy) == 0:
            continue
        b_avg = sum(busy) / len(busy)
        a_avg = sum(act) / len(act) / n_xcd
        print(f"| {k} | {g} | {qu} | {len(busy)} | {b_avg:.4g} | {a_avg:.4g} | "
              f"{100 * b_avg / (a_avg * simds):.1f} |")


def summarize_issue(d, cus=256):
    """Per kernel, from one rocprofv3 --pmc run of SQ_WAVE_CYCLES,
    SQ_ACTIVE_INST_ANY, SQ_ACTIVE_INST_VALU, SQ_WAIT_INST_ANY, SQ_WAIT_ANY,
    SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT and GRBM_GUI_ACTIVE: the shares of
    the waves' lifetime spent issuing (any instruction, VALU) and waiting
    (for an instruction's operands or a dependency counter, for anything),
    the LDS unit's active share of the kernel's cycles on each CU, and the
    bank-conflict share of those LDS cycles."""
    import collections
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    n_xcd = 8
    for r in csv.DictReader(open(f)):
        agg[(_short(r["Kernel_Name"]), _grid(r), r.get("Queue_Id", "?"))][
            r["Counter_Name"]].append(float(r["Counter_Value"]))
    print("| kernel | grid (work-items) | queue | dispatches | issuing % | VALU issuing % "
          "| waiting on operands % | waiting on anything % | LDS active % | LDS bank conflicts % |"
          "\n|---|---|---|---|---|---|---|---|---|---|")
    for (k, g, qu), v in agg.items():
        m = {c: sum(x) / len(x) for c, x in v.items() if x}
        wc, act = m.get("SQ_WAVE_CYCLES", 0.0), m.get("GRBM_GUI_ACTIVE", 0.0) / n_xcd
        if wc == 0 or act == 0:
            continue
        lds = m.get("SQ_LDS_IDX_ACTIVE", 0.0)
        pct = lambda c: 100 * m.get(c, 0.0) / wc
        print(f"| {k} | {g} | {qu} | {len(v['SQ_WAVE_CYCLES'])} | {pct('SQ_ACTIVE_INST_ANY'):.1f} | "
              f"{pct('SQ_ACTIVE_INST_VALU'):.1f} | {pct('SQ_WAIT_INST_ANY'):.1f} | "
              f"{pct('SQ_WAIT_ANY'):.1f} | {100 * lds / (act * cus):.1f} | "
              f"{100 * m.get('SQ_LDS_BANK_CONFLICT', 0.0) / lds if lds else 0.0:.1f} |")


# bytes one appended token moves: its bf16 key (256) and latent row (1152)
# read; its FP8 key (128), scale (4) and latent row (1152) written
APPEND_BYTES_PER_TOKEN = 2 * 128 + 2 * 576 + 128 + 4 + 2 * 576


def append_measure(iters=200):
    """dsa_cache_append on the decode batch's shape (64 requests x 2 rows
    onto 131072 cached tokens) and on a 4096-row prefill chunk; the page
    pool holds the pages the new rows land on."""
    import numpy as np
    import torch

    import sparse_attention_02_amd as dsa
    res = {}
    rng = np.random.default_rng(0)
    for name, B, n, L in (("decode-b64-mtp1-ctx131072", 64, 2, 131072),
                          ("prefill-4096-on-61440", 1, 4096, 65536)):
        maxp = L // 64
        need = B * ((n + 63) // 64 + 1)
        pool = rng.permutation(need).astype(np.int32)
        pt = np.full((B, maxp), -1, np.int32)
        per = need // B
        for b in range(B):
            first = (L - n) // 64
            pt[b, first:first + per] = pool[b * per:(b + 1) * per][:maxp - first]
        cu = np.arange(0, B * n + 1, n, dtype=np.int32)
        dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
        batch = dsa.Batch(dev(cu), dev(np.full(B, L, np.int32)), dev(pt), need, n, L)
        T = B * n
        k_new = torch.randn((T, 128), device="cuda").to(torch.bfloat16)
        kv_new = torch.randn((T, 576), device="cuda").to(torch.bfloat16)
        k8 = torch.zeros((need, 64, 128), dtype=torch.uint8, device="cuda")
        ks = torch.zeros((need, 64), dtype=torch.float32, device="cuda")
        kv = torch.zeros((need, 64, 576), dtype=torch.bfloat16, device="cuda")
        fn = lambda: dsa.dsa_cache_append(batch, k_new, kv_new, k8, ks, kv)  # noqa: E731
        # a single call is shorter than the host's launch cost, so the calls
        # are captured in a graph and replayed (device time per call)
        fn()
        torch.cuda.synchronize()
        reps = 50
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        ms = wall_ms(g.replay, max(2, iters // reps), warmup=2) / reps
        res[name] = {"tokens": T, "us_per_call": ms * 1e3,
                     "algorithmic_bytes": T * APPEND_BYTES_PER_TOKEN,
                     "gbs": T * APPEND_BYTES_PER_TOKEN / (ms * 1e-3) / 1e9}
    return res


def index_space_measure(b, d, iters=20):
    """Top-k + attention with logical positions against the fused transform
    to physical slots + attention over slots (no page-table lookups in the
    attention), on the bench workload's scores."""
    import torch

    import sparse_attention_02_amd as dsa
    import synth
    T, k = b.T, synth.TOPK
    ld = (int(b.max_seqlen_k) + 63) // 64 * 64
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_index_score(d.meta, d.q8, d.q_scale, d.w, d.k8[0], d.k_scale[0], scores, ld)
    tk = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, d.meta, k)
    mk = dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, d.meta, k)
    ws_t = torch.empty(tk, dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(max(mk, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")

    def logical():
        dsa.dsa_topk(d.meta, scores, ld, k, idx, ws_t, tk)
        dsa.dsa_sparse_mla_decode(d.meta, d.q[0], d.kv[0], idx, k, synth.SM_SCALE, out, lse, 0,
                                  ws_m, mk)

    def paged():
        dsa.dsa_topk_transform(d.meta, scores, ld, k, dsa.DSA_IDX_PAGED, None, idx, ws_t, tk)
        dsa.dsa_sparse_mla_decode_paged(d.meta, d.q[0], d.kv[0], idx, k, synth.SM_SCALE, out, lse,
                                        0, ws_m, mk)

    res = {"logical_ms": [], "paged_ms": []}
    for _ in range(3):  # interleaved rounds
        res["logical_ms"].append(wall_ms(logical, iters))
        res["paged_ms"].append(wall_ms(paged, iters))
    res = {key: min(v) for key, v in res.items()}
    del scores, ws_t, ws_m, idx, out, lse
    torch.cuda.empty_cache()
    return res


def short_measure(steps):
    """The short-context form: 64 requests x 2 rows onto 2048 cached tokens
    (every row keeps all its tokens).  The step selects without scanning and
    attends densely; against it, the scan path the step would otherwise take
    (indexer scores, top-k, sparse attention), same results."""
    import torch

    import sparse_attention_02_amd as dsa
    import synth
    from synth.device import to_device
    b = synth.make_batch([2] * 64, [2048] * 64, seed=83, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    step = Step(b, d)
    k = synth.TOPK
    ld = 2048
    scores = torch.empty((b.T, ld), dtype=torch.float32, device="cuda")
    tk = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, d.meta, k)
    mk = dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, d.meta, k)
    ws_t = torch.empty(tk, dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(max(mk, 1), dtype=torch.uint8, device="cuda")

    def scan_path():
        dsa.dsa_index_score(d.meta, d.q8, d.q_scale, d.w, d.k8[0], d.k_scale[0], scores, ld)
        dsa.dsa_topk(d.meta, scores, ld, k, step.idx, ws_t, tk)
        dsa.dsa_sparse_mla_decode(d.meta, d.q[0], d.kv[0], step.idx, k, synth.SM_SCALE, step.out,
                                  step.lse, 0, ws_m, mk)

    res = {"workload": "decode-b64-mtp1-ctx2048", "query_rows": b.T}
    dense, scan = [], []
    for _ in range(3):
        dense.append(wall_ms(step, steps))
        scan.append(wall_ms(scan_path, steps))
    res["ms_dense_step"], res["ms_scan_path"] = min(dense), min(scan)
    res["speedup"] = res["ms_scan_path"] / res["ms_dense_step"]
    del step, d, scores, ws_t, ws_m
    torch.cuda.empty_cache()
    return res


def short_prefill_measure(steps, n=4096):
    """A prefill chunk on an empty cache (n rows, row j sees j + 1 tokens):
    the sparse step (indexer over the causal n x n block, top-2048, sparse
    attention in the absorbed form) against the masked multi-head form the
    pages give for short prefills (the same indexer and top-k, then the
    expanded attention over the selection: up-projection of the latent
    rows, selection mask, flash attention), and against dense absorbed
    attention over every visible token (dsa_dense_mla_decode).  The sparse
    step and the masked form compute the same attention (up to the W_UV
    projection the absorbed output still needs); the dense absorbed one
    attends more positions beyond 2048 and is only timed."""
    import numpy as np
    import torch

    import sparse_attention_02_amd as dsa
    import synth
    from synth.device import to_device
    from sparse_attention_02_amd import accounting
    b = synth.make_batch([n], [n], seed=84, paging="identity", heavy=64, pool_extra_pages=1)
    d = to_device(b)
    step = Step(b, d)
    mk = dsa.dsa_workspace_size(dsa.DSA_OP_DENSE_MLA, d.meta, 1, 0)
    ws = torch.empty(max(mk, 1), dtype=torch.uint8, device="cuda")

    def dense():
        dsa.dsa_dense_mla_decode(d.meta, d.q[0], d.kv[0], synth.SM_SCALE, step.out, step.lse, 0,
                                 ws, mk)

    # the masked multi-head step: indexer, top-k, expanded attention
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    qn, qr, wk, wv = (dev(a) for a in synth.mha_inputs(85, b.T))
    ld = (n + 63) // 64 * 64
    scores = torch.empty((b.T, ld), dtype=torch.float32, device="cuda")
    tk = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, d.meta, synth.TOPK)
    ws_t = torch.empty(max(tk, 1), dtype=torch.uint8, device="cuda")
    mm = dsa.dsa_workspace_size(dsa.DSA_OP_MASKED_MHA, d.meta, 1, 0)
    ws_m = torch.empty(mm, dtype=torch.uint8, device="cuda")
    idx = torch.empty((b.T, synth.TOPK), dtype=torch.int32, device="cuda")
    out_m = torch.empty((b.T, 128, 128), dtype=torch.bfloat16, device="cuda")
    lse_m = torch.empty((b.T, 128), dtype=torch.float32, device="cuda")

    def select():
        dsa.dsa_index_score(d.meta, d.q8, d.q_scale, d.w, d.k8[0], d.k_scale[0], scores, ld)
        dsa.dsa_topk(d.meta, scores, ld, synth.TOPK, idx, ws_t, tk)

    def masked_attention():
        dsa.dsa_masked_mha_prefill(d.meta, qn, qr, wk, wv, d.kv[0], idx, synth.TOPK,
                                   synth.SM_SCALE, out_m, lse_m, ws_m, mm)

    def masked_step():
        select()
        masked_attention()

    select()
    sparse_ms, dense_ms, mstep_ms, mattn_ms = [], [], [], []
    for _ in range(3):
        sparse_ms.append(wall_ms(step, steps))
        dense_ms.append(wall_ms(dense, steps))
        mstep_ms.append(wall_ms(masked_step, steps))
        mattn_ms.append(wall_ms(masked_attention, steps))
    res = {"workload": f"prefill-{n}-on-empty-cache", "query_rows": b.T,
           "ms_sparse_step": min(sparse_ms), "ms_dense_attention": min(dense_ms),
           "ms_masked_mha_step": min(mstep_ms), "ms_masked_mha_attention": min(mattn_ms)}
    res["sparse_over_dense"] = res["ms_sparse_step"] / res["ms_dense_attention"]
    res["sparse_over_masked_mha_step"] = res["ms_sparse_step"] / res["ms_masked_mha_step"]
    # the masked form's work: every causal pair at the expanded per-pair
    # cost, plus the up-projection of the n cached rows (2 x 128 heads x 128
    # dims x 512 per row, keys and values)
    pairs = n * (n + 1) // 2
    flops = pairs * accounting.expanded_pair_flops() + n * 2 * 2 * 128 * 128 * 512
    res["masked_mha_attention_tflops"] = flops / (res["ms_masked_mha_attention"] * 1e-3) / 1e12
    res["masked_mha_attention_frac_bf16_peak"] = res["masked_mha_attention_tflops"] / 2500.0
    del step, d, ws, scores, ws_t, ws_m
    torch.cuda.empty_cache()
    return res


def mli_measure(steps):
    """Two-stream MLI step vs the same kernels back to back on one stream."""
    import numpy as np
    import torch

    import sparse_attention_02_amd as dsa
    import synth
    from synth.device import to_device
    b = synth.make_workload(MLI_WORKLOAD)
    d = to_device(b)
    first = Step(b, d, layer=0)
    first()
    # one stream: layer 1's indexer + top-k, then attention (layer 0's latent)
    seq = Step(b, d, layer=1, mla_layer=0)
    # two streams: the attention reads layer 0's selection while layer 1's
    # indexer + top-k run beside it
    mli = Step(b, d, mode=dsa.DSA_MODE_MLI, attend_idx=first.idx, layer=1, mla_layer=0)
    ms_seq = wall_ms(seq, steps)
    ms_mli = wall_ms(mli, steps)
    torch.cuda.synchronize()
    a, c = first.idx.cpu().numpy(), mli.idx.cpu().numpy()
    ov = [len(np.intersect1d(a[i][a[i] >= 0], c[i][c[i] >= 0])) / max(1, int((a[i] >= 0).sum()))
          for i in range(b.T)]
    res = {"workload": b.name, "query_rows": b.T, "ms_one_stream": ms_seq,
           "ms_two_streams": ms_mli, "speedup": ms_seq / ms_mli,
           "overlap_mean": float(np.mean(ov)), "overlap_min": float(np.min(ov))}
    res["layers"] = layers_measure(b, d, steps)
    del first, seq, mli, d
    torch.cuda.empty_cache()
    return res


def layers_measure(b, d, steps, n_layers=8):
    """An n_layers stack (alternating the workload's two layers) under the
    multi-layer indexer schedule: every layer indexed one stream at a time
    (retention 1, no MLI: the unmodified model), and IndexCache retention
    1/r with and without MLI."""
    import torch

    import sparse_attention_02_amd as dsa
    import synth
    T, k = b.T, synth.TOPK
    outs = [torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    lses = [torch.empty((T, 128), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, k, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sel = torch.empty((n_layers, T, k), dtype=torch.int32, device="cuda")
    aux = torch.cuda.Stream()
    layers = []
    for i in range(n_layers):
        li = i % len(d.k8)
        layers.append(dict(ix=dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[li],
                                   k_scale=d.k_scale[li]),
                           mla=dict(q=d.q[li], kv_cache=d.kv[li], sm_scale=synth.SM_SCALE),
                           out=outs[i], lse=lses[i]))
    res = {"layers": n_layers}
    for r in (1, 2, 4):
        for mli in (0, 1):
            def run(r=r, mli=mli):
                dsa.dsa_decode_layers(d.meta, layers, k, r, mli, 0, sel, ws, ws_bytes,
                                      stream_aux=aux if mli else None)
            res[f"r{r}_mli{mli}_ms"] = wall_ms(run, max(3, steps // 4))
    base = res["r1_mli0_ms"]
    res["speedup_vs_every_layer"] = {key[:-3]: base / v for key, v in res.items()
                                     if key.endswith("_ms")}
    del outs, lses, ws, sel
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=128,
                    help="query rows the CPU oracle baseline covers (all 128 of the workload: about 10 s)")
    ap.add_argument("--extras", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill-chunk form (for counter runs) and print it")
    ap.add_argument("--short-prefill-only", action="store_true",
                    help="time only the 4096-row prefill on an empty cache (sparse step, masked "
                         "multi-head step, dense absorbed attention) and print it")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-mfma", metavar="DIR")
    ap.add_argument("--summarize-issue", metavar="DIR")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.summarize_mfma:
        return summarize_mfma(args.summarize_mfma)
    if args.summarize_issue:
        return summarize_issue(args.summarize_issue)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DSA decode path here runs on a single "
              "MI355X (no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_02_amd as dsa
    import synth
    from sparse_attention_02_amd import accounting
    from synth.device import to_device

    dsa.lib()
    if args.prefill_only:
        print(json.dumps(prefill_measure(args.steps)), flush=True)
        return
    if args.short_prefill_only:
        print(json.dumps(short_prefill_measure(max(3, args.steps // 10))), flush=True)
        return
    t0 = time.perf_counter()
    b = synth.make_workload(DECODE_WORKLOAD)
    log(f"generated {b.name} in {time.perf_counter() - t0:.1f}s")
    d = to_device(b)
    torch.cuda.synchronize()
    step = Step(b, d)
    ms_step, (ms_idx, ms_topk, ms_attn) = timed_steps(step, args.steps, args.warmup)
    step_dev = percentiles(timed_steps.last_step_ms)
    T = b.T
    work = accounting.batch_work(b.seqlens_k, b.n_q)
    idx_gbs = work["indexer_bytes"] / (ms_idx * 1e-3) / 1e9
    traffic = recorded_traffic()
    attn_gbs = work["attention_bytes"] / (ms_attn * 1e-3) / 1e9
    step_gbs = work["bytes"] / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms | indexer {ms_idx:.3f} ms {idx_gbs:.0f} GB/s | top-k "
        f"{ms_topk:.3f} ms | attention {ms_attn:.3f} ms {attn_gbs:.0f} GB/s | step "
        f"{step_gbs:.0f} GB/s")
    space = index_space_measure(b, d) if args.extras else None
    union = union_bytes(b, step.idx) if args.extras else None
    ceil = read_ceilings(d)
    log(f"read ceilings: linear {ceil['linear_read_gbs']:.0f} GB/s, key stream in scan order "
        f"{ceil['key_stream_read_gbs']:.0f} GB/s ({ceil['key_stream_read_us']:.1f} us)")
    del step, d
    torch.cuda.empty_cache()
    copy_gbs = copy_bandwidth()
    log(f"device copy {copy_gbs:.0f} GB/s")
    b32 = decode_b32_measure(max(20, args.steps // 2))
    log(f"{b32['workload']}: step {b32['ms_per_step']:.3f} ms, "
        f"{b32['query_tokens_per_s']:.0f} query-tokens/s, {b32['achieved_gbs']:.0f} GB/s")
    # the 4096-row prefill on an empty cache: sparse step against the masked
    # multi-head form; and the single-request latency workload
    short_prefill = short_prefill_measure(max(3, args.steps // 20))
    log(f"short prefill {short_prefill}")
    latency = latency_measure()
    log(f"single-request latency {latency}")

    result = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": timed_steps.warmup_run,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "config": {"workload": b.name, "requests": b.B, "query_rows": T,
                   "context": int(b.max_seqlen_k), "topk": synth.TOPK, "page_size": 64,
                   "indexer": "64x128 fp8", "mla": "128 heads x 576 bf16"},
        "step_hbm": {"algorithmic_bytes": work["bytes"], "achieved_gbs": step_gbs,
                     "frac": step_gbs / HBM_PEAK_GBS, "device_copy_gbs": copy_gbs,
                     "linear_read_gbs": ceil["linear_read_gbs"],
                     "key_stream_read_gbs": ceil["key_stream_read_gbs"],
                     "scan_vs_key_stream_read": ceil["key_stream_read_us"] / (ms_idx * 1e3)},
        "stages_ms": {"index_score": ms_idx, "topk": ms_topk, "attention": ms_attn},
        "step_device_ms": step_dev,
        "roofline": {"kernel": "index_score_page_kernel", "bound": "hbm", "achieved": idx_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": idx_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": work["indexer_bytes"]},
        "attention_roofline": {"kernel": "sparse_mla_kernel + mla_merge_kernel", "bound": "hbm",
                               "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": attn_gbs / HBM_PEAK_GBS},
        "decode_b32_mtp1_ctx32768": b32,
        "short_prefill": short_prefill,
        "latency": latency,
    }
    if args.extras:
        result["prefill"] = prefill_measure(max(3, args.steps // 10))
        log(f"prefill {result['prefill']}")
        result["mli"] = mli_measure(max(5, args.steps // 2))
        log(f"mli {result['mli']}")
        result["short_context"] = short_measure(max(5, args.steps // 2))
        log(f"short context {result['short_context']}")
        result["cache_append"] = append_measure()
        log(f"cache append {result['cache_append']}")
        result["index_space"] = space
        result["step_hbm"]["gathered_bytes_union"] = union
        result["step_hbm"]["gathered_bytes_per_row"] = work["attention_gather_bytes"]
        log(f"top-k + attention, logical vs physical-slot indices {result['index_space']}")
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        rows = list(range(min(args.cpu_rows, T)))
        secs = cpu_baseline(b, rows, threads)
        result["cpu_baseline"] = {
            "value": len(rows) / secs, "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"rows 0..{len(rows) - 1} ({len(rows) // 2} requests x 2 rows) of the "
                      f"same workload: float64 index scores over 131072 keys, top-2048, "
                      f"attention; {secs:.1f} s wall",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
        if args.extras:
            # the single-request workload (1 row onto 8192 tokens) on one core
            import synth
            b0 = synth.make_workload(0)
            result["cpu_baseline"]["decode-b1-q1-ctx8192_one_core_s"] = cpu_baseline(b0, [0], 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
