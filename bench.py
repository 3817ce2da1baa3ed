"""Benchmark of the DSA decode hot path on one MI355X.

One step = one dsa_decode_step (lightning-indexer scan + top-2048 + sparse
absorbed-MLA split-KV decode + LSE merge) over the decode batch of 64
requests x 2 query rows (1 + MTP) at a 131072-token context, on seeded
synthetic inputs resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
WORKLOAD = 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_stream(fn, iters, warmup=2):
    """Average ms of fn() over iters, by HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DSA decode path here runs on a single "
              "MI355X (no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_02_amd as dsa
    import synth
    from sparse_attention_02_amd import accounting
    from synth.device import to_device

    dsa.lib()
    t0 = time.perf_counter()
    b = synth.make_workload(WORKLOAD)
    log(f"generated {b.name} in {time.perf_counter() - t0:.1f}s")
    d = to_device(b)
    torch.cuda.synchronize()
    k, T = synth.TOPK, b.T
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    ix = dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[0], k_scale=d.k_scale[0])
    ml = dict(q=d.q[0], kv_cache=d.kv[0], sm_scale=synth.SM_SCALE)

    def step():
        dsa.dsa_decode_step(d.meta, ix, ml, k, dsa.DSA_MODE_FUSED, 0, None, idx, out, lse, ws,
                            ws_bytes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = 1e3 * elapsed / args.steps
    log(f"step {ms_step:.3f} ms")

    # dominant kernel: the indexer scan, timed alone by HIP events on its stream
    ld = (b.max_seqlen_k + 63) // 64 * 64
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    ms_idx = time_stream(lambda: dsa.dsa_index_score(d.meta, d.q8, d.q_scale, d.w, d.k8[0],
                                                     d.k_scale[0], scores, ld), 20)
    tk_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, d.meta, k)
    ms_topk = time_stream(lambda: dsa.dsa_topk(d.meta, scores, ld, k, idx, ws, tk_bytes), 20)
    mla_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, d.meta, k, 0)
    ms_mla = time_stream(lambda: dsa.dsa_sparse_mla_decode(d.meta, d.q[0], d.kv[0], idx, k,
                                                           synth.SM_SCALE, out, lse, 0, ws,
                                                           mla_bytes), 20)
    work = accounting.batch_work(b.seqlens_k, b.n_q)
    idx_gbs = work["indexer_bytes"] / (ms_idx * 1e-3) / 1e9
    attn_gbs = work["attention_bytes"] / (ms_mla * 1e-3) / 1e9
    step_gbs = work["bytes"] / (ms_step * 1e-3) / 1e9
    log(f"indexer {ms_idx:.3f} ms {idx_gbs:.0f} GB/s | top-k {ms_topk:.3f} ms | "
        f"attention {ms_mla:.3f} ms {attn_gbs:.0f} GB/s | step {step_gbs:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "config": {"workload": b.name, "requests": b.B, "query_rows": T,
                   "context": int(b.max_seqlen_k), "topk": k, "page_size": 64,
                   "indexer": "64x128 fp8", "mla": "128 heads x 576 bf16"},
        "step_hbm": {"algorithmic_bytes": work["bytes"], "achieved_gbs": step_gbs,
                     "frac": step_gbs / HBM_PEAK_GBS},
        "stages_ms": {"index_score": ms_idx, "topk": ms_topk, "sparse_mla": ms_mla},
        "roofline": {"kernel": "index_score_kernel", "bound": "hbm", "achieved": idx_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": idx_gbs / HBM_PEAK_GBS,
                     "traffic": None},
        "attention_roofline": {"bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        rows = list(range(min(args.cpu_rows, T)))
        secs = cpu_baseline(b, rows, threads)
        result["cpu_baseline"] = {
            "value": len(rows) / secs, "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"rows 0..{len(rows) - 1} ({len(rows) // 2} requests x 2 rows) of the "
                      f"same workload: float64 index scores over 131072 keys, top-2048, "
                      f"attention; {secs:.1f} s wall"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
