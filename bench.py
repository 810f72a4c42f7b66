#!/usr/bin/env python3
"""Benchmark of the CSA layer hot path on one MI355X.

One step = one full pass of the path over the V4-Flash CSA prefill workload
(n = 8192 tokens, c = 512, n_h = 64, n_h^I = 64, c^I = 128, m = 4, k = 512,
w = 128, bf16): main compressor -> indexer compressor -> lightning indexer +
top-k -> sparse shared-KV MQA attention.  Inputs are synthetic (seeded) and
resident in HBM before timing starts.

Prints one JSON line: tokens/s for the whole step, the roofline position of the
dominant kernel (the sparse attention, measured with HIP events on its stream),
and the float64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the MQA attention kernel, from two rocprofv3 PMC passes
# (FETCH_SIZE, WRITE_SIZE) over this benchmark, each divided by the factor the same
# counter reads on a plain device copy of known size (--copy-calibration).  Valid only
# for the kernel source it was measured on: with any other source the figure is null.
TRAFFIC_SOURCE = "compressed_sparse_attention_v4a_amd/csrc/attention_mfma.hip"
TRAFFIC = {"sha256": "36233cb6076ed39974942adfd7fce72bf080cee1ae425be4fdcbc97c70ddec79",
           "fetch_bytes": 859598890, "write_bytes": 536870912}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 4 device-to-device copies of MIB MiB (counter calibration)")
    return ap.parse_args()


def source_sha256(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_bytes():
    if TRAFFIC is None or TRAFFIC.get("sha256") != source_sha256(TRAFFIC_SOURCE):
        return None
    return TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]


def copy_calibration(mib):
    import torch
    nbytes = mib << 20
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "copies": 4}))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import synth
    from compressed_sparse_attention_v4a_amd import binding as B
    from compressed_sparse_attention_v4a_amd import costmodel, ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    cfg = synth.configs.workload("csa_prefill_flash_8k")
    n, c, n_h, n_hI, cI, m, k, w = (cfg[x] for x in ("n", "c", "n_h", "n_hI", "cI", "m", "k", "w"))
    E = n // m
    log(f"generating inputs ({cfg['name']})")
    d = synth.configs.gen_csa_prefill(cfg)
    up = lambda x: ops.upload(x, None, dev)
    T = {key: up(d[key]) for key in ("C", "Z", "B", "CI", "ZI", "BI", "q", "qI", "wI", "local",
                                     "gamma", "gammaI")}
    kv = torch.empty(1, E, c, dtype=torch.bfloat16, device=dev)
    KI = torch.empty(1, E, cI, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(1, n, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, n, dtype=torch.int32, device=dev)
    out = torch.empty(1, n, n_h, c, dtype=torch.bfloat16, device=dev)
    ws_i_bytes = B.v4a_indexer_topk_workspace(1, n, 0, n_hI, cI, m, k, B.BF16)
    ws_i = ops.workspace(ws_i_bytes, dev)
    ws_a_bytes = B.v4a_sparse_mqa_prefill_workspace(1, 0, n, 0, n, n_h, c, k, w, B.BF16)
    ws_a = ops.workspace(ws_a_bytes, dev)
    stream = torch.cuda.current_stream()
    q4 = T["q"].view(1, n, n_h, c)
    qI4 = T["qI"].view(1, n, n_hI, cI)
    wI3 = T["wI"].view(1, n, n_hI)
    loc3 = T["local"].view(1, n, c)

    def step(ev=None, stages=None):
        if stages is not None:
            stages[0].record(stream)
        B.v4a_compress(T["C"], T["Z"], B.BF16, T["B"], 1, n, 0, 0, n, c, m, 1, T["gamma"], 1e-6,
                       64, 10000.0, kv, None, B.BF16, E, stream)
        if stages is not None:
            stages[1].record(stream)
        B.v4a_compress(T["CI"], T["ZI"], B.BF16, T["BI"], 1, n, 0, 0, n, cI, m, 1, T["gammaI"],
                       1e-6, 0, 10000.0, KI, None, B.BF16, E, stream)
        if stages is not None:
            stages[2].record(stream)
        B.v4a_indexer_topk(qI4, None, KI, None, B.BF16, wI3, 1, n, 0, n_hI, cI, m, k, E, idx, cnt,
                           None, ws_i, ws_i_bytes, stream)
        if ev is not None:
            ev[0].record(stream)
        B.v4a_sparse_mqa_prefill(q4, kv, loc3, 0, n, idx, cnt, None, T["gamma"], T["gamma"], 1e-6,
                                 64, 10000.0, 0.0, 1, 0, n, n_h, c, k, w, E, out, B.BF16, ws_a,
                                 ws_a_bytes, stream)
        if ev is not None:
            ev[1].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    attn_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    # one extra, separately timed step for the per-stage split (not part of the timed region)
    st = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev_extra = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    step(ev_extra, st)
    torch.cuda.synchronize()
    stages_ms = {"compress_main": round(st[0].elapsed_time(st[1]), 4),
                 "compress_index": round(st[1].elapsed_time(st[2]), 4),
                 "indexer_topk": round(st[2].elapsed_time(ev_extra[0]), 4),
                 "sparse_mqa": round(ev_extra[0].elapsed_time(ev_extra[1]), 4)}

    counts = costmodel.csa_prefill_counts(n, m, k, w, n_h, c, n_hI, cI)
    attn_tflops = counts["attn_flops"] / (attn_ms * 1e-3) / 1e12
    tokens_per_s = n / (ms_step * 1e-3)
    line = {
        "metric": "CSA layer tokens/s (prefill) and us/token (decode) at 128K ctx; % roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "csa_prefill_v4_flash_n8192", "n": n, "c": c, "n_h": n_h,
                   "n_hI": n_hI, "cI": cI, "m": m, "k": k, "w": w, "global_batch": 1,
                   "seq_len": n, "parallelism": "none"},
        "roofline": {
            "kernel": "v4a_sparse_mqa_prefill",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_bytes(),
            "algorithmic_flops_per_launch": counts["attn_flops"],
            "avg_launch_ms": round(attn_ms, 4),
        },
        "stages_ms": stages_ms,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d, cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def cpu_baseline(d, cfg, target_s):
    """The float64 oracle on a bounded, stratified sample of the same workload: all
    compressed entries (both instances), then indexer scores, top-k and attention for
    S evenly spaced queries.  Reported as tokens/s over the sampled queries."""
    import numpy as np

    import oracle

    n, c, n_h, n_hI, cI, m, k, w = (cfg[x] for x in ("n", "c", "n_h", "n_hI", "cI", "m", "k", "w"))
    E = n // m
    dec = oracle.decode_bf16
    t_start = time.perf_counter()
    kv = oracle.compress(dec(d["C"]), dec(d["Z"]), d["B"], tok_base=0, i_begin=0, i_end=E, c=c,
                         m=m, overlap=True, gamma=d["gamma"], rope_dims=64)
    KI = oracle.compress(dec(d["CI"]), dec(d["ZI"]), d["BI"], tok_base=0, i_begin=0, i_end=E, c=cI,
                         m=m, overlap=True, gamma=d["gammaI"])
    local = dec(d["local"])
    t_fixed = time.perf_counter() - t_start

    def run(nchunks, G):
        # contiguous chunks of G queries (the oracle parallelises over a chunk's queries)
        t0 = time.perf_counter()
        for s0 in np.linspace(0, n - G, nchunks).astype(int):
            s0 = int(s0)
            Et = (s0 + G) // m
            sc = oracle.index_scores(dec(d["qI"][s0:s0 + G]), KI[:max(Et, 1)], d["wI"][s0:s0 + G],
                                     t0=s0, m=m, ld=max(Et, 1))
            idx, cnt = oracle.topk(sc, t0=s0, m=m, k=k)
            lb = max(0, s0 - w + 1)
            oracle.attend_csa(dec(d["q"][s0:s0 + G]), kv, local[lb:s0 + G], idx, cnt, loc_base=lb,
                              t0=s0, w=w, q_gamma=d["gamma"], kv_gamma=d["gamma"], q_norm=True,
                              kv_norm=True, rope_dims=64)
        return time.perf_counter() - t0

    tp = run(16, 16)  # probe: 256 queries
    S = int(max(256, min(n, 256 * (target_s - t_fixed) / max(tp, 1e-3))))
    G = max(16, S // 16)
    ts = run(16, G)
    S = 16 * G
    # per-token cost = sampled query cost + the compressor work amortised over all n tokens
    per_tok = ts / S + t_fixed / n
    return {"value": round(1.0 / per_tok, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{S} of {n} queries in 16 evenly spaced chunks of {G} (indexer scores, "
                      f"top-k, attention) + all {E} entries of both compressors; float64",
            "seconds": round(ts + t_fixed, 2)}


if __name__ == "__main__":
    main()
