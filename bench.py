"""Benchmark: selected-block attention at 75 % sparsity on the 48k-token
edge-video-shaped workload, one MI355X.

One step = the whole hot path over one synthetic input set already in HBM:
block selection (pooling + scores + top-k) followed by block-sparse
attention. Prints one JSON line. ``value`` is effective attention TFLOP/s of
the step (4 * block_q * block_k * head_dim FLOP per selected tile, selection
time included in the denominator); the attention kernel alone is reported in
``roofline`` against the bf16 MFMA peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload edge48k]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 (256 CU x 4096 FLOP/clk x 2.4 GHz)
ATTN_KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_blocks_amd", "csrc", "attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_edge48k_traffic.txt")

WORKLOAD_TEXT = {
    "edge48k": ("edge-video-shaped sparse attention: batch 1, 32 query / 8 KV heads, head_dim 128, "
                "512 protected prefix + 48,360 generation tokens (31x30x52) padded to 48,384, "
                "64x64 blocks, 75% target sparsity (191 of 764 KV blocks per row)"),
    "dense8k": "dense GQA: batch 1, 32 query / 8 KV heads, head_dim 128, 8,192 tokens, 128x128 blocks",
    "video720p": ("720p-video-shaped sparse attention: 32/8 heads, head_dim 128, 512 prefix + "
                  "172,800 generation tokens, 128x128 blocks, 75% target"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="edge48k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--input-sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=756)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="also run one plain device copy of BYTES bytes (a known-size kernel "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    with open(ATTN_KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(case, keep, n_blocks):
    """The fp64 oracle, untouched, on a bounded sample of the same workload:
    selection for query head 0 (all its query blocks) and attention for the
    first ``n_blocks`` query blocks of that head. Reported as effective
    TFLOP/s of the sampled blocks, the selection time pro-rated to them."""
    import oracle
    from threadpoolctl import threadpool_info

    lay = case.layout
    hq, hkv = lay["num_q_heads"], lay["num_kv_heads"]
    g = 0
    lay1 = dict(lay, num_q_heads=1, num_kv_heads=1)
    q1 = np.ascontiguousarray(case.q[:, :, 0:1])
    k1 = np.ascontiguousarray(case.k[:, :, g:g + 1])
    v1 = np.ascontiguousarray(case.v[:, :, g:g + 1])
    t0 = time.perf_counter()
    idx, cnt = oracle.select(lay1, q1, k1, keep)
    t_sel = time.perf_counter() - t0
    nq = lay["q_len"] // lay["block_q"]
    n_blocks = min(n_blocks, nq)
    idx_s = idx[:, :, :n_blocks]
    cnt_s = cnt[:, :, :n_blocks]
    lay_s = dict(lay1, q_len=n_blocks * lay["block_q"], q_valid=min(lay["q_valid"], n_blocks * lay["block_q"]))
    t0 = time.perf_counter()
    oracle.attend(lay_s, q1[:, :lay_s["q_len"]], k1, v1, idx_s, cnt_s)
    t_att = time.perf_counter() - t0
    flops = 4.0 * lay["block_q"] * lay["block_k"] * lay["head_dim"] * float(cnt_s.sum())
    t = t_sel * n_blocks / nq + t_att
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    return {
        "value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"query head 0 of {hq}: selection over all {nq} query blocks "
                   f"({t_sel:.2f} s, pro-rated) + fp64 attention for {n_blocks} query blocks "
                   f"({t_att:.2f} s); effective FLOPs of those blocks"),
        "seconds": round(t_sel + t_att, 2),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the kernel on one GPU's share); "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_blocks_amd as bsa
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    sets = []
    for layer in range(max(1, args.input_sets)):
        case = synth.make_config(name, layer=layer)
        t = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
             for a in (case.q, case.k, case.v)]
        sets.append((case, t))
        print(f"bench: input set {layer} of {name} ready", file=sys.stderr, flush=True)
    case0 = sets[0][0]
    lay = case0.layout
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, case0.sparsity)
    b, hq = lay["batch"], lay["num_q_heads"]
    idx = torch.empty((b, hq, nq, keep), dtype=torch.int32, device=dev)
    cnt = torch.empty((b, hq, nq), dtype=torch.int32, device=dev)
    ws = torch.empty(max(bsa.select_workspace_size(lay), 256), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(t[0]) for _, t in sets]
    stream = torch.cuda.current_stream()

    def step(s, ev=None):
        _, (q, k, v) = sets[s]
        if ev is not None:
            ev[0].record(stream)
        bsa.select_blocks(q, k, lay, keep, keep, block_idx=idx, block_cnt=cnt, workspace=ws,
                          stream=stream)
        if ev is not None:
            ev[1].record(stream)
        bsa.block_sparse_attention(q, k, v, idx, cnt, lay, out=outs[s], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Warm up every layout (each input set) before timing.
    for w in range(max(args.warmup, len(sets))):
        step(w % len(sets))
    torch.cuda.synchronize()
    # Expected sparse dispatch: every real query block keeps exactly `keep` blocks.
    real_rows = (torch.arange(nq, device=dev) * lay["block_q"] < lay["q_valid"])
    if not bool((cnt[:, :, real_rows] == keep).all()):
        raise RuntimeError("unexpected block counts after selection")
    selected_tiles = float(cnt.sum().item())
    eff_flops = 4.0 * lay["block_q"] * lay["block_k"] * lay["head_dim"] * selected_tiles

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s % len(sets), events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_ms = [e[0].elapsed_time(e[1]) for e in events]
    att_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    att_avg = float(np.mean(att_ms))
    att_tflops = eff_flops / (att_avg * 1e-3) / 1e12
    value = eff_flops / (ms_per_step * 1e-3) / 1e12

    traffic = recorded_traffic()
    result = {
        "metric": "effective attention TFLOP/s + ms/call at 75% sparsity, 48k tokens, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; no model weights or videos)",
        "config": {"workload": WORKLOAD_TEXT[name], "name": name, "batch": b,
                   "q_heads": hq, "kv_heads": lay["num_kv_heads"], "head_dim": lay["head_dim"],
                   "q_len": lay["q_len"], "kv_len": lay["kv_len"],
                   "block": f"{lay['block_q']}x{lay['block_k']}", "kv_blocks": nk,
                   "kept_blocks": keep, "sparsity_pct": case0.sparsity,
                   "input_sets": len(sets)},
        "attn_ms_per_call": round(att_avg, 4),
        "attn_ms_min": round(float(np.min(att_ms)), 4),
        "attn_tflops": round(att_tflops, 2),
        "select_ms_per_call": round(float(np.mean(sel_ms)), 4),
        "effective_tflop_per_call": round(eff_flops / 1e12, 4),
        "roofline": {
            "kernel": "attn_fwd_kernel<128,64,64,sparse>",
            "bound": "mfma",
            "achieved": round(att_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case0, keep, args.cpu_sample_blocks)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
