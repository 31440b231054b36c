"""Benchmark: selected-block attention at 75 % sparsity on the 48k-token
edge-video-shaped workload, one MI355X.

One step = the whole hot path over synthetic inputs already in HBM: block
selection (pooling + scores + top-k) followed by block-sparse attention
(``edge48k``, ``video720p``, and at the 48k token shape ``edge48k_256x128``
with 256x128 blocks, ``mha64_48k``, ``mqa48k`` and ``edge48k_cp8``, one GPU's
4-head share of the head-sharded workload); dense attention alone
(``dense8k``); causal dense attention of the understanding stream over itself
(``undcausal``); or the 36-layer two-stream schedule (``twostream``): per
layer the understanding stream's causal self-attention, then the generation
stream over cat(und, gen), dense for the first 8 layers and selected-sparse
for the other 28. Prints one JSON line. ``value`` is effective attention
TFLOP/s of the step (4 * block_q * block_k * head_dim FLOP per selected tile,
selection time included in the denominator); the attention kernel alone is
reported in ``roofline`` against the bf16 MFMA peak, timed with HIP events on
the stream the kernels are launched on.

After the timed region the step runs back to back for a few more seconds
while the driver's energy counter is read (``power``: average socket power
against the power cap, per-XCD shader clocks); these launches are not timed.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload edge48k]
                       [--no-cpu-baseline] [--power-seconds S]
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
FP64_PEAK_TFLOPS = 78.6          # MI355X fp64 (vector and matrix)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
ATTN_KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_blocks_amd", "csrc", "attention.hip")
SELECT_KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_blocks_amd", "csrc", "select.hip")
PROFILES = os.path.join(ROOT, "profiles")

WORKLOAD_TEXT = {
    "edge48k": ("edge-video-shaped sparse attention: batch 1, 32 query / 8 KV heads, head_dim 128, "
                "512 protected prefix + 48,360 generation tokens (31x30x52) padded to 48,384, "
                "64x64 blocks, 75% target sparsity (191 of 764 KV blocks per row)"),
    "dense8k": "dense GQA: batch 1, 32 query / 8 KV heads, head_dim 128, 8,192 tokens, 128x128 blocks",
    "video720p": ("720p-video-shaped sparse attention: 32/8 heads, head_dim 128, 512 prefix + "
                  "172,800 generation tokens (48x45x80), 128x128 blocks, 75% target (339 of 1354)"),
    "twostream": ("two-stream schedule, 36 layers with fresh inputs, 32/8 heads, head_dim 128, "
                  "128x128 blocks; per layer the understanding stream (1,000 tokens padded to "
                  "1,024) attends to itself causally, then the generation stream (20,000 tokens "
                  "padded to 20,096) attends to cat(understanding, generation): dense in layers "
                  "0-7, 75% target (42 of 165 blocks) in layers 8-35"),
    "edge48k_256x128": ("edge-video-shaped sparse attention with 256x128 blocks: 32/8 heads, "
                        "head_dim 128, 512 prefix + 48,360 generation tokens (31x30x52) padded to "
                        "48,384, 75% target (96 of 382 KV blocks per 256-row block)"),
    "mha64_48k": ("edge-video-shaped sparse attention, MHA at head_dim 64: 32 query / 32 KV heads, "
                  "512 prefix + 48,360 generation tokens, 64x64 blocks, 75% target (191 of 764)"),
    "mqa48k": ("edge-video-shaped sparse attention, MQA: 32 query heads / 1 KV head, head_dim 128, "
               "512 prefix + 48,360 generation tokens, 64x64 blocks, 75% target (191 of 764)"),
    "edge48k_cp8": ("one GPU's share of the edge-video-shaped sparse attention split over 8 GPUs "
                    "by heads: 4 query heads / 1 KV head, head_dim 128, 512 prefix + 48,360 "
                    "generation tokens (31x30x52), 64x64 blocks, 75% target (191 of 764)"),
    "undcausal": ("understanding-stream causal self-attention: 1,000 tokens padded to 1,024, "
                  "32/8 heads, head_dim 128, 128x128 blocks, bottom-right causal mask"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="edge48k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--input-sets", type=int, default=3,
                    help="distinct input sets rotated over the steps (twostream: always its 36 layers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power-seconds", type=float, default=4.0,
                    help="after the timed region, run the step back to back for about this long "
                         "and report average socket power and shader clocks from the driver's "
                         "energy counter (0: skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="also run one plain device copy of BYTES bytes (a known-size kernel "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


def kernel_source_hash(path=ATTN_KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_fields(path):
    vals = {}
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#") and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
    return vals


def selector_kernels(name, lay, keep):
    """The two selector kernels, each against its own roof, from the
    committed rocprofv3 statistics of this workload (average duration of the
    profiled run's launches) when they were taken on the current selector
    source: pooling against HBM bandwidth (algorithmic bytes: the real rows
    of Q and K read once, the pooled vectors and norms written once; the
    counters' bytes beside them), scoring and top-k against the fp64 matrix
    peak (2 D FLOP per (query block, candidate block) pair)."""
    stats = _profile_fields(os.path.join(PROFILES, f"attn_fwd_{name}_kernel_stats.txt"))
    if stats.get("select_source_sha256_16") != kernel_source_hash(SELECT_KERNEL_SRC):
        return None
    try:
        pool_ms = float(stats["pool_kernel_avg_ms"])
        score_ms = float(stats["score_topk_kernel_avg_ms"])
    except (KeyError, ValueError):
        return None
    b, hq, hkv, d = lay["batch"], lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"]
    nq, nk = lay["q_len"] // lay["block_q"], lay["kv_len"] // lay["block_k"]
    real_keys = lay["kv_prefix_valid"] + lay["kv_suffix_valid"]
    read = 2 * d * b * (lay["q_valid"] * hq + real_keys * hkv)
    written = b * hq * nq * (8 * d + 8) + b * hkv * nk * (4 * d + 8)
    pool_bytes = read + written
    real_qblocks = -(-lay["q_valid"] // lay["block_q"])
    n_cand = -(-lay["kv_suffix_valid"] // lay["block_k"])
    score_flops = 2.0 * d * b * hq * real_qblocks * n_cand
    traffic = _profile_fields(os.path.join(PROFILES, f"attn_fwd_{name}_traffic.txt"))
    counted = None
    if traffic.get("select_source_sha256_16") == kernel_source_hash(SELECT_KERNEL_SRC):
        try:
            counted = float(traffic["pool_hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            counted = None
    return {
        "source": "rocprofv3 kernel statistics in profiles/ (same selector source)",
        "pool_kernel": {"bound": "hbm", "ms": pool_ms, "algorithmic_bytes": pool_bytes,
                        "achieved": round(pool_bytes / (pool_ms * 1e-3) / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(pool_bytes / (pool_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": counted},
        "score_topk_kernel": {"bound": "fp64 matrix", "ms": score_ms, "flops": score_flops,
                              "achieved": round(score_flops / (score_ms * 1e-3) / 1e12, 3),
                              "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(score_flops / (score_ms * 1e-3) / 1e12 / FP64_PEAK_TFLOPS, 4)},
    }


def recorded_traffic(name):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(PROFILES, f"attn_fwd_{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
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


def recorded_mfma_busy(name):
    """Share of the attention dispatch's cycles in which the matrix cores were
    busy (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs),
    from the committed counter summary, if it covers this workload and was
    taken on the current kernel source; else None. Unlike the fraction of
    the published peak it does not depend on the shader clock."""
    path = os.path.join(PROFILES, "attn_fwd_mfma_busy_edge48k_dense8k.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#") and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals[f"{name}_mfma_busy_frac"])
    except (KeyError, ValueError):
        return None


class SclkSampler:
    """Samples the GPU's current shader clock (the starred level of the
    driver's sysfs table) from a thread while the timed steps run; reports
    the highest value seen, or None where the table is not readable or the
    timed region was too short for `min_samples` readings (a short region
    mostly sees the idle clock, from before the load ramps it up)."""

    def __init__(self, period_s=0.02, min_samples=8):
        self.min_samples = min_samples
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.seen = []
        self.done = threading.Event()
        self.thread = threading.Thread(target=self._run, args=(period_s,), daemon=True)
        if self.path:
            self.thread.start()

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self, period_s):
        while not self.done.is_set():
            v = self._read()
            if v is not None:
                self.seen.append(v)
            self.done.wait(period_s)

    def stop(self):
        if not self.path:
            return None
        self.done.set()
        self.thread.join(timeout=1.0)
        return max(self.seen) if len(self.seen) >= self.min_samples else None


def power_from_readings(readings, cap_w=None):
    """Average socket power over the driver's energy-counter windows.

    `readings` are (timestamp_ns, energy_count, resolution_uJ, gfxclks_mhz)
    tuples, one per counter update (the counter advances about once a
    second), all taken while the step ran back to back. The average is the
    energy between the first and the last update over the time between
    them; the clocks are the per-XCD means over the updates after the first
    (each update reports the clocks of the window it closes). None with
    fewer than two updates."""
    if len(readings) < 2:
        return None
    t0, e0, res, _ = readings[0]
    t1, e1, _, _ = readings[-1]
    if t1 <= t0:
        return None
    avg_w = (e1 - e0) * res * 1e-6 / ((t1 - t0) * 1e-9)
    clks = [r[3] for r in readings[1:] if r[3]]
    per_xcd = None
    if clks and all(len(c) == len(clks[0]) for c in clks):
        per_xcd = [round(float(np.mean([c[x] for c in clks])), 1) for x in range(len(clks[0]))]
    windows = []
    for (ta, ea, ra, _), (tb, eb, _, _) in zip(readings, readings[1:]):
        if tb > ta:
            windows.append((eb - ea) * ra * 1e-6 / ((tb - ta) * 1e-9))
    return {
        "avg_w": round(avg_w, 1),
        "window_w_min": round(min(windows), 1),
        "window_w_max": round(max(windows), 1),
        "windows": len(readings) - 1,
        "seconds": round((t1 - t0) * 1e-9, 3),
        "cap_w": cap_w,
        "gfxclk_mhz_per_xcd": per_xcd,
        "gfxclk_mhz_mean": round(float(np.mean(per_xcd)), 1) if per_xcd else None,
    }


def measure_power(run_step, dev, seconds):
    """Runs `run_step(i)` back to back for about `seconds` after the timed
    region (at most two steps queued) and reads the driver's energy counter
    and shader clocks through amdsmi at each counter update. Returns
    power_from_readings() of those updates, or None where amdsmi is missing,
    the device is not found, an amdsmi call fails or fewer than two updates
    fell inside. Errors of the step itself propagate."""
    if seconds <= 0:
        return None
    try:
        import amdsmi
    except ImportError:
        return None
    import torch
    try:
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        prop = torch.cuda.get_device_properties(dev)
        bdf = f"{prop.pci_domain_id:04x}:{prop.pci_bus_id:02x}:{prop.pci_device_id:02x}"
        handle = None
        try:
            for h in amdsmi.amdsmi_get_processor_handles():
                if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(bdf):
                    handle = h
        except Exception:
            return None
        if handle is None:
            return None
        try:
            cap_w = round(amdsmi.amdsmi_get_power_cap_info(handle)["power_cap"] / 1e6, 1)
        except Exception:
            cap_w = None
        ring = [torch.cuda.Event() for _ in range(2)]
        readings, last_ts = [], None
        t_end = time.perf_counter() + seconds
        next_poll = 0.0
        i = 0
        while time.perf_counter() < t_end:
            if i >= len(ring):
                ring[i % len(ring)].synchronize()
            run_step(i)
            ring[i % len(ring)].record()
            i += 1
            now = time.perf_counter()
            if now < next_poll or i < len(ring):
                continue
            next_poll = now + 0.02
            try:
                e = amdsmi.amdsmi_get_energy_count(handle)
            except Exception:
                readings = []
                break
            if e["timestamp"] != last_ts:
                last_ts = e["timestamp"]
                try:
                    clks = [int(c) for c in amdsmi.amdsmi_get_gpu_metrics_info(handle)
                            .get("current_gfxclks", []) if str(c).isdigit() and int(c) < 0xFFFF]
                except Exception:
                    clks = []
                readings.append((e["timestamp"], e["energy_accumulator"],
                                 e["counter_resolution"], clks))
        torch.cuda.synchronize()
        # The first reading is the counter as the loop found it, the second
        # closes a window that began before the loop: average from the second.
        return power_from_readings(readings[1:], cap_w)
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def causal_tiles(lay):
    """(query block, KV block) tiles the causal kernel visits per head: block
    j is visited for query block i when its first real key's rank is within
    reach of block i's last real row (rank <= row + n_k - n_q), and the count
    of (real row, real key) pairs the causal mask keeps."""
    bq, bk = lay["block_q"], lay["block_k"]
    nq = lay["q_len"] // bq
    pv, sv, pl = lay["kv_prefix_valid"], lay["kv_suffix_valid"], lay["kv_prefix_len"]
    off = pv + sv - lay["q_valid"]
    firsts = [j * bk for j in range((pv + bk - 1) // bk)] + \
        [pv + m * bk for m in range((sv + bk - 1) // bk)]
    tiles = 0
    for i in range(nq):
        if i * bq >= lay["q_valid"]:
            continue
        last = min((i + 1) * bq, lay["q_valid"]) - 1 + off
        tiles += sum(1 for f in firsts if f <= last)
    t = np.arange(lay["q_valid"])
    pairs = int(np.clip(t + off + 1, 0, pv + sv).sum())
    return tiles, pairs


def cpu_baseline_causal(case):
    """The fp64 oracle's causal dense attention, untouched, on the whole
    understanding-stream case (every head); effective FLOPs of the visited
    tiles, like the GPU figure."""
    import oracle
    from threadpoolctl import threadpool_info

    lay = case.layout
    t0 = time.perf_counter()
    oracle.dense_causal(lay, case.q, case.k, case.v)
    t = time.perf_counter() - t0
    tiles, _ = causal_tiles(lay)
    flops = 4.0 * lay["block_q"] * lay["block_k"] * lay["head_dim"] * tiles * lay["batch"] * \
        lay["num_q_heads"]
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    return {
        "value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"understanding stream layer {case.meta.get('layer', 0)}, all "
                   f"{lay['num_q_heads']} query heads, fp64 causal attention ({t:.2f} s); "
                   "effective FLOPs of the visited tiles"),
        "seconds": round(t, 2),
        "cpu_model": cpu_model(),
    }


def _cpu_oracle_head(args):
    """One worker of the CPU baseline: the oracle, untouched, for one query
    head (BLAS limited to one thread): its selection over every query block
    (skipped for a dense layer, ``keep`` None) and its attention for the
    first ``n_blocks`` query blocks. Returns the two phases' seconds, the
    effective FLOPs of the attended blocks (4 bq bk D per listed tile) and
    their valid-only FLOPs (4 D per real (row, key) pair)."""
    lay1, q1, k1, v1, keep, n_blocks = args
    from threadpoolctl import threadpool_limits

    import oracle
    bq, bk, d = lay1["block_q"], lay1["block_k"], lay1["head_dim"]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if keep is None:
            idx, cnt = oracle.identity_selection(lay1)
        else:
            idx, cnt = oracle.select(lay1, q1, k1, keep)
        t_sel = time.perf_counter() - t0 if keep is not None else 0.0
        lay_s = dict(lay1, q_len=n_blocks * bq, q_valid=min(lay1["q_valid"], n_blocks * bq))
        idx_s, cnt_s = idx[:, :, :n_blocks], cnt[:, :, :n_blocks]
        t0 = time.perf_counter()
        oracle.attend(lay_s, q1[:, :lay_s["q_len"]], k1, v1, idx_s, cnt_s)
        t_att = time.perf_counter() - t0
    kvalid = oracle.valid_key_mask(lay1).reshape(-1, bk).sum(axis=1)
    qvalid = oracle.valid_query_mask(lay_s).reshape(-1, bq).sum(axis=1)
    flops = valid = 0.0
    for i in range(n_blocks):
        c = int(cnt_s[0, 0, i])
        blocks = idx_s[0, 0, i, :c]
        flops += 4.0 * bq * bk * d * c
        valid += 4.0 * d * float(qvalid[i]) * float(kvalid[blocks].sum())
    return t_sel, t_att, flops, valid


def cpu_baseline(case, keep, target_flop_per_head=3e11):
    """The fp64 oracle, untouched, on a bounded sample of the same workload:
    one worker process per query head (BLAS limited to one thread each), as
    many heads as the host lets this process run on (at most 16); each
    selects over all its query blocks (skipped for a dense layer, ``keep``
    None) and attends for its first query blocks, about 0.3 TFLOP of
    attention per head. Reported as effective TFLOP/s of the attended
    blocks, the selection pro-rated to them, over the slowest worker."""
    import multiprocessing as mp

    lay = case.layout
    hq, hkv = lay["num_q_heads"], lay["num_kv_heads"]
    grp = hq // hkv
    nq = lay["q_len"] // lay["block_q"]
    per_block = 4.0 * lay["block_q"] * lay["block_k"] * lay["head_dim"] * \
        (keep if keep is not None else lay["kv_len"] // lay["block_k"])
    n_blocks = int(max(1, min(nq, target_flop_per_head // per_block)))
    workers = max(1, min(16, len(os.sched_getaffinity(0)), hq))
    lay1 = dict(lay, num_q_heads=1, num_kv_heads=1)
    tasks = [(lay1, np.ascontiguousarray(case.q[:, :, h:h + 1]),
              np.ascontiguousarray(case.k[:, :, h // grp:h // grp + 1]),
              np.ascontiguousarray(case.v[:, :, h // grp:h // grp + 1]), keep, n_blocks)
             for h in range(workers)]
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_cpu_oracle_head, tasks, chunksize=1)
    wall = time.perf_counter() - t0
    per_head = [t_sel * n_blocks / nq + t_att for t_sel, t_att, _, _ in res]
    t = max(per_head)
    flops = sum(r[2] for r in res)
    valid = sum(r[3] for r in res)
    what = "dense (no selection)" if keep is None else \
        f"selection over all {nq} query blocks (pro-rated)"
    return {
        "value": flops / t / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
        "sample": (f"{case.name} layer {case.meta.get('layer', 0)}, query heads 0-{workers - 1} of "
                   f"{hq}, one single-threaded worker process each: {what} + fp64 attention for "
                   f"the first {n_blocks} of {nq} query blocks; effective FLOPs of those blocks "
                   f"over the slowest worker"),
        "valid_only_value": valid / t / 1e12,
        "effective_tflop": round(flops / 1e12, 4),
        "valid_only_tflop": round(valid / 1e12, 4),
        "seconds": round(wall, 2),
        "cpu_model": cpu_model(),
        "select_seconds_per_head": round(float(np.mean([r[0] for r in res])), 2),
        "attend_seconds_per_head": round(float(np.mean([r[1] for r in res])), 2),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only; --gpus above 1 is not supported (one GPU's share "
              "of the head-sharded 48k workload is --workload edge48k_cp8)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_blocks_amd as bsa
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    schedule = name == "twostream"
    und_only = name == "undcausal"
    n_sets = synth.CONFIGS["twostream"]["layers"] if schedule else max(1, args.input_sets)

    def gpu(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    sets, und_sets = [], []
    for layer in range(n_sets):
        if und_only:
            case = synth.make_und_case(layer)
        else:
            case = synth.make_config(name, layer=layer)
        t = [gpu(a) for a in (case.q, case.k, case.v)]
        sets.append((case, t))
        if schedule:
            # The understanding stream's keys and values are the first segment
            # of this layer's K/V (views, no copy); its queries are its own.
            uc = synth.make_und_case(layer)
            ul = uc.layout["kv_len"]
            und_sets.append((uc, [gpu(uc.q), t[1][:, :ul], t[2][:, :ul]]))
        print(f"bench: input set {layer} of {name} ready", file=sys.stderr, flush=True)
    case0 = sets[0][0]
    lay = case0.layout
    nq, nk, p = bsa.num_blocks(lay)
    b, hq = lay["batch"], lay["num_q_heads"]
    sparse_case = next((c for c, _ in sets if c.sparsity > 0), None)
    keep = bsa.keep_blocks(nk, p, sparse_case.sparsity) if sparse_case else nk
    idx = torch.empty((b, hq, nq, keep), dtype=torch.int32, device=dev)
    cnt = torch.empty((b, hq, nq), dtype=torch.int32, device=dev)
    ws = torch.empty(max(bsa.select_workspace_size(lay), 256), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(t[0]) for _, t in sets]
    und_outs = [torch.empty_like(t[0]) for _, t in und_sets]
    stream = torch.cuda.current_stream()

    # One step: a list of layer calls (input set, kind); kind is "sparse"
    # (selection + block-sparse attention), "dense", "causal" (the measured
    # kernel is the causal one) or "und" (the understanding stream's causal
    # attention inside the two-stream schedule, timed on its own).
    if schedule:
        # The library's step/layer strategy decides each generation-stream
        # call: the Cosmos3 mixed recipe (10 dense steps, then layers 8-35
        # sparse) at its first sparse step.
        tc = synth.CONFIGS["twostream"]
        strategy = bsa.make_strategy(tc["layers"], 10, range(tc["dense_layers"], tc["layers"]),
                                     tc["sparsity"])
        kinds = ["sparse" if bsa.strategy_is_sparse(strategy, 10, s) else "dense"
                 for s in range(len(sets))]
        if any((kd == "dense") != (sets[s][0].sparsity == 0) for s, kd in enumerate(kinds)):
            raise RuntimeError("strategy decisions disagree with the schedule's inputs")
        _, (q0, k0, v0) = sets[0]
        bsa.strategy_warmup(q0, k0, v0, lay, strategy, out=outs[0])
        plan = [[c for s in range(len(sets)) for c in ((s, "und"), (s, kinds[s]))]]
    elif und_only:
        plan = [[(s, "causal")] for s in range(len(sets))]
    else:
        plan = [[(s, "dense" if case0.sparsity == 0 else "sparse")] for s in range(len(sets))]

    def layer_call(s, kind, ev=None):
        if kind == "und":
            uc, (q, k, v) = und_sets[s]
            if ev is not None:
                ev[3].record(stream)
            bsa.dense_attention(q, k, v, uc.layout, causal=True, out=und_outs[s], stream=stream)
            if ev is not None:
                ev[4].record(stream)
            return
        _, (q, k, v) = sets[s]
        if ev is not None:
            ev[0].record(stream)
        if kind == "sparse":
            bsa.select_blocks(q, k, lay, keep, keep, block_idx=idx, block_cnt=cnt, workspace=ws,
                              stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if kind == "sparse":
            bsa.block_sparse_attention(q, k, v, idx, cnt, lay, out=outs[s], stream=stream)
        else:
            bsa.dense_attention(q, k, v, lay, causal=kind == "causal", out=outs[s], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    def step(i, evs=None):
        for j, (s, kind) in enumerate(plan[i % len(plan)]):
            layer_call(s, kind, None if evs is None else evs[j])

    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Warm up every layout (each input set) before timing; count the effective
    # work of each step from the counts the selector actually produced.
    tile_flops = 4.0 * lay["block_q"] * lay["block_k"] * lay["head_dim"]
    real_rows = (torch.arange(nq, device=dev) * lay["block_q"] < lay["q_valid"])
    step_flops, und_flops = [], 0.0
    for i in range(len(plan)):
        f = 0.0
        for s, kind in plan[i]:
            layer_call(s, kind)
            if kind == "dense":
                f += tile_flops * b * hq * nq * nk
            elif kind in ("causal", "und"):
                ul = (und_sets[s][0] if kind == "und" else sets[s][0]).layout
                tf = 4.0 * ul["block_q"] * ul["block_k"] * ul["head_dim"]
                fc = tf * causal_tiles(ul)[0] * ul["batch"] * ul["num_q_heads"]
                f += fc
                if kind == "und":
                    und_flops += fc
            else:
                torch.cuda.synchronize()
                if not bool((cnt[:, :, real_rows] == keep).all()):
                    raise RuntimeError("unexpected block counts after selection")
                f += tile_flops * float(cnt.sum().item())
        step_flops.append(f)
    for w in range(args.warmup):
        step(w)
    torch.cuda.synchronize()

    n_calls = len(plan[0])
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_calls)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    clock = SclkSampler()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = clock.stop()
    power = measure_power(step, dev, args.power_seconds)
    kinds = [kind for _, kind in plan[0]]
    main_calls = [j for j, kind in enumerate(kinds) if kind != "und"]
    und_calls = [j for j, kind in enumerate(kinds) if kind == "und"]
    sel_ms = [sum(ev[j][0].elapsed_time(ev[j][1]) for j in main_calls) for ev in events]
    att_ms = [sum(ev[j][1].elapsed_time(ev[j][2]) for j in main_calls) for ev in events]
    und_ms = [sum(ev[j][3].elapsed_time(ev[j][4]) for j in und_calls) for ev in events]
    eff_flops = float(np.mean([step_flops[i % len(plan)] for i in range(args.steps)]))
    ms_per_step = wall * 1e3 / args.steps
    att_avg = float(np.mean(att_ms))
    # the roofline covers the main attention launches; the understanding
    # stream's causal launches of the schedule are reported beside it
    att_tflops = (eff_flops - und_flops) / (att_avg * 1e-3) / 1e12
    value = eff_flops / (ms_per_step * 1e-3) / 1e12
    n_main = len(main_calls)

    mode = "causal" if und_only else ("dense" if all(k == "dense" for k in kinds) else "sparse")
    kname = f"attn_fwd_kernel<{lay['head_dim']},{lay['block_q']},{lay['block_k']},{mode}>"
    if schedule:
        kname += " (8 dense + 28 sparse generation-stream launches per step)"
    traffic = recorded_traffic(name)
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
                   "kept_blocks": keep, "sparsity_pct": sparse_case.sparsity if sparse_case else 0,
                   "input_sets": len(sets), "calls_per_step": n_calls},
        "und_causal_ms_per_step": round(float(np.mean(und_ms)), 4) if und_calls else None,
        "und_causal_tflops": (round(und_flops / (float(np.mean(und_ms)) * 1e-3) / 1e12, 2)
                              if und_calls else None),
        "attn_ms_per_call": round(att_avg / n_main, 4),
        "attn_ms_per_step": round(att_avg, 4),
        "attn_ms_median": round(float(np.median(att_ms)) / n_main, 4),
        "attn_ms_min": round(float(np.min(att_ms)) / n_main, 4),
        "attn_tflops": round(att_tflops, 2),
        "select_ms_per_step": round(float(np.mean(sel_ms)), 4),
        "selector": None,
        "gpu_sclk_mhz_max_seen": sclk,
        # average socket power and shader clocks with the step running back to back
        "power": power,
        # the bf16 MFMA peak at the mean shader clock of that phase
        "attn_frac_of_peak_at_sustained_clock": (
            round(att_tflops / (256 * 4096 * power["gfxclk_mhz_mean"] * 1e6 / 1e12), 4)
            if power and power.get("gfxclk_mhz_mean") else None),
        # the bf16 MFMA peak scales with the shader clock (4096 FLOP per CU per cycle)
        "attn_frac_of_peak_at_seen_clock": (round(att_tflops / (256 * 4096 * sclk * 1e6 / 1e12), 4)
                                            if sclk else None),
        "attn_mfma_busy_frac_counters": recorded_mfma_busy(name),
        "effective_tflop_per_step": round(eff_flops / 1e12, 4),
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(att_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    n_sel = sum(1 for _, kind in plan[0] if kind == "sparse")
    if n_sel:
        sel_call_ms = float(np.mean(sel_ms)) / n_sel
        result["selector"] = {"ms_per_call": round(sel_call_ms, 4),
                              "kernels": selector_kernels(name, lay, keep)}
    if und_only:
        tiles, pairs = causal_tiles(lay)
        result["config"]["causal_tiles_per_head"] = tiles
        result["config"]["causal_pairs_per_head"] = pairs
    if not args.no_cpu_baseline:
        if und_only:
            result["cpu_baseline"] = cpu_baseline_causal(case0)
        else:
            cb_case = sparse_case if sparse_case is not None else case0
            result["cpu_baseline"] = cpu_baseline(cb_case, keep if sparse_case is not None else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
