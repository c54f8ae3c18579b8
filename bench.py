"""Benchmark: one step = the whole block-sparse attention path on one GPU.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--keep K]

A step runs, on one stream, every stage of the path over one batch of
synthetic inputs already resident in HBM: tile order (BUILD), gather of Q, K
and V into tile order, the plan (pooling, pooled scores, top-k), the sparse
attention forward, and the scatter of O back to raster order.  The default
workload is the 720p Prism-scale grid: 32 x 48 x 80 tokens (1,920 tiles of
4x4x4), batch 2, 24 heads, head_dim 128, 480 kept tiles per query tile.

Prints one JSON line: effective TFLOP/s over the kept tiles (4*B*H*D * sum of
attended key tokens per query) for the whole step, the forward kernel's
roofline against the bf16 dense MFMA peak, per-stage times from HIP events on
the launch stream, and the CPU oracle timed on a bounded sample.

    python bench.py --backward [...]

times the backward instead (bsa_backward: dQ, dK, dV from the forward's
output and lse and a synthetic dO, inputs resident in HBM) and prints its own
line: 2.5 x the forward's effective FLOPs (the five products of the gradient:
S and dP recomputed, dV, dK, dQ) per second.

    python bench.py --structured 1,2 [...]

times structured lists (bsa_plan_structured / bsa_forward_csr): even heads
spatial (radius 1 tile-frame), odd heads temporal (radius 2 tiles); effective
FLOPs from the lists' lengths.

    python bench.py --varkeep 480,192,120,96 [...]

times the variable-keep path instead (bsa_plan_csr / bsa_forward_csr): head h
keeps the (h mod 4)-th count of the list; effective FLOPs from those counts.
With --backward it times bsa_backward_csr over those lists.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 (256 CUs x 2.4 GHz)
HBM_PEAK_GBS = 8000.0
METRIC = "effective TFLOP/s (kept tiles) + ms/call, 122,880-token grid @25% keep, 1 GPU"
METRIC_BWD = "backward effective TFLOP/s (2.5x forward FLOPs, kept tiles) + ms/call, 1 GPU"
METRIC_VAR = "variable-keep effective TFLOP/s (kept tiles, per-head keep) + ms/call, 1 GPU"
METRIC_STRUCT = "structured-list effective TFLOP/s (spatial/temporal heads, kept tiles) + ms/call, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prism720p")
    ap.add_argument("--keep", type=int, default=None, help="override kept tiles per query tile")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=4096, help="query tiles in the CPU oracle sample")
    ap.add_argument("--backward", action="store_true", help="time the backward pass (bsa_backward)")
    ap.add_argument("--cpu-bwd-tiles", type=int, default=120, help="query and key tiles in the backward CPU sample")
    ap.add_argument("--structured", default=None,
                    help="RT,RS: time structured lists, even heads spatial (radius RT), odd heads temporal (RS)")
    ap.add_argument("--varkeep", default=None,
                    help="comma-separated keep counts cycled over the heads: time the CSR (variable keep) path")
    ap.add_argument("--tiled-io", action="store_true",
                    help="time the path through tiled Q and O (gather, forward, scatter) instead of the raster-I/O "
                         "forward")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (reference for HBM byte counters)")
    return ap.parse_args()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none or
    the forward kernel's source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{re.sub(r'<.*', '', kernel)}_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"sha256 \(first 16 hex\s+digits\): `([0-9a-f]{16})`", txt)
    m_bytes = re.search(r"traffic_bytes_per_launch: (\d+)", txt)
    if not (m_hash and m_bytes):
        return None
    src = os.path.join(ROOT, "block_sparse_attention_39_amd", "csrc", "forward.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != m_hash.group(1):
        return None
    return int(m_bytes.group(1))


def step_stats(times):
    """Median, min and 90th percentile of the per-step times (ms)."""
    t = np.asarray(times, np.float64)
    return {"median": float(np.median(t)), "min": float(t.min()), "p90": float(np.percentile(t, 90))}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_SAMPLE_BH = ((0, 0), (1, 23), (0, 13), (1, 5))


def cpu_baseline(wl, q, k, v, n_tiles: int, gpu_idx=None):
    """The oracle on a few (batch, head) slices: gather, pooling and top-k
    over all of each head's rows, attention on `n_tiles` sampled query tiles
    split over the slices; extrapolated linearly over the query tiles and
    heads.  With `gpu_idx` (the GPU's block_idx, [B, H, nVT, k]) the GPU's
    kept lists of those heads are compared with the oracle's on every row, and
    the rows in the contract's near-tie band (relative k-th / (k+1)-th gap
    below 1e-4) and in the float rounding band are counted."""
    import oracle
    pairs = [(b % wl.batch, h % wl.heads) for b, h in CPU_SAMPLE_BH]
    pairs = list(dict.fromkeys(pairs))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    nqt = wl.n_tiled_tokens // 64
    per = max(1, min(nqt, n_tiles // len(pairs)))
    rng = np.random.default_rng(1234)
    scale = float(np.float32(wl.scale))
    t_plan = t_attn = 0.0
    sel = {"rows": 0, "mismatch_rows": 0, "near_tie_rows": 0, "float_band_rows": 0}
    for b, h in pairs:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qs, ks, vs = sl(q), sl(k), sl(v)
        t0 = time.perf_counter()
        if wl.padded:
            perm = oracle.perm_static_padded(wl.grid, wl.tile)[None]
            qt, kt, vt = (oracle.gather_padded(x, perm, wl.n_prefix) for x in (qs, ks, vs))
            qp, kp = oracle.pool_padded(qt, perm, wl.n_prefix), oracle.pool_padded(kt, perm, wl.n_prefix)
        else:
            if wl.dynamic:
                st = oracle.shape_stats(qs, wl.n_prefix, wl.grid)
                shape, _ = oracle.shape_choose(st, wl.grid, float(np.float32(wl.tau)))
                perm = oracle.perm_dynamic(shape, wl.grid)
            else:
                perm = oracle.perm_static(wl.grid, wl.tile)[None]
            qt, kt, vt = (oracle.gather(x, perm, wl.n_prefix) for x in (qs, ks, vs))
            qp, kp = oracle.pool(qt, wl.n_prefix), oracle.pool(kt, wl.n_prefix)
        idx, s_k, s_k1, mag = oracle.topk(qp, kp, wl.keep_tiles)
        t_plan += time.perf_counter() - t0
        if gpu_idx is not None and wl.n_video_tiles:
            # the dynamic shapes of a slice follow the GPU's choice only where
            # the statistic is clear of a threshold; static grids compare fully
            gi = gpu_idx[b, h]
            sel["rows"] += gi.shape[0]
            sel["mismatch_rows"] += int(np.any(gi != idx[0, 0], axis=-1).sum())
            gap = s_k - s_k1
            den = np.maximum(np.abs(s_k), np.abs(s_k1))
            ok = ~np.isnan(s_k1)
            sel["near_tie_rows"] += int((ok & ((den == 0) | (gap < 1e-4 * den))).sum())
            u = 2.0 ** -24
            gam = wl.head_dim * u / (1 - wl.head_dim * u)
            sel["float_band_rows"] += int((ok & (gap <= 2 * gam * mag)).sum())
        tiles = np.sort(rng.choice(nqt, size=per, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        if wl.padded:
            oracle.attention_padded(qt[0, 0], kt[0, 0], vt[0, 0], wl.n_prefix, idx[0, 0],
                                    oracle.key_real(perm[0], wl.n_prefix), scale, tiles)
        else:
            oracle.attention(qt[0, 0], kt[0, 0], vt[0, 0], wl.n_prefix, idx[0, 0], scale, tiles)
        t_attn += time.perf_counter() - t0
    n_s = len(pairs)
    head_seconds = (t_plan + t_attn * nqt / per) / n_s
    head_flops = wl.effective_flops() / (wl.batch * wl.heads)
    res = {
        "value": head_flops / head_seconds / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "ms_per_call_extrapolated": head_seconds * wl.batch * wl.heads * 1e3,
        "sample": (f"{n_s} (batch, head) slices {pairs} of the same workload: gather + pool + top-k over all "
                   f"{wl.n_video_tiles} query tiles of each ({t_plan:.2f} s) and fp64 attention on {per} sampled "
                   f"query tiles of each, {per * n_s} of the call's {nqt * wl.batch * wl.heads} "
                   f"({100.0 * per * n_s / (nqt * wl.batch * wl.heads):.1f}%) ({t_attn:.2f} s), extrapolated "
                   f"linearly over the query tiles and heads"),
    }
    if gpu_idx is not None:
        sel["sample"] = f"every row of the {n_s} (batch, head) slices of the CPU sample, against the oracle"
        res["selection_check"] = sel
    return res


def varkeep_flops(wl, keep_h):
    """4 * B * D * sum over heads and query tokens of the keys attended, with
    head h keeping keep_h[h] tiles per video query tile."""
    pairs = 0
    for kh in keep_h:
        pairs += wl.n_prefix * wl.n_tiled_tokens + wl.n_video_slots * (wl.n_prefix + kh * 64)
    return 4.0 * wl.batch * wl.head_dim * pairs


def cpu_baseline_varkeep(wl, q, k, v, keep_h, n_tiles: int):
    """The oracle's variable-keep path on one (batch, head) slice per distinct
    count: gather, pooling and the per-row top-k over all of the head's rows,
    CSR attention on `n_tiles` sampled query tiles, extrapolated linearly over
    the query tiles and scaled by the heads of each count."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    perm = oracle.perm_static(wl.grid, wl.tile)[None]
    nqt = wl.n_tokens // 64
    rng = np.random.default_rng(2468)
    tiles = np.sort(rng.choice(nqt, size=min(n_tiles, nqt), replace=False)).astype(np.int32)
    scale = float(np.float32(wl.scale))
    total_s, total_f, parts = 0.0, 0.0, []
    for h, kh in enumerate(keep_h[:len(set(keep_h))]):
        sl = lambda x: np.ascontiguousarray(x[0:1, :, h:h + 1])
        t0 = time.perf_counter()
        qt, kt, vt = (oracle.gather(sl(x), perm, wl.n_prefix) for x in (q, k, v))
        qp, kp = oracle.pool(qt, wl.n_prefix), oracle.pool(kt, wl.n_prefix)
        row_ptr, col = oracle.plan_csr(qp, kp, [kh])
        t_plan = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.attention_csr(qt[0, 0], kt[0, 0], vt[0, 0], wl.n_prefix, row_ptr, col, scale, tiles)
        t_attn = time.perf_counter() - t0
        heads = sum(1 for x in keep_h if x == kh) * wl.batch
        total_s += (t_plan + t_attn * nqt / len(tiles)) * heads
        total_f += varkeep_flops(wl, [kh]) / wl.batch * heads
        parts.append(f"k={kh}: plan {t_plan:.2f} s, attention on {len(tiles)} tiles {t_attn:.2f} s")
    return {
        "value": total_f / total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "ms_per_call_extrapolated": total_s * 1e3,
        "sample": ("one (batch, head) slice per distinct keep count of the same workload (" + "; ".join(parts) +
                   f"), fp64, extrapolated linearly over the {nqt} query tiles and over the heads of each count"),
    }


def bench_varkeep(args, wl, q, k, v):
    import torch

    import block_sparse_attention_39_amd as bsa
    counts = [int(x) for x in args.varkeep.split(",")]
    keep_h = [counts[h % len(counts)] for h in range(wl.heads)]
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    desc = bsa.make_desc(wl.batch, wl.heads, wl.head_dim, wl.grid, max(keep_h), scale=wl.scale,
                         n_prefix=wl.n_prefix, dynamic=wl.dynamic, tile=wl.tile, tau=wl.tau, padded=wl.padded)
    raster = not args.tiled_io
    att = bsa.BlockSparseAttention(desc, pool_in_gather=raster)
    out = torch.empty_like(qd)
    rows = wl.batch * wl.heads * wl.n_video_tiles
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device="cuda")
    col = torch.empty(bsa.csr_entries(desc, keep_h), dtype=torch.int32, device="cuda")
    # raster I/O: Q's means alone, K and V gathered (K with its means), the CSR
    # selection from the means, the forward reading raster Q and writing raster
    # O; tiled: the three gathers, bsa_plan_csr (its own pooling), the tiled
    # forward and the scatter
    stages = ["build", "gather", "plan", "forward"] if raster else ["build", "gather", "plan", "forward", "scatter"]

    def step(ev=None):
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        mark(0)
        att.build(qd)
        mark(1)
        if raster:
            att.pool_qk(qd, kd)
            att.gather_v(vd)
            mark(2)
            bsa.select_csr(desc, row_ptr, col, att.workspace, keep_per_head=keep_h)
            mark(3)
            bsa.forward_csr_raster(desc, qd, att.perm, att.k_f, att.v_f, row_ptr, col, out, workspace=att.workspace)
            mark(4)
            return
        att.gather_qkv(qd, kd, vd)
        mark(2)
        bsa.plan_csr(desc, att.q_t, att.k_f, row_ptr, col, att.workspace, keep_per_head=keep_h)
        mark(3)
        bsa.forward_csr(desc, att.q_t, att.k_f, att.v_f, row_ptr, col, att.o_t, workspace=att.workspace)
        mark(4)
        att.scatter_out(out)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_stage = {s: [] for s in stages}
    totals = []
    for ev in events:
        for j, s in enumerate(stages):
            per_stage[s].append(ev[j].elapsed_time(ev[j + 1]))
        totals.append(ev[0].elapsed_time(ev[len(stages)]))
    ms_step = float(np.mean(totals))
    F = varkeep_flops(wl, keep_h)
    fwd_ms = float(np.mean(per_stage["forward"]))
    achieved = F / (fwd_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC_VAR,
        "value": F / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "grid_thw": list(wl.grid), "tokens": wl.n_tokens,
                   "video_tiles": wl.n_video_tiles, "batch": wl.batch, "heads": wl.heads,
                   "head_dim": wl.head_dim, "keep_per_head": keep_h, "effective_tflop_per_call": F / 1e12,
                   "io": "raster Q and O (bsa_forward_csr_raster)" if raster else "tiled Q and O (gather, scatter)"},
        "roofline": {"bound": "mfma",
                     "kernel": f"sparse_fwd_grouped_kernel<{wl.head_dim}, {str(wl.padded).lower()}, "
                               f"{str(raster).lower()}> (CSR lists)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "stages_ms": {s: float(np.mean(per_stage[s])) for s in stages},
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "ms_per_step_stats": step_stats(totals),
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline_varkeep(wl, q, k, v, keep_h, 240)
        print(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def bench_structured(args, wl, q, k, v):
    import torch

    import block_sparse_attention_39_amd as bsa
    rt, rs = (int(x) for x in args.structured.split(","))
    mask = [h % 2 for h in range(wl.heads)]
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    desc = bsa.make_desc(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.keep_tiles, scale=wl.scale,
                         n_prefix=wl.n_prefix, tile=wl.tile, padded=wl.padded)
    raster = not args.tiled_io
    att = bsa.BlockSparseAttention(desc, pool_in_gather=False)   # structured lists need no tile means
    out = torch.empty_like(qd)
    rows = wl.batch * wl.heads * wl.n_video_tiles
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device="cuda")
    entries = bsa.structured_entries(desc, mask, rt, rs)
    col = torch.empty(entries, dtype=torch.int32, device="cuda")
    # raster I/O: only K and V are gathered, the forward reads raster Q and
    # writes raster O; tiled: the three gathers, the tiled forward, the scatter
    stages = ["build", "gather", "plan", "forward"] if raster else ["build", "gather", "plan", "forward", "scatter"]

    def step(ev=None):
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        mark(0)
        att.build(qd)
        mark(1)
        if raster:
            bsa.gather_kf(desc, kd, att.k_f, att.perm)
            att.gather_v(vd)
        else:
            att.gather_qkv(qd, kd, vd)
        mark(2)
        bsa.plan_structured(desc, mask, rt, rs, row_ptr, col)
        mark(3)
        if raster:
            bsa.forward_csr_raster(desc, qd, att.perm, att.k_f, att.v_f, row_ptr, col, out, workspace=att.workspace)
            mark(4)
            return
        bsa.forward_csr(desc, att.q_t, att.k_f, att.v_f, row_ptr, col, att.o_t, workspace=att.workspace)
        mark(4)
        att.scatter_out(out)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_stage = {s: [] for s in stages}
    totals = []
    for ev in events:
        for j, s in enumerate(stages):
            per_stage[s].append(ev[j].elapsed_time(ev[j + 1]))
        totals.append(ev[0].elapsed_time(ev[len(stages)]))
    ms_step = float(np.mean(totals))
    # every video query token attends the prefix and 64 keys per kept tile
    pairs = wl.heads * wl.batch * (wl.n_prefix * wl.n_tiled_tokens + wl.n_video_slots * wl.n_prefix)
    pairs += entries * 64 * 64
    F = 4.0 * wl.head_dim * pairs
    fwd_ms = float(np.mean(per_stage["forward"]))
    achieved = F / (fwd_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC_STRUCT,
        "value": F / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "grid_thw": list(wl.grid), "tokens": wl.n_tokens,
                   "video_tiles": wl.n_video_tiles, "batch": wl.batch, "heads": wl.heads,
                   "head_dim": wl.head_dim, "head_mask": "even spatial, odd temporal", "radius_t": rt,
                   "radius_hw": rs, "kept_entries": entries,
                   "mean_kept_tiles": entries / rows, "effective_tflop_per_call": F / 1e12,
                   "io": "raster Q and O (bsa_forward_csr_raster)" if raster else "tiled Q and O (gather, scatter)"},
        "roofline": {"bound": "mfma",
                     "kernel": f"sparse_fwd_grouped_kernel<{wl.head_dim}, {str(wl.padded).lower()}, "
                               f"{str(raster).lower()}> (CSR lists)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "stages_ms": {s: float(np.mean(per_stage[s])) for s in stages},
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "ms_per_step_stats": step_stats(totals),
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline_structured(wl, q, k, v, rt, rs, args.cpu_tiles)
        print(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def cpu_baseline_structured(wl, q, k, v, rt: int, rs: int, n_tiles: int):
    """The oracle's structured path on one spatial and one temporal (batch,
    head) slice: the lists over the whole tile grid, CSR attention on
    `n_tiles` sampled query tiles, extrapolated linearly over the query tiles
    and over the heads of each kind."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if wl.padded:
        perm = oracle.perm_static_padded(wl.grid, wl.tile)[None]
        gather = lambda x: oracle.gather_padded(x, perm, wl.n_prefix)
    else:
        perm = oracle.perm_static(wl.grid, wl.tile)[None]
        gather = lambda x: oracle.gather(x, perm, wl.n_prefix)
    tgrid = tuple(-(-g // t) for g, t in zip(wl.grid, wl.tile))
    nqt = wl.n_tiled_tokens // 64
    rng = np.random.default_rng(1357)
    tiles = np.sort(rng.choice(nqt, size=min(n_tiles, nqt), replace=False)).astype(np.int32)
    scale = float(np.float32(wl.scale))
    total_s, total_f, parts = 0.0, 0.0, []
    for h, kind in ((0, 0), (1, 1)):
        sl = lambda x: np.ascontiguousarray(x[0:1, :, h:h + 1])
        t0 = time.perf_counter()
        qt, kt, vt = (gather(sl(x)) for x in (q, k, v))
        row_ptr, col = oracle.plan_structured(tgrid, [kind], rt, rs, 1)
        t_plan = time.perf_counter() - t0
        t0 = time.perf_counter()
        if wl.padded:
            oracle.attention_padded_csr(qt[0, 0], kt[0, 0], vt[0, 0], wl.n_prefix, row_ptr, col,
                                        oracle.key_real(perm[0], wl.n_prefix), scale, tiles)
        else:
            oracle.attention_csr(qt[0, 0], kt[0, 0], vt[0, 0], wl.n_prefix, row_ptr, col, scale, tiles)
        t_attn = time.perf_counter() - t0
        heads = sum(1 for x in range(wl.heads) if x % 2 == kind) * wl.batch
        pairs = wl.n_prefix * wl.n_tiled_tokens + wl.n_video_slots * wl.n_prefix + int(row_ptr[-1]) * 64 * 64
        total_s += (t_plan + t_attn * nqt / len(tiles)) * heads
        total_f += 4.0 * wl.head_dim * pairs * heads
        parts.append(f"{('spatial', 'temporal')[kind]}: lists {t_plan:.2f} s, attention on {len(tiles)} tiles "
                     f"{t_attn:.2f} s")
    return {
        "value": total_f / total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "ms_per_call_extrapolated": total_s * 1e3,
        "sample": ("one spatial and one temporal (batch, head) slice of the same workload (" + "; ".join(parts) +
                   f"), fp64, extrapolated linearly over the {nqt} query tiles and over the heads of each kind"),
    }


def cpu_baseline_backward(wl, q, k, v, do, n_tiles: int):
    """The oracle's backward on one (batch, head) slice: lse, Delta and dQ of
    `n_tiles` sampled query tiles, dK and dV of `n_tiles` sampled key tiles
    (given lse and Delta of every query: the work does not depend on their
    values), each extrapolated linearly over the head's tiles."""
    import oracle
    b, h = 0, 0
    sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if wl.padded:
        perm = oracle.perm_static_padded(wl.grid, wl.tile)[None]
        qt, kt, vt, dt = (oracle.gather_padded(sl(x), perm, wl.n_prefix)[0, 0] for x in (q, k, v, do))
        real = oracle.key_real(perm[0], wl.n_prefix)
    else:
        perm = oracle.perm_static(wl.grid, wl.tile)[None]
        qt, kt, vt, dt = (oracle.gather(sl(x), perm, wl.n_prefix)[0, 0] for x in (q, k, v, do))
    t0 = time.perf_counter()
    if wl.padded:
        qp = oracle.pool_padded(qt[None, None], perm, wl.n_prefix)
        kp = oracle.pool_padded(kt[None, None], perm, wl.n_prefix)
    else:
        qp, kp = oracle.pool(qt[None, None], wl.n_prefix), oracle.pool(kt[None, None], wl.n_prefix)
    idx, *_ = oracle.topk(qp, kp, wl.keep_tiles)
    t_plan = time.perf_counter() - t0
    nqt = wl.n_tiled_tokens // 64
    rng = np.random.default_rng(4321)
    tiles = np.sort(rng.choice(nqt, size=min(n_tiles, nqt), replace=False)).astype(np.int32)
    scale = float(np.float32(wl.scale))
    lse = np.zeros(wl.n_tiled_tokens)
    delta = np.zeros(wl.n_tiled_tokens)
    t0 = time.perf_counter()
    if wl.padded:
        oracle.attention_padded(qt, kt, vt, wl.n_prefix, idx[0, 0], real, scale, tiles)
        oracle.backward_dq_padded(qt, kt, vt, dt, lse, delta, wl.n_prefix, idx[0, 0], real, scale, tiles)
    else:
        oracle.attention(qt, kt, vt, wl.n_prefix, idx[0, 0], scale, tiles)
        oracle.backward_dq(qt, kt, vt, dt, lse, delta, wl.n_prefix, idx[0, 0], scale, tiles)
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    if wl.padded:
        oracle.backward_dkdv_padded(qt, kt, vt, dt, lse, delta, wl.n_prefix, idx[0, 0], real, scale, tiles)
    else:
        oracle.backward_dkdv(qt, kt, vt, dt, lse, delta, wl.n_prefix, idx[0, 0], scale, tiles)
    t_k = time.perf_counter() - t0
    head_seconds = t_plan + (t_q + t_k) * nqt / len(tiles)
    head_flops = 2.5 * wl.effective_flops() / (wl.batch * wl.heads)
    return {
        "value": head_flops / head_seconds / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "ms_per_call_extrapolated": head_seconds * wl.batch * wl.heads * 1e3,
        "sample": (f"one (batch, head) slice of the same workload: plan over all rows ({t_plan:.2f} s), lse, "
                   f"Delta and dQ of {len(tiles)} query tiles ({t_q:.2f} s) and dK, dV of {len(tiles)} key tiles "
                   f"({t_k:.2f} s) of {nqt}, fp64, extrapolated linearly to the head and scaled by the head's "
                   f"share of 2.5x the effective FLOPs"),
    }


def bench_backward(args, wl, q, k, v):
    import torch

    import block_sparse_attention_39_amd as bsa
    import synthetic as S
    do = S.tensor(wl, "do")
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    keep_h = None  # --varkeep: CSR lists, head h keeping keep_h[h] tiles
    if args.varkeep:
        counts = [int(x) for x in args.varkeep.split(",")]
        keep_h = [counts[h % len(counts)] for h in range(wl.heads)]
    desc = bsa.make_desc(wl.batch, wl.heads, wl.head_dim, wl.grid, max(keep_h) if keep_h else wl.keep_tiles,
                         scale=wl.scale, n_prefix=wl.n_prefix, dynamic=wl.dynamic, tile=wl.tile, tau=wl.tau,
                         padded=wl.padded)
    att = bsa.BlockSparseAttention(desc, with_lse=True)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    if keep_h is None:
        out = att(qd, kd, vd)
        ws = torch.empty(max(bsa.backward_workspace_size(desc), 256), dtype=torch.uint8, device="cuda")
        call = lambda: bsa.backward(desc, qd, kd, vd, out, dod, att.lse, att.perm, att.block_idx, dq, dk, dv, ws)
    else:
        att.build(qd)
        att.gather_qkv(qd, kd, vd)
        row_ptr = torch.empty(wl.batch * wl.heads * wl.n_video_tiles + 1, dtype=torch.int64, device="cuda")
        col = torch.empty(bsa.csr_entries(desc, keep_h), dtype=torch.int32, device="cuda")
        bsa.plan_csr(desc, att.q_t, att.k_f, row_ptr, col, att.workspace, keep_per_head=keep_h)
        bsa.forward_csr(desc, att.q_t, att.k_f, att.v_f, row_ptr, col, att.o_t, att.lse, workspace=att.workspace)
        out = torch.empty_like(qd)
        att.scatter_out(out)
        ws = torch.empty(max(bsa.backward_csr_workspace_size(desc, col.numel()), 256), dtype=torch.uint8,
                         device="cuda")
        call = lambda: bsa.backward_csr(desc, qd, kd, vd, out, dod, att.lse, att.perm, row_ptr, col, dq, dk, dv,
                                        ws)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = float(np.mean(times))
    # of the last timed call
    dq_gave_up, dq_rounds, kv_gave_up, kv_rounds = bsa.backward_stats(desc, ws, col.numel() if keep_h else 0)
    F = 2.5 * (varkeep_flops(wl, keep_h) if keep_h else wl.effective_flops())
    achieved = F / (ms * 1e-3) / 1e12
    res = {
        "metric": METRIC_BWD,
        "value": achieved,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "grid_thw": list(wl.grid), "tokens": wl.n_tokens,
                   "video_tiles": wl.n_video_tiles, "prefix_tokens": wl.n_prefix, "batch": wl.batch,
                   "heads": wl.heads, "head_dim": wl.head_dim, "keep_tiles": wl.keep_tiles,
                   "tile": "dynamic" if wl.dynamic else "x".join(map(str, wl.tile)),
                   "keep_per_head": keep_h, "padded_video_tokens": wl.n_video_slots if wl.padded else None,
                   "backward_effective_tflop_per_call": F / 1e12},
        "roofline": {"bound": "mfma", "kernel": "bsa_backward%s (all kernels of the call)" % ("_csr" if keep_h else ""),
                     "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None},
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "ms_per_step_stats": step_stats(times),
        "lockstep": {"dq": {"block_rounds": dq_rounds, "waits_gave_up": dq_gave_up},
                     "dkdv": {"block_rounds": kv_rounds, "waits_gave_up": kv_gave_up},
                     "note": "block rounds of the grouped dQ and dK/dV launches in the last timed call (one per "
                             "query tile, one per key tile), and those whose bounded start wait gave up before "
                             "every block of its XCD group arrived"},
    }
    if not args.no_cpu_baseline and keep_h is None:
        t0 = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline_backward(wl, q, k, v, do, args.cpu_bwd_tiles)
        print(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_39_amd as bsa
    import synthetic as S

    wl = S.WORKLOADS[args.workload]
    if args.keep:
        wl = wl.with_keep(args.keep)
    t0 = time.perf_counter()
    q, k, v = S.qkv(wl)
    gen_s = time.perf_counter() - t0
    print(f"[bench] {wl.name}: inputs generated in {gen_s:.1f} s", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    if args.backward:
        if wl.dynamic:
            print("bench.py --backward times static-tile workloads", file=sys.stderr)
            sys.exit(2)
        bench_backward(args, wl, q, k, v)
        return
    if args.structured:
        if wl.dynamic:
            print("bench.py --structured times static-tile workloads", file=sys.stderr)
            sys.exit(2)
        bench_structured(args, wl, q, k, v)
        return
    if args.varkeep:
        if wl.dynamic:
            print("bench.py --varkeep times static-tile workloads", file=sys.stderr)
            sys.exit(2)
        bench_varkeep(args, wl, q, k, v)
        return
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        c = torch.empty_like(a)
        torch.cuda.synchronize()
        c.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done", file=sys.stderr, flush=True)
        del a, c
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    desc = bsa.make_desc(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.keep_tiles, scale=wl.scale,
                         n_prefix=wl.n_prefix, dynamic=wl.dynamic, tile=wl.tile, tau=wl.tau, padded=wl.padded)
    raster = not args.tiled_io
    att = bsa.BlockSparseAttention(desc, raster_io=raster)
    out = torch.empty_like(qd)
    torch.cuda.synchronize()

    if raster:
        # Q's means alone, K gathered with its means; the forward reads raster
        # Q and writes raster O itself
        stages = ["build", "pool_q+gather_k", "gather_v+plan", "forward"]
    else:
        stages = ["build", "gather_qk", "gather_v+plan", "forward", "scatter"]

    def step(ev=None):
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        mark(0)
        att.build(qd)
        mark(1)
        if raster:
            att.pool_qk(qd, kd)
        else:
            att.gather_qk(qd, kd)
        mark(2)
        att.gather_v_and_plan(vd)  # the V gather on a side stream, beside the plan
        mark(3)
        if raster:
            att.forward_raster(qd, out)
            mark(4)
            return
        att.forward()
        mark(4)
        att.scatter_out(out)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_ev = len(stages) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_stage = {s: [] for s in stages}
    totals = []
    for ev in events:
        for j, s in enumerate(stages):
            per_stage[s].append(ev[j].elapsed_time(ev[j + 1]))
        totals.append(ev[0].elapsed_time(ev[len(stages)]))
    ms_step = float(np.mean(totals))
    F = wl.effective_flops()
    fwd_ms = float(np.mean(per_stage["forward"]))
    gave_up, rounds = bsa.forward_stats(desc, att.workspace)   # of the last timed step's forward
    kernels = kernel_breakdown(bsa, att, desc, wl, qd, kd, vd, out, raster)
    # the forward stage is the attention kernel (plus a 4 us counter clear; a
    # dense prefix adds the plain kernel for the prefix query tiles)
    kernel = f"sparse_fwd_grouped_kernel<{wl.head_dim}, {str(wl.padded).lower()}, {str(raster).lower()}>"
    achieved = F / (fwd_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": F / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "grid_thw": list(wl.grid), "tokens": wl.n_tokens,
                   "video_tiles": wl.n_video_tiles, "prefix_tokens": wl.n_prefix, "batch": wl.batch,
                   "heads": wl.heads, "head_dim": wl.head_dim, "keep_tiles": wl.keep_tiles,
                   "tile": "dynamic" if wl.dynamic else "x".join(map(str, wl.tile)),
                   "padded_video_tokens": wl.n_video_slots if wl.padded else None,
                   "io": "raster Q and O (bsa_forward_raster)" if raster else "tiled Q and O (gather, scatter)",
                   "effective_tflop_per_call": F / 1e12},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(kernel, wl.name)},
        "stages_ms": {s: float(np.mean(per_stage[s])) for s in stages},
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "ms_per_step_stats": step_stats(totals),
        "non_forward_ms": ms_step - fwd_ms,
        "skipped_tile_ratio": 1.0 - wl.keep_tiles / wl.n_video_tiles,
        "lockstep": {"block_rounds": rounds, "waits_gave_up": gave_up,
                     "note": "block rounds of the grouped forward launch in the last timed step (one per video "
                             "query tile), and those whose bounded start wait gave up before every block of its "
                             "XCD group arrived"},
        "kernels": kernels,
    }
    if wl.dynamic:
        hist = np.bincount(att.shape_map.cpu().numpy().reshape(-1), minlength=9)
        res["shape_histogram"] = {"order": SHAPE_NAMES, "regions": hist.tolist()}
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        gidx = None if wl.dynamic else att.block_idx.cpu().numpy()
        res["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_tiles, gidx)
        print(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


SHAPE_NAMES = ["4x4x4", "2x4x8", "2x8x4", "8x4x2", "4x2x8", "4x8x2", "8x2x4", "2x2x16", "16x2x2"]


def kernel_breakdown(bsa, att, desc, wl, qd, kd, vd, out, raster: bool, reps: int = 5):
    """Each stage of the step alone on the stream (HIP events, mean of `reps`
    calls after one untimed call), with its HBM bytes and rate against 8 TB/s:
    Q's means alone (the raster-I/O path), the pooling gathers of Q and K, the
    plain gathers they replace, the V gather, the selection, bsa_plan's own
    pooling + selection (the unfused path), the output scatter, and the
    attention kernel with tiled and with raster Q and O.  plan_ms:
    what the plan adds to the step, against the plan's roofline (reading Q and
    K once and writing the lists): on the raster-I/O path Q's means plus the
    K gather's time above the plain one plus the selection; on the tiled path
    the pooling gathers' time above the plain gathers plus the selection."""
    import torch
    cur = torch.cuda.current_stream()
    bf = 2 * wl.batch * wl.heads * wl.n_tiled_tokens * wl.head_dim   # one bf16 tiled tensor, bytes
    pooled = wl.batch * wl.heads * wl.n_video_tiles * wl.head_dim * 4
    idx_bytes = wl.batch * wl.heads * wl.n_video_tiles * wl.keep_tiles * 4
    q_t2, k_f2 = torch.empty_like(att.q_t), torch.empty_like(att.k_f)

    def t(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(cur)
        for _ in range(reps):
            fn()
        ev[1].record(cur)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    ms = {
        "pool_q": t(lambda: bsa.pool(desc, qd, att.perm, att.workspace)),
        "gather_pool_q": t(lambda: bsa.gather_pool(desc, qd, att.q_t, att.perm, att.workspace)),
        "gather_kf_pool_k": t(lambda: bsa.gather_kf_pool(desc, kd, att.k_f, att.perm, att.workspace)),
        "gather_q_plain": t(lambda: bsa.gather(desc, qd, q_t2, att.perm)),
        "gather_kf_k_plain": t(lambda: bsa.gather_kf(desc, kd, k_f2, att.perm)),
        "gather_vf_v": t(lambda: att.gather_v(vd)),
        "select": t(lambda: bsa.select(desc, att.block_idx, att.workspace)),
        "plan_unfused": t(lambda: bsa.plan(desc, att.q_t, att.k_f, att.block_idx, att.workspace)),
        "scatter_o": t(lambda: att.scatter_out(out)),
        # the attention kernel in both forms, same process (after the gathers above
        # filled the tiled Q)
        "forward_tiled_io": t(lambda: bsa.forward(desc, att.q_t, att.k_f, att.v_f, att.block_idx, att.o_t,
                                                  workspace=att.workspace)),
        "forward_raster_io": t(lambda: bsa.forward_raster(desc, qd, att.perm, att.k_f, att.v_f, att.block_idx, out,
                                                          workspace=att.workspace)),
    }
    moved = {"pool_q": bf + pooled, "gather_pool_q": 2 * bf + pooled, "gather_kf_pool_k": 2 * bf + pooled, "gather_q_plain": 2 * bf,
             "gather_kf_k_plain": 2 * bf, "gather_vf_v": 2 * bf, "scatter_o": 2 * bf}
    res = {"note": "each stage alone on the stream, mean of %d calls; hbm = algorithmic bytes moved / time" % reps}
    for k_, v_ in ms.items():
        e = {"ms": v_}
        if k_ in moved:
            gbs = moved[k_] / (v_ * 1e-3) / 1e9
            e.update({"bytes": moved[k_], "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS})
        res[k_] = e
    k_extra = max(0.0, ms["gather_kf_pool_k"] - ms["gather_kf_k_plain"])
    q_extra = max(0.0, ms["gather_pool_q"] - ms["gather_q_plain"])
    pool_ms = ms["pool_q"] + k_extra if raster else q_extra + k_extra
    plan_ms = pool_ms + ms["select"]
    tiled_plan_ms = q_extra + k_extra + ms["select"]
    roof_ms = (2 * bf + idx_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3
    res["plan"] = {"pooling_ms": pool_ms, "select_ms": ms["select"], "plan_ms": plan_ms,
                   "pooling": "Q's means alone plus the K gather's extra" if raster else
                              "the pooling gathers' extra over the plain gathers",
                   "roofline_ms": roof_ms, "frac": roof_ms / plan_ms if plan_ms > 0 else None,
                   "roofline": "read Q and K once (pooling) and write the kept lists, at 8 TB/s",
                   "tiled_path_plan_ms": tiled_plan_ms,
                   "unfused_plan_ms": ms["plan_unfused"],
                   "unfused_frac": roof_ms / ms["plan_unfused"]}
    return res


if __name__ == "__main__":
    main()
