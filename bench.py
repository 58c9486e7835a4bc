#!/usr/bin/env python3
"""Benchmark of one content-adaptive block-sparse attention layer on one MI355X.

A step is the whole path on one batch of synthetic input already resident in
HBM: fractal permute of Q, K, V -> block mask (pool, block softmax, CDF cut)
-> block-sparse attention over the kept tiles -> unpermute of the output.
The default workload is the Wan-2.1-14B-like 720p layer (40 heads, head_dim
128, 21 x 45x80 latent grid padded to 48x80, bf16) with the threshold
calibrated to 80% block sparsity.

Prints one JSON line. ``value`` is the effective TFLOP/s of the whole step,
counting 4*64*64*head_dim flops per kept (query block, key block) tile.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import platform
import shutil
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse attn effective TFLOP/s + ms/layer, Wan-14B 720p shape, 80% sparse"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan14b-720p")
    ap.add_argument("--sparsity", type=float, default=0.80)
    ap.add_argument("--sta", action="store_true", help="union the +-1 sliding-tile window")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--unfused", action="store_true",
                    help="reorder and pool in separate passes (default: cabf_permute_pool)")
    ap.add_argument("--deterministic", action="store_true",
                    help="walk every block list from its first entry (bit-reproducible attention)")
    ap.add_argument("--variants", type=int, default=1,
                    help="also time the 90%% and window variants (0 to skip)")
    ap.add_argument("--backward", type=int, default=1,
                    help="also time the block-sparse attention backward at the main sparsity (0 to skip)")
    ap.add_argument("--semantic", type=int, default=1,
                    help="also time the semantic-permutation (k-means + top-p) variant (0 to skip)")
    ap.add_argument("--power", type=int, default=1,
                    help="sample package power and clock with amd-smi (0: skip, e.g. under a "
                         "profiler, which does not let a child process start another program)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle CPU-baseline sample (0 to skip)")
    return ap.parse_args()


def calibrate_thr(cabf, qp, kp, geom, target, sta, ws, kv_count, kv_index, iters=30):
    """Bisection on thr so that the final mask's block sparsity meets the target."""
    import torch
    nb = geom.sizes()["n_blocks"]
    total = geom.batch * geom.heads * nb * nb
    scale = cabf.default_scale(geom)

    def sparsity(thr):
        cabf.cabf_build_block_mask(geom, qp, kp, scale, thr, sta, kv_count, kv_index, None, ws)
        return 1.0 - kv_count.sum(dtype=torch.int64).item() / total

    lo, hi = 0.0, 1.0
    best = (1.0, abs(sparsity(1.0) - target))
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        sp = sparsity(mid)
        if abs(sp - target) < best[1]:
            best = (mid, abs(sp - target))
        if sp < target:
            lo = mid
        else:
            hi = mid
    return best[0]


def run_steps(cabf, geom, bufs, thr, sta, n, timed, flags=0, select="cdf", topk=0, fused=False):
    """n steps of the whole path; returns per-stage event times (ms) if timed.
    fused: the reorder also pools the blocks (cabf_permute_pool) and the mask is
    built from those means (cabf_build_block_mask_pooled)."""
    import torch
    q, k, v, qp, kp, vp, op, o, cnt, idx, ws = bufs
    scale = cabf.default_scale(geom)
    stage = {"permute": [], "mask": [], "attention": [], "unpermute": []}
    for _ in range(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if timed else None
        if timed:
            ev[0].record()
        if fused and select != "sta":
            cabf.cabf_permute_pool(geom, q, k, v, qp, kp, vp, ws)
        else:
            cabf.cabf_permute(geom, q, k, v, qp, kp, vp)
        if timed:
            ev[1].record()
        if select == "sta":
            cabf.cabf_build_sta_mask(geom, sta, cnt, idx)
        elif fused:
            cabf.cabf_build_block_mask_pooled(geom, scale, 0.0 if select == "topk" else thr,
                                              topk if select == "topk" else 0, sta, cnt, idx,
                                              None, ws)
        elif select == "cdf":
            cabf.cabf_build_block_mask(geom, qp, kp, scale, thr, sta, cnt, idx, None, ws)
        else:
            cabf.cabf_build_block_mask(geom, qp, kp, scale, 0.0, sta, cnt, idx, None, ws, topk=topk)
        if timed:
            ev[2].record()
        cabf.cabf_bsa_forward(geom, qp, kp, vp, cnt, idx, scale, op, None, flags)
        if timed:
            ev[3].record()
        cabf.cabf_unpermute(geom, op, o)
        if timed:
            ev[4].record()
            stage["_ev"] = stage.get("_ev", []) + [ev]
    if timed:
        torch.cuda.synchronize()
        for ev in stage.pop("_ev"):
            for i, name in enumerate(("permute", "mask", "attention", "unpermute")):
                stage[name].append(ev[i].elapsed_time(ev[i + 1]))
    return stage


def progress(msg: str):
    """One line on stderr per finished stage (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def kernel_source_digest(read=None) -> str:
    """sha256 of the attention kernel's sources with comments and blank lines removed (ties a
    counter profile to a kernel version; comment edits do not change it). read(name) -> text
    reads another version of the sources."""
    import hashlib
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "content_adaptive_block_fractal_amd", "csrc", name)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in ("attention_mfma.hip", "attention_common.hpp", "attention_tiles.hpp", "geometry.hpp"):
        text = re.sub(r"/\*.*?\*/", "", read(f), flags=re.S)
        code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in code if ln.strip()).encode())
    return h.hexdigest()


def profiled_traffic(workload: str):
    """Bytes per attention launch beyond L2 (MALL/HBM) from the committed rocprofv3 counter
    summary, or None when that summary was taken on a different kernel source or workload."""
    path = os.path.join(ROOT, "profiles", f"bsa_fwd_mfma.{workload}.hbm.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    m = re.search(r"[0-9a-f]{64}", fields.get("kernel_code_sha256", ""))
    if m is None or m.group(0) != kernel_source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline(attn_tflops: float, attn_ms: float, traffic, kernel: str):
    """The attention kernel against the bf16 matrix-core roofline (its algorithmic bound: a dense
    64x64xd contraction per kept tile), with the measured bytes it moves beyond L2 per launch
    (rocprofv3 counters, scaled by the bytes the permute kernel of the same profiled run is known
    to move) and the rate they imply, with the roof the kernel comes closest to."""
    r = {
        "bound": "mfma",
        "kernel": kernel,
        "achieved": attn_tflops,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": attn_tflops / PEAK_BF16_TFLOPS,
        "traffic": traffic,
        "traffic_unit": ("bytes per launch beyond L2 (MALL/HBM): FETCH_SIZE and WRITE_SIZE, each "
                         "scaled by the bytes reorder_pool_blocks is known to read and write in the "
                         "same profiled run"),
        "algorithmic_unit": "4*64*64*head_dim flops per kept 64x64 tile",
        "avg_launch_ms": attn_ms,
    }
    if traffic is not None:
        rate = traffic / (attn_ms * 1e-3) / 1e9
        r["traffic_GBps"] = rate
        r["traffic_frac_of_hbm_peak"] = rate / PEAK_HBM_GBS
        # the roof the kernel comes closest to (not necessarily what holds it there)
        r["nearest_roof"] = ("beyond-L2 traffic vs the HBM peak" if rate / PEAK_HBM_GBS > r["frac"]
                             else "matrix cores")
    return r


def measure_subset(cabf, geom, bufs, thr, sta, flags, steps: int, frac: float = 0.25):
    """cabf_bsa_forward_subset over a seeded random quarter of the query blocks
    (the active set), on the lists of the main run: time and tile rate."""
    import numpy as np
    import torch
    q, k, v, qp, kp, vp, op, o, cnt, idx, ws = bufs
    scale = cabf.default_scale(geom)
    cabf.cabf_permute(geom, q, k, v, qp, kp, vp)
    cabf.cabf_build_block_mask(geom, qp, kp, scale, thr, sta, cnt, idx, None, ws)
    total = cnt.numel()
    rng = np.random.default_rng(11)
    ids = np.nonzero(rng.random(total) < frac)[0].astype(np.int32)
    qb = torch.from_numpy(ids).to(qp.device)
    kept = int(cnt.view(-1)[qb.long()].sum(dtype=torch.int64).item())
    flops = 4.0 * 64 * 64 * geom.head_dim * kept
    for _ in range(2):
        cabf.cabf_bsa_forward_subset(geom, qp, kp, vp, cnt, idx, qb, scale, op, None, flags)
    times = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cabf.cabf_bsa_forward_subset(geom, qp, kp, vp, cnt, idx, qb, scale, op, None, flags)
        e1.record()
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = statistics.fmean(a.elapsed_time(b) for a, b in times)
    return dict(active_blocks=int(ids.size), of_blocks=total, kept_tiles=kept, attention_ms=ms,
                attention_tflops=flops / (ms * 1e-3) / 1e12)


def _smi_sample(exe):
    """(socket power W, mean gfx clock MHz over the XCDs) from one amd-smi reading, or None."""
    try:
        r = subprocess.run([exe, "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                           timeout=10)
        gpu = json.loads(r.stdout)["gpu_data"][0]
        watts = float(gpu["power"]["socket_power"]["value"])
        clks = [float(v["clk"]["value"]) for k, v in gpu["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        return watts, (sum(clks) / len(clks) if clks else None)
    except Exception:
        return None


def package_power(run, seconds=2.0):
    """Median socket power (W) and gfx clock (MHz) that amd-smi reports while run() (which
    enqueues GPU work) is repeated for about `seconds`, outside every timed region; None where
    amd-smi is not available. Tells whether a kernel runs at the package power limit, where
    the firmware lowers the clock."""
    import threading

    import torch
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            smp = _smi_sample(exe)
            if smp is not None:
                samples.append(smp)
            stop.wait(0.2)

    run()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        run()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    use = samples[1:] or samples          # the first reading can precede the load
    if not use:
        return None
    watts = statistics.median(w for w, _ in use)
    clks = [c for _, c in use if c is not None]
    return {"socket_w": watts, "gfx_mhz": statistics.median(clks) if clks else None,
            "samples": len(use)}


def measured_peaks(cabf, dev):
    """What this GPU sustains: a dense bf16 matrix-core loop (the measurement aid
    libcabf_probe.so) and a plain 2 GiB device copy, timed with HIP events."""
    import torch

    from content_adaptive_block_fractal_amd import peak_probe
    wgs, iters = 2048, 20000
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    peak_probe.mfma_peak(wgs, 200, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    peak_probe.mfma_peak(wgs, iters, out)
    e1.record()
    torch.cuda.synchronize()
    flops = wgs * 4 * iters * 8 * 2.0 * 32 * 32 * 16
    mfma_tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    n = (2 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del src, dst
    copy_gbs = 2.0 * n * 4 / (min(times) * 1e-3) / 1e9
    return {"mfma_bf16_tflops": mfma_tflops, "hbm_copy_gbs": copy_gbs,
            "mfma_probe": f"{wgs} workgroups x 4 waves x {iters} x 8 v_mfma_f32_32x32x16_bf16",
            "copy_probe": "2 GiB fp32 device-to-device copy (read + write counted), best of 5"}


def hbm_fractions(geom, sizes, stages, kept, elem_bytes, fused):
    """Algorithmic bytes of the memory-bound stages over their measured time, against
    the HBM peak: permute moves Q, K, V raster -> padded (fused: and writes the fp32
    block means); the mask reads Qp, Kp (unfused only), writes and reads the block
    means (unfused) or reads them (fused), and writes the lists; unpermute moves O
    back."""
    row = geom.batch * geom.heads * geom.head_dim * elem_bytes
    raster, padded = sizes["tokens_raster"] * row, sizes["tokens_padded"] * row
    nb = sizes["n_blocks"]
    pooled = 2 * geom.batch * geom.heads * nb * geom.head_dim * 4
    lists = 4 * kept + 4 * geom.batch * geom.heads * nb
    if fused:
        work = {"permute": 3 * (raster + padded) + pooled, "mask": pooled + lists}
    else:
        work = {"permute": 3 * (raster + padded), "mask": 2 * padded + 2 * pooled + lists}
    work["unpermute"] = 2 * raster      # real rows read from the reordered tensor, written back
    out = {}
    for k, b in work.items():
        gbs = b / (stages[k] * 1e-3) / 1e9
        out[k] = {"bytes": b, "gbs": gbs, "frac": gbs / PEAK_HBM_GBS}
    return out


def measure_backward(cabf, geom, bufs, thr, sta, steps: int):
    """cabf_bsa_backward on the main workload's lists (after a forward that
    keeps lse), timed with HIP events, in the default clock-phased order and
    in deterministic order. Effective TFLOP/s counts 2.5x the forward's flops
    (five 64x64xd products per kept tile); the kernels actually run seven
    (S and dP in both the dQ pass and the dK/dV pass)."""
    import torch
    q, k, v, qp, kp, vp, op, o, cnt, idx, ws = bufs
    scale = cabf.default_scale(geom)
    cabf.cabf_permute(geom, q, k, v, qp, kp, vp)
    cabf.cabf_build_block_mask(geom, qp, kp, scale, thr, sta, cnt, idx, None, ws)
    lse = torch.empty(qp.shape[:3], dtype=torch.float32, device=qp.device)
    cabf.cabf_bsa_forward(geom, qp, kp, vp, cnt, idx, scale, op, lse)
    dop = torch.randn(qp.shape, generator=torch.Generator(device=qp.device).manual_seed(1),
                      device=qp.device).to(qp.dtype)
    dq, dk, dv = (torch.empty_like(qp) for _ in range(3))
    bws = cabf._ws(cabf._lib.cabf_bsa_backward_workspace_bytes(cabf.ctypes.byref(geom.c())),
                   qp.device)
    kept = int(cnt.sum(dtype=torch.int64).item())
    fwd_flops = 4.0 * 64 * 64 * geom.head_dim * kept
    out = {"kept_tiles": kept}
    for label, flags in (("", 0), ("deterministic_", cabf.BSA_DETERMINISTIC)):
        for _ in range(2):
            cabf.cabf_bsa_backward(geom, qp, kp, vp, op, lse, dop, cnt, idx, scale, dq, dk, dv, bws,
                                   flags)
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            cabf.cabf_bsa_backward(geom, qp, kp, vp, op, lse, dop, cnt, idx, scale, dq, dk, dv, bws,
                                   flags)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = statistics.fmean(times)
        out.update({label + "ms": ms, label + "ms_median": statistics.median(times),
                    label + "effective_tflops": 2.5 * fwd_flops / (ms * 1e-3) / 1e12})
    out["executed_tflops"] = 3.5 * fwd_flops / (out["ms"] * 1e-3) / 1e12
    return out


def measure_semantic(cabf, steps: int, warmup: int, seed: int):
    """The semantic-permutation layer at the Wan-14B 720p token count: every
    stage timed with HIP events on the current stream. The attention's work is
    4 * head_dim flops per kept (query, key) token pair."""
    import torch
    from synth import SEMANTIC_WORKLOADS, gaussian_mixture_qk, kmeans_init_indices

    w = SEMANTIC_WORKLOADS["svg2-wan14b-720p"]
    dev = torch.device("cuda:0")
    n, h, d = w.n, w.heads, w.head_dim
    q, k = gaussian_mixture_qk(n, h, d, components=w.components, spread=w.spread,
                               amplitude=w.amplitude, seed=seed, dtype="bf16", device=dev)
    v = torch.randn(1, h, n, d, generator=torch.Generator(device=dev).manual_seed(seed + 1),
                    device=dev).to(torch.bfloat16)
    init_q = torch.from_numpy(kmeans_init_indices(n, w.cq, h, seed + 2)[None]).to(dev)
    init_k = torch.from_numpy(kmeans_init_indices(n, w.ck, h, seed + 3)[None]).to(dev)
    seq = cabf.Seq(1, h, d, n)
    rows = n + cabf.SEQ_PAD_ROWS
    scale = 1.0 / math.sqrt(d)
    B = 1
    km = {}
    for name, C in (("q", w.cq), ("k", w.ck)):
        km[name] = dict(centroids=torch.empty(B, h, C, d, dtype=torch.float32, device=dev),
                        counts=torch.empty(B, h, C, dtype=torch.int32, device=dev),
                        labels=torch.empty(B, h, n, dtype=torch.int32, device=dev),
                        perm=torch.empty(B, h, n, dtype=torch.int32, device=dev),
                        offsets=torch.empty(B, h, C + 1, dtype=torch.int32, device=dev),
                        ws=cabf._ws(cabf._lib.cabf_kmeans_workspace_bytes(
                            cabf.ctypes.byref(seq.c()), C), dev))
    qp, kp, vp, op = (torch.empty(B, h, rows, d, dtype=torch.bfloat16, device=dev) for _ in range(4))
    o = torch.empty_like(q)
    cnt = torch.empty(B, h, w.cq, dtype=torch.int32, device=dev)
    idx = torch.empty(B, h, w.cq, w.ck, dtype=torch.int32, device=dev)
    ws_sel = cabf._ws(cabf._lib.cabf_cluster_select_workspace_bytes(
        cabf.ctypes.byref(seq.c()), w.cq, w.ck), dev)
    ws_att = cabf._ws(cabf._lib.cabf_cluster_attention_workspace_bytes(
        cabf.ctypes.byref(seq.c()), w.cq, w.ck), dev)
    names = ("kmeans_q", "kmeans_k", "gather", "select", "attention", "scatter")
    side = torch.cuda.Stream(device=dev)          # default priority

    def run_kmeans(name, x, C, init):
        m = km[name]
        cabf.cabf_kmeans(seq, x, C, init, w.iters, m["centroids"], m["counts"], m["labels"],
                         m["perm"], m["offsets"], m["ws"])

    def step(ev, overlap):
        ev[0].record()
        if overlap:
            # the two clusterings are independent: K's runs on a second stream
            # while Q's runs on this one; stage "kmeans_q" then covers both
            side.wait_event(ev[0])
            with torch.cuda.stream(side):
                run_kmeans("k", k, w.ck, init_k)
                done_k = torch.cuda.Event()
                done_k.record()
            run_kmeans("q", q, w.cq, init_q)
            torch.cuda.current_stream().wait_event(done_k)
            ev[1].record()
            ev[2].record()
        else:
            run_kmeans("q", q, w.cq, init_q)
            ev[1].record()
            run_kmeans("k", k, w.ck, init_k)
            ev[2].record()
        cabf.cabf_gather_rows(seq, q, km["q"]["perm"], qp, rows)
        cabf.cabf_gather_rows(seq, k, km["k"]["perm"], kp, rows)
        cabf.cabf_gather_rows(seq, v, km["k"]["perm"], vp, rows)
        ev[3].record()
        cabf.cabf_cluster_select(seq, w.cq, w.ck, km["q"]["centroids"], km["k"]["centroids"],
                                 km["k"]["counts"], scale, w.top_p, cnt, idx, None, ws_sel)
        ev[4].record()
        cabf.cabf_cluster_attention(seq, w.cq, w.ck, qp, kp, vp, km["q"]["offsets"],
                                    km["k"]["offsets"], cnt, idx, scale, op, None, ws_att)
        ev[5].record()
        cabf.cabf_scatter_rows(seq, op, rows, km["q"]["perm"], o)
        ev[6].record()

    def timed(overlap):
        times = {nm: [] for nm in names}
        for it in range(warmup + steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
            step(ev, overlap)
            torch.cuda.synchronize()
            if it >= warmup:
                for i, nm in enumerate(names):
                    times[nm].append(ev[i].elapsed_time(ev[i + 1]))
        return {nm: statistics.fmean(t) for nm, t in times.items()}

    serial = timed(False)
    mean = timed(True)
    # kept (query, key) token pairs of the selection, from the cluster sizes
    qs = torch.diff(km["q"]["offsets"].long(), dim=-1)            # [1, h, cq]
    ks = torch.diff(km["k"]["offsets"].long(), dim=-1)            # [1, h, ck]
    # entries past kv_count are undefined: replace them by 0 before indexing
    valid = torch.arange(w.ck, device=dev).view(1, 1, 1, -1) < cnt.long().unsqueeze(-1)
    safe = torch.where(valid, idx.long(), torch.zeros_like(idx, dtype=torch.long)).clamp(0, w.ck - 1)
    sizes = torch.gather(ks.unsqueeze(2).expand(-1, -1, w.cq, -1), 3, safe)
    kept_keys = (sizes * valid).sum(-1)                            # [1, h, cq]
    pairs = int((kept_keys * qs).sum().item())
    flops = 4.0 * d * pairs
    total = sum(mean.values())
    return {
        "workload": f"{w.name}: 1x{h} heads, head_dim {d}, n={n} tokens, {w.cq} query / {w.ck} "
                    f"key clusters, {w.iters} Lloyd iterations, top-p {w.top_p}",
        "data": f"Gaussian mixture Q/K ({w.components} components, amplitude {w.amplitude}), "
                f"normal V, seeded",
        "density": pairs / float(h * n * n),
        "stage_ms": mean,
        "kmeans_streams": "Q and K clustered concurrently on two streams (kmeans_q covers both)",
        "ms_per_layer": total,
        "ms_per_layer_serial_kmeans": sum(serial.values()),
        "kmeans_serial_ms": {"q": serial["kmeans_q"], "k": serial["kmeans_k"]},
        "attention_tflops": flops / (mean["attention"] * 1e-3) / 1e12,
        "layer_tflops": flops / (total * 1e-3) / 1e12,
        "steps": steps,
    }


def _oracle_head_sample(job):
    """One worker of the CPU baseline: the oracle on one head (float32 copies of its raster Q, K,
    V): permute and block mask of all rows, then attention of query blocks in order until the
    time budget is spent. Single thread (BLAS pinned to one thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    qh, kh, vh, grid, head_dim, thr, sta, budget_s = job
    g = oracle.Grid(*grid)
    scale = 1.0 / math.sqrt(head_dim)
    qh, kh, vh = (x.astype(np.float64) for x in (qh, kh, vh))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        qp, kp, vp = oracle.permute(qh, g), oracle.permute(kh, g), oracle.permute(vh, g)
        info = oracle.build_block_mask(qp, kp, g, scale, thr, sta)
        t_mask = time.perf_counter() - t0
        cnt_all = info["kv_count"]
        done, t_attn, tiles = 0, 0.0, 0
        while done < g.nb and t_attn + t_mask * done / g.nb < budget_s:
            cnt = np.zeros_like(cnt_all)
            cnt[done] = cnt_all[done]
            t1 = time.perf_counter()
            oracle.bsa_forward(qp, kp, vp, cnt, info["kv_index"], g, scale)
            t_attn += time.perf_counter() - t1
            tiles += int(cnt_all[done])
            done += 1
    return dict(flops=4.0 * 64 * 64 * head_dim * tiles, tiles=tiles, done=done, nb=g.nb,
                t_mask=t_mask, t_attn=t_attn, t_equiv=t_attn + t_mask * done / g.nb)


def _cpu_worker(job_path: str, out_path: str):
    """Entry of one CPU-baseline worker process (``bench.py --cpu-worker JOB OUT``): reads its
    head from an .npz file, runs _oracle_head_sample, writes the result as JSON."""
    import numpy as np
    with np.load(job_path, allow_pickle=False) as z:
        sta = tuple(int(x) for x in z["sta"]) if z["sta"].size else None
        job = (z["q"], z["k"], z["v"], tuple(int(x) for x in z["grid"]), int(z["head_dim"]),
               float(z["thr"]), sta, float(z["budget_s"]))
    with open(out_path, "w") as fh:
        json.dump(_oracle_head_sample(job), fh)


def host_cpu_model() -> str:
    """The CPU model name as lscpu reports it (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(q, k, v, w, thr, sta, budget_s):
    """The CPU oracle on a bounded sample of the same layer, heads sharded over worker processes
    (one per host core, up to 16 and up to the head count): each worker runs head h's permute and
    block mask (all rows) plus attention for the first query blocks that fit the time budget, on
    one thread. value = the sum of the workers' throughputs (each measured while all run).
    Workers are plain child processes (this script with --cpu-worker), each given its head in an
    .npz file and waited for, so none outlives the benchmark."""
    import subprocess
    import tempfile

    import numpy as np
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 16, w.heads))
    f = lambda t, hd: t[0, hd].float().cpu().numpy()
    results = None
    with tempfile.TemporaryDirectory(prefix="cabf_cpu_") as tmp:
        procs = []
        try:
            for hd in range(workers):
                job = os.path.join(tmp, f"job{hd}.npz")
                np.savez(job, q=f(q, hd), k=f(k, hd), v=f(v, hd),
                         grid=np.array([w.T, w.H, w.W, w.P]), head_dim=w.head_dim, thr=thr,
                         sta=np.array(sta if sta else [], dtype=np.int64), budget_s=budget_s)
                out = os.path.join(tmp, f"out{hd}.json")
                env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1",
                           MKL_NUM_THREADS="1")
                procs.append((subprocess.Popen([sys.executable, os.path.abspath(__file__),
                                                "--cpu-worker", job, out], env=env), out))
            results = []
            for p, out in procs:
                if p.wait() != 0:
                    raise RuntimeError(f"worker exited with {p.returncode}")
                with open(out) as fh:
                    results.append(json.load(fh))
        except Exception as exc:       # a host without working worker processes: one core
            for p, _ in procs:
                if p.poll() is None:
                    p.kill()
                    p.wait()
            print(f"cpu baseline: worker processes failed ({exc!r}); using one core",
                  file=sys.stderr)
            results = None
    if results is None:
        workers = 1
        results = [_oracle_head_sample((f(q, 0), f(k, 0), f(v, 0), (w.T, w.H, w.W, w.P),
                                        w.head_dim, thr, sta, budget_s))]
    value = sum(r["flops"] / r["t_equiv"] for r in results) / 1e12
    r0 = results[0]
    per_layer_s = (r0["t_mask"] + r0["t_attn"] / r0["done"] * r0["nb"]) * w.heads * w.batch
    tiles = sum(r["tiles"] for r in results)
    done = sum(r["done"] for r in results)
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"heads 0-{workers - 1} of {w.heads}, one worker process and thread each: "
                   f"permute + block mask of all {r0['nb']} rows of the head ({r0['t_mask']:.2f} s "
                   f"on head 0, charged pro rata) + attention of its first query blocks "
                   f"({done} query blocks, {tiles} kept tiles in all, ~{budget_s:.0f} s per worker); "
                   f"fp64 numpy"),
        "extrapolated_s_per_layer_one_core": per_layer_s,
        "host_cpu": host_cpu_model(),
        "host_cores_available": cores,
    }


def main():
    if len(sys.argv) == 4 and sys.argv[1] == "--cpu-worker":
        _cpu_worker(sys.argv[2], sys.argv[3])
        return
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the block-sparse attention path has no "
              f"multi-GPU mode (asked for --gpus {args.gpus}, WORLD_SIZE {world}). "
              f"Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import content_adaptive_block_fractal_amd as cabf
    from synth import WORKLOADS, fourier_video_qkv

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    geom = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    sizes = geom.sizes()
    nb = sizes["n_blocks"]
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=args.seed,
                                dtype=w.dtype, batch=w.batch, device=dev)
    pshape = (w.batch, w.heads, sizes["tokens_padded"], w.head_dim)
    qp, kp, vp, op = (torch.empty(pshape, dtype=q.dtype, device=dev) for _ in range(4))
    o = torch.empty_like(q)
    cnt = torch.empty((w.batch, w.heads, nb), dtype=torch.int32, device=dev)
    idx = torch.empty((w.batch, w.heads, nb, nb), dtype=torch.int32, device=dev)
    ws = cabf.mask_workspace(geom, dev)
    bufs = (q, k, v, qp, kp, vp, op, o, cnt, idx, ws)

    def measure(sparsity, sta, steps, warmup, flags, select="cdf", topk=0, fused=None):
        fused = (not args.unfused) if fused is None else fused
        cabf.cabf_permute(geom, q, k, v, qp, kp, vp)
        thr = (calibrate_thr(cabf, qp, kp, geom, sparsity, sta, ws, cnt, idx) if select == "cdf"
               else None)
        kw = dict(flags=flags, select=select, topk=topk, fused=fused)
        run_steps(cabf, geom, bufs, thr, sta, warmup, timed=False, **kw)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(cabf, geom, bufs, thr, sta, steps, timed=False, **kw)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        stages = run_steps(cabf, geom, bufs, thr, sta, steps, timed=True, **kw)
        kept = int(cnt.sum(dtype=torch.int64).item())
        flops = 4.0 * 64 * 64 * w.head_dim * kept
        med = {kk: statistics.median(vv) for kk, vv in stages.items()}
        mean = {kk: statistics.fmean(vv) for kk, vv in stages.items()}
        return dict(thr=thr, sta=sta, kept_tiles=kept,
                    sparsity=1.0 - kept / (w.batch * w.heads * nb * nb), flops=flops,
                    wall_ms=wall_ms, stage_ms_median=med, stage_ms_mean=mean,
                    stage_ms_min={kk: min(vv) for kk, vv in stages.items()})

    sta = (1, 1, 1) if args.sta else None
    flags = cabf.BSA_DETERMINISTIC if args.deterministic else 0
    main_run = measure(args.sparsity, sta, args.steps, args.warmup, flags, fused=not args.unfused)
    ms = main_run["wall_ms"]
    progress(f"main step {ms:.2f} ms (thr {main_run['thr']:.6f})")
    # spread of the block logits (scaled, base e): mean over rows of the row std of log p
    _, _, probs = cabf.build_block_mask(qp, kp, geom, main_run["thr"], sta, return_probs=True)
    logit_std = float(torch.log(probs.clamp_min(1e-30)).std(dim=-1).mean().item())
    del probs
    attn_ms = main_run["stage_ms_mean"]["attention"]
    mask_ms = main_run["stage_ms_mean"]["mask"]
    attn_tflops = main_run["flops"] / (attn_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": main_run["flops"] / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded smooth Fourier field + noise Q/K/V, no model weights)",
        "config": {
            "workload": f"{w.name}: 1x{w.heads} heads, head_dim {w.head_dim}, "
                        f"T={w.T} x {w.H}x{w.W} (padded {sizes['Hp']}x{sizes['Wp']}), "
                        f"N={sizes['tokens_padded']}, {nb} blocks of 64",
            "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
            "grid": [w.T, w.H, w.W], "patch": w.P,
            "target_sparsity": args.sparsity, "sparsity": main_run["sparsity"],
            "thr": main_run["thr"], "sta_window": list(sta) if sta else None,
            "block_logit_row_std": logit_std,
            "parallelism": "single GPU",
            "attention_order": ("list order, paired kernel in device-sized launches (rows of "
                                ">= 2048 blocks, either flag)" if nb >= 2048 else
                                "list order in device-sized launches (deterministic)"
                                if args.deterministic else "clock-phased start (default)"),
            "reorder": "separate reorder and block pooling" if args.unfused
                       else "reorder fused with block pooling (cabf_permute_pool, "
                            "cabf_build_block_mask_pooled)",
        },
        # the committed counter profile is of the default order
        "roofline": roofline(attn_tflops, attn_ms,
                             None if args.deterministic else profiled_traffic(w.name),
                             "bsa_fwd_pair (cabf_bsa_forward, rows of >= 2048 blocks; one pass = "
                             "device-sized launches, timed together)" if nb >= 2048 else
                             "bsa_fwd_mfma (cabf_bsa_forward)"),
        "stages_ms": main_run["stage_ms_mean"],
        "stages_ms_median": main_run["stage_ms_median"],
        "stages_ms_min": main_run["stage_ms_min"],
        "ms_per_layer": mask_ms + attn_ms,
        "mask_share": mask_ms / (mask_ms + attn_ms),
        "kept_tiles": main_run["kept_tiles"],
        "hbm_fractions": hbm_fractions(geom, sizes, main_run["stage_ms_mean"], main_run["kept_tiles"],
                                       2 if w.dtype == "bf16" else 4, not args.unfused),
    }
    peaks = measured_peaks(cabf, dev)
    line["measured_peaks"] = peaks
    progress("measured peaks")
    # package power and clock under each load (amd-smi; outside the timed regions): the
    # attention runs at the package power limit, where the firmware lowers the clock
    scale = cabf.default_scale(geom)
    q0, k0, v0, qp0, kp0, vp0, op0, o0, cnt0, idx0, ws0 = bufs
    pw_attn = pw_mfma = None
    if args.power:
        pw_attn = package_power(lambda: cabf.cabf_bsa_forward(geom, qp0, kp0, vp0, cnt0, idx0,
                                                               scale, op0, None, flags))
        from content_adaptive_block_fractal_amd import peak_probe
        probe_out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
        pw_mfma = package_power(lambda: peak_probe.mfma_peak(2048, 2000, probe_out))
    line["package_power"] = {
        "attention": pw_attn, "mfma_probe": pw_mfma, "tool": "amd-smi metric -p -c",
        "note": "median socket power and XCD gfx clock over ~2 s of back-to-back launches"}
    progress(f"package power: attention {pw_attn}, matrix-core loop {pw_mfma}")
    line["roofline"]["frac_of_measured_peak"] = attn_tflops / peaks["mfma_bf16_tflops"]
    if args.variants:
        var = {}
        cases = [(0.90, None, flags), (0.80, (1, 1, 1), flags), (0.90, (1, 1, 1), flags),
                 (args.sparsity, sta, flags ^ cabf.BSA_DETERMINISTIC)]
        for sp, st, fl in cases:
            if sp == args.sparsity and st == sta and fl == flags:
                continue
            r = measure(sp, st, max(3, args.steps // 4), 2, fl)
            a = r["stage_ms_mean"]["attention"]
            name = f"{int(round(sp * 100))}%{'+window' if st else ''}"
            if fl != flags:
                name += " deterministic" if fl else " clock-phased"
            var[name] = dict(
                thr=r["thr"], sparsity=r["sparsity"], ms_per_step=r["wall_ms"],
                attention_ms=a, mask_ms=r["stage_ms_mean"]["mask"],
                attention_tflops=r["flops"] / (a * 1e-3) / 1e12,
                step_tflops=r["flops"] / (r["wall_ms"] * 1e-3) / 1e12)
            progress(f"variant {name}: attention {a:.2f} ms")
        # the other selection rules at the same shape: a static keep ratio of
        # 20% (top-k per row) and the sliding-tile window alone
        k20 = cabf.topk_for_ratio(geom, 0.20)
        for name, sel, st, kk in (("static top-k 20%", "topk", None, k20),
                                  ("STA-only +-1", "sta", (1, 1, 1), 0)):
            r = measure(None, st, max(3, args.steps // 4), 2, flags, select=sel, topk=kk)
            a = r["stage_ms_mean"]["attention"]
            var[name] = dict(k=kk or None, sparsity=r["sparsity"], ms_per_step=r["wall_ms"],
                             attention_ms=a, mask_ms=r["stage_ms_mean"]["mask"],
                             attention_tflops=r["flops"] / (a * 1e-3) / 1e12,
                             step_tflops=r["flops"] / (r["wall_ms"] * 1e-3) / 1e12)
        # the other reorder: separate passes if the main run fused them, or fused
        r = measure(args.sparsity, sta, max(3, args.steps // 4), 2, flags, fused=args.unfused)
        a = r["stage_ms_mean"]["attention"]
        pm = lambda x: x["stage_ms_mean"]["permute"] + x["stage_ms_mean"]["mask"]
        fused_r, unfused_r = (r, main_run) if args.unfused else (main_run, r)
        var["fused permute+pool" if args.unfused else "unfused permute, mask"] = dict(
            thr=r["thr"], sparsity=r["sparsity"], ms_per_step=r["wall_ms"],
            permute_ms=r["stage_ms_mean"]["permute"], mask_ms=r["stage_ms_mean"]["mask"],
            attention_ms=a, step_tflops=r["flops"] / (r["wall_ms"] * 1e-3) / 1e12,
            unfused_permute_plus_mask_ms=pm(unfused_r), fused_permute_plus_mask_ms=pm(fused_r))
        line["variants"] = var
        line["active_query_subset"] = measure_subset(cabf, geom, bufs, main_run["thr"], sta,
                                                     flags, max(3, args.steps // 4))
        progress("selection variants, reorder variant, active-query subset")
    if args.backward:
        line["backward"] = measure_backward(cabf, geom, bufs, main_run["thr"], sta,
                                            max(3, args.steps // 4))
        progress(f"backward {line['backward']['ms']:.2f} ms")
    if args.semantic:
        line["semantic_variant"] = measure_semantic(cabf, max(3, args.steps // 4), 2, args.seed)
        progress(f"semantic-permutation layer {line['semantic_variant']['ms_per_layer']:.2f} ms")
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(q, k, v, w, main_run["thr"], sta, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
