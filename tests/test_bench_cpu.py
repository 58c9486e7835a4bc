"""Host-side checks of bench.py's oracle CPU baseline (no GPU): the worker-process
sharding runs the oracle on several heads at once and reports their summed rate."""
import bench
from synth import WORKLOADS, fourier_video_qkv


def test_cpu_baseline_shards_heads_over_workers():
    w = WORKLOADS["tiny"]
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=0,
                                dtype=w.dtype)
    r = bench.cpu_baseline(q, k, v, w, w.thr, w.sta, budget_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert 1 <= r["cores"] <= min(w.heads, 16)
    assert r["value"] > 0
    assert r["extrapolated_s_per_layer_one_core"] > 0


def test_oracle_head_sample_counts_whole_rows():
    w = WORKLOADS["tiny"]
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=1,
                                dtype=w.dtype)
    f = lambda t: t[0, 0].float().numpy()
    r = bench._oracle_head_sample((f(q), f(k), f(v), (w.T, w.H, w.W, w.P), w.head_dim, w.thr,
                                   w.sta, 10.0))
    assert r["done"] == r["nb"] == 16          # a 10 s budget covers every query block here
    assert r["flops"] == 4.0 * 64 * 64 * w.head_dim * r["tiles"]


def test_cpu_baseline_leaves_no_process_behind():
    """The workers are plain child processes that the baseline waits for: no
    child of this process remains afterwards, and the CPU model is named."""
    import psutil
    w = WORKLOADS["tiny"]
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=2,
                                dtype=w.dtype)
    before = {p.pid for p in psutil.Process().children(recursive=True)}
    r = bench.cpu_baseline(q, k, v, w, w.thr, w.sta, budget_s=0.1)
    after = {p.pid for p in psutil.Process().children(recursive=True)}
    assert after <= before
    assert r["cores"] == min(w.heads, 16, r["host_cores_available"])
    assert r["host_cpu"] and r["host_cpu"] != "x86_64"
