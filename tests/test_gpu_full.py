"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses (the same C-ABI calls on full [1, heads, N, d] tensors).

The oracle cannot redo a whole layer here, so each case samples: the block
mask of two heads (every row of them) and the attention of query blocks spread
over those heads, chosen to include padded patches and the first and last
blocks. Attention rows are compared where the GPU kept the same blocks as the
oracle (rows of ill-posed cuts are counted by the mask check); a second check
feeds the oracle's own lists of the sampled heads to cabf_bsa_forward (in
deterministic list order; the first check uses the default clock-phased order).
"""
import math

import numpy as np
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from synth import WORKLOADS, fourier_video_qkv
from tests.parity import compare_attention, compare_masks, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def calibrate(qp, kp, g, target, sta, ws):
    nb = g.sizes()["n_blocks"]
    cnt = torch.empty((1, g.heads, nb), dtype=torch.int32, device=DEV)
    idx = torch.empty((1, g.heads, nb, nb), dtype=torch.int32, device=DEV)
    total = g.heads * nb * nb
    lo, hi = 0.0, 1.0
    for _ in range(24):
        mid = 0.5 * (lo + hi)
        cabf.cabf_build_block_mask(g, qp, kp, cabf.default_scale(g), mid, sta, cnt, idx, None, ws)
        sp = 1.0 - cnt.sum(dtype=torch.int64).item() / total
        if sp < target:
            lo = mid
        else:
            hi = mid
    return hi


def sample_blocks(og, n):
    """Query blocks to check: first, last, padded patches and a spread."""
    bt, bty, btx = oracle.block_coords(og)
    padded = np.nonzero((bty == og.Ty - 1) | (btx == og.Tx - 1))[0]
    pick = {0, og.nb - 1, int(padded[0]), int(padded[-1]), int(padded[len(padded) // 2])}
    pick |= set(np.linspace(0, og.nb - 1, n).astype(int).tolist())
    return sorted(pick)


CASES = [
    ("wan1.3b-480p", 0.80, None),
    ("wan14b-720p", 0.80, None),
    ("wan14b-720p", 0.90, (1, 1, 1)),
    ("hunyuan-241f-768p", 0.85, None),
]


@pytest.mark.parametrize("name,target,sta", CASES)
def test_full_size_layer(name, target, sta):
    w = WORKLOADS[name]
    say(f"full-size {name} sparsity {target} sta {sta}")
    g = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    og = oracle.Grid(w.T, w.H, w.W, w.P)
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=1,
                                dtype=w.dtype, device=DEV)
    scale = cabf.default_scale(g)
    ws = cabf.mask_workspace(g, DEV)
    qp, kp, vp = cabf.permute(q, k, v, g)
    thr = calibrate(qp, kp, g, target, sta, ws)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr, sta, scale, workspace=ws)
    op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, scale, return_lse=True)
    o = cabf.unpermute(op, g)
    torch.cuda.synchronize()
    sparsity = 1.0 - cnt.sum(dtype=torch.int64).item() / (w.heads * og.nb ** 2)
    say(f"thr={thr:.6f} sparsity={sparsity:.4f}")
    assert abs(sparsity - target) < 0.01

    heads = [0, w.heads - 1]
    blocks = sample_blocks(og, 6)
    for hd in heads:
        qh, kh, vh = (to_np(t[0, hd]) for t in (qp, kp, vp))
        info = oracle.build_block_mask(qh, kh, og, scale, thr, sta)
        compare_masks(cnt[0, hd], idx[0, hd], info, thr, label=f"{name} head {hd}")
        gmask = oracle.lists_to_mask(cnt[0, hd].cpu().numpy(), idx[0, hd].cpu().numpy(), og.nb)
        same = ~(gmask != info["mask"]).any(-1)
        use = [b for b in blocks if same[b]]
        assert len(use) >= len(blocks) - 2
        sub_cnt = np.zeros_like(info["kv_count"])
        sub_cnt[use] = info["kv_count"][use]
        ref_o, ref_lse = oracle.bsa_forward(qh, kh, vh, sub_cnt, info["kv_index"], og, scale)
        rows = np.concatenate([np.arange(b * 64, (b + 1) * 64) for b in use])
        compare_attention(op[0, hd], ref_o, True, lse[0, hd], ref_lse, rows=rows,
                          label=f"{name} head {hd} blocks {use}")
        # raster output of the same rows equals the reordered output
        pos = oracle.fractal_positions(og)
        inv = np.full(og.N, -1)
        inv[pos] = np.arange(pos.size)
        real_rows = rows[inv[rows] >= 0]
        assert torch.equal(o[0, hd, torch.from_numpy(inv[real_rows]).to(DEV)],
                           op[0, hd, torch.from_numpy(real_rows).to(DEV)])

        # attention fed the oracle's lists for this head (the rest keeps the
        # GPU's), in deterministic list order
        cnt2, idx2 = cnt.clone(), idx.clone()
        cnt2[0, hd] = torch.from_numpy(info["kv_count"]).to(DEV)
        idx2[0, hd] = torch.from_numpy(info["kv_index"]).to(DEV)
        op2 = cabf.bsa_forward(qp, kp, vp, cnt2, idx2, g, scale, deterministic=True)
        torch.cuda.synchronize()
        sub_cnt = np.zeros_like(info["kv_count"])
        sub_cnt[blocks] = info["kv_count"][blocks]
        ref_o2, _ = oracle.bsa_forward(qh, kh, vh, sub_cnt, info["kv_index"], og, scale)
        rows2 = np.concatenate([np.arange(b * 64, (b + 1) * 64) for b in blocks])
        compare_attention(op2[0, hd], ref_o2, True, rows=rows2, label=f"{name} head {hd} oracle lists")


def test_longest_supported_rows():
    """nb close to the 8192-block limit of the mask kernels (register-held rows)."""
    T, H, W, d = 125, 64, 64, 64          # nb = 125 * 8 * 8 = 8000
    g = cabf.Geom(1, 1, d, T, H, W, 8)
    og = oracle.Grid(T, H, W, 8)
    say(f"longest rows nb={og.nb}")
    q, k, v = fourier_video_qkv(T, H, W, 1, d, 1.0, seed=2, dtype="bf16", device=DEV)
    qp, kp, vp = cabf.permute(q, k, v, g)
    thr = 0.6
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr, None, 1.0)
    torch.cuda.synchronize()
    qn, kn = to_np(qp[0, 0]), to_np(kp[0, 0])
    qb = oracle.pool_blocks(qn, og)
    kb = oracle.pool_blocks(kn, og)
    p = oracle.block_probs(oracle.block_logits(qb, kb, 1.0))
    rows = [0, 1, 777, og.nb // 2, og.nb - 2, og.nb - 1]
    info = dict(mask=np.zeros((len(rows), og.nb), dtype=bool), k=np.zeros(len(rows), dtype=np.int64),
                s_prev=np.zeros(len(rows)), s_k=np.zeros(len(rows)), p_k=np.zeros(len(rows)),
                p_next=np.zeros(len(rows)))
    for n, i in enumerate(rows):
        kept, kk, a, b, c, dd = oracle.cdf_cut_details(p[i], thr)
        info["mask"][n, kept] = True
        info["k"][n], info["s_prev"][n], info["s_k"][n], info["p_k"][n], info["p_next"][n] = kk, a, b, c, dd
    sel = torch.tensor(rows, device=DEV)
    compare_masks(cnt[0, 0, sel], idx[0, 0, sel], info, thr, label=f"nb={og.nb}")
    assert not math.isnan(float(cnt.float().mean()))


@pytest.mark.parametrize("ratio,sta", [(0.20, None), (0.10, (1, 1, 1))])
def test_full_size_topk_static_ratio(ratio, sta):
    """Static-ratio selection at the Wan-14B 720p shape: k = ceil(ratio * nb)
    per row, both edge heads' lists against the oracle, and the attention of
    sampled query blocks on those lists."""
    w = WORKLOADS["wan14b-720p"]
    g = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    og = oracle.Grid(w.T, w.H, w.W, w.P)
    k = cabf.topk_for_ratio(g, ratio)
    say(f"full-size top-k {w.name} ratio {ratio} k {k} sta {sta}")
    q, kk, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=3,
                                 dtype=w.dtype, device=DEV)
    scale = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, kk, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, 0.0, sta, scale, topk=k)
    op = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, scale)
    torch.cuda.synchronize()
    if sta is None:
        assert np.all(cnt.cpu().numpy() == k)
    blocks = sample_blocks(og, 4)
    for hd in (0, w.heads - 1):
        qh, kh, vh = (to_np(t[0, hd]) for t in (qp, kp, vp))
        info = oracle.build_block_mask(qh, kh, og, scale, 0.0, sta, topk=k)
        compare_masks(cnt[0, hd], idx[0, hd], info, 0.0, label=f"top-k head {hd}")
        gmask = oracle.lists_to_mask(cnt[0, hd].cpu().numpy(), idx[0, hd].cpu().numpy(), og.nb)
        same = ~(gmask != info["mask"]).any(-1)
        use = [b for b in blocks if same[b]]
        sub = np.zeros_like(info["kv_count"])
        sub[use] = info["kv_count"][use]
        ref_o, _ = oracle.bsa_forward(qh, kh, vh, sub, info["kv_index"], og, scale)
        rows = np.concatenate([np.arange(b * 64, (b + 1) * 64) for b in use])
        compare_attention(op[0, hd], ref_o, True, rows=rows, label=f"top-k head {hd}")
