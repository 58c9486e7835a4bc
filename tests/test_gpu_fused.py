"""GPU checks of the fused entry points, through the C ABI:

* cabf_permute_pool writes the same reordered tensors as cabf_permute, bit for
  bit, and the mask that cabf_build_block_mask_pooled builds from its block
  means matches the oracle's (NABLA summary, Methodology items 1-3) to the
  same bar as the unfused mask (block probabilities within 2e-5 relative,
  lists equal outside the ill-posed rows);
* cabf_bsa_forward_subset (HSA summary, section 2.2: only the active queries
  are computed) writes exactly the rows that cabf_bsa_forward writes for the
  listed query blocks, bit for bit in deterministic mode, within the bf16
  attention tolerance of the oracle otherwise, and leaves every other row
  untouched.
"""
import numpy as np
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from synth import WORKLOADS, fourier_video_qkv
from tests.parity import compare_attention, compare_masks, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (T, H, W, heads, d, dtype, amplitude)
GRIDS = {
    "tiny-f32-d64": (4, 16, 16, 2, 64, "f32", 1.0),
    "ragged-bf16-d128": (3, 21, 35, 3, 128, "bf16", 0.7),
    "ragged-bf16-d64": (5, 9, 17, 2, 64, "bf16", 1.0),
    "one-partial-block-f32": (1, 3, 5, 2, 128, "f32", 1.0),
    "wide-bf16-d128": (3, 24, 88, 2, 128, "bf16", 0.7),
}


def make(name, seed=0, batch=1):
    T, H, W, heads, d, dt, amp = GRIDS[name]
    qs, ks, vs = [], [], []
    for b in range(batch):
        q, k, v = fourier_video_qkv(T, H, W, heads, d, amp, seed=seed + 17 * b, dtype=dt)
        qs.append(q), ks.append(k), vs.append(v)
    q, k, v = (torch.cat(t, 0).to(DEV) for t in (qs, ks, vs))
    return cabf.Geom(batch, heads, d, T, H, W, 8), oracle.Grid(T, H, W, 8), q, k, v


@pytest.mark.parametrize("name", sorted(GRIDS))
@pytest.mark.parametrize("with_v", [True, False])
def test_permute_pool_reorders_like_permute(name, with_v):
    g, og, q, k, v = make(name, batch=2)
    qp, kp, vp = cabf.permute(q, k, v, g)
    fq, fk, fv, _ = cabf.permute_pool(q, k, v if with_v else None, g)
    torch.cuda.synchronize()
    assert torch.equal(to_cmp(qp), to_cmp(fq))
    assert torch.equal(to_cmp(kp), to_cmp(fk))
    if with_v:
        assert torch.equal(to_cmp(vp), to_cmp(fv))
    else:
        assert fv is None
    assert np.array_equal(to_np(fq[1, 0]), oracle.permute(to_np(q[1, 0]), og))


def to_cmp(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


POOLED_CASES = [
    ("tiny-f32-d64", 0.2, (1, 1, 1), None, None),
    ("ragged-bf16-d128", 0.3, None, None, None),
    ("ragged-bf16-d128", 0.75, (1, 1, 1), 1.0, None),
    ("ragged-bf16-d64", 0.9, (1, 0, 0), 1.0, None),
    ("one-partial-block-f32", 0.5, (1, 1, 1), None, None),
    ("wide-bf16-d128", 0.8, None, 1.0, None),
    ("ragged-bf16-d128", 0.0, None, None, 7),          # top-k from the pooled means
    ("ragged-bf16-d64", 0.0, (1, 1, 1), None, 3),
]


@pytest.mark.parametrize("name,thr,sta,scale,topk", POOLED_CASES)
def test_pooled_mask_matches_oracle(name, thr, sta, scale, topk):
    say(f"pooled mask {name} thr={thr} sta={sta} scale={scale} topk={topk}")
    g, og, q, k, v = make(name)
    s = cabf.default_scale(g) if scale is None else scale
    qp, kp, vp, ws = cabf.permute_pool(q, k, v, g)
    cnt, idx, probs = cabf.build_block_mask_pooled(ws, g, thr, sta, s, return_probs=True,
                                                   topk=topk)
    torch.cuda.synchronize()
    info = oracle.build_block_mask(to_np(qp), to_np(kp), og, s, thr, sta, topk=topk)
    rel = np.abs(probs.cpu().numpy().astype(np.float64) - info["p"]) / info["p"]
    say(f"pooled block prob max rel err {rel.max():.3e}")
    assert rel.max() < 2e-5
    compare_masks(cnt, idx, info, thr, label=f"pooled {name}")
    if topk is not None and sta is None:
        assert np.all(cnt.cpu().numpy() == min(topk, og.nb))


def test_pooled_mask_full_size_agrees_with_unfused():
    """Wan-14B 720p: the fused pair and the unfused pair reorder identically and
    their probabilities agree to 2e-5 relative; on every head where their lists
    differ, both are checked against the oracle (every differing row must be a
    correct cut of the fp64 row). The fused path alone is checked against the
    oracle at full size in test_gpu_full."""
    w = WORKLOADS["wan14b-720p"]
    g = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    og = oracle.Grid(w.T, w.H, w.W, w.P)
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=2,
                                dtype=w.dtype, device=DEV)
    thr = 0.7935
    scale = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, k, v, g)
    c1, i1, p1 = cabf.build_block_mask(qp, kp, g, thr, return_probs=True)
    fq, fk, fv, ws = cabf.permute_pool(q, k, v, g)
    c2, i2, p2 = cabf.build_block_mask_pooled(ws, g, thr, return_probs=True)
    torch.cuda.synchronize()
    for a, b in ((qp, fq), (kp, fk), (vp, fv)):
        assert torch.equal(to_cmp(a), to_cmp(b))
    rel = ((p1.double() - p2.double()).abs() / p1.double()).max().item()
    say(f"full-size fused vs unfused prob rel diff {rel:.3e}")
    assert rel < 2e-5
    same = (c1 == c2) & (i1 == i2).logical_or(
        torch.arange(i1.shape[-1], device=DEV) >= c1.unsqueeze(-1)).all(-1)
    differ = int((~same).sum())
    heads = sorted({h for _, h, _ in torch.nonzero(~same).tolist()})
    say(f"full-size fused vs unfused: {differ} of {same.numel()} rows differ, heads {heads}")
    for hd in heads:
        info = oracle.build_block_mask(to_np(qp[0, hd]), to_np(kp[0, hd]), og, scale, thr)
        compare_masks(c1[0, hd], i1[0, hd], info, thr, label=f"unfused head {hd}")
        compare_masks(c2[0, hd], i2[0, hd], info, thr, label=f"fused head {hd}")


SUBSET_CASES = [
    ("ragged-bf16-d128", 0.4, None, 0.3),
    ("ragged-bf16-d128", 0.7, (1, 1, 1), 0.6),
    ("ragged-bf16-d64", 0.5, None, 0.5),
    ("wide-bf16-d128", 0.8, None, 0.25),
]


def subset_ids(total, frac, seed):
    rng = np.random.default_rng(seed)
    ids = np.nonzero(rng.random(total) < frac)[0].astype(np.int32)
    rng.shuffle(ids)
    return ids


@pytest.mark.parametrize("name,thr,sta,frac", SUBSET_CASES)
def test_subset_forward_writes_exactly_the_listed_blocks(name, thr, sta, frac):
    say(f"subset forward {name} thr={thr} sta={sta} frac={frac}")
    g, og, q, k, v = make(name, batch=2)
    s = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr, sta, s)
    full, full_lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True,
                                      deterministic=True)
    nb = og.nb
    total = g.batch * g.heads * nb
    ids = subset_ids(total, frac, seed=3)
    # ids outside the range are skipped; a repeated id rewrites the same rows
    extra = np.array([-1, total, total + 5, ids[0] if ids.size else 0], dtype=np.int32)
    qb = torch.from_numpy(np.concatenate([ids, extra])).to(DEV)
    listed = np.zeros(total, bool)
    listed[ids] = True
    listed[extra[-1]] = True
    op = torch.full_like(qp, 3.0)
    lse = torch.full(qp.shape[:3], -7.0, device=DEV)
    cabf.bsa_forward_subset(qp, kp, vp, cnt, idx, qb, g, op, lse, deterministic=True)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.repeat(listed, 64)).to(DEV).view(g.batch, g.heads, -1)
    assert torch.equal(op[rows].view(torch.int16), full[rows].view(torch.int16))
    assert torch.equal(lse[rows], full_lse[rows])
    assert torch.all(op[~rows] == 3.0) and torch.all(lse[~rows] == -7.0)
    say(f"{int(listed.sum())} of {total} blocks written; others untouched")
    # the clock-phased order: same rows, within the attention tolerance of the oracle
    op2 = torch.full_like(qp, 3.0)
    lse2 = torch.full(qp.shape[:3], -7.0, device=DEV)
    cabf.bsa_forward_subset(qp, kp, vp, cnt, idx, qb, g, op2, lse2)
    torch.cuda.synchronize()
    assert torch.all(op2[~rows] == 3.0) and torch.all(lse2[~rows] == -7.0)
    valid = oracle.valid_slots(og)
    for b in range(g.batch):
        for hd in range(g.heads):
            blocks = np.nonzero(listed[(b * g.heads + hd) * nb:(b * g.heads + hd + 1) * nb])[0]
            if blocks.size == 0:
                continue
            rws = np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in blocks])
            rws = rws[valid[rws]]
            sub_cnt = cnt[b, hd].cpu().numpy().copy()
            ref_op, ref_lse = oracle.bsa_forward(to_np(qp[b, hd]), to_np(kp[b, hd]),
                                                 to_np(vp[b, hd]), sub_cnt,
                                                 idx[b, hd].cpu().numpy(), og, s)
            compare_attention(op2[b, hd], ref_op, True, lse2[b, hd], ref_lse, rows=rws,
                              label=f"subset {name} b{b} h{hd}")


def test_subset_forward_empty_and_all():
    g, og, q, k, v = make("ragged-bf16-d64")
    s = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, 0.5, None, s)
    op = torch.full_like(qp, 1.5)
    cabf.bsa_forward_subset(qp, kp, vp, cnt, idx, torch.empty(0, dtype=torch.int32, device=DEV),
                            g, op, deterministic=True)
    torch.cuda.synchronize()
    assert torch.all(op == 1.5)
    total = g.batch * g.heads * og.nb
    every = torch.arange(total - 1, -1, -1, dtype=torch.int32, device=DEV)   # reversed order
    cabf.bsa_forward_subset(qp, kp, vp, cnt, idx, every, g, op, deterministic=True)
    full = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(op.view(torch.int16), full.view(torch.int16))


def test_subset_forward_full_size():
    """Wan-14B 720p at 80% sparsity, a quarter of the query blocks active:
    the listed blocks equal the full deterministic forward bit for bit."""
    w = WORKLOADS["wan14b-720p"]
    g = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=4,
                                dtype=w.dtype, device=DEV)
    qp, kp, vp = cabf.permute(q, k, v, g)
    s = cabf.default_scale(g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, 0.7935, None, s)
    full = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, deterministic=True)
    nb = g.sizes()["n_blocks"]
    total = g.batch * g.heads * nb
    ids = subset_ids(total, 0.25, seed=5)
    op = torch.zeros_like(qp)
    cabf.bsa_forward_subset(qp, kp, vp, cnt, idx, torch.from_numpy(ids).to(DEV), g, op,
                            deterministic=True)
    torch.cuda.synchronize()
    listed = np.zeros(total, bool)
    listed[ids] = True
    rows = torch.from_numpy(np.repeat(listed, 64)).to(DEV).view(g.batch, g.heads, -1)
    assert torch.equal(op[rows].view(torch.int16), full[rows].view(torch.int16))
    assert torch.all(op[~rows] == 0)
