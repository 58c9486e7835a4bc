"""Visit orders of the bf16 forward where they differ in structure.

Rows of fewer than 2048 blocks: by default one workgroup per query block over
the whole grid, clock-phased; in list order the same kernel in launches of a
device-full of workgroups each. Rows of 2048 blocks or more, in both modes:
the paired kernel (the same patch in frames 2t and 2t+1 over the union of
their lists; with an odd frame count the last frame's patches pair with their
right neighbours, and an odd patch count leaves its last block single) in
such launches. Each case checks the attention of sampled query blocks (first
and last blocks, partial patches, the last frame) against the oracle over the
GPU's own lists, on token-independent inputs at scale 3.5/sqrt(d) that a
wrong kernel cannot pass; and the list-order result bit for bit against the
one-block kernel walking the same lists in a single launch (the subset entry
point over every query block) and against a second run.
"""
import math

import numpy as np
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from synth import gaussian_video_qkv
from tests.parity import (assert_inputs_discriminate, attention_on_gpu_lists, compare_attention,
                          sample_blocks, sample_rows, say, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHARP_SCALE = 3.5        # kernel scale, times 1/sqrt(d)

CASES = [
    # name, T, H, W, heads, d, thr
    # 21 frames of 5 x 7 patches: nb 735, 1470 one-block workgroups, more than
    # the device holds at once
    ("one-block-d64", 21, 40, 56, 2, 64, 0.6),
    # 33 frames (odd) of 7 x 9 patches (odd, partial last row and column):
    # nb 2079, the paired kernel
    ("paired-d128", 33, 52, 68, 2, 128, 0.6),
    ("paired-d64", 33, 52, 68, 1, 64, 0.6),
]


@pytest.mark.parametrize("name,T,H,W,heads,d,thr", CASES)
def test_visit_orders(name, T, H, W, heads, d, thr):
    g = cabf.Geom(1, heads, d, T, H, W, 8)
    og = oracle.Grid(T, H, W, 8)
    say(f"visit orders {name}: nb={og.nb} heads={heads} d={d} thr={thr}")
    s = SHARP_SCALE / math.sqrt(d)
    q, k, v = gaussian_video_qkv(T, H, W, heads, d, seed=7, device=DEV)
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr, None, s)
    o_def, l_def = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True)
    o_det, l_det = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    o_rep, l_rep = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    every = torch.arange(heads * og.nb, dtype=torch.int32, device=DEV)
    o_one = torch.zeros_like(qp)
    l_one = torch.zeros(qp.shape[:3], dtype=torch.float32, device=DEV)
    cabf.bsa_forward_subset(qp, kp, vp, cnt, idx, every, g, o_one, l_one, scale=s, deterministic=True)
    torch.cuda.synchronize()
    say(f"mean list length {cnt.float().mean().item():.1f}")
    assert torch.equal(o_det.view(torch.int16), o_rep.view(torch.int16))
    assert torch.equal(l_det, l_rep)
    assert torch.equal(o_det.view(torch.int16), o_one.view(torch.int16))
    assert torch.equal(l_det, l_one)
    # blocks of the last frame (paired with their right neighbours when the
    # frame count is odd, the last one single when the patch count is odd)
    blocks = sorted(set(sample_blocks(og, 4)) | {og.nb - 2, og.nb - 1 - og.Tx * og.Ty // 2})
    for hd in range(heads):
        qh, kh, vh = (to_np(t[0, hd]) for t in (qp, kp, vp))
        cnt_h, idx_h = cnt[0, hd].cpu().numpy(), idx[0, hd].cpu().numpy()
        ref_o, ref_lse = attention_on_gpu_lists(qh, kh, vh, cnt_h, idx_h, og, s, blocks)
        rows = sample_rows(blocks)
        compare_attention(o_def[0, hd], ref_o, True, l_def[0, hd], ref_lse, rows=rows,
                          label=f"{name} head {hd} default order")
        compare_attention(o_det[0, hd], ref_o, True, l_det[0, hd], ref_lse, rows=rows,
                          label=f"{name} head {hd} list order")
        if hd == 0:
            assert_inputs_discriminate(qh, kh, vh, cnt_h, idx_h, og, s, blocks, ref_o)
        assert np.all(cnt_h >= 1)
