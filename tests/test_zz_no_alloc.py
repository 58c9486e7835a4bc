"""cabf_build_block_mask_noalloc (the mask for callers that cannot allocate:
its workspace is a static device array) through the C ABI, against
cabf_build_block_mask with a caller workspace: the same lists and
probabilities bit for bit, on two calls in a row, the second on a smaller
input (the array keeps the first call's contents)."""
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
from synth import fourier_video_qkv
from tests.parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(T, H, W, heads, d, amp, seed, thr, sta, scale):
    g = cabf.Geom(1, heads, d, T, H, W, 8)
    q, k, v = fourier_video_qkv(T, H, W, heads, d, amp, seed=seed, dtype="bf16", device=DEV)
    qp, kp, _ = cabf.permute(q, k, v, g)
    s = cabf.default_scale(g) if scale is None else scale
    nb = g.sizes()["n_blocks"]
    lead = (1, heads, nb)
    want_c, want_i, want_p = cabf.build_block_mask(qp, kp, g, thr, sta, s, return_probs=True)
    got_c = torch.full(lead, -5, dtype=torch.int32, device=DEV)
    got_i = torch.full(lead + (nb,), -5, dtype=torch.int32, device=DEV)
    got_p = torch.full(lead + (nb,), -5.0, dtype=torch.float32, device=DEV)
    cabf.cabf_build_block_mask_noalloc(g, qp, kp, s, thr, sta, got_c, got_i, got_p)
    torch.cuda.synchronize()
    assert torch.equal(got_c, want_c)
    assert torch.equal(got_p, want_p)
    used = torch.arange(nb, device=DEV) < want_c.unsqueeze(-1)
    assert torch.equal(got_i[used], want_i[used])
    say(f"no-alloc mask {T}x{H}x{W} heads {heads} d {d}: {int(want_c.sum())} kept blocks, equal")


def test_noalloc_mask_equals_workspace_mask_twice():
    # 720p shape, 40 heads: 7.7 MB per (batch, head) pair, several passes of the array
    _case(21, 45, 80, 40, 128, 0.7, 3, 0.7935, None, None)
    # then a smaller ragged input with a window and unit scale
    _case(3, 21, 35, 3, 64, 1.0, 4, 0.6, (1, 1, 1), 1.0)


def test_noalloc_mask_largest_pair():
    """768p: one (batch, head) pair (69 MB) per pass of the 96 MiB array."""
    _case(61, 48, 84, 2, 128, 0.7, 5, 0.8447, None, None)
