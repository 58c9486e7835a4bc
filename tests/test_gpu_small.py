"""GPU parity at sizes the oracle finishes in seconds: every stage of the HIP
path against the CPU oracle on the same seeded inputs, through the C ABI.

Grids include ragged ones (H, W not multiples of 8) so that partially padded
blocks, several tiles and a ragged tail are covered.
"""
import math

import numpy as np
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from synth import fourier_video_qkv, gaussian_video_qkv
from tests.parity import (assert_inputs_discriminate, compare_attention, compare_masks,
                          rescale_rows, say, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (T, H, W, heads, d, dtype, amplitude)
GRIDS = {
    "tiny-f32-d64": (4, 16, 16, 2, 64, "f32", 1.0),
    "ragged-bf16-d128": (3, 21, 35, 3, 128, "bf16", 0.7),
    "ragged-f32-d128": (2, 13, 27, 2, 128, "f32", 0.7),
    "ragged-bf16-d64": (5, 9, 17, 2, 64, "bf16", 1.0),
    "wide-bf16-d128": (3, 24, 88, 2, 128, "bf16", 0.7),
    "one-block-bf16": (1, 8, 8, 2, 64, "bf16", 1.0),
    "one-partial-block-f32": (1, 3, 5, 2, 128, "f32", 1.0),
    "one-row-high-bf16": (7, 1, 40, 1, 128, "bf16", 1.0),
}


def make(name, seed=0):
    T, H, W, heads, d, dt, amp = GRIDS[name]
    q, k, v = fourier_video_qkv(T, H, W, heads, d, amp, seed=seed, dtype=dt)
    g = cabf.Geom(1, heads, d, T, H, W, 8)
    og = oracle.Grid(T, H, W, 8)
    return g, og, q.to(DEV), k.to(DEV), v.to(DEV)


@pytest.mark.parametrize("name", sorted(GRIDS))
def test_permute_unpermute_bitexact(name):
    say(f"permute {name}")
    g, og, q, k, v = make(name)
    qp, kp, vp = cabf.permute(q, k, v, g)
    torch.cuda.synchronize()
    for src, dst in ((q, qp), (k, kp), (v, vp)):
        want = oracle.permute(src.cpu().view(torch.int16 if src.dtype == torch.bfloat16 else torch.int32).numpy(), og)
        got = dst.cpu().view(torch.int16 if dst.dtype == torch.bfloat16 else torch.int32).numpy()
        assert np.array_equal(got, want)
    back = cabf.unpermute(vp, g)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu().view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32),
                       v.cpu().view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32))


def test_permute_skips_null_pairs():
    g, og, q, k, v = make("ragged-bf16-d64")
    n = g.sizes()["tokens_padded"]
    kp = torch.full((1, g.heads, n, g.head_dim), 7.0, dtype=q.dtype, device=DEV)
    cabf.cabf_permute(g, None, k, None, None, kp, None)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(kp), oracle.permute(to_np(k), og))


MASK_CASES = [
    ("tiny-f32-d64", 0.2, (1, 1, 1), None),
    ("tiny-f32-d64", 0.5, None, None),
    ("ragged-bf16-d128", 0.3, None, None),
    ("ragged-bf16-d128", 0.75, (1, 1, 1), None),
    ("ragged-bf16-d128", 0.6, None, 1.0),          # unit scale: sharper block softmax
    ("ragged-f32-d128", 0.4, (0, 1, 2), None),
    ("ragged-bf16-d64", 0.9, (1, 0, 0), 1.0),
    ("wide-bf16-d128", 0.8, None, 1.0),
    ("one-block-bf16", 0.5, None, None),
    ("one-partial-block-f32", 0.5, (1, 1, 1), None),
    ("one-row-high-bf16", 0.3, (1, 0, 1), 1.0),
]


@pytest.mark.parametrize("name,thr,sta,scale", MASK_CASES)
def test_block_mask_matches_oracle(name, thr, sta, scale):
    say(f"mask {name} thr={thr} sta={sta} scale={scale}")
    g, og, q, k, v = make(name)
    s = cabf.default_scale(g) if scale is None else scale
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx, probs = cabf.build_block_mask(qp, kp, g, thr, sta, s, return_probs=True)
    torch.cuda.synchronize()
    info = oracle.build_block_mask(to_np(qp), to_np(kp), og, s, thr, sta)
    p_gpu = probs.cpu().numpy().astype(np.float64)
    rel = np.abs(p_gpu - info["p"]) / info["p"]
    say(f"block prob max rel err {rel.max():.3e}")
    assert rel.max() < 2e-5
    compare_masks(cnt, idx, info, thr, label=f"{name} thr={thr} sta={sta}")
    # the same decision taken by the oracle in fp32 as well
    info32 = oracle.build_block_mask(to_np(qp), to_np(kp), og, s, thr, sta, precision=np.float32)
    info32.update({kk: info[kk] for kk in ("s_prev", "s_k", "p_k", "p_next", "k")})
    compare_masks(cnt, idx, info32, thr, label=f"{name} (fp32 oracle)")


@pytest.mark.parametrize("thr", [0.0, 1.0])
def test_block_mask_threshold_extremes(thr):
    g, og, q, k, v = make("ragged-bf16-d128")
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr)
    torch.cuda.synchronize()
    info = oracle.build_block_mask(to_np(qp), to_np(kp), og, cabf.default_scale(g), thr)
    c = cnt.cpu().numpy()
    if thr == 0.0:
        assert np.all(c == og.nb)
    else:
        assert np.all(c == 1)
    compare_masks(cnt, idx, info, thr, label=f"thr={thr}")


@pytest.mark.parametrize("n_blocks_t,thr", [(4, 0.2), (6, 0.37)])
def test_block_mask_uniform_rows_keep_lowest_indices(n_blocks_t, thr):
    """Constant K: every block probability is equal, so the cut keeps the
    ceil((1-thr) nb) lowest block indices (NABLA CDF cut with index tie-break)."""
    T, H, W, d = n_blocks_t, 16, 16, 64
    g = cabf.Geom(1, 1, d, T, H, W, 8)
    torch.manual_seed(3)
    q = torch.randn(1, 1, T * H * W, d, device=DEV).to(torch.bfloat16)
    k = torch.full((1, 1, T * H * W, d), 0.25, device=DEV).to(torch.bfloat16)
    qp, kp, _ = cabf.permute(q, k, k, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr)
    torch.cuda.synchronize()
    nb = g.sizes()["n_blocks"]
    want = math.ceil((1 - thr) * nb)
    assert np.all(cnt.cpu().numpy() == want)
    assert np.all(idx.cpu().numpy()[..., :want] == np.arange(want))


TOPK_CASES = [
    ("tiny-f32-d64", 3, None, None),
    ("ragged-bf16-d128", 1, None, None),
    ("ragged-bf16-d128", 17, (1, 1, 1), None),
    ("ragged-bf16-d128", 10_000, None, None),        # k >= nb keeps every block
    ("ragged-f32-d128", 9, (0, 1, 2), 1.0),
    ("wide-bf16-d128", 40, None, 1.0),
    ("one-block-bf16", 1, None, None),
    ("one-row-high-bf16", 5, (1, 0, 1), 1.0),
]


@pytest.mark.parametrize("name,k,sta,scale", TOPK_CASES)
def test_topk_mask_matches_oracle(name, k, sta, scale):
    """Fixed-budget selection: the k most probable blocks (ties to the lower
    index) OR the window; rows with a near-tie at the k-th block are exempt."""
    say(f"topk mask {name} k={k} sta={sta} scale={scale}")
    g, og, q, k_, v = make(name)
    s = cabf.default_scale(g) if scale is None else scale
    qp, kp, vp = cabf.permute(q, k_, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, 0.0, sta, s, topk=k)
    torch.cuda.synchronize()
    info = oracle.build_block_mask(to_np(qp), to_np(kp), og, s, 0.0, sta, topk=k)
    compare_masks(cnt, idx, info, 0.0, label=f"{name} topk={k} sta={sta}")
    if sta is None:
        assert np.all(cnt.cpu().numpy() == min(k, og.nb))


@pytest.mark.parametrize("grid,win", [((4, 16, 16, 8), (1, 1, 1)), ((5, 24, 40, 8), (1, 1, 2)),
                                      ((3, 21, 35, 8), (0, 2, 1)), ((7, 1, 40, 8), (2, 0, 0))])
def test_sta_only_lists_match_oracle(grid, win):
    T, H, W, P = grid
    g = cabf.Geom(2, 3, 64, T, H, W, P)
    og = oracle.Grid(T, H, W, P)
    cnt, idx = cabf.build_sta_mask(g, win, DEV)
    torch.cuda.synchronize()
    want_cnt, want_idx = oracle.sta_only_lists(og, *win)
    c, ix = cnt.cpu().numpy(), idx.cpu().numpy()
    for pos in np.ndindex(*c.shape):
        assert np.array_equal(c[pos], want_cnt[pos[-1]])
        n = c[pos]
        assert np.array_equal(ix[pos][:n], want_idx[pos[-1]][:n])


ATTN_CASES = [
    ("tiny-f32-d64", 0.2, (1, 1, 1)),
    ("ragged-f32-d128", 0.4, None),
    ("ragged-bf16-d128", 0.3, (1, 1, 1)),
    ("ragged-bf16-d64", 0.5, None),
    ("wide-bf16-d128", 0.8, None),
    ("ragged-bf16-d128", 0.0, None),
    ("one-block-bf16", 0.5, None),
    ("one-partial-block-f32", 0.5, None),
    ("one-row-high-bf16", 0.3, (1, 0, 1)),
]


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("name,thr,sta", ATTN_CASES)
def test_attention_on_oracle_lists(name, thr, sta, deterministic):
    """bsa_forward fed the oracle's own block lists equals the oracle's attention,
    in the default order (bf16: clock-phased start) and in list order."""
    say(f"attention {name} thr={thr} sta={sta} deterministic={deterministic}")
    g, og, q, k, v = make(name)
    s = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, k, v, g)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(qp), to_np(kp), to_np(vp)
    info = oracle.build_block_mask(qn, kn, og, s, thr, sta)
    cnt = torch.from_numpy(info["kv_count"]).to(DEV)
    idx = torch.from_numpy(info["kv_index"]).to(DEV)
    op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True,
                               deterministic=deterministic)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.bsa_forward(qn, kn, vn, info["kv_count"], info["kv_index"], og, s)
    compare_attention(op, ref_o, q.dtype == torch.bfloat16, lse, ref_lse, label=name)


SHARP_SCALE = 3.5   # times 1/sqrt(d): token-independent inputs, weights on a few keys


@pytest.mark.parametrize("name,thr", [("ragged-bf16-d128", 0.3), ("wide-bf16-d128", 0.6),
                                      ("ragged-bf16-d64", 0.5), ("one-row-high-bf16", 0.2)])
def test_attention_sharp_on_oracle_lists(name, thr):
    """Inputs that a wrong kernel cannot pass: token-independent Q, K, V at
    scale 3.5/sqrt(d), on ragged grids with partial patches, over the oracle's
    lists. A kernel with uniform weights or a wrong V key order misses by more
    than ten times the tolerance (planted in the oracle's inputs on the CPU),
    and the lazy rescale of the online softmax fires; the GPU, in both visit
    orders, stays within the tolerance."""
    T, H, W, heads, d, _, _ = GRIDS[name]
    say(f"sharp attention {name} thr={thr}")
    q, k, v = gaussian_video_qkv(T, H, W, heads, d, seed=6, device=DEV)
    g = cabf.Geom(1, heads, d, T, H, W, 8)
    og = oracle.Grid(T, H, W, 8)
    s = SHARP_SCALE / math.sqrt(d)
    qp, kp, vp = cabf.permute(q, k, v, g)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(qp), to_np(kp), to_np(vp)
    info = oracle.build_block_mask(qn, kn, og, s, thr, None)
    cnt = torch.from_numpy(info["kv_count"]).to(DEV)
    idx = torch.from_numpy(info["kv_index"]).to(DEV)
    ref_o, ref_lse = oracle.bsa_forward(qn, kn, vn, info["kv_count"], info["kv_index"], og, s)
    blocks = list(range(og.nb))
    hits = 0
    for hd in range(heads):
        c, ix = info["kv_count"][0, hd], info["kv_index"][0, hd]
        assert_inputs_discriminate(qn[0, hd], kn[0, hd], vn[0, hd], c, ix, og, s, blocks,
                                   ref_o[0, hd])
        hits += rescale_rows(qn[0, hd], kn[0, hd], c, ix, og, s, blocks)[0]
    say(f"rows whose list-order pass must rescale: {hits}")
    assert hits > 0
    for det in (True, False):
        op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=det)
        torch.cuda.synchronize()
        compare_attention(op, ref_o, True, lse, ref_lse, label=f"sharp {name} det={det}")


@pytest.mark.parametrize("name", ["wide-bf16-d128", "ragged-bf16-d64"])
def test_attention_visit_orders(name):
    """Deterministic mode (lists walked from their first entry) is bit-identical
    run to run; the default clock-phased start (a rotation of each list, which
    varies between runs) stays within the same tolerance of the oracle."""
    say(f"attention visit orders {name}")
    g, og, q, k, v = make(name)
    s = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, k, v, g)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(qp), to_np(kp), to_np(vp)
    info = oracle.build_block_mask(qn, kn, og, s, 0.3, None)
    cnt = torch.from_numpy(info["kv_count"]).to(DEV)
    idx = torch.from_numpy(info["kv_index"]).to(DEV)
    ref_o, ref_lse = oracle.bsa_forward(qn, kn, vn, info["kv_count"], info["kv_index"], og, s)
    o1, l1 = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    o2, l2 = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    compare_attention(o1, ref_o, True, l1, ref_lse, label=f"{name} deterministic")
    for rep in range(3):
        o3, l3 = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True)
        torch.cuda.synchronize()
        compare_attention(o3, ref_o, True, l3, ref_lse, label=f"{name} clock-phased #{rep}")


@pytest.mark.parametrize("name", ["ragged-bf16-d128", "ragged-bf16-d64", "ragged-f32-d128"])
def test_attention_ignores_finite_pad_values(name):
    """Pad slots of qp, kp, vp holding large finite values (instead of the
    zeros cabf_permute writes) leave every real row within the tolerance of
    the oracle's attention computed with zero pads (pad keys get weight 0).
    fp32 rows are bit-identical; bf16 rows may differ in the last bits,
    because a running max raised for any row of a wave (pad rows included)
    re-bases the exponentials of all its rows."""
    g, og, q, k, v = make(name)
    s = cabf.default_scale(g)
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, 0.4, None, s)
    o1, l1 = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.bsa_forward(to_np(qp), to_np(kp), to_np(vp), cnt.cpu().numpy(),
                                        idx.cpu().numpy(), og, s)
    pad_np = ~oracle.valid_slots(og)
    pad = torch.from_numpy(pad_np).to(DEV)
    assert bool(pad.any())
    for t, val in ((qp, -300.0), (kp, 250.0), (vp, 1000.0)):
        t[:, :, pad] = val
    o2, l2 = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    torch.cuda.synchronize()
    real = np.nonzero(~pad_np)[0]
    assert torch.isfinite(o2[:, :, ~pad]).all()
    bf16 = q.dtype == torch.bfloat16
    compare_attention(o2[0].permute(1, 0, 2), ref_o[0].transpose(1, 0, 2), bf16,
                      l2[0].T, ref_lse[0].T, rows=real, label=f"{name} pad values")
    if not bf16:
        assert torch.equal(o1[:, :, ~pad], o2[:, :, ~pad])
        assert torch.equal(l1[:, :, ~pad], l2[:, :, ~pad])


@pytest.mark.parametrize("deterministic", [False, True])
def test_attention_rows_with_no_blocks_and_arbitrary_lists(deterministic):
    """Random lists (no structure) with an empty row: in list order the empty
    block shares its workgroup with a block that keeps tiles."""
    g, og, q, k, v = make("ragged-bf16-d128")
    nb = og.nb
    qp, kp, vp = cabf.permute(q, k, v, g)
    rng = np.random.default_rng(5)
    mask = rng.random((1, g.heads, nb, nb)) < 0.3
    mask[0, 0, 3] = False            # a row that keeps nothing
    mask[0, 1, :5] = False
    cnt_np, idx_np = oracle.mask_to_lists(mask)
    op, lse = cabf.bsa_forward(qp, kp, vp, torch.from_numpy(cnt_np).to(DEV),
                               torch.from_numpy(idx_np).to(DEV), g, return_lse=True,
                               deterministic=deterministic)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.bsa_forward(to_np(qp), to_np(kp), to_np(vp), cnt_np, idx_np, og,
                                        cabf.default_scale(g))
    compare_attention(op, ref_o, True, lse, ref_lse, label=f"arbitrary lists det={deterministic}")
    assert torch.all(op[0, 0, 3 * 64:4 * 64] == 0)
    assert torch.all(torch.isneginf(lse[0, 0, 3 * 64:4 * 64]))


@pytest.mark.parametrize("name,thr,sta", [("tiny-f32-d64", 0.2, (1, 1, 1)),
                                          ("ragged-bf16-d128", 0.5, (1, 1, 1)),
                                          ("wide-bf16-d128", 0.8, None)])
def test_layer_end_to_end(name, thr, sta):
    """permute_pool -> build_block_mask_pooled -> bsa_forward -> unpermute (the
    layer helper) on the GPU against the oracle: the lists against the
    oracle's cut (differing rows must be correct cuts), every raster row
    against the oracle's attention over the GPU's own lists."""
    say(f"layer {name}")
    g, og, q, k, v = make(name)
    s = cabf.default_scale(g)
    o, (cnt, idx) = cabf.layer(q, k, v, g, thr, sta, s)
    torch.cuda.synchronize()
    qn, kn, vn = (oracle.permute(to_np(t), og) for t in (q, k, v))
    info = oracle.build_block_mask(qn, kn, og, s, thr, sta)
    compare_masks(cnt, idx, info, thr, label=f"layer {name}")
    ref_op, _ = oracle.bsa_forward(qn, kn, vn, cnt.cpu().numpy(), idx.cpu().numpy(), og, s)
    ref_o = oracle.unpermute(ref_op, og)
    err = np.abs(to_np(o) - ref_o)
    say(f"layer {name}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    if q.dtype == torch.bfloat16:
        assert err.max() <= 2e-2 and err.mean() <= 2e-3
    else:
        assert err.max() <= 1e-4


def test_mfma_peak_probe_runs():
    """The benchmark's measurement aid (its own library): every lane writes the
    sum of its accumulators, finite and positive (products of positive inputs)."""
    from content_adaptive_block_fractal_amd import peak_probe
    out = torch.full((8 * 256,), -1.0, device=DEV)
    peak_probe.mfma_peak(8, 3, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out > 0).all()
