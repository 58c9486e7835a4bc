"""Pins of the CPU oracle against what the NABLA page and the mathematics fix.

Each test names the property it pins. None of them re-types the oracle's own
formula: they use hand-derived values (tests/golden), closed forms, special
cases that reduce to textbook routines, invariants and brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.nabla import brute_force_cut, brute_force_topk

RNG = np.random.default_rng(1234)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# --- fractal flattening --------------------------------------------------------

def test_fractal_positions_golden(golden_dir):
    data = _load(golden_dir, "fractal_positions.json")
    for case in data["cases"]:
        g = oracle.Grid(*case["grid"])
        pos = oracle.fractal_positions(g)
        for (t, y, x), want in zip(case["txy"], case["expected"]):
            assert pos[(t * g.H + y) * g.W + x] == want, (case["grid"], (t, y, x))


@pytest.mark.parametrize("grid", [(1, 16, 16, 8), (3, 5, 7, 2), (2, 9, 17, 8), (21, 30, 52, 8)])
def test_fractal_is_injective_into_padded_grid(grid):
    g = oracle.Grid(*grid)
    pos = oracle.fractal_positions(g)
    assert pos.size == g.n_valid
    assert np.unique(pos).size == pos.size
    assert pos.min() >= 0 and pos.max() < g.N
    # every block keeps its real tokens together: block of a token = its patch
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.H), np.arange(g.W), indexing="ij")
    patch = ((t * g.Ty + y // g.P) * g.Tx + x // g.P).reshape(-1)
    assert np.array_equal(pos // g.block, patch)
    # time order kept: all tokens of frame t come before those of frame t+1
    frame = t.reshape(-1)
    for f in range(g.T - 1):
        assert pos[frame == f].max() < pos[frame == f + 1].min()


@pytest.mark.parametrize("grid", [(1, 16, 16, 8), (3, 5, 7, 2), (2, 9, 17, 8)])
def test_permute_roundtrip_bitwise(grid):
    g = oracle.Grid(*grid)
    x = RNG.standard_normal((2, 3, g.n_valid, 5)).astype(np.float32)
    xp = oracle.permute(x, g)
    assert xp.shape == (2, 3, g.N, 5)
    back = oracle.unpermute(xp, g)
    assert back.dtype == x.dtype and np.array_equal(back.view(np.uint32), x.view(np.uint32))
    valid = oracle.valid_slots(g)
    assert np.all(xp[..., ~valid, :] == 0)
    assert valid.sum() == g.n_valid


# --- block pooling ---------------------------------------------------------------

def test_pool_golden(golden_dir):
    data = _load(golden_dir, "block_pool_cases.json")
    g = oracle.Grid(*data["grid"])
    x = np.array(data["values_raster"], dtype=np.float64)[:, None]
    qb = oracle.pool_blocks(oracle.permute(x, g), g)
    assert np.array_equal(qb[:, 0], np.array(data["expected_block_means"]))


def test_pool_constant_and_pad_garbage():
    g = oracle.Grid(2, 5, 7, 2)
    x = np.full((g.n_valid, 3), 0.37)
    xp = oracle.permute(x, g)
    xp[~oracle.valid_slots(g)] = 123.0        # pads must not enter the mean
    assert np.allclose(oracle.pool_blocks(xp, g), 0.37, rtol=0, atol=1e-15)


def test_pool_affine_ramp_equals_ramp_at_centre_of_real_region():
    g = oracle.Grid(3, 13, 11, 4)
    a, by, bx, c = 0.3, -1.7, 2.25, 0.5
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.H), np.arange(g.W), indexing="ij")
    ramp = (a * t + by * y + bx * x + c).reshape(-1, 1)
    qb = oracle.pool_blocks(oracle.permute(ramp, g), g)[:, 0]
    bt, bty, btx = oracle.block_coords(g)
    y0, x0 = bty * g.P, btx * g.P
    y1 = np.minimum(y0 + g.P, g.H) - 1
    x1 = np.minimum(x0 + g.P, g.W) - 1
    want = a * bt + by * (y0 + y1) / 2 + bx * (x0 + x1) / 2 + c
    assert np.allclose(qb, want, rtol=0, atol=1e-12)


# --- reduced attention and the CDF cut ----------------------------------------------

def test_block_logits_and_probs_golden(golden_dir):
    data = _load(golden_dir, "block_cut_cases.json")
    lg = data["logits"]
    z = oracle.block_logits(np.array(lg["qb"]), np.array(lg["kb"]), lg["scale"])
    assert np.allclose(z, np.array(lg["expected_z"]), rtol=0, atol=1e-15)
    pr = data["probs"]
    p = oracle.block_probs(np.array(pr["z"]))
    assert np.allclose(p, np.array(pr["expected_p"]), rtol=0, atol=1e-15)


def test_cut_golden(golden_dir):
    data = _load(golden_dir, "block_cut_cases.json")
    for case in data["cuts"]:
        got = oracle.cdf_cut(np.array(case["p"], dtype=np.float64), case["thr"])
        assert got.tolist() == case["expected"], case


@pytest.mark.parametrize("n,thr", [(16, 0.2), (64, 0.05), (1000, 0.2345), (1260, 0.8123), (4026, 0.8519)])
def test_cut_uniform_rows_keep_lowest_ceil(n, thr):
    p = np.full(n, 1.0 / n)
    got = oracle.cdf_cut(p, thr)
    k = math.ceil((1 - thr) * n)
    assert abs((1 - thr) * n - round((1 - thr) * n)) > 1e-6   # not on a rounding boundary
    assert got.tolist() == list(range(k))


def test_cut_one_hot_keeps_one():
    p = np.full(50, 1e-9)
    p[17] = 1.0 - 49e-9
    for thr in (0.01, 0.2, 0.9):
        assert oracle.cdf_cut(p, thr).tolist() == [17]


def test_cut_invariants_random_rows():
    for trial in range(200):
        n = int(RNG.integers(1, 300))
        z = RNG.standard_normal(n) * RNG.uniform(0.01, 5)
        p = np.exp(z - z.max()); p /= p.sum()
        thr = float(RNG.uniform(0.001, 0.999))
        kept, k, s_prev, s_k, p_k, p_next = oracle.cdf_cut_details(p, thr)
        assert kept.size == k >= 1
        assert np.all(np.diff(kept) > 0)
        mass = p[kept].sum()
        assert mass >= (1 - thr) - 1e-12 or k == n
        assert s_prev < 1 - thr
        # every dropped block has probability <= every kept block
        dropped = np.setdiff1d(np.arange(n), kept)
        if dropped.size:
            assert p[dropped].max() <= p[kept].min()


def test_cut_matches_brute_force_subsets():
    for trial in range(120):
        n = int(RNG.integers(1, 11))
        p = RNG.uniform(0.05, 1.0, n)
        p /= p.sum()
        thr = float(RNG.uniform(0.01, 0.95))
        # keep the case away from exact mass ties that floating order could flip
        got = oracle.cdf_cut(p, thr)
        want = brute_force_cut(p, thr)
        assert got.tolist() == sorted(want.tolist()), (p, thr)


def test_exempt_rows_classification():
    info = dict(k=np.array([3, 3, 3]), s_prev=np.array([0.79995, 0.5, 0.7]),
                s_k=np.array([0.9, 0.80008, 0.9]), p_k=np.array([0.1, 0.3, 0.2]),
                p_next=np.array([0.05, 0.1, 0.2 * (1 - 1e-7)]))
    e1, e2 = oracle.exempt_rows(info, 0.2)
    assert e1.tolist() == [True, True, False]
    assert e2.tolist() == [False, False, True]


# --- fixed-budget (top-k) selection ------------------------------------------------

@pytest.mark.parametrize("n,k", [(16, 3), (64, 64), (1260, 252), (4026, 604), (10, 25)])
def test_topk_uniform_rows_keep_lowest_k(n, k):
    p = np.full(n, 1.0 / n)
    assert oracle.topk_cut(p, k).tolist() == list(range(min(k, n)))


def test_topk_one_is_argmax_lowest_index():
    for trial in range(50):
        n = int(RNG.integers(1, 200))
        p = RNG.integers(0, 5, n).astype(np.float64) + 1.0   # many exact ties
        p /= p.sum()
        assert oracle.topk_cut(p, 1).tolist() == [int(np.argmax(p))]


def test_topk_matches_brute_force_subsets():
    for trial in range(120):
        n = int(RNG.integers(1, 11))
        p = RNG.uniform(0.05, 1.0, n)
        p /= p.sum()
        k = int(RNG.integers(1, n + 1))
        assert oracle.topk_cut(p, k).tolist() == brute_force_topk(p, k).tolist(), (p, k)


def test_topk_invariants_random_rows():
    for trial in range(200):
        n = int(RNG.integers(1, 300))
        z = RNG.standard_normal(n) * RNG.uniform(0.01, 5)
        p = np.exp(z - z.max()); p /= p.sum()
        k = int(RNG.integers(1, n + 3))
        kept, kk, p_k, p_next = oracle.topk_cut_details(p, k)
        assert kept.size == kk == min(k, n)
        assert np.all(np.diff(kept) > 0)
        dropped = np.setdiff1d(np.arange(n), kept)
        if dropped.size:
            assert p[dropped].max() <= p[kept].min() == p_k
            assert p_next == p[dropped].max()


def test_topk_mask_exempts_only_near_ties():
    g = oracle.Grid(2, 16, 24, 8)
    q = RNG.standard_normal((1, g.n_valid, 16))
    k = RNG.standard_normal((1, g.n_valid, 16))
    qp, kp = oracle.permute(q, g), oracle.permute(k, g)
    info = oracle.build_block_mask(qp, kp, g, 0.25, 0.0, sta=(0, 1, 1), topk=4)
    assert info["mode"] == "topk"
    assert np.all(info["adaptive"].sum(-1) == 4)
    assert np.array_equal(info["mask"], info["adaptive"] | oracle.sta_mask(g, 0, 1, 1)[None])
    e1, e2 = oracle.exempt_rows(info, 0.0)
    assert not e1.any()
    assert np.array_equal(e2, (info["p_k"] - info["p_next"]) <= 1e-6 * info["p_k"])


def test_sta_only_lists_are_the_window():
    g = oracle.Grid(5, 24, 40, 8)
    cnt, idx = oracle.sta_only_lists(g, 1, 1, 2)
    m = oracle.sta_mask(g, 1, 1, 2)
    assert np.array_equal(cnt, m.sum(-1))
    assert np.array_equal(oracle.lists_to_mask(cnt, idx, g.nb), m)
    for i in range(g.nb):
        assert np.all(np.diff(idx[i][: cnt[i]]) > 0)


# --- sliding tile window ----------------------------------------------------------

@pytest.mark.parametrize("grid,win", [((4, 16, 16, 8), (1, 1, 1)), ((5, 24, 40, 8), (1, 1, 2)),
                                      ((3, 7, 9, 2), (0, 2, 1))])
def test_sta_window_counts_closed_form(grid, win):
    g = oracle.Grid(*grid)
    m = oracle.sta_mask(g, *win)
    bt, bty, btx = oracle.block_coords(g)
    def span(c, r, L):
        return np.minimum(c + r, L - 1) - np.maximum(c - r, 0) + 1
    want = span(bt, win[0], g.T) * span(bty, win[1], g.Ty) * span(btx, win[2], g.Tx)
    assert np.array_equal(m.sum(axis=1), want)
    assert np.array_equal(m, m.T) and np.all(np.diag(m))


def test_mask_is_cut_union_window():
    g = oracle.Grid(3, 16, 24, 8)
    q = RNG.standard_normal((2, g.n_valid, 16))
    k = RNG.standard_normal((2, g.n_valid, 16))
    qp, kp = oracle.permute(q, g), oracle.permute(k, g)
    a = oracle.build_block_mask(qp, kp, g, 0.25, 0.4)
    b = oracle.build_block_mask(qp, kp, g, 0.25, 0.4, sta=(1, 1, 1))
    assert np.array_equal(a["adaptive"], b["adaptive"])
    assert np.array_equal(b["mask"], a["adaptive"] | oracle.sta_mask(g, 1, 1, 1)[None])
    cnt, idx = b["kv_count"], b["kv_index"]
    assert np.array_equal(oracle.lists_to_mask(cnt, idx, g.nb), b["mask"])
    assert np.all(cnt >= 1)


# --- attention over kept tiles -------------------------------------------------------

def test_attention_golden(golden_dir):
    data = _load(golden_dir, "attention_cases.json")
    g = oracle.Grid(*data["grid"])
    q, k, v = (np.array(data[n]) for n in ("q", "k", "v"))
    lists = data["kv_lists"]
    cnt = np.array([len(l) for l in lists], dtype=np.int32)
    idx = np.full((g.nb, g.nb), -1, dtype=np.int32)
    for i, l in enumerate(lists):
        idx[i, : len(l)] = l
    o, lse = oracle.bsa_forward(q, k, v, cnt, idx, g, data["scale"])
    assert np.allclose(o, np.array(data["expected_o"]), rtol=0, atol=1e-15)
    assert np.allclose(lse, np.array(data["expected_lse"]), rtol=0, atol=1e-15)
    dense = oracle.dense_attention(q[:1], k, v, data["scale"])
    assert np.allclose(dense, np.array(data["expected_o"][:1]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("grid", [(2, 16, 16, 8), (2, 9, 13, 4)])
def test_thr_zero_is_dense_attention(grid):
    g = oracle.Grid(*grid)
    d = 8
    q, k, v = (RNG.standard_normal((2, g.n_valid, d)) for _ in range(3))
    scale = 1 / math.sqrt(d)
    o, info = oracle.layer(q, k, v, g, scale, thr=0.0)
    assert np.all(info["kv_count"] == g.nb)
    want = oracle.dense_attention(q, k, v, scale)
    assert np.allclose(o, want, rtol=0, atol=1e-12)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
    assert np.allclose(o, sdpa, rtol=0, atol=1e-12)
    # lse over all real keys
    qp, kp = oracle.permute(q, g), oracle.permute(k, g)
    vp = oracle.permute(v, g)
    _, lse = oracle.bsa_forward(qp, kp, vp, info["kv_count"], info["kv_index"], g, scale)
    s = scale * q @ np.swapaxes(k, -1, -2)
    want_lse = np.log(np.exp(s).sum(-1))
    assert np.allclose(oracle.unpermute(lse[..., None], g)[..., 0], want_lse, rtol=0, atol=1e-12)


def test_block_sparse_matches_token_bruteforce():
    g = oracle.Grid(2, 3, 5, 2)     # 12 blocks of 4 tokens, pads in the last patch row/column
    d = 3
    q, k, v = (RNG.standard_normal((g.n_valid, d)) for _ in range(3))
    qp, kp, vp = (oracle.permute(a, g) for a in (q, k, v))
    mask = RNG.random((g.nb, g.nb)) < 0.4
    mask[np.arange(g.nb), RNG.integers(0, g.nb, g.nb)] = True
    cnt, idx = oracle.mask_to_lists(mask)
    o, _ = oracle.bsa_forward(qp, kp, vp, cnt, idx, g, 0.7)
    want = oracle.masked_attention_bruteforce(qp, kp, vp, g, mask, 0.7)
    assert np.allclose(o, want, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    g = oracle.Grid(2, 10, 12, 4)
    q, k = (RNG.standard_normal((g.n_valid, 6)) for _ in range(2))
    v = np.tile(RNG.standard_normal((1, 6)), (g.n_valid, 1))
    o, _ = oracle.layer(q, k, v, g, 0.5, thr=0.3, sta=(1, 1, 1))
    assert np.allclose(o, v, rtol=0, atol=1e-13)


def test_pad_slot_contents_do_not_change_real_outputs():
    g = oracle.Grid(2, 10, 13, 4)
    q, k, v = (RNG.standard_normal((g.n_valid, 5)) for _ in range(3))
    qp, kp, vp = (oracle.permute(a, g) for a in (q, k, v))
    info = oracle.build_block_mask(qp, kp, g, 0.4, 0.25)
    o1, _ = oracle.bsa_forward(qp, kp, vp, info["kv_count"], info["kv_index"], g, 0.4)
    pad = ~oracle.valid_slots(g)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[pad] = 50.0
    vp2[pad] = -9.0
    info2 = oracle.build_block_mask(qp, kp2, g, 0.4, 0.25)
    assert np.array_equal(info["mask"], info2["mask"])
    o2, _ = oracle.bsa_forward(qp, kp2, vp2, info["kv_count"], info["kv_index"], g, 0.4)
    assert np.allclose(o1[~pad], o2[~pad], rtol=0, atol=1e-13)


def test_result_does_not_depend_on_order_inside_a_patch():
    """Sparse VideoGen2 summary, section 2A: a token permutation undone at the output
    leaves attention unchanged; here the order inside every block is shuffled."""
    g = oracle.Grid(3, 12, 16, 4)
    q, k, v = (RNG.standard_normal((g.n_valid, 4)) for _ in range(3))
    qp, kp, vp = (oracle.permute(a, g) for a in (q, k, v))
    perm = np.concatenate([b * g.block + RNG.permutation(g.block) for b in range(g.nb)])
    info = oracle.build_block_mask(qp, kp, g, 0.6, 0.35, sta=(0, 1, 1))
    o1, l1 = oracle.bsa_forward(qp, kp, vp, info["kv_count"], info["kv_index"], g, 0.6)

    class Shuffled(oracle.Grid):
        pass
    valid = oracle.valid_slots(g)
    # shuffled copies: slot j of the new layout holds old slot perm[j]
    qs, ks, vs = qp[perm], kp[perm], vp[perm]
    # pooling and the mask only see block membership, so they are unchanged
    qb = qs.reshape(g.nb, g.block, -1)
    vmask = valid[perm].reshape(g.nb, g.block)
    means = (qb * vmask[..., None]).sum(1) / vmask.sum(1)[:, None]
    assert np.allclose(means, oracle.pool_blocks(qp, g), rtol=0, atol=1e-13)
    # attention row by row on the shuffled layout, with the same block lists
    for i in range(g.nb):
        keys = np.concatenate([np.arange(b * g.block, (b + 1) * g.block)
                               for b in info["kv_index"][i][: info["kv_count"][i]]])
        keys = keys[valid[perm][keys]]
        s = 0.6 * qs[i * g.block:(i + 1) * g.block] @ ks[keys].T
        w = np.exp(s - s.max(1, keepdims=True))
        o = (w @ vs[keys]) / w.sum(1, keepdims=True)
        assert np.allclose(o, o1[perm[i * g.block:(i + 1) * g.block]], rtol=0, atol=1e-13)


# --- backward --------------------------------------------------------------------

def _bwd_case(seed=0, thr=0.4):
    g = oracle.Grid(2, 11, 13, 8)          # partially padded blocks
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((g.n_valid, 6)) for _ in range(4))
    qp, kp, vp = oracle.permute(q, g), oracle.permute(k, g), oracle.permute(v, g)
    dop = oracle.permute(do, g)              # pad rows of the gradient are zero
    info = oracle.build_block_mask(qp, kp, g, 0.9, thr)
    return g, qp, kp, vp, dop, info


def test_backward_matches_finite_differences():
    """Central differences of L = <dop, bsa_forward(...)> over real rows."""
    g, qp, kp, vp, dop, info = _bwd_case()
    cnt, idx = info["kv_count"], info["kv_index"]
    dq, dk, dv = oracle.bsa_backward(qp, kp, vp, dop, cnt, idx, g, 0.9)
    valid = oracle.valid_slots(g)
    def loss(q_, k_, v_):
        o, _ = oracle.bsa_forward(q_, k_, v_, cnt, idx, g, 0.9)
        return float((o[valid] * dop[valid]).sum())
    h = 1e-6
    rng = np.random.default_rng(1)
    for name, x, grad in (("q", qp, dq), ("k", kp, dk), ("v", vp, dv)):
        for _ in range(6):
            r = int(rng.choice(np.nonzero(valid)[0]))
            c = int(rng.integers(0, x.shape[1]))
            xp_, xm_ = x.copy(), x.copy()
            xp_[r, c] += h
            xm_[r, c] -= h
            args_p = {"q": (xp_, kp, vp), "k": (qp, xp_, vp), "v": (qp, kp, xp_)}[name]
            args_m = {"q": (xm_, kp, vp), "k": (qp, xm_, vp), "v": (qp, kp, xm_)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[r, c]) < 1e-6 * max(1.0, abs(fd)), (name, r, c, fd, grad[r, c])
    pad = ~valid
    assert np.all(dq[pad] == 0) and np.all(dk[pad] == 0) and np.all(dv[pad] == 0)


def test_backward_matches_autograd_of_masked_dense_attention():
    torch = pytest.importorskip("torch")
    g, qp, kp, vp, dop, info = _bwd_case(seed=2, thr=0.3)
    dq, dk, dv = oracle.bsa_backward(qp, kp, vp, dop, info["kv_count"], info["kv_index"], g, 0.9)
    valid = oracle.valid_slots(g)
    blk = np.arange(g.N) // g.block
    allowed = info["mask"][blk][:, blk] & valid[None, :]           # [N, N] token mask
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in
         (("q", qp), ("k", kp), ("v", vp))}
    s = 0.9 * t["q"] @ t["k"].T
    s = s.masked_fill(~torch.from_numpy(allowed), float("-inf"))
    o = torch.softmax(s, dim=-1) @ t["v"]
    rows = torch.from_numpy(valid)
    (o[rows] * torch.from_numpy(dop)[rows]).sum().backward()
    assert np.allclose(dq, t["q"].grad.numpy(), atol=1e-12)
    assert np.allclose(dk, t["k"].grad.numpy(), atol=1e-12)
    assert np.allclose(dv, t["v"].grad.numpy(), atol=1e-12)
