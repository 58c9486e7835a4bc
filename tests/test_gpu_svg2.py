"""GPU parity of the semantic-permutation variant (k-means, permutation,
centroid top-p, cluster attention) against oracle.svg2, through the C ABI.

k-means is checked step by step: the GPU's assignment against the oracle's
nearest centroid for the same centroids (rows whose two nearest centroids are
within a relative 1e-5 in squared distance are exempt: fp32 and fp64 may pick
either), and the GPU's update against the oracle's mean of the GPU's own
previous labels. Later stages are fed the GPU's own earlier outputs, so each
stage is compared on identical inputs.
"""
import numpy as np
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from oracle import svg2
from synth import SEMANTIC_WORKLOADS, gaussian_mixture_qk, kmeans_init_indices
from tests.parity import compare_attention, compare_masks, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GAP_REL = 1e-5


def mixture(n, heads, d, seed, amplitude=8.5, components=10):
    q, k = gaussian_mixture_qk(n, heads, d, components=components, spread=0.15,
                               amplitude=amplitude, seed=seed, dtype="bf16", device=DEV)
    v = torch.randn(1, heads, n, d, generator=torch.Generator(device=DEV).manual_seed(seed + 9),
                    device=DEV).to(torch.bfloat16)
    return q, k, v


def init_idx(n, C, heads, seed):
    return torch.from_numpy(kmeans_init_indices(n, C, heads, seed)[None]).to(DEV)


def check_labels(x, cent, labels, what):
    """GPU labels = oracle nearest centroid of the same centroids, except near ties."""
    a, gap = svg2.kmeans_assign(x, cent)
    d2_scale = float(np.mean(np.sum((x - cent[a]) ** 2, axis=1))) + 1e-30
    exempt = gap <= GAP_REL * max(d2_scale, float(np.mean(np.sum(cent ** 2, axis=1))))
    bad = (labels != a) & ~exempt
    say(f"{what}: labels differ {int((labels != a).sum())} of {labels.size}, "
        f"exempt {int(exempt.sum())}, not exempt {int(bad.sum())}")
    assert not bad.any()


def check_permutation(labels, perm, offsets, counts, C):
    want_perm, want_off = svg2.cluster_permutation(labels, C)
    assert np.array_equal(perm, want_perm)
    assert np.array_equal(offsets, want_off)
    assert np.array_equal(counts, np.diff(want_off))


@pytest.mark.parametrize("d,C", [(128, 40), (64, 17), (128, 1), (128, 1500), (64, 2900)])
def test_kmeans_steps_match_oracle(d, C):
    n, heads = 3000, 2
    q, _, _ = mixture(n, heads, d, seed=4)
    init = init_idx(n, C, heads, seed=5)
    out0 = cabf.kmeans(q, C, init, 0)
    out1 = cabf.kmeans(q, C, init, 1)
    torch.cuda.synchronize()
    for hd in range(heads):
        x = to_np(q[0, hd])
        c0 = x[init[0, hd].cpu().numpy()]
        assert np.array_equal(out0["centroids"][0, hd].cpu().numpy().astype(np.float64), c0)
        l0 = out0["labels"][0, hd].cpu().numpy()
        check_labels(x, c0, l0, f"d={d} C={C} head {hd} assign 0")
        check_permutation(l0, out0["perm"][0, hd].cpu().numpy(), out0["offsets"][0, hd].cpu().numpy(),
                          out0["counts"][0, hd].cpu().numpy(), C)
        # one update from the GPU's own labels
        c1_ref, _ = svg2.kmeans_update(x, l0, c0)
        c1 = out1["centroids"][0, hd].cpu().numpy().astype(np.float64)
        err = np.abs(c1 - c1_ref).max()
        say(f"update 1 max abs err {err:.3e}")
        assert err <= 1e-5 * max(1.0, np.abs(c1_ref).max())
        l1 = out1["labels"][0, hd].cpu().numpy()
        check_labels(x, c1, l1, f"d={d} C={C} head {hd} assign 1")


def test_kmeans_converged_state_and_determinism():
    w = SEMANTIC_WORKLOADS["svg2-tiny"]
    q, k, _ = mixture(w.n, w.heads, w.head_dim, seed=6, amplitude=w.amplitude,
                      components=w.components)
    init = init_idx(w.n, w.ck, w.heads, seed=7)
    a = cabf.kmeans(k, w.ck, init, w.iters)
    b = cabf.kmeans(k, w.ck, init, w.iters)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    for hd in range(w.heads):
        x = to_np(k[0, hd])
        cent = a["centroids"][0, hd].cpu().numpy().astype(np.float64)
        labels = a["labels"][0, hd].cpu().numpy()
        check_labels(x, cent, labels, f"converged head {hd}")
        check_permutation(labels, a["perm"][0, hd].cpu().numpy(), a["offsets"][0, hd].cpu().numpy(),
                          a["counts"][0, hd].cpu().numpy(), w.ck)
        ref = svg2.kmeans(x, init[0, hd].cpu().numpy(), w.iters)
        agree = float((ref["assign"] == labels).mean())
        say(f"head {hd}: labels equal to the fp64 oracle's {w.iters}-iteration run: {agree:.4f}")
        assert agree >= 0.99


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gather_scatter_rows_bitexact(dtype):
    n, heads, d = 1000, 3, 64
    seq = cabf.Seq(1, heads, d, n)
    x = torch.randn(1, heads, n, d, device=DEV).to(dtype)
    perm = torch.stack([torch.randperm(n, device=DEV) for _ in range(heads)])[None].to(torch.int32)
    rows = n + cabf.SEQ_PAD_ROWS
    xp = torch.full((1, heads, rows, d), 7.0, device=DEV).to(dtype)
    cabf.cabf_gather_rows(seq, x, perm, xp, rows)
    back = torch.empty_like(x)
    cabf.cabf_scatter_rows(seq, xp, rows, perm, back)
    torch.cuda.synchronize()
    for hd in range(heads):
        assert torch.equal(xp[0, hd, :n], x[0, hd, perm[0, hd].long()])
    assert torch.all(xp[:, :, n:] == 0)
    assert torch.equal(back, x)


def _clustered(w, seed):
    q, k, v = mixture(w.n, w.heads, w.head_dim, seed=seed, amplitude=w.amplitude,
                      components=w.components)
    kq = cabf.kmeans(q, w.cq, init_idx(w.n, w.cq, w.heads, seed + 1), w.iters)
    kk = cabf.kmeans(k, w.ck, init_idx(w.n, w.ck, w.heads, seed + 2), w.iters)
    return q, k, v, kq, kk


@pytest.mark.parametrize("top_p", [0.9, 0.5, 1.0])
def test_cluster_select_matches_oracle(top_p):
    w = SEMANTIC_WORKLOADS["svg2-tiny"]
    q, k, v, kq, kk = _clustered(w, seed=10)
    seq = cabf.Seq(1, w.heads, w.head_dim, w.n)
    scale = 1.0 / np.sqrt(w.head_dim)
    cnt = torch.empty(1, w.heads, w.cq, dtype=torch.int32, device=DEV)
    idx = torch.empty(1, w.heads, w.cq, w.ck, dtype=torch.int32, device=DEV)
    probs = torch.empty(1, w.heads, w.cq, w.ck, dtype=torch.float32, device=DEV)
    ws = cabf._ws(cabf._lib.cabf_cluster_select_workspace_bytes(
        cabf.ctypes.byref(seq.c()), w.cq, w.ck), DEV)
    cabf.cabf_cluster_select(seq, w.cq, w.ck, kq["centroids"], kk["centroids"], kk["counts"],
                             scale, top_p, cnt, idx, probs, ws)
    torch.cuda.synchronize()
    for hd in range(w.heads):
        p = svg2.centroid_probs(kq["centroids"][0, hd].cpu().numpy(), kk["centroids"][0, hd].cpu().numpy(),
                                kk["counts"][0, hd].cpu().numpy(), scale)
        got = probs[0, hd].cpu().numpy().astype(np.float64)
        nz = p > 1e-30
        rel = np.abs(got[nz] - p[nz]) / p[nz]
        assert rel.max() < 5e-5, rel.max()
        sel = svg2.top_p_select(p, top_p)
        compare_masks(cnt[0, hd], idx[0, hd], sel, 1.0 - top_p, label=f"top_p={top_p} head {hd}")


def test_cluster_attention_matches_oracle_and_empty_rows():
    w = SEMANTIC_WORKLOADS["svg2-tiny"]
    q, k, v, kq, kk = _clustered(w, seed=20)
    seq = cabf.Seq(1, w.heads, w.head_dim, w.n)
    scale = 1.0 / np.sqrt(w.head_dim)
    rows = w.n + cabf.SEQ_PAD_ROWS
    qp, kp, vp, op = (torch.empty(1, w.heads, rows, w.head_dim, dtype=torch.bfloat16, device=DEV)
                      for _ in range(4))
    cabf.cabf_gather_rows(seq, q, kq["perm"], qp, rows)
    cabf.cabf_gather_rows(seq, k, kk["perm"], kp, rows)
    cabf.cabf_gather_rows(seq, v, kk["perm"], vp, rows)
    # lists: a random subset of key clusters per query cluster, one row empty
    rng = np.random.default_rng(3)
    mask = rng.random((1, w.heads, w.cq, w.ck)) < 0.3
    mask[0, 0, 2] = False
    cnt_np, idx_np = oracle.mask_to_lists(mask)
    cnt, idx = torch.from_numpy(cnt_np).to(DEV), torch.from_numpy(idx_np).to(DEV)
    lse = torch.empty(1, w.heads, rows, dtype=torch.float32, device=DEV)
    ws = cabf._ws(cabf._lib.cabf_cluster_attention_workspace_bytes(
        cabf.ctypes.byref(seq.c()), w.cq, w.ck), DEV)
    cabf.cabf_cluster_attention(seq, w.cq, w.ck, qp, kp, vp, kq["offsets"], kk["offsets"], cnt, idx,
                                scale, op, lse, ws)
    torch.cuda.synchronize()
    for hd in range(w.heads):
        q_off = kq["offsets"][0, hd].cpu().numpy()
        k_off = kk["offsets"][0, hd].cpu().numpy()
        ref_o, ref_lse = svg2.cluster_attention(to_np(qp[0, hd, :w.n]), to_np(kp[0, hd, :w.n]),
                                                to_np(vp[0, hd, :w.n]), q_off, k_off,
                                                cnt_np[0, hd], idx_np[0, hd], scale)
        compare_attention(op[0, hd, :w.n], ref_o, True, lse[0, hd, :w.n], ref_lse,
                          label=f"cluster attention head {hd}")
    r0, r1 = kq["offsets"][0, 0, 2].item(), kq["offsets"][0, 0, 3].item()
    assert torch.all(op[0, 0, r0:r1] == 0) and torch.all(torch.isneginf(lse[0, 0, r0:r1]))


def test_layer_keep_all_is_dense_attention():
    """Sparse VideoGen2 summary, Methodology A: with every cluster pair kept,
    the permuted computation undone is dense attention."""
    w = SEMANTIC_WORKLOADS["svg2-tiny"]
    q, k, v = mixture(w.n, w.heads, w.head_dim, seed=30, amplitude=w.amplitude,
                      components=w.components)
    o = cabf.svg_layer(q, k, v, w.cq, w.ck, init_idx(w.n, w.cq, w.heads, 31),
                       init_idx(w.n, w.ck, w.heads, 32), w.iters, 1.0)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(w.head_dim)
    for hd in range(w.heads):
        ref = oracle.dense_attention(to_np(q[0, hd]), to_np(k[0, hd]), to_np(v[0, hd]), scale)
        compare_attention(o[0, hd], ref, True, label=f"keep-all head {hd}")


def test_layer_matches_oracle_on_the_gpu_clustering():
    """End to end at top-p 0.9: the GPU's selection and attention against the
    oracle's, both fed the GPU's k-means result (checked above)."""
    w = SEMANTIC_WORKLOADS["svg2-tiny"]
    q, k, v = mixture(w.n, w.heads, w.head_dim, seed=40, amplitude=w.amplitude,
                      components=w.components)
    o, info = cabf.svg_layer(q, k, v, w.cq, w.ck, init_idx(w.n, w.cq, w.heads, 41),
                             init_idx(w.n, w.ck, w.heads, 42), w.iters, w.top_p, return_info=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(w.head_dim)
    kq, kk = info["kq"], info["kk"]
    for hd in range(w.heads):
        p = svg2.centroid_probs(kq["centroids"][0, hd].cpu().numpy(), kk["centroids"][0, hd].cpu().numpy(),
                                kk["counts"][0, hd].cpu().numpy(), scale)
        sel = svg2.top_p_select(p, w.top_p)
        compare_masks(info["kv_count"][0, hd], info["kv_index"][0, hd], sel, 1.0 - w.top_p,
                      label=f"layer head {hd}")
        gmask = oracle.lists_to_mask(info["kv_count"][0, hd].cpu().numpy(),
                                     info["kv_index"][0, hd].cpu().numpy(), w.ck)
        same = ~(gmask != sel["mask"]).any(-1)
        perm_q = kq["perm"][0, hd].cpu().numpy()
        perm_k = kk["perm"][0, hd].cpu().numpy()
        q_off = kq["offsets"][0, hd].cpu().numpy()
        ref_op, _ = svg2.cluster_attention(to_np(q[0, hd])[perm_q], to_np(k[0, hd])[perm_k],
                                           to_np(v[0, hd])[perm_k], q_off,
                                           kk["offsets"][0, hd].cpu().numpy(), sel["kv_count"],
                                           sel["kv_index"], scale)
        ref_o = np.zeros_like(ref_op)
        ref_o[perm_q] = ref_op
        rows = np.zeros(w.n, dtype=bool)
        for a in np.nonzero(same)[0]:
            rows[perm_q[q_off[a]:q_off[a + 1]]] = True
        say(f"head {hd}: rows compared {int(rows.sum())} of {w.n}, density "
            f"{svg2.kept_density(dict(q_off=q_off, k_off=kk['offsets'][0, hd].cpu().numpy(), sel=sel)):.3f}")
        compare_attention(o[0, hd], ref_o, True, rows=np.nonzero(rows)[0], label=f"layer head {hd}")


def test_full_size_semantic_layer_sampled():
    """The Wan-14B 720p token count (75,600 tokens, 40 heads, 100 / 500
    clusters, 10 iterations, top-p 0.9) in the configuration the benchmark
    times. Head 0 is checked: k-means labels on a token sample, the whole
    selection, and the attention of sampled query clusters."""
    w = SEMANTIC_WORKLOADS["svg2-wan14b-720p"]
    say(f"full-size {w.name}")
    q, k, v = mixture(w.n, w.heads, w.head_dim, seed=50, amplitude=w.amplitude,
                      components=w.components)
    o, info = cabf.svg_layer(q, k, v, w.cq, w.ck, init_idx(w.n, w.cq, w.heads, 51),
                             init_idx(w.n, w.ck, w.heads, 52), w.iters, w.top_p, return_info=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(w.head_dim)
    kq, kk = info["kq"], info["kk"]
    hd = 0
    sample = np.random.default_rng(0).choice(w.n, 4000, replace=False)
    for name, x, km in (("Q", q, kq), ("K", k, kk)):
        xs = to_np(x[0, hd])[sample]
        cent = km["centroids"][0, hd].cpu().numpy().astype(np.float64)
        check_labels(xs, cent, km["labels"][0, hd].cpu().numpy()[sample], f"full-size {name} labels")
        check_permutation(km["labels"][0, hd].cpu().numpy(), km["perm"][0, hd].cpu().numpy(),
                          km["offsets"][0, hd].cpu().numpy(), km["counts"][0, hd].cpu().numpy(),
                          cent.shape[0])
    p = svg2.centroid_probs(kq["centroids"][0, hd].cpu().numpy(), kk["centroids"][0, hd].cpu().numpy(),
                            kk["counts"][0, hd].cpu().numpy(), scale)
    sel = svg2.top_p_select(p, w.top_p)
    compare_masks(info["kv_count"][0, hd], info["kv_index"][0, hd], sel, 1.0 - w.top_p,
                  label="full-size selection")
    q_off = kq["offsets"][0, hd].cpu().numpy()
    k_off = kk["offsets"][0, hd].cpu().numpy()
    say(f"kept density {svg2.kept_density(dict(q_off=q_off, k_off=k_off, sel=sel)):.4f}")
    cnt = info["kv_count"][0, hd].cpu().numpy()
    idx = info["kv_index"][0, hd].cpu().numpy()
    clusters = [0, w.cq // 2, w.cq - 1]
    n = w.n
    ref_op, ref_lse = svg2.cluster_attention(to_np(info["qp"][0, hd, :n]), to_np(info["kp"][0, hd, :n]),
                                             to_np(info["vp"][0, hd, :n]), q_off, k_off, cnt, idx,
                                             scale, clusters=clusters)
    rows = np.concatenate([np.arange(q_off[a], q_off[a + 1]) for a in clusters])
    compare_attention(info["op"][0, hd, :n], ref_op, True, info["lse"][0, hd, :n], ref_lse,
                      rows=rows, label="full-size cluster attention")
    perm_q = kq["perm"][0, hd].cpu().numpy()
    assert torch.equal(o[0, hd, torch.from_numpy(perm_q[rows]).to(DEV)],
                       info["op"][0, hd, torch.from_numpy(rows).to(DEV)])
    # every query row of every head, into outputs filled with NaN beforehand:
    # written once, bit for bit as in the layer (the pass runs in list order;
    # its work items are spread over the XCDs by head groups)
    seq = cabf.Seq(1, w.heads, w.head_dim, w.n)
    op2 = torch.full_like(info["op"], float("nan"))
    lse2 = torch.full_like(info["lse"], float("nan"))
    ws = cabf._ws(cabf._lib.cabf_cluster_attention_workspace_bytes(cabf.ctypes.byref(seq.c()), int(w.cq),
                                                                    int(w.ck)), DEV)
    cabf.cabf_cluster_attention(seq, w.cq, w.ck, info["qp"], info["kp"], info["vp"], kq["offsets"],
                                kk["offsets"], info["kv_count"], info["kv_index"], scale, op2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(op2[:, :, :n], info["op"][:, :, :n]), "rows left unwritten or different"
    assert torch.equal(lse2[:, :, :n], info["lse"][:, :, :n]), "lse rows left unwritten or different"
