"""Plain fp64 CPU oracle of the semantic-permutation top-p variant.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: Sparse VideoGen2 technical summary (gist.science, paper 2505.18875),
section 2 "Methodology":
  A "semantic-aware permutation": Q and K tokens are clustered by k-means,
    independently, into C_q and C_k groups, and each tensor is reordered so
    that the tokens of a cluster are contiguous; the permutations are undone
    on the output, so with every cluster pair kept the result is exactly
    dense attention;
  B "centroid-based top-p selection": attention scores are estimated between
    cluster centroids, key clusters are sorted by the estimate and taken until
    their cumulative score reaches p;
  C the attention kernel visits, for each query cluster, the key tokens of
    its selected clusters (variable-size blocks, dense contiguous queries).

Readings taken where the page is silent (each is also stated at its function):
  * k-means is Lloyd's algorithm on the raw feature vectors with squared
    Euclidean distance; assignment ties go to the lowest cluster index; an
    empty cluster keeps its previous centroid; the initial centroids are the
    feature vectors of given token indices (the random draw is an input).
    After the last update every token is assigned to its nearest final
    centroid, so labels and centroids are consistent.
  * the permutation is a stable sort by cluster id (tokens of a cluster keep
    their original order).
  * the score of key cluster b for query cluster a is the share of attention
    mass that the query centroid gives to the tokens of b when each of them
    is represented by the key centroid: p_ab proportional to
    |K_b| exp(scale <cq_a, ck_b>), normalised over b (empty clusters: 0).
  * top-p keeps the shortest prefix (p descending, ties to the lower index)
    whose mass reaches p: the NABLA CDF cut with thr = 1 - p.
"""
from __future__ import annotations

import numpy as np

from .nabla import cdf_cut_details


def kmeans_assign(x: np.ndarray, cent: np.ndarray):
    """Nearest centroid of every row of x ([n, d]) among cent ([C, d]).

    Squared Euclidean distance, ties to the lowest index (np.argmin returns
    the first minimum). Also returns the gap between the second-nearest and
    the nearest squared distance of every row (inf when C = 1), which tells
    how well-posed the assignment is.
    Pinned by: brute-force loops on small inputs, separated blobs.
    """
    x = np.asarray(x, dtype=np.float64)
    cent = np.asarray(cent, dtype=np.float64)
    n = x.shape[0]
    assign = np.zeros(n, dtype=np.int64)
    gap = np.full(n, np.inf)
    rows = max(1, (1 << 24) // max(1, cent.size))     # bound the [rows, C, d] temporary
    for r0 in range(0, n, rows):
        d2 = ((x[r0:r0 + rows, None, :] - cent[None, :, :]) ** 2).sum(-1)   # [rows, C]
        assign[r0:r0 + rows] = np.argmin(d2, axis=1)
        if cent.shape[0] > 1:
            part = np.partition(d2, 1, axis=1)
            gap[r0:r0 + rows] = part[:, 1] - part[:, 0]
    return assign, gap


def kmeans_update(x: np.ndarray, assign: np.ndarray, cent_prev: np.ndarray):
    """Lloyd update: each centroid becomes the mean of its members; an empty
    cluster keeps its previous centroid. Returns (cent [C, d], counts [C])."""
    x = np.asarray(x, dtype=np.float64)
    C = cent_prev.shape[0]
    counts = np.bincount(assign, minlength=C)
    cent = np.array(cent_prev, dtype=np.float64, copy=True)
    for c in range(C):
        if counts[c] > 0:
            cent[c] = x[assign == c].mean(axis=0)
    return cent, counts


def kmeans(x: np.ndarray, init_idx: np.ndarray, iters: int):
    """Lloyd's k-means on the rows of x ([n, d]) from the centroids
    x[init_idx], ``iters`` assign+update rounds, then a final assignment.

    Returns dict(cent [C, d], assign [n], counts [C], gap [n], inertia list
    (sum of squared distances to the assigned centroid before each update)).
    Pinned by: objective never increases, separated blobs are recovered,
    labels are the nearest final centroid, centroids are member means.
    """
    x = np.asarray(x, dtype=np.float64)
    cent = x[np.asarray(init_idx)].copy()
    inertia = []
    for _ in range(iters):
        assign, _ = kmeans_assign(x, cent)
        inertia.append(float(((x - cent[assign]) ** 2).sum()))
        cent, _ = kmeans_update(x, assign, cent)
    assign, gap = kmeans_assign(x, cent)
    counts = np.bincount(assign, minlength=cent.shape[0])
    return dict(cent=cent, assign=assign, counts=counts, gap=gap, inertia=inertia)


def cluster_permutation(assign: np.ndarray, C: int):
    """Stable sort of the tokens by cluster id.

    Returns (perm, offsets): perm[i] is the original token at permuted
    position i; the tokens of cluster c occupy positions offsets[c] ..
    offsets[c+1]-1 in their original order.
    """
    assign = np.asarray(assign)
    perm = np.argsort(assign, kind="stable")
    counts = np.bincount(assign, minlength=C)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return perm.astype(np.int64), offsets.astype(np.int64)


def centroid_probs(cq: np.ndarray, ck: np.ndarray, ck_counts: np.ndarray, scale: float):
    """Estimated attention share of every key cluster for every query cluster:
    p_ab = |K_b| exp(scale <cq_a, ck_b>) / sum_b' |K_b'| exp(scale <cq_a, ck_b'>).

    Pinned by: with singleton clusters it equals the token attention
    probabilities of the query centroid; duplicating a key token m times
    equals a count of m.
    """
    z = scale * (np.asarray(cq, dtype=np.float64) @ np.asarray(ck, dtype=np.float64).T)
    w = np.asarray(ck_counts, dtype=np.float64)[None, :]
    e = np.where(w > 0, w * np.exp(z - z.max(axis=1, keepdims=True)), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def top_p_select(p: np.ndarray, top_p: float):
    """Per query cluster, the key clusters kept by the cumulative-score rule.

    Returns dict(mask bool [Cq, Ck], kv_count, kv_index (ascending, tail -1),
    k, s_prev, s_k, p_k, p_next) with the cut quantities of cdf_cut_details
    (thr = 1 - top_p), for judging ill-posed rows.
    """
    Cq, Ck = p.shape
    thr = 1.0 - top_p
    mask = np.zeros((Cq, Ck), dtype=bool)
    k = np.zeros(Cq, dtype=np.int64)
    s_prev, s_k, p_k, p_next = (np.zeros(Cq) for _ in range(4))
    for a in range(Cq):
        kept, kk, sp, sk, pk, pn = cdf_cut_details(p[a], thr)
        mask[a, kept] = True
        k[a], s_prev[a], s_k[a], p_k[a], p_next[a] = kk, sp, sk, pk, pn
    kv_count = mask.sum(1).astype(np.int32)
    kv_index = np.full((Cq, Ck), -1, dtype=np.int32)
    for a in range(Cq):
        idx = np.nonzero(mask[a])[0]
        kv_index[a, : idx.size] = idx
    return dict(mask=mask, kv_count=kv_count, kv_index=kv_index, k=k, s_prev=s_prev, s_k=s_k,
                p_k=p_k, p_next=p_next, p=p, mode="cdf")


def cluster_attention(qp, kp, vp, q_off, k_off, kv_count, kv_index, scale: float, clusters=None):
    """Variable-size block-sparse attention in permuted order.

    Query cluster a (permuted rows q_off[a] .. q_off[a+1]-1) attends to the
    keys of its selected key clusters (rows k_off[b] .. k_off[b+1]-1 of the
    permuted K, V). Returns (op [n, d], lse [n]); rows of clusters not listed
    in ``clusters`` (default: all) are left at 0 / -inf.
    Pinned by: keeping every cluster pair gives dense attention once
    unpermuted; brute-force token masks on small inputs.
    """
    qp, kp, vp = (np.asarray(t, dtype=np.float64) for t in (qp, kp, vp))
    n, d = qp.shape
    op = np.zeros((n, vp.shape[1]))
    lse = np.full(n, -np.inf)
    Cq = len(q_off) - 1
    for a in range(Cq) if clusters is None else clusters:
        r0, r1 = int(q_off[a]), int(q_off[a + 1])
        if r1 == r0:
            continue
        keys = [np.arange(int(k_off[b]), int(k_off[b + 1])) for b in kv_index[a][: kv_count[a]]]
        keys = np.concatenate(keys) if keys else np.zeros(0, dtype=np.int64)
        if keys.size == 0:
            continue
        s = scale * (qp[r0:r1] @ kp[keys].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        op[r0:r1] = (e @ vp[keys]) / l
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return op, lse


def svg_layer(q, k, v, init_q, init_k, iters: int, scale: float, top_p: float):
    """One head, raster order in and out: k-means of Q and K, permutation,
    centroid scores, top-p, cluster attention, inverse permutation.
    q, k, v: [n, d]. Returns (o [n, d], info dict)."""
    kq = kmeans(q, init_q, iters)
    kk = kmeans(k, init_k, iters)
    Cq, Ck = len(init_q), len(init_k)
    perm_q, q_off = cluster_permutation(kq["assign"], Cq)
    perm_k, k_off = cluster_permutation(kk["assign"], Ck)
    p = centroid_probs(kq["cent"], kk["cent"], kk["counts"], scale)
    sel = top_p_select(p, top_p)
    op, lse = cluster_attention(np.asarray(q)[perm_q], np.asarray(k)[perm_k], np.asarray(v)[perm_k],
                                q_off, k_off, sel["kv_count"], sel["kv_index"], scale)
    o = np.zeros_like(op)
    o[perm_q] = op
    return o, dict(kq=kq, kk=kk, perm_q=perm_q, perm_k=perm_k, q_off=q_off, k_off=k_off, sel=sel,
                   op=op, lse=lse)


def kept_density(info) -> float:
    """Fraction of (query, key) token pairs the selection keeps: the sum over
    query clusters of |cluster| times the tokens of its kept key clusters,
    over all query tokens times all key tokens.
    Pinned by: keep-all = 1, a hand-counted selection (tests/test_oracle_svg2.py)."""
    q_sizes = np.diff(info["q_off"])
    k_sizes = np.diff(info["k_off"])
    sel = info["sel"]
    kept = sum(int(q_sizes[a]) * int(k_sizes[sel["mask"][a]].sum()) for a in range(len(q_sizes)))
    n = int(q_sizes.sum())
    return kept / float(n * int(k_sizes.sum()))


__all__ = ["kmeans_assign", "kmeans_update", "kmeans", "cluster_permutation", "centroid_probs",
           "top_p_select", "cluster_attention", "svg_layer", "kept_density"]
