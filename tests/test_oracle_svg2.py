"""Pins of the semantic-permutation oracle (oracle.svg2) against values and
properties fixed by the Sparse VideoGen2 summary and by the mathematics,
independently of the oracle's own formulas."""
import numpy as np
import pytest

import oracle
from oracle import svg2
from synth import gaussian_mixture_qk, kmeans_init_indices

RNG = np.random.default_rng(7)


# --- k-means ---------------------------------------------------------------------

def test_assign_and_update_hand_example():
    x = np.array([[0.0, 0.0], [1.0, 0.0], [5.0, 5.0], [6.0, 5.0], [0.0, 1.0]])
    cent = np.array([[0.0, 0.0], [6.0, 6.0]])
    a, gap = svg2.kmeans_assign(x, cent)
    assert a.tolist() == [0, 0, 1, 1, 0]
    # squared distances of x1 to (0,0) and (6,6): 1 and 25 + 36
    assert gap[1] == pytest.approx(61.0 - 1.0)
    new, counts = svg2.kmeans_update(x, a, cent)
    assert counts.tolist() == [3, 2]
    assert np.allclose(new, [[1.0 / 3.0, 1.0 / 3.0], [5.5, 5.0]])


def test_assignment_tie_goes_to_lowest_index_and_empty_cluster_keeps_centroid():
    x = np.array([[1.0, 0.0], [1.0, 0.0]])
    cent = np.array([[2.0, 0.0], [0.0, 0.0], [9.0, 9.0]])
    a, gap = svg2.kmeans_assign(x, cent)
    assert a.tolist() == [0, 0] and gap.tolist() == [0.0, 0.0]
    new, counts = svg2.kmeans_update(x, a, cent)
    assert counts.tolist() == [2, 0, 0]
    assert np.array_equal(new[1:], cent[1:])          # empty clusters keep their centroids
    assert np.array_equal(new[0], [1.0, 0.0])


def test_separated_blobs_are_recovered():
    centres = np.array([[0.0, 0.0, 0.0], [10.0, 0.0, 0.0], [0.0, 10.0, 0.0], [0.0, 0.0, 10.0]])
    member = RNG.integers(0, 4, 400)
    x = centres[member] + RNG.normal(0, 0.3, (400, 3))
    init = [int(np.nonzero(member == c)[0][0]) for c in range(4)]
    out = svg2.kmeans(x, init, 3)
    assert np.array_equal(out["assign"], member)
    for c in range(4):
        assert np.allclose(out["cent"][c], x[member == c].mean(axis=0))


def test_objective_never_increases_and_labels_are_nearest():
    x = RNG.standard_normal((300, 8))
    init = RNG.choice(300, 12, replace=False)
    out = svg2.kmeans(x, init, 8)
    inert = out["inertia"]
    assert all(b <= a + 1e-9 for a, b in zip(inert, inert[1:]))
    d2 = ((x[:, None] - out["cent"][None]) ** 2).sum(-1)
    assert np.all(d2[np.arange(300), out["assign"]] <= d2.min(axis=1) + 1e-12)


def test_kmeans_matches_library_lloyd():
    """Lloyd's algorithm as a library implements it (scikit-learn, lloyd, one
    run from the same initial centroids, the same number of rounds, final
    labels re-assigned to the final centroids): same labels, same centroids,
    on data where no cluster empties (the library relocates empty clusters,
    the oracle keeps their centroid)."""
    sk = pytest.importorskip("sklearn.cluster")
    q, _ = gaussian_mixture_qk(600, 1, 16, components=6, spread=0.6, amplitude=3.0, seed=2,
                               dtype="f32")
    x = q[0, 0].numpy().astype(np.float64)
    init = kmeans_init_indices(600, 9, 1, seed=3)[0]
    for iters in (1, 4, 9):
        out = svg2.kmeans(x, init, iters)
        assert out["counts"].min() > 0
        km = sk.KMeans(n_clusters=9, init=x[init], n_init=1, max_iter=iters, tol=0.0,
                       algorithm="lloyd").fit(x)
        assert np.array_equal(km.labels_, out["assign"]), iters
        assert np.allclose(km.cluster_centers_, out["cent"], rtol=0, atol=1e-9), iters


# --- permutation -----------------------------------------------------------------

def test_stable_permutation_hand_example():
    perm, off = svg2.cluster_permutation(np.array([2, 0, 2, 1, 0]), 4)
    assert perm.tolist() == [1, 4, 3, 0, 2]
    assert off.tolist() == [0, 2, 3, 5, 5]


# --- centroid scores ---------------------------------------------------------------

def test_singleton_clusters_give_token_attention_weights():
    """One token per cluster: the estimate is the exact attention distribution
    of the query (taken here as the output of dense attention with one-hot
    values)."""
    q = RNG.standard_normal((3, 6))
    k = RNG.standard_normal((9, 6))
    p = svg2.centroid_probs(q, k, np.ones(9), 0.7)
    w = oracle.dense_attention(q, k, np.eye(9), 0.7)
    assert np.allclose(p, w, atol=1e-13)


def test_cluster_count_weights_like_duplicated_keys():
    q = RNG.standard_normal((2, 5))
    k = RNG.standard_normal((4, 5))
    counts = np.array([3, 1, 0, 2])
    p = svg2.centroid_probs(q, k, counts, 0.9)
    dup = np.repeat(k, counts, axis=0)               # key b repeated counts[b] times
    w = oracle.dense_attention(q, dup, np.eye(dup.shape[0]), 0.9)
    owner = np.repeat(np.arange(4), counts)
    merged = np.stack([w[:, owner == b].sum(1) for b in range(4)], axis=1)
    assert np.allclose(p, merged, atol=1e-13)
    assert np.all(p[:, 2] == 0)


def test_top_p_keeps_shortest_prefix_reaching_p():
    for trial in range(50):
        p = RNG.dirichlet(np.full(40, 0.3), size=5)
        top = float(RNG.uniform(0.3, 0.99))
        sel = svg2.top_p_select(p, top)
        for a in range(5):
            kept = sel["kv_index"][a][: sel["kv_count"][a]]
            assert p[a, kept].sum() >= top - 1e-12
            order = np.sort(p[a])[::-1]
            assert np.cumsum(order)[len(kept) - 2] < top if len(kept) > 1 else True


# --- attention ---------------------------------------------------------------------

def _layer_inputs(n=300, d=16, seed=1):
    q, k = gaussian_mixture_qk(n, 1, d, components=6, spread=0.3, amplitude=2.0, seed=seed,
                               dtype="f32")
    q, k = q[0, 0].numpy().astype(np.float64), k[0, 0].numpy().astype(np.float64)
    v = RNG.standard_normal((n, d))
    iq = kmeans_init_indices(n, 7, 1, seed=seed)[0]
    ik = kmeans_init_indices(n, 11, 1, seed=seed + 1)[0]
    return q, k, v, iq, ik


def test_keeping_every_cluster_is_dense_attention():
    """The summary's equivalence: with every cluster pair kept, permuting,
    attending and un-permuting gives dense attention."""
    q, k, v, iq, ik = _layer_inputs()
    o, info = svg2.svg_layer(q, k, v, iq, ik, 4, 0.25, 1.0)
    assert info["sel"]["mask"].all()
    assert np.allclose(o, oracle.dense_attention(q, k, v, 0.25), atol=1e-12)


def test_cluster_attention_matches_token_mask_bruteforce():
    q, k, v, iq, ik = _layer_inputs(n=120, seed=3)
    o, info = svg2.svg_layer(q, k, v, iq, ik, 3, 0.5, 0.7)
    assert not info["sel"]["mask"].all()
    lab_q, lab_k = info["kq"]["assign"], info["kk"]["assign"]
    for n in range(0, 120, 7):
        keys = info["sel"]["mask"][lab_q[n]][lab_k]           # token mask of row n
        want = oracle.dense_attention(q[n:n + 1], k, v, 0.5, key_valid=keys)
        assert np.allclose(o[n], want[0], atol=1e-12)


def test_mixture_generator_has_recoverable_clusters():
    q, _ = gaussian_mixture_qk(2000, 1, 32, components=8, spread=0.2, amplitude=3.0, seed=5,
                               dtype="f32")
    x = q[0, 0].numpy().astype(np.float64)
    init = kmeans_init_indices(2000, 8, 1, seed=5)[0]
    out = svg2.kmeans(x, init, 10)
    sizes = np.sort(out["counts"])
    assert sizes[0] > 100          # no component lost: every cluster holds a real group


def test_kept_density_counts_token_pairs():
    """Hand-counted: query clusters of 2 and 3 tokens, key clusters of 1, 3
    and 2 tokens; the first query cluster keeps key clusters 0 and 2 (2 x 3
    pairs), the second keeps cluster 1 (3 x 3 pairs): 15 of 5 x 6 pairs."""
    q_off = np.array([0, 2, 5])
    k_off = np.array([0, 1, 4, 6])
    mask = np.array([[True, False, True], [False, True, False]])
    assert svg2.kept_density(dict(q_off=q_off, k_off=k_off, sel=dict(mask=mask))) == 0.5
    every = np.ones((2, 3), dtype=bool)
    assert svg2.kept_density(dict(q_off=q_off, k_off=k_off, sel=dict(mask=every))) == 1.0
