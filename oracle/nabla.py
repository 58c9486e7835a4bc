"""Plain fp64 CPU oracle of NABLA block-sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.

Source: NABLA technical summary, gist.science paper 2507.13546,
"Methodology":
  item 1 "token reordering (fractal flattening)";
  item 2 "adaptive mask construction" (down-sampling by block mean pooling,
         reduced attention, per-row CDF threshold, expansion to token
         resolution);
  item 3 "hybrid integration with STA" (M = M_nabla OR M_STA).
Where that page is silent the reading taken is stated at the function.

Every function here is written for clarity, not speed: a library primitive
(matmul, sort, cumulative sum, exp) may serve as one step, nothing is blocked,
fused or reordered. Arrays use the layout [..., tokens, d] with any number of
leading (batch, head) axes.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

BLOCK_E1_WINDOW = 1e-4   # cut within this mass of 1-thr: the row's set is ill-posed
BLOCK_E2_RATIO = 1e-6    # p_(k) and p_(k+1) this close (relative): the set is ill-posed


class Grid:
    """Latent video grid of T frames x H rows x W columns, patch side P.

    The NABLA page (Methodology item 1) groups the tokens of each P x P spatial
    patch into a contiguous run while keeping time order; each such patch of
    one frame is one attention block (Methodology item 2 says "N x N blocks";
    read as one P x P patch = P*P tokens). H and W are padded up to multiples
    of P with pad tokens that are never keys.
    """

    def __init__(self, T: int, H: int, W: int, P: int):
        if min(T, H, W, P) < 1:
            raise ValueError("grid sizes must be positive")
        self.T, self.H, self.W, self.P = int(T), int(H), int(W), int(P)
        self.Ty = -(-self.H // self.P)          # patch rows per frame
        self.Tx = -(-self.W // self.P)          # patch columns per frame
        self.Hp = self.Ty * self.P
        self.Wp = self.Tx * self.P
        self.block = self.P * self.P            # tokens per block
        self.nb = self.T * self.Ty * self.Tx    # blocks
        self.N = self.nb * self.block           # tokens incl. pads
        self.n_valid = self.T * self.H * self.W

    def __repr__(self):
        return f"Grid(T={self.T}, H={self.H}, W={self.W}, P={self.P})"


# ----------------------------------------------------------------------------
# Methodology item 1: fractal flattening
# ----------------------------------------------------------------------------

def fractal_positions(g: Grid) -> np.ndarray:
    """Position in the reordered sequence of every raster token (t, y, x).

    Reading of Methodology item 1: frames stay outermost in time order; inside
    a frame the P x P patches follow in raster order (patch row, patch column);
    inside a patch the tokens follow in raster order. Returns int64 [T*H*W]
    indexed by the raster index (t*H + y)*W + x.
    Pinned by: hand-derived spot indices (tests/golden/fractal_positions.json),
    bijection and round-trip tests.
    """
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.H), np.arange(g.W), indexing="ij")
    patch = (t * g.Ty + y // g.P) * g.Tx + x // g.P
    inside = (y % g.P) * g.P + (x % g.P)
    return (patch * g.block + inside).reshape(-1).astype(np.int64)


def valid_slots(g: Grid) -> np.ndarray:
    """bool [N]: True at reordered positions that hold a real token."""
    valid = np.zeros(g.N, dtype=bool)
    valid[fractal_positions(g)] = True
    return valid


def block_coords(g: Grid):
    """(t, ty, tx) of every block index b in reordered order: b = (t*Ty+ty)*Tx+tx."""
    b = np.arange(g.nb)
    return b // (g.Ty * g.Tx), (b // g.Tx) % g.Ty, b % g.Tx


def permute(x: np.ndarray, g: Grid) -> np.ndarray:
    """Raster [..., T*H*W, d] -> reordered [..., N, d]; pad slots are zero.

    Pinned by: unpermute(permute(x)) == x bitwise, pads exactly zero.
    """
    if x.shape[-2] != g.n_valid:
        raise ValueError(f"expected {g.n_valid} raster tokens, got {x.shape[-2]}")
    out = np.zeros(x.shape[:-2] + (g.N, x.shape[-1]), dtype=x.dtype)
    out[..., fractal_positions(g), :] = x
    return out


def unpermute(xp: np.ndarray, g: Grid) -> np.ndarray:
    """Reordered [..., N, d] -> raster [..., T*H*W, d] (real tokens only).

    Sparse VideoGen2 summary, section 2A ("mathematical equivalence"): undoing
    the permutation restores the original token order of the output.
    """
    if xp.shape[-2] != g.N:
        raise ValueError(f"expected {g.N} reordered tokens, got {xp.shape[-2]}")
    return xp[..., fractal_positions(g), :]


# ----------------------------------------------------------------------------
# Methodology item 2: adaptive mask construction
# ----------------------------------------------------------------------------

def pool_blocks(xp: np.ndarray, g: Grid, precision=np.float64) -> np.ndarray:
    """Block mean-pooling ("down-sampling" bullet of Methodology item 2).

    [..., N, d] -> [..., nb, d]: the mean over the real tokens of each block.
    Reading: pad tokens are left out of the mean (a block always holds at
    least one real token because H and W are padded by less than P).
    ``precision`` is float64 for the definition; float32 evaluates the same
    steps in single precision.
    Pinned by: constant input, affine ramp (mean = ramp at the centre of the
    real part of the patch).
    """
    xs = xp.astype(precision).reshape(xp.shape[:-2] + (g.nb, g.block, xp.shape[-1]))
    valid = valid_slots(g).reshape(g.nb, g.block)
    count = valid.sum(axis=1).astype(precision)            # [nb]
    masked = np.where(valid[:, :, None], xs, precision(0))
    return (masked.sum(axis=-2) / count[:, None]).astype(precision)


def block_logits(qb: np.ndarray, kb: np.ndarray, scale: float, precision=np.float64) -> np.ndarray:
    """Reduced attention logits z_ij = scale * <Qb_i, Kb_j> ("reduced attention" bullet).

    Reading: the same softmax scale as the token attention (an argument).
    Pinned by: hand-computed asymmetric example (tests/golden/block_cut_cases.json).
    """
    qb = qb.astype(precision)
    kb = kb.astype(precision)
    return (precision(scale) * (qb @ np.swapaxes(kb, -1, -2))).astype(precision)


def block_probs(z: np.ndarray, precision=np.float64) -> np.ndarray:
    """Row softmax of the reduced attention map ("full attention map" on pooled blocks)."""
    z = z.astype(precision)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(precision)


def _descending_order(p_row: np.ndarray) -> np.ndarray:
    """Block indices ordered by probability descending, ties by index ascending."""
    idx = np.arange(p_row.shape[0])
    return np.lexsort((idx, -p_row))


def cdf_cut_details(p_row: np.ndarray, thr: float):
    """Per-row CDF threshold ("CDF thresholding" bullet), with the quantities
    used to judge how well-posed the cut is.

    Reading (the bullet's wording is garbled): order the blocks by probability
    descending (ties: lower index first), form prefix sums S_m, keep the
    shortest prefix whose mass reaches 1 - thr, i.e. k = min{m >= 1 : S_m >=
    1 - thr}. thr <= 0 keeps every block (so thr = 0 is dense attention even
    when rounding keeps S_n below 1); if rounding keeps S_n < 1 - thr the row
    keeps all blocks.

    Returns (kept_indices, k, S_{k-1}, S_k, p_(k), p_(k+1)) with S_0 = 0 and
    p_(n+1) = 0. The prefix sums are formed in the array's own precision.
    Pinned by: uniform rows (k = ceil((1-thr) n), lowest indices), one-hot
    rows (k = 1), hand-computed rows, brute-force subset search for n <= 10.
    """
    p_row = np.asarray(p_row)
    n = p_row.shape[0]
    order = _descending_order(p_row)
    ps = p_row[order]
    S = np.cumsum(ps)
    if thr <= 0:
        k = n
    else:
        target = p_row.dtype.type(1.0) - p_row.dtype.type(thr)
        hit = np.nonzero(S >= target)[0]
        k = int(hit[0]) + 1 if hit.size else n
    s_prev = float(S[k - 2]) if k >= 2 else 0.0
    s_k = float(S[k - 1])
    p_k = float(ps[k - 1])
    p_next = float(ps[k]) if k < n else 0.0
    return np.sort(order[:k]), k, s_prev, s_k, p_k, p_next


def cdf_cut(p_row: np.ndarray, thr: float) -> np.ndarray:
    """Kept block indices (ascending) of one row; see ``cdf_cut_details``."""
    return cdf_cut_details(p_row, thr)[0]


def topk_cut_details(p_row: np.ndarray, k: int):
    """Fixed-budget selection of one row: the k most probable blocks.

    Source: DynamicRad summary, "Dual-Mode Strategy", Static-Ratio mode: a
    fixed ratio of the candidates is kept, for throughput. The page gives
    neither the candidate set nor the ranking; the reading taken here keeps a
    fixed count k = ceil(ratio * nb) per row, ranked by the same block
    probabilities as the CDF cut (descending, ties: lower index first). k >= n
    keeps every block.

    Returns (kept_indices, k_eff, p_(k), p_(k+1)) with p_(n+1) = 0.
    Pinned by: uniform rows (the k lowest indices), k = 1 equals argmax,
    brute-force maximum-mass subsets for n <= 10, invariants.
    """
    p_row = np.asarray(p_row)
    n = p_row.shape[0]
    kk = max(1, min(int(k), n))
    order = _descending_order(p_row)
    ps = p_row[order]
    p_k = float(ps[kk - 1])
    p_next = float(ps[kk]) if kk < n else 0.0
    return np.sort(order[:kk]), kk, p_k, p_next


def topk_cut(p_row: np.ndarray, k: int) -> np.ndarray:
    """Kept block indices (ascending) of one row; see ``topk_cut_details``."""
    return topk_cut_details(p_row, k)[0]


# ----------------------------------------------------------------------------
# Methodology item 3: union with Sliding Tile Attention
# ----------------------------------------------------------------------------

def sta_mask(g: Grid, dt: int, dy: int, dx: int) -> np.ndarray:
    """Static sliding-tile window at block granularity, bool [nb, nb].

    Reading (the page gives no window shape): query block (t, ty, tx) sees
    every key block with |dt'| <= dt frames, |dty| <= dy patch rows and
    |dtx| <= dx patch columns, clipped at the grid edges (not shifted).
    Pinned by: closed-form window counts per block.
    """
    t, ty, tx = block_coords(g)
    return ((np.abs(t[:, None] - t[None, :]) <= dt)
            & (np.abs(ty[:, None] - ty[None, :]) <= dy)
            & (np.abs(tx[:, None] - tx[None, :]) <= dx))


def lists_to_mask(kv_count: np.ndarray, kv_index: np.ndarray, nb: int) -> np.ndarray:
    """Per-row block lists -> bool mask [..., nb, nb] (entries past the count ignored)."""
    lead = kv_count.shape
    mask = np.zeros(lead + (nb,), dtype=bool)
    for pos in np.ndindex(*lead):
        c = int(kv_count[pos])
        mask[pos][kv_index[pos][:c]] = True
    return mask


def mask_to_lists(mask: np.ndarray):
    """bool mask [..., nb, nb] -> (kv_count int32 [..., nb], kv_index int32 [..., nb, nb]).

    Lists are ascending; unused tail entries are -1.
    """
    nb = mask.shape[-1]
    kv_count = mask.sum(axis=-1).astype(np.int32)
    kv_index = np.full(mask.shape, -1, dtype=np.int32)
    for pos in np.ndindex(*mask.shape[:-1]):
        idx = np.nonzero(mask[pos])[0]
        kv_index[pos][: idx.size] = idx
    assert kv_index.shape[-1] == nb
    return kv_count, kv_index


def build_block_mask(qp, kp, g: Grid, scale: float, thr: float, sta=None, precision=np.float64,
                     topk=None):
    """Methodology items 2-3: pooled block attention -> CDF cut -> OR STA window.

    qp, kp: reordered [..., N, d]. sta: None or (dt, dy, dx). With ``topk`` set,
    the CDF cut is replaced by the fixed-budget selection of ``topk_cut_details``
    (thr is then unused).
    Returns a dict with
      mask       bool [..., nb, nb]  final kept blocks (M = M_nabla OR M_STA)
      adaptive   bool [..., nb, nb]  the CDF (or top-k) part alone
      window     bool [nb, nb]       the sliding-tile window (all False without one)
      p          [..., nb, nb]       block probabilities
      k, s_prev, s_k, p_k, p_next    per-row cut quantities (see cdf_cut_details;
                                     s_prev and s_k are NaN for top-k)
      kv_count, kv_index             ascending per-row lists of ``mask``
      mode                           "cdf" or "topk"
    The selection runs over all blocks; the window is OR-ed in afterwards.
    """
    qb = pool_blocks(qp, g, precision)
    kb = pool_blocks(kp, g, precision)
    p = block_probs(block_logits(qb, kb, scale, precision), precision)
    lead = p.shape[:-2]
    adaptive = np.zeros(p.shape, dtype=bool)
    k = np.zeros(lead + (g.nb,), dtype=np.int64)
    s_prev = np.zeros(lead + (g.nb,))
    s_k = np.zeros(lead + (g.nb,))
    p_k = np.zeros(lead + (g.nb,))
    p_next = np.zeros(lead + (g.nb,))
    for pos in np.ndindex(*lead):
        for i in range(g.nb):
            if topk is None:
                kept, kk, a, b, c, d = cdf_cut_details(p[pos][i], thr)
            else:
                kept, kk, c, d = topk_cut_details(p[pos][i], topk)
                a = b = math.nan
            adaptive[pos][i][kept] = True
            k[pos][i], s_prev[pos][i], s_k[pos][i], p_k[pos][i], p_next[pos][i] = kk, a, b, c, d
    window = sta_mask(g, *sta) if sta is not None else np.zeros((g.nb, g.nb), dtype=bool)
    mask = adaptive | window
    kv_count, kv_index = mask_to_lists(mask)
    return dict(mask=mask, adaptive=adaptive, window=window, p=p, k=k, s_prev=s_prev, s_k=s_k,
                p_k=p_k, p_next=p_next, kv_count=kv_count, kv_index=kv_index,
                mode="cdf" if topk is None else "topk")


def sta_only_lists(g: Grid, dt: int, dy: int, dx: int):
    """The pure sliding-tile configuration (NABLA summary, comparison with
    static methods: an STA-only mask): every row keeps exactly its window.
    Returns (kv_count int32 [nb], kv_index int32 [nb, nb]), ascending lists."""
    return mask_to_lists(sta_mask(g, dt, dy, dx))


def exempt_rows(info: dict, thr: float, e1: float = BLOCK_E1_WINDOW, e2: float = BLOCK_E2_RATIO):
    """Rows whose kept set is numerically ill-posed, from fp64 cut quantities.

    E1: the cut lies within ``e1`` of the threshold, |S_{k-1} - (1-thr)| <= e1
        or |S_k - (1-thr)| <= e1 (rounding can move the cut by one block).
    E2: the k-th and (k+1)-th probabilities differ by at most e2 * p_(k)
        (rounding can swap which of the two is kept).
    thr <= 0 rows are never exempt (every block is kept by definition). For a
    top-k selection (info["mode"] == "topk") only E2 applies: the count is fixed.
    Returns (e1_rows, e2_rows) as bool arrays over the rows.
    """
    if info.get("mode") == "topk":
        r2 = (info["p_k"] - info["p_next"]) <= e2 * info["p_k"]
        return np.zeros(info["k"].shape, dtype=bool), r2
    if thr <= 0:
        z = np.zeros(info["k"].shape, dtype=bool)
        return z, z.copy()
    target = 1.0 - thr
    r1 = (np.abs(info["s_prev"] - target) <= e1) | (np.abs(info["s_k"] - target) <= e1)
    r2 = (info["p_k"] - info["p_next"]) <= e2 * info["p_k"]
    return r1, r2


# ----------------------------------------------------------------------------
# Methodology item 2, "expansion": attention over the kept tiles
# ----------------------------------------------------------------------------

def bsa_forward(qp, kp, vp, kv_count, kv_index, g: Grid, scale: float):
    """Softmax attention of every reordered query row over the real keys of its
    block's kept key blocks (the binary block mask expanded to token level).

    For a row n in block i with key set K(i) = {m : block(m) in list(i), m real}:
      o_n = sum_{m in K(i)} exp(s q_n.k_m) v_m / sum_{m in K(i)} exp(s q_n.k_m)
      lse_n = ln sum_{m in K(i)} exp(s q_n.k_m)
    Pad query rows are computed like the others. A row with no keys gets o = 0
    and lse = -inf. Returns (op [..., N, d] float64, lse [..., N] float64).
    Pinned by: thr = 0 equals dense attention (textbook + torch fp64 SDPA),
    token-level brute force, constant V, pad-slot invariance.
    """
    qp = np.asarray(qp, dtype=np.float64)
    kp = np.asarray(kp, dtype=np.float64)
    vp = np.asarray(vp, dtype=np.float64)
    valid = valid_slots(g)
    lead = qp.shape[:-2]
    d = qp.shape[-1]
    op = np.zeros(lead + (g.N, vp.shape[-1]))
    lse = np.full(lead + (g.N,), -np.inf)
    B = g.block
    for pos in np.ndindex(*lead):
        for i in range(g.nb):
            blocks = np.asarray(kv_index[pos][i][: int(kv_count[pos][i])], dtype=np.int64)
            keys = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1)
            keys = keys[valid[keys]]
            if keys.size == 0:
                continue
            q = qp[pos][i * B:(i + 1) * B]                      # [B, d]
            s = scale * (q @ kp[pos][keys].T)                   # [B, m]
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            l = e.sum(axis=1, keepdims=True)
            op[pos][i * B:(i + 1) * B] = (e @ vp[pos][keys]) / l
            lse[pos][i * B:(i + 1) * B] = (mx + np.log(l))[:, 0]
    assert d == kp.shape[-1]
    return op, lse


def bsa_backward(qp, kp, vp, dop, kv_count, kv_index, g: Grid, scale: float):
    """Gradients of the block-sparse attention (NABLA summary, closing remarks:
    the method accelerates training as well as inference, so the sparse
    attention needs its backward pass).

    With L a scalar loss of the real output rows and dop = dL/dop (pad query
    rows, which the layer discards, do not enter the function): for a real row
    n of block i with key set K(i) (as in ``bsa_forward``),
      P_nm = exp(s q_n.k_m) / sum_{m' in K(i)} exp(s q_n.k_m')
      dv_m += P_nm do_n
      dP_nm = do_n . v_m,  D_n = sum_m P_nm dP_nm,  dS_nm = P_nm (dP_nm - D_n)
      dq_n = s sum_m dS_nm k_m,  dk_m += s dS_nm q_n
    Returns (dq, dk, dv) [..., N, d] float64 with zero pad rows.
    Pinned by: central finite differences of ``bsa_forward``, and torch
    autograd through a token-masked dense attention.
    """
    qp, kp, vp, dop = (np.asarray(t, dtype=np.float64) for t in (qp, kp, vp, dop))
    valid = valid_slots(g)
    lead = qp.shape[:-2]
    dq, dk, dv = np.zeros_like(qp), np.zeros_like(kp), np.zeros_like(vp)
    B = g.block
    for pos in np.ndindex(*lead):
        for i in range(g.nb):
            blocks = np.asarray(kv_index[pos][i][: int(kv_count[pos][i])], dtype=np.int64)
            keys = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1)
            keys = keys[valid[keys]]
            rows = np.arange(i * B, (i + 1) * B)
            rows = rows[valid[rows]]
            if keys.size == 0 or rows.size == 0:
                continue
            q, do = qp[pos][rows], dop[pos][rows]
            k, v = kp[pos][keys], vp[pos][keys]
            s = scale * (q @ k.T)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            dP = do @ v.T
            D = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[pos][rows] += scale * (dS @ k)
            dk[pos][keys] += scale * (dS.T @ q)
            dv[pos][keys] += P.T @ do
    return dq, dk, dv


def dense_attention(q, k, v, scale: float, key_valid=None):
    """Textbook softmax(scale q k^T) v over the token axis, fp64; optional key mask."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if key_valid is not None:
        s = np.where(key_valid, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return (e @ v) / e.sum(axis=-1, keepdims=True)


def masked_attention_bruteforce(qp, kp, vp, g: Grid, block_mask, scale: float):
    """Token-by-token masked attention for tiny inputs (pure Python loops).

    Token mask M[n, m] = block_mask[block(n), block(m)] and m is a real token.
    qp/kp/vp: [N, d] (one head). Returns [N, d] float64.
    """
    valid = valid_slots(g)
    N = g.N
    out = np.zeros((N, vp.shape[-1]))
    for n in range(N):
        bn = n // g.block
        logits = []
        for m in range(N):
            if block_mask[bn, m // g.block] and valid[m]:
                dot = 0.0
                for c in range(qp.shape[-1]):
                    dot += float(qp[n, c]) * float(kp[m, c])
                logits.append((scale * dot, m))
        if not logits:
            continue
        mx = max(z for z, _ in logits)
        den = 0.0
        acc = [0.0] * vp.shape[-1]
        for z, m in logits:
            w = math.exp(z - mx)
            den += w
            for c in range(vp.shape[-1]):
                acc[c] += w * float(vp[m, c])
        out[n] = np.array(acc) / den
    return out


def layer(q, k, v, g: Grid, scale: float, thr: float, sta=None):
    """One attention layer: reorder, build the mask, attend, restore raster order.

    q, k, v: raster [..., T*H*W, d]. Returns (o raster [..., T*H*W, d], mask info).
    """
    qp, kp, vp = permute(q, g), permute(k, g), permute(v, g)
    info = build_block_mask(qp, kp, g, scale, thr, sta)
    op, _ = bsa_forward(qp, kp, vp, info["kv_count"], info["kv_index"], g, scale)
    return unpermute(op, g), info


def brute_force_topk(p_row, k: int):
    """Exhaustive reference for the top-k selection on small rows (n <= ~12):
    the size-k subset of largest mass, ties broken by the lexicographically
    smallest sorted index tuple. Returns ascending indices."""
    p_row = np.asarray(p_row, dtype=np.float64)
    n = p_row.shape[0]
    k = max(1, min(int(k), n))
    best = None
    for comb in itertools.combinations(range(n), k):
        mass = float(sum(p_row[list(comb)]))
        if best is None or mass > best[0]:
            best = (mass, comb)
    return np.array(best[1])


def brute_force_cut(p_row, thr: float):
    """Exhaustive reference for the CDF cut on small rows (n <= ~12).

    Among all subsets whose mass reaches 1 - thr, take those of smallest size;
    among them the one of largest mass; ties in mass broken by preferring the
    lexicographically smallest sorted index tuple. Returns ascending indices.
    Used only to pin ``cdf_cut`` on small rows with distinct probabilities.
    """
    p_row = np.asarray(p_row, dtype=np.float64)
    n = p_row.shape[0]
    if thr <= 0:
        return np.arange(n)
    target = 1.0 - thr
    for size in range(1, n + 1):
        best = None
        for comb in itertools.combinations(range(n), size):
            mass = float(sum(p_row[list(comb)]))
            if mass >= target and (best is None or mass > best[0]):
                best = (mass, comb)
        if best is not None:
            return np.array(best[1])
    return np.arange(n)
