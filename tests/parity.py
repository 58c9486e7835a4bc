"""Shared helpers of the GPU parity tests: comparisons with the CPU oracle.
The oracle computes every expected value; the checks here only judge the GPU's
results against it (and, where several results are correct, judge validity)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3   # attention output, bf16 inputs
F32_MAX_ABS = 1e-4                         # attention output, fp32 inputs
LSE_ABS = 1e-4


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_lists_wellformed(cnt: np.ndarray, idx: np.ndarray, nb: int):
    assert cnt.min() >= 1 and cnt.max() <= nb
    for pos in np.ndindex(*cnt.shape):
        row = idx[pos][: cnt[pos]]
        assert row.min() >= 0 and row.max() < nb, pos
        assert np.all(np.diff(row) > 0), pos


TIE_REL = 1e-6    # probabilities this close (relative) may be ordered either way
MASS_TOL = 1e-6   # a kept prefix may reach 1 - thr only within this much (fp64 mass)


def valid_cut(kept: np.ndarray, p: np.ndarray, window: np.ndarray, k_oracle: int, thr: float,
              mode: str) -> bool:
    """Whether ``kept`` (bool [nb]) is a correct selection for one row whose
    fp64 block probabilities are ``p`` (NABLA summary, Methodology item 2,
    CDF bullet, with the window of item 3 OR-ed in):

    kept = T OR window, where T holds the k' most probable blocks for some k'
    within one of the oracle's k (top-k: k' = k). Blocks whose probabilities
    lie within TIE_REL of the k'-th may be exchanged with one another; every
    block clearly above it must be kept, no block clearly below it may be.
    For the CDF cut the first k' blocks must reach 1 - thr (less MASS_TOL) and
    the first k' - 1 must not pass it by MASS_TOL: a longer or shorter cut is
    only correct where rounding could have put the row's mass on either side.
    """
    n = p.size
    order = np.lexsort((np.arange(n), -p))
    ps = p[order]
    S = np.cumsum(ps)
    target = 1.0 - thr
    if (window & ~kept).any():
        return False
    free = kept & ~window          # kept blocks that only the adaptive part explains
    if mode == "topk" or thr <= 0:
        cands = [k_oracle]
    else:
        cands = [kk for kk in (k_oracle - 1, k_oracle, k_oracle + 1) if 1 <= kk <= n]
    for kk in cands:
        if mode != "topk" and thr > 0:
            if S[kk - 1] < target - MASS_TOL and kk < n:
                continue
            if kk >= 2 and S[kk - 2] >= target + MASS_TOL:
                continue
        tau = ps[kk - 1]
        must = p > tau * (1.0 + TIE_REL)
        may = p >= tau * (1.0 - TIE_REL)
        if (must & ~kept).any() or (free & ~may).any():
            continue
        if int((must | free).sum()) <= kk <= int((kept & may).sum()):
            return True
    return False


def compare_masks(cnt_gpu, idx_gpu, info, thr, label=""):
    """Kept-block lists must agree except on rows whose cut is ill-posed, and
    every row that differs must still be a correct cut (``valid_cut``).

    Counts (reported, then asserted):
      mismatched              rows whose set differs from the oracle's
      not_exempt              ... outside the 1e-4 window E1 and the near-tie rule E2 (must be 0)
      mismatched_outside_1e6  ... outside a 1e-6 window and E2 (must be 0)
      invalid                 ... that are not a correct cut of the fp64 row (must be 0)
    Returns the dict of counts."""
    nb = info["mask"].shape[-1]
    cnt = cnt_gpu.cpu().numpy()
    idx = idx_gpu.cpu().numpy()
    check_lists_wellformed(cnt, idx, nb)
    gmask = oracle.lists_to_mask(cnt, idx, nb)
    mism = (gmask != info["mask"]).any(axis=-1)
    e1, e2 = oracle.exempt_rows(info, thr)
    tight1, _ = oracle.exempt_rows(info, thr, e1=1e-6)
    bad = mism & ~(e1 | e2)
    window = info.get("window")
    if window is None:
        window = np.zeros((mism.shape[-1], nb), dtype=bool)
    mode = info.get("mode", "cdf")
    invalid = 0
    for pos in zip(*np.nonzero(mism)):
        i = pos[-1]
        if not valid_cut(gmask[pos], info["p"][pos], window[i], int(info["k"][pos]), thr, mode):
            invalid += 1
            say(f"  invalid cut at row {pos}: k={int(info['k'][pos])} kept={int(gmask[pos].sum())}")
    out = dict(rows=int(mism.size), mismatched=int(mism.sum()), not_exempt=int(bad.sum()),
               e1=int(e1.sum()), e2=int(e2.sum()),
               mismatched_outside_1e6=int((mism & ~(tight1 | e2)).sum()), invalid=invalid)
    say(f"mask parity {label}: {out}")
    assert out["not_exempt"] == 0, out
    assert out["mismatched_outside_1e6"] == 0, out
    assert out["invalid"] == 0, out
    return out


def compare_attention(op_gpu, ref_op, bf16: bool, lse_gpu=None, ref_lse=None, rows=None, label=""):
    o = to_np(op_gpu)
    r = np.asarray(ref_op)
    if rows is not None:
        o, r = o[rows], r[rows]
    err = np.abs(o - r)
    mx, mean = float(err.max()), float(err.mean())
    say(f"attention parity {label}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    if bf16:
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    else:
        assert mx <= F32_MAX_ABS, mx
    if lse_gpu is not None:
        lg = lse_gpu.detach().cpu().numpy().astype(np.float64)
        lr = np.asarray(ref_lse)
        if rows is not None:
            lg, lr = lg[rows], lr[rows]
        fin = np.isfinite(lr)
        assert np.array_equal(fin, np.isfinite(lg))
        lerr = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
        say(f"lse parity {label}: max_abs={lerr:.3e}")
        assert lerr <= LSE_ABS, lerr


def sample_blocks(og, n):
    """Query blocks to check: first, last, padded patches and a spread."""
    bt, bty, btx = oracle.block_coords(og)
    padded = np.nonzero((bty == og.Ty - 1) | (btx == og.Tx - 1))[0]
    pick = {0, og.nb - 1, int(padded[0]), int(padded[-1]), int(padded[len(padded) // 2])}
    pick |= set(np.linspace(0, og.nb - 1, n).astype(int).tolist())
    return sorted(pick)


def sample_rows(blocks, block=64):
    return np.concatenate([np.arange(b * block, (b + 1) * block) for b in blocks])


def attention_on_gpu_lists(qn, kn, vn, cnt_h, idx_h, og, scale, blocks):
    """The oracle's attention of the given query blocks of one head, over the
    GPU's own kept lists (kv_count / kv_index of that head, numpy)."""
    sub = np.zeros_like(cnt_h)
    sub[blocks] = cnt_h[blocks]
    return oracle.bsa_forward(qn, kn, vn, sub, idx_h, og, scale)


def assert_inputs_discriminate(qn, kn, vn, cnt_h, idx_h, og, scale, blocks, ref_o, factor=10.0):
    """The inputs must tell a correct attention kernel from two plausible
    wrong ones, each computed by the oracle on the CPU: uniform weights over
    the kept keys (scale 0), and P.V with the V rows of neighbouring keys
    exchanged. Each must miss the correct output by more than ``factor`` times
    the bf16 output tolerance (max-abs or mean-abs)."""
    rows = sample_rows(blocks)
    uni, _ = attention_on_gpu_lists(qn, kn, vn, cnt_h, idx_h, og, 0.0, blocks)
    swapped = vn.reshape(-1, 2, vn.shape[-1])[:, ::-1].reshape(vn.shape)
    swp, _ = attention_on_gpu_lists(qn, kn, swapped, cnt_h, idx_h, og, scale, blocks)
    for label, m in (("uniform weights", uni), ("neighbouring V rows swapped", swp)):
        err = np.abs(m[rows] - ref_o[rows])
        mx, mean = float(err.max()), float(err.mean())
        say(f"planted mistake ({label}): max_abs={mx:.3e} mean_abs={mean:.3e}")
        assert mx > factor * BF16_MAX_ABS or mean > factor * BF16_MEAN_ABS, (label, mx, mean)


def rescale_rows(qn, kn, cnt_h, idx_h, og, scale, blocks, slack_log2=8.0):
    """Rows of the given query blocks whose running maximum over real keys,
    walking the kept list in order, rises by more than ``slack_log2`` (base-2
    logits) above the first tile's: rows where a lazily rescaled online softmax
    must rescale. Returns (such rows, rows examined)."""
    block, d = og.block, qn.shape[-1]
    kt = kn.reshape(-1, block, d)
    real = oracle.valid_slots(og).reshape(-1, block)
    hit = total = 0
    for b in blocks:
        lst = idx_h[b][: cnt_h[b]]
        z = scale * 1.4426950408889634 * (kt[lst] @ qn[b * block:(b + 1) * block].T)
        z = np.where(real[lst][:, :, None], z, -np.inf)
        tile_max = z.max(axis=1)                        # [tiles, rows]
        run = np.maximum.accumulate(tile_max, axis=0)
        hit += int((run[-1] > tile_max[0] + slack_log2).sum())
        total += block
    return hit, total
