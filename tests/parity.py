"""Shared helpers of the GPU parity tests: input upload and comparisons with
the CPU oracle. No method arithmetic lives here; the oracle computes every
expected value."""
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


def compare_masks(cnt_gpu, idx_gpu, info, thr, label=""):
    """Kept-block lists must agree except on rows whose cut is ill-posed
    (oracle.exempt_rows: within 1e-4 of the threshold, or a near-tie at the cut).
    Returns a dict of counts for reporting."""
    nb = info["mask"].shape[-1]
    cnt = cnt_gpu.cpu().numpy()
    idx = idx_gpu.cpu().numpy()
    check_lists_wellformed(cnt, idx, nb)
    gmask = oracle.lists_to_mask(cnt, idx, nb)
    mism = (gmask != info["mask"]).any(axis=-1)
    e1, e2 = oracle.exempt_rows(info, thr)
    tight1, _ = oracle.exempt_rows(info, thr, e1=1e-6)
    bad = mism & ~(e1 | e2)
    out = dict(rows=int(mism.size), mismatched=int(mism.sum()), not_exempt=int(bad.sum()),
               e1=int(e1.sum()), e2=int(e2.sum()),
               mismatched_outside_1e6=int((mism & ~(tight1 | e2)).sum()))
    say(f"mask parity {label}: {out}")
    assert out["not_exempt"] == 0, out
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
