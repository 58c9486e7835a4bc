"""GPU parity of the block-sparse attention backward (cabf_bsa_backward)
against the oracle's gradients, through the C ABI.

Tolerance: the gradients run through bf16 products (P, dS and the inputs
rounded to bf16, fp32 accumulation), so their errors scale with the
gradient's own magnitude: max |err| <= 2e-2 * max |ref| and mean |err| <=
1e-2 * mean |ref| over the compared rows, per tensor.
"""
import math

import numpy as np
import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from synth import WORKLOADS, fourier_video_qkv, gaussian_video_qkv
from tests.parity import say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL_MAX, REL_MEAN = 2e-2, 1e-2
SHARP_SCALE = 3.5        # kernel scale of the sharp cases, times 1/sqrt(d)


def compare_grad(got, ref, rows, label):
    g = to_np(got)[rows]
    r = np.asarray(ref)[rows]
    err = np.abs(g - r)
    scale_max, scale_mean = float(np.abs(r).max()), float(np.abs(r).mean())
    say(f"{label}: max_err {err.max():.3e} (ref max {scale_max:.3e}), mean_err {err.mean():.3e} "
        f"(ref mean {scale_mean:.3e})")
    assert err.max() <= REL_MAX * scale_max + 1e-6
    assert err.mean() <= REL_MEAN * scale_mean + 1e-7


def setup(T, H, W, heads, d, thr, sta, seed=0, amp=0.7, batch=1):
    g = cabf.Geom(batch, heads, d, T, H, W, 8)
    og = oracle.Grid(T, H, W, 8)
    q, k, v = fourier_video_qkv(T, H, W, heads, d, amp, seed=seed, dtype="bf16", batch=batch)
    qp, kp, vp = cabf.permute(q.to(DEV), k.to(DEV), v.to(DEV), g)
    s = cabf.default_scale(g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr, sta, s)
    op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    gen = torch.Generator(device=DEV).manual_seed(seed + 5)
    dop = torch.randn(qp.shape, generator=gen, device=DEV).to(torch.bfloat16)   # pad rows too
    return g, og, s, qp, kp, vp, cnt, idx, op, lse, dop


CASES = [
    ("ragged-d128", (3, 21, 35, 2, 128), 0.4, None),
    ("ragged-d128-window", (3, 21, 35, 2, 128), 0.7, (1, 1, 1)),
    ("ragged-d64", (5, 9, 17, 2, 64), 0.5, None),
    ("wide-d128", (3, 24, 88, 2, 128), 0.8, None),
    ("dense-d128", (2, 16, 16, 1, 128), 0.0, None),
]


@pytest.mark.parametrize("name,shape,thr,sta", CASES)
def test_backward_matches_oracle(name, shape, thr, sta):
    say(f"backward {name} thr={thr} sta={sta}")
    g, og, s, qp, kp, vp, cnt, idx, op, lse, dop = setup(*shape, thr, sta)
    dq, dk, dv = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    dq2, dk2, dv2 = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    pq, pk, pv = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s)     # clock-phased
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))      # deterministic
    valid = oracle.valid_slots(og)
    for hd in range(g.heads):
        ref = oracle.bsa_backward(to_np(qp[0, hd]), to_np(kp[0, hd]), to_np(vp[0, hd]),
                                  to_np(dop[0, hd]), cnt[0, hd].cpu().numpy(),
                                  idx[0, hd].cpu().numpy(), og, s)
        for nm, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            compare_grad(got[0, hd], r, valid, f"{name} head {hd} {nm}")
            assert torch.all(got[0, hd][torch.from_numpy(~valid).to(DEV)] == 0)
        for nm, got, r in (("dq", pq, ref[0]), ("dk", pk, ref[1]), ("dv", pv, ref[2])):
            compare_grad(got[0, hd], r, valid, f"{name} head {hd} {nm} (clock-phased)")
            assert torch.all(got[0, hd][torch.from_numpy(~valid).to(DEV)] == 0)


def test_backward_batch_of_two():
    """Two batch entries of two heads (the key-block order and every pass index
    (batch, head) pairs as one flat axis): both orders against the oracle for
    each (batch, head), and the list order repeats bit for bit."""
    g, og, s, qp, kp, vp, cnt, idx, op, lse, dop = setup(3, 21, 35, 2, 128, 0.5, None, seed=13,
                                                         batch=2)
    det = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    det2 = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    pha = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s)
    torch.cuda.synchronize()
    for a, b in zip(det, det2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    valid = oracle.valid_slots(og)
    for b in range(2):
        for hd in range(g.heads):
            ref = oracle.bsa_backward(to_np(qp[b, hd]), to_np(kp[b, hd]), to_np(vp[b, hd]),
                                      to_np(dop[b, hd]), cnt[b, hd].cpu().numpy(),
                                      idx[b, hd].cpu().numpy(), og, s)
            for tag, grads in (("list order", det), ("clock-phased", pha)):
                for nm, got, r in zip(("dq", "dk", "dv"), grads, ref):
                    compare_grad(got[b, hd], r, valid, f"batch {b} head {hd} {nm} ({tag})")


@pytest.mark.parametrize("name,shape,thr", [("ragged-d128", (3, 21, 35, 2, 128), 0.4),
                                            ("ragged-d64", (5, 9, 17, 2, 64), 0.5)])
def test_backward_sharp_inputs(name, shape, thr):
    """Token-independent Q, K, V at scale 3.5/sqrt(d), where each query's
    weights sit on a few keys, on ragged grids with partial patches: two
    plausible mistakes, planted in the oracle's inputs on the CPU (uniform
    weights; dO rows of neighbouring queries exchanged, as a wrong row order in
    the transposed dO or in dP would do), move every gradient by more than ten
    times the tolerance, and the GPU's gradients, in both visit orders, stay
    within it."""
    T, H, W, heads, d = shape
    say(f"sharp backward {name} thr={thr}")
    g = cabf.Geom(1, heads, d, T, H, W, 8)
    og = oracle.Grid(T, H, W, 8)
    s = SHARP_SCALE / math.sqrt(d)
    q, k, v = gaussian_video_qkv(T, H, W, heads, d, seed=11, device=DEV)
    qp, kp, vp = cabf.permute(q, k, v, g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, thr, None, s)
    op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    gen = torch.Generator(device=DEV).manual_seed(12)
    dop = torch.randn(qp.shape, generator=gen, device=DEV).to(torch.bfloat16)
    dq, dk, dv = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    pq, pk, pv = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s)     # clock-phased
    torch.cuda.synchronize()
    valid = oracle.valid_slots(og)
    for hd in range(heads):
        qn, kn, vn, don = (to_np(t[0, hd]) for t in (qp, kp, vp, dop))
        cnt_h, idx_h = cnt[0, hd].cpu().numpy(), idx[0, hd].cpu().numpy()
        ref = oracle.bsa_backward(qn, kn, vn, don, cnt_h, idx_h, og, s)
        if hd == 0:
            swapped = don.reshape(-1, 2, d)[:, ::-1].reshape(don.shape)
            mistakes = {"uniform weights": oracle.bsa_backward(qn, kn, vn, don, cnt_h, idx_h, og, 0.0),
                        "dO rows exchanged": oracle.bsa_backward(qn, kn, vn, swapped, cnt_h, idx_h, og, s)}
            for label, wrong in mistakes.items():
                for nm, a, b in zip(("dq", "dk", "dv"), wrong, ref):
                    if label == "uniform weights" and nm != "dv":
                        continue      # scale 0 zeroes dq and dk outright
                    err = np.abs(np.asarray(a)[valid] - np.asarray(b)[valid])
                    ref_v = np.abs(np.asarray(b)[valid])
                    say(f"planted mistake ({label}) {nm}: max_err {err.max():.3e} "
                        f"(tolerance {REL_MAX * ref_v.max():.3e}), mean_err {err.mean():.3e} "
                        f"(tolerance {REL_MEAN * ref_v.mean():.3e})")
                    assert (err.max() > 10 * REL_MAX * ref_v.max()
                            or err.mean() > 10 * REL_MEAN * ref_v.mean()), (label, nm)
        for nm, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            compare_grad(got[0, hd], r, valid, f"sharp {name} head {hd} {nm}")
        for nm, got, r in (("dq", pq, ref[0]), ("dk", pk, ref[1]), ("dv", pv, ref[2])):
            compare_grad(got[0, hd], r, valid, f"sharp {name} head {hd} {nm} (clock-phased)")


def test_backward_rows_without_blocks_and_unused_keys():
    g, og, s, qp, kp, vp, cnt, idx, op, lse, dop = setup(3, 21, 35, 2, 128, 0.5, None, seed=3)
    nb = og.nb
    rng = np.random.default_rng(4)
    mask = rng.random((1, g.heads, nb, nb)) < 0.25
    mask[0, 0, 5] = False                  # a query block that keeps nothing
    mask[0, 1, :, 7] = False               # a key block nobody keeps
    cnt_np, idx_np = oracle.mask_to_lists(mask)
    cnt, idx = torch.from_numpy(cnt_np).to(DEV), torch.from_numpy(idx_np).to(DEV)
    op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True, deterministic=True)
    dq, dk, dv = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s)
    torch.cuda.synchronize()
    assert torch.all(dq[0, 0, 5 * 64:6 * 64] == 0)
    assert torch.all(dk[0, 1, 7 * 64:8 * 64] == 0) and torch.all(dv[0, 1, 7 * 64:8 * 64] == 0)
    valid = oracle.valid_slots(og)
    for hd in range(g.heads):
        ref = oracle.bsa_backward(to_np(qp[0, hd]), to_np(kp[0, hd]), to_np(vp[0, hd]),
                                  to_np(dop[0, hd]), cnt_np[0, hd], idx_np[0, hd], og, s)
        for nm, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            compare_grad(got[0, hd], r, valid, f"arbitrary lists head {hd} {nm}")



def test_backward_nonfinite_lse_rows_contribute_nothing():
    """A row whose lse is not finite gets P = 0 (documented for cabf_bsa_backward): its dq is 0
    and dK, dV equal those of a run where that row's dO is zero instead (whose P is finite but
    whose dS and dO products vanish). Deterministic order, so the sums agree exactly."""
    g, og, s, qp, kp, vp, cnt, idx, op, lse, dop = setup(3, 21, 35, 2, 128, 0.5, None, seed=6)
    rows = [(0, 64 + 3), (1, 2 * 64 + 17), (0, 5 * 64 + 40)]     # real rows of kept blocks
    lse_bad = lse.clone()
    dop_zero = dop.clone()
    for (hd, r), val in zip(rows, (float("inf"), float("nan"), float("-inf"))):
        assert torch.isfinite(lse[0, hd, r])
        lse_bad[0, hd, r] = val
        dop_zero[0, hd, r] = 0
    dq_a, dk_a, dv_a = cabf.bsa_backward(qp, kp, vp, op, lse_bad, dop, cnt, idx, g, s,
                                         deterministic=True)
    dq_b, dk_b, dv_b = cabf.bsa_backward(qp, kp, vp, op, lse, dop_zero, cnt, idx, g, s,
                                         deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(dk_a.float(), dk_b.float()) and torch.equal(dv_a.float(), dv_b.float())
    for hd, r in rows:
        assert torch.all(dq_a[0, hd, r] == 0)
        dq_b[0, hd, r] = 0
    assert torch.equal(dq_a.float(), dq_b.float())

def test_backward_full_size_sampled():
    """Wan-14B 720p at 80% sparsity, in both visit orders (clock-phased; list
    order, whose dQ pass runs in several device-sized launches and whose dK/dV
    pass runs the key blocks longest transposed list first): the gradients of
    two key blocks (every query block that keeps them is included, so those
    rows are exact) and the dq of those query blocks, head 0, against the
    oracle; the list-order gradients repeat bit for bit; and the two orders
    agree over the whole of dq, dk and dv (the same sums in another order),
    so no key block or query block is left out by either."""
    w = WORKLOADS["wan14b-720p"]
    g = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    og = oracle.Grid(w.T, w.H, w.W, w.P)
    q, k, v = fourier_video_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.amplitude, seed=8,
                                dtype=w.dtype, device=DEV)
    qp, kp, vp = cabf.permute(q, k, v, g)
    s = cabf.default_scale(g)
    cnt, idx = cabf.build_block_mask(qp, kp, g, 0.7935, None, s)
    op, lse = cabf.bsa_forward(qp, kp, vp, cnt, idx, g, s, return_lse=True)
    dop = torch.randn(qp.shape, generator=torch.Generator(device=DEV).manual_seed(9),
                      device=DEV).to(torch.bfloat16)
    dq, dk, dv = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s)
    det = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    det2 = cabf.bsa_backward(qp, kp, vp, op, lse, dop, cnt, idx, g, s, deterministic=True)
    torch.cuda.synchronize()
    for nm, a, b, c in zip(("dq", "dk", "dv"), (dq, dk, dv), det, det2):
        assert torch.equal(b.view(torch.int16), c.view(torch.int16)), nm
        diff = float((a.float() - b.float()).abs().max())
        big = float(a.float().abs().max())
        say(f"full-size {nm}: clock-phased vs list order max diff {diff:.3e} (max {big:.3e})")
        assert diff <= 1e-2 * big, nm
    # into gradients filled with NaN beforehand, both orders: every row of
    # every head is written (pad rows with 0), so the comparison above cannot
    # pass on untouched memory
    bws = cabf._ws(cabf._lib.cabf_bsa_backward_workspace_bytes(cabf.ctypes.byref(g.c())), DEV)
    for flags, ref_grads in ((0, det), (cabf.BSA_DETERMINISTIC, det)):
        grads = [torch.full_like(qp, float("nan")) for _ in range(3)]
        cabf.cabf_bsa_backward(g, qp, kp, vp, op, lse, dop, cnt, idx, s, *grads, bws, flags)
        torch.cuda.synchronize()
        for nm, a, b in zip(("dq", "dk", "dv"), grads, ref_grads):
            assert torch.isfinite(a.float()).all(), f"{nm} rows left unwritten (flags {flags})"
            if flags:
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
            else:
                assert float((a.float() - b.float()).abs().max()) <= 1e-2 * float(b.float().abs().max()), nm
    hd = 0
    c0, i0 = cnt[0, hd].cpu().numpy(), idx[0, hd].cpu().numpy()
    key_blocks = [0, og.nb - 1]
    keeps = np.array([np.isin(key_blocks, i0[i][: c0[i]]).any() for i in range(og.nb)])
    sub = np.where(keeps, c0, 0)
    say(f"full-size backward: {int(keeps.sum())} query blocks keep key blocks {key_blocks}")
    ref = oracle.bsa_backward(to_np(qp[0, hd]), to_np(kp[0, hd]), to_np(vp[0, hd]),
                              to_np(dop[0, hd]), sub, i0, og, s)
    valid = oracle.valid_slots(og)
    krows = np.concatenate([np.arange(b * 64, (b + 1) * 64) for b in key_blocks])
    krows = krows[valid[krows]]
    qrows = np.concatenate([np.arange(b * 64, (b + 1) * 64) for b in np.nonzero(keeps)[0][:40]])
    qrows = qrows[valid[qrows]]
    for tag, (gq, gk, gv) in (("clock-phased", (dq, dk, dv)), ("list order", det)):
        compare_grad(gk[0, hd], ref[1], krows, f"full-size dk ({tag})")
        compare_grad(gv[0, hd], ref[2], krows, f"full-size dv ({tag})")
        compare_grad(gq[0, hd], ref[0], qrows, f"full-size dq ({tag})")
