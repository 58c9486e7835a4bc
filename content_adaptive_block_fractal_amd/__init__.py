"""Content-adaptive block-sparse video attention on MI355X (gfx950).

Thin Python binding of libcabf.so, the C ABI declared in include/cabf.h.
Each ``cabf_*`` function here has the same name and arguments as its C
counterpart: it checks tensor shapes, dtypes and devices, passes raw device
pointers and the current HIP stream, and raises ``CabfError`` on a non-zero
status. Every step of the path runs in the HIP kernels; PyTorch only provides
device memory and the stream. The helpers at the bottom (``permute``,
``build_block_mask``, ``bsa_forward``, ``unpermute``, ``layer``) allocate the
outputs and call the same entry points.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CABF_LIB may point at another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("CABF_LIB") or os.path.join(_HERE, "libcabf.so")

CABF_OK, CABF_EINVAL, CABF_EUNSUPPORTED, CABF_EWORKSPACE, CABF_EHIP = 0, -1, -2, -3, -4
CABF_BF16, CABF_F32 = 0, 1

EXPORTED = ("cabf_geom_sizes", "cabf_permute", "cabf_permute_pool", "cabf_unpermute",
            "cabf_mask_workspace_bytes", "cabf_build_block_mask", "cabf_build_block_mask_topk",
            "cabf_build_block_mask_noalloc",
            "cabf_build_block_mask_pooled", "cabf_build_sta_mask", "cabf_bsa_forward",
            "cabf_bsa_forward_subset", "cabf_bsa_backward_workspace_bytes", "cabf_bsa_backward",
            "cabf_kmeans_workspace_bytes", "cabf_kmeans", "cabf_gather_rows",
            "cabf_scatter_rows", "cabf_cluster_select_workspace_bytes", "cabf_cluster_select",
            "cabf_cluster_attention_workspace_bytes", "cabf_cluster_attention",
            "cabf_status_string")

SEQ_PAD_ROWS = 64      # extra zero rows of permuted tensors for cabf_cluster_attention


class CabfError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({cabf_status_string(status)})")
        self.status = status


class _Geom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("P", ctypes.c_int32)]


class _Seq(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n", ctypes.c_int32)]


class _Sta(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int32), ("dt", ctypes.c_int32), ("dy", ctypes.c_int32),
                ("dx", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python content_adaptive_block_fractal_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    G = ctypes.POINTER(_Geom)
    Q = ctypes.POINTER(_Seq)
    sig = {
        "cabf_geom_sizes": (ctypes.c_int, [G, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                           ctypes.POINTER(I32), ctypes.POINTER(I32),
                                           ctypes.POINTER(I32)]),
        "cabf_permute": (ctypes.c_int, [G, ctypes.c_int, P, P, P, P, P, P, P]),
        "cabf_permute_pool": (ctypes.c_int, [G, ctypes.c_int, P, P, P, P, P, P, P, SZ, P]),
        "cabf_unpermute": (ctypes.c_int, [G, ctypes.c_int, P, P, P]),
        "cabf_mask_workspace_bytes": (SZ, [G]),
        "cabf_build_block_mask": (ctypes.c_int, [G, ctypes.c_int, P, P, F32, F32,
                                                 ctypes.POINTER(_Sta), P, P, P, P, SZ, P]),
        "cabf_build_block_mask_topk": (ctypes.c_int, [G, ctypes.c_int, P, P, F32, I32,
                                                      ctypes.POINTER(_Sta), P, P, P, P, SZ, P]),
        "cabf_build_block_mask_noalloc": (ctypes.c_int, [G, ctypes.c_int, P, P, F32, F32,
                                                         ctypes.POINTER(_Sta), P, P, P, P]),
        "cabf_build_block_mask_pooled": (ctypes.c_int, [G, F32, F32, I32, ctypes.POINTER(_Sta),
                                                        P, P, P, P, SZ, P]),
        "cabf_build_sta_mask": (ctypes.c_int, [G, ctypes.POINTER(_Sta), P, P, P]),
        "cabf_bsa_forward": (ctypes.c_int, [G, ctypes.c_int, P, P, P, P, P, F32, P, P,
                                            ctypes.c_uint, P]),
        "cabf_bsa_forward_subset": (ctypes.c_int, [G, ctypes.c_int, P, P, P, P, P, P, I64, F32, P,
                                                   P, ctypes.c_uint, P]),
        "cabf_bsa_backward_workspace_bytes": (SZ, [G]),
        "cabf_bsa_backward": (ctypes.c_int, [G, ctypes.c_int, P, P, P, P, P, P, P, P, F32, P, P, P,
                                             P, SZ, ctypes.c_uint, P]),
        "cabf_kmeans_workspace_bytes": (SZ, [Q, I32]),
        "cabf_kmeans": (ctypes.c_int, [Q, ctypes.c_int, P, I32, P, I32, P, P, P, P, P, P, SZ, P]),
        "cabf_gather_rows": (ctypes.c_int, [Q, ctypes.c_int, P, P, P, I32, P]),
        "cabf_scatter_rows": (ctypes.c_int, [Q, ctypes.c_int, P, I32, P, P, P]),
        "cabf_cluster_select_workspace_bytes": (SZ, [Q, I32, I32]),
        "cabf_cluster_select": (ctypes.c_int, [Q, I32, I32, P, P, P, F32, F32, P, P, P, P, SZ, P]),
        "cabf_cluster_attention_workspace_bytes": (SZ, [Q, I32, I32]),
        "cabf_cluster_attention": (ctypes.c_int, [Q, ctypes.c_int, I32, I32, P, P, P, P, P, P, P,
                                                  F32, P, P, P, SZ, P]),
        "cabf_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


@dataclass(frozen=True)
class Geom:
    """Layer geometry (cabf_geom): P x P patches of a T x H x W latent grid."""
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    P: int = 8

    def c(self) -> _Geom:
        return _Geom(self.batch, self.heads, self.head_dim, self.T, self.H, self.W, self.P)

    def sizes(self) -> dict:
        """Derived sizes from the library: tokens (raster / padded), blocks, Hp, Wp."""
        nr, npd = ctypes.c_int64(), ctypes.c_int64()
        nb, hp, wp = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = _lib.cabf_geom_sizes(ctypes.byref(self.c()), ctypes.byref(nr), ctypes.byref(npd),
                                  ctypes.byref(nb), ctypes.byref(hp), ctypes.byref(wp))
        _check("cabf_geom_sizes", st)
        return dict(tokens_raster=nr.value, tokens_padded=npd.value, n_blocks=nb.value,
                    Hp=hp.value, Wp=wp.value)


def cabf_status_string(status: int) -> str:
    return _lib.cabf_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != CABF_OK:
        raise CabfError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CABF_BF16
    if t.dtype == torch.float32:
        return CABF_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, shape, dtype=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def cabf_permute(geom: Geom, q, k, v, qp, kp, vp):
    """Fractal reorder raster q, k, v [B, h, T*H*W, d] into qp, kp, vp [B, h, N, d]."""
    s = geom.sizes()
    rs = (geom.batch, geom.heads, s["tokens_raster"], geom.head_dim)
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    first = next((t for t in (q, k, v) if t is not None), None)
    if first is None:
        return
    dt = first.dtype
    ptrs = []
    for src, dst, n in ((q, qp, "q"), (k, kp, "k"), (v, vp, "v")):
        if src is None and dst is None:
            ptrs += [None, None]
            continue
        ptrs += [_dev(src, rs, dt, n), _dev(dst, ps, dt, n + "p")]
    st = _lib.cabf_permute(ctypes.byref(geom.c()), _dtype_code(first), ptrs[0], ptrs[2], ptrs[4],
                           ptrs[1], ptrs[3], ptrs[5], _stream(first))
    _check("cabf_permute", st)


def cabf_permute_pool(geom: Geom, q, k, v, qp, kp, vp, workspace):
    """cabf_permute that also leaves the fp32 block means of q and k in ``workspace``
    (a mask workspace) for cabf_build_block_mask_pooled. v / vp may be None."""
    s = geom.sizes()
    rs = (geom.batch, geom.heads, s["tokens_raster"], geom.head_dim)
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    dt = q.dtype
    vv = (None, None) if v is None and vp is None else (_dev(v, rs, dt, "v"), _dev(vp, ps, dt, "vp"))
    ptr, nbytes = _ws_ptr(workspace)
    st = _lib.cabf_permute_pool(ctypes.byref(geom.c()), _dtype_code(q), _dev(q, rs, None, "q"),
                                _dev(k, rs, dt, "k"), vv[0], _dev(qp, ps, dt, "qp"),
                                _dev(kp, ps, dt, "kp"), vv[1], ptr, nbytes, _stream(q))
    _check("cabf_permute_pool", st)


def cabf_unpermute(geom: Geom, op, o):
    """Restore raster order: op [B, h, N, d] -> o [B, h, T*H*W, d]."""
    s = geom.sizes()
    st = _lib.cabf_unpermute(
        ctypes.byref(geom.c()), _dtype_code(op),
        _dev(op, (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim), None, "op"),
        _dev(o, (geom.batch, geom.heads, s["tokens_raster"], geom.head_dim), op.dtype, "o"),
        _stream(op))
    _check("cabf_unpermute", st)


def cabf_mask_workspace_bytes(geom: Geom) -> int:
    return int(_lib.cabf_mask_workspace_bytes(ctypes.byref(geom.c())))


def cabf_build_block_mask(geom: Geom, qp, kp, scale: float, thr: float, sta, kv_count, kv_index,
                          block_prob, workspace, topk=None):
    """Adaptive block mask into kv_count [B, h, nb] / kv_index [B, h, nb, nb] (int32).
    With ``topk`` set, calls cabf_build_block_mask_topk (thr unused)."""
    s = geom.sizes()
    nb = s["n_blocks"]
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    lead = (geom.batch, geom.heads, nb)
    sta_c = None
    if sta is not None:
        sta_c = ctypes.byref(_Sta(1, int(sta[0]), int(sta[1]), int(sta[2])))
    bp = None
    if block_prob is not None:
        bp = _dev(block_prob, lead + (nb,), torch.float32, "block_prob")
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_cuda:
        raise ValueError("workspace must be a 1-D uint8 device tensor")
    fn, sel = ((_lib.cabf_build_block_mask, float(thr)) if topk is None
               else (_lib.cabf_build_block_mask_topk, int(topk)))
    st = fn(ctypes.byref(geom.c()), _dtype_code(qp), _dev(qp, ps, None, "qp"),
            _dev(kp, ps, qp.dtype, "kp"), float(scale), sel, sta_c,
            _dev(kv_count, lead, torch.int32, "kv_count"),
            _dev(kv_index, lead + (nb,), torch.int32, "kv_index"), bp,
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(qp))
    _check("cabf_build_block_mask" if topk is None else "cabf_build_block_mask_topk", st)


NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024   # CABF_NOALLOC_SCRATCH_BYTES


def cabf_build_block_mask_noalloc(geom: Geom, qp, kp, scale: float, thr: float, sta, kv_count,
                                  kv_index, block_prob=None):
    """cabf_build_block_mask with the library's static device scratch instead of a
    workspace: allocates nothing (for callers that cannot allocate)."""
    s = geom.sizes()
    nb = s["n_blocks"]
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    lead = (geom.batch, geom.heads, nb)
    sta_c = None
    if sta is not None:
        sta_c = ctypes.byref(_Sta(1, int(sta[0]), int(sta[1]), int(sta[2])))
    bp = None if block_prob is None else _dev(block_prob, lead + (nb,), torch.float32,
                                              "block_prob")
    st = _lib.cabf_build_block_mask_noalloc(
        ctypes.byref(geom.c()), _dtype_code(qp), _dev(qp, ps, None, "qp"),
        _dev(kp, ps, qp.dtype, "kp"), float(scale), float(thr), sta_c,
        _dev(kv_count, lead, torch.int32, "kv_count"),
        _dev(kv_index, lead + (nb,), torch.int32, "kv_index"), bp, _stream(qp))
    _check("cabf_build_block_mask_noalloc", st)


def cabf_build_block_mask_pooled(geom: Geom, scale: float, thr: float, k: int, sta, kv_count,
                                 kv_index, block_prob, workspace):
    """Block mask from the means cabf_permute_pool left in ``workspace``: the CDF cut at
    thr (k = 0) or the top-k blocks per row (k >= 1)."""
    nb = geom.sizes()["n_blocks"]
    lead = (geom.batch, geom.heads, nb)
    sta_c = None
    if sta is not None:
        sta_c = ctypes.byref(_Sta(1, int(sta[0]), int(sta[1]), int(sta[2])))
    bp = None if block_prob is None else _dev(block_prob, lead + (nb,), torch.float32,
                                              "block_prob")
    ptr, nbytes = _ws_ptr(workspace)
    st = _lib.cabf_build_block_mask_pooled(
        ctypes.byref(geom.c()), float(scale), float(thr), int(k), sta_c,
        _dev(kv_count, lead, torch.int32, "kv_count"),
        _dev(kv_index, lead + (nb,), torch.int32, "kv_index"), bp, ptr, nbytes,
        _stream(kv_count))
    _check("cabf_build_block_mask_pooled", st)


def cabf_build_sta_mask(geom: Geom, sta, kv_count, kv_index):
    """Sliding-tile window lists alone into kv_count / kv_index (int32)."""
    nb = geom.sizes()["n_blocks"]
    lead = (geom.batch, geom.heads, nb)
    sta_c = None if sta is None else ctypes.byref(_Sta(1, int(sta[0]), int(sta[1]), int(sta[2])))
    st = _lib.cabf_build_sta_mask(ctypes.byref(geom.c()), sta_c,
                                  _dev(kv_count, lead, torch.int32, "kv_count"),
                                  _dev(kv_index, lead + (nb,), torch.int32, "kv_index"),
                                  _stream(kv_count))
    _check("cabf_build_sta_mask", st)


BSA_DETERMINISTIC = 1    # cabf_bsa_forward flag: walk every list from its first entry


def cabf_bsa_forward(geom: Geom, qp, kp, vp, kv_count, kv_index, scale: float, op, lse=None,
                     flags: int = 0):
    """Block-sparse attention over the listed tiles: op [B, h, N, d] (+ lse [B, h, N])."""
    s = geom.sizes()
    nb = s["n_blocks"]
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    lead = (geom.batch, geom.heads, nb)
    lp = None if lse is None else _dev(lse, ps[:3], torch.float32, "lse")
    st = _lib.cabf_bsa_forward(
        ctypes.byref(geom.c()), _dtype_code(qp), _dev(qp, ps, None, "qp"),
        _dev(kp, ps, qp.dtype, "kp"), _dev(vp, ps, qp.dtype, "vp"),
        _dev(kv_count, lead, torch.int32, "kv_count"),
        _dev(kv_index, lead + (nb,), torch.int32, "kv_index"), float(scale),
        _dev(op, ps, qp.dtype, "op"), lp, int(flags), _stream(qp))
    _check("cabf_bsa_forward", st)


def cabf_bsa_forward_subset(geom: Geom, qp, kp, vp, kv_count, kv_index, q_blocks, scale: float,
                            op, lse=None, flags: int = 0):
    """cabf_bsa_forward over the global query blocks in ``q_blocks`` (int32 device
    tensor of (b*heads + h)*nb + i); other rows of op / lse are left untouched."""
    s = geom.sizes()
    nb = s["n_blocks"]
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    lead = (geom.batch, geom.heads, nb)
    lp = None if lse is None else _dev(lse, ps[:3], torch.float32, "lse")
    if q_blocks.dtype != torch.int32 or q_blocks.dim() != 1:
        raise ValueError("q_blocks must be a 1-D int32 tensor")
    n = q_blocks.numel()
    qb = _dev(q_blocks, (n,), torch.int32, "q_blocks") if n > 0 else None
    st = _lib.cabf_bsa_forward_subset(
        ctypes.byref(geom.c()), _dtype_code(qp), _dev(qp, ps, None, "qp"),
        _dev(kp, ps, qp.dtype, "kp"), _dev(vp, ps, qp.dtype, "vp"),
        _dev(kv_count, lead, torch.int32, "kv_count"),
        _dev(kv_index, lead + (nb,), torch.int32, "kv_index"), qb, n, float(scale),
        _dev(op, ps, qp.dtype, "op"), lp, int(flags), _stream(qp))
    _check("cabf_bsa_forward_subset", st)


# --- allocating helpers -----------------------------------------------------------

def default_scale(geom: Geom) -> float:
    return 1.0 / math.sqrt(geom.head_dim)


def permute(q, k, v, geom: Geom):
    n = geom.sizes()["tokens_padded"]
    shape = (geom.batch, geom.heads, n, geom.head_dim)
    qp, kp, vp = (torch.empty(shape, dtype=q.dtype, device=q.device) for _ in range(3))
    cabf_permute(geom, q, k, v, qp, kp, vp)
    return qp, kp, vp


def unpermute(op, geom: Geom):
    n = geom.sizes()["tokens_raster"]
    o = torch.empty((geom.batch, geom.heads, n, geom.head_dim), dtype=op.dtype, device=op.device)
    cabf_unpermute(geom, op, o)
    return o


def mask_workspace(geom: Geom, device) -> torch.Tensor:
    return torch.empty(cabf_mask_workspace_bytes(geom), dtype=torch.uint8, device=device)


def build_block_mask(qp, kp, geom: Geom, thr: float, sta=None, scale=None, return_probs=False,
                     workspace=None, topk=None):
    """(kv_count, kv_index) of the CDF cut at thr, or of the top-``topk`` blocks per row."""
    nb = geom.sizes()["n_blocks"]
    lead = (geom.batch, geom.heads, nb)
    kv_count = torch.empty(lead, dtype=torch.int32, device=qp.device)
    kv_index = torch.empty(lead + (nb,), dtype=torch.int32, device=qp.device)
    probs = torch.empty(lead + (nb,), dtype=torch.float32, device=qp.device) if return_probs else None
    ws = mask_workspace(geom, qp.device) if workspace is None else workspace
    cabf_build_block_mask(geom, qp, kp, default_scale(geom) if scale is None else scale, thr, sta,
                          kv_count, kv_index, probs, ws, topk=topk)
    if return_probs:
        return kv_count, kv_index, probs
    return kv_count, kv_index


def permute_pool(q, k, v, geom: Geom, workspace=None):
    """(qp, kp, vp, workspace): the reordered tensors and a mask workspace holding the
    block means, ready for build_block_mask_pooled."""
    n = geom.sizes()["tokens_padded"]
    shape = (geom.batch, geom.heads, n, geom.head_dim)
    qp, kp = (torch.empty(shape, dtype=q.dtype, device=q.device) for _ in range(2))
    vp = None if v is None else torch.empty(shape, dtype=q.dtype, device=q.device)
    ws = mask_workspace(geom, q.device) if workspace is None else workspace
    cabf_permute_pool(geom, q, k, v, qp, kp, vp, ws)
    return qp, kp, vp, ws


def build_block_mask_pooled(workspace, geom: Geom, thr: float, sta=None, scale=None,
                            return_probs=False, topk=None, device=None):
    """build_block_mask from the block means left by permute_pool."""
    nb = geom.sizes()["n_blocks"]
    lead = (geom.batch, geom.heads, nb)
    dev = workspace.device if device is None else device
    kv_count = torch.empty(lead, dtype=torch.int32, device=dev)
    kv_index = torch.empty(lead + (nb,), dtype=torch.int32, device=dev)
    probs = torch.empty(lead + (nb,), dtype=torch.float32, device=dev) if return_probs else None
    cabf_build_block_mask_pooled(geom, default_scale(geom) if scale is None else scale,
                                 0.0 if topk else thr, int(topk or 0), sta, kv_count, kv_index,
                                 probs, workspace)
    if return_probs:
        return kv_count, kv_index, probs
    return kv_count, kv_index


def topk_for_ratio(geom: Geom, ratio: float) -> int:
    """Blocks kept per row for a static keep ratio: ceil(ratio * nb), at least 1."""
    nb = geom.sizes()["n_blocks"]
    return max(1, min(nb, math.ceil(ratio * nb - 1e-9)))


def build_sta_mask(geom: Geom, sta, device):
    nb = geom.sizes()["n_blocks"]
    lead = (geom.batch, geom.heads, nb)
    kv_count = torch.empty(lead, dtype=torch.int32, device=device)
    kv_index = torch.empty(lead + (nb,), dtype=torch.int32, device=device)
    cabf_build_sta_mask(geom, sta, kv_count, kv_index)
    return kv_count, kv_index


def bsa_forward(qp, kp, vp, kv_count, kv_index, geom: Geom, scale=None, return_lse=False,
                deterministic=False):
    op = torch.empty_like(qp)
    lse = torch.empty(qp.shape[:3], dtype=torch.float32, device=qp.device) if return_lse else None
    cabf_bsa_forward(geom, qp, kp, vp, kv_count, kv_index,
                     default_scale(geom) if scale is None else scale, op, lse,
                     BSA_DETERMINISTIC if deterministic else 0)
    return (op, lse) if return_lse else op


def bsa_forward_subset(qp, kp, vp, kv_count, kv_index, q_blocks, geom: Geom, op, lse=None,
                       scale=None, deterministic=False):
    """Fill the rows of the listed query blocks of op (and lse) in place."""
    cabf_bsa_forward_subset(geom, qp, kp, vp, kv_count, kv_index, q_blocks,
                            default_scale(geom) if scale is None else scale, op, lse,
                            BSA_DETERMINISTIC if deterministic else 0)
    return op


def cabf_bsa_backward(geom: Geom, qp, kp, vp, op, lse, dop, kv_count, kv_index, scale: float,
                      dqp, dkp, dvp, workspace, flags: int = 0):
    """Gradients of cabf_bsa_forward: dqp, dkp, dvp [B, h, N, d] (bf16)."""
    s = geom.sizes()
    nb = s["n_blocks"]
    ps = (geom.batch, geom.heads, s["tokens_padded"], geom.head_dim)
    lead = (geom.batch, geom.heads, nb)
    ptr, nbytes = _ws_ptr(workspace)
    st = _lib.cabf_bsa_backward(
        ctypes.byref(geom.c()), _dtype_code(qp), _dev(qp, ps, None, "qp"),
        _dev(kp, ps, qp.dtype, "kp"), _dev(vp, ps, qp.dtype, "vp"), _dev(op, ps, qp.dtype, "op"),
        _dev(lse, ps[:3], torch.float32, "lse"), _dev(dop, ps, qp.dtype, "dop"),
        _dev(kv_count, lead, torch.int32, "kv_count"),
        _dev(kv_index, lead + (nb,), torch.int32, "kv_index"), float(scale),
        _dev(dqp, ps, qp.dtype, "dqp"), _dev(dkp, ps, qp.dtype, "dkp"),
        _dev(dvp, ps, qp.dtype, "dvp"), ptr, nbytes, int(flags), _stream(qp))
    _check("cabf_bsa_backward", st)


def bsa_backward(qp, kp, vp, op, lse, dop, kv_count, kv_index, geom: Geom, scale=None,
                 deterministic=False):
    """(dqp, dkp, dvp) of the block-sparse attention over the given lists."""
    dqp, dkp, dvp = (torch.empty_like(qp) for _ in range(3))
    ws = _ws(_lib.cabf_bsa_backward_workspace_bytes(ctypes.byref(geom.c())), qp.device)
    cabf_bsa_backward(geom, qp, kp, vp, op, lse, dop, kv_count, kv_index,
                      default_scale(geom) if scale is None else scale, dqp, dkp, dvp, ws,
                      BSA_DETERMINISTIC if deterministic else 0)
    return dqp, dkp, dvp


def layer(q, k, v, geom: Geom, thr: float, sta=None, scale=None):
    """One attention layer: reorder (pooling the blocks on the way), mask,
    block-sparse attention, restore order."""
    qp, kp, vp, ws = permute_pool(q, k, v, geom)
    kv_count, kv_index = build_block_mask_pooled(ws, geom, thr, sta, scale)
    op = bsa_forward(qp, kp, vp, kv_count, kv_index, geom, scale)
    return unpermute(op, geom), (kv_count, kv_index)


# --- semantic-permutation variant ----------------------------------------------------

@dataclass(frozen=True)
class Seq:
    """Token sequences (cabf_seq): batch x heads sequences of n tokens."""
    batch: int
    heads: int
    head_dim: int
    n: int

    def c(self) -> _Seq:
        return _Seq(self.batch, self.heads, self.head_dim, self.n)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ws_ptr(ws: torch.Tensor):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_cuda:
        raise ValueError("workspace must be a 1-D uint8 device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel()


def cabf_kmeans(seq: Seq, x, clusters: int, init, iters: int, centroids, counts, labels, perm,
                offsets, workspace):
    """k-means of [B, h, n, d] bf16 token features and the cluster permutation."""
    lead = (seq.batch, seq.heads)
    ptr, nbytes = _ws_ptr(workspace)
    st = _lib.cabf_kmeans(
        ctypes.byref(seq.c()), _dtype_code(x), _dev(x, lead + (seq.n, seq.head_dim), None, "x"),
        int(clusters), _dev(init, lead + (clusters,), torch.int32, "init"), int(iters),
        _dev(centroids, lead + (clusters, seq.head_dim), torch.float32, "centroids"),
        _dev(counts, lead + (clusters,), torch.int32, "counts"),
        _dev(labels, lead + (seq.n,), torch.int32, "labels"),
        _dev(perm, lead + (seq.n,), torch.int32, "perm"),
        _dev(offsets, lead + (clusters + 1,), torch.int32, "offsets"), ptr, nbytes, _stream(x))
    _check("cabf_kmeans", st)


def cabf_gather_rows(seq: Seq, x, perm, xp, rows_out: int):
    lead = (seq.batch, seq.heads)
    st = _lib.cabf_gather_rows(ctypes.byref(seq.c()), _dtype_code(x),
                               _dev(x, lead + (seq.n, seq.head_dim), None, "x"),
                               _dev(perm, lead + (seq.n,), torch.int32, "perm"),
                               _dev(xp, lead + (rows_out, seq.head_dim), x.dtype, "xp"),
                               int(rows_out), _stream(x))
    _check("cabf_gather_rows", st)


def cabf_scatter_rows(seq: Seq, xp, rows_in: int, perm, x):
    lead = (seq.batch, seq.heads)
    st = _lib.cabf_scatter_rows(ctypes.byref(seq.c()), _dtype_code(xp),
                                _dev(xp, lead + (rows_in, seq.head_dim), None, "xp"), int(rows_in),
                                _dev(perm, lead + (seq.n,), torch.int32, "perm"),
                                _dev(x, lead + (seq.n, seq.head_dim), xp.dtype, "x"), _stream(xp))
    _check("cabf_scatter_rows", st)


def cabf_cluster_select(seq: Seq, cq: int, ck: int, q_centroids, k_centroids, k_counts,
                        scale: float, top_p: float, kv_count, kv_index, probs, workspace):
    lead = (seq.batch, seq.heads)
    ptr, nbytes = _ws_ptr(workspace)
    pr = None if probs is None else _dev(probs, lead + (cq, ck), torch.float32, "probs")
    st = _lib.cabf_cluster_select(
        ctypes.byref(seq.c()), int(cq), int(ck),
        _dev(q_centroids, lead + (cq, seq.head_dim), torch.float32, "q_centroids"),
        _dev(k_centroids, lead + (ck, seq.head_dim), torch.float32, "k_centroids"),
        _dev(k_counts, lead + (ck,), torch.int32, "k_counts"), float(scale), float(top_p),
        _dev(kv_count, lead + (cq,), torch.int32, "kv_count"),
        _dev(kv_index, lead + (cq, ck), torch.int32, "kv_index"), pr, ptr, nbytes,
        _stream(kv_count))
    _check("cabf_cluster_select", st)


def cabf_cluster_attention(seq: Seq, cq: int, ck: int, qp, kp, vp, q_offsets, k_offsets, kv_count,
                           kv_index, scale: float, op, lse, workspace):
    lead = (seq.batch, seq.heads)
    rows = seq.n + SEQ_PAD_ROWS
    ptr, nbytes = _ws_ptr(workspace)
    shape = lead + (rows, seq.head_dim)
    lp = None if lse is None else _dev(lse, lead + (rows,), torch.float32, "lse")
    st = _lib.cabf_cluster_attention(
        ctypes.byref(seq.c()), _dtype_code(qp), int(cq), int(ck), _dev(qp, shape, None, "qp"),
        _dev(kp, shape, qp.dtype, "kp"), _dev(vp, shape, qp.dtype, "vp"),
        _dev(q_offsets, lead + (cq + 1,), torch.int32, "q_offsets"),
        _dev(k_offsets, lead + (ck + 1,), torch.int32, "k_offsets"),
        _dev(kv_count, lead + (cq,), torch.int32, "kv_count"),
        _dev(kv_index, lead + (cq, ck), torch.int32, "kv_index"), float(scale),
        _dev(op, shape, qp.dtype, "op"), lp, ptr, nbytes, _stream(qp))
    _check("cabf_cluster_attention", st)


def kmeans(x, clusters: int, init, iters: int):
    """Returns dict(centroids, counts, labels, perm, offsets) for [B, h, n, d] bf16 x."""
    B, h, n, d = x.shape
    seq = Seq(B, h, d, n)
    dev = x.device
    out = dict(centroids=torch.empty(B, h, clusters, d, dtype=torch.float32, device=dev),
               counts=torch.empty(B, h, clusters, dtype=torch.int32, device=dev),
               labels=torch.empty(B, h, n, dtype=torch.int32, device=dev),
               perm=torch.empty(B, h, n, dtype=torch.int32, device=dev),
               offsets=torch.empty(B, h, clusters + 1, dtype=torch.int32, device=dev))
    ws = _ws(_lib.cabf_kmeans_workspace_bytes(ctypes.byref(seq.c()), int(clusters)), dev)
    cabf_kmeans(seq, x, clusters, init, iters, out["centroids"], out["counts"], out["labels"],
                out["perm"], out["offsets"], ws)
    return out


def svg_layer(q, k, v, cq: int, ck: int, init_q, init_k, iters: int, top_p: float, scale=None,
              return_info=False):
    """One attention layer of the semantic-permutation variant, raster order in
    and out: k-means of Q and K, permutation, centroid top-p, cluster attention,
    inverse permutation. q, k, v: [B, h, n, d] bf16."""
    B, h, n, d = q.shape
    seq = Seq(B, h, d, n)
    dev = q.device
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    # the two clusterings are independent: K's runs on a second stream
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(main)
    with torch.cuda.stream(side):
        kk = kmeans(k, ck, init_k, iters)
    kq = kmeans(q, cq, init_q, iters)
    main.wait_stream(side)
    for t in kk.values():
        t.record_stream(main)
    rows = n + SEQ_PAD_ROWS
    qp, kp, vp, op = (torch.empty(B, h, rows, d, dtype=q.dtype, device=dev) for _ in range(4))
    cabf_gather_rows(seq, q, kq["perm"], qp, rows)
    cabf_gather_rows(seq, k, kk["perm"], kp, rows)
    cabf_gather_rows(seq, v, kk["perm"], vp, rows)
    kv_count = torch.empty(B, h, cq, dtype=torch.int32, device=dev)
    kv_index = torch.empty(B, h, cq, ck, dtype=torch.int32, device=dev)
    ws = _ws(_lib.cabf_cluster_select_workspace_bytes(ctypes.byref(seq.c()), int(cq), int(ck)), dev)
    cabf_cluster_select(seq, cq, ck, kq["centroids"], kk["centroids"], kk["counts"], scale, top_p,
                        kv_count, kv_index, None, ws)
    ws = _ws(_lib.cabf_cluster_attention_workspace_bytes(ctypes.byref(seq.c()), int(cq), int(ck)),
             dev)
    lse = torch.empty(B, h, rows, dtype=torch.float32, device=dev)
    cabf_cluster_attention(seq, cq, ck, qp, kp, vp, kq["offsets"], kk["offsets"], kv_count,
                           kv_index, scale, op, lse, ws)
    o = torch.empty_like(q)
    cabf_scatter_rows(seq, op, rows, kq["perm"], o)
    if return_info:
        return o, dict(kq=kq, kk=kk, kv_count=kv_count, kv_index=kv_index, qp=qp, kp=kp, vp=vp,
                       op=op, lse=lse)
    return o
