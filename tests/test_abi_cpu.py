"""Host-side checks of the C ABI: the library loads, exports every function
include/cabf.h declares, derives the same geometry as the oracle, and rejects
bad arguments before launching anything.

The rejection cases pass dummy pointers, so they must never reach a launch;
each case breaks exactly one rule. They are skipped where a GPU is present
(there the GPU tests exercise real calls).
"""
import ctypes
import os
import re

import pytest
import torch

import content_adaptive_block_fractal_amd as cabf
import oracle
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cabf.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cabf_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(cabf.EXPORTED), names
    lib = ctypes.CDLL(cabf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_library_exports_only_the_c_abi():
    """Built with hidden visibility: the dynamic symbols the library defines
    are exactly the functions the header declares."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", cabf.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    assert funcs == set(declared_functions()), sorted(funcs ^ set(declared_functions()))


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_geometry_matches_oracle_grid(name):
    w = WORKLOADS[name]
    g = cabf.Geom(w.batch, w.heads, w.head_dim, w.T, w.H, w.W, w.P)
    s = g.sizes()
    o = oracle.Grid(w.T, w.H, w.W, w.P)
    assert s == dict(tokens_raster=o.n_valid, tokens_padded=o.N, n_blocks=o.nb, Hp=o.Hp, Wp=o.Wp)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(cabf.cabf_status_string(code), str)
    assert cabf.cabf_status_string(-3) == "workspace too small"


def test_workspace_bytes():
    g = cabf.Geom(1, 2, 64, 4, 16, 16, 8)
    n = cabf.cabf_mask_workspace_bytes(g)
    nb = 16
    assert n >= 2 * 2 * nb * 64 * 4 + 2 * nb * nb * 4
    assert cabf.cabf_mask_workspace_bytes(cabf.Geom(1, 2, 64, 4, 16, 16, 4)) == 0
    assert cabf.cabf_mask_workspace_bytes(cabf.Geom(1, 2, 96, 4, 16, 16, 8)) == 0


no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="dummy-pointer checks run host-only")
L = cabf._lib
G = cabf._Geom
DUMMY = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: every case below fails validation
DUMMY2 = ctypes.c_void_p(0x200000)
NULL = None


def geom(**kw):
    base = dict(batch=1, heads=2, head_dim=64, T=4, H=16, W=16, P=8)
    base.update(kw)
    return ctypes.byref(G(*base.values()))


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(P=4), cabf.CABF_EUNSUPPORTED), (dict(head_dim=96), cabf.CABF_EUNSUPPORTED),
    (dict(T=0), cabf.CABF_EINVAL), (dict(heads=-1), cabf.CABF_EINVAL), (dict(W=0), cabf.CABF_EINVAL),
])
def test_bad_geometry_rejected(kw, code):
    assert L.cabf_permute(geom(**kw), 0, DUMMY, DUMMY, DUMMY, DUMMY2, DUMMY2, DUMMY2, NULL) == code
    assert L.cabf_unpermute(geom(**kw), 0, DUMMY, DUMMY2, NULL) == code
    assert L.cabf_geom_sizes(geom(**kw), None, None, None, None, None) == code


@no_gpu
def test_permute_argument_checks():
    g = geom()
    assert L.cabf_permute(g, 0, DUMMY, NULL, NULL, NULL, NULL, NULL, NULL) == cabf.CABF_EINVAL
    assert L.cabf_permute(g, 5, DUMMY, NULL, NULL, DUMMY2, NULL, NULL, NULL) == cabf.CABF_EINVAL
    mis = ctypes.c_void_p(0x100002)
    assert L.cabf_permute(g, 0, mis, NULL, NULL, DUMMY2, NULL, NULL, NULL) == cabf.CABF_EINVAL
    assert L.cabf_permute(g, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == cabf.CABF_OK
    assert L.cabf_unpermute(g, 0, NULL, DUMMY2, NULL) == cabf.CABF_EINVAL


@no_gpu
def test_mask_argument_checks():
    g = geom()
    need = L.cabf_mask_workspace_bytes(g)
    sta_bad = ctypes.byref(cabf._Sta(1, -1, 1, 1))
    def call(**kw):
        a = dict(qp=DUMMY, kp=DUMMY, scale=0.125, thr=0.2, sta=None, cnt=DUMMY2, idx=DUMMY2,
                 prob=None, ws=ctypes.c_void_p(0x300000), wsb=need, dt=0)
        a.update(kw)
        return L.cabf_build_block_mask(g, a["dt"], a["qp"], a["kp"], a["scale"], a["thr"], a["sta"],
                                       a["cnt"], a["idx"], a["prob"], a["ws"], a["wsb"], NULL)
    assert call(qp=NULL) == cabf.CABF_EINVAL
    assert call(cnt=NULL) == cabf.CABF_EINVAL
    assert call(ws=NULL) == cabf.CABF_EINVAL
    assert call(scale=0.0) == cabf.CABF_EINVAL
    assert call(scale=float("nan")) == cabf.CABF_EINVAL
    assert call(thr=-0.1) == cabf.CABF_EINVAL
    assert call(thr=1.5) == cabf.CABF_EINVAL
    assert call(thr=float("nan")) == cabf.CABF_EINVAL
    assert call(sta=sta_bad) == cabf.CABF_EINVAL
    assert call(wsb=need - 1) == cabf.CABF_EWORKSPACE
    assert call(ws=ctypes.c_void_p(0x300010)) == cabf.CABF_EINVAL   # not 256-byte aligned
    assert call(dt=3) == cabf.CABF_EINVAL


@no_gpu
def test_noalloc_mask_argument_checks():
    """The no-allocation mask rejects bad arguments, and a geometry whose one
    (batch, head) pair needs more than the static scratch, before any launch."""
    def call(g=None, **kw):
        a = dict(qp=DUMMY, scale=0.125, thr=0.2, cnt=DUMMY2, dt=0)
        a.update(kw)
        return L.cabf_build_block_mask_noalloc(geom() if g is None else g, a["dt"], a["qp"], DUMMY,
                                               a["scale"], a["thr"], None, a["cnt"], DUMMY2,
                                               None, NULL)
    assert call(qp=NULL) == cabf.CABF_EINVAL
    assert call(cnt=NULL) == cabf.CABF_EINVAL
    assert call(scale=0.0) == cabf.CABF_EINVAL
    assert call(thr=2.0) == cabf.CABF_EINVAL
    assert call(dt=3) == cabf.CABF_EINVAL
    assert call(geom(P=4)) == cabf.CABF_EUNSUPPORTED
    # nb = 125 * 5 * 8 = 5000 blocks at head_dim 128: 2*5000*128 + 5000*5056 floats > 96 MiB
    big = geom(head_dim=128, T=125, H=40, W=64)
    assert (2 * 5000 * 128 + 5000 * 5056) * 4 > cabf.NOALLOC_SCRATCH_BYTES
    assert call(big) == cabf.CABF_EWORKSPACE
    assert call(geom(head_dim=128, T=9000, H=8, W=8)) == cabf.CABF_EUNSUPPORTED   # nb > 8192


@no_gpu
def test_topk_and_sta_mask_argument_checks():
    g = geom()
    need = L.cabf_mask_workspace_bytes(g)
    ws = ctypes.c_void_p(0x300000)
    def topk(k, **kw):
        a = dict(qp=DUMMY, scale=0.125, wsb=need)
        a.update(kw)
        return L.cabf_build_block_mask_topk(g, 0, a["qp"], DUMMY, a["scale"], k, None, DUMMY2,
                                            DUMMY2, None, ws, a["wsb"], NULL)
    assert topk(0) == cabf.CABF_EINVAL
    assert topk(-3) == cabf.CABF_EINVAL
    assert topk(4, qp=NULL) == cabf.CABF_EINVAL
    assert topk(4, scale=-1.0) == cabf.CABF_EINVAL
    assert topk(4, wsb=need - 1) == cabf.CABF_EWORKSPACE
    on = ctypes.byref(cabf._Sta(1, 1, 1, 1))
    off = ctypes.byref(cabf._Sta(0, 1, 1, 1))
    neg = ctypes.byref(cabf._Sta(1, 0, -1, 0))
    assert L.cabf_build_sta_mask(g, None, DUMMY2, DUMMY2, NULL) == cabf.CABF_EINVAL
    assert L.cabf_build_sta_mask(g, off, DUMMY2, DUMMY2, NULL) == cabf.CABF_EINVAL
    assert L.cabf_build_sta_mask(g, neg, DUMMY2, DUMMY2, NULL) == cabf.CABF_EINVAL
    assert L.cabf_build_sta_mask(g, on, NULL, DUMMY2, NULL) == cabf.CABF_EINVAL
    assert L.cabf_build_sta_mask(g, on, ctypes.c_void_p(0x200002), DUMMY2, NULL) == cabf.CABF_EINVAL
    assert L.cabf_build_sta_mask(geom(P=4), on, DUMMY2, DUMMY2, NULL) == cabf.CABF_EUNSUPPORTED


@no_gpu
def test_semantic_permutation_argument_checks():
    seq = ctypes.byref(cabf._Seq(1, 2, 128, 1000))
    ws = ctypes.c_void_p(0x300000)
    need = L.cabf_kmeans_workspace_bytes(seq, 40)
    assert need > 0
    assert L.cabf_kmeans_workspace_bytes(seq, 0) == 0
    assert L.cabf_kmeans_workspace_bytes(seq, 1001) == 0
    assert L.cabf_kmeans_workspace_bytes(ctypes.byref(cabf._Seq(1, 2, 96, 1000)), 4) == 0
    def km(**kw):
        a = dict(seq=seq, dt=0, x=DUMMY, C=40, init=DUMMY2, iters=3, wsb=need)
        a.update(kw)
        return L.cabf_kmeans(a["seq"], a["dt"], a["x"], a["C"], a["init"], a["iters"], DUMMY2,
                             DUMMY2, DUMMY2, DUMMY2, DUMMY2, ws, a["wsb"], NULL)
    assert km(dt=1) == cabf.CABF_EUNSUPPORTED
    assert km(x=NULL) == cabf.CABF_EINVAL
    assert km(C=0) == cabf.CABF_EINVAL
    assert km(iters=-1) == cabf.CABF_EINVAL
    assert km(wsb=need - 1) == cabf.CABF_EWORKSPACE
    assert km(seq=ctypes.byref(cabf._Seq(1, 2, 128, 0))) == cabf.CABF_EINVAL
    assert km(seq=ctypes.byref(cabf._Seq(1, 2, 128, 1 << 24))) == cabf.CABF_EUNSUPPORTED
    assert L.cabf_gather_rows(seq, 0, DUMMY, DUMMY2, DUMMY2, 999, NULL) == cabf.CABF_EINVAL
    assert L.cabf_gather_rows(seq, 0, ctypes.c_void_p(0x100008), DUMMY2, DUMMY2, 1064, NULL) == cabf.CABF_EINVAL
    assert L.cabf_scatter_rows(seq, 2, DUMMY, 1064, DUMMY2, DUMMY2, NULL) == cabf.CABF_EINVAL
    sneed = L.cabf_cluster_select_workspace_bytes(seq, 10, 40)
    def sel(**kw):
        a = dict(cq=10, ck=40, scale=0.1, top_p=0.9, wsb=sneed)
        a.update(kw)
        return L.cabf_cluster_select(seq, a["cq"], a["ck"], DUMMY, DUMMY, DUMMY2, a["scale"],
                                     a["top_p"], DUMMY2, DUMMY2, None, ws, a["wsb"], NULL)
    assert sel(top_p=0.0) == cabf.CABF_EINVAL
    assert sel(top_p=1.5) == cabf.CABF_EINVAL
    assert sel(scale=0.0) == cabf.CABF_EINVAL
    assert sel(ck=0) == cabf.CABF_EINVAL
    assert sel(ck=9000) == cabf.CABF_EUNSUPPORTED
    assert sel(wsb=sneed - 1) == cabf.CABF_EWORKSPACE
    aneed = L.cabf_cluster_attention_workspace_bytes(seq, 10, 40)
    def att(**kw):
        a = dict(dt=0, cq=10, ck=40, qp=DUMMY, wsb=aneed)
        a.update(kw)
        return L.cabf_cluster_attention(seq, a["dt"], a["cq"], a["ck"], a["qp"], DUMMY, DUMMY,
                                        DUMMY2, DUMMY2, DUMMY2, DUMMY2, 0.1, DUMMY2, None, ws,
                                        a["wsb"], NULL)
    assert att(dt=1) == cabf.CABF_EUNSUPPORTED
    assert att(qp=NULL) == cabf.CABF_EINVAL
    assert att(cq=1001) == cabf.CABF_EINVAL
    assert att(wsb=aneed - 1) == cabf.CABF_EWORKSPACE


@no_gpu
def test_mask_rejects_rows_longer_than_supported():
    g = geom(T=129, H=64, W=64)      # 129 * 64 blocks > 8192
    assert L.cabf_build_block_mask(g, 0, DUMMY, DUMMY, 0.1, 0.2, None, DUMMY2, DUMMY2, None,
                                   ctypes.c_void_p(0x300000), 1 << 40, NULL) == cabf.CABF_EUNSUPPORTED


@no_gpu
def test_attention_argument_checks():
    g = geom()
    def call(**kw):
        a = dict(q=DUMMY, k=DUMMY, v=DUMMY, cnt=DUMMY2, idx=DUMMY2, scale=0.125, op=DUMMY2,
                 lse=None, dt=0, flags=0)
        a.update(kw)
        return L.cabf_bsa_forward(g, a["dt"], a["q"], a["k"], a["v"], a["cnt"], a["idx"],
                                  a["scale"], a["op"], a["lse"], a["flags"], NULL)
    for key in ("q", "k", "v", "cnt", "idx", "op"):
        assert call(**{key: NULL}) == cabf.CABF_EINVAL, key
    assert call(scale=-1.0) == cabf.CABF_EINVAL
    assert call(scale=float("inf")) == cabf.CABF_EINVAL
    assert call(lse=ctypes.c_void_p(0x400002)) == cabf.CABF_EINVAL
    assert call(dt=2) == cabf.CABF_EINVAL
    assert call(flags=2) == cabf.CABF_EINVAL
    assert call(flags=cabf.BSA_DETERMINISTIC | 4) == cabf.CABF_EINVAL


@no_gpu
def test_fused_entry_argument_checks():
    g = geom()
    need = L.cabf_mask_workspace_bytes(g)
    ws = ctypes.c_void_p(0x300000)
    def pp(**kw):
        a = dict(dt=0, q=DUMMY, k=DUMMY, v=NULL, qp=DUMMY2, kp=DUMMY2, vp=NULL, ws=ws, wsb=need)
        a.update(kw)
        return L.cabf_permute_pool(g, a["dt"], a["q"], a["k"], a["v"], a["qp"], a["kp"], a["vp"],
                                   a["ws"], a["wsb"], NULL)
    assert pp(q=NULL, qp=NULL) == cabf.CABF_EINVAL          # q and k are required
    assert pp(k=NULL, kp=NULL) == cabf.CABF_EINVAL
    assert pp(v=DUMMY) == cabf.CABF_EINVAL                  # v without vp
    assert pp(ws=NULL) == cabf.CABF_EINVAL
    assert pp(ws=ctypes.c_void_p(0x300040)) == cabf.CABF_EINVAL
    assert pp(wsb=need - 1) == cabf.CABF_EWORKSPACE
    assert pp(dt=4) == cabf.CABF_EINVAL
    assert L.cabf_permute_pool(geom(T=129, H=64, W=64), 0, DUMMY, DUMMY, NULL, DUMMY2, DUMMY2, NULL,
                               ws, 1 << 40, NULL) == cabf.CABF_EUNSUPPORTED
    def mp(**kw):
        a = dict(scale=0.125, thr=0.2, k=0, cnt=DUMMY2, ws=ws, wsb=need)
        a.update(kw)
        return L.cabf_build_block_mask_pooled(g, a["scale"], a["thr"], a["k"], None, a["cnt"],
                                              DUMMY2, None, a["ws"], a["wsb"], NULL)
    assert mp(k=-1) == cabf.CABF_EINVAL
    assert mp(thr=1.2) == cabf.CABF_EINVAL
    assert mp(scale=0.0) == cabf.CABF_EINVAL
    assert mp(cnt=NULL) == cabf.CABF_EINVAL
    assert mp(wsb=need - 1) == cabf.CABF_EWORKSPACE
    def sub(**kw):
        a = dict(dt=0, qb=DUMMY2, n=4, scale=0.125, flags=0, op=DUMMY2)
        a.update(kw)
        return L.cabf_bsa_forward_subset(g, a["dt"], DUMMY, DUMMY, DUMMY, DUMMY2, DUMMY2, a["qb"],
                                         a["n"], a["scale"], a["op"], None, a["flags"], NULL)
    assert sub(dt=1) == cabf.CABF_EUNSUPPORTED
    assert sub(dt=3) == cabf.CABF_EINVAL
    assert sub(n=-1) == cabf.CABF_EINVAL
    assert sub(qb=NULL) == cabf.CABF_EINVAL
    assert sub(qb=NULL, n=0) == cabf.CABF_OK                # nothing to do
    assert sub(qb=ctypes.c_void_p(0x200002)) == cabf.CABF_EINVAL
    assert sub(op=NULL) == cabf.CABF_EINVAL
    assert sub(flags=8) == cabf.CABF_EINVAL
    assert sub(scale=float("nan")) == cabf.CABF_EINVAL


@no_gpu
def test_probe_library_is_separate_and_checks_arguments():
    """The benchmark's matrix-core probe lives in its own library, outside the C ABI."""
    from content_adaptive_block_fractal_amd import peak_probe
    lib = peak_probe._load()
    assert not hasattr(L, "cabf_mfma_peak_probe")
    assert lib.probe_mfma_peak(0, 10, DUMMY2, NULL) == -1
    assert lib.probe_mfma_peak(4, 0, DUMMY2, NULL) == -1
    assert lib.probe_mfma_peak(4, 10, NULL, NULL) == -1
    assert lib.probe_mfma_peak(4, 10, ctypes.c_void_p(0x200002), NULL) == -1
