"""Workload shapes of the block-sparse video attention path.

Each entry is a latent video grid and head layout of a video diffusion
transformer's self-attention layer, with the seeded input recipe of
``synth.fields``. P = 8 (64-token blocks) throughout.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    P: int
    dtype: str            # "f32" or "bf16"
    amplitude: float      # Fourier-signal amplitude of the generator
    sparsity: tuple = ()  # target block sparsities (thr calibrated to hit them)
    thr: float | None = None
    sta: tuple | None = None   # (dt, dy, dx) window or None
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 4, 16, 16, 8, "f32", 1.0, thr=0.2, sta=(1, 1, 1),
                     notes="4 frames x 16x16, N=1024, 16 blocks; oracle finishes in about a second"),
    "wan1.3b-480p": Workload("wan1.3b-480p", 1, 12, 128, 21, 30, 52, 8, "bf16", 0.7, sparsity=(0.80,),
                             notes="21 x 30x52 padded to 32x56, N=37,632, 588 blocks"),
    "wan14b-720p": Workload("wan14b-720p", 1, 40, 128, 21, 45, 80, 8, "bf16", 0.7,
                            sparsity=(0.80, 0.90), sta=(1, 1, 1),
                            notes="21 x 45x80 padded to 48x80, N=80,640, 1,260 blocks; run with and without the window"),
    "hunyuan-241f-768p": Workload("hunyuan-241f-768p", 1, 24, 128, 61, 48, 84, 8, "bf16", 0.7,
                                  sparsity=(0.85,),
                                  notes="61 x 48x84 padded to 48x88, N=257,664, 4,026 blocks"),
}


@dataclass(frozen=True)
class SemanticWorkload:
    """Semantic-permutation (k-means + top-p) variant: n tokens per head, Q and
    K from a Gaussian mixture (``synth.gaussian_mixture_qk``), V standard
    normal, seeded k-means initial indices (``synth.kmeans_init_indices``)."""
    name: str
    heads: int
    head_dim: int
    n: int
    cq: int               # query clusters
    ck: int               # key clusters
    iters: int            # Lloyd iterations
    top_p: float
    components: int
    spread: float
    amplitude: float
    notes: str = ""


SEMANTIC_WORKLOADS = {
    "svg2-tiny": SemanticWorkload("svg2-tiny", 2, 128, 3000, 12, 40, 5, 0.9, 10, 0.15, 8.5,
                                  notes="oracle finishes in seconds"),
    "svg2-wan14b-720p": SemanticWorkload(
        "svg2-wan14b-720p", 40, 128, 21 * 45 * 80, 100, 500, 10, 0.9, 64, 0.15, 8.5,
        notes="Wan-14B 720p token count (21 x 45x80 = 75,600), 100 query / 500 key clusters, "
              "10 Lloyd iterations, top-p 0.9; amplitude 8.5 puts the kept density near 16%"),
}
