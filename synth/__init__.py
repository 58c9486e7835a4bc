"""Seeded synthetic inputs for the block-sparse video attention path.

This package holds input synthesis only (random fields, shapes and sizes of
the workloads); it contains none of the attention method's arithmetic. Both
the CPU oracle's callers and the HIP path's callers draw their inputs here.
"""
from .fields import (fourier_video_qkv, gaussian_video_qkv, round_to_bf16,  # noqa: F401
                     gaussian_mixture_qk, kmeans_init_indices)
from .workloads import WORKLOADS, Workload, SEMANTIC_WORKLOADS, SemanticWorkload  # noqa: F401
