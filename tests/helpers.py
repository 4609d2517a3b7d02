"""Shared test helpers: tiny workloads and fp64 views.  Holds no attention arithmetic."""
from __future__ import annotations

import numpy as np
import torch

from tree_verification_attention_amd import workloads as W


def tiny_workload(parents, *, B=1, Hq=2, Hkv=1, D=8, L=5, prefix_len=None, dtype=torch.float32,
                  seed=0, scale=None, peaky=0.0):
    if isinstance(parents[0], int):
        parents = [list(parents)] * B
    return W.make_workload("t", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           max_prefix_len=L, parents=parents, prefix_len=prefix_len,
                           dtype=dtype, seed=seed, scale=scale, peaky_frac=peaky)


def f64(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float64)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()
