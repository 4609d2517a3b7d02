"""GPU parity on the full-size workloads (Llama-3-8B 32k / 256k, Vicuna-7B batch 8, the QwQ-32B
decode sweep), in the launch configuration the benchmark times (automatic chunking).

The oracle computes every query row of every workload (its rows spread over the host's
cores); the GPU computes every row, which must all be finite and within the bars.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tree_verification_attention_amd import workloads as W

from test_gpu_parity import check_rows, run_gpu, _log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama3_8b_32k", "llama3_8b_256k", "vicuna7b_b8"])
def test_config_every_row(name):
    _log(f"config {name}")
    w = W.by_name(name)
    out, lse = run_gpu(w)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check_rows(w, out, lse, seed=1)


@pytest.mark.parametrize("prefix", W.QWQ_PREFIXES)
@pytest.mark.parametrize("chain", [False, True])
def test_qwq_sweep(prefix, chain):
    w = W.qwq_32b(prefix, chain=chain)
    _log(f"config {w.name}")
    out, lse = run_gpu(w)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check_rows(w, out, lse, seed=2)


def test_tiny_fp32_config():
    """fp32 inputs run exact fp32 arithmetic: far inside the bf16 bars."""
    w = W.tiny()
    assert w.dtype == torch.float32
    _log(f"config {w.name}")
    out, lse = run_gpu(w)
    # fp32 arithmetic; outputs also carry the 16-bit storage of the split-K partials
    check_rows(w, out, lse, out_tol=1e-4, lse_tol=2e-5)
