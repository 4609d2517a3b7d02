"""GPU parity of hta_chunk_mass (each prefix chunk's and the tree's share of every query
row's attention) against the chunk-mass oracle.

Bar: absolute 2e-3 on each share.  A share is exp(l_s - l) of two log-sum-exps that each
meet the 1e-3 lse bar, so the share's relative error is at most about 2e-3 and shares are
at most 1.  Empty chunks (past prefix_len) must be exactly 0; rows sum to 1 within 1e-5;
the per-sequence scores must equal the fixed-order mean of the rows' shares.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

from test_gpu_parity import _log, sample_rows, to_dev

pytestmark = pytest.mark.gpu

MASS_TOL = 2e-3


def _run(w: W.Workload, chunk: int, fused: bool = True):
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk)
    ws = hta.new_workspace(desc, "cuda")
    B, T, Hq, D = w.q.shape
    out = torch.empty(B, T, Hq, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
    if fused:
        hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                       t["parent_idx"], t["prefix_len"], out, lse, ws)
    else:
        hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
        hta.hta_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                              t["prefix_len"], ws)
        hta.hta_merge(desc, t["prefix_len"], True, out, lse, ws)
    mass, scores = hta.chunk_mass(desc, t["prefix_len"], lse, ws)
    torch.cuda.synchronize()
    p = hta.plan(desc)
    return mass.cpu().double().numpy(), scores.cpu().double().numpy(), p


def _check(w, mass, scores, p, n_rows, seed=0):
    S = p.num_splits
    assert mass.shape == (w.batch, w.num_q_heads, w.tree_size, S + 1)
    b, h, i = sample_rows(w, n_rows, seed)
    ref = oracle.chunk_mass(w.as_numpy(), w.scale, p.chunk, S, b, h, i)
    got = mass[b, h, i]
    err = float(np.max(np.abs(got - ref)))
    _log(f"  [{w.name}] chunk {p.chunk} splits {S} rows={len(b)} max|mass-oracle|={err:.3e}")
    assert np.all(np.isfinite(got)) and err <= MASS_TOL
    assert np.array_equal(got[ref == 0], ref[ref == 0])  # empty chunks exactly 0
    np.testing.assert_allclose(mass.sum(axis=-1), 1.0, atol=1e-5)
    np.testing.assert_allclose(scores, mass.mean(axis=(1, 2)), rtol=0, atol=1e-6)
    return err


def test_tiny_fp32_all_rows():
    w = W.tiny()
    mass, scores, p = _run(w, chunk=256)
    _check(w, mass, scores, p, n_rows=10**9)


def test_llama_32k_sampled_rows():
    w = W.llama3_8b(32768)
    mass, scores, p = _run(w, chunk=1024)
    assert p.num_splits == 32
    _check(w, mass, scores, p, n_rows=48)


def test_vicuna_ragged_batch_sampled_rows():
    w = W.vicuna_7b_b8()
    mass, scores, p = _run(w, chunk=1024)
    _check(w, mass, scores, p, n_rows=48)
    # chunks past each sequence's prefix are exactly 0 for every row
    for b in range(w.batch):
        ns = -(-int(w.prefix_len[b]) // p.chunk)
        assert (mass[b, :, :, ns:p.num_splits] == 0).all()


@pytest.mark.parametrize("chunk", [64, 320])
def test_small_chunks_and_the_unfused_path_agree(chunk):
    gen = torch.Generator().manual_seed(70)
    par = [W.level_tree((3, 5, 5), gen) for _ in range(2)]
    w = W.make_workload("mass_small", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        max_prefix_len=1000, parents=par, prefix_len=[1000, 333],
                        peaky_frac=0.05, seed=71)
    m1, s1, p = _run(w, chunk=chunk, fused=True)
    m2, s2, _ = _run(w, chunk=chunk, fused=False)
    _check(w, m1, s1, p, n_rows=10**9)
    _check(w, m2, s2, p, n_rows=64, seed=1)
    assert float(np.max(np.abs(m1 - m2))) <= MASS_TOL


def test_rejected_sequence_is_nan():
    gen = torch.Generator().manual_seed(72)
    par = [W.level_tree((2, 4), gen) for _ in range(2)]
    par[1][3] = 4  # a forward pointer
    w = W.make_workload("mass_bad", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                        max_prefix_len=512, parents=par, seed=73)
    mass, scores, p = _run(w, chunk=128)
    assert np.isnan(mass[1]).all() and np.isnan(scores[1]).all()
    assert np.isfinite(mass[0]).all()
