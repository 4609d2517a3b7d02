"""Inputs outside the range the bf16 path supports are loud, never silently wrong.

The prefix pass (and the standalone tree pass) feed V to the PV product as fp16, so a bf16 V
value beyond 65504 cannot be represented there.  Such a value makes every output row that
sees it NaN, and the call records HTA_ERR_NONFINITE for its sequence in the workspace status.
The fused tree part of hta_verify runs in fp32 and takes such tree values exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

from test_gpu_parity import _log, check_rows, oracle_rows, to_dev

pytestmark = pytest.mark.gpu

NONFINITE = 10
BIG = 70144.0  # a bf16 value beyond the fp16 range (70000 rounds to it)


def _workload(seed=5):
    gen = torch.Generator().manual_seed(seed)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(2)]
    return W.make_workload("range", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                           max_prefix_len=1000, parents=par, prefix_len=[1000, 800], seed=seed,
                           peaky_frac=0.02, dtype=torch.bfloat16)


def _verify(w, t, desc, ws):
    B, T, Hq, D = w.q.shape
    out = torch.empty(B, T, Hq, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
    hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                   t["parent_idx"], t["prefix_len"], out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def test_prefix_v_beyond_fp16_is_reported_and_nan():
    w = _workload()
    assert float(torch.tensor(BIG).to(torch.bfloat16)) == BIG
    w.v_prefix[1, 0, 517, 9] = BIG  # sequence 1, KV head 0 (query heads 0..3), a valid key
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    ws = hta.new_workspace(desc, "cuda")
    out, lse = _verify(w, t, desc, ws)
    _log(f"  status after planting |v| = {BIG}: {hta.hta_get_device_status(desc, ws)}")
    assert hta.hta_get_device_status(desc, ws) == (NONFINITE, 1)
    # every row of (sequence 1, KV head 0) sees the key: NaN; every other row is exact
    assert np.all(np.isnan(out[1, :, 0:4])) and np.all(np.isnan(lse[1, 0:4]))
    rest = np.ones(out.shape[:3], bool)
    rest[1, :, 0:4] = False
    assert np.all(np.isfinite(out[rest]))
    b, i, h = np.nonzero(rest)
    ro, rl = oracle_rows(w, b, h, i)
    assert float(np.max(np.abs(out[b, i, h] - ro))) <= 2e-3
    assert float(np.max(np.abs(lse[b, h, i] - rl))) <= 1e-3
    # the status words are cleared by the next call: a clean input reports nothing
    w.v_prefix[1, 0, 517, 9] = 0.5
    t = to_dev(w)
    out, lse = _verify(w, t, desc, ws)
    assert hta.hta_get_device_status(desc, ws) == (0, -1)
    check_rows(w, out, lse)


def test_big_tree_v_is_exact_in_the_fused_step_and_reported_unfused():
    w = _workload(6)
    w.v_tree[0, 1, 3, 5] = BIG  # node 3 of sequence 0, KV head 1 (a level-0 node)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    ws = hta.new_workspace(desc, "cuda")
    out, lse = _verify(w, t, desc, ws)
    assert hta.hta_get_device_status(desc, ws) == (0, -1)
    B, T, Hq, D = w.q.shape
    ids = np.arange(B * T * Hq)
    b, h, i = ids // (T * Hq), ids % Hq, (ids // Hq) % T
    ro, rl = oracle_rows(w, b, h, i)
    _, rl_tree = oracle_rows(w, b, h, i, oracle.PART_TREE)
    go = out[b, i, h]
    # The tree part enters with a weight relative to the prefix part whose log-sum-exp is
    # within 2^-11 of exact (fp16 probabilities), so its contribution -- at most the row's
    # tree share times |v| -- carries up to that relative error: with |v| = 7e4 the bar is
    # 2e-3 plus 1e-3 of (tree share x |v|).
    share = np.exp(rl_tree - rl)
    bar = 2e-3 + 1e-3 * share * BIG
    err = np.abs(go - ro).max(axis=1)
    _log(f"  fused step with |v_tree| = {BIG}: max |out - oracle| = {float(err.max()):.3e}, "
         f"worst err / bar = {float((err / bar).max()):.3f}, "
         f"max |lse| err {float(np.max(np.abs(lse[b, h, i] - rl))):.3e}")
    assert np.all(np.isfinite(go))
    assert np.all(err <= bar)
    assert float(np.max(np.abs(lse[b, h, i] - rl))) <= 1e-3
    # the unfused path takes the tree V as fp16: the affected rows are NaN and reported
    hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
    hta.hta_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                          t["prefix_len"], ws)
    o2 = torch.empty(B, T, Hq, D, dtype=torch.float32, device="cuda")
    l2 = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
    hta.hta_merge(desc, t["prefix_len"], True, o2, l2, ws)
    torch.cuda.synchronize()
    assert hta.hta_get_device_status(desc, ws) == (NONFINITE, 0)
    o2 = o2.cpu().numpy()
    assert np.isnan(o2[0, 3, 4:8]).all()  # node 3 itself, query heads of KV head 1
    assert np.isfinite(o2[1]).all() and np.isfinite(o2[0, :, 0:4]).all()
    # the rows the big value does not reach stay exact: a non-finite row recorded in the
    # sequence's status word by the merge must not reject the sequence's other rows
    fin = np.isfinite(o2[b, i, h]).all(axis=1)
    assert fin.sum() >= B * T * Hq - T * (Hq // w.num_kv_heads)
    assert float(np.max(np.abs(o2[b, i, h][fin] - ro[fin]))) <= 2e-3


def test_cross_attention_reports_big_cache_values():
    w = _workload(7)
    w.v_prefix[0, 1, 10, 0] = -BIG
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    ws = hta.new_workspace(desc, "cuda")
    out, lse = hta.cross_attention(t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"],
                                   scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert hta.hta_get_device_status(desc, ws) == (NONFINITE, 0)
    out = out.cpu().numpy()
    assert np.isnan(out[0, :, 4:8]).all() and np.isfinite(out[1]).all()
