"""The allocation-free entry point (hta_verify_noalloc) against hta_verify.

hta_verify_noalloc runs the same launches on the library's static per-GPU scratch instead of
a caller workspace.  Two calls in a row on one GPU -- the second with a smaller input, so the
scratch still holds the first call's larger contents -- must give exactly hta_verify's bits,
and the per-sequence device flags must reach the caller's status buffer.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

from test_gpu_parity import _log, check_rows, to_dev

pytestmark = pytest.mark.gpu


def _inputs(name, B, Hq, Hkv, L, plen, seed, bad_tree=None):
    gen = torch.Generator().manual_seed(seed)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(B)]
    if bad_tree is not None:
        par[bad_tree][10] = 40  # a parent after its child: invalid
    return W.make_workload(name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                           max_prefix_len=L, parents=par, prefix_len=plen, seed=seed,
                           peaky_frac=0.02, dtype=torch.bfloat16)


def _both(w):
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    B, T, Hq, D = w.q.shape
    ref_o, ref_l = hta.verify(t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                              t["parent_idx"], t["prefix_len"], scale=w.scale)
    out = torch.full((B, T, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, T), 7.0, dtype=torch.float32, device="cuda")
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    hta.hta_verify_noalloc(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                           t["parent_idx"], t["prefix_len"], out, lse, status)
    torch.cuda.synchronize()
    return ref_o, ref_l, out, lse, status


def test_noalloc_matches_verify_on_consecutive_calls():
    # a large call, then a smaller one on the same scratch
    big = _inputs("noalloc_big", B=1, Hq=32, Hkv=8, L=32768, plen=[32768], seed=11)
    small = _inputs("noalloc_small", B=2, Hq=8, Hkv=2, L=700, plen=[700, 333], seed=12)
    for w in (big, small):
        _log(f"noalloc {w.name}")
        ref_o, ref_l, out, lse, status = _both(w)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), w.name
        assert torch.all(status == 0)
        check_rows(w, out.cpu().double().numpy(), lse.cpu().double().numpy(), n_rows=300)


def test_noalloc_reports_device_errors_in_the_callers_status():
    w = _inputs("noalloc_bad", B=3, Hq=8, Hkv=2, L=500, plen=[500, 200, 600], seed=13,
                bad_tree=1)
    ref_o, ref_l, out, lse, status = _both(w)
    # sequence 1: invalid tree; sequence 2: prefix_len beyond the cache
    assert status.cpu().tolist() == [0, 1, 2]
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
    assert torch.equal(out[0], ref_o[0]) and torch.equal(lse[0], ref_l[0])
    # the same call without a status buffer still NaN-fills the rows
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    out2 = torch.zeros_like(out)
    lse2 = torch.zeros_like(lse)
    hta.hta_verify_noalloc(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                           t["parent_idx"], t["prefix_len"], out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out2[0], ref_o[0]) and torch.isnan(out2[1:]).all()
