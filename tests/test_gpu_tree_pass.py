"""GPU parity of the standalone tree pass: hta_tree_partials runs the masked matrix-core tree
kernel (ancestor bitmasks, bf16 scores, fp16 probabilities) and leaves its partial in slot S
of the workspace.  That partial is compared element by element with the oracle's tree-only
attention of every row, then the unfused path (prefix partials, tree partial, plain merge)
with the oracle's full answer.  Bars: 2e-3 on outputs, 1e-3 on log-sum-exps.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

from test_gpu_parity import LSE_TOL, OUT_TOL, _log, check_rows, to_dev

pytestmark = pytest.mark.gpu

# (head_dim, query heads per KV head): every tree size runs each pair
DG = [(64, 1), (128, 4), (128, 5), (64, 16)]


def _parents(kind: str, T: int, B: int, seed: int):
    gen = torch.Generator().manual_seed(seed)
    if kind == "forest":
        return [W.random_forest(T, gen) for _ in range(B)]
    if kind == "chain":
        return [W.chain_tree(T)] * B
    return [W.star_tree(T)] * B


def _all_rows(w: W.Workload):
    B, T, Hq = w.batch, w.tree_size, w.num_q_heads
    ids = np.arange(B * T * Hq)
    return ids // (T * Hq), ids % Hq, (ids // Hq) % T


@pytest.mark.parametrize("kind", ["forest", "chain", "star"])
@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 68, 130, 256])
def test_tree_partial_matches_oracle(T, kind):
    for D, G in DG:
        Hkv = 2
        B = 2
        _log(f"tree pass T={T} {kind} D={D} G={G}")
        w = W.make_workload(f"tree_{kind}_{T}_{D}_{G}", batch=B, num_q_heads=G * Hkv,
                            num_kv_heads=Hkv, head_dim=D, max_prefix_len=300,
                            parents=_parents(kind, T, B, 1000 + T), prefix_len=[300, 123],
                            seed=T * 7 + G, peaky_frac=0.02, dtype=torch.bfloat16)
        t = to_dev(w)
        desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk=128)
        ws = hta.new_workspace(desc, "cuda")
        hta.hta_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                              t["prefix_len"], ws)
        torch.cuda.synchronize()
        assert hta.hta_get_device_status(desc, ws) == (0, -1)
        lse_p, o_p = (x.cpu().double().numpy() for x in hta.partial_views(desc, ws))
        S = hta.plan(desc).num_splits
        b, h, i = _all_rows(w)
        ro, rl = oracle.rows(w.as_numpy(), w.scale, b, h, i, oracle.PART_TREE)
        g, r = h // G, i * G + h % G
        go, gl = o_p[b, g, S, r], lse_p[b, g, S, r]
        err_o = float(np.max(np.abs(go - ro)))
        err_l = float(np.max(np.abs(gl - rl)))
        _log(f"  tree partial: rows={len(b)} max|o|={err_o:.3e} max|lse|={err_l:.3e}")
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
        assert err_o <= OUT_TOL and err_l <= LSE_TOL
        # the unfused step: prefix partials + this tree partial through the plain merge
        hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
        out = torch.empty(B, T, G * Hkv, D, dtype=torch.float32, device="cuda")
        lse = torch.empty(B, G * Hkv, T, dtype=torch.float32, device="cuda")
        hta.hta_merge(desc, t["prefix_len"], True, out, lse, ws)
        torch.cuda.synchronize()
        assert hta.hta_get_device_status(desc, ws) == (0, -1)
        check_rows(w, out.cpu().double().numpy(), lse.cpu().double().numpy())


def test_prepared_calls_match_direct_calls():
    """The prepared (checked-once) tree, prefix and merge calls enqueue exactly what the direct
    calls do: the unfused step through either path is bit-identical, also when repeated."""
    B, Hkv, G, D, T = 2, 2, 4, 128, 68
    w = W.make_workload("prepared", batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                        head_dim=D, max_prefix_len=700, prefix_len=[700, 321],
                        tree_widths=W.LONGSPEC_TREE_WIDTHS, seed=77, peaky_frac=0.02,
                        dtype=torch.bfloat16)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk=128)
    res = []
    for prepared in (False, True, True):
        ws = hta.new_workspace(desc, "cuda")
        out = torch.full((B, T, G * Hkv, D), float("nan"), device="cuda")
        lse = torch.full((B, G * Hkv, T), float("nan"), device="cuda")
        if prepared:
            hta.prepare_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                                      t["prefix_len"], ws)()
            hta.prepare_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"],
                                        t["prefix_len"], ws)()
            hta.prepare_merge(desc, t["prefix_len"], True, out, lse, ws)()
        else:
            hta.hta_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                                  t["prefix_len"], ws)
            hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"],
                                    t["prefix_len"], ws)
            hta.hta_merge(desc, t["prefix_len"], True, out, lse, ws)
        torch.cuda.synchronize()
        assert hta.hta_get_device_status(desc, ws) == (0, -1)
        res.append((out.cpu(), lse.cpu()))
    for o, l in res[1:]:
        assert torch.equal(o, res[0][0]) and torch.equal(l, res[0][1])
    check_rows(w, res[0][0].double().numpy(), res[0][1].double().numpy())
