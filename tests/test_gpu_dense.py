"""GPU parity of the single-pass masked baseline (hta_dense_mask, hta_verify_dense).

Bars: the explicit mask bit-exact against the one assembled from the oracle's ancestor masks
and the prefix lengths; outputs within the verification bars (out 2e-3, lse 1e-3) of the
oracle -- the tree definition (oracle.rows) for tree-derived masks, the general masked
attention oracle for arbitrary masks (rows that see nothing: out exactly 0, lse -inf).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

from test_gpu_parity import LSE_TOL, OUT_TOL, check_rows, to_dev

pytestmark = pytest.mark.gpu


def _expected_mask(w: W.Workload) -> np.ndarray:
    """Word-major [B, Wm, T_pad] uint64 from the oracle's ancestor masks and prefix_len."""
    B, T, Lmax = w.batch, w.tree_size, w.max_prefix_len
    Wp, Wt = -(-Lmax // 64), -(-T // 64)
    T_pad = T + (T & 1)
    anc = oracle.ancestor_masks(w.parent_idx.numpy())  # [B, T, Wt]
    m = np.zeros((B, Wp + Wt, T_pad), dtype=np.uint64)
    for b in range(B):
        L = int(w.prefix_len[b])
        for wd in range(Wp):
            n = L - 64 * wd
            m[b, wd, :T] = np.uint64(0) if n <= 0 else (
                np.uint64(0xFFFFFFFFFFFFFFFF) if n >= 64 else np.uint64((1 << n) - 1))
        m[b, Wp:, :T] = anc[b].T
    return m


def _run_dense(w: W.Workload, mask=None):
    t = to_dev(w)
    out, lse, mask = hta.verify_dense(t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"],
                                      t["v_tree"], t["parent_idx"], t["prefix_len"],
                                      scale=w.scale, mask=mask)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy(), mask


CASES = [
    ("llama3_8b_32k", None),
    ("vicuna7b_b8", None),
    ("qwq32b_tree_16k", None),
    ("qwq32b_chain5_4k", None),
]


@pytest.mark.parametrize("name", [c[0] for c in CASES])
def test_dense_matches_oracle_on_the_configs(name):
    w = W.by_name(name)
    out, lse, mask = _run_dense(w)
    got = mask.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, _expected_mask(w))
    check_rows(w, out, lse, n_rows=40, seed=5)


@pytest.mark.parametrize("D,Hq,Hkv,T,L", [(64, 8, 8, 7, 300), (128, 20, 4, 65, 1000),
                                          (128, 4, 1, 256, 130), (64, 8, 2, 1, 0)])
def test_dense_small_shapes_all_rows(D, Hq, Hkv, T, L):
    gen = torch.Generator().manual_seed(80 + T)
    par = [W.random_forest(T, gen) for _ in range(2)]
    w = W.make_workload("dense_small", batch=2, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                        max_prefix_len=max(L, 1), parents=par, prefix_len=[L, L // 3],
                        peaky_frac=0.05, seed=81)
    out, lse, mask = _run_dense(w)
    assert np.array_equal(mask.cpu().numpy().view(np.uint64), _expected_mask(w))
    check_rows(w, out, lse)


def test_dense_agrees_with_the_hybrid_step():
    w = W.llama3_8b(32768)
    out_d, lse_d, _ = _run_dense(w)
    t = to_dev(w)
    out_h, lse_h = hta.verify(t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                              t["parent_idx"], t["prefix_len"], scale=w.scale)
    torch.cuda.synchronize()
    assert float(np.max(np.abs(out_d - out_h.cpu().double().numpy()))) <= OUT_TOL
    assert float(np.max(np.abs(lse_d - lse_h.cpu().double().numpy()))) <= LSE_TOL


def test_dense_arbitrary_masks_against_masked_attention():
    """Random explicit masks (not tree-shaped), prefix bits past prefix_len set on purpose
    (they must stay invisible), and rows that see no key at all."""
    gen = torch.Generator().manual_seed(90)
    B, Hq, Hkv, D, T, Lmax = 2, 8, 2, 128, 40, 700
    par = [W.random_forest(T, gen) for _ in range(B)]
    w = W.make_workload("dense_rand", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                        max_prefix_len=Lmax, parents=par, prefix_len=[700, 450], seed=91)
    Wp, Wt = -(-Lmax // 64), -(-T // 64)
    rng = np.random.default_rng(92)
    bits = rng.random((B, T, Wp * 64 + Wt * 64)) < 0.3
    bits[:, 3, :] = False  # node 3 sees nothing
    m = np.zeros((B, Wp + Wt, T), dtype=np.uint64)
    for wd in range(Wp + Wt):
        for k in range(64):
            m[:, wd, :] |= bits[:, :, 64 * wd + k].astype(np.uint64) << np.uint64(k)
    mask = torch.from_numpy(m.view(np.int64)).cuda()
    out, lse, _ = _run_dense(w, mask=mask)
    G = Hq // Hkv
    for b in range(B):
        L = int(w.prefix_len[b])
        for h in range(Hq):
            g = h // G
            k = torch.cat([w.k_prefix[b, g, :L], w.k_tree[b, g]]).double().numpy()
            v = torch.cat([w.v_prefix[b, g, :L], w.v_tree[b, g]]).double().numpy()
            vis = np.concatenate([bits[b, :, :L], bits[b, :, Wp * 64:Wp * 64 + T]], axis=1)
            ro, rl = oracle.masked_attention(w.q[b, :, h].double().numpy(), k, v, vis, w.scale)
            empty = np.isneginf(rl)
            assert empty[3] and (out[b, 3, h] == 0).all() and np.isneginf(lse[b, h, 3])
            assert np.abs(out[b, ~empty, h] - ro[~empty]).max() <= OUT_TOL
            assert np.abs(lse[b, h, ~empty] - rl[~empty]).max() <= LSE_TOL


def test_dense_mask_of_a_rejected_tree_is_empty():
    gen = torch.Generator().manual_seed(93)
    par = [W.level_tree((2, 4), gen) for _ in range(2)]
    par[1][5] = 5
    w = W.make_workload("dense_bad", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                        max_prefix_len=200, parents=par, seed=94)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    mask = torch.full(hta.dense_mask_shape(desc), -1, dtype=torch.int64, device="cuda")
    ws = hta.new_workspace(desc, "cuda")
    hta.hta_dense_mask(desc, t["parent_idx"], t["prefix_len"], mask, ws)
    assert hta.hta_get_device_status(desc, ws) == (6, 1)
    m = mask.cpu().numpy().view(np.uint64)
    assert (m[1] == 0).all() and (m[0] != 0).any()
