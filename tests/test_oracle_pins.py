"""Pins of the CPU oracle against things other than itself.

The LongSpec pages print no worked example, so the oracle is pinned by brute force on
tiny inputs, by special cases that reduce to a library routine (torch's fp64 scaled dot
product attention), by closed forms and by invariants of the definition:

* a chain-shaped draft tree is ordinary causal attention over prefix + chain;
* a one-node tree is plain decode attention;
* a star tree is attention with an explicit diagonal mask on the tree block;
* merging the partial attentions of any split of the keys through their log-sum-exp
  equals unsplit attention (the aggregation the README's "Hybrid Attention Aggregation"
  performs must be exact, since the decoding is lossless);
* q = 0 gives a uniform softmax, so lse = ln(#visible keys) and out = mean of visible v;
* grouped-query attention equals multi-head attention with K/V repeated;
* renumbering the tree nodes in another topological order permutes the output rows;
* permuting the prefix keys changes nothing.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import bruteforce
from tree_verification_attention_amd import workloads as W

from helpers import f64, tiny_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf_inputs(w):
    """Nested float lists for the brute force (bf16 widened exactly through float32)."""
    def L(t):
        return t.to(torch.float64).tolist()
    return (L(w.q), L(w.k_prefix), L(w.v_prefix), L(w.k_tree), L(w.v_tree),
            w.parent_idx.tolist(), w.prefix_len.tolist(), w.scale)


# ----------------------------------------------------------------------------- brute force


@st.composite
def tiny_cases(draw):
    B = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    D = draw(st.integers(1, 9))
    Lmax = draw(st.integers(0, 11))
    T = draw(st.integers(1, 8))
    seed = draw(st.integers(0, 2**31 - 1))
    gen = torch.Generator().manual_seed(seed)
    parents = [W.random_forest(T, gen) for _ in range(B)]
    plen = [draw(st.integers(0, Lmax)) for _ in range(B)]
    dtype = draw(st.sampled_from([torch.float32, torch.bfloat16]))
    peaky = draw(st.sampled_from([0.0, 0.3]))
    return tiny_workload(parents, B=B, Hq=Hkv * G, Hkv=Hkv, D=D, L=Lmax, prefix_len=plen,
                         dtype=dtype, seed=seed, peaky=peaky)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_cases())
def test_oracle_matches_bruteforce_random_tiny(w):
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    bo, bl = bruteforce.verify(*_bf_inputs(w))
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_oracle_matches_bruteforce_tiny_config_sample():
    """The tiny fp32 configuration (prefix 1024, 7-node binary tree), every 7th row."""
    w = W.tiny()
    a = w.as_numpy()
    rows = [(0, h, i) for h in range(w.num_q_heads) for i in range(w.tree_size)][::3]
    out, lse = oracle.rows(a, w.scale, [r[0] for r in rows], [r[1] for r in rows],
                           [r[2] for r in rows])
    q, kp, vp, kt, vt, par, plen, scale = _bf_inputs(w)
    anc = bruteforce.ancestor_sets(par[0])
    for n, (b, h, i) in enumerate(rows):
        g = h // (w.num_q_heads // w.num_kv_heads)
        keys = kp[b][g][: plen[b]] + [kt[b][g][t] for t in sorted(anc[i])]
        vals = vp[b][g][: plen[b]] + [vt[b][g][t] for t in sorted(anc[i])]
        o, l = bruteforce.attention_row(q[b][i][h], keys, vals, scale)
        np.testing.assert_allclose(out[n], o, rtol=0, atol=1e-12)
        assert abs(lse[n] - l) < 1e-12


# ----------------------------------------------------------------------------- library special cases


def _sdpa(q, k, v, scale, mask=None, causal=False):
    """torch fp64 SDPA; q [H, Nq, D], k/v [H, Nk, D]."""
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal, scale=scale)


@pytest.mark.parametrize("T,L,G", [(1, 0, 1), (5, 0, 2), (5, 17, 4), (9, 33, 1), (3, 1, 3)])
def test_chain_tree_equals_causal_attention(T, L, G):
    """A chain is causal attention over the concatenated sequence (its last T query rows)."""
    Hkv = 2
    w = tiny_workload(W.chain_tree(T), B=1, Hq=Hkv * G, Hkv=Hkv, D=16, L=L, seed=7 + T,
                      dtype=torch.bfloat16, peaky=0.1)
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    for h in range(w.num_q_heads):
        g = h // G
        k = torch.cat([f64(w.k_prefix[0, g]), f64(w.k_tree[0, g])])  # [L+T, D]
        v = torch.cat([f64(w.v_prefix[0, g]), f64(w.v_tree[0, g])])
        qs = torch.zeros(L + T, w.head_dim, dtype=torch.float64)
        qs[L:] = f64(w.q[0, :, h])
        ref = _sdpa(qs[None], k[None], v[None], w.scale, causal=True)[0, L:]
        np.testing.assert_allclose(out[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_single_node_equals_decode_attention():
    w = tiny_workload([-1], B=2, Hq=4, Hkv=2, D=32, L=40, prefix_len=[40, 13], seed=3)
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    for b in range(2):
        Lb = int(w.prefix_len[b])
        for h in range(4):
            g = h // 2
            k = torch.cat([f64(w.k_prefix[b, g, :Lb]), f64(w.k_tree[b, g])])
            v = torch.cat([f64(w.v_prefix[b, g, :Lb]), f64(w.v_tree[b, g])])
            ref = _sdpa(f64(w.q[b, :, h])[None], k[None], v[None], w.scale)[0]
            np.testing.assert_allclose(out[b, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_star_tree_equals_diagonal_mask():
    T, L = 6, 9
    w = tiny_workload(W.star_tree(T), B=1, Hq=2, Hkv=1, D=8, L=L, seed=11)
    out, _ = oracle.verify(w.as_numpy(), w.scale)
    mask = torch.zeros(T, L + T, dtype=torch.bool)
    mask[:, :L] = True
    mask[torch.arange(T), L + torch.arange(T)] = True
    for h in range(2):
        k = torch.cat([f64(w.k_prefix[0, 0]), f64(w.k_tree[0, 0])])
        v = torch.cat([f64(w.v_prefix[0, 0]), f64(w.v_tree[0, 0])])
        ref = _sdpa(f64(w.q[0, :, h])[None], k[None], v[None], w.scale, mask=mask[None])[0]
        np.testing.assert_allclose(out[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_random_tree_equals_sdpa_with_ancestor_mask_from_matrix_closure():
    """Ancestor mask built by boolean matrix closure (a different route), then SDPA."""
    gen = torch.Generator().manual_seed(5)
    T, L = 12, 10
    par = W.random_forest(T, gen)
    w = tiny_workload(par, B=1, Hq=3, Hkv=1, D=8, L=L, seed=5)
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    A = np.eye(T, dtype=bool)
    for i, p in enumerate(par):
        if p >= 0:
            A[i, p] = True
    for _ in range(T):
        A = (A.astype(np.int64) @ A.astype(np.int64)) > 0
    mask = torch.zeros(T, L + T, dtype=torch.bool)
    mask[:, :L] = True
    mask[:, L:] = torch.from_numpy(A)
    for h in range(3):
        k = torch.cat([f64(w.k_prefix[0, 0]), f64(w.k_tree[0, 0])])
        v = torch.cat([f64(w.v_prefix[0, 0]), f64(w.v_tree[0, 0])])
        ref = _sdpa(f64(w.q[0, :, h])[None], k[None], v[None], w.scale, mask=mask[None])[0]
        np.testing.assert_allclose(out[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- merge / split invariance


@pytest.mark.parametrize("nparts", [1, 2, 3, 7])
def test_split_and_merge_equals_unsplit(nparts):
    rng = np.random.default_rng(nparts)
    nk, D = 23, 6
    q = rng.standard_normal((4, D))
    k = rng.standard_normal((nk, D)) * 2
    v = rng.standard_normal((nk, D))
    full_mask = rng.random((4, nk)) < 0.8
    full_mask[:, 0] = True
    o_ref, l_ref = oracle.masked_attention(q, k, v, full_mask, 0.7)
    assign = rng.integers(0, nparts, size=nk)  # arbitrary partition of the keys
    for r in range(4):
        lp, op = [], []
        for p in range(nparts):
            m = full_mask[r:r + 1] & (assign == p)[None, :]
            o, l = oracle.masked_attention(q[r:r + 1], k, v, m, 0.7)
            lp.append(l[0]); op.append(o[0])
        o, l = oracle.lse_merge(np.array(lp), np.array(op))
        np.testing.assert_allclose(o, o_ref[r], rtol=0, atol=1e-12)
        assert abs(l - l_ref[r]) < 1e-12


def test_prefix_and_tree_parts_merge_to_full():
    gen = torch.Generator().manual_seed(9)
    par = [W.level_tree((2, 3, 3), gen) for _ in range(2)]
    w = tiny_workload(par, B=2, Hq=4, Hkv=2, D=8, L=12, prefix_len=[12, 0], seed=9,
                      dtype=torch.bfloat16)
    a = w.as_numpy()
    o_all, l_all = oracle.verify(a, w.scale, oracle.PART_ALL)
    o_p, l_p = oracle.verify(a, w.scale, oracle.PART_PREFIX)
    o_t, l_t = oracle.verify(a, w.scale, oracle.PART_TREE)
    assert np.all(np.isneginf(l_p[1])) and np.all(o_p[1] == 0)  # empty prefix part
    for b in range(2):
        for i in range(w.tree_size):
            for h in range(4):
                o, l = oracle.lse_merge(np.array([l_p[b, h, i], l_t[b, h, i]]),
                                        np.stack([o_p[b, i, h], o_t[b, i, h]]))
                np.testing.assert_allclose(o, o_all[b, i, h], rtol=0, atol=1e-12)
                assert abs(l - l_all[b, h, i]) < 1e-12


def test_merge_identities():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((3, 5))
    l = rng.standard_normal(3)
    base_o, base_l = oracle.lse_merge(l, o)
    # merging with an empty part is the identity
    o2, l2 = oracle.lse_merge(np.append(l, -np.inf), np.vstack([o, rng.standard_normal(5)]))
    np.testing.assert_allclose(o2, base_o, rtol=0, atol=1e-15)
    assert l2 == base_l
    # associativity: ((0,1),2) == (0,(1,2))
    o01, l01 = oracle.lse_merge(l[:2], o[:2])
    oa, la = oracle.lse_merge(np.array([l01, l[2]]), np.vstack([o01, o[2]]))
    np.testing.assert_allclose(oa, base_o, rtol=0, atol=1e-14)
    assert abs(la - base_l) < 1e-14
    # two equal parts: out unchanged, lse + ln 2
    o3, l3 = oracle.lse_merge(np.array([l[0], l[0]]), np.vstack([o[0], o[0]]))
    np.testing.assert_allclose(o3, o[0], rtol=0, atol=1e-15)
    assert abs(l3 - (l[0] + math.log(2))) < 1e-14
    # all empty
    o4, l4 = oracle.lse_merge(np.array([-np.inf, -np.inf]), np.zeros((2, 5)))
    assert l4 == -np.inf and np.all(o4 == 0)


# ----------------------------------------------------------------------------- closed forms


def test_zero_query_closed_form():
    """q = 0: uniform weights, lse = ln(prefix_len + depth + 1), out = mean of visible v."""
    gen = torch.Generator().manual_seed(2)
    par = [W.level_tree((3, 4, 4), gen), W.chain_tree(11)]
    w = tiny_workload(par, B=2, Hq=4, Hkv=2, D=5, L=20, prefix_len=[20, 7], seed=2)
    w.q.zero_()
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    for b in range(2):
        dep = W.depths(par[b])
        Lb = int(w.prefix_len[b])
        for h in range(4):
            g = h // 2
            for i in range(w.tree_size):
                assert abs(lse[b, h, i] - math.log(Lb + dep[i] + 1)) < 1e-13
                chain = []
                p = i
                while p != -1:
                    chain.append(p)
                    p = par[b][p]
                rows = np.concatenate([w.v_prefix[b, g, :Lb].double().numpy(),
                                       w.v_tree[b, g, chain].double().numpy()])
                np.testing.assert_allclose(out[b, i, h], rows.mean(0), rtol=0, atol=1e-13)


def test_hand_worked_golden_example():
    """A two-key example worked by hand (derivation in the fixture file)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        ex = json.load(f)
    a = {k: np.array(v, dtype=np.float32) for k, v in ex["inputs"].items()
         if k not in ("parent_idx", "prefix_len")}
    a["parent_idx"] = np.array(ex["inputs"]["parent_idx"], dtype=np.int32)
    a["prefix_len"] = np.array(ex["inputs"]["prefix_len"], dtype=np.int32)
    out, lse = oracle.verify(a, ex["scale"])
    for row in ex["expected"]:
        b, i, h = row["b"], row["i"], row["h"]
        expect = [eval(e, {"math": math}) for e in row["out"]]
        np.testing.assert_allclose(out[b, i, h], expect, rtol=0, atol=1e-12)
        assert abs(lse[b, h, i] - eval(row["lse"], {"math": math})) < 1e-12


# ----------------------------------------------------------------------------- invariants


def test_gqa_equals_mha_with_repeated_kv():
    gen = torch.Generator().manual_seed(4)
    par = [W.level_tree((2, 4), gen)]
    w = tiny_workload(par, B=1, Hq=6, Hkv=2, D=8, L=9, seed=4, dtype=torch.bfloat16)
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    rep = lambda t: t.repeat_interleave(3, dim=1).contiguous()  # noqa: E731
    w2 = tiny_workload(par, B=1, Hq=6, Hkv=6, D=8, L=9, seed=4, dtype=torch.bfloat16)
    w2.q, w2.k_prefix, w2.v_prefix = w.q, rep(w.k_prefix), rep(w.v_prefix)
    w2.k_tree, w2.v_tree = rep(w.k_tree), rep(w.v_tree)
    out2, lse2 = oracle.verify(w2.as_numpy(), w.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_topological_relabelling_permutes_rows():
    par = [-1, -1, 0, 0, 1, 2, 2, 4]
    w = tiny_workload(par, B=1, Hq=2, Hkv=1, D=8, L=6, seed=8)
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    # another topological order: new position n holds old node perm[n]
    perm = [1, 0, 4, 3, 2, 7, 6, 5]
    inv = {old: new for new, old in enumerate(perm)}
    new_par = [inv[par[old]] if par[old] >= 0 else -1 for old in perm]
    assert all(p < n for n, p in enumerate(new_par))
    w2 = tiny_workload(new_par, B=1, Hq=2, Hkv=1, D=8, L=6, seed=8)
    w2.q = w.q[:, perm].contiguous()
    w2.k_prefix, w2.v_prefix = w.k_prefix, w.v_prefix
    w2.k_tree = w.k_tree[:, :, perm].contiguous()
    w2.v_tree = w.v_tree[:, :, perm].contiguous()
    out2, lse2 = oracle.verify(w2.as_numpy(), w.scale)
    np.testing.assert_allclose(out2, out[:, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, perm], rtol=0, atol=1e-13)


def test_prefix_permutation_invariance():
    w = tiny_workload([-1, 0, 0, 1], B=1, Hq=2, Hkv=1, D=8, L=15, seed=12, prefix_len=[11])
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    perm = torch.randperm(11, generator=torch.Generator().manual_seed(1))
    w.k_prefix[:, :, :11] = w.k_prefix[:, :, perm].clone()
    w.v_prefix[:, :, :11] = w.v_prefix[:, :, perm].clone()
    out2, lse2 = oracle.verify(w.as_numpy(), w.scale)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_padding_beyond_prefix_len_is_never_read():
    w = tiny_workload([-1, 0], B=2, Hq=2, Hkv=1, D=8, L=10, prefix_len=[4, 10], seed=13)
    out, lse = oracle.verify(w.as_numpy(), w.scale)
    w.k_prefix[0, :, 4:] = float("nan")
    w.v_prefix[0, :, 4:] = float("nan")
    out2, lse2 = oracle.verify(w.as_numpy(), w.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


# ----------------------------------------------------------------------------- masks and tree validity


@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 68, 130, 256])
def test_mask_invariants(T):
    gen = torch.Generator().manual_seed(T)
    par = np.array([W.random_forest(T, gen), W.chain_tree(T)], dtype=np.int32)
    masks = oracle.ancestor_masks(par)
    assert masks.shape == (2, T, (T + 63) // 64)
    for b in range(2):
        dep = W.depths(par[b].tolist())
        for i in range(T):
            m = masks[b, i]
            pop = sum(bin(int(x)).count("1") for x in m)
            assert pop == dep[i] + 1
            assert (int(m[i // 64]) >> (i % 64)) & 1 == 1
            p = par[b, i]
            if p >= 0:
                expect = masks[b, p].copy()
                expect[i // 64] |= np.uint64(1) << np.uint64(i % 64)
                np.testing.assert_array_equal(m, expect)
            # no bit beyond i (ancestors precede their descendants)
            for t in range(i + 1, T):
                assert (int(m[t // 64]) >> (t % 64)) & 1 == 0
        # compare with the brute-force fixed point
        anc = bruteforce.ancestor_sets(par[b].tolist())
        for i in range(T):
            bits = {t for t in range(T) if (int(masks[b, i, t // 64]) >> (t % 64)) & 1}
            assert bits == anc[i]


def test_chain_masks_are_lower_triangular_words():
    masks = oracle.ancestor_masks(np.array([W.chain_tree(70)], dtype=np.int32))
    for i in range(70):
        full = sum(int(masks[0, i, w]) << (64 * w) for w in range(2))
        assert full == (1 << (i + 1)) - 1


@pytest.mark.parametrize("bad", [[0, -1], [-1, 1], [-1, 0, 5], [-2, -1]])
def test_invalid_trees_are_rejected(bad):
    par = np.array([bad], dtype=np.int32)
    assert not oracle.check_tree(par)
    with pytest.raises(oracle.OracleError):
        oracle.ancestor_masks(par)
    w = tiny_workload([-1] * len(bad), B=1, Hq=1, Hkv=1, D=2, L=1)
    a = w.as_numpy()
    a["parent_idx"] = par
    with pytest.raises(oracle.OracleError):
        oracle.verify(a, 1.0)


# ----------------------------------------------------------------------------- general masked attention


def test_masked_attention_matches_fp64_sdpa_with_a_boolean_mask():
    """The general masked-attention oracle against torch's fp64 scaled_dot_product_attention
    with a boolean mask and against logsumexp of the masked scores; an all-masked row gives
    out 0, lse -inf."""
    rng = np.random.default_rng(40)
    nq, nk, D, scale = 9, 37, 12, 0.37
    q = rng.standard_normal((nq, D)) * 1.5
    k = rng.standard_normal((nk, D))
    v = rng.standard_normal((nk, D))
    mask = rng.random((nq, nk)) < 0.4
    mask[0, :] = False          # sees nothing
    mask[1, :] = True           # sees everything
    mask[2, :] = False
    mask[2, 17] = True          # sees one key
    out, lse = oracle.masked_attention(q, k, v, mask, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    tm = torch.from_numpy(mask)
    rows = np.nonzero(mask.any(axis=1))[0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq[rows][None], tk[None], tv[None], attn_mask=tm[rows][None], scale=scale)[0].numpy()
    np.testing.assert_allclose(out[rows], ref, rtol=0, atol=1e-13)
    s = (tq @ tk.T) * scale
    ref_lse = torch.logsumexp(s.masked_fill(~tm, float("-inf")), dim=1).numpy()
    np.testing.assert_allclose(lse[rows], ref_lse[rows], rtol=0, atol=1e-13)
    assert lse[0] == -np.inf and (out[0] == 0).all()
    np.testing.assert_allclose(out[2], v[17], atol=1e-15)
