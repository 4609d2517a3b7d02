"""GPU parity of the steps around the attention (libhta.so through the C ABI) against the
step oracle: rotary encoding of the tree, the target's greedy tokens, greedy acceptance and
the KV commit.

Bars: positions, greedy tokens, acceptance outputs and the committed caches bit-exact;
rotated q / k_tree within one unit in the last place of their storage type of the oracle's
single rounding of the exact fp64 rotation, with at most one element in 10^4 off at all
(both sides round the same fp64 value once; they can part only where device and host
sin/cos differ in the last bits of a double right at a rounding boundary).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _np_in(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return _bits16(t) if t.dtype == torch.bfloat16 else t.numpy()


def _ulp_distance(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Distance in representable steps between equal-width float bit patterns."""
    if got.dtype == np.uint16:
        g, w = got.astype(np.int64), want.astype(np.int64)
        sign = 0x8000
    else:
        g = got.view(np.uint32).astype(np.int64)
        w = want.view(np.uint32).astype(np.int64)
        sign = 0x80000000
    # map sign-magnitude to a monotone integer line
    g = np.where(g & sign, -(g & (sign - 1)), g)
    w = np.where(w & sign, -(w & (sign - 1)), w)
    return np.abs(g - w)


def _expected_rope(x: torch.Tensor, par, plen, theta, interleaved, layout):
    ref, pos = oracle.rope(_np_in(x), np.asarray(par), np.asarray(plen), theta, interleaved,
                           layout)
    if x.dtype == torch.bfloat16:
        return oracle.round_bf16(ref), pos
    return ref.astype(np.float32), pos


def _check_rotated(got: torch.Tensor, want: np.ndarray):
    g = _np_in(got)
    d = _ulp_distance(g, want)
    assert d.max() <= 1, f"max distance {d.max()} ulp"
    assert (d > 0).sum() <= max(1, d.size // 10000), f"{(d > 0).sum()} of {d.size} differ"


ROPE_CASES = [
    # name, B, T-tree, Hq, Hkv, D, dtype, prefix_len, theta, interleaved
    ("tiny_fp32", 2, "binary3", 4, 2, 64, torch.float32, [0, 1000], 10000.0, False),
    ("tiny_fp32_inter", 2, "binary3", 4, 2, 64, torch.float32, [5, 77], 10000.0, True),
    ("llama_32k", 1, "longspec", 32, 8, 128, torch.bfloat16, [32768], W.LLAMA3_ROPE_THETA, False),
    ("llama_262k", 1, "longspec", 32, 8, 128, torch.bfloat16, [262144], W.LLAMA3_ROPE_THETA, False),
    ("vicuna_b8", 8, "longspec", 32, 32, 128, torch.bfloat16, "ragged", W.VICUNA_ROPE_THETA, False),
    ("qwq_chain5", 1, "chain5", 40, 8, 128, torch.bfloat16, [16384], W.QWQ_ROPE_THETA, False),
    ("chain256_inter", 1, "chain256", 4, 1, 64, torch.bfloat16, [123456], 10000.0, True),
]


def _parents(kind, B, gen):
    if kind == "binary3":
        return [W.complete_binary_tree(3)] * B
    if kind == "longspec":
        return [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(B)]
    if kind == "chain5":
        return [W.chain_tree(5)] * B
    if kind == "chain256":
        return [W.chain_tree(256)] * B
    raise KeyError(kind)


@pytest.mark.parametrize("case", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope_tree_matches_oracle(case):
    name, B, kind, Hq, Hkv, D, dtype, plen, theta, inter = case
    gen = torch.Generator().manual_seed(31)
    par = _parents(kind, B, gen)
    T = len(par[0])
    if plen == "ragged":
        plen = torch.randint(8192, 16385, (B,), generator=gen).tolist()
    q = torch.randn(B, T, Hq, D, generator=gen).to(dtype)
    k = torch.randn(B, Hkv, T, D, generator=gen).to(dtype)
    want_q, pos = _expected_rope(q, par, plen, theta, inter, "q")
    want_k, _ = _expected_rope(k, par, plen, theta, inter, "k")
    qd, kd = q.to(DEV), k.to(DEV)
    pd = torch.tensor(par, dtype=torch.int32, device=DEV)
    ld = torch.tensor(plen, dtype=torch.int32, device=DEV)
    got_pos = hta.rope_tree(qd, kd, pd, ld, theta, interleaved=inter, max_prefix_len=max(plen))
    torch.cuda.synchronize()
    assert np.array_equal(got_pos.cpu().numpy(), pos)
    _check_rotated(qd, want_q)
    _check_rotated(kd, want_k)


def test_rope_tree_errors_poison_only_the_bad_sequence():
    gen = torch.Generator().manual_seed(32)
    B, T, Hq, Hkv, D = 3, 7, 4, 2, 64
    par = [W.complete_binary_tree(3)] * B
    par = [list(p) for p in par]
    par[1][4] = 5  # points forward: invalid
    plen = [10, 10, 10]
    q = torch.randn(B, T, Hq, D, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Hkv, T, D, generator=gen).to(torch.bfloat16)
    good = [0, 2]
    want_q, pos = _expected_rope(q[good], [par[0], par[2]], [10, 10], 10000.0, False, "q")
    qd, kd = q.to(DEV), k.to(DEV)
    desc = hta.make_desc(B, Hq, Hkv, D, T, 64)
    ws = hta.new_workspace(desc, DEV)
    positions = torch.empty(B, T, dtype=torch.int32, device=DEV)
    pl = torch.tensor(plen, dtype=torch.int32, device=DEV)
    hta.hta_rope_tree(desc, 10000.0, False, qd, kd, torch.tensor(par, dtype=torch.int32,
                      device=DEV), pl, positions, ws)
    code, bad = hta.hta_get_device_status(desc, ws)
    assert (code, bad) == (6, 1)
    assert torch.isnan(qd[1].float()).all() and torch.isnan(kd[1].float()).all()
    assert (positions[1] == -1).all()
    _check_rotated(qd[good], want_q)
    assert np.array_equal(positions[good].cpu().numpy(), pos)
    # prefix_len beyond the cache: HTA_ERR_PREFIX_LEN, rows poisoned
    par_ok = torch.tensor([W.complete_binary_tree(3)] * B, dtype=torch.int32, device=DEV)
    qd, kd = q.to(DEV), k.to(DEV)
    pl = torch.tensor([10, 65, 10], dtype=torch.int32, device=DEV)
    hta.hta_rope_tree(desc, 10000.0, False, qd, kd, par_ok, pl, None, ws)
    code, bad = hta.hta_get_device_status(desc, ws)
    assert (code, bad) == (7, 1)
    assert torch.isnan(qd[1].float()).all() and not torch.isnan(qd[0].float()).any()


# ----------------------------------------------------------------------------- acceptance


def _step_case(B, kind, Hkv, D, Lmax, plen, vocab, ldtype, kvdtype, seed):
    gen = torch.Generator().manual_seed(seed)
    par = _parents(kind, B, gen)
    T = len(par[0])
    st = W.make_step_inputs(par, vocab, dtype=ldtype, seed=seed)
    if B * Hkv * Lmax * D <= 40_000_000:
        kp = torch.randn(B, Hkv, Lmax, D, generator=gen).to(kvdtype)
        vp = torch.randn(B, Hkv, Lmax, D, generator=gen).to(kvdtype)
    else:  # large caches: a cheap pattern that still differs from row to row
        n = B * Hkv * Lmax * D
        kp = ((torch.arange(n) % 509) * 0.01 - 2.5).reshape(B, Hkv, Lmax, D).to(kvdtype)
        vp = ((torch.arange(n) % 503) * 0.01 - 2.5).reshape(B, Hkv, Lmax, D).to(kvdtype)
    kt = torch.randn(B, Hkv, T, D, generator=gen).to(kvdtype)
    vt = torch.randn(B, Hkv, T, D, generator=gen).to(kvdtype)
    return par, st, kp, vp, kt, vt, list(plen)


def _run_and_check(par, st, kp, vp, kt, vt, plen, expect_codes=(0,)):
    B, Hkv, Lmax, D = kp.shape
    T = len(par[0])
    logits = st.logits
    # oracle
    nxt = oracle.argmax(_np_in(logits))
    n_ref, acc_ref, bonus_ref = oracle.accept(np.array(par), st.tokens.numpy(),
                                              st.root_token.numpy(), nxt)
    kp_ref, vp_ref, pl_ref, full = oracle.kv_commit(_np_in(kp), _np_in(vp), _np_in(kt),
                                                    _np_in(vt), np.array(plen, dtype=np.int32),
                                                    n_ref, acc_ref)
    # device
    d = {k: v.to(DEV) for k, v in dict(logits=logits, tok=st.tokens, root=st.root_token,
                                       kp=kp, vp=vp, kt=kt, vt=vt).items()}
    pd = torch.tensor(par, dtype=torch.int32, device=DEV)
    ld = torch.tensor(plen, dtype=torch.int32, device=DEV)
    desc = hta.make_desc(B, Hkv, Hkv, D, T, Lmax, 0 if kp.dtype == torch.bfloat16 else 1)
    ws = torch.empty(hta.accept_workspace_size(desc, logits.shape[-1]), dtype=torch.uint8,
                     device=DEV)
    outs = [torch.full((B, T), -7, dtype=torch.int32, device=DEV),
            torch.full((B,), -7, dtype=torch.int32, device=DEV),
            torch.full((B, T), -7, dtype=torch.int32, device=DEV),
            torch.full((B,), -7, dtype=torch.int32, device=DEV)]
    hta.hta_accept_commit(desc, d["logits"], d["tok"], d["root"], pd, ld, d["kp"], d["vp"],
                          d["kt"], d["vt"], *outs, ws)
    code, bad = hta.hta_get_device_status(desc, ws)
    assert code in expect_codes
    tn, n, acc, bonus = (o.cpu().numpy() for o in outs)
    assert np.array_equal(tn, nxt)
    assert np.array_equal(n, n_ref)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(bonus, bonus_ref)
    assert np.array_equal(ld.cpu().numpy(), pl_ref)
    assert np.array_equal(_np_in(d["kp"]), kp_ref)
    assert np.array_equal(_np_in(d["vp"]), vp_ref)
    return n_ref, full, code, bad


STEP_CASES = [
    # name, B, tree, Hkv, D, Lmax, prefix_len, vocab, logits dtype, kv dtype
    ("llama_32k", 1, "longspec", 8, 128, 32768 + 8, [32768], W.LLAMA3_VOCAB, torch.bfloat16,
     torch.bfloat16),
    ("vicuna_b8", 8, "longspec", 32, 128, 16384 + 8, "ragged", W.VICUNA_VOCAB, torch.bfloat16,
     torch.bfloat16),
    ("qwq_f32_logits", 1, "longspec", 8, 128, 4096 + 8, [4096], W.QWQ_VOCAB, torch.float32,
     torch.bfloat16),
    ("tiny_fp32_odd_vocab", 2, "binary3", 4, 64, 64, [0, 50], 1001, torch.float32,
     torch.float32),
    ("bf16_odd_vocab", 2, "longspec", 2, 64, 200, [100, 7], 12345, torch.bfloat16,
     torch.bfloat16),
    ("vocab_7", 3, "binary3", 1, 64, 32, [1, 2, 3], 7, torch.bfloat16, torch.bfloat16),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_accept_commit_matches_oracle(case):
    name, B, kind, Hkv, D, Lmax, plen, vocab, ldt, kvdt = case
    if plen == "ragged":
        plen = torch.randint(8192, 16385, (B,), generator=torch.Generator().manual_seed(5)).tolist()
    args = _step_case(B, kind, Hkv, D, Lmax, plen, vocab, ldt, kvdt, seed=40 + len(name))
    n, full, code, _ = _run_and_check(*args)
    assert code == 0 and not full.any()


def test_accept_commit_ties_nans_and_signed_zeros():
    B, T, V = 1, 7, 40000  # spans of 8192: several per row
    par = [W.complete_binary_tree(3)]
    st = W.make_step_inputs(par, V, dtype=torch.bfloat16, seed=50)
    lg = st.logits.float()
    lg[0, 0, :] = -1.0
    lg[0, 0, [30000, 9000, 20000]] = 5.0      # equal maxima in three spans: 9000 wins
    lg[0, 1, [39999, 12]] = float("nan")      # the first NaN wins over everything
    lg[0, 1, 100] = float("inf")
    lg[0, 2, :] = float("-inf")               # every value equal: index 0
    lg[0, 3, :] = -0.0
    lg[0, 3, 8191] = 0.0                      # +0 == -0: index 0
    lg[0, 4, :] = -3.0
    lg[0, 4, 8192] = -2.5                     # first element of the second span
    lg[0, 5, V - 1] = 100.0                   # the last element
    st.logits = lg.to(torch.bfloat16)
    gen = torch.Generator().manual_seed(51)
    kp = torch.randn(B, 2, 32, 64, generator=gen).to(torch.bfloat16)
    vp, kt, vt = (torch.randn(s, generator=gen).to(torch.bfloat16)
                  for s in ((B, 2, 32, 64), (B, 2, T, 64), (B, 2, T, 64)))
    _run_and_check(par, st, kp, vp, kt, vt, [4])
    nxt = oracle.argmax(_np_in(st.logits))[0]
    assert nxt[:6].tolist() == [9000, 12, 0, 0, 8192, V - 1]


def test_accept_commit_full_chain_and_cache_full():
    # a 256-node chain whose every draft is right: the whole chain is accepted
    T, V = 256, 512
    par = [W.chain_tree(T)]
    gen = torch.Generator().manual_seed(52)
    toks = torch.randint(0, V, (1, T), generator=gen, dtype=torch.int32)
    logits = torch.randn(1, T, V, generator=gen)
    nxt_tok = torch.cat([toks[0, 1:], torch.tensor([3], dtype=torch.int32)])
    logits[0, torch.arange(T), nxt_tok.long()] = 50.0
    st = W.StepInputs(tokens=toks, root_token=toks[:, 0].clone(),
                      logits=logits.to(torch.bfloat16), planted=nxt_tok[None])
    kp = torch.randn(1, 2, 300, 64, generator=gen).to(torch.bfloat16)
    vp, kt, vt = (torch.randn(s, generator=gen).to(torch.bfloat16)
                  for s in ((1, 2, 300, 64), (1, 2, T, 64), (1, 2, T, 64)))
    n, full, code, _ = _run_and_check(par, st, kp, vp, kt, vt, [44])
    assert n.tolist() == [256] and code == 0
    # the same path into a cache with room for 255 more rows: HTA_ERR_CACHE_FULL, the
    # acceptance outputs are still written and the cache is left alone
    n, full, code, bad = _run_and_check(par, st, kp, vp, kt, vt, [45], expect_codes=(9,))
    assert full.tolist() == [True] and (code, bad) == (9, 0)


def test_accept_commit_invalid_tree_and_prefix_len():
    B, V = 2, 300
    gen = torch.Generator().manual_seed(53)
    par = [W.complete_binary_tree(3), W.complete_binary_tree(3)]
    st = W.make_step_inputs(par, V, seed=54)
    kp = torch.randn(B, 1, 16, 64, generator=gen).to(torch.bfloat16)
    vp, kt, vt = (torch.randn(s, generator=gen).to(torch.bfloat16)
                  for s in ((B, 1, 16, 64), (B, 1, 7, 64), (B, 1, 7, 64)))
    bad_par = [list(par[0]), [-1, 0, 0, 1, 1, 2, 6]]  # node 6 is its own parent
    pd = torch.tensor(bad_par, dtype=torch.int32, device=DEV)
    ld = torch.tensor([3, 3], dtype=torch.int32, device=DEV)
    desc = hta.make_desc(B, 1, 1, 64, 7, 16)
    ws = torch.empty(hta.accept_workspace_size(desc, V), dtype=torch.uint8, device=DEV)
    kd, vd = kp.to(DEV), vp.to(DEV)
    outs = hta.accept_commit(st.logits.to(DEV), st.tokens.to(DEV), st.root_token.to(DEV), pd, ld,
                             kd, vd, kt.to(DEV), vt.to(DEV), workspace=ws)
    code, bad = hta.hta_get_device_status(desc, ws)
    assert (code, bad) == (6, 1)
    tn, n, acc, bonus = (o.cpu().numpy() for o in outs)
    assert np.array_equal(tn, oracle.argmax(_np_in(st.logits)))  # greedy tokens still given
    assert n[1] == 0 and (acc[1] == -1).all() and bonus[1] == -1
    assert ld.cpu().tolist()[1] == 3 and torch.equal(kd[1].cpu(), kp[1])
    n0, acc0, b0 = oracle.accept(np.array(par[:1]), st.tokens.numpy()[:1],
                                 st.root_token.numpy()[:1], tn[:1])
    assert n[0] == n0[0] and np.array_equal(acc[0], acc0[0]) and bonus[0] == b0[0]
    # prefix_len outside [0, Lmax]: acceptance reported, nothing committed
    pd = torch.tensor(par, dtype=torch.int32, device=DEV)
    ld = torch.tensor([3, 17], dtype=torch.int32, device=DEV)
    kd = kp.to(DEV)
    hta.accept_commit(st.logits.to(DEV), st.tokens.to(DEV), st.root_token.to(DEV), pd, ld, kd,
                      vp.to(DEV), kt.to(DEV), vt.to(DEV), workspace=ws)
    code, bad = hta.hta_get_device_status(desc, ws)
    assert (code, bad) == (7, 1)
    assert ld.cpu().tolist()[1] == 17 and torch.equal(kd[1].cpu(), kp[1])


# ----------------------------------------------------------------------------- whole step


def test_greedy_step_rope_verify_accept_commit():
    """rotary positions -> verification attention -> greedy acceptance -> KV commit, on the
    device, against the oracle's chain on the same inputs."""
    w = W.make_workload("step", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        max_prefix_len=2048, prefix_len=[1500, 700],
                        tree_widths=W.LONGSPEC_TREE_WIDTHS, seed=60)
    theta, vocab = W.LLAMA3_ROPE_THETA, 5000
    par = w.parent_idx.numpy()
    st = W.make_step_inputs(par.tolist(), vocab, seed=61)
    # oracle chain
    a = w.as_numpy()
    q_ref, _ = oracle.rope(a["q"], par, a["prefix_len"], theta, False, "q")
    k_ref, _ = oracle.rope(a["k_tree"], par, a["prefix_len"], theta, False, "k")
    a_rot = dict(a, q=oracle.round_bf16(q_ref), k_tree=oracle.round_bf16(k_ref))
    out_ref, lse_ref = oracle.verify(a_rot, w.scale)
    nxt = oracle.argmax(_np_in(st.logits))
    n_ref, acc_ref, bonus_ref = oracle.accept(par, st.tokens.numpy(), st.root_token.numpy(), nxt)
    kp_ref, vp_ref, pl_ref, _ = oracle.kv_commit(a["k_prefix"], a["v_prefix"], a_rot["k_tree"],
                                                 a["v_tree"], a["prefix_len"], n_ref, acc_ref)
    # device chain
    d = {k: getattr(w, k).to(DEV) for k in ("q", "k_prefix", "v_prefix", "k_tree", "v_tree",
                                            "parent_idx", "prefix_len")}
    hta.rope_tree(d["q"], d["k_tree"], d["parent_idx"], d["prefix_len"], theta,
                  max_prefix_len=w.max_prefix_len)
    out, lse = hta.verify(d["q"], d["k_prefix"], d["v_prefix"], d["k_tree"], d["v_tree"],
                          d["parent_idx"], d["prefix_len"])
    tn, n, acc, bonus = hta.accept_commit(st.logits.to(DEV), st.tokens.to(DEV),
                                          st.root_token.to(DEV), d["parent_idx"],
                                          d["prefix_len"], d["k_prefix"], d["v_prefix"],
                                          d["k_tree"], d["v_tree"])
    torch.cuda.synchronize()
    _check_rotated(d["q"], a_rot["q"])
    _check_rotated(d["k_tree"], a_rot["k_tree"])
    np.testing.assert_allclose(out.cpu().numpy(), out_ref, rtol=0, atol=2e-3)
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=1e-3)
    assert np.array_equal(n.cpu().numpy(), n_ref) and np.array_equal(acc.cpu().numpy(), acc_ref)
    assert np.array_equal(bonus.cpu().numpy(), bonus_ref)
    assert np.array_equal(d["prefix_len"].cpu().numpy(), pl_ref)
    assert np.array_equal(_bits16(d["k_prefix"]), kp_ref)
    assert np.array_equal(_bits16(d["v_prefix"]), vp_ref)
    assert n_ref.sum() > 0  # the seeds accept something
