"""Pins of the step oracle (oracle/step_oracle.c): rotary positions of the tree, the
target's greedy token, greedy acceptance, and the KV commit.

Each pin checks the oracle against something other than itself: closed forms (a rotation
by a known angle, positions of a level tree), an independent formulation (complex
exponentials; exact rational rounding), invariants (relative-position property, norms),
library routines (numpy's argmax), and the lossless property of greedy speculation (the
emitted tokens equal plain greedy decoding of a toy target).  Planted mistakes in a copy of
the oracle must each fail one of them (last test).
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tree_verification_attention_amd import workloads as W

ORACLE_DIR = os.path.dirname(oracle.__file__)


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- depths


def test_depths_closed_forms():
    gen = torch.Generator().manual_seed(0)
    par = W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen)
    level = [l for l, w in enumerate(W.LONGSPEC_TREE_WIDTHS) for _ in range(w)]
    assert oracle.depths(np.array([par]))[0].tolist() == level
    assert oracle.depths(np.array([W.chain_tree(9)]))[0].tolist() == list(range(9))
    heap = W.complete_binary_tree(5)
    assert oracle.depths(np.array([heap]))[0].tolist() == [
        int(math.floor(math.log2(i + 1))) for i in range(len(heap))]


@pytest.mark.parametrize("bad", [[-1, 1], [-2, 0], [-1, 0, 3], [0]])
def test_depths_reject_bad_trees(bad):
    with pytest.raises(oracle.OracleError):
        oracle.depths(np.array([bad], dtype=np.int32))


# ----------------------------------------------------------------------------- rotary


def test_rope_d2_rotates_by_the_position_in_radians():
    # D = 2: one pair with frequency theta^0 = 1, so node at position p turns by p radians.
    T = 1
    prefix = np.array([0, 1, 2, 5, 1000], dtype=np.int32)
    B = prefix.size
    par = np.full((B, T), -1, dtype=np.int32)
    x = np.zeros((B, T, 2, 2), dtype=np.float32)
    x[:, :, 0, 0] = 1.0  # head 0: (1, 0)
    x[:, :, 1, 1] = 1.0  # head 1: (0, 1)
    for theta in (10000.0, 3.0):
        out, pos = oracle.rope(x, par, prefix, theta)
        assert pos[:, 0].tolist() == prefix.tolist()
        for b, p in enumerate(prefix.tolist()):
            np.testing.assert_allclose(out[b, 0, 0], [math.cos(p), math.sin(p)], atol=1e-15)
            np.testing.assert_allclose(out[b, 0, 1], [-math.sin(p), math.cos(p)], atol=1e-15)


def test_rope_is_identity_at_position_zero():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 3, 4, 16)).astype(np.float32)
    par = np.array([[-1, -1, -1]], dtype=np.int32)
    for inter in (False, True):
        out, pos = oracle.rope(x, par, np.array([0]), 500000.0, interleaved=inter)
        assert (pos == 0).all()
        assert np.array_equal(out, x.astype(np.float64))


def _complex_rope(x64, pos, theta, interleaved):
    """x as complex pairs times exp(i * pos * theta^(-2j/D)); x64 [..., D], pos [...]."""
    D = x64.shape[-1]
    j = np.arange(D // 2)
    freq = np.power(float(theta), -2.0 * j / D)
    if interleaved:
        z = x64[..., 0::2] + 1j * x64[..., 1::2]
    else:
        z = x64[..., : D // 2] + 1j * x64[..., D // 2:]
    z = z * np.exp(1j * pos[..., None].astype(np.float64) * freq)
    out = np.empty_like(x64)
    if interleaved:
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    else:
        out[..., : D // 2], out[..., D // 2:] = z.real, z.imag
    return out


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_rope_matches_complex_exponentials(interleaved, theta):
    gen = torch.Generator().manual_seed(4)
    par = np.array([W.level_tree((2, 3, 3), gen), W.chain_tree(8)], dtype=np.int32)
    prefix = np.array([262144, 37], dtype=np.int32)
    depth = np.array([W.depths(p) for p in par.tolist()])
    pos_ref = prefix[:, None] + depth
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 8, 3, 16)).astype(np.float32)
    k = rng.standard_normal((2, 2, 8, 16)).astype(np.float32)
    oq, pos = oracle.rope(q, par, prefix, theta, interleaved=interleaved, layout="q")
    ok, _ = oracle.rope(k, par, prefix, theta, interleaved=interleaved, layout="k")
    assert np.array_equal(pos, pos_ref)
    np.testing.assert_allclose(oq, _complex_rope(q.astype(np.float64), pos_ref[:, :, None],
                                                 theta, interleaved), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ok, _complex_rope(k.astype(np.float64), pos_ref[:, None, :],
                                                 theta, interleaved), rtol=0, atol=1e-12)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_scores_depend_on_the_position_difference_only(interleaved):
    # <R(m) q, R(n) k> = <R(m - n) q, k>: one root per sequence, position = prefix_len.
    rng = np.random.default_rng(6)
    D, m, n = 32, 70001, 1234
    v = rng.standard_normal((2, 1, 1, D)).astype(np.float32)
    par = np.full((1, 1), -1, dtype=np.int32)
    rq = lambda x, p: oracle.rope(x, par, np.array([p]), 10000.0, interleaved)[0][0, 0, 0]  # noqa: E731
    lhs = rq(v[:1], m) @ rq(v[1:], n)
    rhs = rq(v[:1], m - n) @ v[1, 0, 0].astype(np.float64)
    assert abs(lhs - rhs) < 1e-10 * (1 + abs(rhs))
    # and every pair keeps its length
    r = rq(v[:1], m)
    x = v[0, 0, 0].astype(np.float64)
    if interleaved:
        a, c = (r[0::2], r[1::2]), (x[0::2], x[1::2])
    else:
        a, c = (r[: D // 2], r[D // 2:]), (x[: D // 2], x[D // 2:])
    np.testing.assert_allclose(a[0] ** 2 + a[1] ** 2, c[0] ** 2 + c[1] ** 2, rtol=1e-13)


def test_rope_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((1, 2, 2, 8)).astype(np.float32)).to(torch.bfloat16)
    par = np.array([[-1, 0]], dtype=np.int32)
    o16, _ = oracle.rope(_bits(x), par, np.array([9]), 10000.0)
    o32, _ = oracle.rope(x.float().numpy(), par, np.array([9]), 10000.0)
    assert np.array_equal(o16, o32)


def test_rope_rejects_bad_trees():
    x = np.zeros((1, 2, 1, 4), dtype=np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.rope(x, np.array([[-1, 1]], dtype=np.int32), np.array([0]), 10000.0)


# ----------------------------------------------------------------------------- bf16 rounding


def _round_bf16_exact(x: float) -> int:
    """Nearest bf16 by exact rational comparison (ties to an even last bit)."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    ax = Fraction(abs(x))
    e = math.floor(math.log2(abs(x)))
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    lo = (ax // ulp) * ulp
    hi = lo + ulp
    if ax - lo < hi - ax:
        r = lo
    elif ax - lo > hi - ax:
        r = hi
    else:
        r = lo if (lo / ulp) % 2 == 0 else hi
    f = np.float32(float(r))  # r has at most 8 significant bits: exact
    return sign | int(np.array([f]).view(np.uint32)[0] >> 16)


def test_round_bf16_single_rounding():
    rng = np.random.default_rng(8)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000)))
    ties = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * 2.0 ** -9]
    # just above a tie: a detour through fp32 would round to the tie and then to even
    above = [1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8 + 2.0 ** -30]
    vals += ties + above + [0.0, -0.0, 1.0, 2.0 ** -100]
    x = np.array(vals, dtype=np.float64)
    got = oracle.round_bf16(x)
    want = np.array([_round_bf16_exact(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert got[len(vals) - 4 - 2 - 4] == 0x3F80  # 1 + 2^-8 -> 1.0 (even)
    assert got[len(vals) - 4 - 2 - 3] == 0x3F82  # 1 + 3 2^-8 -> 1 + 2^-6
    assert got[len(vals) - 4 - 2] == 0x3F81      # above the tie -> up
    assert oracle.round_bf16(np.array([np.nan]))[0] & 0x7F80 == 0x7F80
    assert oracle.round_bf16(np.array([1e300]))[0] == 0x7F80


# ----------------------------------------------------------------------------- argmax


def test_argmax_matches_numpy_first_maximum():
    rng = np.random.default_rng(9)
    x = rng.integers(-3, 4, size=(200, 37)).astype(np.float32)  # many ties
    x[5, 7] = np.nan
    x[5, 30] = np.nan
    x[6, :] = 0.0
    x[6, 3] = -0.0
    x[7, :] = -0.0
    x[7, 9] = 0.0  # -0 == +0: the first element wins
    x[8, 36] = np.inf
    x[9, :] = -np.inf
    assert np.array_equal(oracle.argmax(x), np.argmax(x, axis=1))
    xb = torch.from_numpy(rng.standard_normal((3, 5, 1001)).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(oracle.argmax(_bits(xb)), np.argmax(xb.float().numpy(), axis=-1))
    assert oracle.argmax(np.array([[4.0]], dtype=np.float32)).tolist() == [0]


# ----------------------------------------------------------------------------- acceptance


def _toy_target(context, vocab):
    """A deterministic 'target model': the next token is a fixed function of the context."""
    h = 0
    for t in context:
        h = (h * 1000003 + t + 17) % 2147483647
    return h % vocab


def _tree_drafts(parents, prefix, vocab, rng, p_good):
    """Draft tokens: each node carries the toy target's token for its context with
    probability p_good, else another token; siblings carry distinct tokens."""
    T = len(parents)
    tok = [0] * T
    ctx = {}
    for i, p in enumerate(parents):
        base = prefix if p < 0 else ctx[p]
        good = _toy_target(base, vocab)
        sib = [tok[j] for j in range(i) if parents[j] == p]
        if rng.random() < p_good and good not in sib:
            tok[i] = good
        else:
            choices = [t for t in range(vocab) if t != good and t not in sib]
            tok[i] = int(rng.choice(choices))
        ctx[i] = base + [tok[i]]
    return tok, ctx


def test_accept_is_lossless_greedy_decoding():
    rng = np.random.default_rng(10)
    gen = torch.Generator().manual_seed(11)
    vocab = 50
    seen = set()
    for trial in range(60):
        par = (W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) if trial % 3 else
               W.random_forest(12, gen) if trial % 2 else W.chain_tree(6))
        prefix = [int(t) for t in rng.integers(0, vocab, 5)]
        tok, ctx = _tree_drafts(par, prefix, vocab, rng, p_good=0.6)
        nxt = [_toy_target(ctx[i], vocab) for i in range(len(par))]
        root = _toy_target(prefix, vocab)
        n, acc, bonus = oracle.accept(np.array([par]), np.array([tok]), np.array([root]),
                                      np.array([nxt]))
        n = int(n[0])
        emitted = [tok[i] for i in acc[0, :n]] + [int(bonus[0])]
        # plain greedy decoding of the toy target for n + 1 tokens
        c = list(prefix)
        for _ in range(n + 1):
            c.append(_toy_target(c, vocab))
        assert emitted == c[len(prefix):]
        # the path is a chain of parent links, padded with -1
        assert all(par[acc[0, k]] == (acc[0, k - 1] if k else -1) for k in range(n))
        assert (acc[0, n:] == -1).all()
        # and it is the longest matching path (siblings are distinct here)
        deepest = 0
        for i in range(len(par)):
            path, p = [], i
            while p != -1:
                path.append(p)
                p = par[p]
            path.reverse()
            if all(tok[j] == _toy_target(ctx[j][:-1], vocab) for j in path):
                deepest = max(deepest, len(path))
        assert n == deepest
        seen.add(n)
    assert len(seen) >= 4  # the trials cover several acceptance lengths


def test_accept_hand_cases():
    par = np.array([[-1, -1, 0, 0, 1, 2]], dtype=np.int32)
    tok = np.array([[7, 7, 3, 3, 3, 9]], dtype=np.int32)
    nxt = np.array([[3, 3, 9, 5, 8, 4]], dtype=np.int32)
    # two roots carry the expected token 7: the smaller index (0) is taken; then its
    # children 2 and 3 both carry 3: node 2; then node 5 (token 9); bonus = nxt[5] = 4
    n, acc, bonus = oracle.accept(par, tok, np.array([7]), nxt)
    assert n.tolist() == [3] and acc[0].tolist() == [0, 2, 5, -1, -1, -1] and bonus[0] == 4
    # no root matches: nothing accepted, the target's own token is emitted
    n, acc, bonus = oracle.accept(par, tok, np.array([1]), nxt)
    assert n.tolist() == [0] and (acc == -1).all() and bonus[0] == 1
    # a chain whose every token matches is accepted whole
    chain = np.array([W.chain_tree(4)], dtype=np.int32)
    n, acc, bonus = oracle.accept(chain, np.array([[5, 6, 7, 8]]), np.array([5]),
                                  np.array([[6, 7, 8, 2]]))
    assert n.tolist() == [4] and acc[0].tolist() == [0, 1, 2, 3] and bonus[0] == 2


# ----------------------------------------------------------------------------- KV commit


def test_commit_then_prefix_attention_equals_tree_attention():
    # After committing the accepted path, the last accepted node's query attends to the
    # grown prefix exactly as it attended to prefix + ancestors-or-self during verification.
    from helpers import tiny_workload

    par = [-1, -1, 0, 1, 2, 2, 4]
    w = tiny_workload(par, B=2, Hq=4, Hkv=2, D=8, L=12, prefix_len=[6, 9], seed=12)
    a = w.as_numpy()
    acc = np.array([[0, 2, 4, -1, -1, -1, -1], [1, 3, -1, -1, -1, -1, -1]], dtype=np.int32)
    n = np.array([3, 2], dtype=np.int32)
    kp, vp, pl, full = oracle.kv_commit(a["k_prefix"], a["v_prefix"], a["k_tree"], a["v_tree"],
                                        a["prefix_len"], n, acc)
    assert not full.any() and pl.tolist() == [9, 11]
    ref_out, ref_lse = oracle.verify(a, w.scale)
    b2 = dict(a, k_prefix=kp, v_prefix=vp, prefix_len=pl)
    for b in range(2):
        last = int(acc[b, n[b] - 1])
        rows = [(b, h, last) for h in range(4)]
        out, lse = oracle.rows(b2, w.scale, *zip(*rows), part=oracle.PART_PREFIX)
        np.testing.assert_allclose(out, ref_out[b, last], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse[b, :, last], rtol=0, atol=1e-13)
    # untouched rows stay untouched
    assert np.array_equal(kp[0, :, :6], a["k_prefix"][0, :, :6])
    assert np.array_equal(kp[0, :, 9:], a["k_prefix"][0, :, 9:])
    # a path that does not fit leaves the sequence unchanged
    n_big = np.array([3, 4], dtype=np.int32)
    acc_big = np.array([[0, 2, 4, -1, -1, -1, -1], [1, 3, 6, 5, -1, -1, -1]], dtype=np.int32)
    kp, vp, pl, full = oracle.kv_commit(a["k_prefix"], a["v_prefix"], a["k_tree"], a["v_tree"],
                                        a["prefix_len"], n_big, acc_big)
    assert full.tolist() == [False, True] and pl.tolist() == [9, 9]
    assert np.array_equal(kp[1], a["k_prefix"][1]) and np.array_equal(vp[1], a["v_prefix"][1])


# ----------------------------------------------------------------------------- mutants

STEP_SRC = os.path.join(ORACLE_DIR, "step_oracle.c")
ATTN_SRC = os.path.join(ORACLE_DIR, "hta_oracle.c")

MUTANTS = {
    "depth_from_one": ("            int d = 0;\n            for (int p = par[i]",
                       "            int d = 1;\n            for (int p = par[i]"),
    "position_without_prefix": ("const int64_t pos = (int64_t)prefix_len[b] + depth;",
                                "const int64_t pos = depth;"),
    "pairs_adjacent_in_half_layout": ("const int c = interleaved ? 2 * j + 1 : j + half;",
                                      "const int c = interleaved ? 2 * j + 1 : j + 1;"),
    "rotation_sign": ("out[row + a] = xa * cs - xc * sn;", "out[row + a] = xa * cs + xc * sn;"),
    "frequency_exponent": ("pow(theta, -2.0 * (double)j / (double)D)",
                           "pow(theta, -1.0 * (double)j / (double)D)"),
    "q_layout_transposed": ("const size_t row = layout == 0 ? (((size_t)b * T + i) * H + h) * D",
                            "const size_t row = layout == 0 ? (((size_t)b * H + h) * T + i) * D"),
    "round_truncates": ("const uint64_t half_ulp = (1ull << (drop - 1)) - 1 + ((u >> drop) & 1);",
                        "const uint64_t half_ulp = 0;"),
    "round_ties_up": ("const uint64_t half_ulp = (1ull << (drop - 1)) - 1 + ((u >> drop) & 1);",
                      "const uint64_t half_ulp = (1ull << (drop - 1));"),
    "argmax_last_tie": ("if (isnan(v) || v > bv) {", "if (isnan(v) || v >= bv) {"),
    "argmax_ignores_nan": ("if (isnan(v) || v > bv) {", "if (v > bv) {"),
    "accept_largest_index": ("                    chosen = i;\n                    break;",
                             "                    chosen = i;"),
    "bonus_not_advanced": ("            expect = nxt[chosen];", "            ;"),
    "accept_ignores_parent": ("if (par[i] == last && tok[i] == expect)", "if (tok[i] == expect)"),
}

STEP_PINS = [
    test_depths_closed_forms,
    test_rope_d2_rotates_by_the_position_in_radians,
    lambda: [test_rope_matches_complex_exponentials(i, t) for i in (False, True)
             for t in (10000.0, 500000.0)],
    test_round_bf16_single_rounding,
    test_argmax_matches_numpy_first_maximum,
    test_accept_is_lossless_greedy_decoding,
    test_accept_hand_cases,
]


@contextlib.contextmanager
def _swapped(path):
    old = oracle._lib
    oracle._lib = oracle.configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        oracle._lib = old


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_step_mutant_fails_a_pin(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(STEP_SRC).read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    c = tmp_path / "step_mutant.c"
    so = tmp_path / "libstepmutant.so"
    c.write_text(src.replace(before, after, 1))
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-std=c11", "-shared", "-fPIC",
                           ATTN_SRC, str(c), "-o", str(so), "-lm"])
    failed = []
    with _swapped(str(so)):
        for pin in STEP_PINS:
            try:
                pin()
            except (AssertionError, oracle.OracleError):
                failed.append(pin)
    assert failed, f"mutant {name} survived every pin"


def test_window_commit_keeps_the_last_positions():
    """Commit a stream of paths into a small ring; afterwards slot s must hold the latest
    committed position p with p % W == s (a closed form of the ring), checked against the
    full history written out position by position."""
    rng = np.random.default_rng(13)
    B, Hkv, W, D, T = 2, 2, 5, 3, 7
    kw = np.zeros((B, Hkv, W, D), dtype=np.float32)
    vw = np.zeros_like(kw)
    pos = np.zeros((B,), dtype=np.int32)
    history = [[], []]  # per sequence: (k row, v row) of every committed position
    for step in range(9):
        kt = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
        vt = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
        n = rng.integers(0, T + 1, size=B).astype(np.int32)
        acc = np.full((B, T), -1, dtype=np.int32)
        for b in range(B):
            acc[b, :n[b]] = rng.permutation(T)[:n[b]]
            history[b] += [(kt[b, :, acc[b, k]], vt[b, :, acc[b, k]]) for k in range(n[b])]
        kw, vw, pos = oracle.window_commit(kw, vw, kt, vt, acc, n, pos)
        for b in range(B):
            assert pos[b] == len(history[b])
            for p in range(max(0, pos[b] - W), pos[b]):
                assert np.array_equal(kw[b, :, p % W], history[b][p][0])
                assert np.array_equal(vw[b, :, p % W], history[b][p][1])
