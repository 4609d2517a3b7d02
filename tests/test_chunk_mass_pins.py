"""Pins of the chunk-mass oracle (oracle/hta_oracle.c, hta_oracle_chunk_mass): each prefix
chunk's (and the tree's) share of a query row's attention.

Checked against: the row sum (1), the closed form for a zero query (uniform weights), the
log-sum-exps of the same row restricted to one chunk computed by the general masked
attention oracle (mass = exp(lse_chunk - lse_row)), and a single chunk covering the whole
prefix.  Planted mistakes in a copy of the oracle each fail one of them.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from tree_verification_attention_amd import workloads as W

from helpers import tiny_workload

ORACLE_DIR = os.path.dirname(oracle.__file__)


def _all_rows(B, Hq, T):
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(T)]
    return [list(x) for x in zip(*rows)]


def test_rows_sum_to_one():
    gen = torch.Generator().manual_seed(3)
    par = [W.level_tree((2, 3, 3), gen), W.random_forest(8, gen)]
    w = tiny_workload(par, B=2, Hq=4, Hkv=2, D=8, L=40, prefix_len=[40, 13], seed=4,
                      dtype=torch.bfloat16, peaky=0.3)
    m = oracle.chunk_mass(w.as_numpy(), w.scale, 16, 3, *_all_rows(2, 4, 8))
    np.testing.assert_allclose(m.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (m >= 0).all()
    # sequence 1 has 13 prefix keys: chunks 1 and 2 are empty
    assert (m[32:, 1:3] == 0).all()


def test_zero_query_gives_uniform_weights():
    par = [-1, 0, 0, 1, 3, -1]
    L, chunk = 23, 8
    w = tiny_workload(par, B=1, Hq=2, Hkv=1, D=4, L=30, prefix_len=[L], seed=5)
    w.q.zero_()
    m = oracle.chunk_mass(w.as_numpy(), w.scale, chunk, 4, *_all_rows(1, 2, 6))
    dep = W.depths(par)
    for r, (h, i) in enumerate((h, i) for h in range(2) for i in range(6)):
        n = L + dep[i] + 1
        want = [min(chunk, max(0, L - s * chunk)) / n for s in range(4)] + [(dep[i] + 1) / n]
        np.testing.assert_allclose(m[r], want, rtol=0, atol=1e-15)


def test_mass_is_the_chunk_lse_against_the_row_lse():
    gen = torch.Generator().manual_seed(6)
    par = W.level_tree((2, 2, 4), gen)
    L, chunk, D = 50, 16, 8
    w = tiny_workload(par, B=1, Hq=2, Hkv=1, D=D, L=L, seed=7, peaky=0.2)
    T = len(par)
    m = oracle.chunk_mass(w.as_numpy(), w.scale, chunk, 4, *_all_rows(1, 2, T))
    k = torch.cat([w.k_prefix[0, 0], w.k_tree[0, 0]]).double().numpy()
    v = torch.cat([w.v_prefix[0, 0], w.v_tree[0, 0]]).double().numpy()
    r = 0
    for h in range(2):
        for i in range(T):
            qi = w.q[0, i, h].double().numpy()[None]
            anc = set()
            p = i
            while p != -1:
                anc.add(p)
                p = par[p]
            visible = np.array([j < L or (j - L) in anc for j in range(L + T)])
            _, lse_row = oracle.masked_attention(qi, k, v, visible[None], w.scale)
            for s in range(5):
                sel = (np.arange(L + T) // chunk == s) & (np.arange(L + T) < L) if s < 4 else \
                    (np.arange(L + T) >= L)
                _, lse_s = oracle.masked_attention(qi, k, v, (visible & sel)[None], w.scale)
                want = 0.0 if lse_s[0] == -np.inf else math.exp(lse_s[0] - lse_row[0])
                assert abs(m[r, s] - want) < 1e-13
            r += 1


def test_one_chunk_covering_the_prefix():
    par = W.chain_tree(4)
    w = tiny_workload(par, B=1, Hq=2, Hkv=2, D=8, L=20, seed=8)
    m = oracle.chunk_mass(w.as_numpy(), w.scale, 64, 1, *_all_rows(1, 2, 4))
    np.testing.assert_allclose(m[:, 0] + m[:, 1], 1.0, atol=1e-14)
    assert m.shape == (8, 2) and (m[:, 0] > 0).all()


def test_rejects_bad_arguments():
    w = tiny_workload([-1, 0], B=1, Hq=2, Hkv=1, D=4, L=20, seed=9)
    with pytest.raises(oracle.OracleError):
        oracle.chunk_mass(w.as_numpy(), w.scale, 8, 2, [0], [0], [0])  # 16 < Lmax
    a = w.as_numpy()
    a["parent_idx"] = np.array([[-1, 1]], dtype=np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.chunk_mass(a, w.scale, 8, 3, [0], [0], [0])


# ----------------------------------------------------------------------------- mutants

SRC = os.path.join(ORACLE_DIR, "hta_oracle.c")
STEP_SRC = os.path.join(ORACLE_DIR, "step_oracle.c")

MUTANTS = {
    "chunk_boundary_shifted": ("const int bin = j < L ? j / chunk : nchunks;",
                               "const int bin = j < L ? (j + 1) / chunk : nchunks;"),
    "tree_share_dropped": ("            const int bin = j < L ? j / chunk : nchunks;\n            row[bin] += ",
                           "            if (j >= L) continue;\n            const int bin = j / chunk;\n            row[bin] += "),
    "not_normalised": ("row[bin] += exp(scores[j] - m) / Z;", "row[bin] += exp(scores[j] - m);"),
    "scale_dropped": ("scores[j] = s * scale;", "scores[j] = s;"),
    "self_not_in_tree": ("        for (int p = i; p != -1; p = par[p])\n            in_tree[p] = 1;\n        /* scores",
                         "        for (int p = par[i]; p != -1; p = par[p])\n            in_tree[p] = 1;\n        /* scores"),
}

PINS = [test_rows_sum_to_one, test_zero_query_gives_uniform_weights,
        test_mass_is_the_chunk_lse_against_the_row_lse, test_one_chunk_covering_the_prefix]


@contextlib.contextmanager
def _swapped(path):
    old = oracle._lib
    oracle._lib = oracle.configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        oracle._lib = old


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_chunk_mass_mutant_fails_a_pin(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    start = src.index("int hta_oracle_chunk_mass(")
    assert src.count(before, start) >= 1, f"mutation site for {name} not found"
    mutated = src[:start] + src[start:].replace(before, after, 1)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-std=c11", "-shared", "-fPIC",
                           str(c), STEP_SRC, "-o", str(so), "-lm"])
    failed = []
    with _swapped(str(so)):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, oracle.OracleError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} survived every pin"
