"""Pure-Python brute force of tree verification attention -- TEST INFRASTRUCTURE ONLY.

An independent second reading of the same definition the C oracle implements (LongSpec
paper summary, Summary, "Hybrid Tree Attention"; README, Introduction): each tree token
sees every prefix key and its own ancestors-or-self in the tree, under one softmax.  It is
written differently on purpose -- lists, ``math.exp`` without max subtraction, ``math.fsum``,
the ancestor set built by a fixed-point over child->parent edges rather than by walking up
-- so that a shared mistake is unlikely.  Only for tiny inputs.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def bf16_bits_to_float(bits: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def ancestor_sets(parents: Sequence[int]) -> List[set]:
    """anc[i] = {i} united with everything reachable through parent edges (fixed point)."""
    T = len(parents)
    anc = [{i} for i in range(T)]
    changed = True
    while changed:
        changed = False
        for i in range(T):
            grow = set()
            for a in anc[i]:
                p = parents[a]
                if p >= 0 and p not in anc[i]:
                    grow.add(p)
            if grow:
                anc[i] |= grow
                changed = True
    return anc


def attention_row(qrow: Sequence[float], keys: Sequence[Sequence[float]],
                  vals: Sequence[Sequence[float]], scale: float) -> Tuple[List[float], float]:
    if not keys:
        return [0.0] * len(qrow), -math.inf
    e = [math.exp(scale * math.fsum(a * b for a, b in zip(qrow, k))) for k in keys]
    Z = math.fsum(e)
    D = len(qrow)
    out = [math.fsum(e[j] * vals[j][d] for j in range(len(keys))) / Z for d in range(D)]
    return out, math.log(Z)


def verify(q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, scale):
    """Nested lists (or numpy arrays of floats) in the canonical layouts.

    Returns out[b][i][h][d] and lse[b][h][i] as nested lists.
    """
    B, T, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k_prefix[0])
    G = Hq // Hkv
    out = [[[None] * Hq for _ in range(T)] for _ in range(B)]
    lse = [[[None] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        anc = ancestor_sets([int(x) for x in parent_idx[b]])
        L = int(prefix_len[b])
        for h in range(Hq):
            g = h // G
            for i in range(T):
                keys = [list(map(float, k_prefix[b][g][j])) for j in range(L)]
                vals = [list(map(float, v_prefix[b][g][j])) for j in range(L)]
                for t in sorted(anc[i]):
                    keys.append(list(map(float, k_tree[b][g][t])))
                    vals.append(list(map(float, v_tree[b][g][t])))
                o, l = attention_row(list(map(float, q[b][i][h])), keys, vals, scale)
                out[b][i][h] = o
                lse[b][h][i] = l
    return out, lse
