"""Seeded synthetic inputs for tree verification attention.

This module only draws numbers: it holds none of the attention arithmetic. Both the
CPU oracle (via the tests) and the HIP path consume what it produces, so the two never
share anything else.

Workload shapes stand in for the evaluation runs described on the LongSpec pages:

* the draft tree has level widths 4,16,16,16,16 (LongSpec README, Evaluation: the
  ``--tree_shape`` flag of both inference commands), i.e. 68 nodes; every node's parent is
  drawn uniformly from the previous level, level-0 nodes hang off the prefix (parent -1);
* Llama-3-8B-Instruct-262k layer shape (README, Evaluation) at 32k and 262k prefixes;
* Vicuna-7B at batch 8 (paper summary, Key points: the RepoBench-P throughput figure);
* QwQ-32B decode sweep, outputs up to 32k tokens (paper summary, Key points).

No dataset item is used: attention cost depends only on shapes, so the prefixes are
N(0, 1) noise.  Layouts (row-major, contiguous):

* ``q``                    [B, T, Hq, D]
* ``k_prefix``, ``v_prefix`` [B, Hkv, Lmax, D]
* ``k_tree``, ``v_tree``     [B, Hkv, T, D]
* ``parent_idx``           [B, T] int32, ``-1`` = child of the prefix
* ``prefix_len``           [B] int32
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

LONGSPEC_TREE_WIDTHS = (4, 16, 16, 16, 16)


@dataclasses.dataclass
class Workload:
    """One verification-attention problem (all tensors on the CPU)."""

    name: str
    q: torch.Tensor
    k_prefix: torch.Tensor
    v_prefix: torch.Tensor
    k_tree: torch.Tensor
    v_tree: torch.Tensor
    parent_idx: torch.Tensor
    prefix_len: torch.Tensor
    scale: float
    seed: int = 0

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def tree_size(self) -> int:
        return self.q.shape[1]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[2]

    @property
    def head_dim(self) -> int:
        return self.q.shape[3]

    @property
    def num_kv_heads(self) -> int:
        return self.k_prefix.shape[1]

    @property
    def max_prefix_len(self) -> int:
        return self.k_prefix.shape[2]

    @property
    def dtype(self) -> torch.dtype:
        return self.q.dtype

    def as_numpy(self) -> Dict[str, np.ndarray]:
        """Zero-copy numpy views; bf16 tensors come out as their raw uint16 bit patterns."""

        def view(t: torch.Tensor) -> np.ndarray:
            t = t.contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()

        return {
            "q": view(self.q),
            "k_prefix": view(self.k_prefix),
            "v_prefix": view(self.v_prefix),
            "k_tree": view(self.k_tree),
            "v_tree": view(self.v_tree),
            "parent_idx": self.parent_idx.numpy(),
            "prefix_len": self.prefix_len.numpy(),
        }


# ----------------------------------------------------------------------------- trees


def level_tree(widths: Sequence[int], gen: torch.Generator) -> List[int]:
    """Parents of a tree stored level by level; each parent uniform over the previous level."""
    parents: List[int] = []
    prev_start, prev_width = 0, 0
    for lvl, w in enumerate(widths):
        start = len(parents)
        for _ in range(w):
            if lvl == 0:
                parents.append(-1)
            else:
                parents.append(prev_start + int(torch.randint(0, prev_width, (1,), generator=gen)))
        prev_start, prev_width = start, w
    return parents


def complete_binary_tree(levels: int) -> List[int]:
    """Heap-ordered complete binary tree: node i>0 has parent (i-1)//2; root hangs off the prefix."""
    n = (1 << levels) - 1
    return [-1] + [(i - 1) // 2 for i in range(1, n)]


def chain_tree(depth: int) -> List[int]:
    """A single path of ``depth`` nodes (the degenerate tree: plain causal draft)."""
    return [i - 1 for i in range(depth)]


def star_tree(n: int) -> List[int]:
    """Every node a child of the prefix."""
    return [-1] * n


def random_forest(n: int, gen: torch.Generator) -> List[int]:
    """Random topologically ordered forest: parent of node i uniform over {-1, 0, ..., i-1}."""
    return [int(torch.randint(-1, i, (1,), generator=gen)) if i > 0 else -1 for i in range(n)]


def depths(parents: Sequence[int]) -> List[int]:
    d: List[int] = []
    for i, p in enumerate(parents):
        d.append(0 if p < 0 else d[p] + 1)
    return d


# ----------------------------------------------------------------------------- builder


def make_workload(
    name: str,
    *,
    batch: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    max_prefix_len: int,
    parents: Optional[Sequence[Sequence[int]]] = None,
    tree_widths: Optional[Sequence[int]] = None,
    prefix_len: Optional[Sequence[int]] = None,
    prefix_len_range: Optional[Sequence[int]] = None,
    dtype: torch.dtype = torch.bfloat16,
    peaky_frac: float = 0.0,
    peaky_scale: float = 4.0,
    poison_padding: bool = False,
    seed: int = 0,
    scale: Optional[float] = None,
) -> Workload:
    """Draw one workload.

    Draw order (fixed, so a seed names the bits): prefix lengths, tree parents, q,
    k_prefix, v_prefix, k_tree, v_tree, then the peaky-key selectors.  Peaky keys: an
    independent Bernoulli(``peaky_frac``) per (sequence, kv head, key) over prefix and tree
    keys; selected K rows are multiplied by ``peaky_scale`` before the cast.
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    B, Hq, Hkv, D, Lmax = batch, num_q_heads, num_kv_heads, head_dim, max_prefix_len
    if prefix_len_range is not None:
        lo, hi = prefix_len_range
        plen = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64)
    elif prefix_len is not None:
        plen = torch.tensor(list(prefix_len), dtype=torch.int64)
    else:
        plen = torch.full((B,), Lmax, dtype=torch.int64)
    if parents is None:
        assert tree_widths is not None
        parents = [level_tree(tree_widths, gen) for _ in range(B)]
    parents = [list(p) for p in parents]
    T = len(parents[0])
    assert all(len(p) == T for p in parents)

    q = torch.randn(B, T, Hq, D, generator=gen)
    kp = torch.randn(B, Hkv, Lmax, D, generator=gen)
    vp = torch.randn(B, Hkv, Lmax, D, generator=gen)
    kt = torch.randn(B, Hkv, T, D, generator=gen)
    vt = torch.randn(B, Hkv, T, D, generator=gen)
    if peaky_frac > 0:
        sel_p = torch.rand(B, Hkv, Lmax, generator=gen) < peaky_frac
        sel_t = torch.rand(B, Hkv, T, generator=gen) < peaky_frac
        kp[sel_p] *= peaky_scale
        kt[sel_t] *= peaky_scale
        del sel_p, sel_t
    if poison_padding:
        for b in range(B):
            kp[b, :, int(plen[b]):, :] = float("nan")
            vp[b, :, int(plen[b]):, :] = float("nan")
    if dtype != torch.float32:
        q, kp, vp, kt, vt = (t.to(dtype) for t in (q, kp, vp, kt, vt))
    return Workload(
        name=name,
        q=q.contiguous(),
        k_prefix=kp.contiguous(),
        v_prefix=vp.contiguous(),
        k_tree=kt.contiguous(),
        v_tree=vt.contiguous(),
        parent_idx=torch.tensor(parents, dtype=torch.int32),
        prefix_len=plen.to(torch.int32),
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
        seed=seed,
    )


# ----------------------------------------------------------------------------- step inputs

# Vocabulary sizes and rotary bases of the checkpoints the LongSpec README evaluates (from
# their public model configurations): Llama-3-8B, Vicuna-7B (a Llama-2 model), QwQ-32B.
LLAMA3_VOCAB, VICUNA_VOCAB, QWQ_VOCAB = 128256, 32000, 152064
LLAMA3_ROPE_THETA, VICUNA_ROPE_THETA, QWQ_ROPE_THETA = 500000.0, 10000.0, 1000000.0


@dataclasses.dataclass
class StepInputs:
    """What one greedy verification step needs besides the attention inputs (CPU tensors).

    ``tokens`` [B, T] int32: the drafted token of every tree node; ``root_token`` [B] int32:
    the target's token for the position after the prefix (known from the previous step);
    ``logits`` [B, T, V]: the target's scores after every node; ``planted`` [B, T] int32:
    the token whose score was raised above every other in that row."""

    tokens: torch.Tensor
    root_token: torch.Tensor
    logits: torch.Tensor
    planted: torch.Tensor

    @property
    def vocab(self) -> int:
        return self.logits.shape[-1]


def make_step_inputs(parents: Sequence[Sequence[int]], vocab: int, *, p_root: float = 0.95,
                     p_follow: float = 0.85, dtype: torch.dtype = torch.bfloat16,
                     planted_score: float = 12.0, seed: int = 0) -> StepInputs:
    """Draw tokens and logits for a batch of draft trees.

    Draw order (fixed): tokens uniform in [0, vocab); per sequence a Bernoulli(``p_root``)
    and a uniform root choice -- on success ``root_token`` is that root's token, otherwise a
    uniform token; per node a Bernoulli(``p_follow``) and a uniform child choice -- on
    success (and if the node has children) the planted token is that child's token,
    otherwise a uniform token; then N(0, 1) logits.  The planted token's score is set to
    ``planted_score`` (above every N(0, 1) draw of a realistic vocabulary).  With the
    defaults the greedy walk accepts about 2.4 of the 5 levels of the 4,16,16,16,16 tree
    (3.4 tokens a step with the target's own token), near the mean acceptance length of
    about 3.8 the LongSpec paper summary reports for QwQ-32B."""
    gen = torch.Generator("cpu").manual_seed(seed)
    B = len(parents)
    T = len(parents[0])
    tokens = torch.randint(0, vocab, (B, T), generator=gen, dtype=torch.int64)
    root = torch.empty(B, dtype=torch.int64)
    planted = torch.empty(B, T, dtype=torch.int64)
    for b in range(B):
        par = list(parents[b])
        roots = [i for i in range(T) if par[i] == -1]
        hit = bool(torch.rand(1, generator=gen) < p_root)
        pick = int(torch.randint(0, max(len(roots), 1), (1,), generator=gen))
        other = int(torch.randint(0, vocab, (1,), generator=gen))
        root[b] = int(tokens[b, roots[pick]]) if (hit and roots) else other
        for i in range(T):
            kids = [c for c in range(T) if par[c] == i]
            hit = bool(torch.rand(1, generator=gen) < p_follow)
            pick = int(torch.randint(0, max(len(kids), 1), (1,), generator=gen))
            other = int(torch.randint(0, vocab, (1,), generator=gen))
            planted[b, i] = int(tokens[b, kids[pick]]) if (hit and kids) else other
    logits = torch.randn(B, T, vocab, generator=gen)
    logits.scatter_(2, planted.unsqueeze(-1), planted_score)
    return StepInputs(tokens=tokens.to(torch.int32), root_token=root.to(torch.int32),
                      logits=logits.to(dtype).contiguous(), planted=planted.to(torch.int32))


# ----------------------------------------------------------------------------- named configs

QWQ_PREFIXES = (4096, 8192, 16384, 32768)


def tiny(seed: int = 1001) -> Workload:
    """Batch 1, 4 query heads = 4 KV heads, D 64, prefix 1024, 7-node complete binary tree, fp32."""
    return make_workload(
        "tiny_fp32", batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64, max_prefix_len=1024,
        parents=[complete_binary_tree(3)], dtype=torch.float32, seed=seed, scale=1.0 / 8.0,
    )


def llama3_8b(prefix: int = 32768, seed: Optional[int] = None) -> Workload:
    """Llama-3-8B layer: 32 query / 8 KV heads, D 128, 68-node tree, 2% of keys scaled x4, bf16."""
    if seed is None:
        seed = 1002 if prefix == 32768 else 1003
    return make_workload(
        f"llama3_8b_{prefix // 1024}k", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        max_prefix_len=prefix, tree_widths=LONGSPEC_TREE_WIDTHS, peaky_frac=0.02, seed=seed,
    )


def vicuna_7b_b8(seed: int = 1004, poison_padding: bool = True) -> Workload:
    """Vicuna-7B layer at batch 8: MHA 32/32 heads, D 128, prefixes uniform in [8192, 16384]."""
    return make_workload(
        "vicuna7b_b8", batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128,
        max_prefix_len=16384, prefix_len_range=(8192, 16384), tree_widths=LONGSPEC_TREE_WIDTHS,
        poison_padding=poison_padding, seed=seed,
    )


def qwq_32b(prefix: int, chain: bool = False, seed: Optional[int] = None) -> Workload:
    """QwQ-32B layer: 40 query / 8 KV heads, D 128; the 68-node tree or a depth-5 chain."""
    k = QWQ_PREFIXES.index(prefix)
    if seed is None:
        seed = 1010 + 2 * k + (1 if chain else 0)
    kind = "chain5" if chain else "tree"
    return make_workload(
        f"qwq32b_{kind}_{prefix // 1024}k", batch=1, num_q_heads=40, num_kv_heads=8, head_dim=128,
        max_prefix_len=prefix,
        parents=[chain_tree(5)] if chain else None,
        tree_widths=None if chain else LONGSPEC_TREE_WIDTHS, seed=seed,
    )


CONFIG_NAMES = (
    "tiny_fp32",
    "llama3_8b_32k",
    "llama3_8b_256k",
    "vicuna7b_b8",
) + tuple(f"qwq32b_{k}_{p // 1024}k" for p in QWQ_PREFIXES for k in ("tree", "chain5"))


def by_name(name: str) -> Workload:
    if name == "tiny_fp32":
        return tiny()
    if name == "llama3_8b_32k":
        return llama3_8b(32768)
    if name == "llama3_8b_256k":
        return llama3_8b(262144)
    if name == "vicuna7b_b8":
        return vicuna_7b_b8()
    if name.startswith("qwq32b_"):
        _, kind, size = name.split("_")
        return qwq_32b(int(size[:-1]) * 1024, chain=(kind == "chain5"))
    raise KeyError(name)
