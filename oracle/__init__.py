"""CPU oracle for tree verification attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The HIP library and its Python binding never do: the two sides
share nothing but the seeded input generators.

The arithmetic lives in ``hta_oracle.c`` (the attention) and ``step_oracle.c`` (the steps
around it: rotary positions of the tree, the target's argmax, greedy acceptance); both are
plain C, fp64, single-threaded, and their headers state the definitions and the passages
they follow.  ``kv_commit`` below is plain numpy indexing.  This module only builds it with gcc,
loads it with ctypes and marshals numpy arrays.  ``bruteforce.py`` is an independent
pure-Python version used to pin the C code on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hta_oracle.c")
_SRC_STEP = os.path.join(_HERE, "step_oracle.c")
_LIB = os.path.join(_HERE, "libhta_oracle.so")

PART_ALL, PART_PREFIX, PART_TREE = 0, 1, 2
OK, BAD_TREE, BAD_ARG, NOMEM = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fno-fast-math", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
             _SRC, _SRC_STEP, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib: Optional[ctypes.CDLL] = None


def configure(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    i = ctypes.c_int
    L.hta_oracle_rows.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, P, ctypes.c_double,
                                  i, i, P, P, P, P, P]
    L.hta_oracle_verify.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, P,
                                    ctypes.c_double, i, P, P]
    L.hta_oracle_masks.argtypes = [i, i, P, P]
    L.hta_oracle_check_tree.argtypes = [i, i, P]
    L.hta_oracle_masked_attention.argtypes = [i, i, i, P, P, P, P, ctypes.c_double, P, P]
    L.hta_oracle_lse_merge.argtypes = [i, i, P, P, P, P]
    L.hta_oracle_chunk_mass.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, ctypes.c_double,
                                        i, i, i, P, P, P, P]
    L.step_oracle_depths.argtypes = [i, i, P, P]
    L.step_oracle_rope.argtypes = [i, i, i, i, i, i, P, P, P, ctypes.c_double, i, P, P]
    L.step_oracle_round_bf16.argtypes = [ctypes.c_size_t, P, P]
    L.step_oracle_round_bf16.restype = None
    L.step_oracle_argmax.argtypes = [i, i, i, P, P]
    L.step_oracle_accept.argtypes = [i, i, P, P, P, P, P, P, P]
    for f in (L.hta_oracle_rows, L.hta_oracle_verify, L.hta_oracle_masks,
              L.hta_oracle_check_tree, L.hta_oracle_masked_attention, L.hta_oracle_lse_merge,
              L.hta_oracle_chunk_mass, L.step_oracle_depths, L.step_oracle_rope, L.step_oracle_argmax,
              L.step_oracle_accept):
        f.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    """The oracle library: the in-tree build (rebuilt when a source is newer), or the build
    HTA_ORACLE_LIBRARY names (e.g. one with sanitizers)."""
    global _lib
    if _lib is None and os.environ.get("HTA_ORACLE_LIBRARY"):
        _lib = configure(ctypes.CDLL(os.environ["HTA_ORACLE_LIBRARY"]))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
                os.path.getmtime(_SRC), os.path.getmtime(_SRC_STEP)):
            build(force=True)
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int) -> None:
    if rc == BAD_TREE:
        raise OracleError("invalid tree: parent_idx[i] must lie in [-1, i-1]")
    if rc != OK:
        raise OracleError(f"oracle error code {rc}")


def _inputs(arrs: Dict[str, np.ndarray]):
    q = np.ascontiguousarray(arrs["q"])
    if q.dtype == np.uint16:
        is_bf16 = 1
    elif q.dtype == np.float32:
        is_bf16 = 0
    else:
        raise TypeError("q must be bf16 bits (uint16) or float32")
    out = {"is_bf16": is_bf16, "q": q}
    for name in ("k_prefix", "v_prefix", "k_tree", "v_tree"):
        a = np.ascontiguousarray(arrs[name])
        if a.dtype != q.dtype:
            raise TypeError(f"{name} dtype {a.dtype} != q dtype {q.dtype}")
        out[name] = a
    out["parent_idx"] = np.ascontiguousarray(arrs["parent_idx"], dtype=np.int32)
    out["prefix_len"] = np.ascontiguousarray(arrs["prefix_len"], dtype=np.int32)
    B, T, Hq, D = q.shape
    Hkv, Lmax = out["k_prefix"].shape[1], out["k_prefix"].shape[2]
    assert out["k_prefix"].shape == (B, Hkv, Lmax, D)
    assert out["v_prefix"].shape == (B, Hkv, Lmax, D)
    assert out["k_tree"].shape == (B, Hkv, T, D)
    assert out["v_tree"].shape == (B, Hkv, T, D)
    assert out["parent_idx"].shape == (B, T)
    assert out["prefix_len"].shape == (B,)
    return out, (B, T, Hq, Hkv, D, Lmax)


def verify(arrs: Dict[str, np.ndarray], scale: float, part: int = PART_ALL
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Full verification attention: out [B,T,Hq,D] fp64, lse [B,Hq,T] fp64."""
    a, (B, T, Hq, Hkv, D, Lmax) = _inputs(arrs)
    out = np.empty((B, T, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    rc = lib().hta_oracle_verify(B, T, Hq, Hkv, D, Lmax, a["is_bf16"], _ptr(a["q"]),
                                 _ptr(a["k_prefix"]), _ptr(a["v_prefix"]), _ptr(a["k_tree"]),
                                 _ptr(a["v_tree"]), _ptr(a["parent_idx"]), _ptr(a["prefix_len"]),
                                 float(scale), int(part), _ptr(out), _ptr(lse))
    _check(rc)
    return out, lse


def rows(arrs: Dict[str, np.ndarray], scale: float, row_b: Sequence[int], row_h: Sequence[int],
         row_i: Sequence[int], part: int = PART_ALL) -> Tuple[np.ndarray, np.ndarray]:
    """Selected rows only: out [n, D], lse [n] for rows (b, h, i)."""
    a, (B, T, Hq, Hkv, D, Lmax) = _inputs(arrs)
    rb = np.ascontiguousarray(row_b, dtype=np.int32)
    rh = np.ascontiguousarray(row_h, dtype=np.int32)
    ri = np.ascontiguousarray(row_i, dtype=np.int32)
    n = rb.shape[0]
    assert rh.shape == (n,) and ri.shape == (n,)
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib().hta_oracle_rows(B, T, Hq, Hkv, D, Lmax, a["is_bf16"], _ptr(a["q"]),
                               _ptr(a["k_prefix"]), _ptr(a["v_prefix"]), _ptr(a["k_tree"]),
                               _ptr(a["v_tree"]), _ptr(a["parent_idx"]), _ptr(a["prefix_len"]),
                               float(scale), int(part), n, _ptr(rb), _ptr(rh), _ptr(ri),
                               _ptr(out), _ptr(lse))
    _check(rc)
    return out, lse


def chunk_mass(arrs: Dict[str, np.ndarray], scale: float, chunk: int, nchunks: int,
               row_b: Sequence[int], row_h: Sequence[int], row_i: Sequence[int]) -> np.ndarray:
    """Share of each selected row's attention on prefix chunk s (columns s < nchunks) and on
    the tree (column nchunks): fp64 [n, nchunks + 1], rows summing to 1."""
    a, (B, T, Hq, Hkv, D, Lmax) = _inputs(arrs)
    rb = np.ascontiguousarray(row_b, dtype=np.int32)
    rh = np.ascontiguousarray(row_h, dtype=np.int32)
    ri = np.ascontiguousarray(row_i, dtype=np.int32)
    n = rb.shape[0]
    mass = np.empty((n, nchunks + 1), dtype=np.float64)
    rc = lib().hta_oracle_chunk_mass(B, T, Hq, Hkv, D, Lmax, a["is_bf16"], _ptr(a["q"]),
                                     _ptr(a["k_prefix"]), _ptr(a["k_tree"]),
                                     _ptr(a["parent_idx"]), _ptr(a["prefix_len"]), float(scale),
                                     int(chunk), int(nchunks), n, _ptr(rb), _ptr(rh), _ptr(ri),
                                     _ptr(mass))
    _check(rc)
    return mass


def ancestor_masks(parent_idx: np.ndarray) -> np.ndarray:
    """Packed ancestor-or-self masks, uint64 [B, T, ceil(T/64)]."""
    par = np.ascontiguousarray(parent_idx, dtype=np.int32)
    B, T = par.shape
    W = (T + 63) // 64
    masks = np.zeros((B, T, W), dtype=np.uint64)
    _check(lib().hta_oracle_masks(B, T, _ptr(par), _ptr(masks)))
    return masks


def check_tree(parent_idx: np.ndarray) -> bool:
    par = np.ascontiguousarray(parent_idx, dtype=np.int32)
    B, T = par.shape
    return lib().hta_oracle_check_tree(B, T, _ptr(par)) == OK


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """General fp64 softmax attention with an explicit boolean mask [nq, nk]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    nq, D = q.shape
    nk = k.shape[0]
    assert k.shape == (nk, D) and v.shape == (nk, D) and m.shape == (nq, nk)
    out = np.empty((nq, D), dtype=np.float64)
    lse = np.empty((nq,), dtype=np.float64)
    _check(lib().hta_oracle_masked_attention(nq, nk, D, _ptr(q), _ptr(k), _ptr(v), _ptr(m),
                                             float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def lse_merge(lse_parts: np.ndarray, o_parts: np.ndarray) -> Tuple[np.ndarray, float]:
    """Exact LSE merge of partial attentions over disjoint key sets of one row."""
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    n, D = o.shape
    assert l.shape == (n,)
    out = np.empty((D,), dtype=np.float64)
    lse = np.empty((1,), dtype=np.float64)
    _check(lib().hta_oracle_lse_merge(n, D, _ptr(l), _ptr(o), _ptr(out), _ptr(lse)))
    return out, float(lse[0])


# ----------------------------------------------------------------------------- around the attention


def depths(parent_idx: np.ndarray) -> np.ndarray:
    """Depth of every tree node (0 for a node whose parent is -1), int32 [B, T]."""
    par = np.ascontiguousarray(parent_idx, dtype=np.int32)
    B, T = par.shape
    d = np.empty((B, T), dtype=np.int32)
    _check(lib().step_oracle_depths(B, T, _ptr(par), _ptr(d)))
    return d


def rope(x: np.ndarray, parent_idx: np.ndarray, prefix_len: np.ndarray, theta: float,
         interleaved: bool = False, layout: str = "q") -> Tuple[np.ndarray, np.ndarray]:
    """Rotary encoding of tree rows at positions prefix_len + depth, exact in fp64.

    x: bf16 bits (uint16) or float32, [B, T, H, D] for layout "q", [B, H, T, D] for "k".
    Returns (rotated fp64 array of x's shape, positions int32 [B, T])."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        is_bf16 = 1
    elif x.dtype == np.float32:
        is_bf16 = 0
    else:
        raise TypeError("x must be bf16 bits (uint16) or float32")
    par = np.ascontiguousarray(parent_idx, dtype=np.int32)
    pl = np.ascontiguousarray(prefix_len, dtype=np.int32)
    if layout == "q":
        B, T, H, D = x.shape
        lay = 0
    elif layout == "k":
        B, H, T, D = x.shape
        lay = 1
    else:
        raise ValueError(layout)
    assert par.shape == (B, T) and pl.shape == (B,)
    out = np.empty(x.shape, dtype=np.float64)
    pos = np.empty((B, T), dtype=np.int32)
    rc = lib().step_oracle_rope(B, T, H, D, lay, is_bf16, _ptr(x), _ptr(par), _ptr(pl),
                                float(theta), 1 if interleaved else 0, _ptr(out), _ptr(pos))
    _check(rc)
    return out, pos


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), nearest-even, one rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().step_oracle_round_bf16(x.size, _ptr(x), _ptr(out))
    return out


def argmax(logits: np.ndarray) -> np.ndarray:
    """Greedy token of each row of logits [..., V] (bf16 bits or float32): first maximum,
    NaN largest.  Returns int32 of shape logits.shape[:-1]."""
    lg = np.ascontiguousarray(logits)
    if lg.dtype == np.uint16:
        is_bf16 = 1
    elif lg.dtype == np.float32:
        is_bf16 = 0
    else:
        raise TypeError("logits must be bf16 bits (uint16) or float32")
    V = lg.shape[-1]
    rows = lg.size // V
    idx = np.empty(lg.shape[:-1], dtype=np.int32)
    _check(lib().step_oracle_argmax(rows, V, is_bf16, _ptr(lg), _ptr(idx)))
    return idx


def accept(parent_idx: np.ndarray, tokens: np.ndarray, root_token: np.ndarray,
           target_next: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Greedy acceptance along each tree: (accept_len [B], accepted [B, T] (-1 padded),
    bonus [B]), all int32."""
    par = np.ascontiguousarray(parent_idx, dtype=np.int32)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    root = np.ascontiguousarray(root_token, dtype=np.int32)
    nxt = np.ascontiguousarray(target_next, dtype=np.int32)
    B, T = par.shape
    assert tok.shape == (B, T) and nxt.shape == (B, T) and root.shape == (B,)
    n = np.empty((B,), dtype=np.int32)
    acc = np.empty((B, T), dtype=np.int32)
    bonus = np.empty((B,), dtype=np.int32)
    _check(lib().step_oracle_accept(B, T, _ptr(par), _ptr(tok), _ptr(root), _ptr(nxt), _ptr(n),
                                    _ptr(acc), _ptr(bonus)))
    return n, acc, bonus


def kv_commit(k_prefix: np.ndarray, v_prefix: np.ndarray, k_tree: np.ndarray,
              v_tree: np.ndarray, prefix_len: np.ndarray, accept_len: np.ndarray,
              accepted: np.ndarray):
    """Append the accepted path's tree keys and values to each sequence's prefix cache.

    Row k of the path (node accepted[b, k]) goes to cache row prefix_len[b] + k of every KV
    head, and prefix_len[b] grows by accept_len[b].  A sequence whose cache cannot hold the
    path (prefix_len + accept_len > Lmax) is left unchanged and reported in the returned
    ``full`` flags.  Returns new arrays (k_prefix, v_prefix, prefix_len, full)."""
    kp, vp = k_prefix.copy(), v_prefix.copy()
    pl = np.array(prefix_len, dtype=np.int32, copy=True)
    B, Hkv, Lmax, D = kp.shape
    full = np.zeros((B,), dtype=bool)
    for b in range(B):
        L, n = int(prefix_len[b]), int(accept_len[b])
        if L + n > Lmax:
            full[b] = True
            continue
        for k in range(n):
            node = int(accepted[b, k])
            kp[b, :, L + k, :] = k_tree[b, :, node, :]
            vp[b, :, L + k, :] = v_tree[b, :, node, :]
        pl[b] = L + n
    return kp, vp, pl, full


def window_commit(k_win: np.ndarray, v_win: np.ndarray, k_tree: np.ndarray, v_tree: np.ndarray,
                  accepted: np.ndarray, accept_len: np.ndarray, win_pos: np.ndarray):
    """Append each sequence's accepted path to its ring of the last W positions.

    The ring [B, Hkv, W, D] holds position p in slot p % W.  Path row k (node accepted[b, k])
    is position win_pos[b] + k; rows are written in path order, so of a path longer than W
    only its last W rows remain.  Returns new arrays (k_win, v_win, win_pos)."""
    kw, vw = k_win.copy(), v_win.copy()
    pos = np.array(win_pos, dtype=np.int32, copy=True)
    B, Hkv, Wn, D = kw.shape
    for b in range(B):
        for k in range(int(accept_len[b])):
            node = int(accepted[b, k])
            slot = (int(win_pos[b]) + k) % Wn
            kw[b, :, slot, :] = k_tree[b, :, node, :]
            vw[b, :, slot, :] = v_tree[b, :, node, :]
        pos[b] = int(win_pos[b]) + int(accept_len[b])
    return kw, vw, pos
