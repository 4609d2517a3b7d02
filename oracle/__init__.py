"""CPU oracle for tree verification attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The HIP library and its Python binding never do: the two sides
share nothing but the seeded input generators.

The arithmetic lives in ``hta_oracle.c`` (plain C, fp64, single-threaded; its header
states the definition and the passages it follows).  This module only builds it with gcc,
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
             _SRC, "-o", tmp, "-lm"]
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
    for f in (L.hta_oracle_rows, L.hta_oracle_verify, L.hta_oracle_masks,
              L.hta_oracle_check_tree, L.hta_oracle_masked_attention, L.hta_oracle_lse_merge):
        f.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
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
