"""Host-side contract of libhta.so (no GPU needed).

The library must load on a machine without a GPU, export every entry point that
include/hta.h declares, and reject bad arguments on the host, before any HIP call, with
the documented status codes.  Pointers below are fake non-null addresses: every case here
fails validation, so nothing is ever dereferenced or launched.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

import pytest

import tree_verification_attention_amd as hta
from tree_verification_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hta.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(hta_[a-z_]+)\s*\(", text,
                                 re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = hta.load()
    names = declared_functions()
    assert "hta_verify" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/hta.h but not exported"
    assert set(names) == set(B.EXPORTED)


def test_status_strings_cover_every_code():
    for code, name in B.STATUS_NAMES.items():
        assert hta.status_str(code).startswith(name)
    assert hta.status_str(99) == "HTA_ERR_UNKNOWN"


def _desc(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, tree_size=68,
                max_prefix_len=32768)
    base.update(kw)
    return B.make_desc(**base)


def _plan_code(d):
    info = B.hta_plan_info()
    return hta.load().hta_plan(ctypes.byref(d), ctypes.byref(info))


def test_plan_llama_shape():
    p = hta.plan(_desc())
    assert p.rows == 272 and p.rows_padded == 272
    assert p.num_splits * p.chunk >= 32768 and p.chunk % 64 == 0
    assert p.workspace_bytes == hta.workspace_size(_desc())
    # partial buffers hold (splits + 1) slots: the last one is the tree partial
    n = 8 * (p.num_splits + 1) * 272
    assert p.o_scale_offset >= p.lse_part_offset + 4 * n
    assert p.o_part_offset >= p.o_scale_offset + 4 * n
    # o_part rows: 128 int16 values each
    assert p.workspace_bytes >= p.o_part_offset + 2 * n * 128


def test_partial_views_decode_the_documented_encoding():
    """The o_part rows and their factors written out from their description in include/hta.h
    (an encoder of its own) and read back through partial_views, on the CPU."""
    d = _desc(batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64, tree_size=3,
              max_prefix_len=256)
    p = hta.plan(d)
    n = 1 * 4 * (p.num_splits + 1) * p.rows_padded
    rng = np.random.default_rng(5)
    vals = (rng.standard_normal((n, 64)) * np.exp2(rng.integers(-20, 20, (n, 1)))).astype(np.float32)
    vals[1] = 0.0                                       # an all-zero row: factor 0
    vals[2] = np.linspace(-1.0, 1.0, 64, dtype=np.float32)
    vals[2, :3] = [-3.0, 1.5, 0.75]                     # -3 is the largest magnitude
    m = np.max(np.abs(vals), axis=1)
    scale = (m / np.float32(32767)).astype(np.float32)
    enc = np.where(m > 0, np.float32(32767) / np.where(m > 0, m, 1), 0).astype(np.float32)
    q = np.rint(vals * enc[:, None]).astype(np.int16)   # nearest, ties to even
    assert q[2, 0] == -32767 and np.abs(q).max() == 32767
    ws = torch.zeros(p.workspace_bytes, dtype=torch.uint8)
    ws[p.o_scale_offset:p.o_scale_offset + 4 * n] = torch.from_numpy(scale.view(np.uint8))
    ws[p.o_part_offset:p.o_part_offset + 2 * n * 64] = torch.from_numpy(
        q.reshape(-1).view(np.uint8))
    _, o = hta.partial_views(d, ws)
    got = o.reshape(n, 64).numpy()
    assert np.array_equal(got, q.astype(np.float32) * scale[:, None])
    assert not got[1].any()
    # the documented bound: 2^-16 of the row's largest magnitude, plus fp32 rounding (of the
    # factors and of the products: a few 2^-24 of the magnitude, i.e. under 1% of the bound)
    err = np.abs(got.astype(np.float64) - vals) / np.maximum(m, 1e-30)[:, None]
    assert err.max() <= 2.0 ** -16 * 1.01


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), SHAPE),
    (dict(head_dim=256), SHAPE),
    (dict(num_q_heads=30), SHAPE),          # not a multiple of num_kv_heads
    (dict(num_q_heads=8 * 17), SHAPE),      # group of 17 > 16
    (dict(tree_size=0), SHAPE),
    (dict(tree_size=257), SHAPE),
    (dict(batch=0), SHAPE),
    (dict(max_prefix_len=-1), SHAPE),
    (dict(chunk=100), SHAPE),               # not a multiple of 64
    (dict(scale=-1.0), SHAPE),
    (dict(scale=float("nan")), SHAPE),
    (dict(batch=65536), SHAPE),                                  # a grid dimension
    (dict(batch=40000, tree_size=256, num_q_heads=256, num_kv_heads=16), SHAPE),  # 2^31 rows
    (dict(num_q_heads=16 * 65536, num_kv_heads=65536), SHAPE),   # KV heads x row blocks
    (dict(in_dtype=2), DTYPE),
    (dict(in_dtype=7), DTYPE),
])
def test_bad_descriptors_are_rejected(kw, code):
    d = _desc(**kw)
    assert _plan_code(d) == code
    assert hta.workspace_size(d) == 0


def test_launch_limits_admit_their_edges():
    # the largest batch, and a row count just under the merge's 32-bit limit
    assert _plan_code(_desc(batch=65535, tree_size=1, num_q_heads=1, num_kv_heads=1)) == 0
    assert _plan_code(_desc(batch=32767, tree_size=256, num_q_heads=256, num_kv_heads=16)) == 0


def test_fp32_inputs_plan_like_bf16():
    # fp32 inputs take their own kernels but the same plan, workspace and partial layout
    a, b = hta.plan(_desc()), hta.plan(_desc(in_dtype=1))
    for f in ("chunk", "num_splits", "rows", "rows_padded", "workspace_bytes"):
        assert getattr(a, f) == getattr(b, f)


def test_null_descriptor():
    L = hta.load()
    info = B.hta_plan_info()
    assert L.hta_plan(None, ctypes.byref(info)) == NULL
    assert L.hta_workspace_size(None) == 0


FAKE = 0x10000  # 64 KiB-aligned fake device address; never dereferenced


def _verify_code(d, ptrs=None, ws=FAKE, ws_bytes=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    if ws_bytes is None:
        ws_bytes = max(hta.workspace_size(d), 1)
    return hta.load().hta_verify(ctypes.byref(d), *p, ws, ws_bytes, None)


@pytest.mark.parametrize("i", range(9))
def test_verify_rejects_each_null_pointer(i):
    p = [FAKE] * 9
    p[i] = None
    assert _verify_code(_desc(), p) == NULL


@pytest.mark.parametrize("i", range(9))
def test_verify_rejects_each_misaligned_pointer(i):
    p = [FAKE] * 9
    p[i] = FAKE + 8
    assert _verify_code(_desc(), p) == ALIGN


def test_verify_workspace_checks():
    d = _desc()
    n = hta.workspace_size(d)
    assert _verify_code(d, ws=None) == WORKSPACE
    assert _verify_code(d, ws_bytes=n - 1) == WORKSPACE
    assert _verify_code(d, ws=FAKE + 16) == ALIGN


def test_empty_cache_allows_null_prefix_pointers_in_validation():
    # with max_prefix_len = 0 the prefix pointers are never read; validation then only
    # fails on the workspace (the fake workspace size is too small on purpose)
    d = _desc(max_prefix_len=0)
    p = [FAKE] * 9
    p[1] = p[2] = None
    assert _verify_code(d, p, ws_bytes=1) == WORKSPACE


def test_other_entry_points_validate_before_launching():
    L = hta.load()
    d = _desc()
    n = hta.workspace_size(d)
    assert L.hta_prefix_partials(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, n, None) == NULL
    assert L.hta_prefix_partials(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, n - 1, None) == WORKSPACE
    assert L.hta_tree_partials(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, n, None) == NULL
    assert L.hta_merge(ctypes.byref(d), FAKE, 1, FAKE, FAKE + 4, FAKE, n, None) == ALIGN
    assert L.hta_ancestor_masks(ctypes.byref(d), FAKE, None, FAKE, n, None) == NULL
    bad = _desc(head_dim=80)
    assert L.hta_merge(ctypes.byref(bad), FAKE, 1, FAKE, FAKE, FAKE, n, None) == SHAPE
    assert L.hta_get_device_status(ctypes.byref(d), None, None, None) == WORKSPACE


def test_mfma_peak_probe_validates_before_launching():
    L = hta.load()
    f = ctypes.c_double(0.0)
    assert L.hta_mfma_peak_probe(256, 16, None, None, ctypes.byref(f)) == NULL
    assert L.hta_mfma_peak_probe(256, 16, 0x1000, None, None) == NULL
    for blocks, iters in ((0, 16), (1 << 21, 16), (256, 0), (256, 1 << 25)):
        assert L.hta_mfma_peak_probe(blocks, iters, 0x1000, None, ctypes.byref(f)) == SHAPE
    assert L.hta_mfma_peak_probe(256, 16, 0x1004, None, ctypes.byref(f)) == ALIGN


def test_version():
    assert hta.load().hta_version() >= 100


def test_rope_tree_validates_before_launching():
    L = hta.load()
    d = _desc()
    small = 256  # the status words of one sequence
    args = lambda **kw: [kw.get("theta", 500000.0), 0, kw.get("q", FAKE), kw.get("k", FAKE),  # noqa: E731
                         kw.get("par", FAKE), kw.get("pl", FAKE), kw.get("pos", None),
                         kw.get("ws", FAKE), kw.get("n", small), None]
    assert L.hta_rope_tree(ctypes.byref(d), *args(q=None)) == NULL
    assert L.hta_rope_tree(ctypes.byref(d), *args(k=FAKE + 2)) == ALIGN
    assert L.hta_rope_tree(ctypes.byref(d), *args(pos=FAKE + 4)) == ALIGN
    assert L.hta_rope_tree(ctypes.byref(d), *args(theta=0.0)) == SHAPE
    assert L.hta_rope_tree(ctypes.byref(d), *args(theta=float("inf"))) == SHAPE
    assert L.hta_rope_tree(ctypes.byref(d), *args(theta=float("nan"))) == SHAPE
    assert L.hta_rope_tree(ctypes.byref(d), *args(n=small - 1)) == WORKSPACE
    assert L.hta_rope_tree(ctypes.byref(d), *args(ws=FAKE + 16)) == ALIGN
    assert L.hta_rope_tree(ctypes.byref(_desc(head_dim=80)), *args()) == SHAPE


def test_accept_workspace_size():
    d = _desc()
    base = hta.workspace_size(d)
    # fp32 logits: 4096-element spans; Llama-3's 128256 -> 32 spans per row, 68 rows
    n = hta.accept_workspace_size(d, 128256)
    assert n >= base + 8 * 68 * 32 and n % 256 == 0
    assert hta.accept_workspace_size(d, 1) >= base + 8 * 68
    assert hta.accept_workspace_size(d, 0) == 0
    assert hta.accept_workspace_size(_desc(tree_size=0), 100) == 0


def test_accept_commit_validates_before_launching():
    L = hta.load()
    d = _desc()
    n = hta.accept_workspace_size(d, 128256)

    def code(vocab=128256, dtype=0, i=None, val=None, ws=FAKE, nbytes=n, desc=d):
        p = [FAKE] * 13
        if i is not None:
            p[i] = val
        return L.hta_accept_commit(ctypes.byref(desc), vocab, dtype, *p, ws, nbytes, None)

    for i in range(13):
        assert code(i=i, val=None) == NULL, i
    for i in range(1, 13):  # logits only need element alignment
        assert code(i=i, val=FAKE + 4) == ALIGN, i
    assert code(vocab=0) == SHAPE
    assert code(dtype=5) == DTYPE
    assert code(dtype=1, nbytes=n - 1) == WORKSPACE  # fp32 logits need the most spans
    assert code(ws=None) == WORKSPACE
    assert code(ws=FAKE + 64) == ALIGN
    assert code(desc=_desc(num_q_heads=30)) == SHAPE


def test_chunk_mass_validates_before_launching():
    L = hta.load()
    d = _desc()
    n = hta.workspace_size(d)
    call = lambda *p, nbytes=n, desc=d: L.hta_chunk_mass(ctypes.byref(desc), *p, nbytes, None)  # noqa: E731
    assert call(None, FAKE, FAKE, FAKE, FAKE) == NULL
    assert call(FAKE, None, FAKE, FAKE, FAKE) == NULL
    assert call(FAKE, FAKE, None, FAKE, FAKE) == NULL
    assert call(FAKE, FAKE, FAKE + 4, FAKE, FAKE) == ALIGN
    assert call(FAKE, FAKE, FAKE, FAKE + 4, FAKE) == ALIGN
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, nbytes=n - 1) == WORKSPACE
    assert call(FAKE, FAKE, FAKE, FAKE, None) == WORKSPACE
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, desc=_desc(head_dim=80)) == SHAPE


def test_dense_mask_bytes_and_validation():
    L = hta.load()
    d = _desc()  # Lmax 32768, T 68: 512 + 2 words per node, T_pad 68
    assert hta.load().hta_dense_mask_bytes(ctypes.byref(d)) == 8 * 1 * 514 * 68
    d7 = _desc(tree_size=7, max_prefix_len=100)  # 2 + 1 words, T_pad 8
    assert hta.load().hta_dense_mask_bytes(ctypes.byref(d7)) == 8 * 3 * 8
    assert hta.load().hta_dense_mask_bytes(ctypes.byref(_desc(head_dim=80))) == 0
    assert B.dense_mask_shape(d7) == (1, 3, 8)
    assert L.hta_dense_mask(ctypes.byref(d), None, FAKE, FAKE, FAKE, 256, None) == NULL
    assert L.hta_dense_mask(ctypes.byref(d), FAKE, FAKE, FAKE + 8, FAKE, 256, None) == ALIGN
    assert L.hta_dense_mask(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 255, None) == WORKSPACE
    p = [FAKE] * 9  # q, k/v_prefix, k/v_tree, mask, prefix_len, out, lse (never launched)
    for i in (0, 3, 4, 5, 6, 7, 8):
        q = list(p)
        q[i] = None
        assert L.hta_verify_dense(ctypes.byref(d), *q, None) == NULL, i
    q = list(p)
    q[5] = FAKE + 8
    assert L.hta_verify_dense(ctypes.byref(d), *q, None) == ALIGN
    assert L.hta_verify_dense(ctypes.byref(_desc(in_dtype=1)), *p, None) == DTYPE


# ----------------------------------------------------------------------------- binding checks


def _verify_tensors(B=2, T=5, Hq=8, Hkv=2, D=64, L=40, dtype=torch.bfloat16):
    """Correctly shaped CPU tensors for hta_verify (the binding checks them before any call)."""
    t = dict(q=torch.zeros(B, T, Hq, D, dtype=dtype),
             k_prefix=torch.zeros(B, Hkv, L, D, dtype=dtype),
             v_prefix=torch.zeros(B, Hkv, L, D, dtype=dtype),
             k_tree=torch.zeros(B, Hkv, T, D, dtype=dtype),
             v_tree=torch.zeros(B, Hkv, T, D, dtype=dtype),
             parent_idx=torch.full((B, T), -1, dtype=torch.int32),
             prefix_len=torch.full((B,), L, dtype=torch.int32),
             out=torch.zeros(B, T, Hq, D, dtype=torch.float32),
             lse=torch.zeros(B, Hq, T, dtype=torch.float32))
    desc = hta.make_desc(B, Hq, Hkv, D, T, L, 0 if dtype == torch.bfloat16 else 1)
    ws = torch.zeros(hta.workspace_size(desc), dtype=torch.uint8)
    return desc, t, ws


def _call_verify(desc, t, ws):
    hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                   t["parent_idx"], t["prefix_len"], t["out"], t["lse"], ws)


@pytest.mark.parametrize("name,bad,exc", [
    ("prefix_len", lambda t: t["prefix_len"].to(torch.int64), TypeError),
    ("parent_idx", lambda t: t["parent_idx"].to(torch.int64), TypeError),
    ("k_tree", lambda t: t["k_tree"].permute(0, 2, 1, 3).contiguous(), ValueError),
    ("v_prefix", lambda t: t["v_prefix"][:, :, :-1].contiguous(), ValueError),
    ("q", lambda t: t["q"].to(torch.float32), TypeError),
    ("out", lambda t: t["out"].to(torch.bfloat16), TypeError),
    ("lse", lambda t: t["lse"].transpose(1, 2), ValueError),
    ("v_tree", lambda t: t["v_tree"].transpose(2, 3), ValueError),
])
def test_binding_rejects_mismatched_tensors(name, bad, exc):
    """Every tensor the wrapper hands to the C ABI is checked against the descriptor first:
    a wrong dtype, layout, length or stride is an error, never a misread on the device."""
    desc, t, ws = _verify_tensors()
    t[name] = bad(t)
    with pytest.raises(exc, match=name):
        _call_verify(desc, t, ws)


def test_binding_rejects_small_workspace_and_host_tensors():
    desc, t, ws = _verify_tensors()
    with pytest.raises(ValueError, match="workspace"):
        _call_verify(desc, t, ws[:-1])
    with pytest.raises(TypeError, match="workspace"):
        _call_verify(desc, t, ws.to(torch.int32))
    # every shape and dtype right, but on the host: refused before the C call
    with pytest.raises(ValueError, match="GPU"):
        _call_verify(desc, t, ws)
    with pytest.raises(ValueError, match="GPU"):
        hta.prepare_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                           t["parent_idx"], t["prefix_len"], t["out"], t["lse"], ws)


def test_binding_checks_the_other_wrappers():
    desc, t, ws = _verify_tensors()
    with pytest.raises(TypeError, match="prefix_len"):
        hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"],
                                t["prefix_len"].to(torch.int64), ws)
    with pytest.raises(ValueError, match="k_tree"):
        hta.hta_tree_partials(desc, t["q"], t["k_tree"][:, :1].contiguous(), t["v_tree"],
                              t["parent_idx"], t["prefix_len"], ws)
    with pytest.raises(ValueError, match="out"):
        hta.hta_merge(desc, t["prefix_len"], True, t["out"][:1].contiguous(), t["lse"], ws)
    with pytest.raises(ValueError, match="out"):
        hta.prepare_merge(desc, t["prefix_len"], True, t["out"][:1].contiguous(), t["lse"], ws)
    with pytest.raises(TypeError, match="parent_idx"):
        hta.prepare_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"],
                                  t["parent_idx"].to(torch.int64), t["prefix_len"], ws)
    with pytest.raises(ValueError, match="k_cache"):
        hta.hta_cross_attention(desc, t["q"], t["k_prefix"][:, :, :3].contiguous(),
                                t["v_prefix"], t["prefix_len"], t["out"], t["lse"], ws)
    with pytest.raises(ValueError, match="GPU"):
        hta.hta_cross_attention(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"],
                                t["out"], t["lse"], ws)


def test_noalloc_refuses_plans_beyond_its_scratch():
    """The allocation-free entry point checks the plan against its static scratch first."""
    L = hta.load()
    big = _desc(batch=64, max_prefix_len=262144)
    assert hta.workspace_size(big) > (64 << 20)
    fake = [16 * (i + 1) for i in range(10)]
    code = L.hta_verify_noalloc(ctypes.byref(big), *fake, None, None)
    assert code == 11 and hta.status_str(code).startswith("HTA_ERR_SCRATCH")
    # a plan that fits gets as far as the pointer checks (nothing dereferenced or launched)
    small = _desc()
    assert hta.workspace_size(small) <= (64 << 20)
    assert L.hta_verify_noalloc(ctypes.byref(small), None, *fake[1:], None, None) == NULL
    assert L.hta_verify_noalloc(ctypes.byref(small), *fake[:9], 8, None, None) == ALIGN
