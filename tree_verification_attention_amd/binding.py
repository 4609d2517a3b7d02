"""ctypes binding of libhta.so (the C ABI in include/hta.h).

Argument marshalling only: every step of the verification attention runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory (tensors, the workspace) and the
stream.  If the shared library has not been built, loading raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhta.so")

HTA_BF16, HTA_F32 = 0, 1

STATUS_NAMES = {
    0: "HTA_OK",
    1: "HTA_ERR_NULL",
    2: "HTA_ERR_SHAPE",
    3: "HTA_ERR_DTYPE",
    4: "HTA_ERR_ALIGN",
    5: "HTA_ERR_WORKSPACE",
    6: "HTA_ERR_TREE",
    7: "HTA_ERR_PREFIX_LEN",
    8: "HTA_ERR_HIP",
    9: "HTA_ERR_CACHE_FULL",
    10: "HTA_ERR_NONFINITE",
    11: "HTA_ERR_SCRATCH",
}
EXPORTED = (
    "hta_plan",
    "hta_workspace_size",
    "hta_verify",
    "hta_verify_noalloc",
    "hta_ancestor_masks",
    "hta_prefix_partials",
    "hta_tree_partials",
    "hta_merge",
    "hta_get_device_status",
    "hta_chunk_mass",
    "hta_cross_attention",
    "hta_window_commit",
    "hta_dense_mask_bytes",
    "hta_dense_mask",
    "hta_verify_dense",
    "hta_rope_tree",
    "hta_accept_workspace_size",
    "hta_accept_commit",
    "hta_status_str",
    "hta_version",
    "hta_mfma_peak_probe",
)


class HtaError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        name = status_str(code) if _lib is not None else STATUS_NAMES.get(code, str(code))
        super().__init__(f"{what}: {name}" if what else name)


class hta_desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tree_size", ctypes.c_int32),
        ("max_prefix_len", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("chunk", ctypes.c_int32),
    ]


class hta_plan_info(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("rows_padded", ctypes.c_int32),
        ("status_offset", ctypes.c_size_t),
        ("masks_offset", ctypes.c_size_t),
        ("lse_part_offset", ctypes.c_size_t),
        ("o_part_offset", ctypes.c_size_t),
        ("o_scale_offset", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libhta.so (raises if it is missing: the HIP path is the only path).  The path is
    the in-tree build unless HTA_LIBRARY names another build of the same sources."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("HTA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m tree_verification_attention_amd.build`"
        )
    L = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    D = ctypes.POINTER(hta_desc)
    L.hta_plan.argtypes = [D, ctypes.POINTER(hta_plan_info)]
    L.hta_workspace_size.argtypes = [D]
    L.hta_workspace_size.restype = S
    L.hta_verify.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
    L.hta_verify_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
    L.hta_ancestor_masks.argtypes = [D, P, P, P, S, P]
    L.hta_prefix_partials.argtypes = [D, P, P, P, P, P, S, P]
    L.hta_tree_partials.argtypes = [D, P, P, P, P, P, P, S, P]
    L.hta_merge.argtypes = [D, P, I, P, P, P, S, P]
    L.hta_get_device_status.argtypes = [D, P, P, ctypes.POINTER(ctypes.c_int32)]
    L.hta_rope_tree.argtypes = [D, ctypes.c_double, I, P, P, P, P, P, P, S, P]
    L.hta_chunk_mass.argtypes = [D, P, P, P, P, P, S, P]
    L.hta_cross_attention.argtypes = [D, P, P, P, P, P, P, P, S, P]
    L.hta_window_commit.argtypes = [D, I, P, P, P, P, P, P, P, P, S, P]
    L.hta_dense_mask_bytes.argtypes = [D]
    L.hta_dense_mask_bytes.restype = S
    L.hta_dense_mask.argtypes = [D, P, P, P, P, S, P]
    L.hta_verify_dense.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    L.hta_accept_workspace_size.argtypes = [D, I]
    L.hta_accept_workspace_size.restype = S
    L.hta_accept_commit.argtypes = [D, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    L.hta_status_str.argtypes = [ctypes.c_int]
    L.hta_status_str.restype = ctypes.c_char_p
    L.hta_version.argtypes = []
    L.hta_mfma_peak_probe.argtypes = [I, I, P, P, ctypes.POINTER(ctypes.c_double)]
    for f in (L.hta_plan, L.hta_verify, L.hta_verify_noalloc, L.hta_ancestor_masks, L.hta_prefix_partials,
              L.hta_tree_partials, L.hta_merge, L.hta_get_device_status, L.hta_version,
              L.hta_rope_tree, L.hta_accept_commit, L.hta_chunk_mass, L.hta_dense_mask,
              L.hta_verify_dense, L.hta_cross_attention, L.hta_window_commit,
              L.hta_mfma_peak_probe):
        f.restype = ctypes.c_int
    _lib = L
    return L


def status_str(code: int) -> str:
    return load().hta_status_str(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise HtaError(code, what)


def _enqueue(fn, args, keep, what: str):
    """A callable that enqueues fn(*args) again on every call (arguments checked and marshalled
    once by the caller); keep holds the buffers alive as long as the callable."""
    def call() -> None:
        code = fn(*args)
        if code != 0:
            raise HtaError(code, what)
    call.keep = keep
    return call


def make_desc(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, tree_size: int,
              max_prefix_len: int, in_dtype: int = HTA_BF16, scale: float = 0.0,
              chunk: int = 0) -> hta_desc:
    return hta_desc(batch, num_q_heads, num_kv_heads, head_dim, tree_size, max_prefix_len,
                    in_dtype, float(scale), chunk)


def plan(desc: hta_desc) -> hta_plan_info:
    info = hta_plan_info()
    _check(load().hta_plan(ctypes.byref(desc), ctypes.byref(info)), "hta_plan")
    return info


def workspace_size(desc: hta_desc) -> int:
    return int(load().hta_workspace_size(ctypes.byref(desc)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _used_on(stream, *tensors) -> None:
    """Tensors a wrapper allocated (on the current stream) and handed to work on another torch
    stream: recorded on that stream, so the caching allocator does not reuse their memory
    before the work there has finished.  (With a raw stream handle the caller passes its own
    workspace and keeps the outputs alive until that stream has finished.)"""
    if isinstance(stream, torch.cuda.Stream) and stream != torch.cuda.current_stream(stream.device):
        for t in tensors:
            t.record_stream(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HTA_BF16
    if t.dtype == torch.float32:
        return HTA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def desc_for(q: torch.Tensor, k_prefix: torch.Tensor, scale: Optional[float] = None,
             chunk: int = 0) -> hta_desc:
    B, T, Hq, D = q.shape
    Hkv, Lmax = k_prefix.shape[1], k_prefix.shape[2]
    return make_desc(B, Hq, Hkv, D, T, Lmax, _dtype_code(q), 0.0 if scale is None else scale,
                     chunk)


def new_workspace(desc: hta_desc, device) -> torch.Tensor:
    n = workspace_size(desc)
    if n == 0:
        _check(2, "hta_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _contig(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


_I32 = (torch.int32,)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def _in_dtype(desc: hta_desc):
    return (torch.bfloat16,) if desc.in_dtype == HTA_BF16 else (torch.float32,)


def _validate(specs, workspace: Optional[torch.Tensor] = None, ws_bytes: int = 0) -> None:
    """Check every tensor a wrapper hands to the C ABI before the call: its dtype, shape and
    contiguity against the descriptor (specs: (name, tensor, shape, dtypes), shape None = any),
    then that all of them and the workspace (a 1-D uint8 buffer of at least ws_bytes) live on
    one GPU.  The C ABI sees only pointers, so a mismatch here would otherwise be misread or
    read out of bounds on the device."""
    named = [x for x in specs if x[1] is not None]
    if workspace is not None:
        named.append(("workspace", workspace, None, _U8))
    for name, t, shape, dtypes in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype not in dtypes:
            want = " or ".join(str(d) for d in dtypes)
            raise TypeError(f"{name} has dtype {t.dtype}, expected {want}")
        if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if workspace is not None:
        if workspace.dim() != 1 or workspace.numel() < ws_bytes:
            raise ValueError(f"workspace must be a 1-D uint8 buffer of at least {ws_bytes} bytes,"
                             f" got shape {tuple(workspace.shape)}")
    dev = named[0][1].device
    for name, t, _, _ in named:
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}: every tensor must be on a GPU")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, {named[0][0]} on {dev}")


def _dims(desc: hta_desc):
    return (desc.batch, desc.tree_size, desc.num_q_heads, desc.num_kv_heads, desc.head_dim,
            desc.max_prefix_len)


# ----------------------------------------------------------------------------- entry points


def hta_verify(desc, q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, out, lse,
               workspace, stream=None) -> None:
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_prefix", k_prefix, (B, Hkv, L, D), X),
               ("v_prefix", v_prefix, (B, Hkv, L, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("v_tree", v_tree, (B, Hkv, T, D), X), ("parent_idx", parent_idx, (B, T), _I32),
               ("prefix_len", prefix_len, (B,), _I32), ("out", out, (B, T, Hq, D), _F32),
               ("lse", lse, (B, Hq, T), _F32)], workspace, workspace_size(desc))
    _check(load().hta_verify(ctypes.byref(desc), _ptr(q), _ptr(k_prefix), _ptr(v_prefix),
                             _ptr(k_tree), _ptr(v_tree), _ptr(parent_idx), _ptr(prefix_len),
                             _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                             _stream(stream)), "hta_verify")


def hta_verify_noalloc(desc, q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len,
                       out, lse, status=None, stream=None) -> None:
    """hta_verify on the library's static scratch: no workspace, nothing allocated.  status
    (int32 [B] on the device, optional) receives the per-sequence device flags."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_prefix", k_prefix, (B, Hkv, L, D), X),
               ("v_prefix", v_prefix, (B, Hkv, L, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("v_tree", v_tree, (B, Hkv, T, D), X), ("parent_idx", parent_idx, (B, T), _I32),
               ("prefix_len", prefix_len, (B,), _I32), ("out", out, (B, T, Hq, D), _F32),
               ("lse", lse, (B, Hq, T), _F32), ("status", status, (B,), _I32)])
    _check(load().hta_verify_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_prefix),
                                     _ptr(v_prefix), _ptr(k_tree), _ptr(v_tree),
                                     _ptr(parent_idx), _ptr(prefix_len), _ptr(out), _ptr(lse),
                                     _ptr(status), _stream(stream)), "hta_verify_noalloc")


def prepare_verify(desc, q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, out,
                   lse, workspace, stream=None):
    """hta_verify with its arguments checked and marshalled once: returns a callable that
    enqueues the same call again (for loops that repeat one step on fixed buffers, where the
    per-call checks would cost more host time than the GPU spends on the step)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_prefix", k_prefix, (B, Hkv, L, D), X),
               ("v_prefix", v_prefix, (B, Hkv, L, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("v_tree", v_tree, (B, Hkv, T, D), X), ("parent_idx", parent_idx, (B, T), _I32),
               ("prefix_len", prefix_len, (B,), _I32), ("out", out, (B, T, Hq, D), _F32),
               ("lse", lse, (B, Hq, T), _F32)], workspace, workspace_size(desc))
    fn = load().hta_verify
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_prefix), _ptr(v_prefix), _ptr(k_tree),
            _ptr(v_tree), _ptr(parent_idx), _ptr(prefix_len), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(stream))
    keep = (desc, q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, out, lse,
            workspace)

    def call() -> None:
        code = fn(*args)
        if code != 0:
            raise HtaError(code, "hta_verify")
    call.keep = keep  # the buffers stay alive as long as the call
    return call


def prepare_prefix_partials(desc, q, k_prefix, v_prefix, prefix_len, workspace, stream=None):
    """hta_prefix_partials checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_prefix", k_prefix, (B, Hkv, L, D), X),
               ("v_prefix", v_prefix, (B, Hkv, L, D), X), ("prefix_len", prefix_len, (B,), _I32)],
              workspace, workspace_size(desc))
    fn = load().hta_prefix_partials
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_prefix), _ptr(v_prefix), _ptr(prefix_len),
            _ptr(workspace), workspace.numel(), _stream(stream))
    keep = (desc, q, k_prefix, v_prefix, prefix_len, workspace)

    def call() -> None:
        code = fn(*args)
        if code != 0:
            raise HtaError(code, "hta_prefix_partials")
    call.keep = keep
    return call


def hta_ancestor_masks(desc, parent_idx, masks, workspace, stream=None) -> None:
    B, T = desc.batch, desc.tree_size
    _validate([("parent_idx", parent_idx, (B, T), _I32),
               ("masks", masks, (B, T, (T + 63) // 64), (torch.int64,))],
              workspace, workspace_size(desc))
    _check(load().hta_ancestor_masks(ctypes.byref(desc), _ptr(parent_idx), _ptr(masks),
                                     _ptr(workspace), workspace.numel(), _stream(stream)),
           "hta_ancestor_masks")


def hta_prefix_partials(desc, q, k_prefix, v_prefix, prefix_len, workspace, stream=None) -> None:
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_prefix", k_prefix, (B, Hkv, L, D), X),
               ("v_prefix", v_prefix, (B, Hkv, L, D), X), ("prefix_len", prefix_len, (B,), _I32)],
              workspace, workspace_size(desc))
    _check(load().hta_prefix_partials(ctypes.byref(desc), _ptr(q), _ptr(k_prefix),
                                      _ptr(v_prefix), _ptr(prefix_len), _ptr(workspace),
                                      workspace.numel(), _stream(stream)),
           "hta_prefix_partials")


def prepare_tree_partials(desc, q, k_tree, v_tree, parent_idx, prefix_len, workspace,
                          stream=None):
    """hta_tree_partials checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("v_tree", v_tree, (B, Hkv, T, D), X), ("parent_idx", parent_idx, (B, T), _I32),
               ("prefix_len", prefix_len, (B,), _I32)], workspace, workspace_size(desc))
    fn = load().hta_tree_partials
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(parent_idx),
            _ptr(prefix_len), _ptr(workspace), workspace.numel(), _stream(stream))
    keep = (desc, q, k_tree, v_tree, parent_idx, prefix_len, workspace)

    def call() -> None:
        code = fn(*args)
        if code != 0:
            raise HtaError(code, "hta_tree_partials")
    call.keep = keep
    return call


def prepare_merge(desc, prefix_len, include_tree: bool, out, lse, workspace, stream=None):
    """hta_merge checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    _validate([("prefix_len", prefix_len, (B,), _I32), ("out", out, (B, T, Hq, D), _F32),
               ("lse", lse, (B, Hq, T), _F32)], workspace, workspace_size(desc))
    fn = load().hta_merge
    args = (ctypes.byref(desc), _ptr(prefix_len), 1 if include_tree else 0, _ptr(out),
            _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
    keep = (desc, prefix_len, out, lse, workspace)

    def call() -> None:
        code = fn(*args)
        if code != 0:
            raise HtaError(code, "hta_merge")
    call.keep = keep
    return call


def hta_tree_partials(desc, q, k_tree, v_tree, parent_idx, prefix_len, workspace,
                      stream=None) -> None:
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("v_tree", v_tree, (B, Hkv, T, D), X), ("parent_idx", parent_idx, (B, T), _I32),
               ("prefix_len", prefix_len, (B,), _I32)], workspace, workspace_size(desc))
    _check(load().hta_tree_partials(ctypes.byref(desc), _ptr(q), _ptr(k_tree), _ptr(v_tree),
                                    _ptr(parent_idx), _ptr(prefix_len), _ptr(workspace),
                                    workspace.numel(), _stream(stream)), "hta_tree_partials")


def hta_merge(desc, prefix_len, include_tree: bool, out, lse, workspace, stream=None) -> None:
    B, T, Hq, Hkv, D, L = _dims(desc)
    _validate([("prefix_len", prefix_len, (B,), _I32), ("out", out, (B, T, Hq, D), _F32),
               ("lse", lse, (B, Hq, T), _F32)], workspace, workspace_size(desc))
    _check(load().hta_merge(ctypes.byref(desc), _ptr(prefix_len), 1 if include_tree else 0,
                            _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                            _stream(stream)), "hta_merge")


def hta_get_device_status(desc, workspace, stream=None) -> Tuple[int, int]:
    bad = ctypes.c_int32(-1)
    code = load().hta_get_device_status(ctypes.byref(desc), _ptr(workspace), _stream(stream),
                                        ctypes.byref(bad))
    return int(code), int(bad.value)


def prepare_chunk_mass(desc, prefix_len, lse, mass, chunk_scores, workspace, stream=None):
    """hta_chunk_mass checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    S1 = plan(desc).num_splits + 1
    _validate([("prefix_len", prefix_len, (B,), _I32), ("lse", lse, (B, Hq, T), _F32),
               ("mass", mass, (B, Hq, T, S1), _F32),
               ("chunk_scores", chunk_scores, (B, S1), _F32)], workspace, workspace_size(desc))
    args = (ctypes.byref(desc), _ptr(prefix_len), _ptr(lse), _ptr(mass), _ptr(chunk_scores),
            _ptr(workspace), workspace.numel(), _stream(stream))
    return _enqueue(load().hta_chunk_mass, args,
                    (desc, prefix_len, lse, mass, chunk_scores, workspace), "hta_chunk_mass")


def hta_chunk_mass(desc, prefix_len, lse, mass, chunk_scores, workspace, stream=None) -> None:
    prepare_chunk_mass(desc, prefix_len, lse, mass, chunk_scores, workspace, stream)()


def prepare_cross_attention(desc, q, k_cache, v_cache, cache_len, out, lse, workspace,
                            stream=None):
    """hta_cross_attention checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_cache", k_cache, (B, Hkv, L, D), X),
               ("v_cache", v_cache, (B, Hkv, L, D), X), ("cache_len", cache_len, (B,), _I32),
               ("out", out, (B, T, Hq, D), _F32), ("lse", lse, (B, Hq, T), _F32)],
              workspace, workspace_size(desc))
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
            _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
    return _enqueue(load().hta_cross_attention, args,
                    (desc, q, k_cache, v_cache, cache_len, out, lse, workspace),
                    "hta_cross_attention")


def hta_cross_attention(desc, q, k_cache, v_cache, cache_len, out, lse, workspace,
                        stream=None) -> None:
    prepare_cross_attention(desc, q, k_cache, v_cache, cache_len, out, lse, workspace, stream)()


def cross_attention(q, k_cache, v_cache, cache_len, *, scale=None, chunk: int = 0,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """The drafter's cross-attention into a target KV cache (no mask): (out, lse)."""
    desc = desc_for(q, k_cache, scale, chunk)
    B, Tq, Hq, D = q.shape
    out = torch.empty(B, Tq, Hq, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(desc, q.device)
    hta_cross_attention(desc, q, k_cache, v_cache, cache_len, out, lse, workspace, stream)
    _used_on(stream, out, lse, workspace)
    return out, lse


def hta_window_commit(desc, window: int, k_win, v_win, k_tree, v_tree, accepted, accept_len,
                      win_pos, workspace, stream=None) -> None:
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("k_win", k_win, (B, Hkv, window, D), X), ("v_win", v_win, (B, Hkv, window, D), X),
               ("k_tree", k_tree, (B, Hkv, T, D), X), ("v_tree", v_tree, (B, Hkv, T, D), X),
               ("accepted", accepted, (B, T), _I32), ("accept_len", accept_len, (B,), _I32),
               ("win_pos", win_pos, (B,), _I32)], workspace, 4 * B)
    _check(load().hta_window_commit(ctypes.byref(desc), int(window), _ptr(k_win), _ptr(v_win),
                                    _ptr(k_tree), _ptr(v_tree), _ptr(accepted),
                                    _ptr(accept_len), _ptr(win_pos), _ptr(workspace),
                                    workspace.numel(), _stream(stream)), "hta_window_commit")


def dense_mask_shape(desc: hta_desc) -> Tuple[int, int, int]:
    """(B, W, T_pad) of the word-major explicit mask (include/hta.h)."""
    B, T = desc.batch, desc.tree_size
    t_pad = T + (T & 1)
    n = int(load().hta_dense_mask_bytes(ctypes.byref(desc)))
    if n == 0:
        _check(2, "hta_dense_mask_bytes")
    return B, n // (8 * B * t_pad), t_pad


def hta_dense_mask(desc, parent_idx, prefix_len, mask, workspace, stream=None) -> None:
    B, T = desc.batch, desc.tree_size
    _validate([("parent_idx", parent_idx, (B, T), _I32), ("prefix_len", prefix_len, (B,), _I32),
               ("mask", mask, dense_mask_shape(desc), (torch.int64,))], workspace, 4 * B)
    _check(load().hta_dense_mask(ctypes.byref(desc), _ptr(parent_idx), _ptr(prefix_len),
                                 _ptr(mask), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "hta_dense_mask")


def hta_verify_dense(desc, q, k_prefix, v_prefix, k_tree, v_tree, mask, prefix_len, out, lse,
                     stream=None) -> None:
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_prefix", k_prefix, (B, Hkv, L, D), X),
               ("v_prefix", v_prefix, (B, Hkv, L, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("v_tree", v_tree, (B, Hkv, T, D), X),
               ("mask", mask, dense_mask_shape(desc), (torch.int64,)),
               ("prefix_len", prefix_len, (B,), _I32), ("out", out, (B, T, Hq, D), _F32),
               ("lse", lse, (B, Hq, T), _F32)])
    _check(load().hta_verify_dense(ctypes.byref(desc), _ptr(q), _ptr(k_prefix), _ptr(v_prefix),
                                   _ptr(k_tree), _ptr(v_tree), _ptr(mask), _ptr(prefix_len),
                                   _ptr(out), _ptr(lse), _stream(stream)), "hta_verify_dense")


def verify_dense(q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, *, scale=None,
                 mask: Optional[torch.Tensor] = None, stream=None):
    """The single-pass masked baseline: builds the explicit mask (unless one is given) and
    runs one masked attention pass over all L + T keys.  Returns (out, lse, mask)."""
    desc = desc_for(q, k_prefix, scale)
    B, T, Hq, D = q.shape
    if mask is None:
        mask = torch.empty(*dense_mask_shape(desc), dtype=torch.int64, device=q.device)
        ws = torch.empty(256 * ((4 * B + 255) // 256), dtype=torch.uint8, device=q.device)
        hta_dense_mask(desc, parent_idx, prefix_len, mask, ws, stream)
        _used_on(stream, mask, ws)
    out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    hta_verify_dense(desc, q, k_prefix, v_prefix, k_tree, v_tree, mask, prefix_len, out, lse,
                     stream)
    _used_on(stream, out, lse)
    return out, lse, mask


def chunk_mass(desc, prefix_len, lse, workspace, stream=None):
    """Each chunk's share of every query row's attention after hta_verify on this workspace:
    (mass float [B, Hq, T, S+1], chunk_scores float [B, S+1]); column S is the tree."""
    p = plan(desc)
    B, Hq, T = desc.batch, desc.num_q_heads, desc.tree_size
    mass = torch.empty(B, Hq, T, p.num_splits + 1, dtype=torch.float32, device=lse.device)
    scores = torch.empty(B, p.num_splits + 1, dtype=torch.float32, device=lse.device)
    hta_chunk_mass(desc, prefix_len, lse, mass, scores, workspace, stream)
    _used_on(stream, mass, scores)
    return mass, scores


def prepare_rope_tree(desc, rope_theta: float, interleaved: bool, q, k_tree, parent_idx,
                      prefix_len, positions, workspace, stream=None):
    """hta_rope_tree checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    _validate([("q", q, (B, T, Hq, D), X), ("k_tree", k_tree, (B, Hkv, T, D), X),
               ("parent_idx", parent_idx, (B, T), _I32), ("prefix_len", prefix_len, (B,), _I32),
               ("positions", positions, (B, T), _I32)], workspace, 4 * B)
    args = (ctypes.byref(desc), float(rope_theta), 1 if interleaved else 0, _ptr(q),
            _ptr(k_tree), _ptr(parent_idx), _ptr(prefix_len), _ptr(positions), _ptr(workspace),
            workspace.numel(), _stream(stream))
    return _enqueue(load().hta_rope_tree, args,
                    (desc, q, k_tree, parent_idx, prefix_len, positions, workspace),
                    "hta_rope_tree")


def hta_rope_tree(desc, rope_theta: float, interleaved: bool, q, k_tree, parent_idx, prefix_len,
                  positions, workspace, stream=None) -> None:
    prepare_rope_tree(desc, rope_theta, interleaved, q, k_tree, parent_idx, prefix_len,
                      positions, workspace, stream)()


def accept_workspace_size(desc: hta_desc, vocab: int) -> int:
    return int(load().hta_accept_workspace_size(ctypes.byref(desc), int(vocab)))


def prepare_accept_commit(desc, logits, tokens, root_token, parent_idx, prefix_len, k_prefix,
                          v_prefix, k_tree, v_tree, target_next, accept_len, accepted,
                          bonus_token, workspace, stream=None):
    """hta_accept_commit checked and marshalled once (see prepare_verify)."""
    B, T, Hq, Hkv, D, L = _dims(desc)
    X = _in_dtype(desc)
    vocab = logits.shape[-1] if isinstance(logits, torch.Tensor) and logits.dim() == 3 else 0
    _validate([("logits", logits, (B, T, vocab), (torch.bfloat16, torch.float32)),
               ("tokens", tokens, (B, T), _I32), ("root_token", root_token, (B,), _I32),
               ("parent_idx", parent_idx, (B, T), _I32), ("prefix_len", prefix_len, (B,), _I32),
               ("k_prefix", k_prefix, (B, Hkv, L, D), X), ("v_prefix", v_prefix, (B, Hkv, L, D), X),
               ("k_tree", k_tree, (B, Hkv, T, D), X), ("v_tree", v_tree, (B, Hkv, T, D), X),
               ("target_next", target_next, (B, T), _I32), ("accept_len", accept_len, (B,), _I32),
               ("accepted", accepted, (B, T), _I32), ("bonus_token", bonus_token, (B,), _I32)],
              workspace, accept_workspace_size(desc, max(vocab, 1)))
    args = (ctypes.byref(desc), int(vocab), _dtype_code(logits), _ptr(logits), _ptr(tokens),
            _ptr(root_token), _ptr(parent_idx), _ptr(prefix_len), _ptr(k_prefix),
            _ptr(v_prefix), _ptr(k_tree), _ptr(v_tree), _ptr(target_next), _ptr(accept_len),
            _ptr(accepted), _ptr(bonus_token), _ptr(workspace), workspace.numel(),
            _stream(stream))
    keep = (desc, logits, tokens, root_token, parent_idx, prefix_len, k_prefix, v_prefix,
            k_tree, v_tree, target_next, accept_len, accepted, bonus_token, workspace)
    return _enqueue(load().hta_accept_commit, args, keep, "hta_accept_commit")


def hta_accept_commit(desc, logits, tokens, root_token, parent_idx, prefix_len, k_prefix,
                      v_prefix, k_tree, v_tree, target_next, accept_len, accepted, bonus_token,
                      workspace, stream=None) -> None:
    prepare_accept_commit(desc, logits, tokens, root_token, parent_idx, prefix_len, k_prefix,
                          v_prefix, k_tree, v_tree, target_next, accept_len, accepted,
                          bonus_token, workspace, stream)()


def prepare_mfma_peak_probe(blocks: int, iters: int, out: torch.Tensor, stream=None):
    """hta_mfma_peak_probe (a measurement helper, not part of the path) checked and marshalled
    once: returns (call, flops per launch); the preparation enqueues one launch (a warm-up).
    out: float32 on the GPU, blocks * 512 elements."""
    _validate([("out", out, (int(blocks) * 512,), _F32)])
    flops = ctypes.c_double(0.0)
    fn = load().hta_mfma_peak_probe
    args = (int(blocks), int(iters), _ptr(out), _stream(stream), ctypes.byref(flops))
    call = _enqueue(fn, args, (out, flops), "hta_mfma_peak_probe")
    call()
    return call, float(flops.value)


# ----------------------------------------------------------------------------- convenience


def verify(q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, *, scale=None,
           chunk: int = 0, workspace: Optional[torch.Tensor] = None, stream=None
           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Tree verification attention on device tensors: returns (out fp32 [B,T,Hq,D],
    lse fp32 [B,Hq,T]).  A workspace is allocated through torch if none is given."""
    desc = desc_for(q, k_prefix, scale, chunk)
    B, T, Hq, D = q.shape
    out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(desc, q.device)
    hta_verify(desc, q, k_prefix, v_prefix, k_tree, v_tree, parent_idx, prefix_len, out, lse,
               workspace, stream)
    _used_on(stream, out, lse, workspace)
    return out, lse


def ancestor_masks(parent_idx: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Packed ancestor-or-self masks uint64 [B, T, ceil(T/64)] (as int64 storage)."""
    B, T = parent_idx.shape
    desc = make_desc(B, 1, 1, 64, T, 0)
    W = (T + 63) // 64
    masks = torch.empty(B, T, W, dtype=torch.int64, device=parent_idx.device)
    if workspace is None:
        workspace = new_workspace(desc, parent_idx.device)
    hta_ancestor_masks(desc, parent_idx, masks, workspace, stream)
    _used_on(stream, masks, workspace)
    return masks


def rope_tree(q, k_tree, parent_idx, prefix_len, rope_theta: float, *, interleaved: bool = False,
              max_prefix_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Rotate q [B,T,Hq,D] and k_tree [B,Hkv,T,D] in place at positions prefix_len + depth;
    returns the positions int32 [B, T].  max_prefix_len bounds the valid prefix_len values
    (default: no bound below 2^31 - 1 - T)."""
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[1]
    Lmax = (2 ** 31 - 1 - T) if max_prefix_len is None else int(max_prefix_len)
    desc = make_desc(B, Hq, Hkv, D, T, 0, _dtype_code(q))
    desc.max_prefix_len = Lmax
    positions = torch.empty(B, T, dtype=torch.int32, device=q.device)
    if workspace is None:
        ws_desc = make_desc(B, Hq, Hkv, D, T, 0, _dtype_code(q))
        workspace = new_workspace(ws_desc, q.device)
    hta_rope_tree(desc, rope_theta, interleaved, q, k_tree, parent_idx, prefix_len, positions,
                  workspace, stream)
    _used_on(stream, positions, workspace)
    return positions


def accept_commit(logits, tokens, root_token, parent_idx, prefix_len, k_prefix, v_prefix,
                  k_tree, v_tree, *, workspace: Optional[torch.Tensor] = None, stream=None):
    """Greedy acceptance along the draft trees and KV commit of the accepted paths (in place
    on k_prefix, v_prefix, prefix_len).  Returns (target_next [B,T], accept_len [B],
    accepted [B,T], bonus_token [B]), int32."""
    B, Hkv, Lmax, D = k_prefix.shape
    T = tokens.shape[1]
    desc = make_desc(B, Hkv, Hkv, D, T, Lmax, _dtype_code(k_prefix))
    dev = logits.device
    target_next = torch.empty(B, T, dtype=torch.int32, device=dev)
    accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    accepted = torch.empty(B, T, dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    if workspace is None:
        n = accept_workspace_size(desc, logits.shape[-1])
        if n == 0:
            _check(2, "hta_accept_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    hta_accept_commit(desc, logits, tokens, root_token, parent_idx, prefix_len, k_prefix,
                      v_prefix, k_tree, v_tree, target_next, accept_len, accepted, bonus,
                      workspace, stream)
    _used_on(stream, target_next, accept_len, accepted, bonus, workspace)
    return target_next, accept_len, accepted, bonus


def partial_views(desc: hta_desc, workspace: torch.Tensor):
    """(lse_part [B,Hkv,S+1,R_pad] view, o_part [B,Hkv,S+1,R_pad,D] decoded fp32 copy) of a
    workspace.  o_part rows are stored as int16 values with one fp32 factor per row
    (include/hta.h); this decodes them with torch ops on the workspace's device (inspection
    and tests only)."""
    p = plan(desc)
    B, Hkv, D = desc.batch, desc.num_kv_heads, desc.head_dim
    S1, Rp = p.num_splits + 1, p.rows_padded
    n = B * Hkv * S1 * Rp
    lse = workspace[p.lse_part_offset:p.lse_part_offset + 4 * n].view(torch.float32)
    scale = workspace[p.o_scale_offset:p.o_scale_offset + 4 * n].view(torch.float32)
    q = workspace[p.o_part_offset:p.o_part_offset + 2 * n * D].view(torch.int16)
    o = q.view(n, D).to(torch.float32) * scale.view(n, 1)
    return lse.view(B, Hkv, S1, Rp), o.reshape(B, Hkv, S1, Rp, D)
