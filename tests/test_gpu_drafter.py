"""GPU parity of the drafter's attention (libhta.so through the C ABI) against the oracle.

* hta_cross_attention: the drafter's queries over one layer of the target's KV cache, no
  mask -- the oracle's prefix-only attention (oracle.rows, part=PREFIX); bars out 2e-3,
  lse 1e-3; an empty cache gives out 0, lse -inf.
* windowed self-attention while drafting a tree = hta_verify with the window ring as the
  prefix: against the oracle's verification attention over the same last-W positions stored
  in chronological order (a different key order: the result must not depend on it).
* hta_window_commit: the ring after appending accepted paths, bit-exact against the oracle's
  ring append.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

from test_gpu_parity import LSE_TOL, OUT_TOL, _log, check_rows, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


CROSS = [
    # name, B, Hq, Hkv, Tq, Lmax, cache lengths
    ("llama_level16_32k", 1, 32, 8, 16, 32768, None),
    ("llama_level4_32k", 1, 32, 8, 4, 32768, None),
    ("llama_one_token_32k", 1, 32, 8, 1, 32768, None),
    ("qwq_level16_16k", 1, 40, 8, 16, 16384, None),
    ("vicuna_b8_level16", 8, 32, 32, 16, 16384, "ragged"),
]


@pytest.mark.parametrize("case", CROSS, ids=[c[0] for c in CROSS])
def test_cross_attention_matches_oracle(case):
    name, B, Hq, Hkv, Tq, Lmax, lens = case
    if lens == "ragged":
        lens = torch.randint(8192, Lmax + 1, (B,), generator=torch.Generator().manual_seed(3)).tolist()
        lens[1] = 0  # an empty cache
    w = W.make_workload(name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                        max_prefix_len=Lmax, parents=[W.chain_tree(Tq)] * B, prefix_len=lens,
                        peaky_frac=0.02, poison_padding=lens is not None, seed=100 + Tq)
    t = to_dev(w)
    out, lse = hta.cross_attention(t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"],
                                   scale=w.scale)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    check_rows(w, out, lse, n_rows=48, seed=1, part=oracle.PART_PREFIX)
    for b in range(B):
        if int(w.prefix_len[b]) == 0:
            assert (out[b] == 0).all() and np.isneginf(lse[b]).all()


@pytest.mark.parametrize("committed", [2000, 300, 512])
def test_window_self_attention_is_verification_over_the_ring(committed):
    """Drafter self-attention with a 512-position window while drafting a 4,16,16 tree."""
    W_ = 512
    B, Hq, Hkv, D = 2, 32, 8, 128
    gen = torch.Generator().manual_seed(110 + committed)
    par = [W.level_tree((4, 16, 16), gen) for _ in range(B)]
    T = len(par[0])
    hist_k = torch.randn(B, Hkv, committed, D, generator=gen).to(torch.bfloat16)
    hist_v = torch.randn(B, Hkv, committed, D, generator=gen).to(torch.bfloat16)
    q = torch.randn(B, T, Hq, D, generator=gen).to(torch.bfloat16)
    kt = torch.randn(B, Hkv, T, D, generator=gen).to(torch.bfloat16)
    vt = torch.randn(B, Hkv, T, D, generator=gen).to(torch.bfloat16)
    n = min(committed, W_)
    first = committed - n
    # the ring: position p in slot p % W (slots past n unused when fewer were committed)
    ring_k = torch.zeros(B, Hkv, W_, D, dtype=torch.bfloat16)
    ring_v = torch.zeros(B, Hkv, W_, D, dtype=torch.bfloat16)
    for p in range(first, committed):
        ring_k[:, :, p % W_] = hist_k[:, :, p]
        ring_v[:, :, p % W_] = hist_v[:, :, p]
    if committed < W_:
        ring_k[:, :, n:] = float("nan")  # never read: prefix_len = n
        ring_v[:, :, n:] = float("nan")
    plen = torch.full((B,), n, dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    out, lse = hta.verify(q.to(DEV), ring_k.to(DEV), ring_v.to(DEV), kt.to(DEV), vt.to(DEV),
                          torch.tensor(par, dtype=torch.int32, device=DEV), plen.to(DEV),
                          scale=scale)
    torch.cuda.synchronize()
    # the oracle over the same positions in chronological order
    arrs = {"q": _np(q), "k_prefix": _np(hist_k[:, :, first:].contiguous()),
            "v_prefix": _np(hist_v[:, :, first:].contiguous()), "k_tree": _np(kt),
            "v_tree": _np(vt), "parent_idx": np.array(par, dtype=np.int32),
            "prefix_len": plen.numpy()}
    ro, rl = oracle.verify(arrs, scale)
    eo = float(np.max(np.abs(out.cpu().double().numpy() - ro)))
    el = float(np.max(np.abs(lse.cpu().double().numpy() - rl)))
    _log(f"  window {W_}, committed {committed}: max|out|={eo:.3e} max|lse|={el:.3e}")
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_window_commit_matches_oracle():
    rng = np.random.default_rng(120)
    B, Hkv, D, T = 3, 8, 128, 68
    for W_ in (512, 5):
        kw = torch.from_numpy(rng.standard_normal((B, Hkv, W_, D)).astype(np.float32)).to(torch.bfloat16)
        vw = torch.from_numpy(rng.standard_normal((B, Hkv, W_, D)).astype(np.float32)).to(torch.bfloat16)
        kw_d, vw_d = kw.to(DEV), vw.to(DEV)
        pos = np.array([0, 510, 1023], dtype=np.int32)
        pos_d = torch.from_numpy(pos).to(DEV)
        desc = hta.make_desc(B, Hkv, Hkv, D, T, W_)
        ws = hta.new_workspace(desc, DEV)
        kw_ref, vw_ref = _np(kw), _np(vw)
        for step in range(4):
            kt = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
            vt = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
            n = rng.integers(0, 8, size=B).astype(np.int32)
            if step == 3:
                n[2] = 7  # longer than a 5-slot ring: only its last 5 rows stay
            acc = np.full((B, T), -1, dtype=np.int32)
            for b in range(B):
                acc[b, :n[b]] = rng.permutation(T)[:n[b]]
            hta.hta_window_commit(desc, W_, kw_d, vw_d, kt.to(DEV), vt.to(DEV),
                                  torch.from_numpy(acc).to(DEV), torch.from_numpy(n).to(DEV),
                                  pos_d, ws)
            kw_ref, vw_ref, pos = oracle.window_commit(kw_ref, vw_ref, _np(kt), _np(vt), acc, n,
                                                       pos)
        torch.cuda.synchronize()
        assert hta.hta_get_device_status(desc, ws)[0] == 0
        assert np.array_equal(pos_d.cpu().numpy(), pos)
        assert np.array_equal(_np(kw_d), kw_ref) and np.array_equal(_np(vw_d), vw_ref)
    # an accepted length beyond T is refused on the device, nothing written
    bad = torch.tensor([0, T + 1, 0], dtype=torch.int32, device=DEV)
    before = _np(kw_d).copy()
    hta.hta_window_commit(desc, W_, kw_d, vw_d, kt.to(DEV), vt.to(DEV),
                          torch.from_numpy(acc).to(DEV), bad, pos_d, ws)
    assert hta.hta_get_device_status(desc, ws) == (7, 1)
    assert np.array_equal(_np(kw_d)[1], before[1])
