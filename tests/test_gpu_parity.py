"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (bf16 inputs, fp32 accumulation): max |out - oracle| <= 2e-3, max |lse - oracle| <= 1e-3;
ancestor masks bit-exact.  Every input is seeded and synthetic (tree_verification_attention_amd
.workloads); the oracle sees exactly the same bits.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_amd as hta
from tree_verification_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3


def _log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w: W.Workload):
    d = "cuda"
    return dict(q=w.q.to(d), k_prefix=w.k_prefix.to(d), v_prefix=w.v_prefix.to(d),
                k_tree=w.k_tree.to(d), v_tree=w.v_tree.to(d), parent_idx=w.parent_idx.to(d),
                prefix_len=w.prefix_len.to(d))


def run_gpu(w: W.Workload, chunk: int = 0):
    t = to_dev(w)
    out, lse = hta.verify(t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                          t["parent_idx"], t["prefix_len"], scale=w.scale, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def sample_rows(w: W.Workload, n: int, seed: int = 0):
    B, T, Hq = w.batch, w.tree_size, w.num_q_heads
    total = B * T * Hq
    rng = np.random.default_rng(seed)
    if n >= total:
        ids = np.arange(total)
    else:
        ids = rng.choice(total, size=n, replace=False)
        # always include the first and last rows of every sequence (ragged edges)
        extra = [b * T * Hq for b in range(B)] + [(b + 1) * T * Hq - 1 for b in range(B)]
        ids = np.unique(np.concatenate([ids, extra]))
    b = ids // (T * Hq)
    i = (ids // Hq) % T
    h = ids % Hq
    return b, h, i


def oracle_rows(w: W.Workload, b, h, i, part=oracle.PART_ALL):
    """The oracle's rows (b, h, i), spread over the host's cores (each row is the same
    single-threaded C code; the C call releases the GIL)."""
    arrs = w.as_numpy()
    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(16, ncpu or 1, len(b) // 8 or 1))
    idx = np.array_split(np.arange(len(b)), threads)
    with cf.ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(lambda k: oracle.rows(arrs, w.scale, b[k], h[k], i[k], part), idx))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def check_rows(w: W.Workload, out, lse, n_rows: int = 10**9, seed: int = 0, part=oracle.PART_ALL,
               out_tol=OUT_TOL, lse_tol=LSE_TOL):
    b, h, i = sample_rows(w, n_rows, seed)
    ro, rl = oracle_rows(w, b, h, i, part)
    go = out[b, i, h]
    gl = lse[b, h, i]
    if part == oracle.PART_PREFIX:
        empty = np.isneginf(rl)
        assert np.all(np.isneginf(gl[empty])) and np.all(go[empty] == 0)
        ro, rl, go, gl = ro[~empty], rl[~empty], go[~empty], gl[~empty]
    err_o = float(np.max(np.abs(go - ro))) if go.size else 0.0
    err_l = float(np.max(np.abs(gl - rl))) if gl.size else 0.0
    _log(f"  [{w.name}] rows={len(b)} max|out-oracle|={err_o:.3e} max|lse-oracle|={err_l:.3e}")
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert err_o <= out_tol, err_o
    assert err_l <= lse_tol, err_l
    return err_o, err_l


# ----------------------------------------------------------------------------- ancestor masks


@pytest.mark.parametrize("T", [1, 5, 7, 63, 64, 65, 68, 130, 256])
def test_ancestor_masks_bit_exact(T):
    _log(f"masks T={T}")
    gen = torch.Generator().manual_seed(100 + T)
    par = [W.random_forest(T, gen), W.chain_tree(T), W.star_tree(T)]
    if T == 68:
        par.append(W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen))
    pi = torch.tensor(par, dtype=torch.int32)
    got = hta.ancestor_masks(pi.cuda()).cpu().numpy().view(np.uint64)
    ref = oracle.ancestor_masks(pi.numpy())
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------------------- the parts


def _small(name, parents, *, B=2, Hq=8, Hkv=2, D=128, L=1000, plen=None, seed=0, peaky=0.02,
           dtype=torch.bfloat16):
    return W.make_workload(name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           max_prefix_len=L, parents=parents, prefix_len=plen, seed=seed,
                           peaky_frac=peaky, dtype=dtype)


def test_tree_part_alone_prefix_len_zero():
    """prefix_len = 0: the whole answer is the tree pass."""
    gen = torch.Generator().manual_seed(1)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(2)]
    w = _small("tree_only", par, L=128, plen=[0, 0], seed=1)
    out, lse = run_gpu(w)
    check_rows(w, out, lse)


def test_prefix_partials_match_oracle_per_chunk():
    """Each split-K partial against the oracle's attention over exactly that key chunk."""
    gen = torch.Generator().manual_seed(2)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(2)]
    w = _small("chunks", par, L=1000, plen=[1000, 777], seed=2)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk=256)
    ws = hta.new_workspace(desc, "cuda")
    hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
    torch.cuda.synchronize()
    lse_p, o_p = (x.cpu().double().numpy() for x in hta.partial_views(desc, ws))
    info = hta.plan(desc)
    G = w.num_q_heads // w.num_kv_heads
    rng = np.random.default_rng(0)
    worst_o = worst_l = 0.0
    for b in range(w.batch):
        Lb = int(w.prefix_len[b])
        for s in range((Lb + info.chunk - 1) // info.chunk):
            k0, k1 = s * info.chunk, min((s + 1) * info.chunk, Lb)
            for g in range(w.num_kv_heads):
                K = w.k_prefix[b, g, k0:k1].double().numpy()
                V = w.v_prefix[b, g, k0:k1].double().numpy()
                rows = rng.choice(w.tree_size * G, size=24, replace=False)
                Q = np.stack([w.q[b, r // G, g * G + r % G].double().numpy() for r in rows])
                ro, rl = oracle.masked_attention(Q, K, V, np.ones((len(rows), k1 - k0), bool),
                                                 w.scale)
                worst_o = max(worst_o, float(np.max(np.abs(o_p[b, g, s, rows] - ro))))
                worst_l = max(worst_l, float(np.max(np.abs(lse_p[b, g, s, rows] - rl))))
    _log(f"  per-chunk partials: max|o|={worst_o:.3e} max|lse|={worst_l:.3e}")
    assert worst_o <= OUT_TOL and worst_l <= LSE_TOL


def test_partial_rows_zero_and_wide_range():
    """The 16-bit partial rows against their contract in include/hta.h, read straight from the
    workspace: value = q * o_scale with o_scale = m / 32767, m at least the row's largest
    magnitude and at most the largest |v| the row attends to, and each value within half a
    step.  A KV head whose V is all zero gives factors of 0 and exact zeros; a KV head whose
    V dims span six orders of magnitude exercises the bound on the small dims."""
    gen = torch.Generator().manual_seed(3)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(2)]
    w = _small("partial_rows", par, L=700, plen=[700, 300], seed=3)
    w.v_prefix[:, 0] = 0
    dim_scale = torch.logspace(-3, 3, w.head_dim)
    w.v_prefix[:, 1] = (w.v_prefix[:, 1].float() * dim_scale).to(w.v_prefix.dtype)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk=256)
    ws = hta.new_workspace(desc, "cuda")
    hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
    torch.cuda.synchronize()
    lse_p, o_p = (x.cpu().double().numpy() for x in hta.partial_views(desc, ws))
    info = hta.plan(desc)
    S1, Rp = info.num_splits + 1, info.rows_padded
    n = w.batch * w.num_kv_heads * S1 * Rp
    fac = ws[info.o_scale_offset:info.o_scale_offset + 4 * n].view(torch.float32)
    fac = fac.view(w.batch, w.num_kv_heads, S1, Rp).cpu().double().numpy()
    G = w.num_q_heads // w.num_kv_heads
    R = w.tree_size * G
    worst = 0.0
    for b in range(w.batch):
        Lb = int(w.prefix_len[b])
        for s in range((Lb + info.chunk - 1) // info.chunk):
            assert np.all(fac[b, 0, s, :R] == 0.0) and np.all(o_p[b, 0, s, :R] == 0.0)
            assert np.all(np.isfinite(lse_p[b, 0, s, :R]))
            k0, k1 = s * info.chunk, min((s + 1) * info.chunk, Lb)
            K = w.k_prefix[b, 1, k0:k1].double().numpy()
            V = w.v_prefix[b, 1, k0:k1].double().numpy()
            Q = np.stack([w.q[b, r // G, G + r % G].double().numpy() for r in range(R)])
            ro, _ = oracle.masked_attention(Q, K, V, np.ones((R, k1 - k0), bool), w.scale)
            # the kernel's own error: the fp16 probabilities move each weight by at most
            # 2^-11 relative, so a dim's error is at most ~2 * 2^-11 of its largest |v|
            kern = 2.0 * 2.0 ** -11 * np.max(np.abs(V), axis=0)
            m = fac[b, 1, s, :R] * 32767.0
            assert np.all(m >= np.max(np.abs(ro), axis=1) - np.max(kern)), "factor below the row"
            assert np.all(m <= np.max(np.abs(V)) * (1 + 1e-6)), "factor above max |v|"
            err = np.abs(o_p[b, 1, s, :R] - ro)
            bound = kern[None, :] + 0.5 * 1.01 * fac[b, 1, s, :R, None]
            worst = max(worst, float(np.max(err / bound)))
    _log(f"  wide-range partial rows: worst error / (kernel + half-step) bound = {worst:.3f}")
    assert worst <= 1.0


def test_merge_matches_oracle_merge_of_gpu_partials():
    """lse_merge against the oracle's merge applied to the very partials the GPU produced."""
    gen = torch.Generator().manual_seed(3)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(2)]
    w = _small("merge", par, L=1000, plen=[1000, 321], seed=3)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk=128)
    ws = hta.new_workspace(desc, "cuda")
    hta.hta_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                          t["prefix_len"], ws)
    hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
    B, T, Hq, D = w.q.shape
    out = torch.empty(B, T, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, T, device="cuda")
    hta.hta_merge(desc, t["prefix_len"], True, out, lse, ws)
    torch.cuda.synchronize()
    lse_p, o_p = (x.cpu().double().numpy() for x in hta.partial_views(desc, ws))
    info = hta.plan(desc)
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    G = Hq // w.num_kv_heads
    worst = 0.0
    for b in range(B):
        n = (int(w.prefix_len[b]) + info.chunk - 1) // info.chunk
        slots = list(range(n)) + [info.num_splits]
        for i in range(0, T, 5):
            for h in range(Hq):
                g, r = h // G, i * G + h % G
                ro, rl = oracle.lse_merge(lse_p[b, g, slots, r], o_p[b, g, slots, r])
                worst = max(worst, float(np.max(np.abs(out[b, i, h] - ro))),
                            abs(lse[b, h, i] - rl))
    _log(f"  merge vs oracle merge of the same partials: {worst:.3e}")
    assert worst <= 1e-5


# ----------------------------------------------------------------------------- whole step


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 5, 8])
def test_verify_small_shapes(D, G):
    gen = torch.Generator().manual_seed(10 * G + D)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen), W.random_forest(68, gen)]
    w = _small(f"small_D{D}_G{G}", par, B=2, Hq=2 * G, Hkv=2, D=D, L=1100, plen=[1100, 613],
               seed=G + D)
    _log(f"verify small D={D} G={G}")
    out, lse = run_gpu(w)
    check_rows(w, out, lse)


@pytest.mark.parametrize("G,T", [(4, 4), (8, 4), (4, 40), (2, 68), (4, 36), (4, 68), (1, 64),
                                 (5, 50), (16, 17), (8, 40), (4, 12), (4, 16)])
def test_verify_row_tilings(G, T):
    """Row counts T*G covering every way the prefix pass splits query-row tiles over its
    waves: 1 or 2 tiles only, leftover tiles of 1 and 2 (their keys split over waves),
    several row blocks."""
    gen = torch.Generator().manual_seed(300 + 7 * G + T)
    par = [W.random_forest(T, gen), W.level_tree((T // 2, T - T // 2), gen)]
    w = _small(f"tiles_G{G}_T{T}", par, B=2, Hq=2 * G, Hkv=2, D=128, L=777, plen=[777, 350],
               seed=300 + G + T)
    _log(f"verify row tilings G={G} T={T} rows={T * G}")
    for chunk in (256, 0):
        out, lse = run_gpu(w, chunk=chunk)
        check_rows(w, out, lse, n_rows=3000)


@pytest.mark.parametrize("T", [16, 19, 22, 25, 35, 38, 41, 44, 68])
def test_verify_row_shapes_g5(T):
    """Five query heads per KV head (T*G = 80 .. 340 rows, a ragged last tile each): every
    split of 5 to 14 row tiles between the two wave groups, including second-group waves
    with fewer tiles than first-group ones, and 22 tiles in two blocks of 11."""
    G = 5
    gen = torch.Generator().manual_seed(500 + T)
    par = [W.random_forest(T, gen), W.level_tree((T // 3, T - T // 3), gen)]
    w = _small(f"shapes_G5_T{T}", par, B=2, Hq=2 * G, Hkv=2, D=128, L=650, plen=[650, 301],
               seed=500 + T)
    _log(f"verify row shapes G=5 T={T} rows={T * G}")
    for chunk in (192, 0):
        out, lse = run_gpu(w, chunk=chunk)
        check_rows(w, out, lse, n_rows=3000)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130, 256])
def test_verify_tree_sizes(T):
    gen = torch.Generator().manual_seed(T)
    par = [W.chain_tree(T), W.random_forest(T, gen)]
    w = _small(f"T{T}", par, B=2, Hq=4, Hkv=1, D=128, L=300, plen=[300, 65], seed=T)
    _log(f"verify T={T}")
    out, lse = run_gpu(w)
    check_rows(w, out, lse, n_rows=4000)


@pytest.mark.parametrize("chunk", [64, 192, 320, 448, 1024, 4096])
def test_verify_chunk_sizes_all_within_tolerance(chunk):
    """2999 keys in 47, 16, 10, 7, 3 and 1 splits: every size of the merge's per-lane batch
    of partials (9, 4, 4, 2, 1, 1 splits per lane) and its pass beyond the first batch."""
    gen = torch.Generator().manual_seed(7)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen)]
    w = _small("chunks", par, B=1, Hq=8, Hkv=2, L=3000, plen=[2999], seed=7)
    out, lse = run_gpu(w, chunk=chunk)
    check_rows(w, out, lse, n_rows=2000)


def test_verify_more_than_64_splits():
    """79 splits of 64 keys: the merge's pass over splits beyond its first 36 and its maximum
    over splits beyond the first 64 (every row checked)."""
    gen = torch.Generator().manual_seed(9)
    par = [W.level_tree((2, 3, 3), gen), W.chain_tree(8)]
    w = _small("splits79", par, B=2, Hq=8, Hkv=2, L=5000, plen=[5000, 4200], seed=9)
    _log("verify 79 splits")
    out, lse = run_gpu(w, chunk=64)
    check_rows(w, out, lse)


def test_largest_tree_and_group_at_32k():
    """The largest tree (T = 256) with the largest query group (G = 16: 4096 query rows per KV
    head, 16 row blocks of the prefix pass) over a 32k prefix, one random forest and one
    LongSpec-style level tree."""
    gen = torch.Generator().manual_seed(31)
    par = [W.random_forest(256, gen), W.level_tree((4, 16, 16, 60, 80, 80), gen)]
    w = _small("T256_G16_32k", par, B=2, Hq=32, Hkv=2, D=128, L=32768, plen=[32768, 20000],
               seed=31)
    _log("verify T=256 G=16 at 32k")
    out, lse = run_gpu(w)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check_rows(w, out, lse, n_rows=48, seed=4)


def test_million_token_prefix_sampled_rows():
    """The longest prefix in the suite: the Llama-3-8B layer shape at 2^20 prefix tokens (4 GiB
    of bf16 K/V, 128 splits of 8192 keys in the automatic plan)."""
    w = W.llama3_8b(1 << 20, seed=1005)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    assert hta.plan(desc).num_splits == 128
    _log(f"config {w.name}")
    out, lse = hta.verify(t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                          t["parent_idx"], t["prefix_len"], scale=w.scale)
    torch.cuda.synchronize()
    del t
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check_rows(w, out, lse, n_rows=16, seed=3)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 8), (128, 20, 4)])
def test_late_score_spikes(D, Hq, Hkv):
    """Keys far above every score of their chunk's first 32 keys (the prefix pass must not
    saturate its fp16 probabilities): keys equal to a multiple of one query's vector, placed
    early, mid-chunk and in a chunk's last tile, for rows of full and leftover row tiles."""
    gen = torch.Generator().manual_seed(21)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen)]
    w = _small(f"spikes_D{D}", par, B=1, Hq=Hq, Hkv=Hkv, D=D, L=3000, plen=[2990], seed=21,
               peaky=0.0)
    G = Hq // Hkv
    T = w.tree_size
    # (key position, query node, head in group, factor): score ~ factor * |q|^2 * scale
    spikes = [(5, 0, 0, 1.5), (700, T - 1, G - 1, 2.0), (1024 + 40, T // 2, 0, 3.0),
              (2047, T - 2, G // 2, 2.5), (2960, 3, G - 1, 2.0)]
    for g in range(Hkv):
        for pos, node, hg, f in spikes:
            qv = w.q[0, node, g * G + hg].float()
            w.k_prefix[0, g, pos] = (f * qv).to(w.k_prefix.dtype)
    _log(f"late spikes D={D} Hq={Hq} Hkv={Hkv}")
    for chunk in (1024, 0):
        out, lse = run_gpu(w, chunk=chunk)
        check_rows(w, out, lse)


@pytest.mark.parametrize("chunk,Lmax,plen", [
    # chunks whose first two tiles run past the prefix end (loaded before the length is known,
    # then loaded again with the rows past the end replaced): 70, 1, 127 and 100 keys in the
    # last chunk; a full cache; a last chunk too close to Lmax for the early loads
    (1024, 4096, [1024 + 70, 2048 + 1, 3072 + 127, 100, 4096]),
    (256, 1500, [256 + 64, 512 + 65, 1, 1500, 1280 + 127]),
    (128, 700, [128, 129, 640 + 1, 700, 63]),
])
def test_prefix_end_inside_first_tiles(chunk, Lmax, plen):
    """Prefix ends inside a chunk's first two 64-key tiles, with NaN in every cache row past
    the end: those rows are never read (a NaN V row times a zero probability would poison
    the row), for several chunk sizes and ragged lengths."""
    gen = torch.Generator().manual_seed(chunk)
    par = [W.level_tree((2, 3), gen) for _ in range(len(plen))]
    w = W.make_workload(f"prefix_end_{chunk}", batch=len(plen), num_q_heads=8, num_kv_heads=2,
                        head_dim=128, max_prefix_len=Lmax, parents=par, prefix_len=plen,
                        poison_padding=True, peaky_frac=0.02, seed=chunk + 5)
    _log(f"prefix end inside the first tiles: chunk={chunk} Lmax={Lmax} plen={plen}")
    out, lse = run_gpu(w, chunk=chunk)
    check_rows(w, out, lse)


def test_empty_and_tiny_prefixes():
    gen = torch.Generator().manual_seed(8)
    par = [W.level_tree((2, 3), gen) for _ in range(4)]
    w = _small("edge_prefix", par, B=4, Hq=4, Hkv=2, L=70, plen=[0, 1, 63, 70], seed=8)
    out, lse = run_gpu(w)
    check_rows(w, out, lse)


def test_empty_cache_capacity():
    w = _small("lmax0", [W.chain_tree(5)], B=1, Hq=4, Hkv=2, L=0, plen=[0], seed=9)
    out, lse = run_gpu(w)
    check_rows(w, out, lse)


def test_nan_padding_is_never_read():
    w = W.make_workload("poison", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=128,
                        max_prefix_len=700, prefix_len=[700, 300, 5],
                        tree_widths=W.LONGSPEC_TREE_WIDTHS, poison_padding=True, seed=11)
    out, lse = run_gpu(w)
    check_rows(w, out, lse)


def test_bitwise_deterministic():
    w = W.llama3_8b(4096, seed=5)
    a = run_gpu(w)
    b = run_gpu(w)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- device errors


def test_side_stream_matches_the_current_stream():
    """The wrappers on a second torch stream (default priority): the same bits as on the
    current stream, the outputs recorded on that stream by the wrapper."""
    gen = torch.Generator().manual_seed(41)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen) for _ in range(2)]
    w = _small("side_stream", par, B=2, Hq=8, Hkv=2, L=2000, plen=[2000, 1200], seed=41)
    t = to_dev(w)
    args = (t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"], t["parent_idx"],
            t["prefix_len"])
    ref_out, ref_lse = hta.verify(*args, scale=w.scale)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        out, lse = hta.verify(*args, scale=w.scale, stream=side)
    side.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_invalid_tree_is_flagged_and_poisons_only_its_sequence():
    gen = torch.Generator().manual_seed(12)
    good = W.level_tree((2, 3), gen)
    bad = list(good)
    bad[3] = 4  # parent after the child
    w = _small("badtree", [good, bad], B=2, Hq=4, Hkv=2, L=100, seed=12)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    ws = hta.new_workspace(desc, "cuda")
    B, T, Hq, D = w.q.shape
    out = torch.empty(B, T, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, T, device="cuda")
    hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                   t["parent_idx"], t["prefix_len"], out, lse, ws)
    code, seq = hta.hta_get_device_status(desc, ws)
    assert code == 6 and seq == 1
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(l[1]))
    assert np.all(np.isfinite(o[0])) and np.all(np.isfinite(l[0]))
    # a later good call clears the status
    t["parent_idx"][1] = torch.tensor(good, dtype=torch.int32)
    hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                   t["parent_idx"], t["prefix_len"], out, lse, ws)
    assert hta.hta_get_device_status(desc, ws) == (0, -1)


def test_prefix_len_out_of_range_is_flagged():
    w = _small("badlen", [W.chain_tree(3)] * 2, B=2, Hq=2, Hkv=1, L=64, seed=13)
    t = to_dev(w)
    t["prefix_len"] = torch.tensor([64, 65], dtype=torch.int32, device="cuda")
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale)
    ws = hta.new_workspace(desc, "cuda")
    out = torch.empty(2, 3, 2, 128, device="cuda")
    lse = torch.empty(2, 2, 3, device="cuda")
    hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                   t["parent_idx"], t["prefix_len"], out, lse, ws)
    code, seq = hta.hta_get_device_status(desc, ws)
    assert code == 7 and seq == 1
    assert np.all(np.isnan(out[1].cpu().numpy())) and np.all(np.isfinite(out[0].cpu().numpy()))


# ----------------------------------------------------------------------------- fp32 inputs

F32_TOL = 2e-5  # exact fp32 arithmetic against the fp64 oracle (log-sum-exp)
# outputs: the split-K partials pass through memory as 16-bit values with one factor per row
# (error at most 2^-16 of the row's largest magnitude, include/hta.h); a partial row is a
# convex combination of V rows, so |out - oracle| <= 2^-16 max|v| + fp32 rounding; max|v| < 6
# here
F32_OUT_TOL = 1e-4


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4])
def test_fp32_verify(D, G):
    gen = torch.Generator().manual_seed(40 + G + D)
    par = [W.level_tree(W.LONGSPEC_TREE_WIDTHS, gen), W.chain_tree(68)]
    w = _small(f"f32_D{D}_G{G}", par, B=2, Hq=2 * G, Hkv=2, D=D, L=700, plen=[700, 129],
               seed=41 + G + D, dtype=torch.float32)
    _log(f"fp32 verify D={D} G={G}")
    out, lse = run_gpu(w, chunk=256)
    check_rows(w, out, lse, out_tol=F32_OUT_TOL, lse_tol=F32_TOL)


def test_fp32_entry_points_match_oracle_parts():
    """fp32 through the separate entry points: tree partial alone, prefix partials alone, the
    plain merge, each against the oracle's part-wise attention."""
    gen = torch.Generator().manual_seed(50)
    par = [W.random_forest(130, gen)]
    w = _small("f32_parts", par, B=1, Hq=4, Hkv=2, D=64, L=600, plen=[577], seed=50,
               dtype=torch.float32)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, chunk=256)
    ws = hta.new_workspace(desc, "cuda")
    hta.hta_tree_partials(desc, t["q"], t["k_tree"], t["v_tree"], t["parent_idx"],
                          t["prefix_len"], ws)
    hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
    B, T, Hq, D = w.q.shape
    out = torch.empty(B, T, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, T, device="cuda")
    hta.hta_merge(desc, t["prefix_len"], True, out, lse, ws)
    torch.cuda.synchronize()
    assert hta.hta_get_device_status(desc, ws) == (0, -1)
    check_rows(w, out.cpu().double().numpy(), lse.cpu().double().numpy(), out_tol=F32_OUT_TOL,
               lse_tol=F32_TOL)
    lse_p, o_p = (x.cpu().double().numpy() for x in hta.partial_views(desc, ws))
    info = hta.plan(desc)
    G = Hq // w.num_kv_heads
    b_idx = np.zeros(T * Hq, dtype=np.int64)
    h_idx = np.tile(np.arange(Hq), T)
    i_idx = np.repeat(np.arange(T), Hq)
    ro, rl = oracle.rows(w.as_numpy(), w.scale, b_idx, h_idx, i_idx, oracle.PART_TREE)
    go = o_p[0, h_idx // G, info.num_splits, i_idx * G + h_idx % G]
    gl = lse_p[0, h_idx // G, info.num_splits, i_idx * G + h_idx % G]
    assert float(np.max(np.abs(go - ro))) <= F32_OUT_TOL
    assert float(np.max(np.abs(gl - rl))) <= F32_TOL


def test_fp32_invalid_tree_and_prefix_len():
    gen = torch.Generator().manual_seed(51)
    good = W.level_tree((2, 3), gen)
    bad = list(good)
    bad[2] = 2  # a node as its own parent
    w = _small("f32_bad", [good, bad], B=2, Hq=2, Hkv=1, D=64, L=100, seed=51,
               dtype=torch.float32)
    out, lse = run_gpu(w)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(lse[0]))


def test_stale_workspace_is_never_read():
    """A workspace whose every byte is 0xFF (NaN in every float slot) before the call: the
    whole step, the prefix-only merge (its tree slot is never written) and the drafter's
    cross-attention must not pick up anything they did not write themselves."""
    gen = torch.Generator().manual_seed(12)
    par = [W.level_tree((2, 6), gen) for _ in range(3)]
    w = W.make_workload("stale_ws", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        max_prefix_len=900, parents=par, prefix_len=[900, 0, 333],
                        poison_padding=True, seed=13)
    t = to_dev(w)
    desc = hta.desc_for(t["q"], t["k_prefix"], w.scale, 256)
    B, T, Hq, D = w.q.shape
    for mode in ("verify", "prefix_only", "cross"):
        ws = torch.full((hta.workspace_size(desc),), 0xFF, dtype=torch.uint8, device="cuda")
        out = torch.empty(B, T, Hq, D, dtype=torch.float32, device="cuda")
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
        if mode == "verify":
            hta.hta_verify(desc, t["q"], t["k_prefix"], t["v_prefix"], t["k_tree"], t["v_tree"],
                           t["parent_idx"], t["prefix_len"], out, lse, ws)
            part = oracle.PART_ALL
        elif mode == "prefix_only":
            hta.hta_prefix_partials(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"], ws)
            hta.hta_merge(desc, t["prefix_len"], False, out, lse, ws)
            part = oracle.PART_PREFIX
        else:
            hta.hta_cross_attention(desc, t["q"], t["k_prefix"], t["v_prefix"], t["prefix_len"],
                                    out, lse, ws)
            part = oracle.PART_PREFIX
        torch.cuda.synchronize()
        _log(f"  stale workspace, {mode}")
        check_rows(w, out.cpu().double().numpy(), lse.cpu().double().numpy(), part=part)
