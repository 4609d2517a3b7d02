#!/usr/bin/env python3
"""Benchmark of one tree-verification-attention step on one MI355X.

A step is one ``hta_verify`` call: ancestor masks + tree pass, split-K prefix pass, LSE
merge -- the whole verification attention of one layer -- on the Llama-3-8B layer shape
with a 32k-token prefix and the 68-node LongSpec draft tree (4,16,16,16,16).  Inputs are
seeded synthetic tensors already resident in HBM.  To time HBM rather than the 256 MB
Infinity Cache, consecutive steps rotate over copies of the prefix KV cache totalling at
least 1 GiB.

Prints ONE JSON line: the step time (us/step) plus, for the dominant kernel
(prefix_attn_splitk), its roofline figures measured live with HIP events around launches
of that kernel alone, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tree_verification_attention_amd as hta  # noqa: E402
from tree_verification_attention_amd import workloads as W  # noqa: E402

METRIC = "verification-attention µs/step + achieved HBM GB/s, Llama-3-8B shape, 32k prefix"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix, published
ROTATE_BYTES = 1 << 30
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "tree_verification_attention_amd", "csrc",
                          "prefix_attn_splitk.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def settle(fn, seconds: float) -> int:
    """Call fn until `seconds` of wall time have passed, so the engine clock has reached its
    steady state under this load before anything is timed.  Returns the calls made."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(20):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_loop(fn, n: int, stream):
    """n calls of fn timed two ways at once: wall clock between device synchronisations, and
    HIP events recorded on the launch stream around the same calls.  µs per call each."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(n):
        fn(k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n * 1e6
    return wall, e0.elapsed_time(e1) / n * 1e3


def kv_rotation(w: W.Workload, dev):
    """The prefix cache on the device plus copies, so that consecutive calls together touch at
    least ROTATE_BYTES (more than the 256 MB Infinity Cache) and time HBM."""
    kv_copy_bytes = w.k_prefix.numel() * w.k_prefix.element_size() * 2
    n_copies = max(1, min(64, math.ceil(ROTATE_BYTES / kv_copy_bytes)))
    kp0, vp0 = w.k_prefix.to(dev), w.v_prefix.to(dev)
    kps = [kp0] + [kp0.clone() for _ in range(n_copies - 1)]
    vps = [vp0] + [vp0.clone() for _ in range(n_copies - 1)]
    return kps, vps, n_copies, kv_copy_bytes


def roofline_figures(fig: dict, step_us: float, prefix_us: float) -> dict:
    """Achieved rates of a step against the published peaks; the bound is whichever of the
    HBM time and the matrix-core time of the algorithmic work is longer."""
    t_hbm = fig["step_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = fig["step_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    gbs = fig["step_bytes"] / (step_us * 1e-6) / 1e9
    tfs = fig["step_flops"] / (step_us * 1e-6) / 1e12
    return {
        "us_per_step": round(step_us, 3),
        "prefix_us": round(prefix_us, 3),
        "alg_bytes": fig["step_bytes"], "alg_flops": fig["step_flops"],
        "GBps": round(gbs, 1), "TFLOPs": round(tfs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
        "bound": "mfma" if t_mfma > t_hbm else "hbm",
        "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 3),
        "roofline_frac": round(max(t_hbm, t_mfma) / (step_us * 1e-6), 4),
        "prefix_GBps": round(fig["prefix_bytes"] / (prefix_us * 1e-6) / 1e9, 1),
        "prefix_TFLOPs": round(fig["prefix_flops"] / (prefix_us * 1e-6) / 1e12, 1),
    }


def alg_figures(w: W.Workload):
    """Algorithmic bytes and flops of one step and of the prefix kernel alone.

    Per KV head and prefix key the prefix pass must read 2*D*2 bytes of K and V (bf16) and
    performs 4*D*T*G flops (QK^T and PV for all T*G query rows that share the head).
    """
    B, T, Hq, D = w.q.shape
    Hkv = w.num_kv_heads
    G = Hq // Hkv
    el = w.q.element_size()
    sum_L = int(w.prefix_len.sum())
    depths = [W.depths(p) for p in w.parent_idx.tolist()]
    vis_tree = sum(sum(d) + len(d) for d in depths)  # sum over nodes of (depth + 1)
    kv_bytes = 2 * Hkv * sum_L * D * el
    q_bytes = B * T * Hq * D * el
    prefix_bytes = kv_bytes + q_bytes
    prefix_flops = 4 * D * G * T * Hkv * sum_L
    step_bytes = (prefix_bytes + 2 * B * Hkv * T * D * el + B * T * 4
                  + B * T * Hq * D * 4 + B * Hq * T * 4 + B * 4)
    step_flops = prefix_flops + 4 * D * Hq * vis_tree
    return dict(step_bytes=step_bytes, step_flops=step_flops, prefix_bytes=prefix_bytes,
                prefix_flops=prefix_flops, kv_bytes_per_unit=2 * D * el,
                kv_units=Hkv * sum_L)


KERNEL_HEADERS = [os.path.join(os.path.dirname(KERNEL_SRC), h)
                  for h in ("hta_internal.h", "lds_tiles.h")]


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (string literals are not
    special-cased: the kernel sources hold none with comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the prefix kernel's code (its source and the two headers it includes, comments
    and layout ignored): the committed counters are reported only for this code."""
    h = hashlib.sha256()
    for path in [KERNEL_SRC, *KERNEL_HEADERS]:
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic of the prefix kernel from committed rocprofv3 counter runs, only if they
    were taken on the current kernel source."""
    p = os.path.join(PROFILE_DIR, f"prefix_attn_splitk_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256_16") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def _counter_means(run_dir: str, kernel_substr: str, counter: str):
    """Mean per-dispatch value of one rocprofv3 counter over the dispatches of one kernel."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples of {kernel_substr} under {run_dir}")
    return sum(vals) / len(vals), len(vals)


def summarize_counters(workload: str, fetch_dir: str, write_dir: str, fetch_copy_dir: str,
                       write_copy_dir: str) -> str:
    """HBM traffic of the prefix kernel per launch from four rocprofv3 --pmc runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the prefix kernel (--mode prefix-only) are
    scaled by what the same counters read for the plain 256 MiB copy (--mode copy), so the
    result is in bytes actually moved.  Written next to the other profiles, with the kernel
    source hash: the bench reports the figure only while the kernel source is unchanged.
    """
    copy_bytes = 256 << 20
    kern = "prefix_attn_splitk"
    f_k, nf = _counter_means(fetch_dir, kern, "FETCH_SIZE")
    w_k, nw = _counter_means(write_dir, kern, "WRITE_SIZE")
    f_c, _ = _counter_means(fetch_copy_dir, "copyBuffer", "FETCH_SIZE")
    w_c, _ = _counter_means(write_copy_dir, "copyBuffer", "WRITE_SIZE")
    f_factor = copy_bytes / (f_c * 1024)
    w_factor = copy_bytes / (w_c * 1024)
    rd = f_k * 1024 * f_factor
    wr = w_k * 1024 * w_factor
    w = W.by_name(workload)
    alg = alg_figures(w)["prefix_bytes"]
    rec = {
        "kernel": kern, "workload": workload, "kernel_sha256_16": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": round(f_k, 2), "write_size_kib_per_dispatch": round(w_k, 2),
        "dispatches_sampled": {"fetch": nf, "write": nw},
        "copy_calibration": {"bytes_copied": copy_bytes, "fetch_size_kib": round(f_c, 2),
                             "write_size_kib": round(w_c, 2), "fetch_factor": round(f_factor, 4),
                             "write_factor": round(w_factor, 4)},
        "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
        "traffic_bytes_per_launch": int(rd + wr), "alg_bytes_per_launch": alg,
        "read_over_alg": round(rd / alg, 4),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
            "python3 bench.py --mode prefix-only --steps 10 --warmup 2",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- "
            "python3 bench.py --mode prefix-only --steps 10 --warmup 2",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_copy_dir} -o run -- "
            "python3 bench.py --mode copy --steps 5 --warmup 1",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_copy_dir} -o run -- "
            "python3 bench.py --mode copy --steps 5 --warmup 1",
            f"python3 bench.py --summarize-counters {fetch_dir} {write_dir} {fetch_copy_dir} "
            f"{write_copy_dir}",
        ],
    }
    out = os.path.join(PROFILE_DIR, f"prefix_attn_splitk_{workload}_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return out


def cpu_baseline(w: W.Workload, max_seconds: float = 12.0):
    """Time the oracle (plain fp64 C, one row per call of its loop nest) on a bounded sample of
    the workload's query rows, scaled per step: once on one thread, then with the same rows
    spread over the host's cores (the identical single-threaded code per row; the outputs
    must be bitwise equal)."""
    import concurrent.futures as cf
    import platform

    import oracle  # test infrastructure: only this baseline leg uses it
    a = w.as_numpy()
    B, T, Hq = w.batch, w.tree_size, w.num_q_heads
    total = B * T * Hq
    rng = np.random.default_rng(0)
    # calibrate with a few rows, then size the sample to the time budget
    rb, ri, rh = [0] * 8, list(range(8)), [0] * 8
    t0 = time.perf_counter()
    oracle.rows(a, w.scale, rb, rh, ri)
    per_row = (time.perf_counter() - t0) / 8
    n = int(min(total, max(16, max_seconds / max(per_row, 1e-9))))
    ids = np.sort(rng.choice(total, size=n, replace=False))
    b, i, h = ids // (T * Hq), (ids // Hq) % T, ids % Hq
    t0 = time.perf_counter()
    o1, l1 = oracle.rows(a, w.scale, b, h, i)
    dt1 = time.perf_counter() - t0
    # every core this process may run on, up to the 16-core host share one GPU has on the
    # benchmark machines (their rule for worker pools)
    allowed = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    host_cores = os.cpu_count() or 1
    threads = max(1, min(16, allowed or host_cores))
    parts = np.array_split(np.arange(n), threads)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:  # the C call releases the GIL
        res = list(ex.map(lambda ix: oracle.rows(a, w.scale, b[ix], h[ix], i[ix]), parts))
    dtn = time.perf_counter() - t0
    on = np.concatenate([r[0] for r in res])
    ln = np.concatenate([r[1] for r in res])
    cpu = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(x.split(":", 1)[1].strip() for x in f if x.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": dtn / n * total * 1e6, "unit": "µs/step", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {total} query rows (b, head, node) of the same workload, fp64 C "
                      f"oracle, rows spread over {threads} threads ({dtn:.1f} s), scaled to the "
                      f"full step",
            "host_cores": host_cores, "cores_allowed": allowed,
            "threads_note": "threads = the cores this process may use, capped at the 16-core "
                            "host share of one GPU on the benchmark machines",
            "single_thread_value": dt1 / n * total * 1e6,
            "bitwise_equal_across_threads": bool(np.array_equal(o1, on) and np.array_equal(l1, ln)),
            "cpu_model": cpu}


SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_COEXEC_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT "
    "SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_INSTS_VALU SQ_INSTS_MFMA",
    "SQ_CYCLES SQ_WAVES SQ_INSTS_LDS SQ_INSTS_SALU SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VMEM "
    "SQ_INST_LEVEL_LDS SQ_ACTIVE_INST_MISC",
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_LDS_IDX_ACTIVE "
    "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE GRBM_COUNT",
)
# GRBM counters are summed over the chip's XCDs (one instance each)
XCDS = 8


def summarize_sq(workload: str, dirs) -> str:
    """SQ counters of the prefix kernel from the rocprofv3 --pmc passes of SQ_PASSES (each on
    --mode prefix-only) as a markdown table plus the per-wave and per-SIMD ratios; with the
    fourth pass also the matrix-core and LDS utilisation over the kernel's active cycles and
    the matrix-core flops executed against the algorithmic ones."""
    kern = "prefix_attn_splitk"
    vals = {}
    for i, (d, counters) in enumerate(zip(dirs, SQ_PASSES)):
        for c in counters.split():
            key = c if i < 3 or c not in vals else c + " (4th pass)"
            vals[key] = _counter_means(d, kern, c)[0]
    waves = vals["SQ_WAVES"]
    per = lambda c: vals[c] / waves  # noqa: E731
    life = per("SQ_WAVE_CYCLES")
    simds = 1024
    mfma_busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    cmds = "\n".join(
        f"rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python3 bench.py "
        f"--workload {workload} --mode prefix-only --steps 10 --warmup 2"
        for d, c in zip(dirs, SQ_PASSES))
    lines = [f"# SQ counters: prefix_attn_splitk, {workload}", "",
             f"Commands (from the repository root, on one MI355X; {len(dirs)} passes of at most "
             "eight SQ and two GRBM counters each), then `python3 bench.py --workload " + workload +
             " --summarize-sq " + " ".join(dirs) + "`:", "", "```",
             "cd /tmp && export TMPDIR=/tmp && cd -", cmds, "```", "",
             f"Kernel code sha256[:16] (source and included headers, comments ignored) = `{kernel_source_hash()}`.  Values: per dispatch, "
             "summed over the chip's counter instances, averaged over the sampled dispatches.",
             "", "| Counter | Per dispatch |", "|---|---:|"]
    for c in sorted(vals):
        lines.append(f"| `{c}` | {vals[c]:,.0f} |")
    lines += ["",
              f"Per wave ({waves:,.0f} waves; wave-cycle counters count 4-cycle units): lifetime "
              f"{life:,.0f} units; issuing (ACTIVE_INST_ANY) {per('SQ_ACTIVE_INST_ANY') / life:.0%}, "
              f"stalled on dependencies (WAIT_INST_ANY) {per('SQ_WAIT_INST_ANY') / life:.0%}, "
              f"waiting at s_waitcnt / barriers (WAIT_ANY) {per('SQ_WAIT_ANY') / life:.0%}.  "
              f"Matrix core: VALU_MFMA_BUSY {mfma_busy:,.0f} cycles per SIMD; VALU and MFMA "
              f"co-execute in {vals['SQ_VALU_MFMA_COEXEC_CYCLES'] / vals['SQ_VALU_MFMA_BUSY_CYCLES']:.0%} "
              f"of the MFMA-busy cycles.  Instructions per wave: {per('SQ_INSTS_MFMA'):,.0f} MFMA, "
              f"{per('SQ_INSTS_VALU'):,.0f} VALU (MFMA included), {per('SQ_INSTS_LDS'):,.0f} LDS, "
              f"{per('SQ_INSTS_SALU'):,.0f} SALU; LDS bank-conflict cycles "
              f"{per('SQ_LDS_BANK_CONFLICT'):,.0f} per wave."]
    if "GRBM_GUI_ACTIVE" in vals:
        active = vals["GRBM_GUI_ACTIVE"] / XCDS  # the kernel's active cycles (one XCD's count)
        busy4 = vals.get("SQ_VALU_MFMA_BUSY_CYCLES (4th pass)", vals["SQ_VALU_MFMA_BUSY_CYCLES"])
        mops = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + vals["SQ_INSTS_VALU_MFMA_MOPS_F16"]
        alg = alg_figures(W.by_name(workload))["prefix_flops"]
        lines += ["",
                  f"Over the kernel's active cycles (GRBM_GUI_ACTIVE / {XCDS} XCDs = {active:,.0f} "
                  f"cycles per dispatch): matrix core busy {busy4 / (active * simds):.0%} of SIMD "
                  f"cycles; LDS busy (SQ_LDS_IDX_ACTIVE) {vals['SQ_LDS_IDX_ACTIVE'] / (active * 256):.0%} "
                  f"of CU cycles.  Matrix-core flops executed (MFMA MOPS x 512: bf16 "
                  f"{vals['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.2f} G, fp16 "
                  f"{vals['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512 / 1e9:.2f} G) = {mops * 512 / alg:.3f}x "
                  f"the pass's algorithmic {alg / 1e9:.2f} GFLOP (row-sum products, padded rows and "
                  f"the zero half of the leftover products included)."]
    out = os.path.join(PROFILE_DIR, f"prefix_attn_splitk_{workload}_sq_counters.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


# The configurations of the pages' evaluation besides the headline: the 262k-context Llama-3
# checkpoint, Vicuna-7B at batch 8 with ragged prefixes, and the QwQ-32B long-reasoning sweep
# on the LongSpec tree and on a 5-token chain.
OTHER_CONFIGS = ("llama3_8b_256k", "vicuna7b_b8",
                 "qwq32b_tree_4k", "qwq32b_tree_8k", "qwq32b_tree_16k", "qwq32b_tree_32k",
                 "qwq32b_chain5_4k", "qwq32b_chain5_8k", "qwq32b_chain5_16k",
                 "qwq32b_chain5_32k")


def bench_config(name: str, dev, stream, settle_s: float = 0.25, target_s: float = 0.2) -> dict:
    """One configuration: its step (hta_verify) and its prefix pass alone, timed like the
    headline (clock settled, warm-up, then wall clock and HIP events over the same calls),
    with the step's algorithmic bytes and flops against both peaks."""
    w = W.by_name(name)
    fig = alg_figures(w)
    B, T, Hq, D = w.q.shape
    q = w.q.to(dev)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    par, plen = w.parent_idx.to(dev), w.prefix_len.to(dev)
    kps, vps, n_copies, _ = kv_rotation(w, dev)
    desc = hta.desc_for(q, kps[0], w.scale)
    info = hta.plan(desc)
    ws = hta.new_workspace(desc, dev)
    out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    steps = [hta.prepare_verify(desc, q, kps[c], vps[c], kt, vt, par, plen, out, lse, ws, stream)
             for c in range(n_copies)]
    pres = [hta.prepare_prefix_partials(desc, q, kps[c], vps[c], plen, ws, stream)
            for c in range(n_copies)]
    t0 = time.perf_counter()
    n_settle = settle(lambda k: steps[k % n_copies](), settle_s)
    per_call = (time.perf_counter() - t0) / n_settle
    code, _ = hta.hta_get_device_status(desc, ws, stream)
    if code != 0:
        raise RuntimeError(f"{name}: device status {hta.status_str(code)}")
    n = int(min(2000, max(50, target_s / per_call)))
    wall, ev = time_loop(lambda k: steps[k % n_copies](), n, stream)
    for k in range(50):
        pres[k % n_copies]()
    _, pre = time_loop(lambda k: pres[k % n_copies](), n, stream)
    rec = roofline_figures(fig, wall, pre)
    rec.update({
        "events_us": round(ev, 3), "steps_timed": n,
        "batch": B, "num_q_heads": Hq, "num_kv_heads": w.num_kv_heads, "tree_nodes": T,
        "prefix_len_sum": int(w.prefix_len.sum()), "prefix_len_max": int(w.prefix_len.max()),
        "chunk": info.chunk, "splits": info.num_splits, "kv_copies_rotated": n_copies,
    })
    log(f"[bench] {name}: {wall:.2f} us/step (events {ev:.2f}), prefix {pre:.2f} us, "
        f"{rec['GBps']:.0f} GB/s, {rec['TFLOPs']:.0f} TFLOP/s, {rec['bound']}-bound, "
        f"roofline {rec['roofline_frac']:.3f}")
    del steps, pres, kps, vps, q, kt, vt, par, plen, ws, out, lse, w
    torch.cuda.empty_cache()
    return rec


def summarize_trace(run_dir: str, workload: str, command: str) -> str:
    """A kernel-trace summary (rocprofv3 --kernel-trace --stats) of a --mode step-only run as a
    markdown table under profiles/: calls, average, min, max and share per kernel."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["Percentage"])))
    rows.sort(key=lambda x: -x[5])
    w = W.by_name(workload)
    fig = alg_figures(w)
    whole = "--mode step-only" not in command
    title = (f"the whole bench.py run on {workload} (headline, kernels alone, baselines, other "
             f"configurations)" if whole else f"one verification step per call, {workload}")
    lines = [f"# Kernel trace: {title}", "",
             "Command (from the repository root, on one MI355X):", "", "```",
             "cd /tmp && export TMPDIR=/tmp && cd - && " + command, "```", "",
             f"Workload: batch {w.batch}, {w.num_q_heads} query / {w.num_kv_heads} KV heads, "
             f"head_dim {w.head_dim}, {w.tree_size} tree nodes, prefix lengths summing to "
             f"{int(w.prefix_len.sum())} (max {int(w.prefix_len.max())}).  Algorithmic bytes "
             f"per step {fig['step_bytes']}, flops {fig['step_flops']}.  Counts include "
             "the clock-settling and warm-up launches; the copies are the rotated prefix caches "
             "being made.", "",
             "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |",
             "|---|---:|---:|---:|---:|---:|"]
    for name, calls, avg, mn, mx, pct in rows:
        short = name.replace("hta::(anonymous namespace)::", "").replace("void ", "")
        short = short.split("(")[0] if not short.startswith("__amd") else short
        lines.append(f"| `{short}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f}% |")
    out = os.path.join(PROFILE_DIR, f"{'bench' if whole else 'verify_step'}_{workload}"
                                    "_kernel_stats.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


def measured_peaks(dev) -> dict:
    """What this GPU sustains right now: a 512 MiB device copy (HBM read + write) and a large
    bf16 GEMM (the vendor BLAS, matrix cores).  Context for the spec peaks."""
    n = 512 << 20
    src = torch.empty(n // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    copy_gbs = 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    m = 8192
    x = torch.randn(m, m, device=dev).to(torch.bfloat16)
    y = torch.randn(m, m, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, y)
    e0.record()
    for _ in range(10):
        torch.matmul(x, y)
    e1.record()
    e1.synchronize()
    gemm_tf = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y
    # the matrix cores alone: independent bf16 products on register operands (no memory),
    # with 2 waves per SIMD (the prefix pass's occupancy) and with 8
    stream = torch.cuda.current_stream()
    loop_tf = {}
    for label, blocks in (("2_waves_per_simd", 256), ("8_waves_per_simd", 1024)):
        out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
        call, flops = hta.prepare_mfma_peak_probe(blocks, 8192 * 256 // blocks, out, stream)
        for _ in range(3):
            call()
        e0.record(stream)
        for _ in range(10):
            call()
        e1.record(stream)
        e1.synchronize()
        loop_tf[label] = round(flops * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del out
    return {"hbm_copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tf, 1),
            "bf16_mfma_loop_TFLOPs": loop_tf,
            "how": "512 MiB device copy (bytes read + written); 8192^3 bf16 torch.matmul; "
                   "hta_mfma_peak_probe: eight independent v_mfma_f32_16x16x32_bf16 chains per "
                   "wave on register operands"}


def around_figures(name: str):
    """Vocabulary and rotary base of the checkpoint a workload stands for."""
    if name.startswith("vicuna"):
        return W.VICUNA_VOCAB, W.VICUNA_ROPE_THETA
    if name.startswith("qwq"):
        return W.QWQ_VOCAB, W.QWQ_ROPE_THETA
    return W.LLAMA3_VOCAB, W.LLAMA3_ROPE_THETA


def bench_around(w: W.Workload, dev, stream, steps: int, warmup: int) -> dict:
    """The steps on either side of the attention, timed with HIP events on the launch
    stream: rotary encoding of the tree (hta_rope_tree), then the target's greedy tokens,
    acceptance and KV commit (hta_accept_commit: the argmax launch and the acceptance
    launch).  The caches grow by the accepted path on every call, as in decoding."""
    vocab, theta = around_figures(w.name)
    B, T, Hq, D = w.q.shape
    Hkv = w.num_kv_heads
    st = W.make_step_inputs(w.parent_idx.tolist(), vocab, dtype=torch.bfloat16, seed=w.seed + 7)
    calls = warmup + 2 * steps
    depth = max(max(W.depths(p)) for p in w.parent_idx.tolist()) + 1
    Lmax = w.max_prefix_len + calls * depth
    q = w.q.to(dev)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    par = w.parent_idx.to(dev)
    plen0 = w.prefix_len.to(dev)
    kp = torch.empty(B, Hkv, Lmax, D, dtype=w.dtype, device=dev)
    vp = torch.empty_like(kp)
    logits, tok, root = st.logits.to(dev), st.tokens.to(dev), st.root_token.to(dev)
    desc = hta.make_desc(B, Hq, Hkv, D, T, Lmax, hta.binding._dtype_code(w.q))
    ws = torch.empty(hta.accept_workspace_size(desc, vocab), dtype=torch.uint8, device=dev)
    plen = plen0.clone()
    outs = [torch.empty(B, T, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(B, T, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev)]

    # prepared calls (checked once), so the loops are not paced by the host
    rope = hta.prepare_rope_tree(desc, theta, False, q, kt, par, plen, None, ws, stream)
    accept = hta.prepare_accept_commit(desc, logits, tok, root, par, plen, kp, vp, kt, vt, *outs,
                                       ws, stream)

    for _ in range(warmup):
        rope()
        accept()
    torch.cuda.synchronize()
    code, _ = hta.hta_get_device_status(desc, ws, stream)
    if code != 0:
        raise RuntimeError(f"device status {hta.status_str(code)}")
    n_acc = outs[1].float().mean().item()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        rope()
    e1.record(stream)
    e1.synchronize()
    rope_us = e0.elapsed_time(e1) / steps * 1e3
    e0.record(stream)
    for _ in range(steps):
        accept()
    e1.record(stream)
    e1.synchronize()
    accept_us = e0.elapsed_time(e1) / steps * 1e3
    code, _ = hta.hta_get_device_status(desc, ws, stream)
    if code != 0:
        raise RuntimeError(f"device status {hta.status_str(code)}")
    esz = w.q.element_size()
    rope_bytes = 2 * (B * T * Hq * D + B * Hkv * T * D) * esz
    logits_bytes = B * T * vocab * 2
    log(f"[bench] rope_tree {rope_us:.2f} us; accept_commit (argmax + acceptance) "
        f"{accept_us:.2f} us; {n_acc:.2f} nodes accepted per sequence")
    return {
        "vocab": vocab, "rope_theta": theta, "logits_dtype": "bf16",
        "accepted_nodes_per_sequence": round(n_acc, 3),
        "rope_tree_us": round(rope_us, 3),
        "rope_tree_alg_bytes": rope_bytes,
        "accept_commit_us": round(accept_us, 3),
        "logits_bytes": logits_bytes,
        "accept_commit_GBps": round(logits_bytes / (accept_us * 1e-6) / 1e9, 1),
        "accept_commit_frac_of_hbm_peak": round(logits_bytes / (accept_us * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4),
        "note": "accept_commit = the vocabulary argmax launch plus the acceptance/commit "
                "launch, per call (prepared calls, HIP events around the loop); the kernel "
                "trace splits the two",
    }


def bench_drafter(w: W.Workload, dev, stream, steps: int, kps, vps, n_copies: int) -> dict:
    """The drafter's attention on the same target cache, HIP events on the launch stream:
    cross-attention of one drafted level (16 queries) into the target's KV cache, and the
    windowed self-attention (512-position ring as the prefix) of a 4,16 draft tree."""
    B, T, Hq, D = w.q.shape
    Hkv = w.num_kv_heads
    gen = torch.Generator().manual_seed(w.seed + 11)
    qc = torch.randn(B, 16, Hq, D, generator=gen).to(w.dtype).to(dev)
    plen = w.prefix_len.to(dev)
    dc = hta.desc_for(qc, kps[0], w.scale)
    wsc = hta.new_workspace(dc, dev)
    oc = torch.empty(B, 16, Hq, D, dtype=torch.float32, device=dev)
    lc = torch.empty(B, Hq, 16, dtype=torch.float32, device=dev)
    win = 512
    par = torch.tensor([W.level_tree((4, 16), gen) for _ in range(B)], dtype=torch.int32,
                       device=dev)
    Tw = par.shape[1]
    qw = torch.randn(B, Tw, Hq, D, generator=gen).to(w.dtype).to(dev)
    kr = torch.randn(B, Hkv, win, D, generator=gen).to(w.dtype).to(dev)
    vr = torch.randn(B, Hkv, win, D, generator=gen).to(w.dtype).to(dev)
    kt = torch.randn(B, Hkv, Tw, D, generator=gen).to(w.dtype).to(dev)
    vt = torch.randn(B, Hkv, Tw, D, generator=gen).to(w.dtype).to(dev)
    wl = torch.full((B,), win, dtype=torch.int32, device=dev)
    dw = hta.desc_for(qw, kr, w.scale)
    wsw = hta.new_workspace(dw, dev)
    ow = torch.empty(B, Tw, Hq, D, dtype=torch.float32, device=dev)
    lw = torch.empty(B, Hq, Tw, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for k in range(50):
            fn(k)
        e0.record(stream)
        for k in range(steps):
            fn(k)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    # prepared calls (checked once), so the loops are not paced by the host
    cross = [hta.prepare_cross_attention(dc, qc, kps[c], vps[c], plen, oc, lc, wsc, stream)
             for c in range(n_copies)]
    window = hta.prepare_verify(dw, qw, kr, vr, kt, vt, par, wl, ow, lw, wsw, stream)
    cross_us = timed(lambda k: cross[k % n_copies]())
    window_us = timed(lambda k: window())
    kv_bytes = int(w.prefix_len.sum()) * Hkv * D * 2 * w.k_prefix.element_size()
    log(f"[bench] drafter: cross-attention (16 queries) {cross_us:.2f} us, window self-attention "
        f"(512 + 4,16 tree) {window_us:.2f} us")
    return {
        "cross_attention_us": round(cross_us, 3), "cross_attention_queries": 16,
        "cross_attention_GBps": round(kv_bytes / (cross_us * 1e-6) / 1e9, 1),
        "window_self_attention_us": round(window_us, 3), "window": win, "window_tree_nodes": Tw,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first: the engine clock settles after a few hundred")
    ap.add_argument("--workload", default="llama3_8b_32k", choices=W.CONFIG_NAMES)
    ap.add_argument("--chunk", type=int, default=0, help="split-K chunk (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="bench", choices=["bench", "prefix-only", "step-only",
                                                         "copy"],
                    help="prefix-only / step-only / copy: launch only that (for profiler runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (the configs object)")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up, so the engine clock is "
                         "at its steady state under this load")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="write the prefix kernel's SQ counters from the rocprofv3 --pmc passes "
                         "of SQ_PASSES (three or all four, in order) into profiles/ and exit; "
                         "needs no GPU")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "COMMAND"),
                    help="write a kernel-trace summary of --workload from a rocprofv3 "
                         "--kernel-trace --stats output folder into profiles/ and exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar="DIR",
                    help="write the prefix kernel's HBM traffic from four rocprofv3 --pmc "
                         "output folders (FETCH_SIZE, WRITE_SIZE, then the same for --mode "
                         "copy) into profiles/ and exit; needs no GPU")
    args = ap.parse_args()

    if args.summarize_counters:
        print(summarize_counters(args.workload, *args.summarize_counters))
        return 0
    if args.summarize_sq:
        print(summarize_sq(args.workload, args.summarize_sq))
        return 0
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace[0], args.workload, args.summarize_trace[1]))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU (the work shards by KV head with no "
              "communication); run with --gpus 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    hta.load()

    if args.mode == "copy":
        # plain copy of known size: calibrates the FETCH_SIZE / WRITE_SIZE counters
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n,
                          "launches": args.warmup + args.steps}))
        return 0

    log(f"[bench] workload {args.workload}: generating inputs")
    w = W.by_name(args.workload)
    fig = alg_figures(w)
    B, T, Hq, D = w.q.shape
    q = w.q.to(dev)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    par, plen = w.parent_idx.to(dev), w.prefix_len.to(dev)
    kps, vps, n_copies, kv_copy_bytes = kv_rotation(w, dev)
    desc = hta.desc_for(q, kps[0], w.scale, args.chunk)
    info = hta.plan(desc)
    ws = hta.new_workspace(desc, dev)
    out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] chunk {info.chunk}, splits {info.num_splits}, rows {info.rows}, "
        f"{n_copies} KV copies of {kv_copy_bytes / 1e6:.1f} MB")

    # one prepared call per KV copy: arguments checked and marshalled once, so the timed loops
    # measure the GPU and not the binding's per-call checks
    step_calls = [hta.prepare_verify(desc, q, kps[c], vps[c], kt, vt, par, plen, out, lse, ws,
                                     stream) for c in range(n_copies)]
    prefix_calls = [hta.prepare_prefix_partials(desc, q, kps[c], vps[c], plen, ws, stream)
                    for c in range(n_copies)]

    def step(k):
        step_calls[k % n_copies]()

    def prefix_only(k):
        prefix_calls[k % n_copies]()

    if args.mode in ("prefix-only", "step-only"):
        fn = prefix_only if args.mode == "prefix-only" else step
        if args.mode == "step-only":  # (not under counter collection: too slow there)
            settle(fn, args.settle)
        for k in range(args.warmup + args.steps):
            fn(k)
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "workload": args.workload,
                          "launches": args.warmup + args.steps,
                          "alg_bytes_per_launch": fig["prefix_bytes"]}))
        return 0

    # ---- whole step: clock settled, W warm-up steps, then exactly K timed steps, each loop
    # bracketed by device synchronisations; wall clock (the headline) and HIP events on the
    # launch stream measure the same K calls
    settle_calls = settle(step, args.settle)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    code, _ = hta.hta_get_device_status(desc, ws, stream)
    if code != 0:
        raise RuntimeError(f"device status {hta.status_str(code)}")
    us_per_step, step_events_us = time_loop(step, args.steps, stream)
    log(f"[bench] step: {us_per_step:.2f} us wall clock, {step_events_us:.2f} us HIP events "
        f"({settle_calls} settle + {args.warmup} warm-up steps first)")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # secondary loops (kernels alone, the spread of single calls) run at least this many
    # calls, each after a warm-up of its own
    n_side = max(args.steps, 200)
    # each call between its own event pair: the spread of single steps
    n_calls = n_side
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_calls)]
    for k, (a0, a1) in enumerate(evs):
        a0.record(stream)
        step(k)
        a1.record(stream)
    torch.cuda.synchronize()
    per_call = np.array([a0.elapsed_time(a1) * 1e3 for a0, a1 in evs])
    p10, p50, p90 = (float(np.percentile(per_call, q)) for q in (10, 50, 90))
    log(f"[bench] single steps: p10 {p10:.2f} p50 {p50:.2f} p90 {p90:.2f} us")

    # ---- dominant kernel alone, HIP events on the launch stream
    for k in range(max(args.warmup, 50)):
        prefix_only(k)
    _, prefix_us = time_loop(prefix_only, n_side, stream)
    achieved_gbs = fig["prefix_bytes"] / (prefix_us * 1e-6) / 1e9
    achieved_tflops = fig["prefix_flops"] / (prefix_us * 1e-6) / 1e12
    log(f"[bench] prefix_attn_splitk: {prefix_us:.2f} us, {achieved_gbs:.0f} GB/s, "
        f"{achieved_tflops:.0f} TFLOP/s")

    # ---- the other two kernels alone (context for the step time), each warmed up first
    tree_call = hta.prepare_tree_partials(desc, q, kt, vt, par, plen, ws, stream)
    merge_call = hta.prepare_merge(desc, plen, True, out, lse, ws, stream)

    def tree_only(k):
        tree_call()

    def merge_only(k):
        merge_call()

    for k in range(50):
        tree_only(k)
    _, tree_us = time_loop(tree_only, n_side, stream)
    for k in range(50):
        merge_only(k)
    _, merge_us = time_loop(merge_only, n_side, stream)
    log(f"[bench] tree_attn_masked: {tree_us:.2f} us, lse_merge: {merge_us:.2f} us")

    result = {
        "metric": METRIC,
        "value": round(us_per_step, 3),
        "unit": "µs/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": B, "num_q_heads": Hq, "num_kv_heads": w.num_kv_heads, "head_dim": D,
            "prefix_len": int(w.prefix_len.max()), "tree_nodes": T,
            "tree_widths": list(W.LONGSPEC_TREE_WIDTHS), "chunk": info.chunk,
            "splits": info.num_splits, "kv_copies_rotated": n_copies,
        },
        "step": {
            "alg_bytes": fig["step_bytes"], "alg_flops": fig["step_flops"],
            "achieved_GBps": round(fig["step_bytes"] / (us_per_step * 1e-6) / 1e9, 1),
            "roofline_frac": round(max(fig["step_bytes"] / (HBM_PEAK_GBS * 1e9),
                                       fig["step_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                                   / (us_per_step * 1e-6), 4),
            "wall_us": round(us_per_step, 3),
            "events_us": round(step_events_us, 3),
            "settle_steps": settle_calls,
            "timing_note": "value = wall clock over the K timed steps between device "
                           "synchronisations; events_us = HIP events on the launch stream "
                           "around the same K calls (GPU time, without the host's first-launch "
                           "and final-synchronisation latency)",
            "per_call_us": {"p10": round(p10, 3), "p50": round(p50, 3), "p90": round(p90, 3),
                            "calls": n_calls},
            "kernel_us": {"prefix_attn_splitk": round(prefix_us, 3),
                          "tree_attn_masked": round(tree_us, 3),
                          "lse_merge": round(merge_us, 3)},
        },
        "roofline": {
            "kernel": "prefix_attn_splitk",
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(w.name),
            "alg_bytes_per_launch": fig["prefix_bytes"],
            "kernel_us": round(prefix_us, 3),
            "mfma": {"achieved": round(achieved_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        },
    }
    # ---- each chunk's share of every row's attention, from the partials the steps left
    mass = torch.empty(B, Hq, T, info.num_splits + 1, dtype=torch.float32, device=dev)
    scores = torch.empty(B, info.num_splits + 1, dtype=torch.float32, device=dev)
    step(0)
    mass_call = hta.prepare_chunk_mass(desc, plen, lse, mass, scores, ws, stream)
    for _ in range(50):
        mass_call()
    _, mass_us = time_loop(lambda k: mass_call(), n_side, stream)
    log(f"[bench] chunk_mass: {mass_us:.2f} us")
    result["chunk_mass"] = {
        "us": round(mass_us, 3), "columns": info.num_splits + 1,
        "bytes": int((mass.numel() * 2 + lse.numel() * (info.num_splits + 1)) * 4),
    }
    # ---- the method's "before": one masked pass over all L + T keys, explicit mask
    dmask = torch.empty(hta.dense_mask_shape(desc), dtype=torch.int64, device=dev)
    hta.hta_dense_mask(desc, par, plen, dmask, ws, stream)
    dense_steps = max(20, n_side // 5)
    for k in range(20):
        hta.hta_verify_dense(desc, q, kps[k % n_copies], vps[k % n_copies], kt, vt, dmask, plen,
                             out, lse, stream)
    e0.record(stream)
    for k in range(dense_steps):
        hta.hta_verify_dense(desc, q, kps[k % n_copies], vps[k % n_copies], kt, vt, dmask, plen,
                             out, lse, stream)
    e1.record(stream)
    e1.synchronize()
    dense_us = e0.elapsed_time(e1) / dense_steps * 1e3
    e0.record(stream)
    for _ in range(dense_steps):
        hta.hta_dense_mask(desc, par, plen, dmask, ws, stream)
    e1.record(stream)
    e1.synchronize()
    dmask_us = e0.elapsed_time(e1) / dense_steps * 1e3
    log(f"[bench] single-pass masked baseline: {dense_us:.1f} us (+ mask {dmask_us:.1f} us), "
        f"{(dense_us + dmask_us) / step_events_us:.2f}x the hybrid step")
    dense_wgs = (info.rows_padded // 16 + 3) // 4 * w.num_kv_heads * B
    result["dense_masked_baseline"] = {
        "us": round(dense_us, 3), "mask_build_us": round(dmask_us, 3),
        "mask_bytes": int(dmask.numel() * 8), "launches_timed": dense_steps,
        "before_over_after": round((dense_us + dmask_us) / step_events_us, 3),
        "workgroups": dense_wgs, "simds_busy": 4 * dense_wgs, "simds": 1024,
        "note": f"one masked pass over all L+T keys per (64 query rows, KV head), explicit "
                f"mask; before_over_after = (mask build + pass) / the hybrid step (HIP events). "
                f"That pass runs {dense_wgs} workgroups of 4 waves ({4 * dense_wgs} of the "
                f"1024 SIMDs) with no split over the keys, so the ratio also counts the "
                f"parallelism the split-K prefix pass adds",
    }
    result["drafter"] = bench_drafter(w, dev, stream, n_side, kps, vps, n_copies)
    result["around_attention"] = bench_around(w, dev, stream, n_side, args.warmup)
    peaks = measured_peaks(dev)
    log(f"[bench] measured peaks: {peaks}")
    result["measured_peaks"] = peaks
    result["roofline"]["frac_of_measured_peak"] = round(achieved_gbs / peaks["hbm_copy_GBps"], 4)
    # measured matrix-core peak: the register-only product loop at full occupancy (the torch
    # GEMM falls far short of it and is reported beside it only as context)
    loop_peak = peaks["bf16_mfma_loop_TFLOPs"]["8_waves_per_simd"]
    result["roofline"]["mfma"]["frac_of_measured_peak"] = round(achieved_tflops / loop_peak, 4)
    result["roofline"]["mfma"]["measured_peak"] = loop_peak
    result["roofline"]["mfma"]["frac_of_gemm"] = round(achieved_tflops / peaks["bf16_gemm_TFLOPs"], 4)
    # ---- the other configurations, each timed like the headline
    del kps, vps
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = {"llama3_8b_32k": roofline_figures(fig, us_per_step, prefix_us)}
        result["configs"]["llama3_8b_32k"]["events_us"] = round(step_events_us, 3)
        for name in OTHER_CONFIGS:
            result["configs"][name] = bench_config(name, dev, stream)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
