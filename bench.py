#!/usr/bin/env python3
"""Benchmark of the paged-KV attention step on one MI355X.

One step = the whole hot path on synthetic inputs already resident in HBM:

* the decode step of a Qwen3-8B-shaped layer (32 q / 8 kv heads, head_dim 128,
  bf16, batch 256, lognormal context lengths, page_size 1 by default) as one
  replay of the captured HIP graph: store_kv of the 256 new tokens, then
  split-K decode attention (and its merge);
* the same step at the other page size (16 by default: same lengths and
  logical K/V, shuffled pages);
* the decode step of a Qwen3-0.6B-shaped layer (16 q / 8 kv heads, batch 64,
  contexts U[512, 4096]), captured the same way;
* a ragged causal prefill/extend step (Qwen3-0.6B heads, 8 requests, extend
  U[128, 2048] on a cached prefix U[0, 1024]): store_kv, then MFMA prefill
  attention.

``value`` is the first decode leg's achieved HBM bandwidth (algorithmic bytes
/ leg time); the line carries the other decode legs' figures (and the captured
steps of both page sizes replayed one at a time after a cache flush),
req-tokens/s of the decode leg and the prefill
leg's TFLOP/s, a roofline object for the dominant kernel (decode attention,
timed with HIP events on its own stream) and the fp64 CPU oracle timed on the
same decode workload as a reported baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# template arguments of the Qwen3-8B-shaped decode kernels in profiler kernel names
# (element type, head_dim 128, 4 q heads per kv head)
QWEN3_8B_DECODE = ", 128, 4"
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_DIR = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILE_DIR, "decode_attn_qwen3_8b_bs256_traffic.txt")
# sources that define the decode attention kernels (a counter summary is only
# valid for the sources it was taken on)
DECODE_SOURCES = ("paged_kv_attention_slots_amd/csrc/decode.hip",
                  "paged_kv_attention_slots_amd/csrc/attend_valu.h",
                  "paged_kv_attention_slots_amd/csrc/common.h",
                  "paged_kv_attention_slots_amd/csrc/launch.h")


def decode_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode-attention launch from the committed counter summary,
    or None when it is missing or was taken on other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_hash") != decode_source_hash():
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(w) -> int:
    """Algorithmic HBM bytes of one decode-attention launch: every visible
    token's K and V slice once per kv head, q in, out written, one 4-byte
    page-table id per visible token."""
    e = w.dtype.itemsize
    L = int(w.seq_lens.long().sum())
    kv = L * w.kv_heads * w.head_dim * 2 * e
    qo = 2 * w.bs * w.q_heads * w.head_dim * e
    return kv + qo + 4 * L


def store_bytes(w) -> int:
    e = w.dtype.itemsize
    return 2 * 2 * w.num_tokens * w.kv_heads * w.head_dim * e + 4 * w.num_tokens


def rope_store_bytes(w) -> int:
    """Algorithmic HBM bytes of one fused RoPE + KV write: q and k read and
    written once each, v read and written once, a position and a slot id per
    token."""
    e = w.dtype.itemsize
    return 2 * w.num_tokens * (w.q_heads + 2 * w.kv_heads) * w.head_dim * e + 8 * w.num_tokens


ROPE_BASE = 1e6  # Qwen3's rotary base
PREFILL_WARM_LAUNCHES = 400  # ~40 ms of the ragged prefill kernel before it is timed alone
KERNEL_ITERS = 20  # default number of eager decode-attention launches timed for the roofline
SETTLE_STEPS = 60  # untimed full steps before the warm-up steps (~45 ms of GPU work)


def prefill_flops(w) -> float:
    """Matrix flops of the unmasked (query, key) pairs: 2 matmuls x 2 flop x d per pair and head."""
    ext = (w.seq_lens - w.cached_lens).double()
    C = w.cached_lens.double()
    pairs = float((ext * C + ext * (ext + 1) / 2).sum())
    return 4.0 * w.head_dim * w.q_heads * pairs


def _read_csv(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirname}")


def summarize_profiles(stats_dir, fetch_dir, write_dir, command, workload_bytes, rope_bytes=None):
    """Write the committed text summaries from rocprofv3 output directories:
    the kernel-trace statistics of the bench command, and the decode kernels'
    HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs, scaled by what the
    same counters read for the plain copy kernel (torch.neg over a known size)."""
    stats = _read_csv(_find(stats_dir, "kernel_stats.csv"))
    os.makedirs(PROFILE_DIR, exist_ok=True)
    lines = ["# rocprofv3 --kernel-trace --stats summary of the benchmark command",
             f"# command: rocprofv3 --kernel-trace --stats --output-format csv -- {command}",
             "# workload: Qwen3-8B decode bs 256 as captured steps at page sizes 1 and 16, the Qwen3-0.6B",
             "#           decode bs 64 captured step, ragged prefill 8 requests (Qwen3-0.6B heads), eager",
             "#           decode-attention launches (bs 256, page size 1), then the fused RoPE, vocabulary",
             "#           indexing and shared-prefix legs; durations in microseconds", ""]
    head = f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel"
    mine = [r for r in stats if "msgl::" in r["Name"]]
    other = [r for r in stats if "msgl::" not in r["Name"]]

    def row(r):
        name = r["Name"].replace('"', "")
        return (f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}  {name[:110]}")

    # per leg, from the trace: the decode / prefill step legs come before the
    # first fused-RoPE launch; the RoPE, vocabulary and shared-prefix legs after
    trace = _read_csv(_find(stats_dir, "kernel_trace.csv"))
    cut = min([int(r["Dispatch_Id"]) for r in trace if "rope_store_kv_kernel" in r["Kernel_Name"]] or [1 << 62])

    def legs(before):
        per = {}
        for r in trace:
            if "msgl::" in r["Kernel_Name"] and (int(r["Dispatch_Id"]) < cut) == before:
                per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out = []
        for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{len(d):6d} {sum(d) / len(d):10.2f} {min(d):10.2f} {max(d):10.2f} {'':>8}  {name[:110]}")
        return out
    lines += ["## library kernels, whole run", head] + [row(r) for r in mine]
    lines += ["", "## the step's legs (decode graph replays at bs 256 ps1 and ps16 and at bs 64, the ragged prefill),",
              "## then the eager launches the bench times alone (decode attention, prefill attention)",
              head] + legs(True)
    # the roofline's kernel: the eager decode-attention launches the bench line times (the
    # last KERNEL_ITERS split + merge pairs before the cut) against its HIP-event average
    def eager(kind):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
             if kind in r["Kernel_Name"] and QWEN3_8B_DECODE in r["Kernel_Name"] and int(r["Dispatch_Id"]) < cut]
        return d[-KERNEL_ITERS:]
    sp, mg = eager("decode_split_kernel"), eager("decode_merge_kernel")
    if sp and mg:
        lines += ["", f"## the roofline's kernel: the {len(sp)} eager decode-attention launches the bench line times",
                  f"split {sum(sp) / len(sp):.2f} us + merge {sum(mg) / len(mg):.2f} us = "
                  f"{sum(sp) / len(sp) + sum(mg) / len(mg):.2f} us per launch"]
    lines += ["", "## after them: fused RoPE (decode and prefill batches), vocabulary indexing (4288 and 256 tokens),",
              "## shared-prefix batch (cascade call: prefix MFMA pass, suffix decode, merge; then plain decode)",
              head] + legs(False)
    lines += ["", "## largest other kernels (seeded input generation, torch copies)", head]
    lines += [row(r) for r in other[:6]]
    with open(os.path.join(PROFILE_DIR, "step_qwen3_8b_decode_bs256_ragged_prefill_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_dispatch(dirname, counter):
        # only the dispatches before the first fused-RoPE launch: the decode
        # kernels after it belong to the shared-prefix leg's batch
        rows = _read_csv(_find(dirname, "counter_collection.csv"))
        cut = min([int(r["Dispatch_Id"]) for r in rows if "rope_store_kv_kernel" in r["Kernel_Name"]] or [1 << 62])
        out = {}
        for r in rows:
            if r["Counter_Name"] != counter or ("neg_kernel" not in r["Kernel_Name"] and int(r["Dispatch_Id"]) > cut):
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)  # KiB -> B
        return out

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")

    def one(d, key, shape=""):
        names = [n for n in d if key in n and shape in n]
        if not names:
            raise KeyError(key)
        vals = d[names[0]]
        return sum(vals) / len(vals), len(vals)

    def copies(d):
        # the calibration copies: 3 of 1 GiB, then 3 of a quarter of that (see --copy-calibration-gib)
        names = [n for n in d if "neg_kernel" in n]
        vals = sorted(v for n in names for v in d[n])
        if len(vals) < 6:
            raise KeyError("calibration copies")
        return sum(vals[-3:]) / 3, sum(vals[:3]) / 3

    cal = float(1 << 30)  # the bench negates 1 GiB (--copy-calibration-gib 1): 1 GiB read, 1 GiB written
    (neg_f, neg_f4), (neg_w, neg_w4) = copies(fetch), copies(write)
    f_scale, w_scale = cal / neg_f, cal / neg_w
    f_scale4, w_scale4 = cal / 4 / neg_f4, cal / 4 / neg_w4
    split_f, n_split = one(fetch, "decode_split_kernel", QWEN3_8B_DECODE)
    split_w, _ = one(write, "decode_split_kernel", QWEN3_8B_DECODE)
    merge_f, _ = one(fetch, "decode_merge_kernel", QWEN3_8B_DECODE)
    merge_w, _ = one(write, "decode_merge_kernel", QWEN3_8B_DECODE)
    traffic = (split_f + merge_f) * f_scale + (split_w + merge_w) * w_scale
    lines = [
        "# HBM traffic of one decode-attention launch (split + merge kernels), Qwen3-8B shape, bs 256",
        f"# command (three runs): rocprofv3 --kernel-trace --stats | --pmc FETCH_SIZE | --pmc WRITE_SIZE "
        f"-- {command}",
        "# counters are per dispatch (KiB), averaged over the launches of the Qwen3-8B kernels (graph",
        "# replays at page sizes 1 and 16 and the eager launches, all before the bench's fused-RoPE leg);",
        "# each is scaled by (known bytes / counter reading) of a plain copy kernel: torch.neg over 1 GiB",
        "# of fp32; the same copy over a quarter of that gives the second pair of factors (a check)",
        f"copy_fetch_scale = {f_scale:.4f}",
        f"copy_write_scale = {w_scale:.4f}",
        f"copy_fetch_scale_quarter_size = {f_scale4:.4f}",
        f"copy_write_scale_quarter_size = {w_scale4:.4f}",
        f"split_fetch_bytes = {split_f:.0f}",
        f"split_write_bytes = {split_w:.0f}",
        f"merge_fetch_bytes = {merge_f:.0f}",
        f"merge_write_bytes = {merge_w:.0f}",
        f"dispatches_averaged = {n_split}",
        f"algorithmic_bytes_per_launch = {workload_bytes}",
        f"traffic_bytes_per_launch = {traffic:.0f}",
        f"traffic_over_algorithmic = {traffic / workload_bytes:.4f}",
        f"source_hash = {decode_source_hash()}",
    ]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if rope_bytes:
        summarize_rope_traffic(fetch_dir, write_dir, command, f_scale, w_scale, rope_bytes)


def summarize_rope_traffic(fetch_dir, write_dir, command, f_scale, w_scale, rope_bytes):
    """HBM bytes per launch of the fused RoPE + KV-write kernel, per batch (the
    bench launches it on the decode batch and on the prefill batch; the
    dispatches are told apart by their grid size, smaller grid first)."""
    def groups(dirname, counter):
        out = {}
        for r in _read_csv(_find(dirname, "counter_collection.csv")):
            if r["Counter_Name"] == counter and "rope_store_kv_kernel" in r["Kernel_Name"]:
                out.setdefault(int(r["Grid_Size"]), []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    fetch, write = groups(fetch_dir, "FETCH_SIZE"), groups(write_dir, "WRITE_SIZE")
    lines = ["# HBM traffic of one fused RoPE + KV-write launch (rope_store_kv_kernel), per batch",
             f"# command (two runs): rocprofv3 --pmc FETCH_SIZE | --pmc WRITE_SIZE -- {command}",
             "# counters per dispatch (KiB -> bytes), averaged, scaled by the plain-copy factors below",
             f"copy_fetch_scale = {f_scale:.4f}", f"copy_write_scale = {w_scale:.4f}"]
    for (tag, algo), grid in zip(sorted(rope_bytes.items(), key=lambda kv: kv[1]), sorted(fetch)):
        fb = sum(fetch[grid]) / len(fetch[grid]) * f_scale
        wb = sum(write.get(grid, [0.0])) / max(1, len(write.get(grid, []))) * w_scale
        lines += [f"{tag}.grid_threads = {grid}", f"{tag}.dispatches_averaged = {len(fetch[grid])}",
                  f"{tag}.fetch_bytes = {fb:.0f}", f"{tag}.write_bytes = {wb:.0f}",
                  f"{tag}.algorithmic_bytes_per_launch = {algo}",
                  f"{tag}.traffic_over_algorithmic = {(fb + wb) / algo:.4f}"]
    with open(os.path.join(PROFILE_DIR, "rope_store_kv_qwen3_traffic.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _time_stream(fn, stream, iters, warm=3):
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def shared_prefix_leg(iters: int, stream) -> dict:
    """Cascade decode (msgl_decode_attn_shared_prefix) and plain decode attention
    on one decode batch whose requests share radix prefixes.  Unique bytes count
    each shared prefix's K/V rows once per group, everything else as decode."""
    import torch

    from paged_kv_attention_slots_amd import _lib, runner, workloads as wl

    sp = wl.shared_prefix_decode(device=stream.device)
    w = sp.w
    out = torch.empty_like(w.q)
    lse = torch.empty(w.bs, w.q_heads, dtype=torch.float32, device=w.q.device)
    ws = _lib.shared_prefix_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len, device=w.q.device)
    ws_d = _lib.decode_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len, device=w.q.device)

    def cascade():
        _lib.msgl_decode_attn_shared_prefix(out, lse, w.q, w.k_pool, w.v_pool, w.page_table, w.table_idx,
                                            w.seq_lens, sp.group_start, sp.prefix_lens, sp.max_group_size,
                                            sp.max_prefix_len, w.max_seq_len, ws, page_size=w.page_size,
                                            stream=stream)

    def plain():
        runner.decode_attn(w, w.k_pool, w.v_pool, out=out, lse=lse, workspace=ws_d, stream=stream)

    c_ms = _time_stream(cascade, stream, iters)
    p_ms = _time_stream(plain, stream, iters)
    e = w.dtype.itemsize
    row = w.kv_heads * w.head_dim * 2 * e  # K and V of one token
    gs = sp.group_start.cpu().tolist()
    shared_tok = sum(int(sp.prefix_lens[gs[g]]) for g in range(len(gs) - 1))
    own_tok = int((w.seq_lens - sp.prefix_lens).long().sum())
    qo = 2 * w.bs * w.q_heads * w.head_dim * e
    unique = (shared_tok + own_tok) * (row + 4) + qo
    plain_bytes = decode_bytes(w)
    return {"batch": w.bs, "groups": len(gs) - 1, "shared_prefix_tokens": shared_tok,
            "context_tokens": int(w.seq_lens.sum()), "cascade_ms": round(c_ms, 4), "plain_decode_ms": round(p_ms, 4),
            "speedup": round(p_ms / c_ms, 2), "cascade_unique_GBs": round(unique / (c_ms * 1e-3) / 1e9, 1),
            "cascade_frac_hbm": round(unique / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "plain_GBs": round(plain_bytes / (p_ms * 1e-3) / 1e9, 1), "unique_bytes": unique,
            "plain_bytes": plain_bytes}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def prefill_cpu_baseline(oracle, w, threads: int) -> dict:
    """The fp64 oracle on a bounded sample of the ragged prefill batch: every
    4th query row, each as a one-query request at its own position (same
    page-table row and keys), on all host threads, passes repeated to ~4 s;
    then every 32nd row on one thread (~2 s).  TFLOP/s of the same
    algorithmic flops (4 d H per visible key)."""
    import numpy as np
    import torch

    kp, vp = oracle.store_kv(w.k_pool.cpu(), w.v_pool.cpu(), w.k_new, w.v_new, w.out_loc)
    cu = w.cu_q.cpu().numpy()
    C = w.cached_lens.cpu().numpy()
    tix_all = w.table_idx.cpu().numpy()
    q_all = w.q.cpu()
    pt = w.page_table.cpu()

    def run(step: int, n_threads: int, min_seconds: float):
        rows = np.arange(0, w.num_tokens, step)
        b = np.searchsorted(cu, rows, side="right") - 1
        pos = C[b] + (rows - cu[b])
        tix = torch.from_numpy(tix_all[b].astype(np.int32))
        seq = torch.from_numpy((pos + 1).astype(np.int32))
        qs = torch.arange(len(rows) + 1, dtype=torch.int32)
        q = q_all[torch.from_numpy(rows)]
        oracle.set_threads(n_threads)
        reps, t0 = 0, time.perf_counter()
        while True:  # repeat the pass until min_seconds of CPU time
            oracle.attention(q, kp, vp, pt, tix, seq, qs)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
        flops = 4.0 * w.head_dim * w.q_heads * float((pos + 1).sum())
        return len(rows), el / reps, flops * reps / el / 1e12

    n_all, s_all, tf_all = run(4, threads, 4.0)
    n_one, s_one, tf_one = run(32, 1, 2.0)
    oracle.set_threads(threads)
    return {"value": round(tf_all, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 C oracle, ragged prefill attention of every 4th query row ({n_all} of "
                      f"{w.num_tokens}), {s_all:.2f} s per pass on {threads} OpenMP threads",
            "one_thread": {"value": round(tf_one, 6), "unit": "TFLOP/s",
                           "sample": f"every 32nd query row ({n_one}), {s_one:.2f} s per pass on 1 thread"}}


def oracle_pass_time(oracle, w, n_threads: int, min_seconds: float, max_seconds: float) -> tuple:
    """Seconds per pass of the oracle's attention over workload ``w`` (host
    copies, store_kv applied first, outside the clock), repeated until
    ``min_seconds`` (or before passing ``max_seconds``); and the pass count."""
    kp, vp = oracle.store_kv(w.k_pool.cpu(), w.v_pool.cpu(), w.k_new.cpu(), w.v_new.cpu(), w.out_loc.cpu())
    args_h = (w.q.cpu(), kp, vp, w.page_table.cpu(), w.table_idx.cpu(), w.seq_lens.cpu(), w.cu_q.cpu())
    return oracle_pass_time_h(oracle, args_h, n_threads, min_seconds, max_seconds)


def oracle_pass_time_h(oracle, args_h, n_threads: int, min_seconds: float, max_seconds: float) -> tuple:
    """The same on host arguments already prepared (q, pools, page table, table_idx, seq_lens, cu_q)."""
    prev = oracle.num_threads()
    oracle.set_threads(n_threads)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(*args_h)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el * (reps + 1) / reps > max_seconds:
            break
    oracle.set_threads(prev)
    return el / reps, reps


def small_config_cpu_baselines(oracle, w2, threads: int) -> dict:
    """The oracle on the small configurations, whole: Qwen3-0.6B decode at
    bs 64 on all threads and on one, and the tiny fp32 decode and prefill on one
    thread (GB/s of algorithmic bytes for decode, TFLOP/s for prefill)."""
    from paged_kv_attention_slots_amd import workloads as wl

    out = {}
    sb = decode_bytes(w2)
    for tag, n in (("all_threads", threads), ("one_thread", 1)):
        s, reps = oracle_pass_time(oracle, w2, n, 2.0, 6.0)
        out[f"qwen3_06b_decode_bs64_{tag}"] = {
            "value": round(sb / s / 1e9, 4), "unit": "GB/s", "threads": n,
            "sample": f"the whole batch ({int(w2.seq_lens.sum())} context tokens), {reps} passes, {s:.3f} s each"}
    t1d = wl.tiny("decode")
    s, reps = oracle_pass_time(oracle, t1d, 1, 0.5, 2.0)
    out["tiny_fp32_decode_one_thread"] = {"value": round(decode_bytes(t1d) / s / 1e9, 4), "unit": "GB/s",
                                          "threads": 1, "sample": f"both requests, {reps} passes, {s * 1e6:.1f} us each"}
    t1p = wl.tiny("prefill")
    ext = (t1p.seq_lens - t1p.cached_lens).double()
    fl = 4.0 * t1p.head_dim * t1p.q_heads * float((ext * t1p.cached_lens.double() + ext * (ext + 1) / 2).sum())
    s, reps = oracle_pass_time(oracle, t1p, 1, 0.5, 2.0)
    out["tiny_fp32_prefill_one_thread"] = {"value": round(fl / s / 1e12, 8), "unit": "TFLOP/s", "threads": 1,
                                           "sample": f"both requests ({t1p.num_tokens} query rows), {reps} passes, "
                                                     f"{s * 1e6:.1f} us each"}
    return out


def flushed_timing(fn, stream, iters: int, flush_bytes: int = 1 << 30, warm: int = 10,
                   read_bytes: int = 1 << 29) -> dict:
    """Per-launch times of ``fn``, each after a cache flush outside the events:
    a write of ``flush_bytes`` to a scratch buffer, then a read of
    ``read_bytes`` from another, so that the last-level cache (256 MB) holds
    none of the kernel's inputs and no dirty lines.  A flush by writes alone
    leaves up to a cache's worth of dirty lines, whose write-back then lands
    inside the timed launch; that variant is timed too and reported under
    ``write_only``.  Median, p10 and p90 in ms."""
    import torch

    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device=stream.device)
    clean = torch.ones(read_bytes // 4, dtype=torch.float32, device=stream.device)
    sink = torch.empty((), dtype=torch.float32, device=stream.device)
    torch.cuda.synchronize()
    for _ in range(warm):
        fn()

    def run(read_after: bool) -> list:
        times = []
        for _ in range(iters):
            with torch.cuda.stream(stream):
                scratch.fill_(1.0)
                if read_after:
                    torch.sum(clean, dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        return times

    times = run(True)
    times_w = run(False)
    del scratch, clean, sink
    q = lambda t, f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]
    return {"median_ms": round(q(times, 0.5), 4), "p10_ms": round(q(times, 0.1), 4), "p90_ms": round(q(times, 0.9), 4),
            "iters": iters, "flush_bytes": flush_bytes,
            "flush": f"write {flush_bytes >> 20} MiB, then read {read_bytes >> 20} MiB of another buffer",
            "write_only": {"median_ms": round(q(times_w, 0.5), 4), "p10_ms": round(q(times_w, 0.1), 4),
                           "p90_ms": round(q(times_w, 0.9), 4)}}


def sweep(iters: int) -> int:
    """Secondary measurements (one JSON line each): the captured decode step at
    every padded batch size for page sizes 1 and 16, padding runs, eager
    decode attention, and prefill on the ragged and chunked shapes."""
    import torch

    from paged_kv_attention_slots_amd import _lib, runner, workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    for ps in (1, 16):
        full = wl.qwen3_8b_decode(page_size=ps, device=dev)
        if ps == 1:  # the clocks settle after some tens of ms of sustained work: warm up before the first timing
            wout = torch.empty_like(full.q)
            wws = _lib.decode_workspace(full.bs, full.q_heads, full.head_dim, full.max_seq_len, device=dev)
            for _ in range(100):
                runner.decode_attn(full, full.k_pool, full.v_pool, out=wout, workspace=wws, with_lse=False,
                                   stream=stream)
            torch.cuda.synchronize()
            del wout, wws
            # the first graph a process creates and replays runs slow for a while: one untimed graph first
            w = wl.pad_decode(wl.subset_decode(full, 1), 1)
            out = torch.empty_like(w.q)
            ws = _lib.decode_workspace(1, w.q_heads, w.head_dim, w.max_seq_len, device=dev)
            torch.cuda.synchronize()
            g = _lib.msgl_decode_graph_create(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc, out, None, w.q,
                                              w.page_table, w.table_idx, w.seq_lens, w.max_seq_len, ws,
                                              page_size=ps, stream=stream)
            _time_stream(lambda: g.launch(stream), stream, 200)
            g.destroy()
        runs = [(n, n) for n in wl.GRAPH_BATCH_SIZES] + [(3, 4), (100, 128), (200, 256)]
        for real, padded in runs:
            w = wl.pad_decode(wl.subset_decode(full, real), padded)
            out = torch.empty_like(w.q)
            lse = torch.empty(padded, w.q_heads, dtype=torch.float32, device=dev)
            ws = _lib.decode_workspace(padded, w.q_heads, w.head_dim, w.max_seq_len, device=dev)
            torch.cuda.synchronize()
            g = _lib.msgl_decode_graph_create(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc, out, lse, w.q,
                                              w.page_table, w.table_idx, w.seq_lens, w.max_seq_len, ws,
                                              page_size=ps, stream=stream)
            ms = _time_stream(lambda: g.launch(stream), stream, iters)
            g.destroy()
            real_w = wl.subset_decode(full, real)
            byts = decode_bytes(real_w) + store_bytes(real_w)
            print(json.dumps({"sweep": "decode_graph_step", "page_size": ps, "batch": real, "padded": padded,
                              "ms": round(ms, 4), "GBs": round(byts / ms / 1e6, 1),
                              "frac_hbm": round(byts / ms / 1e6 / HBM_PEAK_GBS, 4),
                              "req_tokens_per_s": round(real / ms * 1e3, 1),
                              "context_tokens": int(real_w.seq_lens.sum())}), flush=True)
        out = torch.empty_like(full.q)
        ws = _lib.decode_workspace(full.bs, full.q_heads, full.head_dim, full.max_seq_len, device=dev)
        ms = _time_stream(lambda: runner.decode_attn(full, full.k_pool, full.v_pool, out=out, workspace=ws,
                                                     with_lse=False, stream=stream), stream, iters)
        byts = decode_bytes(full)
        print(json.dumps({"sweep": "decode_attn_eager", "page_size": ps, "batch": full.bs, "ms": round(ms, 4),
                          "GBs": round(byts / ms / 1e6, 1), "frac_hbm": round(byts / ms / 1e6 / HBM_PEAK_GBS, 4)}),
              flush=True)
        del full
        torch.cuda.empty_cache()
    cases = [("ragged_prefill_8req", wl.ragged_prefill(device=dev)),
             ("chunked_prefill_2x2048_on_8192", wl.ragged_prefill(
                 device=dev, n_req=2, e_lo=2048, e_hi=2048, c_lo=8192, c_hi=8192, num_slots=1 << 15,
                 heads=wl.QWEN3_8B, seed=1005))]
    for name, w in cases:
        runner.store_kv(w, w.k_pool, w.v_pool)  # the new tokens' K/V in the pools, as in the step
        out = torch.empty_like(w.q)
        ms = _time_stream(lambda: runner.prefill_attn(w, w.k_pool, w.v_pool, out=out, with_lse=False,
                                                      stream=stream), stream, iters, warm=PREFILL_WARM_LAUNCHES)
        fl = prefill_flops(w)
        print(json.dumps({"sweep": "prefill_attn", "case": name, "tokens": w.num_tokens,
                          "context_tokens": int(w.seq_lens.sum()), "ms": round(ms, 4),
                          "TFLOPs": round(fl / ms / 1e9, 1),
                          "frac_bf16_peak": round(fl / ms / 1e9 / BF16_DENSE_PEAK_TFLOPS, 4)}), flush=True)
    return 0


def mixed(iters: int) -> int:
    """The mixed step alone (`--mixed N`): one JSON line."""
    import torch

    stream = torch.cuda.Stream(device=torch.device("cuda:0"))
    print(json.dumps(mixed_leg(iters, stream)), flush=True)
    return 0


def mixed_leg(iters: int, stream) -> dict:
    """The mixed multi-layer step (36 layers, 192 decode requests + 2 chunked
    prefills of 2048 on 8192-token prefixes, pool 60% of 288 GB), eager, per
    layer store_kv -> decode -> prefill, timed over `iters` steps after 4
    warm-up steps.  Returns its record; the pools are freed on return."""
    import torch

    from paged_kv_attention_slots_amd import _lib, workloads as wl

    dev = stream.device
    t0 = time.time()
    log("building the mixed step (36 layers, pool 60% of 288 GB)")
    m = wl.mixed_step(device=dev)
    torch.cuda.synchronize()
    log(f"  built in {time.time() - t0:.1f}s")
    d0, p0 = m.layer_views(0)
    od = torch.empty_like(d0.q)
    op = torch.empty_like(p0.q)
    ws = _lib.decode_workspace(d0.bs, d0.q_heads, d0.head_dim, d0.max_seq_len, device=dev)
    max_ext = int((p0.seq_lens - p0.cached_lens).max())
    views = [m.layer_views(layer) for layer in range(m.layers)]

    def step():
        for d, p in views:
            _lib.msgl_store_kv(d.k_pool, d.v_pool, m.k_new[d.layer], m.v_new[d.layer], m.out_loc, stream=stream)
            _lib.msgl_decode_attn(od, None, d.q, d.k_pool, d.v_pool, d.page_table, d.table_idx, d.seq_lens,
                                  d.max_seq_len, ws, stream=stream)
            _lib.msgl_prefill_attn(op, None, p.q, p.k_pool, p.v_pool, p.page_table, p.table_idx, p.seq_lens,
                                   p.cached_lens, p.cu_q, max_ext, stream=stream)

    ms = _time_stream(step, stream, iters, warm=4)  # past the start-up transient of matrix work
    dbytes = decode_bytes(d0) * m.layers
    sbytes = (2 * 2 * m.num_tokens * d0.kv_heads * d0.head_dim * 2 + 4 * m.num_tokens) * m.layers
    flops = prefill_flops(p0) * m.layers
    roof_ms = ((dbytes + sbytes) / (HBM_PEAK_GBS * 1e9) + flops / (BF16_DENSE_PEAK_TFLOPS * 1e12)) * 1e3
    rec = {"mixed_step": "qwen3-8b 36 layers: 192 decode + 2x2048 prefill on 8192 prefix",
           "ms_per_step": round(ms, 3), "steps": iters, "tokens_per_step": m.num_tokens,
           "tokens_per_s": round(m.num_tokens / ms * 1e3, 1),
           "roofline_ms": round(roof_ms, 3), "frac_of_roofline": round(roof_ms / ms, 4),
           "decode_bytes": dbytes, "store_bytes": sbytes, "prefill_flops": flops,
           "slots_per_layer": d0.num_slots, "decode_context_tokens": int(d0.seq_lens.sum())}
    del views, d0, p0, od, op, ws, m
    torch.cuda.empty_cache()
    return rec


def prefill_profile(iters: int, zero_new: bool = False) -> int:
    """Only the ragged prefill attention (8 requests, Qwen3-0.6B heads),
    launched back to back: the command the prefill counter profiles run.  The
    new tokens' K/V are written into the pools first, as in the step: with
    their slots still zero the kernel runs several percent faster (the matrix
    cores draw less power on zero operands and the clocks stay higher)."""
    import torch
    from paged_kv_attention_slots_amd import _lib, runner, workloads as wl

    dev = torch.device("cuda:0")
    w = wl.ragged_prefill(device=dev)
    if not zero_new:  # --zero-new: leave the new tokens' slots zero (to show the effect above)
        runner.store_kv(w, w.k_pool, w.v_pool)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.num_tokens, w.q_heads, dtype=torch.float32, device=dev)
    me = int((w.seq_lens - w.cached_lens).max())
    stream = torch.cuda.Stream(device=dev)

    def call():
        _lib.msgl_prefill_attn(out, lse, w.q, w.k_pool, w.v_pool, w.page_table, w.table_idx, w.seq_lens,
                               w.cached_lens, w.cu_q, me, page_size=w.page_size, sm_scale=w.sm_scale,
                               stream=stream)

    ms = _time_stream(call, stream, iters, warm=PREFILL_WARM_LAUNCHES)
    print(json.dumps({"prefill_profile": "ragged prefill 8 req", "new_token_slots": "zero" if zero_new else "stored",
                      "launches": iters + PREFILL_WARM_LAUNCHES,
                      "timed_launches": iters, "ms": round(ms, 4),
                      "tflops": round(prefill_flops(w) / (ms * 1e-3) / 1e12, 2)}), flush=True)
    return 0


def ceilings(iters: int) -> int:
    """Measured ceilings beside the vendor peaks: a large bf16 GEMM through the
    vendor BLAS (torch.matmul, 2-D contiguous operands) and a plain device copy
    (read once, write once).  One JSON line each."""
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    for n in (8192, 16384):
        a = torch.randn(n, n, device=dev).to(torch.bfloat16)
        b = torch.randn(n, n, device=dev).to(torch.bfloat16)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        with torch.cuda.stream(stream):
            ms = _time_stream(lambda: torch.matmul(a, b, out=c), stream, iters, warm=20)
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"ceiling": "bf16 gemm (torch.matmul)", "m=n=k": n, "ms": round(ms, 4),
                          "TFLOPs": round(tf, 1), "frac_bf16_peak": round(tf / BF16_DENSE_PEAK_TFLOPS, 4)}),
              flush=True)
        del a, b, c
    n = (2 << 30) // 4
    x = torch.ones(n, device=dev)
    y = torch.empty_like(x)
    with torch.cuda.stream(stream):
        ms = _time_stream(lambda: y.copy_(x), stream, iters, warm=5)
    gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    print(json.dumps({"ceiling": "device copy (torch copy_, 2 GiB read + 2 GiB written)", "ms": round(ms, 4),
                      "GBs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
    del x, y
    read_ceilings(iters, stream)
    mfma_ceilings(stream)
    return 0


def mfma_ceilings(stream) -> None:
    """Matrix-core ceilings of the prefill kernel's inner loop, from the probe
    kernel in csrc/probes/mfma_ceilings.hip: 16 bf16 MFMAs (32x32x16) per 32 keys
    per 32 query columns, with operands from registers, with the kernel's LDS
    operand reads, and with those plus a softmax-like vector load; 32 or 64
    columns per wave.  Run on random N(0,1) bf16 data and on zeros: the clock the
    loop holds (shader cycles over the 100 MHz constant clock, mean over blocks)
    depends on the data.  mfma_busy = MFMA cycles (32 per instruction, from the
    dense peak) over elapsed cycles per SIMD.  One JSON line each."""
    import ctypes

    import torch

    from paged_kv_attention_slots_amd import build as _build

    lib = ctypes.CDLL(_build.PROBES_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.msglp_mfma_loop.argtypes = [I, I, P, I, I, P, P, P]
    dev = stream.device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    gen = torch.Generator(device="cpu")
    gen.manual_seed(5)
    data = {"random": torch.randn(16384, generator=gen).to(torch.bfloat16).to(dev),
            "zero": torch.zeros(16384, dtype=torch.bfloat16, device=dev)}
    units = 2000
    names = {0: "MFMA only (operands in registers)", 1: "MFMA + LDS operand reads",
             2: "MFMA + LDS operand reads + softmax-like VALU", 3: "MFMA only, 16x16x32 (operands in registers)"}
    for dname, src in data.items():
        for wide, v in ((0, 3), (0, 0), (0, 1), (0, 2), (1, 1), (1, 2)):
            nc = 2 if wide else 1
            waves = 4 * nc
            blocks = (4 if nc == 1 else 2) * cus
            sink = torch.zeros(blocks * 64 * waves, device=dev)
            clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
            call = lambda: lib.msglp_mfma_loop(v, wide, src.data_ptr(), blocks, units, sink.data_ptr(),
                                               clk.data_ptr(), stream.cuda_stream)
            assert call() == 0
            ms = _time_stream(call, stream, 3, warm=1)
            c = clk.view(-1, 2).double().cpu()
            ghz = float((c[:, 0] / (c[:, 1] / 100e6)).mean()) / 1e9
            mfmas = blocks * waves * units * 16 * nc
            tf = mfmas * 32768 / (ms * 1e-3) / 1e12
            busy = mfmas * 32 / (4 * cus) / (ms * 1e-3 * ghz * 1e9)
            print(json.dumps({"ceiling": names[v], "query_columns_per_wave": 32 * nc, "data": dname,
                              "ms": round(ms, 4), "TFLOPs": round(tf, 1),
                              "frac_bf16_peak": round(tf / BF16_DENSE_PEAK_TFLOPS, 4),
                              "clock_GHz": round(ghz, 3), "mfma_busy": round(busy, 3)}), flush=True)


def read_ceilings(iters: int, stream) -> None:
    """Read ceilings of the decode kernel's access patterns, from the probe
    kernels in csrc/probes (libmsgl_probes.so): a sequential stream of 16-byte
    loads over 4 GiB, and a 4 GiB pool of 2 KB rows (8 kv heads x 128 bf16)
    read as 256-byte per-head slices of rows in random order (page size 1) and
    of random 16-row pages (page size 16).  Each is the best over a few grid
    sizes (and, for the gathers, 4 or 8 loads in flight per lane); one JSON line
    each."""
    import ctypes

    import torch

    from paged_kv_attention_slots_amd import build as _build

    lib = ctypes.CDLL(_build.PROBES_PATH)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.msglp_stream_read.argtypes = [P, I64, P, I, P]
    lib.msglp_gather_heads.argtypes = [P, P, I, I, I, P, I, I, P]
    dev = stream.device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    heads, row_bytes = 8, 8 * 256
    rows = nbytes // row_bytes
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    row_ids = torch.randperm(rows, generator=gen, device=dev).to(torch.int32)
    page_ids = torch.randperm(rows // 16, generator=gen, device=dev).to(torch.int32)
    assert int(row_ids.max()) < rows and int(page_ids.max()) < rows // 16
    s = stream.cuda_stream

    def best(call, grids):
        out = []
        for g in grids:
            assert call(g) == 0
            out.append((_time_stream(lambda: call(g), stream, iters, warm=3), g))
        return min(out)

    for name, call, grids in (
            ("sequential read, 16-byte nontemporal loads, 4 GiB",
             lambda g: lib.msglp_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), g, s), (cus, 2 * cus, 4 * cus)),
            ("random 2 KB rows read as 256-byte head slices (page size 1), 4 GiB pool",
             lambda g: lib.msglp_gather_heads(buf.data_ptr(), row_ids.data_ptr(), rows, heads, 0, sink.data_ptr(),
                                              g[0], g[1], s),
             [(b, f) for f in (4, 8) for b in (cus // 4, cus // 2, cus, 2 * cus)]),
            ("random 16-row pages read as 256-byte head slices (page size 16), 4 GiB pool",
             lambda g: lib.msglp_gather_heads(buf.data_ptr(), page_ids.data_ptr(), rows // 16, heads, 1,
                                              sink.data_ptr(), g[0], g[1], s),
             [(b, f) for f in (4, 8) for b in (cus // 4, cus // 2, cus, 2 * cus)])):
        ms, g = best(call, grids)
        gbs = nbytes / (ms * 1e-3) / 1e9
        rec = {"ceiling": name, "ms": round(ms, 4), "GBs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        if isinstance(g, tuple):
            rec.update(blocks=g[0], loads_in_flight_per_lane=g[1])
        else:
            rec["blocks"] = g
        print(json.dumps(rec), flush=True)


def main() -> int:
    if len(sys.argv) > 1 and sys.argv[1] == "--prefill-profile":
        return prefill_profile(int(sys.argv[2]) if len(sys.argv) > 2 else 20, "--zero-new" in sys.argv)
    if len(sys.argv) > 1 and sys.argv[1] == "--mixed":
        return mixed(int(sys.argv[2]) if len(sys.argv) > 2 else 5)
    if len(sys.argv) > 1 and sys.argv[1] == "--ceilings":
        return ceilings(int(sys.argv[2]) if len(sys.argv) > 2 else 20)
    if len(sys.argv) > 1 and sys.argv[1] == "--sweep":
        return sweep(int(sys.argv[2]) if len(sys.argv) > 2 else 20)
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profiles":
        # bench.py --summarize-profiles STATS_DIR FETCH_DIR WRITE_DIR ALGO_BYTES "COMMAND" [BENCH_JSON]
        rope_bytes = None
        if len(sys.argv) > 7:  # the bench line gives the RoPE kernel's algorithmic bytes per batch
            with open(sys.argv[7]) as f:
                rec = json.loads([ln for ln in f if ln.startswith("{")][-1])
            rope_bytes = {k: v["bytes_per_launch"] for k, v in rec["rope_store_kv"].items()}
        summarize_profiles(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[6], int(sys.argv[5]), rope_bytes)
        return 0
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--page-size", type=int, default=1, choices=(1, 16))
    ap.add_argument("--chunk", type=int, default=0, help="decode split size (0 = library default)")
    ap.add_argument("--kernel-iters", type=int, default=KERNEL_ITERS, help="eager decode launches timed for the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed 36-layer step (config 5)")
    ap.add_argument("--cpu-sample-reqs", type=int, default=256,
                    help="decode requests the CPU oracle is timed on (first N of the batch)")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="after the run, negate a tensor of this many GiB into another (a plain "
                         "read-once / write-once kernel used to scale HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this attention step has no cross-GPU path "
              "(each GPU would run it on its own share of heads or requests). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from paged_kv_attention_slots_amd import _lib, runner, workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    log("building decode workloads (Qwen3-8B shape, bs 256, page sizes 1 and 16) on the GPU")
    w4 = wl.qwen3_8b_decode(page_size=args.page_size, device=dev)
    # the same lengths and logical K/V at the other page size (both are the decode gate)
    w4o = wl.qwen3_8b_decode(page_size=17 - args.page_size, device=dev)
    log(f"  sum(L)={int(w4.seq_lens.sum())} max L={int(w4.seq_lens.max())} ({time.time() - t0:.1f}s)")
    w2 = wl.qwen3_06b_decode(device=dev)
    log(f"  qwen3-0.6b decode bs {w2.bs}: sum(L)={int(w2.seq_lens.sum())} ({time.time() - t0:.1f}s)")
    w3 = wl.ragged_prefill(device=dev)
    log(f"  prefill tokens={w3.num_tokens} ctx={int(w3.seq_lens.sum())} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=dev)
    # fixed buffers recorded by the graph
    out4 = torch.empty_like(w4.q)
    lse4 = torch.empty(w4.bs, w4.q_heads, dtype=torch.float32, device=dev)
    ws4 = _lib.decode_workspace(w4.bs, w4.q_heads, w4.head_dim, w4.max_seq_len, args.chunk, device=dev)
    k_pool4, v_pool4 = w4.k_pool, w4.v_pool
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph = _lib.msgl_decode_graph_create(k_pool4, v_pool4, w4.k_new, w4.v_new, w4.out_loc, out4, lse4,
                                              w4.q, w4.page_table, w4.table_idx, w4.seq_lens,
                                              w4.max_seq_len, ws4, page_size=w4.page_size,
                                              chunk=args.chunk, sm_scale=w4.sm_scale, stream=stream)
    # the other page size's step, and the Qwen3-0.6B decode batch (bs 64), each
    # as a captured step of its own (store_kv + decode attention)
    side = {}
    for tag, w in ((f"ps{w4o.page_size}", w4o), ("qwen3_06b_bs64", w2)):
        o = torch.empty_like(w.q)
        l = torch.empty(w.bs, w.q_heads, dtype=torch.float32, device=dev)
        ws = _lib.decode_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len, args.chunk, device=dev)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g = _lib.msgl_decode_graph_create(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc, o, l, w.q,
                                              w.page_table, w.table_idx, w.seq_lens, w.max_seq_len, ws,
                                              page_size=w.page_size, chunk=args.chunk, sm_scale=w.sm_scale,
                                              stream=stream)
        side[tag] = (w, g, (o, l, ws))
    out3 = torch.empty_like(w3.q)
    lse3 = torch.empty(w3.num_tokens, w3.q_heads, dtype=torch.float32, device=dev)
    max_ext3 = int((w3.seq_lens - w3.cached_lens).max())

    def prefill_leg():
        _lib.msgl_store_kv(w3.k_pool, w3.v_pool, w3.k_new, w3.v_new, w3.out_loc, stream=stream)
        _lib.msgl_prefill_attn(out3, lse3, w3.q, w3.k_pool, w3.v_pool, w3.page_table, w3.table_idx,
                               w3.seq_lens, w3.cached_lens, w3.cu_q, max_ext3, page_size=w3.page_size,
                               sm_scale=w3.sm_scale, stream=stream)

    # settle: the first few tens of steps after matrix work starts run the decode leg 10-15%
    # slower (a start-up transient of the clocks or power state: it is gone after ~50 steps
    # and does not come back); full steps, untimed, before the W warm-up steps
    # One step: the captured decode step at page size 1, the same at page size
    # 16, the Qwen3-0.6B decode step, then the prefill leg.
    g_o, g_2 = side[f"ps{w4o.page_size}"][1], side["qwen3_06b_bs64"][1]

    legs = [lambda: graph.launch(stream), lambda: g_o.launch(stream), lambda: g_2.launch(stream), prefill_leg]

    log(f"settle {SETTLE_STEPS} steps, warmup {args.warmup} steps")
    for _ in range(SETTLE_STEPS + args.warmup):
        for leg in legs:
            leg()
    torch.cuda.synchronize()

    K = args.steps
    n_legs = len(legs)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_legs + 1)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        for j, leg in enumerate(legs):
            leg()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    leg_ms = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / K for j in range(n_legs)]
    dec_ms, dec_o_ms, dec2_ms, pre_ms = leg_ms
    ms_per_step = wall * 1e3 / K

    # dominant kernel: decode attention on its own, eager, HIP events on its stream
    log(f"timing {args.kernel_iters} eager decode-attention launches")
    ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        runner.decode_attn(w4, k_pool4, v_pool4, out=out4, lse=lse4, workspace=ws4, chunk=args.chunk,
                           stream=stream)
    torch.cuda.synchronize()
    ka.record(stream)
    for _ in range(args.kernel_iters):
        runner.decode_attn(w4, k_pool4, v_pool4, out=out4, lse=lse4, workspace=ws4, chunk=args.chunk,
                           stream=stream)
    kb.record(stream)
    torch.cuda.synchronize()
    attn_ms = ka.elapsed_time(kb) / args.kernel_iters

    # prefill attention on its own: back-to-back launches (the step's leg above
    # also holds store_kv and starts with the pools just swept by the decode)
    log("timing prefill-attention launches (5 rounds)")

    def prefill_attn_only():
        _lib.msgl_prefill_attn(out3, lse3, w3.q, w3.k_pool, w3.v_pool, w3.page_table, w3.table_idx,
                               w3.seq_lens, w3.cached_lens, w3.cu_q, max_ext3, page_size=w3.page_size,
                               sm_scale=w3.sm_scale, stream=stream)

    # the compute clocks take some tens of milliseconds of sustained matrix work
    # to settle: warm up on the kernel itself (~40 ms) before timing it
    for _ in range(PREFILL_WARM_LAUNCHES):
        prefill_attn_only()
    # the median of 5 rounds of back-to-back launches (a single window varies by a few percent)
    p_rounds = []
    for _ in range(5):
        ka.record(stream)
        for _ in range(max(100, args.kernel_iters)):
            prefill_attn_only()
        kb.record(stream)
        torch.cuda.synchronize()
        p_rounds.append(ka.elapsed_time(kb) / max(100, args.kernel_iters))
    pattn_ms = statistics.median(p_rounds)

    # the same launch without the lse output (an engine's prefill asks for none): the kernels then
    # skip the unrounded weight sums; bit-identical outputs
    out3n = torch.empty_like(out3)

    def prefill_attn_no_lse():
        _lib.msgl_prefill_attn(out3n, None, w3.q, w3.k_pool, w3.v_pool, w3.page_table, w3.table_idx,
                               w3.seq_lens, w3.cached_lens, w3.cu_q, max_ext3, page_size=w3.page_size,
                               sm_scale=w3.sm_scale, stream=stream)

    nolse_ms = _time_stream(prefill_attn_no_lse, stream, max(100, args.kernel_iters), warm=100)
    torch.cuda.synchronize()
    nolse = {"ms": round(nolse_ms, 4), "tflops": round(prefill_flops(w3) / (nolse_ms * 1e-3) / 1e12, 1),
             "frac_bf16_peak": round(prefill_flops(w3) / (nolse_ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 4),
             "bit_identical": bool(torch.equal(out3n.view(torch.int16), out3.view(torch.int16)))}

    # the same launch with the host plan (block list made on the host, copied
    # once): bit-identical outputs, timed in interleaved rounds with the
    # unplanned launch
    log("timing the planned prefill launch (host plan)")
    meta_h = (w3.seq_lens.cpu(), w3.cached_lens.cpu(), w3.cu_q.cpu(), w3.table_idx.cpu())  # host copies
    make_plan = lambda: _lib.msgl_prefill_plan(*meta_h, w3.page_table.shape[0], w3.page_table.shape[1],
                                               w3.q_heads, w3.kv_heads)
    plan_h = make_plan()
    plan_times = []
    for _ in range(20):  # the host plan's own time (metadata already on the host), median of 20 calls
        h0 = time.perf_counter()
        make_plan()
        plan_times.append((time.perf_counter() - h0) * 1e6)
    plan_us = statistics.median(plan_times)
    plan_d = plan_h.to(dev)
    out3p = torch.empty_like(out3)
    lse3p = torch.empty_like(lse3)

    def prefill_attn_planned():
        _lib.msgl_prefill_attn_planned(out3p, lse3p, w3.q, w3.k_pool, w3.v_pool, w3.page_table, plan_h, plan_d,
                                       page_size=w3.page_size, sm_scale=w3.sm_scale, stream=stream)

    prefill_attn_planned()
    torch.cuda.synchronize()
    plan_same = bool(torch.equal(out3p.view(torch.int16), out3.view(torch.int16)) and torch.equal(lse3p, lse3))
    rounds = {"planned": [], "unplanned": []}
    n_round = max(100, args.kernel_iters)
    for _ in range(4):
        for tag, fn in (("planned", prefill_attn_planned), ("unplanned", prefill_attn_only)):
            for _ in range(n_round):  # the clocks stay up: no idle gap before the timed launches
                fn()
            ka.record(stream)
            for _ in range(n_round):
                fn()
            kb.record(stream)
            torch.cuda.synchronize()
            rounds[tag].append(ka.elapsed_time(kb) / n_round)
    plan_ms = statistics.median(rounds["planned"])
    planned = {"median_ms": round(plan_ms, 4), "tflops": round(prefill_flops(w3) / (plan_ms * 1e-3) / 1e12, 1),
               "unplanned_median_ms": round(statistics.median(rounds["unplanned"]), 4),
               "rounds": 4, "launches_per_round": n_round, "entries": int(plan_h[3]),
               "host_plan_us": round(plan_us, 1), "bit_identical": plan_same}

    # the next step on the layer's path: RoPE of q and k fused with the KV write,
    # on the decode batch and on the prefill batch (back-to-back launches)
    log(f"timing {args.kernel_iters} fused RoPE + KV-write launches per batch")
    rope = {}
    for tag, w in (("decode_bs256", w4), ("prefill_8req", w3)):
        q_rot = torch.empty_like(w.q)

        def rope_call(w=w, q_rot=q_rot):
            _lib.msgl_rope_store_kv(q_rot, w.q, w.k_pool, w.v_pool, w.k_new, w.v_new, w.positions, w.out_loc,
                                    ROPE_BASE, stream=stream)

        r_ms = _time_stream(rope_call, stream, args.kernel_iters)
        r_gbs = rope_store_bytes(w) / (r_ms * 1e-3) / 1e9
        rope[tag] = {"tokens": w.num_tokens, "ms": round(r_ms, 4), "GBs": round(r_gbs, 1),
                     "frac_hbm": round(r_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": rope_store_bytes(w)}

    # vocabulary indexing on the Qwen3-8B table (151936 x 4096 bf16): the mixed
    # step's 4288 new tokens and a decode batch of 256
    log(f"timing {args.kernel_iters} vocabulary-indexing launches per batch")
    vocab = {}
    for tag, n in (("tokens4288", 4288), ("decode_bs256", 256)):
        vb = wl.vocab_batch(device=dev, num_tokens=n)
        e_out = torch.empty(n, vb.hidden, dtype=vb.weight.dtype, device=dev)
        v_ms = _time_stream(lambda: _lib.msgl_vocab_embed(e_out, vb.weight, vb.ids, vb.vocab_start, stream=stream),
                            stream, args.kernel_iters)
        vbytes = 2 * n * vb.hidden * vb.weight.element_size() + 4 * n
        vocab[tag] = {"tokens": n, "ms": round(v_ms, 4), "GBs": round(vbytes / (v_ms * 1e-3) / 1e9, 1),
                      "frac_hbm": round(vbytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": vbytes}
        del vb, e_out

    # decode over shared radix prefixes (4 groups of 64 requests on 4096-token
    # prefixes, Qwen3-8B heads): the cascade call against plain decode attention
    log("building the shared-prefix decode batch and timing it")
    cascade = shared_prefix_leg(args.kernel_iters, stream)

    # both attention kernels again, one launch at a time after a cache flush (1 GiB written,
    # then 512 MiB read: no input and no dirty line left in the last-level cache)
    log("timing flushed launches (1 GiB written and 512 MiB read between launches)")
    dflush = flushed_timing(lambda: runner.decode_attn(w4, k_pool4, v_pool4, out=out4, lse=lse4, workspace=ws4,
                                                       chunk=args.chunk, stream=stream), stream, 50)
    dflush["GBs"] = round(decode_bytes(w4) / (dflush["median_ms"] * 1e-3) / 1e9, 1)
    # the captured steps at both page sizes, replayed one at a time after the flush
    gflush = {}
    for tag, w, g in ((f"ps{w4.page_size}", w4, graph), (f"ps{w4o.page_size}", w4o, g_o)):
        f = flushed_timing(lambda g=g: g.launch(stream), stream, 50)
        gbs = (decode_bytes(w) + store_bytes(w)) / (f["median_ms"] * 1e-3) / 1e9
        f["GBs"] = round(gbs, 1)
        f["frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
        f["write_only"]["frac_hbm"] = round((decode_bytes(w) + store_bytes(w)) / (f["write_only"]["median_ms"] * 1e-3)
                                            / 1e9 / HBM_PEAK_GBS, 4)
        gflush[tag] = f
    pflush = flushed_timing(prefill_attn_only, stream, 50)
    pflush["TFLOPs"] = round(prefill_flops(w3) / (pflush["median_ms"] * 1e-3) / 1e12, 1)
    pflush["frac_bf16_peak"] = round(pflush["TFLOPs"] / BF16_DENSE_PEAK_TFLOPS, 4)

    # config 5: the mixed 36-layer step (its own 172 GB pool), unless --no-mixed
    mixed_rec = None
    if not args.no_mixed:
        try:
            mixed_rec = mixed_leg(5, stream)
        except torch.cuda.OutOfMemoryError as e:  # the pool does not fit beside the other legs' buffers
            torch.cuda.empty_cache()
            mixed_rec = {"skipped": f"out of device memory: {str(e)[:120]}"}

    dbytes = decode_bytes(w4)
    sbytes = store_bytes(w4)
    flops3 = prefill_flops(w3)
    value = (dbytes + sbytes) / (dec_ms * 1e-3) / 1e9
    attn_gbs = dbytes / (attn_ms * 1e-3) / 1e9
    prefill_tflops = flops3 / (pre_ms * 1e-3) / 1e12
    pattn_tflops = flops3 / (pattn_ms * 1e-3) / 1e12
    req_tok_s = w4.bs / (dec_ms * 1e-3)

    def graph_leg(w, ms):
        gbs = (decode_bytes(w) + store_bytes(w)) / (ms * 1e-3) / 1e9
        return {"batch": w.bs, "q_heads": w.q_heads, "kv_heads": w.kv_heads, "page_size": w.page_size,
                "context_tokens": int(w.seq_lens.sum()), "ms": round(ms, 4), "GBs": round(gbs, 1),
                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "req_tokens_per_s": round(w.bs / (ms * 1e-3), 1),
                "bytes": decode_bytes(w) + store_bytes(w)}

    decode_graph = {f"ps{w4.page_size}": graph_leg(w4, dec_ms), f"ps{w4o.page_size}": graph_leg(w4o, dec_o_ms)}
    config2 = graph_leg(w2, dec2_ms)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        n = max(1, min(args.cpu_sample_reqs, w4.bs))
        log(f"CPU oracle on the first {n} decode requests (host copies)")
        ws = wl.subset_decode(w4, n)
        kp_h, vp_h = oracle.store_kv(w4.k_pool.cpu(), w4.v_pool.cpu(), ws.k_new, ws.v_new, ws.out_loc)
        q_h = ws.q.cpu()
        args_h = (ws.page_table.cpu(), ws.table_idx.cpu(), ws.seq_lens.cpu(), ws.cu_q.cpu())
        threads = oracle.num_threads()
        # repeat the sample until about 10 s of CPU time (at most 30 s)
        reps, c0 = 0, time.perf_counter()
        while True:
            oracle.attention(q_h, kp_h, vp_h, *args_h)
            reps += 1
            el = time.perf_counter() - c0
            if el >= 10.0 or el * (reps + 1) / reps > 30.0:
                break
        cpu_s = el / reps
        sb = decode_bytes(ws)
        cpu = {"value": round(sb / cpu_s / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"fp64 C oracle, decode attention of the first {n} of {w4.bs} requests "
                         f"({int(ws.seq_lens.sum())} context tokens), {reps} passes, {cpu_s:.2f} s each on "
                         f"{threads} OpenMP threads ({cpu_model()}; {len(os.sched_getaffinity(0))} cores "
                         f"in this process's affinity set)",
               "seconds_per_pass": round(cpu_s, 3)}
        log(f"  oracle {cpu_s:.2f}s with {threads} threads")
        # the first 8 of the same requests on one thread (the pools as stored above)
        n1 = min(8, n)
        w1t = wl.subset_decode(ws, n1)
        s1, r1 = oracle_pass_time_h(oracle, (q_h[:n1], kp_h, vp_h, args_h[0], args_h[1][:n1], args_h[2][:n1],
                                             args_h[3][:n1 + 1]), 1, 2.0, 8.0)
        cpu["one_thread"] = {"value": round(decode_bytes(w1t) / s1 / 1e9, 4), "unit": "GB/s",
                             "sample": f"the first {n1} requests ({int(w1t.seq_lens.sum())} context tokens), "
                                       f"{r1} passes, {s1:.2f} s each on 1 thread"}
        cpu_prefill = prefill_cpu_baseline(oracle, w3, threads)
        cpu["prefill"] = cpu_prefill
        log("CPU oracle on the small configurations")
        cpu["small_configs"] = small_config_cpu_baselines(oracle, w2, threads)

    rec = {
        "metric": "paged decode-attn achieved HBM GB/s + req-tokens/s; prefill attn TFLOP/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": SETTLE_STEPS,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"qwen3-8b decode bs256 ps{w4.page_size} (hipGraph: store_kv + decode attn; value) "
                        f"+ the same at ps{w4o.page_size} + qwen3-0.6b decode bs64 (hipGraph) "
                        f"+ ragged prefill 8 req (store_kv + prefill attn)",
            "decode": {"batch": w4.bs, "q_heads": w4.q_heads, "kv_heads": w4.kv_heads,
                       "head_dim": w4.head_dim, "page_size": w4.page_size,
                       "context_tokens": int(w4.seq_lens.sum()), "max_len": int(w4.seq_lens.max()),
                       "min_units_per_block": args.chunk or 64},
            "prefill": {"requests": w3.bs, "q_heads": w3.q_heads, "kv_heads": w3.kv_heads,
                        "head_dim": w3.head_dim, "extend_tokens": w3.num_tokens,
                        "context_tokens": int(w3.seq_lens.sum())},
        },
        "decode_leg_ms": round(dec_ms, 4),
        "decode_graph_step": decode_graph,
        "decode_graph_flushed": gflush,
        "qwen3_06b_decode_bs64": config2,
        "prefill_leg_ms": round(pre_ms, 4),
        "req_tokens_per_s": round(req_tok_s, 1),
        "prefill_tflops": round(prefill_tflops, 2),
        "prefill_frac_of_bf16_peak": round(prefill_tflops / BF16_DENSE_PEAK_TFLOPS, 4),
        "prefill_attn_ms": round(pattn_ms, 4),
        "prefill_attn_tflops": round(pattn_tflops, 2),
        "prefill_attn_frac_of_bf16_peak": round(pattn_tflops / BF16_DENSE_PEAK_TFLOPS, 4),
        "prefill_attn_no_lse": nolse,
        "prefill_attn_planned": planned,
        "decode_attn_flushed": dflush,
        "prefill_attn_flushed": pflush,
        "rope_store_kv": rope,
        "vocab_embed": vocab,
        "shared_prefix_decode": cascade,
        "mixed_step": mixed_rec,
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "decode attention (split + merge), eager, bs 256",
                     "bytes_per_launch": dbytes, "avg_launch_ms": round(attn_ms, 4)},
        "cpu_baseline": cpu,
    }
    graph.destroy()
    for _, g, _ in side.values():
        g.destroy()
    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30)) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        xq, yq = x[:n // 4], y[:n // 4]
        for _ in range(3):
            torch.neg(xq, out=yq)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = [n * 4, n // 4 * 4]
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
