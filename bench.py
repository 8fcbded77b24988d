#!/usr/bin/env python3
"""Benchmark of the DeepSeek-V4 indexed-attention prefill hot path on one MI355X.

One step = one pass of the whole hot path over one prefill chunk of the
workload: compress the chunk's raw KV rows into the attention PoolingCache,
compress its raw index keys into the indexer PoolingCache, indexer score +
top-k (dsv4_indexer_select), fused windowed + pooled attention.  Before each
step the caches' host counters are reset to the prefix state, so every step
appends the same rows at the same offsets.  Inputs are resident in HBM before
the timed region.

Prints one JSON line.  `value` is the headline metric, indexer score+top-k
query rows per second (chunk rows / mean time of dsv4_indexer_select inside the
timed steps, measured with HIP events on the launch stream).  `roofline` is
for the dominant kernel, the MFMA indexer score, timed with HIP events over
its own launches in the same configuration; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload's query rows.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds S]

`roofline.traffic` (HBM bytes per score-kernel launch) comes from the
rocprofv3 counter summary profiles/traffic_indexer_score_<workload>.md and is
reported only while the score kernel's sources still hash to the value
recorded there (otherwise null).  It is written, with the counter summary
profiles/counters_<workload>.md, by `bench.py --summarize-counters OUT_MD DB..`
from rocprofv3 --pmc runs of `bench.py --lean --calibration-copy` (one
counter set per run); the calibration copy scales FETCH_SIZE / WRITE_SIZE to
bytes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic_inputs as SI  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 1 << 30        # the calibration copy kernel moves this many bytes each way
SCORE_SOURCES = ("sparse_indexed_attention_amd/csrc/indexer_score.hip",
                 "sparse_indexed_attention_amd/csrc/dsv4_device.h")
SCORE_KERNEL = "indexer_score_kernel"


def score_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_indexer_score_{workload}.md")


def recorded_traffic(workload: str):
    """Bytes per score launch from the counter summary, if its source hash matches."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("score_source_hash") != score_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


KERNEL_CLASSES = (("indexer_score", "indexer_score_kernel"), ("topk", "topk_reg_kernel"),
                  ("attention", "sparse_attn_kernel"), ("attention", "attn_h64_kernel"),
                  ("compress", "compress_kernel"),
                  ("copy", "copy_kernel"))


def read_counter_db(db: str) -> dict:
    """{class: {"duration_ns": [...], counter: [...per dispatch...]}} from one
    rocprofv3 --pmc database: SQ / TCC counters summed over their instances
    per dispatch, GRBM_GUI_ACTIVE the largest instance (the XCDs run in
    parallel)."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select name, dispatch_id, counter_name, counter_value, duration "
                     "from pmc_events").fetchall()
    per = {}
    for name, disp, cname, val, dur in rows:
        cls = next((k for k, pat in KERNEL_CLASSES if pat in name), None)
        if cls is None:
            continue
        d = per.setdefault(cls, {}).setdefault(disp, {"duration_ns": dur})
        if cname.startswith("GRBM"):
            d[cname] = max(d.get(cname, 0.0), val)
        else:
            d[cname] = d.get(cname, 0.0) + val
    out = {}
    for cls, disps in per.items():
        keys = set().union(*[set(v) for v in disps.values()])
        out[cls] = {k: [v[k] for v in disps.values() if k in v] for k in keys}
    return out


def summarize_counters(out_md: str, dbs: list, workload: str, cmds: str):
    """Counter summary of the hot path's kernels from several rocprofv3 --pmc
    runs of `bench.py --lean --calibration-copy` (one counter set per run):
    MFMA utilisation and engine clock of the score and attention kernels,
    counter-measured HBM bytes of the score, top-k and attention kernels
    (FETCH_SIZE / WRITE_SIZE scaled by the same counters' reading for the
    1 GiB probe copy), LDS bank conflicts, instruction mix and wait shares.
    Also rewrites the score kernel's traffic file the bench line reads."""
    merged = {}
    for db in dbs:
        for cls, vals in read_counter_db(db).items():
            m = merged.setdefault(cls, {})
            for k, v in vals.items():
                if k == "duration_ns":
                    m.setdefault(k, []).extend(v)
                else:
                    m[k] = v
    mean = lambda cls, k: float(np.mean(merged[cls][k])) if cls in merged and k in merged[cls] else None
    wl = SI.WORKLOADS[workload]
    T, H, D, k = wl.chunk, wl.heads, wl.head_dim, wl.topk
    tile = wl.tile_rows or T
    S = wl.n_rows_after
    pos = range(wl.q_pos0 + T - tile, wl.q_pos0 + T)
    pairs = sum((p + 1) // 4 for p in pos)
    keys_q = [min(wl.window, p + 1) + min(k, (p + 1) // 4) for p in range(wl.q_pos0, wl.q_pos0 + T)]
    algo = {
        "indexer_score": {"flop": pairs * 2 * wl.idx_heads * wl.idx_dim,
                          "bytes": S * wl.idx_dim * 2 + tile * wl.idx_heads * (wl.idx_dim * 2 + 4)
                          + tile * S * 4},
        "topk": {"bytes": pairs * 4 + tile * k * 4},
        "attention": {"flop": sum(4 * H * D * n for n in keys_q),
                      "bytes": sum(2 * D * n for n in keys_q) + 2 * T * H * D * 2 + T * k * 4},
    }
    # counter units per byte moved, from the probe copy (reads and writes COPY_BYTES)
    kf = mean("copy", "FETCH_SIZE") * 1024.0 / COPY_BYTES if mean("copy", "FETCH_SIZE") else None
    kw = mean("copy", "WRITE_SIZE") * 1024.0 / COPY_BYTES if mean("copy", "WRITE_SIZE") else None
    lines = [f"# Counters of the hot-path kernels, {workload}", "",
             "rocprofv3 --pmc runs of `bench.py --lean --calibration-copy` (warmup 1, 3 steps; each",
             "kernel also runs in its own timed loop), one counter set per run.  Per dispatch, SQ",
             "and TCC counters are summed over their instances and GRBM_GUI_ACTIVE is the largest",
             "instance; figures are means over the kernel's dispatches.  Durations are those of the",
             "counter runs (dispatches are serialised under counters).", "",
             "Commands:", "", "```", cmds.strip(), "```", "",
             f"- workload: `{workload}` ({T} query rows, tile {tile}, {S} pooled rows, k {k})",
             f"- score_source_hash: `{score_source_hash()}`"]
    if kf and kw:
        lines += [f"- copy calibration: FETCH_SIZE {kf:.4f} KiB-units per byte read, "
                  f"WRITE_SIZE {kw:.4f} per byte written (1 GiB probe copy, "
                  f"{len(merged['copy']['FETCH_SIZE'])} dispatches)"]
    lines += ["", "| kernel | dispatches | us (counters) | clock GHz | MFMA busy % | bf16 MFMA FLOP / algorithmic "
              "| HBM read MB | HBM write MB | HBM total / algorithmic | LDS bank conflict % "
              "| VALU / MFMA / LDS / SALU instr per wave | wait any % / dependency % |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    res = {}
    for cls in ("indexer_score", "topk", "attention", "compress", "copy"):
        if cls not in merged:
            continue
        dur = mean(cls, "duration_ns")
        grbm = mean(cls, "GRBM_GUI_ACTIVE")
        # (too short a dispatch gives no usable clock: the counter window
        # is wider than the kernel)
        clock = grbm / dur if grbm and dur and dur > 50e3 else None
        busy = mean(cls, "SQ_VALU_MFMA_BUSY_CYCLES")
        util = 100.0 * busy / (grbm * 1024) if busy is not None and grbm else None
        mops = mean(cls, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        fl = algo.get(cls, {}).get("flop")
        fl_ratio = (mops * 512 / fl) if mops is not None and fl else None
        rd = mean(cls, "FETCH_SIZE") * 1024.0 / kf if kf and mean(cls, "FETCH_SIZE") is not None else None
        wr = mean(cls, "WRITE_SIZE") * 1024.0 / kw if kw and mean(cls, "WRITE_SIZE") is not None else None
        ab = algo.get(cls, {}).get("bytes")
        tot_ratio = (rd + wr) / ab if rd is not None and wr is not None and ab else None
        bc, la = mean(cls, "SQ_LDS_BANK_CONFLICT"), mean(cls, "SQ_LDS_IDX_ACTIVE")
        conf = 100.0 * bc / la if bc is not None and la else None
        waves = mean(cls, "SQ_WAVES")
        mix = None
        if waves:
            mix = " / ".join(f"{(mean(cls, c) or 0) / waves:.0f}" for c in
                             ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"))
        wc = mean(cls, "SQ_WAVE_CYCLES")
        waits = None
        if wc:
            waits = f"{100 * (mean(cls, 'SQ_WAIT_ANY') or 0) / wc:.0f} / {100 * (mean(cls, 'SQ_WAIT_INST_ANY') or 0) / wc:.0f}"
        f = lambda x, fmt: "—" if x is None else format(x, fmt)
        n_disp = len(merged[cls]["duration_ns"])
        lines.append(f"| {cls} | {n_disp} | {f(dur / 1e3 if dur else None, '.1f')} | {f(clock, '.2f')} "
                     f"| {f(util, '.1f')} | {f(fl_ratio, '.3f')} | {f(rd / 1e6 if rd is not None else None, '.1f')} "
                     f"| {f(wr / 1e6 if wr is not None else None, '.1f')} | {f(tot_ratio, '.3f')} "
                     f"| {f(conf, '.1f')} | {mix or '—'} | {waits or '—'} |")
        res[cls] = {"util": util, "clock": clock, "rd": rd, "wr": wr, "algo_bytes": ab}
    lines += ["", "Algorithmic work per launch (the bench's roofline units):"]
    lines += [f"- indexer_score: {algo['indexer_score']['flop']:.4e} FLOP (16,384 per visible pair, "
              f"{pairs} pairs); {algo['indexer_score']['bytes']} B (keys once, q, w, scores written)",
              f"- topk: {algo['topk']['bytes']} B (4 per visible pair read, 4 k per row written)",
              f"- attention: {algo['attention']['flop']:.4e} FLOP (4 H D per query and key); "
              f"{algo['attention']['bytes']} B logical (one {D}-dim bf16 row per query and key, "
              "q and out, the selection)",
              "", "MFMA busy % = sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1,024 SIMDs): "
              "the share of SIMD cycles the matrix cores were busy, at the clock the kernel ran at.",
              "clock = GRBM_GUI_ACTIVE / duration."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(out_md).read())
    sc = res.get("indexer_score")
    if sc and sc["rd"] is not None and sc["wr"] is not None:
        with open(traffic_file(workload), "w") as fh:
            fh.write(f"# HBM traffic of the indexer score kernel, {workload}\n\n")
            fh.write("FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the same counter's reading "
                     "for the 1 GiB probe copy; taken with the counter runs of "
                     f"`{os.path.basename(out_md)}` (commands there).\n\n")
            fh.write(f"- workload: `{workload}`\n- score_source_hash: `{score_source_hash()}`\n")
            fh.write(f"- hbm_fetch_bytes_per_launch: {sc['rd']:.0f}\n")
            fh.write(f"- hbm_write_bytes_per_launch: {sc['wr']:.0f}\n")
            fh.write(f"- hbm_bytes_per_launch: {sc['rd'] + sc['wr']:.0f}\n")
            fh.write(f"- algorithmic_bytes_per_launch: {sc['algo_bytes']}\n")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=SI.CTX_128K.name, choices=sorted(SI.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the CPU oracle baseline (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--matrix", action="store_true",
                    help="instead of the benchmark, time the (global chunk, indexer tile) matrix "
                         "at 1M context, serial and ping-pong, one JSON line per pair")
    ap.add_argument("--all-configs", action="store_true",
                    help="one bench line per named workload (tiny .. 1M), without the extras")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the sibling-mode and narrow-query measurements")
    ap.add_argument("--lean", action="store_true",
                    help="only the timed steps and per-kernel timings (for profiler runs)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the benchmark, run a 1 GiB copy kernel three times (counter scale)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="OUT_MD DB [DB ...]: write the counter summary of the hot-path kernels "
                         "(and the score kernel's traffic file) from rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DB", "BENCH_LOG", "OUT_MD"),
                    help="write the kernel-trace summary of a profiled bench run and exit")
    ap.add_argument("--commands", default="",
                    help="text of the commands, for --summarize-counters / --summarize-trace")
    ap.add_argument("--ab", nargs=2, metavar=("LIB_A", "LIB_B"),
                    help="instead of the benchmark, time one operation of two builds of the "
                         "library in this process, alternating rounds (see ab_compare)")
    ap.add_argument("--ab-op", default="attention", choices=("attention", "select", "score", "topk"))
    ap.add_argument("--ab-rounds", type=int, default=8)
    return ap.parse_args()


class Setup:
    """Device state of one chunk of the workload (caches at the prefix state)."""

    def __init__(self, wl: SI.Workload, seed: int):
        import sparse_indexed_attention_amd as dsv4
        self.dsv4 = dsv4
        self.wl = wl
        inp = SI.make_inputs(wl, seed)
        if not wl.bf16:
            for k in list(inp):
                if isinstance(inp[k], np.ndarray) and k != "w":
                    inp[k], inp[k + "_t"] = SI.as_bf16(inp[k])[1], SI.as_bf16(inp[k])[0]
        self.inp = inp
        self.n_prefix = wl.prefix_tokens // 4
        self.icache = dsv4.PoolCache(wl.capacity_rows, wl.idx_dim)
        self.acache = dsv4.PoolCache(wl.capacity_rows, wl.head_dim)
        if self.n_prefix:
            self.icache.rows[:self.n_prefix].copy_(inp["prefix_idx_rows_t"])
            self.acache.rows[:self.n_prefix].copy_(inp["prefix_attn_rows_t"])
        self.raw_pos0 = inp["raw_pos0"]
        self.raw_kv = inp["raw_kv_t"].cuda()
        self.chunk_kv = self.raw_kv[wl.q_pos0 - self.raw_pos0:]
        self.idx_keys = inp["idx_keys_t"].cuda()
        self.q_idx = inp["q_idx_t"].cuda()
        self.w = inp["w_t"].cuda()
        self.q_attn = inp["q_attn_t"].cuda()
        T = wl.chunk
        self.tile = wl.tile_rows if wl.tile_rows else T
        self.S_after = wl.n_rows_after
        self.scratch = torch.empty(dsv4.dsv4_indexer_scratch_bytes(self.tile, self.S_after) // 4,
                                   device="cuda")
        self.idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
        self.out = torch.empty((T, wl.heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")

    def reset(self):
        self.icache.set_state(self.n_prefix, 0)
        self.acache.set_state(self.n_prefix, 0)

    def step(self, ev=None):
        d, wl = self.dsv4, self.wl
        self.reset()
        if ev: ev[0].record()
        d.dsv4_compress(self.acache, self.chunk_kv)
        d.dsv4_compress(self.icache, self.idx_keys)
        if ev: ev[1].record()
        ap = d.dsv4_indexer_select(self.icache, self.acache.n_rows, self.q_idx, self.w, wl.chunk,
                                   wl.q_pos0, wl.idx_heads, wl.topk, self.idx, self.scratch,
                                   wl.tile_rows)
        if ev: ev[2].record()
        d.dsv4_sparse_prefill_attn(self.q_attn, wl.q_pos0, self.raw_kv, self.raw_pos0, wl.window,
                                   self.acache, self.idx, self.out)
        if ev: ev[3].record()
        return ap


def timed_kernel(fn, reps: int) -> float:
    """Mean ms per call of fn() measured with HIP events on the current stream."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def per_call_stats(fn, reps: int, scrub=None) -> dict:
    """Median and min ms of single calls of fn(), each bracketed by its own HIP
    events on the current stream.  With `scrub` (a large tensor), the buffer
    is overwritten before every call so the call starts with cold caches
    (the 256 MB MALL and the L2s hold none of its inputs)."""
    fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        if scrub is not None:
            scrub.fill_(float(len(times) + 1))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return {"median": float(np.median(times)), "min": float(np.min(times))}


def probe_lib():
    """The ceiling probes (libdsv4_probe.so, built beside libdsv4.so)."""
    import ctypes
    path = os.path.join(ROOT, "sparse_indexed_attention_amd", "libdsv4_probe.so")
    L = ctypes.CDLL(path)
    L.dsv4_probe_mfma_flops.restype = ctypes.c_double
    L.dsv4_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.dsv4_probe_mfma.restype = ctypes.c_int
    L.dsv4_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.dsv4_probe_copy.restype = ctypes.c_int
    L.dsv4_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p]
    return L


def probe_copy(L, src, dst, workgroups=4096):
    rc = L.dsv4_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(),
                           workgroups, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"copy probe launch failed ({rc})")


def achievable_peaks() -> dict:
    """What this machine reaches on plain work in the same process:
    - a register-resident v_mfma_f32_32x32x16_bf16 loop over varied bf16
      operands (two and four waves per SIMD on every CU), with the engine
      clock it ran at (shader-clock and 100 MHz counters of one wave);
    - a 16-byte-per-lane copy of 1 GiB (reads 1 GiB, writes 1 GiB);
    - for context, an 8192^3 bf16 torch.matmul (hipBLASLt)."""
    L = probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for wg in (512, 1024):
        iters = 2000
        out = torch.empty(wg * 256, device="cuda")
        stamps = torch.zeros(2, dtype=torch.int64, device="cuda")
        run = lambda: L.dsv4_probe_mfma(wg, iters, out.data_ptr(), stamps.data_ptr(), stream)
        if run() != 0:
            raise RuntimeError("mfma probe launch failed")
        ms = timed_kernel(run, 5)
        ticks, real = stamps.cpu().tolist()
        tflops = L.dsv4_probe_mfma_flops(wg, iters) / (ms * 1e-3) / 1e12
        rec = {"TFLOPs": tflops, "workgroups": wg, "ms": ms,
               "clock_GHz": ticks / (real / 1e8) / 1e9 if real > 0 else None}
        if best is None or tflops > best["TFLOPs"]:
            best = rec
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms_copy = min(timed_kernel(lambda: probe_copy(L, src, dst, wg), 10) for wg in (2048, 8192))
    del src, dst
    m = 8192
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    ms_gemm = timed_kernel(lambda: torch.matmul(a, b), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"mfma_loop_bf16_TFLOPs": best["TFLOPs"], "mfma_loop": best,
            "hbm_copy_GBps": 2 * n * 4 / (ms_copy * 1e-3) / 1e9,
            "library_gemm_bf16_TFLOPs": 2 * m ** 3 / (ms_gemm * 1e-3) / 1e12,
            "how": "register-resident 32x32x16 bf16 MFMA loop and 1 GiB 16-byte copy "
                   "(libdsv4_probe.so); 8192^3 bf16 torch.matmul for context; same process"}


def measure_modes(setup: Setup, reps: int) -> dict:
    """The sibling attention modes of the same fused kernel on this chunk:
    window-only (LocalAttention) and window + every visible ratio-128 pooled
    row (CompressedAttention, after the chunk's ratio-128 compress).  Each is
    timed with HIP events over `reps` launches; FLOPs are 4*H*D per (query,
    key) and the gather is one head_dim row of bf16 per (query, key)."""
    d, wl = setup.dsv4, setup.wl
    T, H, D, W = wl.chunk, wl.heads, wl.head_dim, wl.window
    rows_t, _ = SI.prefix_rows_ratio(wl, 0, 128)
    n128 = rows_t.shape[0]
    c128 = d.PoolCache(n128 + T // 128 + 1, D, ratio=128)
    c128.rows[:n128].copy_(rows_t)

    def comp128():
        c128.set_state(n128, 0)
        d.dsv4_compress(c128, setup.chunk_kv)

    ms_c128 = timed_kernel(comp128, reps)
    comp128()
    out = setup.out
    ms_local = timed_kernel(lambda: d.dsv4_sparse_prefill_attn(
        setup.q_attn, wl.q_pos0, setup.raw_kv, setup.raw_pos0, W, None, None, out), reps)
    ms_comp = timed_kernel(lambda: d.dsv4_sparse_prefill_attn(
        setup.q_attn, wl.q_pos0, setup.raw_kv, setup.raw_pos0, W, c128, None, out), reps)
    res = {}
    for name, ms, pooled in (("local_attention", ms_local, lambda p: 0),
                             ("compressed_attention_r128", ms_comp, lambda p: (p + 1) // 128)):
        keys = sum(min(W, p + 1) + pooled(p) for p in range(wl.q_pos0, wl.q_pos0 + T))
        tflops = 4 * H * D * keys / (ms * 1e-3) / 1e12
        gbs = keys * D * 2 / (ms * 1e-3) / 1e9
        res[name] = {"ms": ms, "query_rows_per_s": T / (ms * 1e-3), "keys_per_query": keys / T,
                     "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS},
                     "gather_GBps": gbs}
    res["compress_r128_ms"] = ms_c128
    return res


def measure_narrow(setup: Setup, reps: int) -> dict:
    """Narrow-query steps (T = 1, 2, 4 query rows: decode, draft verification,
    short prefill bands) at the end of this workload's context, against the
    same caches: the indexer select (scratch as dsv4_indexer_scratch_bytes
    sizes it) and the key-split attention with its planned split count.
    HIP-event means over `reps` calls of each, eager and as a replayed HIP
    graph of the whole step."""
    d, wl = setup.dsv4, setup.wl
    S = setup.S_after
    H, D, W, k = wl.heads, wl.head_dim, wl.window, wl.topk
    res = {}
    for T in (1, 2, 4):
        q0 = 4 * S - T                      # the last T positions the caches cover
        scratch = torch.empty(d.dsv4_indexer_scratch_bytes(T, S) // 4, device="cuda")
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        qi, w, qa = setup.q_idx[:T], setup.w[:T], setup.q_attn[:T]
        ns, nb = d.dsv4_sparse_attn_narrow_plan(T, H, D, W, k)
        ws = torch.empty(max(nb // 4, 4), device="cuda")
        raw_lo = q0 - W + 1
        raw = setup.raw_kv[raw_lo - setup.raw_pos0:q0 + T - setup.raw_pos0]

        def sel():
            d.dsv4_indexer_select(setup.icache, setup.acache.n_rows, qi, w, T, q0, wl.idx_heads,
                                  k, idx, scratch, 0)

        def attn():
            d.dsv4_sparse_attn_narrow(qa, q0, raw, raw_lo, W, setup.acache, idx, out, ns, ws)

        ms_sel = timed_kernel(sel, reps)
        ms_attn = timed_kernel(attn, reps)
        ms_step = timed_kernel(lambda: (sel(), attn()), reps)
        # the same step captured once in a HIP graph and replayed (no host
        # launch work per kernel)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sel(); attn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sel(); attn()
        torch.cuda.synchronize()
        ms_graph = timed_kernel(graph.replay, reps)
        res[f"T{T}"] = {"select_ms": ms_sel, "attention_ms": ms_attn, "attention_splits": ns,
                        "step_ms": ms_step, "query_rows_per_s": T / (ms_step * 1e-3),
                        "graph_step_ms": ms_graph,
                        "graph_query_rows_per_s": T / (ms_graph * 1e-3)}
    return res


# (global chunk, indexer tile) pairs of the tiling proposal's benchmark matrix
MATRIX = ((4096, 4096), (2048, 2048), (1024, 1024), (4096, 2048), (4096, 1024))


def tile_matrix(steps: int):
    """Each (chunk, tile) pair at 1M tokens of context (the chunk ends at
    position 2^20): score scratch bytes, whole-chunk indexer select time with
    one scratch reused by every tile (serial), the same tiles with two scratch
    buffers and the top-k of tile i on a second stream beside the scoring of
    tile i+1 (ping-pong), and the whole step (compress, select, attention)."""
    import dataclasses
    for chunk, tile in MATRIX:
        wl = dataclasses.replace(SI.CTX_1M, name=f"ctx1m-chunk{chunk}-tile{tile}",
                                 prefix_tokens=(1 << 20) - chunk, chunk=chunk,
                                 tile_rows=0 if tile == chunk else tile)
        st = Setup(wl, 0)
        d = st.dsv4
        st.step()
        torch.cuda.synchronize()
        S, T, q0 = st.S_after, wl.chunk, wl.q_pos0
        stride = d.dsv4_score_stride(S)
        bufs = [st.scratch[:st.tile * stride].view(st.tile, stride)]
        n_tiles = (T + st.tile - 1) // st.tile
        if n_tiles > 1:
            bufs.append(torch.empty(st.tile * stride, device="cuda").view(st.tile, stride))
        main, aux = torch.cuda.current_stream(), torch.cuda.Stream()
        # the top-k the select runs: the two-pass chunk top-k over long rows,
        # here with a workspace per buffer (the select keeps the chunk winners
        # in its scratch, but a ping-pong buffer is rescored while its top-k runs)
        nb_ws = d.dsv4_topk_split_workspace_bytes(st.tile, q0 + T - st.tile, wl.topk)
        wss = [torch.empty(nb_ws // 4, device="cuda") if nb_ws else None for _ in bufs]

        def serial():
            d.dsv4_indexer_select(st.icache, st.acache.n_rows, st.q_idx, st.w, T, q0,
                                  wl.idx_heads, wl.topk, st.idx, st.scratch, wl.tile_rows)

        def pingpong():
            ev_sc = [torch.cuda.Event() for _ in bufs]
            ev_tk = [torch.cuda.Event() for _ in bufs]
            start = torch.cuda.Event()
            start.record(main)
            aux.wait_event(start)
            for i, t0 in enumerate(range(0, T, st.tile)):
                b, n = i % len(bufs), min(st.tile, T - t0)
                if i >= len(bufs):
                    main.wait_event(ev_tk[b])
                d.dsv4_indexer_scores(st.icache, st.q_idx[t0:t0 + n], st.w[t0:t0 + n], q0 + t0,
                                      bufs[b][:n], True, stream=main)
                ev_sc[b].record(main)
                aux.wait_event(ev_sc[b])
                if nb_ws:
                    d.dsv4_topk_select_split(bufs[b][:n], q0 + t0, S, wl.topk, st.idx[t0:t0 + n],
                                             wss[b], stream=aux)
                else:
                    d.dsv4_topk_select(bufs[b][:n], q0 + t0, S, wl.topk, st.idx[t0:t0 + n],
                                       stream=aux)
                ev_tk[b].record(aux)
            for e in ev_tk:
                main.wait_event(e)

        serial()
        torch.cuda.synchronize()
        ref = st.idx.clone()
        pingpong()
        torch.cuda.synchronize()
        same = bool(torch.equal(ref, st.idx))
        ms_serial = timed_kernel(serial, steps)
        ms_pp = timed_kernel(pingpong, steps)
        ms_step = timed_kernel(st.step, steps)
        one = d.dsv4_indexer_scratch_bytes(st.tile, S)
        print(json.dumps({
            "workload": wl.name, "context_tokens": q0 + T, "chunk": T, "tile_rows": st.tile,
            "pooled_rows": S, "scratch_bytes": one,
            "pingpong_scratch_bytes": (one + nb_ws) * len(bufs),
            "select_ms": ms_serial, "select_rows_per_s": T / (ms_serial * 1e-3),
            "pingpong_select_ms": ms_pp, "pingpong_equal_selection": same,
            "step_ms": ms_step, "step_rows_per_s": T / (ms_step * 1e-3)}))
        sys.stdout.flush()
        del st, bufs, wss
        torch.cuda.empty_cache()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(setup: Setup, budget_s: float):
    """The CPU oracle (score + top-k) on a bounded sample of the chunk's query
    rows, on every host core this process may run on (BLAS threads set to
    that count)."""
    from oracle import dsv4_oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
        limiter = threadpool_limits(limits=cores)
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        limiter, threads = None, None
    wl, inp = setup.wl, setup.inp
    S = setup.S_after
    st = O.PoolingCacheState(wl.idx_dim, S)
    st.rows[:setup.n_prefix] = inp["prefix_idx_rows"]
    st.n_rows = setup.n_prefix
    O.compress(st, inp["idx_keys"])
    keys = st.rows[:S]
    rng = np.random.default_rng(1)
    order = rng.permutation(wl.chunk)
    t0 = time.perf_counter()
    n = 0
    while n < len(order) and (n < 4 or time.perf_counter() - t0 < budget_s):
        t = int(order[n])
        sc = O.indexer_scores(inp["q_idx"][t:t + 1], inp["w"][t:t + 1], keys, wl.q_pos0 + t, S)
        O.topk_select(sc, wl.q_pos0 + t, wl.topk)
        n += 1
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": n / dt, "unit": "query rows/s", "cores": cores, "blas_threads": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} random query rows of the chunk (score + top-k, numpy fp64), {dt:.1f} s"}


def summarize_trace(db: str, log: str, out_md: str, cmds: str):
    """Per-kernel dispatch statistics from a rocprofv3 --kernel-trace database,
    beside the bench line the same run printed."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), avg(duration), min(duration), max(duration), "
                     "sum(duration) from kernels group by name order by sum(duration) desc").fetchall()
    line = None
    with open(log) as fh:
        for ln in fh:
            if ln.startswith('{"metric"'):
                line = json.loads(ln)
    with open(out_md, "w") as fh:
        fh.write("# Kernel trace of the hot-path benchmark\n\n")
        fh.write("Command:\n\n```\n" + cmds.strip() + "\n```\n\n")
        fh.write("| kernel | calls | avg us | min us | max us | total ms |\n|---|---|---|---|---|---|\n")
        for name, n, avg, mn, mx, tot in rows:
            short = name if len(name) < 90 else name[:87] + "..."
            fh.write(f"| `{short}` | {n} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | "
                     f"{tot / 1e6:.2f} |\n")
        if line:
            fh.write("\nThe same run's bench line (HIP-event times, ms):\n\n")
            fh.write(f"- ms: `{json.dumps(line['ms'])}`\n")
            fh.write(f"- value: {line['value']:.0f} {line['unit']}\n")
            fh.write(f"- roofline: `{json.dumps(line['roofline'])}`\n")
    print(open(out_md).read())


def engine_clocks_mhz() -> list:
    """Current shader clock of each GPU the host's sysfs lists (the line the
    driver marks with '*' in pp_dpm_sclk), where readable; else empty."""
    import glob
    out = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if "*" in line:
                    out.append(int("".join(ch for ch in line.split(":")[1] if ch.isdigit())))
        except (OSError, ValueError, IndexError):
            pass
    return out


def ab_compare(args, wl: SI.Workload) -> dict:
    """One operation of two library builds, A and B, in one process: both are
    loaded side by side and called alternately on the same inputs (the chunk
    state of the benchmark, prepared with A), `rounds` rounds of `reps` calls
    each per build, HIP events around each round.  Reports per build the
    median, min and max of the round means, and B / A of the medians; the
    engine clock read from sysfs before and after each round where the host
    exposes it."""
    import sparse_indexed_attention_amd as dsv4
    la = dsv4.use_library(os.path.abspath(args.ab[0]))
    lb = dsv4._load(os.path.abspath(args.ab[1]))
    dsv4.use_library(la)
    st = Setup(wl, args.seed)
    st.step()
    torch.cuda.synchronize()
    d, T = dsv4, wl.chunk
    S = st.S_after
    stride = d.dsv4_score_stride(S)
    sc = st.scratch[:st.tile * stride].view(st.tile, stride)
    t0 = T - st.tile
    if args.ab_op == "topk":
        # the scores of the last query tile, then the top-k the select runs
        # on them (as in the benchmark: the two-pass kernel with a workspace
        # over rows longer than one chunk, so the scores stay intact)
        d.dsv4_indexer_scores(st.icache, st.q_idx[t0:], st.w[t0:], wl.q_pos0 + t0, sc, True)
        torch.cuda.synchronize()
        split_ws = d.dsv4_topk_split_workspace_bytes(st.tile, wl.q_pos0 + t0, wl.topk)
        ws_t = torch.empty(max(1, split_ws // 4), dtype=torch.float32, device="cuda")
    ops = {
        "attention": lambda: d.dsv4_sparse_prefill_attn(st.q_attn, wl.q_pos0, st.raw_kv,
                                                        st.raw_pos0, wl.window, st.acache,
                                                        st.idx, st.out),
        "select": lambda: d.dsv4_indexer_select(st.icache, st.acache.n_rows, st.q_idx, st.w,
                                                wl.chunk, wl.q_pos0, wl.idx_heads, wl.topk,
                                                st.idx, st.scratch, wl.tile_rows),
        "score": lambda: d.dsv4_indexer_scores(st.icache, st.q_idx[t0:], st.w[t0:],
                                               wl.q_pos0 + t0, sc, True),
        "topk": (lambda: d.dsv4_topk_select_split(sc, wl.q_pos0 + t0, S, wl.topk, st.idx[t0:], ws_t))
        if args.ab_op == "topk" and split_ws > 0 else
        (lambda: d.dsv4_topk_select(sc, wl.q_pos0 + t0, S, wl.topk, st.idx[t0:])),
    }
    fn = ops[args.ab_op]
    reps = max(10, args.steps)
    times = {"A": [], "B": []}
    clocks = {"A": [], "B": []}
    for name, L in (("A", la), ("B", lb)):  # warm both
        d.use_library(L)
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    for r in range(args.ab_rounds):
        order = (("A", la), ("B", lb)) if r % 2 == 0 else (("B", lb), ("A", la))
        for name, L in order:
            d.use_library(L)
            c0 = engine_clocks_mhz()
            times[name].append(timed_kernel(fn, reps))
            clocks[name].append([c0, engine_clocks_mhz()])
    d.use_library(la)
    summ = {}
    for name in ("A", "B"):
        v = np.array(times[name])
        summ[name] = {"lib": args.ab[0 if name == "A" else 1], "median_ms": float(np.median(v)),
                      "min_ms": float(v.min()), "max_ms": float(v.max()),
                      "rounds_ms": [round(float(x), 4) for x in v], "clock_mhz": clocks[name]}
    return {"ab": args.ab_op, "workload": wl.name, "rounds": args.ab_rounds, "calls_per_round": reps,
            "A": summ["A"], "B": summ["B"],
            "B_over_A": summ["B"]["median_ms"] / summ["A"]["median_ms"]}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.commands)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:], args.workload,
                           args.commands)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path runs on one MI355X and this build "
              "has no multi-GPU path (see the sharding note in the design notes).", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    if args.ab:
        print(json.dumps(ab_compare(args, SI.WORKLOADS[args.workload])))
        return
    if args.matrix:
        tile_matrix(max(3, args.steps // 4))
        return
    if args.all_configs:
        # one line per named workload (the headline line is the default run)
        for name in ("tiny-64tok", "ctx4k-chunk2048", "ctx16k-chunk2048", "ctx128k-chunk2048",
                     "ctx1m-chunk4096-tile1024"):
            rec = run_workload(args, SI.WORKLOADS[name], extras=False)
            print(json.dumps(rec))
            sys.stdout.flush()
            torch.cuda.empty_cache()
        return
    rec = run_workload(args, SI.WORKLOADS[args.workload], extras=not args.lean)
    print(json.dumps(rec))
    sys.stdout.flush()
    if args.calibration_copy:
        L = probe_lib()
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            probe_copy(L, src, dst)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()


def run_workload(args, wl: SI.Workload, extras: bool) -> dict:
    """Warmup, the timed steps and the per-kernel measurements of one
    workload; `extras` adds the per-call, achievable-peak, sibling-mode and
    narrow-step measurements."""
    setup = Setup(wl, args.seed)
    d = setup.dsv4
    T = wl.chunk
    for _ in range(args.warmup):
        setup.step()
    torch.cuda.synchronize()

    # ---- timed steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_pooled = False
    for k in range(args.steps):
        all_pooled = setup.step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    comp = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    sel = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    attn = np.mean([e[2].elapsed_time(e[3]) for e in evs])

    # ---- per-kernel times, same launch configuration as inside the step
    pairs = wl.visible_pairs()
    S = setup.S_after
    tile = setup.tile
    tile_pairs = sum((p + 1) // 4 for p in range(wl.q_pos0 + T - tile, wl.q_pos0 + T))
    stride = d.dsv4_score_stride(S)
    sc_view = setup.scratch[:tile * stride].view(tile, stride)
    t_last0 = T - tile
    q_t, w_t = setup.q_idx[t_last0:], setup.w[t_last0:]
    ms_score = timed_kernel(lambda: d.dsv4_indexer_scores(setup.icache, q_t, w_t, wl.q_pos0 + t_last0,
                                                          sc_view, True), max(5, args.steps))
    # the top-k the select runs: over rows longer than one 32,768-column chunk,
    # the two-pass chunk top-k (timed here with a workspace, so that the scores
    # just written stay intact; the select keeps the chunk winners in its
    # scratch instead), else the per-row kernel
    split_ws = d.dsv4_topk_split_workspace_bytes(tile, wl.q_pos0 + t_last0, wl.topk)
    if split_ws > 0:
        ws_t = torch.empty(split_ws // 4, dtype=torch.float32, device="cuda")
        topk_fn = lambda: d.dsv4_topk_select_split(sc_view, wl.q_pos0 + t_last0, S, wl.topk,
                                                   setup.idx[t_last0:], ws_t)
    else:
        topk_fn = lambda: d.dsv4_topk_select(sc_view, wl.q_pos0 + t_last0, S, wl.topk,
                                             setup.idx[t_last0:])
    ms_topk = timed_kernel(topk_fn, max(5, args.steps))
    flops_per_pair = 2 * wl.idx_heads * wl.idx_dim
    score_tflops = tile_pairs * flops_per_pair / (ms_score * 1e-3) / 1e12
    topk_bytes = tile_pairs * 4 + tile * wl.topk * 4
    topk_gbs = topk_bytes / (ms_topk * 1e-3) / 1e9

    attn_flops = sum(4 * wl.heads * wl.head_dim
                     * (min(wl.window, p + 1) + min(wl.topk, (p + 1) // 4))
                     for p in range(wl.q_pos0, wl.q_pos0 + T))
    attn_tflops = attn_flops / (attn * 1e-3) / 1e12
    attn_gather = sum(2 * wl.head_dim * (min(wl.window, p + 1) + min(wl.topk, (p + 1) // 4))
                      for p in range(wl.q_pos0, wl.q_pos0 + T))

    # per-call median / min, warm and cold (a 512 MiB write between calls)
    sel_fn = lambda: d.dsv4_indexer_select(setup.icache, setup.acache.n_rows, setup.q_idx, setup.w,
                                           T, wl.q_pos0, wl.idx_heads, wl.topk, setup.idx,
                                           setup.scratch, wl.tile_rows)
    attn_fn = lambda: d.dsv4_sparse_prefill_attn(setup.q_attn, wl.q_pos0, setup.raw_kv,
                                                 setup.raw_pos0, wl.window, setup.acache,
                                                 setup.idx, setup.out)
    reps = max(5, args.steps // 2)
    calls = peaks = modes = narrow = None
    if extras:
        scrub = torch.empty(512 << 18, dtype=torch.float32, device="cuda")
        calls = {"indexer_select": {"warm": per_call_stats(sel_fn, reps),
                                    "cold": per_call_stats(sel_fn, reps, scrub)},
                 "attention": {"warm": per_call_stats(attn_fn, reps),
                               "cold": per_call_stats(attn_fn, reps, scrub)}}
        del scrub
        torch.cuda.empty_cache()
        peaks = achievable_peaks()
        if not args.no_modes:
            modes = measure_modes(setup, max(5, args.steps // 2))
            narrow = measure_narrow(setup, max(10, args.steps))
    budget = args.cpu_seconds if extras else min(args.cpu_seconds, 4.0)
    if args.lean:
        budget = 0
    cpu = cpu_baseline(setup, budget) if budget > 0 else None
    ach = (lambda x, key: x / peaks[key]) if peaks else (lambda x, key: None)
    rec = {
        "metric": "indexer score+top-k query rows/s and pooled-row scores/s at 128K ctx; MFMA util",
        "value": T / (sel * 1e-3),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the pages' 4K-1M contexts)",
        "config": {"workload": wl.name, "context_tokens": wl.q_pos0 + T, "chunk": T,
                   "tile_rows": tile, "pooled_rows": S, "topk": wl.topk,
                   "indexer_heads": wl.idx_heads, "indexer_dim": wl.idx_dim,
                   "heads": wl.heads, "head_dim": wl.head_dim, "window": wl.window},
        "pair_scores_per_s": pairs / (sel * 1e-3),
        "step_query_rows_per_s": T / (ms_step * 1e-3),
        "ms": {"compress_both": comp, "indexer_select": sel, "attention": attn,
               "score_kernel": ms_score, "topk_kernel": ms_topk},
        "all_pooled_path": bool(all_pooled),
        "roofline": {"bound": "mfma", "kernel": "indexer_score", "achieved": score_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": score_tflops / PEAK_BF16_TFLOPS,
                     "traffic": recorded_traffic(wl.name),
                     "frac_of_achievable": ach(score_tflops, "mfma_loop_bf16_TFLOPs")},
        "per_call_ms": calls,
        "achievable": peaks,
        "topk_roofline": {"bound": "hbm", "achieved": topk_gbs, "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": topk_gbs / PEAK_HBM_GBS,
                          "frac_of_achievable": ach(topk_gbs, "hbm_copy_GBps")},
        "attn_roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                          "frac_of_achievable": ach(attn_tflops, "mfma_loop_bf16_TFLOPs"),
                          "gather_GBps": attn_gather / (attn * 1e-3) / 1e9},
        "modes": modes,
        "narrow": narrow,
        "cpu_baseline": cpu,
    }
    return rec


if __name__ == "__main__":
    main()
