#!/usr/bin/env python3
"""Benchmark of the ForwardPass attention step on one MI355X.

A step is one whole pass through the ABI calls (append -> attend ->
fold + readout) over one batch of synthetic input that is already resident
in HBM. The reset of committed_len that makes the same pass replayable runs
before each flushed step's first event, beside the cache flush (the
back-to-back figure keeps it inside).

Default workload: the decode wave (64 lanes x 1 row, kv_len ~ U{512..8192},
H_q=32, H_kv=8, d=128, bf16, pages of 16 in a permuted pool). `value` is the
decode KV read rate of the whole step: algorithmic KV bytes (each lane's
kv_len slots x 2 x H_kv x d x 2 B, read once for all GQA heads) per second.
`roofline` prices the attention kernels alone, timed with HIP events recorded
on the launch stream around them inside every timed step. `cpu_baseline` is
the fp64 oracle timed on the host on a bounded sample of the same workload.

Other workloads: --config 1..5 (3: mixed prefill+decode; 4: guidance +
speculative verify; 5: long-context masked prefill, reported in TFLOP/s).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s + decode KV-read GB/s (1 GPU), % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure

WORKLOAD_TEXT = {
    1: "one lane, 37-row prompt, H_q=4 H_kv=2 d=64, 3 shuffled pages of 16",
    2: "decode wave: 64 lanes x 1 row, kv_len U{512..8192}, H_q=32 H_kv=8 d=128, P=16, permuted pool",
    3: "mixed wave: 8 prefill lanes (1024-4096 rows on 0-2048 cached) + 120 decode lanes (kv 256-16384), "
       "H_q=32 H_kv=8 d=128, P=32",
    4: "guidance pairs (prefix 2048/512) + 32 verify lanes x 8 draft rows, channel fold, H_q=32 H_kv=8 d=128, P=16",
    5: "16 lanes x 512-row chunks over kv_len 32768, window-1024+4-sink / TOVA-30% bitmaps, "
       "H_q=64 H_kv=8 d=128, P=16",
}


# --------------------------------------------------------------------------- algorithmic work

def attended_pairs(wl) -> np.ndarray:
    """|A(r)| per row: slots each row attends (causal rule or bitmap), from the inputs."""
    st = wl.step
    cap = wl.capacity()
    out = np.zeros(st.num_rows, dtype=np.int64)
    for lane in range(wl.num_lanes):
        r0, r1 = int(st.indptr[lane]), int(st.indptr[lane + 1])
        if r1 == r0:
            continue
        eff = min(max(int(st.kv_len[lane]), 0), int(cap[lane]))
        masked = wl.mask_bits is not None and wl.mask_word_offset[lane + 1] > wl.mask_word_offset[lane]
        if not masked:
            out[r0:r1] = np.clip(np.minimum(st.slots[r0:r1].astype(np.int64) + 1, eff), 0, None)
            continue
        o0, o1 = int(wl.mask_word_offset[lane]), int(wl.mask_word_offset[lane + 1])
        wpr = (o1 - o0) // (r1 - r0)
        words = wl.mask_bits[o0:o1].reshape(r1 - r0, wpr)
        nfull = eff // 32
        cnt = np.unpackbits(words[:, :nfull].view(np.uint8), axis=1).sum(axis=1).astype(np.int64)
        if eff % 32 and nfull < wpr:
            tail = words[:, nfull] & np.uint32((1 << (eff % 32)) - 1)
            cnt += np.unpackbits(tail.view(np.uint8).reshape(-1, 4), axis=1).sum(axis=1)
        out[r0:r1] = cnt
    return out


def work(wl):
    """Algorithmic bytes of decode-class lanes and flops of all attention."""
    st = wl.step
    G = wl.H_q // wl.H_kv
    n = np.diff(st.indptr).astype(np.int64)
    eff = np.minimum(np.maximum(st.kv_len.astype(np.int64), 0), wl.capacity())
    decode = (n > 0) & (n * G <= 32)
    kv_bytes = int((eff[decode] * 2 * wl.H_kv * wl.d * 2).sum())
    pairs = attended_pairs(wl)
    lane_of = np.repeat(np.arange(wl.num_lanes), n)
    flops_all = 4.0 * wl.d * wl.H_q * float(pairs.sum())
    flops_prefill = 4.0 * wl.d * wl.H_q * float(pairs[~decode[lane_of]].sum()) if len(pairs) else 0.0
    return dict(kv_bytes_decode=kv_bytes, kv_bytes_all=int((eff * 2 * wl.H_kv * wl.d * 2).sum()),
                flops=flops_all, flops_prefill=flops_prefill, pairs=int(pairs.sum()),
                flops_prefill_executed=executed_prefill_flops(wl))


def executed_prefill_flops(wl) -> float:
    """MFMA flops the prefill kernel issues: each work item (one KV head, a block
    of 256/G rows, all G query heads) runs QK^T and P*V over every 32-slot tile
    it visits (causal lanes: up to the block's furthest row limit; masked lanes:
    the tiles where some row of the block has an allowed slot), for every row
    of the block, padded rows included."""
    st = wl.step
    G = wl.H_q // wl.H_kv
    RB = 256 // G
    cap = wl.capacity()
    tot_tiles_rows = 0
    for lane in range(wl.num_lanes):
        r0, r1 = int(st.indptr[lane]), int(st.indptr[lane + 1])
        n = r1 - r0
        if n == 0 or n * G <= 32:
            continue
        eff = min(max(int(st.kv_len[lane]), 0), int(cap[lane]))
        masked = wl.mask_bits is not None and wl.mask_word_offset[lane + 1] > wl.mask_word_offset[lane]
        if masked:
            o0, o1 = int(wl.mask_word_offset[lane]), int(wl.mask_word_offset[lane + 1])
            wpr = (o1 - o0) // n
            words = wl.mask_bits[o0:o1].reshape(n, wpr)
            ntiles = min((eff + 31) // 32, wpr)
            valid = np.full(ntiles, 0xFFFFFFFF, dtype=np.uint64)
            if ntiles and eff % 32 and ntiles == (eff + 31) // 32:
                valid[-1] = (1 << (eff % 32)) - 1
        for b0 in range(0, n, RB):
            b1 = min(n, b0 + RB)
            if masked:
                anyw = np.bitwise_or.reduce(words[b0:b1, :ntiles].astype(np.uint64), axis=0) & valid
                t = int(np.count_nonzero(anyw))
            else:
                lim = np.minimum(st.slots[r0 + b0:r0 + b1].astype(np.int64) + 1, eff)
                t = (int(lim.max()) + 31) // 32 if b1 > b0 else 0
            tot_tiles_rows += t * RB
    return 4.0 * wl.d * 32 * G * wl.H_kv * float(tot_tiles_rows)


# --------------------------------------------------------------------------- HIP events

class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded (same soname)."""

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.lib.hipEventCreate(self.ct.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        self.lib.hipEventSynchronize(self.ct.c_void_p(b))
        t = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(t), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(self.ct.c_void_p(ev))


# --------------------------------------------------------------------------- CPU baseline

_CPU_JOB = {}  # what the forked oracle workers read (inherited copy-on-write)


def _cpu_attend(rows):
    import oracle

    j = _CPU_JOB
    st, wl = j["st"], j["wl"]
    oracle.attend(j["pool"], st.indptr, st.positions, st.slots, st.kv_len, st.q, wl.H_q, wl.theta, wl.sm_scale,
                  wl.mask_bits, wl.mask_word_offset, rows=rows)
    return len(rows)


def cpu_baseline(wl, cfg: int, unit: str):
    """Time the fp64 oracle on a bounded sample of the same step on the host's
    cores: the append of the sampled lanes, then their attention split by lane
    over a pool of worker processes (one per core of this process's CPU set,
    at most 16, the CPU share of one GPU; BLAS limited to one thread each),
    then fold and readout. Must run before anything in the process touches the
    GPU: the workers are forked from it."""
    import multiprocessing as mp

    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    st = wl.step
    n = np.diff(st.indptr).astype(np.int64)
    order = [l for l in range(wl.num_lanes) if n[l] > 0]
    G = wl.H_q // wl.H_kv
    # bounded sample: whole lanes for decode-class work, sampled rows of prefill lanes
    if cfg in (1, 2, 4):
        lanes, rows = order, None
    else:
        rng = np.random.default_rng(7)
        lanes = sorted(rng.choice(order, size=min(2 * cores, len(order)), replace=False).tolist())
        rows = []
        for l in lanes:
            r0, r1 = int(st.indptr[l]), int(st.indptr[l + 1])
            rows += sorted(set(rng.integers(r0, r1, size=min(8, r1 - r0)).tolist()))
        rows = np.array(rows, dtype=np.int64)
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
    c = np.zeros(wl.num_lanes, np.int32)
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        if wl.prefix is not None:  # untimed set-up, like the GPU prefix pass
            p = wl.prefix
            oracle.append(pool, c, p.indptr, p.positions, p.slots, p.k, p.v, wl.theta, lanes=lanes)
            c, _ = oracle.fold(c, p.indptr, p.fold)
        sample_rows = rows if rows is not None else np.concatenate(
            [np.arange(st.indptr[l], st.indptr[l + 1]) for l in lanes]).astype(np.int64)
        lane_of = np.searchsorted(st.indptr, sample_rows, side="right") - 1
        groups = [sample_rows[lane_of == l] for l in lanes]
        groups = sorted([g for g in groups if len(g)], key=len, reverse=True)
        t0 = time.perf_counter()
        oracle.append(pool, c, st.indptr, st.positions, st.slots, st.k, st.v, wl.theta, lanes=lanes)
        _CPU_JOB.update(pool=pool, st=st, wl=wl)
        with mp.get_context("fork").Pool(cores) as workers:
            workers.map(_cpu_attend, groups, chunksize=1)
        oracle.fold(c, st.indptr, st.fold, wl.channel)
        if rows is None:
            rl = oracle.readout_rows(st.indptr, wl.readout_rows)
            oracle.readout(np.zeros((st.num_rows, 1)), st.num_rows, rl)
        dt = time.perf_counter() - t0
    finally:
        _CPU_JOB.clear()
        if ctx:
            ctx.__exit__(None, None, None)
    eff = np.minimum(np.maximum(st.kv_len.astype(np.int64), 0), wl.capacity())
    if unit == "GB/s":
        work_units = float(sum(eff[l] * 2 * wl.H_kv * wl.d * 2 for l in lanes if n[l] * G <= 32))
        val = work_units / dt / 1e9
        what = f"{len(lanes)} lanes ({len(sample_rows)} rows), decode KV bytes {work_units:.3e}"
    else:
        pairs = attended_pairs(wl)[sample_rows]
        work_units = 4.0 * wl.d * wl.H_q * float(pairs.sum())
        val = work_units / dt / 1e12
        what = f"{len(sample_rows)} sampled rows of {len(lanes)} lanes, {work_units:.3e} algorithmic flop"
    return {"value": val, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{what}; append+attend+fold+readout in {dt:.2f} s, worker start included (fp64 numpy "
                      f"oracle, attention split by lane over {cores} forked processes, BLAS 1 thread each)"}


# --------------------------------------------------------------------------- measured traffic

KERNEL_SOURCES = ("ragged_paged_kv_fp_amd/csrc/fp_lib.hip", "ragged_paged_kv_fp_amd/csrc/fp_kernels.h",
                  "ragged_paged_kv_fp_amd/csrc/fp_decode.h", "ragged_paged_kv_fp_amd/csrc/fp_prefill.h",
                  "ragged_paged_kv_fp_amd/csrc/fp_device.h", "include/fp.h")
TOVA_BUDGET = 2048  # old slots a lane keeps in the timed eviction step
DOMINANT_KERNEL = {2: "decode_kernel", 3: "prefill_kernel", 4: "decode_kernel", 5: "prefill_kernel", 1: "prefill_kernel"}
TRAFFIC_KERNELS = {2: ("merge_kernel", "append_kernel"), 3: ("decode_kernel", "append_kernel"),
                   4: ("merge_kernel",), 5: ("append_kernel",)}


def source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(cfg: int, kernel: str = None) -> str:
    from workloads import CONFIG_NAMES

    return os.path.join(ROOT, "profiles", f"{kernel or DOMINANT_KERNEL[cfg]}_{CONFIG_NAMES[cfg]}_hbm_traffic.txt")


def pmc_summary(fetch_db: str, write_db: str, cfg: int, calib_bytes: int, steps: int) -> list:
    """HBM bytes per step of each library kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch), each counter scaled by what it reads for
    the plain device copy of calib_bytes run in the same process. A kernel with
    several template variants (decode's unmasked and masked launches) counts
    the sum of the variants' per-launch medians: each runs once per step, and
    the median leaves out the untimed prefix pass's one large append. Writes
    one record per kernel of DOMINANT_KERNEL and TRAFFIC_KERNELS for the config."""
    import sqlite3

    def rows_of(db, counter):
        c = sqlite3.connect(db)
        return c.execute("select kernel_name, value from counters_collection where counter_name = ?",
                         (counter,)).fetchall()

    per = {}  # counter -> (scale, copy_kib, {kernel name: [KiB per dispatch]})
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = rows_of(db, counter)
        copies = sorted(v for n, v in rows if "copyBuffer" in n)[-5:]  # the calibration copies are the largest
        calib_kib = float(np.median(copies))
        by = {}
        for n, v in rows:
            if n.startswith("fpk::") or n.startswith("void fpk::"):
                by.setdefault(n, []).append(float(v))
        per[counter] = ((calib_bytes / 1024.0) / calib_kib, calib_kib, by)
    out = []
    for kern in [DOMINANT_KERNEL[cfg]] + [k for k in TRAFFIC_KERNELS.get(cfg, ()) if k != DOMINANT_KERNEL[cfg]]:
        res = {}
        for counter, (scale, calib_kib, by) in per.items():
            variants = {n: v for n, v in by.items() if f"fpk::{kern}<" in n or n.startswith(f"fpk::{kern}(")}
            res[counter] = dict(scale=scale, copy_kib=calib_kib,
                                variants={n: dict(launches=len(v), kib_median=float(np.median(v)),
                                                  kib_min=float(np.min(v)), kib_max=float(np.max(v)))
                                          for n, v in variants.items()},
                                kib_per_step=float(sum(np.median(v) for v in variants.values())))
        traffic = sum(v["kib_per_step"] * v["scale"] * 1024.0 for v in res.values())
        rec = {"kernel": kern, "config": cfg, "source_hash": source_hash(), "calib_copy_bytes": calib_bytes,
               "counters": res, "traffic_bytes_per_step": traffic,
               "command": [f"rocprofv3 --pmc {c} -d <dir> -o c -- python3 bench.py --config {cfg} --no-extra "
                           f"--no-peaks --no-cpu-baseline --steps {steps} --warmup 1 --calib-copy {calib_bytes >> 20}"
                           for c in ("FETCH_SIZE", "WRITE_SIZE")]}
        with open(traffic_file(cfg, kern), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        out.append(rec)
    return out


def trace_summary(db: str, command: str, last: int = 0) -> str:
    """Markdown table of per-kernel durations from a rocprofv3 --kernel-trace
    results db: all launches, and (last > 0) the last `last` launches of each
    kernel by start time, which are the flushed timed steps of bench.py's
    final phase when last = --steps."""
    import sqlite3

    c = sqlite3.connect(db)
    rows = c.execute("select name, start, duration, vgpr_count, lds_size from kernels order by start").fetchall()
    by = {}
    for name, start, dur, vgpr, lds in rows:
        by.setdefault(name, []).append((dur / 1000.0, vgpr, lds))
    head = "| kernel | calls | avg us | min us | max us | total us | VGPRs | LDS B |"
    sep = "|---|---|---|---|---|---|---|---|"
    if last:
        head += f" avg us, last {last} |"
        sep += "---|"
    lines = [f"Command: `{command}`", "", head, sep]
    for name, v in sorted(by.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        d = np.array([x[0] for x in v])
        cell = name.replace("|", "/")[:90]
        line = (f"| `{cell}` | {len(d)} | {d.mean():.2f} | {d.min():.2f} | {d.max():.2f} | {d.sum():.1f} | "
                f"{v[0][1]} | {v[0][2]} |")
        if last:
            line += f" {d[-last:].mean():.2f} |"
        lines.append(line)
    return "\n".join(lines) + "\n"


def measured_traffic(cfg: int, kernel: str = None):
    """Committed counter-based HBM bytes per step of the config's kernel, or
    None if absent or taken on different kernel sources."""
    path = traffic_file(cfg, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return float(rec["traffic_bytes_per_step"])


# --------------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split", type=int, default=None, help="decode KV slots per work item")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="config 2 only: skip configs 5, 3 and 4 and the other seeds")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured read-stream and MFMA peaks")
    ap.add_argument("--no-flush", action="store_true", help="no 1 GiB read between timed steps")
    ap.add_argument("--frame", action="store_true",
                    help="time a two-pass frame (config 3 split per lane) eagerly and as one HIP-graph replay")
    ap.add_argument("--lora", action="store_true",
                    help="time projection-site LoRA (rank 16, 8 adapters, d_in = d_out = 4096) on config 3's rows "
                         "and config 2's rows")
    ap.add_argument("--run-ahead", action="store_true",
                    help="time a repeating speculative decode loop (geometry advanced on the device) eagerly and "
                         "as one HIP-graph replay per pass")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first run 5 plain device copies of MIB MiB (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the measured-traffic record for --config from two rocprofv3 --pmc result dbs")
    ap.add_argument("--trace-summary", nargs=2, metavar=("DB", "COMMAND"),
                    help="print a markdown per-kernel summary of a rocprofv3 --kernel-trace results db "
                         "(with --trace-last N: also the mean of each kernel's last N launches)")
    ap.add_argument("--trace-last", type=int, default=0)
    args = ap.parse_args(argv)
    if args.trace_summary:
        print(trace_summary(*args.trace_summary, last=args.trace_last), end="")
        return 0
    if args.pmc_summary:
        recs = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config, (args.calib_copy or 1024) << 20,
                           args.steps)
        for rec in recs:
            print(json.dumps({"kernel": rec["kernel"], "traffic_bytes_per_step": rec["traffic_bytes_per_step"]}))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        return 2

    import workloads as W

    cpu = None
    pre_wl = None
    if not (args.no_cpu_baseline or args.run_ahead or args.lora or args.frame):
        # the oracle's workers are forked, so this runs before anything touches the GPU
        pre_wl = W.make_config(args.config, seed=args.seed, scale="full")
        unit0 = "TFLOP/s" if args.config == 5 else "GB/s"
        cpu = cpu_baseline(pre_wl, args.config, unit0)
        print(json.dumps({"cpu_baseline": cpu}), file=sys.stderr, flush=True)

    import torch

    from ragged_paged_kv_fp_amd import _lib, runner

    _lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calib_copy:
        nbytes = args.calib_copy << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": nbytes}), file=sys.stderr, flush=True)
        del src, dst
    if args.run_ahead:
        print(json.dumps(run_ahead_bench(W, runner, args.seed, args.steps, args.warmup)), flush=True)
        return 0
    if args.lora:
        print(json.dumps(lora_bench(W, args.seed, args.steps, args.warmup)), flush=True)
        return 0
    if args.frame:
        print(json.dumps(frame_bench(W, runner, args.seed, args.steps, args.warmup)), flush=True)
        return 0
    cfg = args.config
    K, Wm = args.steps, args.warmup
    peaks = None if args.no_peaks else measure_peaks()
    pk_hbm = peaks["hbm_read_GB/s"] if peaks else None
    pk_mfma = peaks["mfma_bf16_TFLOP/s"] if peaks else None
    others, seeds = {}, {}
    if cfg == 2 and not args.no_extra:
        # the other configurations and seeds run first, so that the flushed steps
        # of the main configuration are the last launches of its kernels
        others = extra_configs(W, runner, args.seed, pk_hbm, pk_mfma)
        for sd in (1, 2):
            if sd == args.seed:
                continue
            wls, ws_, rs = measure(W, runner, cfg, sd, args.split, 10, 2, None, flush=not args.no_flush)
            seeds[str(sd)] = round(ws_["kv_bytes_decode"] / (float(np.mean(rs["step_ms"])) * 1e-3) / 1e9, 3)
            del wls
    mass = {}
    wl, w, r = measure(W, runner, cfg, args.seed, args.split, K, Wm, mass, flush=not args.no_flush, wl=pre_wl)
    pre_wl = None
    step_ms = float(np.mean(r["step_ms"]))
    if cfg == 5:
        unit, work_units, scale = "TFLOP/s", w["flops"], 1e12
        bound, peak, r_unit, win, kname = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s", "prefill_ms", "prefill_kernel"
    else:
        unit, work_units, scale = "GB/s", w["kv_bytes_all"] if cfg == 1 else w["kv_bytes_decode"], 1e9
        bound, peak, r_unit = "hbm", HBM_PEAK_GBS, "GB/s"
        win, kname = ("attn_ms", "prefill_kernel") if cfg == 1 else ("decode_ms", "decode_kernel")
    value = work_units / (step_ms * 1e-3) / scale
    achieved = rate(work_units, r[win], scale)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"config {cfg}: " + WORKLOAD_TEXT[cfg], "seed": args.seed,
                   "lanes": wl.num_lanes, "rows": wl.step.num_rows, "kv_bytes_decode": w["kv_bytes_decode"],
                   "attn_flops": w["flops"], "attended_pairs": w["pairs"]},
        "timing": {"protocol": ("per step: untimed 1 GiB read of other data (evicts L2 and MALL) and reset of "
                                "committed_len, then events around append->attend->fold+readout and no marker "
                                "inside; value and ms_per_step are the mean of K such flushed steps; the kernel "
                                "windows come from K other flushed steps with HIP events inside fp_attend "
                                "(step_ms_instrumented), the fp_attend window from K with events around it"
                                if not args.no_flush else "no flush between steps"),
                   "step_ms": _stats(r["step_ms"]),
                   "step_ms_instrumented": _stats(r["step_ms_instrumented"]),
                   "unflushed_ms_per_step": round(r["unflushed_ms_per_step"], 4),
                   "unflushed_value": round(work_units / (r["unflushed_ms_per_step"] * 1e-3) / scale, 3),
                   "host_wall_ms_per_step_unflushed": round(r["host_ms_per_step"], 4)},
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": r_unit,
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(cfg),
                     "kernel": f"{kname}: HIP events recorded by fp_attend around it, per flushed step",
                     "kernel_avg_ms": round(float(np.mean(r[win])), 5), "kernel_ms": _stats(r[win])},
    }
    if peaks:
        line["peaks_measured"] = peaks
        line["roofline"]["measured_peak"] = pk_mfma if bound == "mfma" else pk_hbm
        line["roofline"]["frac_of_measured_peak"] = round(achieved / line["roofline"]["measured_peak"], 4)
    if bound == "hbm" and cfg != 1:
        line["roofline"]["windows"] = decode_windows(w, r, pk_hbm)
    if cfg in (3, 5):
        line["roofline"]["prefill"] = prefill_window(w, r, pk_mfma)
    line["attn_mass"] = {"kernel": "mass_kernel (fp_attn_mass after the step's attention), torch events",
                         "this_config": mass_line(wl, w, mass["ms"], cfg)}
    if "tova_ms" in mass:
        line["tova_step"] = tova_line(wl, mass)
    if others:
        line.update(others)
        line["seeds"] = {str(args.seed): round(value, 3), **seeds}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


def extra_configs(W, runner, seed, pk_hbm, pk_mfma) -> dict:
    """The other measured configurations of the default run: the prefill half of
    the metric on config 5 (long-context masked prefill), config 3 (mixed wave:
    its prefill lanes in TFLOP/s and its decode lanes in GB/s, each on its own
    kernel window) and config 4 (guidance + speculative verify, HBM-bound).
    Each runs 1 warm-up and 5 flushed steps."""
    out = {}
    mass5 = {}
    wl5, w5, r5 = measure(W, runner, 5, seed, None, 5, 1, mass5)
    out["prefill"] = {"workload": "config 5: " + WORKLOAD_TEXT[5], "bound": "mfma", "unit": "TFLOP/s",
                      "peak": BF16_PEAK_TFLOPS, "ms_per_step": round(float(np.mean(r5["step_ms"])), 4),
                      **prefill_window(w5, r5, pk_mfma), "traffic": measured_traffic(5), "steps": 5, "warmup": 1,
                      "attn_mass": mass_line(wl5, w5, mass5["ms"], 5)}
    if "tova_ms" in mass5:
        out["prefill"]["tova_step"] = tova_line(wl5, mass5)
    del wl5
    wl3, w3, r3 = measure(W, runner, 3, seed, None, 5, 1)
    t_pre = w3["flops_prefill"] / (BF16_PEAK_TFLOPS * 1e12) * 1e3
    t_dec = w3["kv_bytes_decode"] / (HBM_PEAK_GBS * 1e9) * 1e3
    t3 = float(np.mean(r3["step_ms"]))
    out["config3"] = {"workload": "config 3: " + WORKLOAD_TEXT[3], "steps": 5, "warmup": 1,
                      "prefill": prefill_window(w3, r3, pk_mfma), "decode": decode_windows(w3, r3, pk_hbm),
                      "step_ms": _stats(r3["step_ms"]),
                      "t_bound_ms": {"prefill_at_peak": round(t_pre, 4), "decode_at_peak": round(t_dec, 4)},
                      "t_bound_over_t_measured": round(max(t_pre, t_dec) / t3, 4),
                      "t_bound_serial_over_t_measured": round((t_pre + t_dec) / t3, 4),
                      "traffic": {"prefill_kernel": measured_traffic(3), "decode_kernel": measured_traffic(3, "decode_kernel")}}
    del wl3
    # a decode wave under a sliding window with sinks: masked decode lanes walk tile lists
    wlw = W.make_window_decode(seed, L=64, kv=32768, window=1024, sinks=4)
    ww, rw = measure(W, runner, None, seed, None, 5, 1, wl=wlw)[1:]
    kvb = 2 * wlw.H_kv * wlw.d * 2  # bytes per slot
    attended = int(attended_pairs(wlw).sum()) * kvb
    tiles = 64 * (len(range(0, 4, 32)) + (1024 + 31) // 32 + 1) * 32 * kvb  # the tiles a lane touches (upper bound)
    gbs = rate(attended, rw["decode_ms"], 1e9)
    out["window_decode"] = {"workload": "64 decode lanes x 1 row at kv_len 32768, window 1024 + 4 sinks bitmaps, "
                                        "H_q=32 H_kv=8 d=128, P=16", "steps": 5, "warmup": 1,
                            "attended_kv_bytes": attended, "kv_bytes_if_unmasked": int(ww["kv_bytes_decode"]),
                            "tile_bytes_upper_bound": tiles,
                            "decode_ms": _stats(rw["decode_ms"]), "decode_merge_ms": _stats(rw["decode_merge_ms"]),
                            "fp_attend_ms": _stats(rw["call_ms"]), "step_ms": _stats(rw["step_ms"]),
                            "GB/s_attended": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del wlw
    wl4, w4, r4 = measure(W, runner, 4, seed, None, 5, 1)
    out["config4"] = {"workload": "config 4: " + WORKLOAD_TEXT[4], "steps": 5, "warmup": 1,
                      "decode": decode_windows(w4, r4, pk_hbm), "step_ms": _stats(r4["step_ms"]),
                      "unflushed_step_ms": round(r4["unflushed_ms_per_step"], 4), "traffic": measured_traffic(4)}
    del wl4
    return out


def run_ahead_bench(W, runner, seed, K, Wm) -> dict:
    """A repeating decode loop at the decode-wave shape (64 lanes, prompts up to
    8192 slots, 32/8 heads, d=128, P=16, each lane drafting 0/1/2/4/8 rows per
    pass and the fold committing a device-channel count), every pass taking
    its geometry from fp_advance. K passes enqueued eagerly (four ABI calls per
    pass) and K as one HIP-graph replay per pass, each after the copies of that
    pass's inputs into the loop's buffers: device and host ms per pass."""
    import torch

    ra = W.make_run_ahead(seed, H_kv=8, G=4, d=128, P=16, num_lanes=64, passes=Wm + K, max_prompt=8192)
    res = {"metric": "run-ahead decode pass (geometry advanced on the device), eager vs HIP-graph replay",
           "config": {"workload": "64 lanes, prompts U{0..8192}, H_q=32 H_kv=8 d=128 P=16, drafts 0/1/2/4/8 rows "
                                  "per lane, channel fold", "rows_per_pass": int(ra.indptr[-1]), "seed": seed},
           "steps": K, "warmup": Wm}
    for mode in ("eager", "graph"):
        lp = runner.RunAheadLoop(ra)
        go = lp.one_pass
        if mode == "graph":
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):  # recording runs nothing: the loop state is unchanged
                lp.one_pass()
            torch.cuda.synchronize()
            go = graph.replay
        for t in range(Wm):
            lp.load(t)
            go()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for t in range(Wm, Wm + K):
            lp.load(t)
            go()
        e1.record()
        h1 = time.perf_counter()
        torch.cuda.synchronize()
        res[mode] = {"device_ms_per_pass": round(e0.elapsed_time(e1) / K, 4),
                     "host_ms_per_pass": round((h1 - h0) * 1e3 / K, 4), "status": int(lp.status.cpu()[0])}
        del lp
    return res


def lora_bench(W, seed, K, Wm) -> dict:
    """fp_adapter_lora at the q projection (d_in = d_out = 4096, rank 16, 8
    adapters, a fifth of the lanes without one), and fp_adapter_ia3 at the
    same site, over the rows of config 3
    (mixed wave) and config 2 (decode wave), inputs resident in HBM, timed with
    torch events over K calls. Algorithmic bytes: x read, y read, out written,
    and each adapter in use read once (A and B); priced against the HBM peak."""
    import torch

    from ragged_paged_kv_fp_amd import api

    res = {"metric": "projection-site LoRA, GB/s of algorithmic HBM bytes (1 GPU)", "unit": "GB/s",
           "peak": HBM_PEAK_GBS, "steps": K, "warmup": Wm, "dtype": "bf16", "data": "synthetic"}
    for cfg in (3, 2):
        wl = W.make_config(cfg, seed=seed, scale="full")
        lw = W.make_lora(seed, wl.step.indptr, d_in=4096, d_out=4096, rank=16, num_adapters=8)
        dev = "cuda"
        bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)  # noqa: E731
        ip = lw.indptr.astype(np.int32)
        geom = api.Geometry(indptr=torch.from_numpy(ip).to(dev), indptr_host=ip.copy(), positions=None, slots=None,
                            kv_len=None, fold=None)
        lora = api.Lora(a=bits(lw.a), b=bits(lw.b), scale=torch.from_numpy(lw.scale).to(dev))
        x, y = bits(lw.x), bits(lw.y)
        out = torch.empty_like(y)
        ws = torch.empty(api.lora_workspace_bytes(geom, lora), dtype=torch.uint8, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        ad = torch.from_numpy(lw.adapter).to(dev)
        call = lambda: api.adapter_lora(geom, lora, ad, x, y, out, ws, status)  # noqa: E731
        for _ in range(Wm):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        N = int(ip[-1])
        used = np.unique(lw.adapter[(lw.adapter >= 0) & (np.diff(ip) > 0)])
        nbytes = N * 4096 * 2 * 3 + len(used) * 16 * (4096 + 4096) * 2
        ach = nbytes / (ms * 1e-3) / 1e9
        # IA3 at the same site: y read, out written, each scale vector in use read once
        sc3 = bits(W.bf16_bits_from_f32(np.random.default_rng(seed).uniform(0.5, 2.0, (8, 4096)).astype(np.float32)))
        call3 = lambda: api.adapter_ia3(geom, sc3, ad, y, out, status)  # noqa: E731
        for _ in range(Wm):
            call3()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            call3()
        e1.record()
        torch.cuda.synchronize()
        ms3 = e0.elapsed_time(e1) / K
        nb3 = N * 4096 * 2 * 2 + len(used) * 4096 * 2
        ach3 = nb3 / (ms3 * 1e-3) / 1e9
        res[f"config{cfg}"] = {"workload": f"rows of config {cfg}: " + WORKLOAD_TEXT[cfg], "rows": N,
                               "adapters_used": int(len(used)), "ms": round(ms, 4), "algorithmic_bytes": nbytes,
                               "achieved": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4),
                               "ia3": {"ms": round(ms3, 4), "algorithmic_bytes": nb3, "achieved": round(ach3, 1),
                                       "frac": round(ach3 / HBM_PEAK_GBS, 4)},
                               "status": int(status.cpu()[0])}
    return res


def frame_bench(W, runner, seed, K, Wm) -> dict:
    """A frame of two passes (config 3 with each lane's rows split at a random
    point: prefix pass folded all, then the continuation) submitted K times
    eagerly (six ABI calls per frame from the host) and K times as one HIP
    graph replay: device ms per frame from torch events and host ms per frame."""
    import torch

    wl = W.make_config(3, seed=seed, scale="full")
    rng = np.random.default_rng(seed)
    first = np.array([int(rng.integers(0, m + 1)) for m in np.diff(wl.step.indptr)])
    A, B = W.split_pass(wl.step, first)
    ds = runner.DeviceStep(wl, device="cuda")
    ds.run_prefix()
    frames = {"eager": runner.Frame(ds.pool, [A, B], wl.H_q, wl.theta, wl.sm_scale),
              "vertical": runner.Frame(ds.pool, [A, B], wl.H_q, wl.theta, wl.sm_scale, vertical=True)}
    frames["graph"] = frames["eager"]
    frames["vertical_graph"] = frames["vertical"]
    assert len(frames["vertical"].items) == 1
    res = {}
    for mode in ("eager", "graph", "vertical", "vertical_graph"):
        fr = frames[mode]
        go = fr.replay if mode.endswith("graph") else fr.run
        if mode.endswith("graph"):
            fr.capture()
        for _ in range(Wm):
            go()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for _ in range(K):
            go()
        e1.record()
        h1 = time.perf_counter()
        torch.cuda.synchronize()
        res[mode] = {"device_ms_per_frame": round(e0.elapsed_time(e1) / K, 4),
                     "host_ms_per_frame": round((h1 - h0) * 1e3 / K, 4)}
    st = int(frames["eager"].status.cpu()[0]) | int(frames["vertical"].status.cpu()[0])
    return {"metric": "two-pass frame (prefix pass + continuation): eager and one HIP-graph replay, each as two "
                      "passes and vertically batched into one pass (fp_vertical_merge)",
            "config": {"workload": "config 3 split per lane at a random row: " + WORKLOAD_TEXT[3], "seed": seed,
                       "rows": [A.num_rows, B.num_rows]},
            "steps": K, "warmup": Wm, "status": st, **res}


def tova_line(wl, mass) -> dict:
    """The timed eviction step: bytes are the fp32 mass it reads (every old slot,
    every KV head) plus the bitmap words it writes."""
    gbs = mass["tova_bytes"] / (mass["tova_ms"] * 1e-3) / 1e9
    return {"what": f"fp_tova_mask from this pass's attention mass: keep {TOVA_BUDGET} of each lane's "
                    f"{mass['tova_old_slots'] // wl.num_lanes} old slots (fp32 mass summed over {wl.H_kv} KV heads, "
                    "radix select), then write the pass's row bitmaps",
            "ms": round(mass["tova_ms"], 4), "bytes": mass["tova_bytes"], "GB/s": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def mass_line(wl, w, ms, cfg) -> dict:
    """Roofline of fp_attn_mass: decode-class lanes read each slot's K once
    (HBM-bound: kv_len x H_kv x d x 2 B); prefill lanes run Q.K over every
    attended pair (MFMA-bound: 2 d flops per pair and query head)."""
    k_bytes = w["kv_bytes_decode"] // 2
    qk_flops = w["flops"] / 2.0
    if cfg == 5:
        ach = qk_flops / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "bound": "mfma", "unit": "TFLOP/s", "achieved": round(ach, 2),
                "peak": BF16_PEAK_TFLOPS, "frac": round(ach / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": qk_flops}
    ach = k_bytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "bound": "hbm", "unit": "GB/s", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": k_bytes}


FLUSH_BYTES = 1 << 30  # read before every flushed step: L2 (8 x 4 MB) and the 256 MB MALL then hold none of its inputs


class Flusher:
    """Evicts the caches between timed steps by reading FLUSH_BYTES of other
    data with the read-stream kernel of libfp_peaks.so (a read leaves no dirty
    lines whose write-back could overlap the next step)."""

    def __init__(self):
        import ctypes

        import torch

        from ragged_paged_kv_fp_amd import build

        if not os.path.exists(build.PEAKS_LIB):
            raise ImportError(f"{build.PEAKS_LIB} is missing: build it with __graft_entry__.build()")
        self.lib = ctypes.CDLL(build.PEAKS_LIB)
        self.lib.fp_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p]
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(256, dtype=torch.int32, device="cuda")
        self.blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count

    def __call__(self, stream):
        rc = self.lib.fp_peak_read(self.buf.data_ptr(), FLUSH_BYTES, self.blocks, self.sink.data_ptr(),
                                   stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"flush read failed: {rc}")


def _stats(xs) -> dict:
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "min": round(float(a.min()), 5), "max": round(float(a.max()), 5)}


def measure(W, runner, cfg, seed, split, K, Wm, mass=None, flush=True, wl=None):
    """Time one configuration with inputs resident in HBM.

    Phase 1 (unflushed): Wm warm-up steps, then K steps back to back between
    two events; gives the back-to-back rate.
    Phases 2-4 are flushed: Wm warm-up steps, then K steps per phase, each
    after an untimed 1 GiB read of other data that evicts L2 and the MALL and
    the untimed reset of committed_len. An event a pass enqueues is a marker
    that adds a few microseconds to the pass, so each window is timed in steps
    that hold only its own markers:
    Phase 2 (the kernel windows): HIP events the library records inside
    fp_attend split it into the prefill kernel, the decode kernel and the
    split merge; events at the step's ends give step_ms_instrumented.
    Phase 3 (the fp_attend window): events around the fp_attend call only.
    Phase 4 (the step time that value and ms_per_step report): events at the
    two ends of the step (append -> attend -> fold + readout) only.
    Every phase is bracketed by torch.cuda.synchronize(). Returns
    (workload, work, dict of per-step millisecond lists and phase-1 totals)."""
    import torch

    print(f"[bench] config {cfg if wl is None else wl.name} seed {seed}: {K} steps after {Wm} warm-ups", file=sys.stderr,
          flush=True)
    if wl is None:
        wl = W.make_config(cfg, seed=seed, scale="full")
    w = work(wl)
    ds = runner.DeviceStep(wl, device="cuda", split=split)
    ds.run_prefix()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = HipEvents()
    hip_ev = [tuple(ev.create() for _ in range(4)) for _ in range(K)]  # begin, end, prefill_end, merge_end
    tev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # ---- phase 1: back to back
    for _ in range(Wm):
        ds.reset()
        ds.step()
    torch.cuda.synchronize()
    b0, b1 = tev(), tev()
    h0 = time.perf_counter()
    b0.record(stream)
    for _ in range(K):
        ds.reset()
        ds.step()
    b1.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    res = {"unflushed_ms_per_step": b0.elapsed_time(b1) / K, "host_ms_per_step": (h1 - h0) * 1e3 / K}
    # ---- phase 2: flushed steps with per-step windows
    flusher = Flusher() if flush else None
    step_ev = [(tev(), tev(), tev(), tev()) for _ in range(K)]  # step begin, call begin, call end, step end
    for i in range(Wm):
        if flusher is not None:
            flusher(stream)
        ds.reset()
        ds.step()
    torch.cuda.synchronize()
    ds.status.zero_()
    torch.cuda.synchronize()
    for i in range(K):
        if flusher is not None:
            flusher(stream)
        sb, _, _, se = step_ev[i]
        ds.reset()  # replay state, not part of the pass
        sb.record(stream)
        ds.append()
        ds.attend(events=hip_ev[i])
        ds.finish()
        se.record(stream)
    torch.cuda.synchronize()
    res["step_ms_instrumented"] = [sb.elapsed_time(se) for sb, _, _, se in step_ev]
    # ---- phase 3: the fp_attend call alone between two events
    for i in range(K):
        if flusher is not None:
            flusher(stream)
        _, cb, ce, _ = step_ev[i]
        ds.reset()
        ds.append()
        cb.record(stream)
        ds.attend()
        ce.record(stream)
        ds.finish()
    torch.cuda.synchronize()
    res["call_ms"] = [cb.elapsed_time(ce) for _, cb, ce, _ in step_ev]
    # ---- phase 4: the step timed at its two ends only
    plain_ev = [(tev(), tev()) for _ in range(K)]
    for i in range(K):
        if flusher is not None:
            flusher(stream)
        sb, se = plain_ev[i]
        ds.reset()  # replay state, not part of the pass
        sb.record(stream)
        ds.append()
        ds.attend()
        ds.finish()
        se.record(stream)
    torch.cuda.synchronize()
    res["step_ms"] = [sb.elapsed_time(se) for sb, se in plain_ev]
    res["attn_ms"] = [ev.elapsed_ms(b, e) for b, e, _, _ in hip_ev]
    res["prefill_ms"] = [ev.elapsed_ms(b, p) for b, _, p, _ in hip_ev]
    res["decode_ms"] = [ev.elapsed_ms(p, e) for _, e, p, _ in hip_ev]
    res["decode_merge_ms"] = [ev.elapsed_ms(p, m) for _, _, p, m in hip_ev]  # decode kernel + split merge
    status = int(ds.status.cpu()[0])
    if status != 0:
        print(f"warning: device status {status} (config {cfg})", file=sys.stderr)
    del flusher
    if mass is not None:
        from ragged_paged_kv_fp_amd import api

        buf = torch.zeros((wl.H_kv, int(wl.page_indptr[-1]) * wl.P), dtype=torch.float32, device="cuda")
        call = lambda: api.attn_mass(ds.pool, ds.geom, wl.H_q, ds.lse, ds.workspace, buf, ds.mask, split)  # noqa: E731
        for _ in range(Wm):
            call()
        torch.cuda.synchronize()
        m0, m1 = tev(), tev()
        m0.record(stream)
        for _ in range(K):
            call()
        m1.record(stream)
        torch.cuda.synchronize()
        mass["ms"] = m0.elapsed_time(m1) / K
        if ds.mask is not None:
            # score-driven eviction from this mass: re-mask the same pass (rows at
            # committed_len..) keeping tova_budget old slots per lane
            ds.reset()
            L = wl.num_lanes
            cap = np.diff(wl.page_indptr) * wl.P
            koff = np.concatenate([[0], np.cumsum((cap + 31) // 32)]).astype(np.int64)
            keep = torch.zeros(int(koff[-1]), dtype=torch.int32, device="cuda")
            koff_t = torch.from_numpy(koff).cuda()
            bits = torch.zeros_like(ds.mask.bits)
            tmask = api.Mask(bits=bits, word_offset=ds.mask.word_offset, word_offset_host=ds.mask.word_offset_host)
            budget = torch.full((L,), TOVA_BUDGET, dtype=torch.int32, device="cuda")
            st = torch.zeros(1, dtype=torch.int32, device="cuda")
            tcall = lambda: api.tova_mask(ds.pool, ds.geom, buf, budget, koff_t, keep, tmask, st)  # noqa: E731
            for _ in range(Wm):
                tcall()
            torch.cuda.synchronize()
            m0.record(stream)
            for _ in range(K):
                tcall()
            m1.record(stream)
            torch.cuda.synchronize()
            c0 = ds.committed0.cpu().numpy().astype(np.int64)
            mass["tova_ms"] = m0.elapsed_time(m1) / K
            mass["tova_bytes"] = int(c0.sum() * wl.H_kv * 4 + ds.mask.bits.numel() * 4)
            mass["tova_old_slots"] = int(c0.sum())
            del keep, bits
        del buf
    for evs in hip_ev:
        for e in evs:
            ev.destroy(e)
    del ds
    torch.cuda.empty_cache()
    return wl, w, res


def rate(units: float, ms_list, scale: float) -> float:
    return units / (float(np.mean(ms_list)) * 1e-3) / scale


def decode_windows(w, r, peak_meas=None) -> dict:
    """HBM-bound decode figures of one measurement: algorithmic KV bytes of the
    decode-class lanes over the decode kernel alone, decode + split merge
    (the split-KV decode with its reduction), the whole fp_attend call (plan,
    Q rotation, tile lists, attention, merge) and the whole step."""
    b = w["kv_bytes_decode"]
    out = {}
    for name, key in (("decode_kernel", "decode_ms"), ("decode_plus_merge", "decode_merge_ms"), ("fp_attend", "call_ms"),
                      ("step", "step_ms")):
        gbs = rate(b, r[key], 1e9)
        out[name] = {"ms": _stats(r[key]), "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if peak_meas:
            out[name]["frac_of_measured_peak"] = round(gbs / peak_meas, 4)
    return out


def prefill_window(w, r, peak_meas=None) -> dict:
    """MFMA-bound prefill figures: algorithmic flops (allowed pairs only) and
    executed flops (every 32-slot tile a work item visits) over the prefill kernel."""
    alg = rate(w["flops_prefill"], r["prefill_ms"], 1e12)
    exe = rate(w["flops_prefill_executed"], r["prefill_ms"], 1e12)
    out = {"ms": _stats(r["prefill_ms"]), "TFLOP/s": round(alg, 2), "frac": round(alg / BF16_PEAK_TFLOPS, 4),
           "TFLOP/s_executed": round(exe, 2), "frac_executed": round(exe / BF16_PEAK_TFLOPS, 4),
           "algorithmic_flops": w["flops_prefill"], "executed_flops": w["flops_prefill_executed"]}
    if peak_meas:
        out["frac_of_measured_peak"] = round(alg / peak_meas, 4)
    return out


# --------------------------------------------------------------------------- measured peaks

def measure_peaks(reps: int = 10) -> dict:
    """The device's own peaks from libfp_peaks.so: a read-only stream of 4 GiB
    (16-byte non-temporal loads, contiguous chunks per workgroup) and a loop of
    independent v_mfma_f32_32x32x16_bf16 chains on every SIMD, each timed with
    events on the launch stream; best of `reps` launches."""
    import ctypes

    import torch

    from ragged_paged_kv_fp_amd import build

    if not os.path.exists(build.PEAKS_LIB):
        raise ImportError(f"{build.PEAKS_LIB} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(build.PEAKS_LIB)
    lib.fp_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.fp_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.fp_peak_mfma_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.fp_peak_mfma_flop.restype = ctypes.c_double
    stream = torch.cuda.current_stream()
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(fn):
        best = float("inf")
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn()
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"peak kernel launch failed: {rc}")
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    read_ms = timed(lambda: lib.fp_peak_read(buf.data_ptr(), nbytes, 8 * cus, sink.data_ptr(), stream.cuda_stream))
    del buf
    iters, blocks = 4096, 2 * cus  # eight waves per CU, two per SIMD
    mfma_ms = timed(lambda: lib.fp_peak_mfma(iters, blocks, sink.data_ptr(), stream.cuda_stream))
    gbs = nbytes / (read_ms * 1e-3) / 1e9
    tf = lib.fp_peak_mfma_flop(iters, blocks) / (mfma_ms * 1e-3) / 1e12
    torch.cuda.empty_cache()
    return {"hbm_read_GB/s": round(gbs, 1), "hbm_frac_of_vendor": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_bf16_TFLOP/s": round(tf, 1), "mfma_frac_of_vendor": round(tf / BF16_PEAK_TFLOPS, 4),
            "read_ms": round(read_ms, 4), "mfma_ms": round(mfma_ms, 4), "reps": reps,
            "how": "libfp_peaks.so: 4 GiB read stream (16-byte non-temporal loads, contiguous chunks), "
                   "4 chains of v_mfma_f32_32x32x16_bf16 per wave on 2 waves/SIMD; best of reps"}


if __name__ == "__main__":
    sys.exit(main())
