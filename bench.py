#!/usr/bin/env python3
"""Benchmark of the ForwardPass attention step on one MI355X.

A step is one whole pass through the four ABI calls (append -> attend ->
fold -> readout) over one batch of synthetic input that is already resident
in HBM, plus the reset of committed_len that makes the step replayable.

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

def cpu_baseline(wl, cfg: int, unit: str, budget_s: float = 20.0):
    """Time the fp64 oracle on a bounded sample of the same step, one host thread."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    st = wl.step
    n = np.diff(st.indptr).astype(np.int64)
    order = [l for l in range(wl.num_lanes) if n[l] > 0]
    G = wl.H_q // wl.H_kv
    # bounded sample: whole lanes for decode-class work, sampled rows of prefill lanes
    if cfg in (1, 2, 4):
        lanes, rows = order, None
    else:
        rng = np.random.default_rng(7)
        lanes = sorted(rng.choice(order, size=min(4, len(order)), replace=False).tolist())
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
        t0 = time.perf_counter()
        oracle.append(pool, c, st.indptr, st.positions, st.slots, st.k, st.v, wl.theta, lanes=lanes)
        sample_rows = rows if rows is not None else np.concatenate(
            [np.arange(st.indptr[l], st.indptr[l + 1]) for l in lanes]).astype(np.int64)
        O, LSE, _ = oracle.attend(pool, st.indptr, st.positions, st.slots, st.kv_len, st.q, wl.H_q, wl.theta,
                                  wl.sm_scale, wl.mask_bits, wl.mask_word_offset, rows=sample_rows)
        oracle.fold(c, st.indptr, st.fold, wl.channel)
        if rows is None:
            rl = oracle.readout_rows(st.indptr, wl.readout_rows)
            oracle.readout(np.zeros((st.num_rows, 1)), st.num_rows, rl)
        dt = time.perf_counter() - t0
    finally:
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
    return {"value": val, "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{what}; append+attend+fold+readout in {dt:.2f} s (fp64 numpy, one thread)"}


# --------------------------------------------------------------------------- measured traffic

KERNEL_SOURCES = ("ragged_paged_kv_fp_amd/csrc/fp_lib.hip", "ragged_paged_kv_fp_amd/csrc/fp_kernels.h",
                  "ragged_paged_kv_fp_amd/csrc/fp_decode.h", "ragged_paged_kv_fp_amd/csrc/fp_prefill.h",
                  "ragged_paged_kv_fp_amd/csrc/fp_device.h", "include/fp.h")
DOMINANT_KERNEL = {2: "decode_kernel", 3: "prefill_kernel", 4: "decode_kernel", 5: "prefill_kernel", 1: "prefill_kernel"}


def source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(cfg: int) -> str:
    return os.path.join(ROOT, "profiles", f"{DOMINANT_KERNEL[cfg]}_config{cfg}_hbm_traffic.txt")


def pmc_summary(fetch_db: str, write_db: str, cfg: int, calib_bytes: int, out: str) -> dict:
    """Per-launch HBM bytes of the dominant kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch), each scaled by what the same counter
    reads for the plain device copy of calib_bytes run in the same process."""
    import sqlite3

    def per_kernel(db, counter):
        c = sqlite3.connect(db)
        rows = c.execute("select kernel_name, value from counters_collection where counter_name = ?",
                         (counter,)).fetchall()
        return rows

    kern = DOMINANT_KERNEL[cfg]
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = per_kernel(db, counter)
        copies = [v for n, v in rows if "copyBuffer" in n]
        kvals = [v for n, v in rows if f"fpk::{kern}<" in n]  # exact kernel (not mass_decode_kernel)
        # the calibration copies are the largest copy dispatches of the run
        copies = sorted(copies)[-5:]
        calib_kib = float(np.median(copies))
        scale = (calib_bytes / 1024.0) / calib_kib
        res[counter] = dict(kernel_kib=float(np.mean(kvals)), launches=len(kvals), copy_kib=calib_kib, scale=scale)
    traffic = sum(v["kernel_kib"] * v["scale"] * 1024.0 for v in res.values())
    rec = {"kernel": kern, "config": cfg, "source_hash": source_hash(), "calib_copy_bytes": calib_bytes,
           "counters": res, "traffic_bytes_per_launch": traffic,
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -d <dir> -o c -- python3 bench.py "
                      f"--config {cfg} --no-cpu-baseline --steps 5 --warmup 1 --calib-copy {calib_bytes >> 20}"}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def trace_summary(db: str, command: str) -> str:
    """Markdown table of per-kernel durations from a rocprofv3 --kernel-trace results db."""
    import sqlite3

    c = sqlite3.connect(db)
    q = ("select name, count(*), avg(duration)/1000.0, min(duration)/1000.0, max(duration)/1000.0, "
         "sum(duration)/1000.0 from kernels group by name order by sum(duration) desc")
    lines = [f"Command: `{command}`", "",
             "| kernel | calls | avg us | min us | max us | total us |", "|---|---|---|---|---|---|"]
    for name, n, avg, mn, mx, tot in c.execute(q):
        name = name.replace("|", "/")
        lines.append(f"| `{name[:90]}` | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {tot:.1f} |")
    return "\n".join(lines) + "\n"


def measured_traffic(cfg: int):
    """Committed counter-based traffic for this config, or None if absent or
    taken on different kernel sources."""
    path = traffic_file(cfg)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return float(rec["traffic_bytes_per_launch"])


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
    ap.add_argument("--no-prefill", action="store_true", help="config 2 only: skip the config 5 prefill measurement")
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
                    help="print a markdown per-kernel summary of a rocprofv3 --kernel-trace results db")
    args = ap.parse_args(argv)
    if args.trace_summary:
        print(trace_summary(*args.trace_summary), end="")
        return 0
    if args.pmc_summary:
        rec = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config, (args.calib_copy or 1024) << 20,
                          traffic_file(args.config))
        print(json.dumps(rec))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import workloads as W
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
    mass = {}
    wl, w, ms_step, attn_avg, host_ms = measure(W, runner, cfg, args.seed, args.split, args.steps, args.warmup, mass)
    K, Wm = args.steps, args.warmup
    if cfg == 5:
        unit, work_units, scale = "TFLOP/s", w["flops"], 1e12
        bound, peak, r_unit = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        unit, work_units, scale = "GB/s", w["kv_bytes_all"] if cfg == 1 else w["kv_bytes_decode"], 1e9
        bound, peak, r_unit = "hbm", HBM_PEAK_GBS, "GB/s"
        if cfg == 3:
            work_units = w["kv_bytes_decode"]
    value = work_units / (ms_step * 1e-3) / scale
    achieved = work_units / (attn_avg * 1e-3) / scale
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"config {cfg}: " + WORKLOAD_TEXT[cfg], "seed": args.seed,
                   "lanes": wl.num_lanes, "rows": wl.step.num_rows, "kv_bytes_decode": w["kv_bytes_decode"],
                   "attn_flops": w["flops"], "attended_pairs": w["pairs"], "host_wall_ms_per_step":
                   round(host_ms, 4)},
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": r_unit,
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(cfg),
                     "kernel": "attention kernels (decode_kernel / prefill_kernel), HIP events per step",
                     "kernel_avg_ms": round(attn_avg, 5)},
    }
    line["attn_mass"] = {"kernel": "mass_kernel (fp_attn_mass after the step's attention), torch events",
                         "this_config": mass_line(wl, w, mass["ms"], cfg)}
    if cfg == 3:
        line["config"]["prefill_tflops_step"] = round(w["flops_prefill"] / (ms_step * 1e-3) / 1e12, 3)
    if cfg == 5:
        line["roofline"]["executed_frac"] = round(w["flops_prefill_executed"] / (attn_avg * 1e-3) / 1e12 / peak, 4)
    if cfg == 2 and not args.no_prefill:
        # the prefill half of the metric, on the long-context masked prefill wave
        mass5 = {}
        wl5, w5, ms5, attn5, _ = measure(W, runner, 5, args.seed, None, 5, 1, mass5)
        alg = w5["flops"] / (attn5 * 1e-3) / 1e12
        exe = w5["flops_prefill_executed"] / (attn5 * 1e-3) / 1e12
        line["prefill"] = {"workload": "config 5: " + WORKLOAD_TEXT[5], "bound": "mfma", "unit": "TFLOP/s",
                           "peak": BF16_PEAK_TFLOPS, "attn_ms": round(attn5, 4), "ms_per_step": round(ms5, 4),
                           "achieved": round(alg, 2), "frac": round(alg / BF16_PEAK_TFLOPS, 4),
                           "achieved_executed": round(exe, 2), "frac_executed": round(exe / BF16_PEAK_TFLOPS, 4),
                           "algorithmic_flops": w5["flops"], "executed_flops": w5["flops_prefill_executed"],
                           "traffic": measured_traffic(5), "steps": 5, "warmup": 1}
        line["attn_mass"]["prefill"] = mass_line(wl5, w5, mass5["ms"], 5)
        del wl5
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, cfg, unit)
    print(json.dumps(line), flush=True)
    return 0


def run_ahead_bench(W, runner, seed, K, Wm) -> dict:
    """A repeating decode loop at the decode-wave shape (64 lanes, prompts up to
    8192 slots, 32/8 heads, d=128, P=16, each lane drafting 0/1/2/4/8 rows per
    pass and the fold committing a device-channel count), every pass taking
    its geometry from fp_advance. K passes enqueued eagerly (five ABI calls per
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
    eagerly (eight ABI calls per frame from the host) and K times as one HIP
    graph replay: device ms per frame from torch events and host ms per frame."""
    import torch

    wl = W.make_config(3, seed=seed, scale="full")
    rng = np.random.default_rng(seed)
    first = np.array([int(rng.integers(0, m + 1)) for m in np.diff(wl.step.indptr)])
    A, B = W.split_pass(wl.step, first)
    ds = runner.DeviceStep(wl, device="cuda")
    ds.run_prefix()
    fr = runner.Frame(ds.pool, [A, B], wl.H_q, wl.theta, wl.sm_scale)
    res = {}
    for mode in ("eager", "graph"):
        go = fr.run if mode == "eager" else fr.replay
        if mode == "graph":
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
    st = int(fr.status.cpu()[0])
    return {"metric": "two-pass frame (prefix pass + continuation), eager vs one HIP-graph replay",
            "config": {"workload": "config 3 split per lane at a random row: " + WORKLOAD_TEXT[3], "seed": seed,
                       "rows": [A.num_rows, B.num_rows]},
            "steps": K, "warmup": Wm, "status": st, **res}


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


def measure(W, runner, cfg, seed, split, K, Wm, mass=None):
    """Time K steps (after Wm warm-ups) of one configuration with inputs resident
    in HBM: returns (workload, work, ms per step, attention-kernel ms per step
    from HIP events on the launch stream, host wall ms per step). With a dict
    as `mass`, also times K calls of fp_attn_mass over the last step's
    attention (torch events on the stream it runs on) into mass["ms"]."""
    import torch

    wl = W.make_config(cfg, seed=seed, scale="full")
    w = work(wl)
    ds = runner.DeviceStep(wl, device="cuda", split=split)
    ds.run_prefix()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = HipEvents()
    pairs_ev = [(ev.create(), ev.create()) for _ in range(K)]
    for _ in range(Wm):
        ds.reset()
        ds.step()
    torch.cuda.synchronize()
    ds.status.zero_()
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    t_begin.record(stream)
    for i in range(K):
        ds.reset()
        ds.step(events=pairs_ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    total_ms = t_begin.elapsed_time(t_end)
    attn_ms = [ev.elapsed_ms(a, b) for a, b in pairs_ev]
    status = int(ds.status.cpu()[0])
    if status != 0:
        print(f"warning: device status {status} (config {cfg})", file=sys.stderr)
    if mass is not None:
        from ragged_paged_kv_fp_amd import api

        buf = torch.zeros((wl.H_kv, int(wl.page_indptr[-1]) * wl.P), dtype=torch.float32, device="cuda")
        call = lambda: api.attn_mass(ds.pool, ds.geom, wl.H_q, ds.lse, ds.workspace, buf, ds.mask, split)  # noqa: E731
        for _ in range(Wm):
            call()
        torch.cuda.synchronize()
        m0 = torch.cuda.Event(enable_timing=True)
        m1 = torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for _ in range(K):
            call()
        m1.record(stream)
        torch.cuda.synchronize()
        mass["ms"] = m0.elapsed_time(m1) / K
        del buf
    for a, b in pairs_ev:
        ev.destroy(a)
        ev.destroy(b)
    del ds
    torch.cuda.empty_cache()
    return wl, w, total_ms / K, float(np.mean(attn_ms)), (h1 - h0) * 1e3 / K


if __name__ == "__main__":
    sys.exit(main())
