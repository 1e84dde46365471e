"""Seeded synthetic workloads shaped like the Pie ForwardPass attention step.

Every array here is an *input*: row offsets, slots, positions, page tables,
mask bitmaps, device-channel counts and bf16 bit patterns of Q/K/V. The
method's arithmetic (RoPE, attention, fold, readout) lives elsewhere.

Workload shapes follow the five configurations of the hot path:
  1  one lane, 37-token prompt, GQA 4/2, d=64, 3 shuffled pages of 16
  2  decode wave: 64 lanes x 1 row, kv_len ~ U{512..8192}, 32/8 heads, d=128, P=16
  3  mixed wave: 8 prefill lanes (1024-4096 rows on 0-2048 cached slots)
     plus 120 decode lanes (kv_len 256-16384), P=32
  4  guidance pairs (cond prefix 2048, uncond prefix 512) plus 32 speculative
     verify lanes of 8 draft rows whose fold count comes from a device channel
  5  16 lanes x 512-row chunks over kv_len 32768 with non-contiguous positions,
     sliding-window+sink masks on half the lanes, TOVA-style random drops on the rest

Random streams are child seeds of one SeedSequence, drawn in a fixed order
(lengths, permutation, prefix K/V, Q, K, V, mask, channel), so a workload is a
pure function of (config, seed, scale).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# Fold sentinels of the C ABI (a literal count is any value >= 0).
FOLD_ALL = -1
FOLD_CHANNEL = -2

CONFIG_NAMES = {
    1: "single_lane_gqa_37",
    2: "decode_wave_64",
    3: "mixed_prefill_decode_128",
    4: "guidance_spec_verify_48",
    5: "long_context_masks_16",
}

_STREAMS = ("lengths", "perm", "prefix_kv", "q", "k", "v", "mask", "channel")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 samples to bf16 (nearest-even); returns uint16 bit patterns.

    Finite floats stay below 0x7F800000 in magnitude bits, so the 32-bit sum
    below cannot carry out of the word.
    """
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 1 << 14) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, generated in row chunks to bound memory."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if out.size == 0:
        return out
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0,) + shape[1:], dtype=np.float32))
    return out


@dataclass
class Pass:
    """One ForwardPass worth of rows (concatenated by lane, offsets in indptr)."""

    indptr: np.ndarray      # int32 [L+1]
    positions: np.ndarray   # int32 [N]
    slots: np.ndarray       # int32 [N]
    kv_len: np.ndarray      # int32 [L]
    fold: np.ndarray        # int32 [L]: >=0 literal, FOLD_ALL, FOLD_CHANNEL
    k: np.ndarray           # uint16 bf16 bits [N][H_kv][d]
    v: np.ndarray           # uint16 bf16 bits [N][H_kv][d]
    q: Optional[np.ndarray] = None  # uint16 bf16 bits [N][H_q][d]

    @property
    def num_lanes(self) -> int:
        return int(self.indptr.shape[0] - 1)

    @property
    def num_rows(self) -> int:
        return int(self.indptr[-1])


@dataclass
class Workload:
    name: str
    H_q: int
    H_kv: int
    d: int
    P: int
    theta: float
    sm_scale: float
    num_pages: int
    page_indptr: np.ndarray          # int32 [L+1]
    page_ids: np.ndarray             # int32 [page_indptr[-1]]
    prefix: Optional[Pass]           # appended and folded (all) before the step
    step: Pass
    mask_bits: Optional[np.ndarray] = None         # uint32 words
    mask_word_offset: Optional[np.ndarray] = None  # int64 [L+1]
    channel: Optional[np.ndarray] = None           # int32 [L]
    readout_rows: Optional[np.ndarray] = None      # int32 list of global rows; None = default
    meta: dict = field(default_factory=dict)

    @property
    def num_lanes(self) -> int:
        return self.step.num_lanes

    def capacity(self) -> np.ndarray:
        return (np.diff(self.page_indptr).astype(np.int64) * self.P).astype(np.int64)


def _rngs(seed: int):
    ss = np.random.SeedSequence(int(seed))
    kids = ss.spawn(len(_STREAMS))
    return {name: np.random.default_rng(kid) for name, kid in zip(_STREAMS, kids)}


def _assemble(
    name: str,
    rngs,
    *,
    H_q: int,
    H_kv: int,
    d: int,
    P: int,
    lanes: List[dict],
    theta: float = 10000.0,
    shuffle_lanes: bool = True,
    extra_pages: int = 0,
    mask_fn=None,
    readout_fn=None,
    channel_fn=None,
) -> Workload:
    """Lay out lanes into a paged pool.

    Each lane dict holds: c (cached prefix length), n (rows this pass), kv_len,
    fold, pos_of_slot (int64 array over all slots the lane uses) and optional
    'slots' (default c..c+n-1), 'pages' (default ceil(kv_len/P)).
    """
    L = len(lanes)
    order = rngs["perm"].permutation(L) if shuffle_lanes and L > 1 else np.arange(L)
    lanes = [lanes[i] for i in order]

    pages = np.array([int(ln.get("pages", -(-max(ln["kv_len"], 1) // P))) for ln in lanes], dtype=np.int64)
    page_indptr = np.zeros(L + 1, dtype=np.int64)
    page_indptr[1:] = np.cumsum(pages)
    num_pages = int(page_indptr[-1]) + int(extra_pages)
    perm = rngs["perm"].permutation(num_pages).astype(np.int32)
    page_ids = perm[: int(page_indptr[-1])].copy()

    # Prefix pass: slots 0..c-1 of each lane at their positions, folded all.
    pre_counts = np.array([ln["c"] for ln in lanes], dtype=np.int64)
    pre_indptr = np.zeros(L + 1, dtype=np.int64)
    pre_indptr[1:] = np.cumsum(pre_counts)
    Np = int(pre_indptr[-1])
    pre_slots = np.concatenate([np.arange(ln["c"], dtype=np.int64) for ln in lanes]) if Np else np.zeros(0, np.int64)
    pre_pos = np.concatenate([ln["pos_of_slot"][: ln["c"]] for ln in lanes]) if Np else np.zeros(0, np.int64)
    pre_k = _normal_bf16(rngs["prefix_kv"], (Np, H_kv, d))
    pre_v = _normal_bf16(rngs["prefix_kv"], (Np, H_kv, d))
    prefix = None
    if Np:
        prefix = Pass(
            indptr=pre_indptr.astype(np.int32),
            positions=pre_pos.astype(np.int32),
            slots=pre_slots.astype(np.int32),
            kv_len=pre_counts.astype(np.int32),
            fold=np.full(L, FOLD_ALL, dtype=np.int32),
            k=pre_k,
            v=pre_v,
        )

    counts = np.array([ln["n"] for ln in lanes], dtype=np.int64)
    indptr = np.zeros(L + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(counts)
    N = int(indptr[-1])
    slot_list, pos_list = [], []
    for ln in lanes:
        s = np.asarray(ln.get("slots", np.arange(ln["c"], ln["c"] + ln["n"])), dtype=np.int64)
        slot_list.append(s)
        pos_list.append(ln["pos_of_slot"][s] if len(s) else np.zeros(0, np.int64))
    slots = np.concatenate(slot_list) if N else np.zeros(0, np.int64)
    positions = np.concatenate(pos_list) if N else np.zeros(0, np.int64)
    q = _normal_bf16(rngs["q"], (N, H_q, d))
    k = _normal_bf16(rngs["k"], (N, H_kv, d))
    v = _normal_bf16(rngs["v"], (N, H_kv, d))
    step = Pass(
        indptr=indptr.astype(np.int32),
        positions=positions.astype(np.int32),
        slots=slots.astype(np.int32),
        kv_len=np.array([ln["kv_len"] for ln in lanes], dtype=np.int32),
        fold=np.array([ln["fold"] for ln in lanes], dtype=np.int32),
        k=k,
        v=v,
        q=q,
    )

    wl = Workload(
        name=name,
        H_q=H_q,
        H_kv=H_kv,
        d=d,
        P=P,
        theta=float(theta),
        sm_scale=float(1.0 / np.sqrt(d)),
        num_pages=num_pages,
        page_indptr=page_indptr.astype(np.int32),
        page_ids=page_ids,
        prefix=prefix,
        step=step,
        meta={"lanes": [{k_: v_ for k_, v_ in ln.items() if k_ != "pos_of_slot"} for ln in lanes]},
    )
    if mask_fn is not None:
        bits, offs = mask_fn(rngs["mask"], lanes, step)
        wl.mask_bits, wl.mask_word_offset = bits, offs
    if channel_fn is not None:
        wl.channel = channel_fn(rngs["channel"], lanes)
    if readout_fn is not None:
        wl.readout_rows = readout_fn(lanes, step)
    return wl


def _ident_pos(n: int) -> np.ndarray:
    return np.arange(n, dtype=np.int64)


def _pack_lsb_first(allowed: np.ndarray) -> np.ndarray:
    """bool [rows, 32*w] -> uint32 [rows, w]; bit b of word w is slot 32*w + b."""
    rows, width = allowed.shape
    w = width // 32
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (allowed.reshape(rows, w, 32).astype(np.uint64) * weights).sum(axis=2).astype(np.uint32)


def _bitmap_rows(lanes, step, rng):
    """Per-row slot bitmaps for lanes that carry a mask (uint32 words, LSB first).

    Each masked lane stores ceil(kv_len/32) words per row, rows in order; its
    span is [offs[l], offs[l+1]). Lanes without a mask get an empty span and
    keep the causal rule.
    """
    L = len(lanes)
    offs = np.zeros(L + 1, dtype=np.int64)
    chunks = []
    for li, ln in enumerate(lanes):
        n = ln["n"]
        if ln.get("mask") is None or n == 0:
            offs[li + 1] = offs[li]
            continue
        kvl = int(ln["kv_len"])
        wpr = -(-kvl // 32)
        r0 = int(step.indptr[li])
        slot = step.slots[r0:r0 + n].astype(np.int64)[:, None]
        allowed = np.zeros((n, wpr * 32), dtype=bool)
        allowed[:, :kvl] = _mask_rule(ln["mask"], slot, np.arange(kvl, dtype=np.int64)[None, :], rng)
        chunks.append(_pack_lsb_first(allowed).reshape(-1))
        offs[li + 1] = offs[li] + n * wpr
    bits = np.concatenate(chunks) if chunks else np.zeros(0, dtype=np.uint32)
    return bits, offs


def _mask_rule(m, slot, j, rng):
    """Slot predicate for one lane: slot is [n,1] (row slots), j is [1,kv_len]."""
    kind = m["kind"]
    if kind == "window":      # sliding window of `window` slots ending at the row, plus sink slots
        return (j < m["sinks"]) | ((j > slot - m["window"]) & (j <= slot))
    if kind == "tova":        # causal, minus a random `drop` fraction; the row's own slot is kept
        u = rng.random((slot.shape[0], j.shape[1]))
        return (j <= slot) & ((j == slot) | (u >= m["drop"]))
    if kind == "causal":
        return np.broadcast_to(j <= slot, (slot.shape[0], j.shape[1]))
    if kind == "random":      # not causal at all: any slot below kv_len may be chosen
        return rng.random((slot.shape[0], j.shape[1])) < m["density"]
    if kind == "empty":
        return np.zeros((slot.shape[0], j.shape[1]), dtype=bool)
    raise ValueError(kind)


def _make_mask(rng, lanes, step):
    return _bitmap_rows(lanes, step, rng)


# --------------------------------------------------------------------------- configs


def _config1(rngs, scale):
    lanes = [dict(c=0, n=37, kv_len=37, fold=FOLD_ALL, pos_of_slot=_ident_pos(37))]
    return _assemble(CONFIG_NAMES[1], rngs, H_q=4, H_kv=2, d=64, P=16, lanes=lanes)


def _config2(rngs, scale):
    L, lo, hi = (64, 512, 8192) if scale == "full" else (6, 33, 700)
    kvs = rngs["lengths"].integers(lo, hi + 1, size=L)
    lanes = [dict(c=int(kv) - 1, n=1, kv_len=int(kv), fold=FOLD_ALL, pos_of_slot=_ident_pos(int(kv))) for kv in kvs]
    return _assemble(CONFIG_NAMES[2], rngs, H_q=32, H_kv=8, d=128, P=16, lanes=lanes)


def _config3(rngs, scale):
    if scale == "full":
        Lp, n_rng, c_rng, Ld, kv_rng = 8, (1024, 4096), (0, 2048), 120, (256, 16384)
    else:
        Lp, n_rng, c_rng, Ld, kv_rng = 2, (40, 150), (0, 90), 5, (20, 500)
    g = rngs["lengths"]
    ns = g.integers(n_rng[0], n_rng[1] + 1, size=Lp)
    cs = g.integers(c_rng[0], c_rng[1] + 1, size=Lp)
    kvs = g.integers(kv_rng[0], kv_rng[1] + 1, size=Ld)
    lanes = [dict(c=int(c), n=int(n), kv_len=int(c + n), fold=FOLD_ALL, pos_of_slot=_ident_pos(int(c + n))) for n, c in zip(ns, cs)]
    lanes += [dict(c=int(kv) - 1, n=1, kv_len=int(kv), fold=FOLD_ALL, pos_of_slot=_ident_pos(int(kv))) for kv in kvs]
    return _assemble(CONFIG_NAMES[3], rngs, H_q=32, H_kv=8, d=128, P=32, lanes=lanes)


def _config4(rngs, scale):
    if scale == "full":
        pairs, c_cond, c_unc, Lv, c_hi = 8, 2048, 512, 32, 4088
    else:
        pairs, c_cond, c_unc, Lv, c_hi = 2, 200, 60, 4, 300
    g = rngs["lengths"]
    lanes = []
    for _ in range(pairs):
        lanes.append(dict(c=c_cond, n=1, kv_len=c_cond + 1, fold=FOLD_ALL, pos_of_slot=_ident_pos(c_cond + 1), role="cond"))
        lanes.append(dict(c=c_unc, n=1, kv_len=c_unc + 1, fold=FOLD_ALL, pos_of_slot=_ident_pos(c_unc + 1), role="uncond"))
    for c in g.integers(0, c_hi + 1, size=Lv):
        c = int(c)
        lanes.append(dict(c=c, n=8, kv_len=c + 8, fold=FOLD_CHANNEL, pos_of_slot=_ident_pos(c + 8), role="verify"))

    def channel_fn(rng, lanes_):
        return np.array([int(rng.integers(0, 9)) if ln["role"] == "verify" else 0 for ln in lanes_], dtype=np.int32)

    def readout_fn(lanes_, step):
        rows = []
        for li, ln in enumerate(lanes_):
            r0, r1 = int(step.indptr[li]), int(step.indptr[li + 1])
            if ln["role"] == "verify":
                rows.extend(range(r0, r1))
            elif r1 > r0:
                rows.append(r1 - 1)
        return np.array(rows, dtype=np.int32)

    return _assemble(CONFIG_NAMES[4], rngs, H_q=32, H_kv=8, d=128, P=16, lanes=lanes,
                     channel_fn=channel_fn, readout_fn=readout_fn)


def _config5(rngs, scale):
    if scale == "full":
        L, n, kvl, window, H_q = 16, 512, 32768, 1024, 64
    else:
        L, n, kvl, window, H_q = 4, 64, 1024, 128, 64
    g = rngs["lengths"]
    kinds = np.array(["window"] * (L // 2) + ["tova"] * (L - L // 2))
    kinds = kinds[g.permutation(L)]
    lanes = []
    for kind in kinds:
        gaps = g.integers(1, 5, size=kvl).astype(np.int64)
        gaps[0] = 0
        pos = np.cumsum(gaps)
        mask = dict(kind="window", window=window, sinks=4) if kind == "window" else dict(kind="tova", drop=0.3)
        lanes.append(dict(c=kvl - n, n=n, kv_len=kvl, fold=FOLD_ALL, pos_of_slot=pos, mask=mask))
    return _assemble(CONFIG_NAMES[5], rngs, H_q=H_q, H_kv=8, d=128, P=16, lanes=lanes, mask_fn=_make_mask)


_BUILDERS = {1: _config1, 2: _config2, 3: _config3, 4: _config4, 5: _config5}


def make_config(k: int, seed: int = 0, scale: str = "full") -> Workload:
    """Build configuration k (1..5). scale='full' gives the benchmark sizes,
    scale='small' a reduced copy (same structure, a few tiles per lane and a
    ragged tail) that the CPU oracle finishes in seconds."""
    if scale not in ("full", "small"):
        raise ValueError(scale)
    wl = _BUILDERS[int(k)](_rngs(seed), scale)
    wl.meta.update(config=int(k), seed=int(seed), scale=scale)
    return wl


def make_random(seed: int, *, H_kv: int = 2, G: int = 2, d: int = 64, P: int = 16,
                num_lanes: int = 6, max_rows: int = 80, max_ctx: int = 300,
                masked: bool = True, fold_modes: bool = True, extra_pages: int = 3) -> Workload:
    """A random small pass mixing prefill, decode, verify and empty lanes, causal
    and bitmap lanes, and every fold mode (literal, all, channel, out-of-range)."""
    rngs = _rngs(seed)
    g = rngs["lengths"]
    lanes = []
    for i in range(num_lanes):
        kind = g.integers(0, 4)
        if kind == 0:      # decode
            n = 1
        elif kind == 1:    # verify-like window
            n = int(g.integers(2, 9))
        elif kind == 2:    # prefill chunk
            n = int(g.integers(9, max_rows + 1))
        else:              # empty lane (reads nothing this pass)
            n = 0
        c = int(g.integers(0, max_ctx + 1))
        kv = c + n
        extra = int(g.integers(0, 2 * P))  # spare capacity beyond kv_len
        ln = dict(c=c, n=n, kv_len=kv, pages=-(-max(kv + extra, 1) // P), pos_of_slot=np.cumsum(g.integers(1, 3, size=kv + extra + 1)) - 1)
        if fold_modes:
            fm = int(g.integers(0, 4))
            ln["fold"] = [FOLD_ALL, FOLD_CHANNEL, int(g.integers(0, n + 1)), 0][fm]
        else:
            ln["fold"] = FOLD_ALL
        if masked and n > 0 and g.random() < 0.5:
            mk = ["window", "tova", "causal", "random"][int(g.integers(0, 4))]
            ln["mask"] = dict(kind=mk, window=int(g.integers(1, 70)), sinks=int(g.integers(0, 5)), drop=0.3, density=0.4)
        lanes.append(ln)

    def channel_fn(rng, lanes_):
        # includes out-of-range counts to exercise clamping
        return np.array([int(rng.integers(-2, 12)) for _ in lanes_], dtype=np.int32)

    return _assemble(f"random_{seed}", rngs, H_q=H_kv * G, H_kv=H_kv, d=d, P=P, lanes=lanes,
                     extra_pages=extra_pages, mask_fn=_make_mask if masked else None,
                     channel_fn=channel_fn)


@dataclass
class RunAhead:
    """A repeating decode loop: a prompt per lane, then `passes` passes of a fixed
    shape (indptr) whose geometry each pass takes from the committed lengths.

    Per pass t the arrays k[t], v[t], q[t] hold that pass's rows and accept[t]
    the per-lane count the fold commits (a device channel, possibly out of
    range to exercise clamping). Slot s of lane l sits at position
    pos_offset[l] + s.
    """

    H_q: int
    H_kv: int
    d: int
    P: int
    theta: float
    sm_scale: float
    num_pages: int
    page_indptr: np.ndarray   # int32 [L+1]
    page_ids: np.ndarray      # int32
    prefix: Optional[Pass]
    pos_offset: np.ndarray    # int32 [L]
    indptr: np.ndarray        # int32 [L+1], the shape of every pass
    k: List[np.ndarray]
    v: List[np.ndarray]
    q: List[np.ndarray]
    accept: List[np.ndarray]  # int32 [L] per pass

    @property
    def num_lanes(self) -> int:
        return int(self.indptr.shape[0] - 1)

    @property
    def passes(self) -> int:
        return len(self.k)


def make_run_ahead(seed: int, *, H_kv: int = 2, G: int = 4, d: int = 128, P: int = 16, num_lanes: int = 8,
                   passes: int = 6, max_prompt: int = 300, extra_pages: int = 2) -> RunAhead:
    """Speculative-decoding style loop: each lane drafts 0..8 rows per pass
    (0 = an idle lane), the channel accepts 0..n of them (sometimes more, to
    be clamped), prompts 0..max_prompt slots, random position offsets."""
    rngs = _rngs(seed)
    g = rngs["lengths"]
    L = int(num_lanes)
    n = np.array([int(g.choice([0, 1, 2, 4, 8])) for _ in range(L)], dtype=np.int64)
    c0 = g.integers(0, max_prompt + 1, size=L).astype(np.int64)
    off = g.integers(0, 5000, size=L).astype(np.int64)
    pages = -(-(c0 + passes * n + 1) // P)
    page_indptr = np.zeros(L + 1, dtype=np.int64)
    page_indptr[1:] = np.cumsum(pages)
    num_pages = int(page_indptr[-1]) + int(extra_pages)
    page_ids = rngs["perm"].permutation(num_pages).astype(np.int32)[: int(page_indptr[-1])].copy()
    pre_indptr = np.zeros(L + 1, dtype=np.int64)
    pre_indptr[1:] = np.cumsum(c0)
    Np = int(pre_indptr[-1])
    prefix = None
    if Np:
        slots = np.concatenate([np.arange(c, dtype=np.int64) for c in c0])
        pos = np.concatenate([np.arange(c, dtype=np.int64) + o for c, o in zip(c0, off)])
        prefix = Pass(indptr=pre_indptr.astype(np.int32), positions=pos.astype(np.int32),
                      slots=slots.astype(np.int32), kv_len=c0.astype(np.int32),
                      fold=np.full(L, FOLD_ALL, dtype=np.int32),
                      k=_normal_bf16(rngs["prefix_kv"], (Np, H_kv, d)),
                      v=_normal_bf16(rngs["prefix_kv"], (Np, H_kv, d)))
    indptr = np.zeros(L + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(n)
    N = int(indptr[-1])
    H_q = H_kv * G
    ks, vs, qs, acc = [], [], [], []
    for _ in range(passes):
        qs.append(_normal_bf16(rngs["q"], (N, H_q, d)))
        ks.append(_normal_bf16(rngs["k"], (N, H_kv, d)))
        vs.append(_normal_bf16(rngs["v"], (N, H_kv, d)))
        a = np.array([int(rngs["channel"].integers(0, m + 1)) for m in n], dtype=np.int32)
        if rngs["channel"].random() < 0.3:
            a[int(rngs["channel"].integers(0, L))] = 99
        acc.append(a)
    return RunAhead(H_q=H_q, H_kv=H_kv, d=d, P=P, theta=10000.0, sm_scale=float(1.0 / np.sqrt(d)),
                    num_pages=num_pages, page_indptr=page_indptr.astype(np.int32), page_ids=page_ids,
                    prefix=prefix, pos_offset=off.astype(np.int32), indptr=indptr.astype(np.int32),
                    k=ks, v=vs, q=qs, accept=acc)


def split_pass(p: Pass, first_rows) -> tuple:
    """Split a pass into two consecutive passes: lane l's first first_rows[l]
    rows (folded all, reading up to the last slot they write) and the rest
    (the original kv_len and fold). Input arrays are copied, not regenerated."""
    L = p.num_lanes
    a_rows, b_rows, a_kv, a_ip, b_ip = [], [], [], [0], [0]
    for lane in range(L):
        r0, r1 = int(p.indptr[lane]), int(p.indptr[lane + 1])
        s = min(max(int(first_rows[lane]), 0), r1 - r0)
        a = list(range(r0, r0 + s))
        b = list(range(r0 + s, r1))
        a_rows += a
        b_rows += b
        a_ip.append(a_ip[-1] + len(a))
        b_ip.append(b_ip[-1] + len(b))
        a_kv.append(int(p.slots[a[-1]]) + 1 if a else 0)
    a_rows = np.asarray(a_rows, dtype=np.int64)
    b_rows = np.asarray(b_rows, dtype=np.int64)

    def sub(rows, ip, kv, fold):
        return Pass(indptr=np.asarray(ip, dtype=np.int32), positions=p.positions[rows].copy(),
                    slots=p.slots[rows].copy(), kv_len=np.asarray(kv, dtype=np.int32),
                    fold=np.asarray(fold, dtype=np.int32), k=p.k[rows].copy(), v=p.v[rows].copy(),
                    q=None if p.q is None else p.q[rows].copy())

    first = sub(a_rows, a_ip, a_kv, [FOLD_ALL] * L)
    second = sub(b_rows, b_ip, p.kv_len, p.fold)
    return first, second


@dataclass
class Lora:
    """Inputs of a projection-site LoRA step: rows of a pass (x, base output y),
    per-lane adapter ids (-1: none) and the adapters' weights and scales."""

    indptr: np.ndarray     # int32 [L+1]
    adapter: np.ndarray    # int32 [L]
    x: np.ndarray          # uint16 bf16 [N][d_in]
    y: np.ndarray          # uint16 bf16 [N][d_out]
    a: np.ndarray          # uint16 bf16 [n_ad][r][d_in]
    b: np.ndarray          # uint16 bf16 [n_ad][d_out][r]
    scale: np.ndarray      # float32 [n_ad]


def make_lora(seed: int, indptr, *, d_in: int, d_out: int, rank: int, num_adapters: int,
              none_frac: float = 0.2) -> Lora:
    """x, y ~ N(0,1); A ~ N(0, 1/d_in), B ~ N(0, 1/rank) so B(Ax) is O(1) like y;
    scales ~ U[0.5, 2); each lane takes a uniform adapter id, or none with
    probability none_frac. All rounded to bf16."""
    rngs = _rngs(seed)
    indptr = np.asarray(indptr, dtype=np.int32)
    L, N = len(indptr) - 1, int(indptr[-1])
    g = rngs["lengths"]
    adapter = g.integers(0, num_adapters, size=L).astype(np.int32)
    adapter[g.random(L) < none_frac] = -1
    x = _normal_bf16(rngs["q"], (N, d_in))
    y = _normal_bf16(rngs["v"], (N, d_out))
    a = bf16_bits_from_f32(rngs["k"].standard_normal((num_adapters, rank, d_in), dtype=np.float32)
                           / np.float32(np.sqrt(d_in)))
    b = bf16_bits_from_f32(rngs["prefix_kv"].standard_normal((num_adapters, d_out, rank), dtype=np.float32)
                           / np.float32(np.sqrt(rank)))
    scale = rngs["channel"].uniform(0.5, 2.0, size=num_adapters).astype(np.float32)
    return Lora(indptr=indptr, adapter=adapter, x=x, y=y, a=a, b=b, scale=scale)


def make_explicit(seed: int, *, H_kv: int = 2, G: int = 2, d: int = 64, P: int = 16, num_lanes: int = 6,
                  max_rows: int = 80, max_ctx: int = 300, masked: bool = True, extra_pages: int = 3,
                  kinds=None, density: float = 0.7) -> Workload:
    """A pass whose rows name their slots explicitly, the way algorithms that
    manage KV slots directly use StateGeometry (Docs, State geometry), instead
    of appending after the committed prefix.

    Per lane: an untimed prefix pass writes a random subset (about `density`)
    of the lane's slots in random order at random positions, and its fold
    freezes the slots below a random k (a literal count). The step's rows
    then write distinct slots drawn from [k, capacity) in random order: some
    rewrite slots the prefix wrote above k, some are fresh, and gaps are left.
    kv_len is the capacity, the largest written slot + 1, or a value between
    the smallest and largest written slot + 1, so some rows write past what
    the lane reads. Slots below kv_len that neither pass writes are holes:
    they keep whatever the pool held (the caller's fill). Positions are random
    and unrelated to slots. Lane kinds: 0 decode (1 row), 1 verify (2..8
    rows), 2 prefill (9..max_rows rows); masks as in make_random; fold modes,
    channel and an explicit readout list (random rows, repeats allowed) too.
    """
    rngs = _rngs(seed)
    g = rngs["lengths"]
    L = int(num_lanes)
    spec = []
    for i in range(L):
        kind = int(kinds[i % len(kinds)]) if kinds is not None else int(g.integers(0, 3))
        n = 1 if kind == 0 else (int(g.integers(2, 9)) if kind == 1 else int(g.integers(9, max_rows + 1)))
        cap = -(-(n + int(g.integers(0, max_ctx + 1)) + int(g.integers(0, 2 * P))) // P) * P
        pre = np.nonzero(g.random(cap) < density)[0].astype(np.int64)
        pre = pre[g.permutation(len(pre))]
        k = int(g.integers(0, min(len(pre), cap - n) + 1))
        step = g.choice(np.arange(k, cap, dtype=np.int64), size=n, replace=False)
        hi = int(step.max()) + 1
        mode = int(g.integers(0, 3))
        kvl = cap if mode == 0 else (hi if mode == 1 else int(g.integers(int(step.min()) + 1, hi + 1)))
        fm = int(g.integers(0, 4))
        fold = [FOLD_ALL, FOLD_CHANNEL, int(g.integers(0, n + 1)), 0][fm]
        mask = None
        if masked and g.random() < 0.5:
            mk = ["window", "tova", "causal", "random"][int(g.integers(0, 4))]
            mask = dict(kind=mk, window=int(g.integers(1, 70)), sinks=int(g.integers(0, 5)), drop=0.3, density=0.4)
        spec.append(dict(n=n, cap=cap, pre=pre, k=k, step=step, kv_len=kvl, fold=fold, mask=mask, kind=kind))
    order = rngs["perm"].permutation(L) if L > 1 else np.arange(L)
    spec = [spec[i] for i in order]
    pages = np.array([s["cap"] // P for s in spec], dtype=np.int64)
    page_indptr = np.zeros(L + 1, dtype=np.int64)
    page_indptr[1:] = np.cumsum(pages)
    num_pages = int(page_indptr[-1]) + int(extra_pages)
    page_ids = rngs["perm"].permutation(num_pages).astype(np.int32)[: int(page_indptr[-1])].copy()

    def cat(arrs):
        return np.concatenate(arrs).astype(np.int64) if arrs else np.zeros(0, np.int64)

    pre_counts = np.array([len(s["pre"]) for s in spec], dtype=np.int64)
    pre_indptr = np.concatenate([[0], np.cumsum(pre_counts)])
    Np = int(pre_indptr[-1])
    pre_pos = g.integers(0, 20000, size=Np)
    prefix = None
    if Np:
        prefix = Pass(indptr=pre_indptr.astype(np.int32), positions=pre_pos.astype(np.int32),
                      slots=cat([s["pre"] for s in spec]).astype(np.int32),
                      kv_len=np.array([s["cap"] for s in spec], dtype=np.int32),
                      fold=np.array([s["k"] for s in spec], dtype=np.int32),
                      k=_normal_bf16(rngs["prefix_kv"], (Np, H_kv, d)),
                      v=_normal_bf16(rngs["prefix_kv"], (Np, H_kv, d)))
    counts = np.array([s["n"] for s in spec], dtype=np.int64)
    indptr = np.concatenate([[0], np.cumsum(counts)])
    N = int(indptr[-1])
    H_q = H_kv * G
    step = Pass(indptr=indptr.astype(np.int32), positions=g.integers(0, 20000, size=N).astype(np.int32),
                slots=cat([s["step"] for s in spec]).astype(np.int32),
                kv_len=np.array([s["kv_len"] for s in spec], dtype=np.int32),
                fold=np.array([s["fold"] for s in spec], dtype=np.int32),
                k=_normal_bf16(rngs["k"], (N, H_kv, d)), v=_normal_bf16(rngs["v"], (N, H_kv, d)),
                q=_normal_bf16(rngs["q"], (N, H_q, d)))
    wl = Workload(name=f"explicit_{seed}", H_q=H_q, H_kv=H_kv, d=d, P=P, theta=10000.0,
                  sm_scale=float(1.0 / np.sqrt(d)), num_pages=num_pages,
                  page_indptr=page_indptr.astype(np.int32), page_ids=page_ids, prefix=prefix, step=step,
                  meta={"lanes": [{k_: v_ for k_, v_ in s.items() if k_ not in ("pre", "step")} for s in spec]})
    if masked:
        lanes_m = [dict(n=s["n"], kv_len=s["kv_len"], mask=s["mask"]) for s in spec]
        wl.mask_bits, wl.mask_word_offset = _bitmap_rows(lanes_m, step, rngs["mask"])
    wl.channel = np.array([int(rngs["channel"].integers(-2, 12)) for _ in range(L)], dtype=np.int32)
    if N:
        wl.readout_rows = rngs["channel"].integers(0, N, size=int(rngs["channel"].integers(1, 2 * L + 1))).astype(np.int32)
    return wl


def make_append_mix(seed: int, *, H_kv: int = 2, d: int = 64, P: int = 16, rows: int = 4096) -> Workload:
    """A pass of at least `rows` rows for the KV write alone, mixing the slot
    patterns a row group of the append can meet: contiguous runs that start
    at any offset of a page and cross page boundaries (prefill chunks),
    single rows (decode), runs in reverse order, runs with gaps, and a few
    rows aimed at frozen slots (below the folded prefix) or outside the
    lane's capacity, which the write must refuse and flag. Lane sizes vary
    from 1 to 300 rows, so row groups straddle lane boundaries. H_q = H_kv."""
    rngs = _rngs(seed)
    g = rngs["lengths"]
    lanes, total = [], 0
    while total < rows:
        kind = int(g.integers(0, 5))
        n = 1 if kind == 1 else int(g.integers(1, 301))
        c = int(g.integers(0, 6 * P))
        cap = -(-(c + 2 * n + int(g.integers(0, 2 * P)) + 1) // P) * P
        if kind in (0, 1):     # contiguous run after the prefix
            slots = np.arange(c, c + n)
        elif kind == 2:        # the same run written back to front
            slots = np.arange(c + n - 1, c - 1, -1)
        elif kind == 3:        # every other slot
            slots = c + 2 * np.arange(n)
        else:                  # contiguous, with a few rows at frozen or out-of-range slots
            slots = np.arange(c, c + n)
            bad = g.random(n) < 0.05
            slots = np.where(bad, g.choice(np.array([-1, cap, cap + P, max(c - 1, -1)]), size=n), slots)
        lanes.append(dict(c=c, n=n, kv_len=int(min(cap, max(c + 1, int(slots.max()) + 1))), fold=FOLD_ALL,
                          pos_of_slot=_ident_pos(cap + 2 * P + 1), pages=cap // P, slots=slots))
        total += n
    wl = _assemble(f"append_mix_{seed}", rngs, H_q=H_kv, H_kv=H_kv, d=d, P=P, lanes=lanes, extra_pages=2)
    return wl


def make_window_decode(seed: int, *, L: int = 64, kv: int = 32768, window: int = 1024, sinks: int = 4,
                       H_q: int = 32, H_kv: int = 8, d: int = 128, P: int = 16) -> Workload:
    """A decode wave under a sliding window with attention sinks (Docs,
    Attention masks), the StreamingLLM shape: L lanes of one row at slot
    kv - 1 (position kv - 1) whose bitmap allows slots j < sinks and the
    window kv - window < j <= kv - 1. The prefix pass writes only the slots
    the rows may read (sinks and window, positions = slots, nothing frozen);
    the others are holes that keep the pool's fill. Lane order and physical
    pages are permuted as in the configurations."""
    rngs = _rngs(seed)
    read = np.concatenate([np.arange(sinks), np.arange(kv - window, kv - 1)]).astype(np.int64)
    n_pre = len(read)
    lanes = [dict(c=0, n=1, kv_len=kv, fold=FOLD_ALL, pos_of_slot=_ident_pos(kv),
                  mask=dict(kind="window", window=window, sinks=sinks)) for _ in range(L)]
    wl = _assemble(f"window_decode_{L}x{kv}", rngs, H_q=H_q, H_kv=H_kv, d=d, P=P, lanes=lanes,
                   mask_fn=_make_mask)
    # the step's single row sits at slot kv - 1; the prefix writes the readable slots only
    st = wl.step
    st.slots = np.full(L, kv - 1, dtype=np.int32)
    st.positions = np.full(L, kv - 1, dtype=np.int32)
    wl.mask_bits, wl.mask_word_offset = _bitmap_rows(lanes, st, rngs["mask"])
    pre_indptr = (np.arange(L + 1, dtype=np.int64) * n_pre).astype(np.int32)
    wl.prefix = Pass(indptr=pre_indptr, positions=np.tile(read, L).astype(np.int32),
                     slots=np.tile(read, L).astype(np.int32), kv_len=np.full(L, kv, dtype=np.int32),
                     fold=np.zeros(L, dtype=np.int32), k=_normal_bf16(rngs["prefix_kv"], (L * n_pre, H_kv, d)),
                     v=_normal_bf16(rngs["prefix_kv"], (L * n_pre, H_kv, d)))
    wl.meta.update(window=window, sinks=sinks)
    return wl


def make_empty_pass(seed: int, *, H_q: int = 32, H_kv: int = 8, d: int = 128, P: int = 16) -> Workload:
    """A pass with lanes but no rows: five lanes with cached prefixes of 0, 17,
    64, 300 and 5 slots and no new rows. Their folds are all, none, a device
    channel count of 2 and a literal 3 (both more than the lane's zero rows)
    and all; the default readout then lists no row."""
    rngs = _rngs(seed)
    cs = [0, 17, 64, 300, 5]
    folds = [FOLD_ALL, 0, FOLD_CHANNEL, 3, FOLD_ALL]
    lanes = [dict(c=c, n=0, kv_len=c, fold=f, pos_of_slot=_ident_pos(max(c, 1)), pages=-(-max(c, 1) // P))
             for c, f in zip(cs, folds)]
    return _assemble(f"empty_pass_{len(lanes)}", rngs, H_q=H_q, H_kv=H_kv, d=d, P=P, lanes=lanes,
                     channel_fn=lambda rng, ls: np.full(len(ls), 2, dtype=np.int32))

