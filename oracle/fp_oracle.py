"""Plain fp64 CPU oracle of the ForwardPass attention step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark import this module. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

What it computes, step by step, following the Pie documentation page "The
forward pass" (pie-project.org/docs/invent/forward-pass) and the paged-KV
accounting of the two Pie reviews (section 2.1/2.2, Eqs. (1) and (2)):

  append   each input row writes its K/V state into the slot its StateGeometry
           names (per-row `slots`), K rotated by RoPE at the row's explicit
           `positions` value ("State geometry" field table). K/V live in a
           paged pool; a lane's working set is an ordered list of pages.
  attend   every row of a lane attends to the lane's first `kv_len` slots
           ("kv_len: number of KV slots the lane reads"), either under the
           folding rule (rows appended causally) or under an explicit per-row
           slot set given by `fwd.mask` ("Attention masks": sliding window,
           sinks, TOVA are all such sets). Exact softmax attention in fp64.
  fold     after the pass, freeze none, all, or a count of the newly written
           slots; the count may come from a device channel written by the
           epilogue ("State geometry", speculative-decoding paragraph).
  readout  by default the last row of each lane, or caller-chosen rows
           ("Readouts").

Readings taken where the pages are silent:
  * RoPE pairs interleaved dims (2i, 2i+1) with w_i = theta^(-2i/d) (the
    RoFormer definition); K is stored rotated, Q is rotated at use, unrounded.
  * Rotated K is rounded once, to nearest-even, from fp64 to bf16.
  * "causal" with explicit slots means slot-index causal: row r reads j <= slots[r].
  * a lane's bitmap replaces the causal rule for that lane; bits >= kv_len are ignored.
  * GQA: query head q reads KV head q // (H_q / H_kv).
  * an empty allowed set gives O = 0 and LSE = -inf.
  * fold adds its count to the lane's committed length; counts are clamped to
    [0, rows of the lane] (flagged); it happens after attention.
  * writes to slots outside the lane's pages, or below its committed length,
    are suppressed and flagged.

Pool layout used here (the oracle's own): k[page][head][offset][dim] and
v[page][head][offset][dim], bf16 bit patterns (uint16).
"""

from __future__ import annotations

import numpy as np

# Device status bits (values fixed by the C ABI documentation).
ST_SLOT_RANGE = 1      # slot outside [0, capacity): write suppressed
ST_FROZEN = 2          # slot below committed length: write suppressed
ST_KVLEN = 4           # kv_len outside [0, capacity]: clamped
ST_FOLD_CLAMP = 8      # fold count outside [0, rows]: clamped
ST_READOUT_RANGE = 16  # readout row outside [0, num_rows): zero row returned
ST_MASK_SHORT = 32     # mask row holds fewer than kv_len bits: missing bits read as 0
ST_PAGE_RANGE = 64     # page id outside [0, num_pages): write suppressed, read clamped
ST_ADAPTER = 256       # adapter id >= number of adapters: the lane keeps y
ST_DUP_WRITE = 512     # a KV cell receives two writes in one pass
ST_SHARED_CELL = 1024  # a KV cell one lane writes is read or written by another lane

FOLD_ALL = -1
FOLD_CHANNEL = -2


# ----------------------------------------------------------------------------- accounting
# Eq. (1) and Eq. (2) of the Pie reviews (section 2.1 / 2.2 "KV cache" and "paging").

def kv_bytes(L: int, H_kv: int, d: int, T: int, b: int) -> int:
    """Dense KV bytes M_KV = 2 * L * H_kv * d * T * b (keys and values, all layers)."""
    return 2 * int(L) * int(H_kv) * int(d) * int(T) * int(b)


def pages_for(T: int, P: int) -> int:
    """Pages a T-token sequence occupies at P tokens per page: ceil(T / P)."""
    return -(-int(T) // int(P))


def page_waste(T: int, P: int) -> int:
    """Unused slots in the last page: W(T, P) = P * ceil(T / P) - T."""
    return int(P) * pages_for(T, P) - int(T)


# ----------------------------------------------------------------------------- bf16

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to bf16 bit patterns, nearest-even, in one correct rounding.

    Method: round to float32 with round-to-odd (truncate toward zero, then set
    the last bit if anything was discarded), then round that to bf16 with
    nearest-even. Float32 keeps 16 more significand bits than bf16, which is
    enough for round-to-odd to make the second rounding exact. Inputs must be
    finite with magnitude in float32's normal range or zero.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    back = f.astype(np.float64)
    fb = np.atleast_1d(f.view(np.uint32)).astype(np.uint64).copy()
    xb = np.atleast_1d(x)
    backb = np.atleast_1d(back)
    away = np.abs(backb) > np.abs(xb)
    fb[away] -= 1                       # one float32 ulp toward zero: now truncated
    fb[backb != xb] |= 1                # sticky bit
    r = (fb + 0x7FFF + ((fb >> 16) & 1)) >> 16
    return r.astype(np.uint16).reshape(x.shape)


# ----------------------------------------------------------------------------- RoPE

def rope_freqs(d: int, theta: float) -> np.ndarray:
    """w_i = theta^(-2i/d), i = 0 .. d/2-1, in fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(d))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]) by angle pos * w_i, in fp64.

    x: [..., H, d] float64, pos: [...] integer positions (one per leading index).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_freqs(d, theta)  # [..., d/2]
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------- pool

class Pool:
    """The oracle's own paged KV pool for one attention layer."""

    def __init__(self, num_pages, page_size, num_kv_heads, head_dim, page_indptr, page_ids, fill_bits=0):
        self.num_pages = int(num_pages)
        self.P = int(page_size)
        self.H = int(num_kv_heads)
        self.d = int(head_dim)
        self.page_indptr = np.asarray(page_indptr, dtype=np.int64)
        self.page_ids = np.asarray(page_ids, dtype=np.int64)
        shape = (self.num_pages, self.H, self.P, self.d)
        self.k = np.full(shape, fill_bits, dtype=np.uint16)
        self.v = np.full(shape, fill_bits, dtype=np.uint16)

    @property
    def nbytes(self) -> int:
        return int(self.k.nbytes + self.v.nbytes)

    def capacity(self, lane: int) -> int:
        return int(self.page_indptr[lane + 1] - self.page_indptr[lane]) * self.P

    def locate(self, lane: int, slot, clamp: bool = True):
        """Physical (page, offset) of a lane's working-set slot(s).

        A page id outside [0, num_pages) is a caller error: reads use the
        nearest valid page (clamp=True); writers check page_ok() first.
        """
        slot = np.asarray(slot, dtype=np.int64)
        page = self.page_ids[self.page_indptr[lane] + slot // self.P]
        if clamp:
            page = np.clip(page, 0, self.num_pages - 1)
        return page, slot % self.P

    def page_ok(self, lane: int, slot):
        page = self.page_ids[self.page_indptr[lane] + np.asarray(slot, dtype=np.int64) // self.P]
        return (page >= 0) & (page < self.num_pages)

    def lane_kv(self, lane: int, n: int):
        """K and V of the lane's first n slots, fp64, [n][H][d]."""
        page, off = self.locate(lane, np.arange(n))
        return bf16_to_f64(self.k[page, :, off, :]), bf16_to_f64(self.v[page, :, off, :])


# ----------------------------------------------------------------------------- step parts

def _lane_rows(indptr, lane):
    return int(indptr[lane]), int(indptr[lane + 1])


def append(pool: Pool, committed, indptr, positions, slots, k_bits, v_bits, theta, lanes=None) -> int:
    """Write every row's rotated K and its V into the row's slot. Returns status bits.

    lanes: optional subset of lanes to process (the others are left untouched);
    used to check large passes on a sample of lanes.
    """
    status = 0
    committed = np.asarray(committed)
    for lane in (range(len(indptr) - 1) if lanes is None else lanes):
        r0, r1 = _lane_rows(indptr, lane)
        if r1 == r0:
            continue
        cap = pool.capacity(lane)
        rows = np.arange(r0, r1)
        s = np.asarray(slots[r0:r1], dtype=np.int64)
        bad = (s < 0) | (s >= cap)
        frozen = (~bad) & (s < int(committed[lane]))
        if bad.any():
            status |= ST_SLOT_RANGE
        if frozen.any():
            status |= ST_FROZEN
        ok = ~(bad | frozen)
        if not ok.any():
            continue
        rows, s = rows[ok], s[ok]
        pok = pool.page_ok(lane, s)
        if not pok.all():
            status |= ST_PAGE_RANGE
            rows, s = rows[pok], s[pok]
        if len(np.unique(s)) != len(s):
            raise ValueError("duplicate slot writes in one pass are undefined")
        kr = rope(bf16_to_f64(k_bits[rows]), np.asarray(positions)[rows], theta)
        page, off = pool.locate(lane, s)
        pool.k[page, :, off, :] = f64_to_bf16(kr)
        pool.v[page, :, off, :] = v_bits[rows]
    return status


def hazards(pool: Pool, committed, indptr, slots, kv_len) -> int:
    """Conflicts of one pass between what its rows write and what its lanes read.

    The reviews' Eq. (4) (section 5, batching that keeps meaning) asks that
    calls batched together do not touch each other's state:
    W(a) ∩ (R(b) ∪ W(b)) = ∅ for two calls a ≠ b. Here a call is a lane, and
    the state is KV cells (physical page, offset):
      W(a): the cells lane a's rows write this pass (writes that append()
            performs: slot inside the lane's capacity, not frozen, page id in
            the pool);
      R(b): the cells of lane b's slots below its kv_len (clamped to its
            capacity) whose page id is in the pool.
    Returns ST_DUP_WRITE if some cell is written more than once in the pass
    (two rows with one slot, or two lanes' writes landing in one cell), and
    ST_SHARED_CELL if a cell lane a writes is read or written by another lane.
    """
    writers = {}
    L = len(indptr) - 1
    for lane in range(L):
        r0, r1 = _lane_rows(indptr, lane)
        cap = pool.capacity(lane)
        for r in range(r0, r1):
            s = int(slots[r])
            if s < 0 or s >= cap or s < int(committed[lane]):
                continue
            page = int(pool.page_ids[pool.page_indptr[lane] + s // pool.P])
            if page < 0 or page >= pool.num_pages:
                continue
            writers.setdefault((page, s % pool.P), []).append(lane)
    status = 0
    for lanes in writers.values():
        if len(lanes) > 1:
            status |= ST_DUP_WRITE
        if len(set(lanes)) > 1:
            status |= ST_SHARED_CELL
    for lane in range(L):
        eff = min(max(int(kv_len[lane]), 0), pool.capacity(lane))
        for j in range(eff):
            page = int(pool.page_ids[pool.page_indptr[lane] + j // pool.P])
            if page < 0 or page >= pool.num_pages:
                continue
            w = writers.get((page, j % pool.P))
            if w is not None and any(a != lane for a in w):
                status |= ST_SHARED_CELL
    return status


def _mask_span(mask_bits, word_offset, indptr, lane):
    if mask_bits is None or word_offset is None:
        return None
    o0, o1 = int(word_offset[lane]), int(word_offset[lane + 1])
    if o1 == o0:
        return None
    n = int(indptr[lane + 1] - indptr[lane])
    if n == 0 or (o1 - o0) % n:
        raise ValueError("mask span of a lane must be rows * words_per_row")
    return o0, (o1 - o0) // n


def allowed_slots(lane, row, eff_len, slots, indptr, mask_bits=None, word_offset=None):
    """Slots j < eff_len that row `row` (global index) attends to.

    Returns (index array, short) where short says the mask row held fewer than eff_len bits.
    """
    span = _mask_span(mask_bits, word_offset, indptr, lane)
    if span is None:
        lim = min(eff_len, int(slots[row]) + 1)
        return np.arange(max(lim, 0)), False
    o0, wpr = span
    local = row - int(indptr[lane])
    words = np.asarray(mask_bits[o0 + local * wpr: o0 + (local + 1) * wpr], dtype=np.uint64)
    nbits = min(eff_len, 32 * wpr)
    j = np.arange(nbits)
    on = ((words[j // 32] >> (j % 32).astype(np.uint64)) & 1).astype(bool)
    return j[on], 32 * wpr < eff_len


def attend(pool: Pool, indptr, positions, slots, kv_len, q_bits, H_q, theta, sm_scale,
           mask_bits=None, word_offset=None, rows=None):
    """Exact softmax attention of the given rows (default: all) over their allowed slots.

    Returns (O [len(rows)][H_q][d] fp64, LSE [len(rows)][H_q] fp64, status).
    """
    N = int(indptr[-1])
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    G = H_q // pool.H
    O = np.zeros((len(rows), H_q, pool.d))
    LSE = np.full((len(rows), H_q), -np.inf)
    status = 0
    lane_of = np.searchsorted(np.asarray(indptr), rows, side="right") - 1
    for lane in np.unique(lane_of):
        lane = int(lane)
        cap = pool.capacity(lane)
        kvl = int(kv_len[lane])
        eff = min(max(kvl, 0), cap)
        if eff != kvl:
            status |= ST_KVLEN
        K, V = pool.lane_kv(lane, eff)
        if not (np.isfinite(K).all() and np.isfinite(V).all()):
            # every slot below kv_len must hold finite K/V (written by append or
            # filled by the caller); such a pass is outside the step's domain
            raise ValueError(f"lane {lane}: a slot below kv_len holds a non-finite K or V")
        idx = np.nonzero(lane_of == lane)[0]
        qr = rope(bf16_to_f64(q_bits[rows[idx]]), np.asarray(positions)[rows[idx]], theta)
        for t, i in enumerate(idx):
            A, short = allowed_slots(lane, int(rows[i]), eff, slots, indptr, mask_bits, word_offset)
            if short:
                status |= ST_MASK_SHORT
            if len(A) == 0:
                continue
            for g in range(pool.H):
                qg = qr[t, g * G:(g + 1) * G, :]            # [G][d]
                s = (K[A, g, :] @ qg.T) * sm_scale          # [|A|][G]
                m = s.max(axis=0)
                p = np.exp(s - m)
                l = p.sum(axis=0)
                O[i, g * G:(g + 1) * G, :] = (p.T @ V[A, g, :]) / l[:, None]
                LSE[i, g * G:(g + 1) * G] = m + np.log(l)
    return O, LSE, status


def attn_mass(pool: Pool, indptr, positions, slots, kv_len, q_bits, H_q, theta, sm_scale,
              mask_bits=None, word_offset=None, lanes=None):
    """Attention mass each slot received in the pass, per KV head: the scores
    returned out of the forward pass so that score-driven eviction (TOVA) can
    use them (review section 7; Docs "Attention masks" names such eviction).

    For lane l, KV head g and slot j below the lane's clamped kv_len, the sum
    over the lane's rows r and the query heads h of g of the softmax
    probability of slot j in row r's attention (0 if r may not read j), under
    the same allowed sets and scaling as attend(). Returns fp64
    [H][page_indptr[L] * P], slot j of lane l at column page_indptr[l] * P + j;
    `lanes` limits the lanes computed (the others stay zero).
    """
    S = int(pool.page_indptr[-1]) * pool.P
    mass = np.zeros((pool.H, S))
    G = H_q // pool.H
    L = len(indptr) - 1
    for lane in (range(L) if lanes is None else lanes):
        r0, r1 = _lane_rows(indptr, lane)
        if r1 == r0:
            continue
        eff = min(max(int(kv_len[lane]), 0), pool.capacity(lane))
        K, _ = pool.lane_kv(lane, eff)
        base = int(pool.page_indptr[lane]) * pool.P
        qr = rope(bf16_to_f64(q_bits[r0:r1]), np.asarray(positions)[r0:r1], theta)
        for t, row in enumerate(range(r0, r1)):
            A, _ = allowed_slots(lane, row, eff, slots, indptr, mask_bits, word_offset)
            if len(A) == 0:
                continue
            for g in range(pool.H):
                s = (K[A, g, :] @ qr[t, g * G:(g + 1) * G, :].T) * sm_scale   # [|A|][G]
                p = np.exp(s - s.max(axis=0))
                p /= p.sum(axis=0)
                mass[g, base + A] += p.sum(axis=1)
    return mass


def order_key(x32) -> np.ndarray:
    """Total order of fp32 values as uint32 (negatives below positives, NaN of
    positive sign above +inf): the key the eviction step compares."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    neg = (b & 0x80000000) != 0
    return np.where(neg, (~b) & 0xFFFFFFFF, b | 0x80000000).astype(np.uint32)


def tova_scores(mass32, page_indptr, P, lane, n):
    """Eviction score of lane `lane`'s slots 0..n-1: its attention mass summed
    over the KV heads in head order, in fp32 (the precision the device step
    decides in). mass32: fp32 [H][S], slot j of the lane at page_indptr[lane]*P + j."""
    base = int(page_indptr[lane]) * P
    acc = np.zeros(n, dtype=np.float32)
    for g in range(mass32.shape[0]):
        acc = (acc + mass32[g, base:base + n].astype(np.float32)).astype(np.float32)
    return acc


def tova_keep(mass32, page_indptr, P, committed, budget, prev_keep=None, prev_limit=None):
    """Score-driven eviction (the Docs' Attention masks section: per-row bitmaps
    express attention-based KV eviction such as TOVA; the review's section 7:
    the forward pass returns the scores such a policy needs). Reading taken:
    a lane's old slots are those below its committed length c; a slot is a
    candidate unless an earlier selection dropped it (prev_keep given, slot
    below prev_limit, its bit clear); the lane keeps the min(budget, #candidates)
    candidates with the largest score (order_key of tova_scores), equal keys
    going to the lower slot. Returns a list of bool arrays, lane l's of length c_l."""
    out = []
    for lane in range(len(committed)):
        c = max(int(committed[lane]), 0)
        keys = order_key(tova_scores(mass32, page_indptr, P, lane, c))
        cand = np.ones(c, dtype=bool)
        if prev_keep is not None:
            pl = min(max(int(prev_limit[lane]), 0), c)
            cand[:pl] = np.asarray(prev_keep[lane][:pl], dtype=bool)
        idx = np.nonzero(cand)[0]
        k = min(max(int(budget[lane]), 0), len(idx))
        # larger key first, then lower slot
        order = sorted(idx.tolist(), key=lambda j: (-int(keys[j]), j))
        keep = np.zeros(c, dtype=bool)
        keep[order[:k]] = True
        out.append(keep)
    return out


def tova_mask(keep, indptr, slots, kv_len, committed, words_per_row):
    """The pass's per-row bitmaps from the lanes' keep sets: row r of lane l
    reads old slot j < c_l iff it is kept, and new slot c_l <= j < kv_len_l iff
    j <= slots[r] (the slot-order rule for the pass's own rows); bits at or past
    kv_len are 0. words_per_row[l] words per row (fewer than ceil(kv_len/32)
    drops the tail and flags ST_MASK_SHORT; none means the lane carries no
    bitmap and keeps the causal rule, as an empty mask span does). Returns (list of uint32 arrays,
    lane l's rows concatenated, status)."""
    out, status = [], 0
    for lane in range(len(indptr) - 1):
        r0, r1 = int(indptr[lane]), int(indptr[lane + 1])
        c = max(int(committed[lane]), 0)
        kv = max(int(kv_len[lane]), 0)
        wpr = int(words_per_row[lane])
        if r1 > r0 and 0 < wpr and wpr * 32 < kv:   # no words at all: the lane keeps the causal rule
            status |= ST_MASK_SHORT
        words = np.zeros((r1 - r0, wpr), dtype=np.uint32)
        for t, row in enumerate(range(r0, r1)):
            for j in range(min(kv, 32 * wpr)):
                ok = bool(keep[lane][j]) if j < c else j <= int(slots[row])
                if ok:
                    words[t, j >> 5] |= np.uint32(1 << (j & 31))
        out.append(words.reshape(-1))
    return out, status


def fold(committed, indptr, fold_spec, channel=None):
    """committed[l] += k_l with k_l = literal | rows (all) | channel[l], clamped to [0, rows]."""
    out = np.array(committed, dtype=np.int64)
    status = 0
    for lane in range(len(indptr) - 1):
        n = int(indptr[lane + 1] - indptr[lane])
        f = int(fold_spec[lane])
        if f == FOLD_ALL:
            k = n
        elif f == FOLD_CHANNEL:
            if channel is None:
                status |= ST_FOLD_CLAMP
                k = 0
            else:
                k = int(channel[lane])
        elif f >= 0:
            k = f
        else:
            status |= ST_FOLD_CLAMP
            k = 0
        if k < 0 or k > n:
            status |= ST_FOLD_CLAMP
            k = min(max(k, 0), n)
        out[lane] += k
    return out.astype(np.int32), status


def advance(committed, indptr, pos_offset=None):
    """Geometry of the next pass of a repeating decode loop ("Pipelines and
    frames": run_ahead; "State geometry": folding appends rows causally after
    the frozen prefix): lane l's rows take slots c_l, c_l+1, ..., their
    positions add the lane's offset (0 if none), and the lane reads c_l + n_l slots.
    Returns (positions, slots, kv_len) as int32 arrays."""
    ip = np.asarray(indptr, dtype=np.int64)
    L = len(ip) - 1
    positions = np.zeros(int(ip[-1]), dtype=np.int64)
    slots = np.zeros(int(ip[-1]), dtype=np.int64)
    kv_len = np.zeros(L, dtype=np.int64)
    for lane in range(L):
        c = int(committed[lane])
        off = 0 if pos_offset is None else int(pos_offset[lane])
        for i, r in enumerate(range(int(ip[lane]), int(ip[lane + 1]))):
            slots[r] = c + i
            positions[r] = c + i + off
        kv_len[lane] = c + int(ip[lane + 1] - ip[lane])
    return positions.astype(np.int32), slots.astype(np.int32), kv_len.astype(np.int32)


def lora(x_bits, y_bits, adapter, indptr, a_bits, b_bits, scale):
    """Projection-site LoRA adapter (Docs "Adapters": an adapter maps the
    projection input x and base output y to y + b * (a * x); requests in one
    batch may use different adapters). For the rows of lane l with
    k = adapter[l] >= 0 the exact value is y + s_k * B_k (A_k x), rounded once
    to bf16; lanes with k < 0 keep y, and an id k >= the number of adapters
    keeps y and sets ST_ADAPTER.

    x_bits [N][d_in], y_bits [N][d_out]: bf16 bits; a_bits [n_ad][r][d_in],
    b_bits [n_ad][d_out][r]: bf16 bits; scale [n_ad] float.
    Returns (out bf16 bits [N][d_out], exact fp64 [N][d_out], status).
    """
    out = np.array(y_bits, dtype=np.uint16, copy=True)
    exact = bf16_to_f64(y_bits)
    n_ad = a_bits.shape[0]
    status = 0
    for lane in range(len(indptr) - 1):
        r0, r1 = _lane_rows(indptr, lane)
        k = int(adapter[lane])
        if r1 == r0 or k < 0:
            continue
        if k >= n_ad:
            status |= ST_ADAPTER
            continue
        X = bf16_to_f64(x_bits[r0:r1])
        v = X @ bf16_to_f64(a_bits[k]).T                  # [rows][r]
        e = exact[r0:r1] + float(scale[k]) * (v @ bf16_to_f64(b_bits[k]).T)
        exact[r0:r1] = e
        out[r0:r1] = f64_to_bf16(e)
    return out, exact, status


def ia3(y_bits, adapter, indptr, scale_bits):
    """IA3 adapter (Docs "Adapters": IA3 scales the base output y): rows of a
    lane with k = adapter[l] >= 0 become bf16(y * scale_k) per output column;
    others keep y, an id past the table also sets ST_ADAPTER.
    Returns (out bf16 bits [N][d_out], status)."""
    out = np.array(y_bits, dtype=np.uint16, copy=True)
    status = 0
    for lane in range(len(indptr) - 1):
        r0, r1 = _lane_rows(indptr, lane)
        k = int(adapter[lane])
        if r1 == r0 or k < 0:
            continue
        if k >= scale_bits.shape[0]:
            status |= ST_ADAPTER
            continue
        out[r0:r1] = f64_to_bf16(bf16_to_f64(y_bits[r0:r1]) * bf16_to_f64(scale_bits[k])[None, :])
    return out, status


def readout_rows(indptr, rows=None):
    """Readout list: given rows in the given order, or the last row of each non-empty lane."""
    if rows is not None:
        return np.asarray(rows, dtype=np.int64)
    ip = np.asarray(indptr, dtype=np.int64)
    n = np.diff(ip)
    return (ip[1:] - 1)[n > 0]


def readout(O_flat, num_rows, rows):
    """Gather readout rows of O ([num_rows][...]); out-of-range rows give zeros and a status bit."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows),) + tuple(O_flat.shape[1:]), dtype=O_flat.dtype)
    ok = (rows >= 0) & (rows < num_rows)
    out[ok] = O_flat[rows[ok]]
    return out, (0 if ok.all() else ST_READOUT_RANGE)


def step(pool: Pool, committed, geom, H_q, theta, sm_scale, mask_bits=None, word_offset=None,
         channel=None, readout_list=None, rows=None):
    """One pass: append -> attend -> fold -> readout, in that order.

    geom: an object with indptr, positions, slots, kv_len, fold, k, v, q.
    Returns dict(O, LSE, committed, readout, readout_rows, status).
    """
    st = append(pool, committed, geom.indptr, geom.positions, geom.slots, geom.k, geom.v, theta)
    O, LSE, st_a = attend(pool, geom.indptr, geom.positions, geom.slots, geom.kv_len, geom.q, H_q,
                          theta, sm_scale, mask_bits, word_offset, rows=rows)
    new_c, st_f = fold(committed, geom.indptr, geom.fold, channel)
    res = dict(O=O, LSE=LSE, committed=new_c, status=st | st_a | st_f)
    if rows is None:
        rl = readout_rows(geom.indptr, readout_list)
        ro, st_r = readout(O.reshape(O.shape[0], O.shape[1] * O.shape[2]), int(geom.indptr[-1]), rl)
        res.update(readout=ro, readout_rows=rl)
        res["status"] |= st_r
    return res
