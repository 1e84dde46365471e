"""Pins of the fp64 oracle against what the pages and mathematics fix.

Sources: Pie docs "The forward pass" (Lanes, State geometry, Attention masks,
Readouts) and the two Pie reviews, section 2.1/2.2, Eqs. (1) and (2), and
section 4 (whole prompt == prefix then continuation through the cache).
"""

import itertools
import json
import math
import os
import struct

import numpy as np
import pytest

import bruteforce as bf
import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- Eq. (1), Eq. (2)

def test_eq1_worked_example():
    for c in _load("eq1_kv_bytes.json")["cases"]:
        assert oracle.kv_bytes(c["L"], c["H_kv"], c["d"], c["T"], c["b"]) == c["bytes"]
    assert oracle.kv_bytes(32, 8, 128, 1, 2) == 128 * 1024
    assert oracle.kv_bytes(32, 8, 128, 8192, 2) == 1 << 30


def test_eq2_golden_and_exhaustive():
    for c in _load("eq2_page_waste.json")["cases"]:
        assert oracle.pages_for(c["T"], c["P"]) == c["pages"]
        assert oracle.page_waste(c["T"], c["P"]) == c["waste"]
    for P in (1, 8, 16, 32):
        for T in range(0, 65537):
            w = oracle.page_waste(T, P)
            assert 0 <= w < P
            assert (T + w) % P == 0 and oracle.pages_for(T, P) * P == T + w


def test_pool_bytes_match_eq1_per_page():
    wl = W.make_config(1)
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
    assert pool.nbytes == wl.num_pages * oracle.kv_bytes(1, wl.H_kv, wl.d, wl.P, 2)
    # 37 tokens in pages of 16: 3 pages, 11 unused slots (Eq. 2)
    assert pool.nbytes == oracle.kv_bytes(1, 2, 64, 37, 2) + oracle.page_waste(37, 16) * 2 * 2 * 64 * 2
    assert pool.nbytes == 24576


# ----------------------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_exact_rationals():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000)))
    # exact bf16 midpoints and their neighbours (tie cases and one-ulp-off cases)
    for bits in rng.integers(0x0080, 0x7F00, size=400):
        lo = bf16_value = struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]
        hi = struct.unpack("<f", struct.pack("<I", (int(bits) + 1) << 16))[0]
        mid = (lo + hi) / 2.0
        xs += [mid, -mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), lo, hi]
    xs = np.array(xs, dtype=np.float64)
    got = oracle.f64_to_bf16(xs)
    want = np.array([bf.bf16_round_exact(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)
    # exact round trip for bf16 values
    b = rng.integers(0, 0x7F80, size=1000).astype(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(oracle.bf16_to_f64(b)), b)


# ----------------------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero_and_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(5, int), 10000.0), x)
    y = oracle.rope(x, rng.integers(0, 100000, 5), 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_equals_complex_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 1, 16))
    pos = np.array([0, 1, 17, 81234])
    y = oracle.rope(x, pos, 10000.0)
    for i in range(4):
        ref = bf.rope_complex(list(x[i, 0]), int(pos[i]), 10000.0)
        np.testing.assert_allclose(y[i, 0], ref, rtol=0, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    base = None
    for m in (0, 5, 1000, 77777):
        s = float((oracle.rope(q, [m + 9], 500.0) * oracle.rope(k, [m], 500.0)).sum())
        base = s if base is None else base
        assert abs(s - base) < 1e-9


# ----------------------------------------------------------------------------- brute force

def _as_bf_inputs(wl, rows_pass):
    p = rows_pass
    d = dict(indptr=p.indptr, positions=p.positions, slots=p.slots, kv_len=p.kv_len, fold=p.fold,
             k=p.k.tolist(), v=p.v.tolist(), q=None if p.q is None else p.q.tolist())
    return d


def _mask_sets(wl):
    """Decode LSB-first mask words into per-row slot sets (independent of the oracle)."""
    if wl.mask_bits is None:
        return None
    st = wl.step
    out = [None] * st.num_rows
    for lane in range(st.num_lanes):
        o0, o1 = int(wl.mask_word_offset[lane]), int(wl.mask_word_offset[lane + 1])
        r0, r1 = int(st.indptr[lane]), int(st.indptr[lane + 1])
        if o1 == o0:
            continue
        wpr = (o1 - o0) // (r1 - r0)
        for r in range(r0, r1):
            words = wl.mask_bits[o0 + (r - r0) * wpr: o0 + (r - r0 + 1) * wpr]
            out[r] = {32 * wi + b for wi, wd in enumerate(words) for b in range(32) if (int(wd) >> b) & 1}
    return out


def _oracle_run(wl, fill=0):
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids, fill_bits=fill)
    committed = np.zeros(wl.num_lanes, np.int32)
    if wl.prefix is not None:
        p = wl.prefix
        oracle.append(pool, committed, p.indptr, p.positions, p.slots, p.k, p.v, wl.theta)
        committed, _ = oracle.fold(committed, p.indptr, p.fold)
    res = oracle.step(pool, committed, wl.step, wl.H_q, wl.theta, wl.sm_scale, wl.mask_bits,
                      wl.mask_word_offset, wl.channel, wl.readout_rows)
    res["pool"] = pool
    res["committed0"] = committed
    return res


def _bf_run(wl, hole_bits=None):
    st = _as_bf_inputs(wl, wl.step)
    st["mask"] = _mask_sets(wl)
    st["channel"] = wl.channel
    pre = _as_bf_inputs(wl, wl.prefix) if wl.prefix is not None else None
    return bf.run(st, H_q=wl.H_q, H_kv=wl.H_kv, d=wl.d, theta=wl.theta, sm_scale=wl.sm_scale,
                  cap=[int(c) for c in wl.capacity()], prefix=pre, hole_bits=hole_bits)


def _compare_to_bruteforce(wl, res, ref):
    O = np.array(ref["O"])
    LSE = np.array(ref["LSE"])
    assert np.max(np.abs(res["O"] - O)) <= 1e-12
    fin = np.isfinite(LSE)
    assert np.array_equal(fin, np.isfinite(res["LSE"]))
    assert np.max(np.abs(res["LSE"][fin] - LSE[fin]), initial=0.0) <= 1e-12
    assert list(res["committed"]) == list(ref["committed"])
    # stored K/V: every slot the brute force holds matches the paged pool bit for bit
    pool = res["pool"]
    for lane, slots in enumerate(ref["store"]):
        for s, (ks, vs) in slots.items():
            pg, off = pool.locate(lane, s)
            got_k = oracle.bf16_to_f64(pool.k[pg, :, off, :])
            got_v = oracle.bf16_to_f64(pool.v[pg, :, off, :])
            assert np.array_equal(got_k, np.array(ks)) and np.array_equal(got_v, np.array(vs))


def _with_page_order(wl, order):
    wl2 = W.make_config(1)
    wl2.page_ids = np.asarray(order, dtype=np.int32)
    return wl2


def test_config1_all_page_orders_match_bruteforce_and_each_other():
    wl = W.make_config(1)
    ref = _bf_run(wl)
    outs = []
    for order in itertools.permutations(range(3)):
        w2 = _with_page_order(wl, order)
        res = _oracle_run(w2)
        _compare_to_bruteforce(w2, res, ref)
        outs.append(res)
        # default readout: the lane's last row (row 36)
        assert list(res["readout_rows"]) == [36]
        assert np.array_equal(res["readout"][0], res["O"][36].reshape(-1))
    for r in outs[1:]:
        assert np.array_equal(r["O"], outs[0]["O"]) and np.array_equal(r["LSE"], outs[0]["LSE"])


@pytest.mark.parametrize("seed,P,G,d", [(0, 1, 2, 16), (1, 2, 1, 16), (2, 4, 4, 8), (3, 16, 2, 16),
                                         (4, 8, 8, 8), (5, 16, 1, 32)])
def test_random_passes_match_bruteforce(seed, P, G, d):
    wl = W.make_random(seed, H_kv=2, G=G, d=d, P=P, num_lanes=5, max_rows=20, max_ctx=40)
    res = _oracle_run(wl)
    ref = _bf_run(wl)
    _compare_to_bruteforce(wl, res, ref)


HOLE_BITS = 0x3FC0  # bf16 1.5: what a never-written slot holds in the explicit-slot pins


@pytest.mark.parametrize("seed,P,G,d", [(0, 4, 2, 16), (1, 8, 1, 8), (2, 2, 4, 16), (3, 16, 2, 8), (4, 1, 8, 8)])
def test_explicit_slots_match_bruteforce(seed, P, G, d):
    """Rows that name their slots (State geometry): permuted and gapped slots,
    prefix slots above the frozen count rewritten, kv_len below some rows'
    slots, holes that keep the pool's fill, random positions; the paged oracle
    equals the dense brute force, which has no page table."""
    wl = W.make_explicit(seed, H_kv=2, G=G, d=d, P=P, num_lanes=5, max_rows=14, max_ctx=30)
    res = _oracle_run(wl, fill=HOLE_BITS)
    ref = _bf_run(wl, hole_bits=HOLE_BITS)
    _compare_to_bruteforce(wl, res, ref)


def test_explicit_generator_covers_the_geometry_cases():
    """Over a few seeds, make_explicit writes out of order, writes past kv_len,
    leaves holes below kv_len and rewrites prefix slots above the frozen count."""
    out_of_order = past = hole = rewrite = False
    for seed in range(5):
        _explicit_cases(W.make_explicit(seed, num_lanes=7), flags := {})
        out_of_order |= flags["out_of_order"]
        past |= flags["past"]
        hole |= flags["hole"]
        rewrite |= flags["rewrite"]
    assert out_of_order and past and hole and rewrite


def _explicit_cases(wl, flags):
    st, pre = wl.step, wl.prefix
    c = np.zeros(wl.num_lanes, np.int32)
    c, _ = oracle.fold(c, pre.indptr, pre.fold)
    out_of_order = past = hole = rewrite = False
    for lane in range(wl.num_lanes):
        r0, r1 = int(st.indptr[lane]), int(st.indptr[lane + 1])
        s_ = st.slots[r0:r1].astype(np.int64)
        ps = pre.slots[int(pre.indptr[lane]):int(pre.indptr[lane + 1])].astype(np.int64)
        k = int(c[lane])
        out_of_order |= bool(np.any(np.diff(s_) != 1))
        past |= bool(np.any(s_ >= int(st.kv_len[lane])))
        written = set(s_.tolist()) | set(ps.tolist())
        hole |= any(j not in written for j in range(int(st.kv_len[lane])))
        rewrite |= bool(set(s_.tolist()) & set(ps[ps >= k].tolist()))
    flags.update(out_of_order=out_of_order, past=past, hole=hole, rewrite=rewrite)


def test_nonfinite_slot_below_kv_len_is_outside_the_domain():
    """The step's precondition: slots below kv_len hold finite K/V. The oracle
    refuses a pass that breaks it and accepts non-finite bytes at or past kv_len."""
    wl = W.make_config(1)
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids, fill_bits=0x7FC0)
    st = wl.step
    c = np.zeros(1, np.int32)
    oracle.append(pool, c, st.indptr, st.positions, st.slots, st.k, st.v, wl.theta)
    O, _, _ = oracle.attend(pool, st.indptr, st.positions, st.slots, st.kv_len, st.q, wl.H_q, wl.theta, wl.sm_scale)
    assert np.isfinite(O).all()  # slots 37..47 hold NaN but lie past kv_len
    pg, off = pool.locate(0, 20)
    pool.v[pg, 1, off, 3] = 0x7FC0
    with pytest.raises(ValueError):
        oracle.attend(pool, st.indptr, st.positions, st.slots, st.kv_len, st.q, wl.H_q, wl.theta, wl.sm_scale)


def _hz(page_indptr, page_ids, indptr, slots, kv_len, committed=None, num_pages=8, P=4):
    pool = oracle.Pool(num_pages, P, 1, 2, page_indptr, page_ids)
    L = len(indptr) - 1
    return oracle.hazards(pool, np.zeros(L, np.int32) if committed is None else np.asarray(committed),
                          np.asarray(indptr), np.asarray(slots), np.asarray(kv_len))


def test_hazards_hand_worked():
    """Eq. (4) (reviews, section 5): W(a) and R(b) ∪ W(b) disjoint for lanes a ≠ b,
    on (page, offset) cells, and no cell written twice; pages of 4 slots."""
    DUP, SH = oracle.ST_DUP_WRITE, oracle.ST_SHARED_CELL
    # two lanes on disjoint pages, each writing and reading its own cells: no hazard
    assert _hz([0, 2, 3], [5, 1, 7], [0, 2, 3], [6, 7, 2], [8, 3]) == 0
    # one lane, two rows naming slot 3: a cell written twice
    assert _hz([0, 1], [2], [0, 2], [3, 3], [4]) == DUP
    # the same page listed twice in one lane: slots 1 and 5 are one cell
    assert _hz([0, 2], [6, 6], [0, 2], [1, 5], [6]) == DUP
    # lane 1 (no rows) shares page 3 read-only with lane 0 and reads slots 0..2; lane 0
    # writes offset 3 of that page (its slot 7): lane 1 does not read offset 3, no hazard ...
    assert _hz([0, 2, 3], [0, 3, 3], [0, 1, 1], [7], [8, 3]) == 0
    # ... but with kv_len 4 it does
    assert _hz([0, 2, 3], [0, 3, 3], [0, 1, 1], [7], [8, 4]) == SH
    # lane 1 writes that shared cell itself (slot 3 of its page 3), lane 0 reads it too
    assert _hz([0, 2, 3], [0, 3, 3], [0, 1, 2], [1, 3], [8, 4]) == SH
    # both lanes write the same cell: written twice, and by two lanes
    assert _hz([0, 1, 2], [4, 4], [0, 1, 2], [2, 2], [0, 0]) == DUP | SH
    # a suppressed write (frozen, or past capacity) is no write
    assert _hz([0, 1, 2], [4, 4], [0, 1, 2], [2, 2], [0, 0], committed=[3, 0]) == 0
    assert _hz([0, 1, 2], [4, 4], [0, 1, 2], [2, 9], [0, 0]) == 0
    # a lane reading cells it writes itself is the normal case
    assert _hz([0, 2], [1, 0], [0, 3], [4, 5, 6], [8]) == 0
    # every valid pass the generators build is hazard-free
    for seed in range(3):
        for wl in (W.make_explicit(seed), W.make_random(seed), W.make_config(3, seed=seed, scale="small")):
            pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
            c = np.zeros(wl.num_lanes, np.int32)
            if wl.prefix is not None:
                p = wl.prefix
                assert oracle.hazards(pool, c, p.indptr, p.slots, p.kv_len) == 0
                c, _ = oracle.fold(c, p.indptr, p.fold)
            st = wl.step
            assert oracle.hazards(pool, c, st.indptr, st.slots, st.kv_len) == 0


# ----------------------------------------------------------------------------- invariants

def _split_config1(split):
    """Config 1 as a prefix pass of `split` rows (folded all) followed by the rest."""
    wl = W.make_config(1)
    st = wl.step
    pre = W.Pass(indptr=np.array([0, split], np.int32), positions=st.positions[:split], slots=st.slots[:split],
                 kv_len=np.array([split], np.int32), fold=np.array([W.FOLD_ALL], np.int32),
                 k=st.k[:split], v=st.v[:split], q=st.q[:split])
    post = W.Pass(indptr=np.array([0, 37 - split], np.int32), positions=st.positions[split:], slots=st.slots[split:],
                  kv_len=np.array([37], np.int32), fold=np.array([W.FOLD_ALL], np.int32),
                  k=st.k[split:], v=st.v[split:], q=st.q[split:])
    return wl, pre, post


def test_whole_prompt_equals_prefix_then_continuation():
    wl = W.make_config(1)
    whole = _oracle_run(wl)
    for split in range(1, 37):
        _, pre, post = _split_config1(split)
        pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
        c = np.zeros(1, np.int32)
        r1 = oracle.step(pool, c, pre, wl.H_q, wl.theta, wl.sm_scale)
        r2 = oracle.step(pool, r1["committed"], post, wl.H_q, wl.theta, wl.sm_scale)
        assert np.array_equal(np.concatenate([r1["O"], r2["O"]]), whole["O"])
        assert np.array_equal(np.concatenate([r1["LSE"], r2["LSE"]]), whole["LSE"])
        assert np.array_equal(pool.k, whole["pool"].k) and np.array_equal(pool.v, whole["pool"].v)
        assert int(r2["committed"][0]) == 37


def test_all_causal_bitmap_equals_folding():
    wl = W.make_config(1)
    base = _oracle_run(wl)
    j = np.arange(64)
    rows = []
    for r in range(37):
        allowed = (j <= wl.step.slots[r])
        rows.append([int(sum(1 << b for b in range(32) if allowed[32 * w + b])) for w in range(2)])
    wl.mask_bits = np.array(rows, dtype=np.uint32).reshape(-1)
    wl.mask_word_offset = np.array([0, 74], dtype=np.int64)
    masked = _oracle_run(wl)
    assert np.array_equal(masked["O"], base["O"]) and np.array_equal(masked["LSE"], base["LSE"])


def test_single_slot_row_returns_its_value_exactly():
    wl = W.make_config(1)
    res = _oracle_run(wl)
    # row 0 of a fresh lane sees only slot 0: softmax weight 1
    pg, off = res["pool"].locate(0, 0)
    V0 = oracle.bf16_to_f64(res["pool"].v[pg, :, off, :])
    G = wl.H_q // wl.H_kv
    for h in range(wl.H_q):
        assert np.array_equal(res["O"][0, h], V0[h // G])


def test_zero_query_gives_mean_of_allowed_values():
    wl = W.make_config(1)
    wl.step.q[:] = 0
    res = _oracle_run(wl)
    K, V = res["pool"].lane_kv(0, 37)
    G = wl.H_q // wl.H_kv
    for r in (0, 5, 36):
        for h in range(wl.H_q):
            np.testing.assert_allclose(res["O"][r, h], V[: r + 1, h // G].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(res["LSE"][r, h] - math.log(r + 1)) < 1e-14


def test_empty_allowed_set_gives_zero_and_minus_inf():
    wl = W.make_config(1)
    wl.mask_bits = np.zeros(37 * 2, dtype=np.uint32)
    wl.mask_word_offset = np.array([0, 74], dtype=np.int64)
    res = _oracle_run(wl)
    assert np.all(res["O"] == 0) and np.all(np.isneginf(res["LSE"]))


def test_page_permutation_with_decoys_is_bit_invariant():
    wl = W.make_random(11, H_kv=2, G=2, d=16, P=4, num_lanes=5, max_rows=20, max_ctx=40, extra_pages=6)
    a = _oracle_run(wl, fill=0x7FC0)
    rng = np.random.default_rng(5)
    wl.page_ids = rng.permutation(wl.num_pages)[: len(wl.page_ids)].astype(np.int32)
    b = _oracle_run(wl, fill=0x7FC0)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["LSE"], b["LSE"])
    assert np.all(np.isfinite(a["O"]))


# ----------------------------------------------------------------------------- fold, readout, errors

def test_fold_closed_form_and_channel_clamp():
    indptr = np.array([0, 3, 3, 11, 19, 27, 28])
    spec = np.array([W.FOLD_ALL, W.FOLD_ALL, 5, W.FOLD_CHANNEL, W.FOLD_CHANNEL, 0])
    chan = np.array([0, 0, 0, 4, 12, 0])
    c0 = np.array([10, 20, 30, 40, 50, 60])
    c1, st = oracle.fold(c0, indptr, spec, chan)
    assert list(c1) == [13, 20, 35, 44, 58, 60]
    assert st == oracle.ST_FOLD_CLAMP
    c2, st2 = oracle.fold(c0, indptr, spec, np.array([0, 0, 0, 4, 8, 0]))
    assert list(c2) == [13, 20, 35, 44, 58, 60] and st2 == 0
    c3, st3 = oracle.fold(c0, indptr, np.array([9, -7, 0, 0, 0, 0]), None)
    assert list(c3) == [13, 20, 30, 40, 50, 60] and st3 == oracle.ST_FOLD_CLAMP


def test_default_readout_is_last_row_of_each_lane():
    g = _load("lanes_indptr.json")
    assert list(oracle.readout_rows(np.array(g["indptr"]))) == g["default_readout_rows"]
    assert list(oracle.readout_rows(np.array([0, 0, 4, 4, 5]))) == [3, 4]
    O = np.arange(12.0).reshape(6, 2)
    out, st = oracle.readout(O, 6, [5, 0, 9])
    assert st == oracle.ST_READOUT_RANGE and out.tolist() == [[10, 11], [0, 1], [0, 0]]


def test_suppressed_writes_and_status():
    wl = W.make_config(1)
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids, fill_bits=0x1234)
    st = wl.step
    slots = st.slots.copy()
    slots[3] = 48          # capacity is 3 pages x 16 = 48
    slots[4] = -1
    s = oracle.append(pool, np.array([2]), st.indptr, st.positions, slots, st.k, st.v, wl.theta)
    assert s == oracle.ST_SLOT_RANGE | oracle.ST_FROZEN
    for bad_slot in (0, 1):  # frozen
        pg, off = pool.locate(0, bad_slot)
        assert np.all(pool.k[pg, :, off, :] == 0x1234)
    pg, off = pool.locate(0, 2)
    assert not np.all(pool.v[pg, :, off, :] == 0x1234)


def test_kv_len_beyond_capacity_is_clamped_and_flagged():
    wl = W.make_config(1)
    wl.step.kv_len[:] = 60
    res = _oracle_run(wl)
    assert res["status"] & oracle.ST_KVLEN
    wl2 = W.make_config(1)
    base = _oracle_run(wl2)
    assert np.array_equal(res["O"], base["O"])


# ----------------------------------------------------------------------------- run-ahead geometry

def test_advance_hand_worked_example():
    # lane 0: one row after 5 committed slots, positions shifted by 10
    # lane 1: three rows on an empty lane; lane 2: no rows; lane 3: two rows after 3, shift -3
    pos, slots, kv = oracle.advance([5, 0, 7, 3], [0, 1, 4, 4, 6], [10, 0, 2, -3])
    assert slots.tolist() == [5, 0, 1, 2, 3, 4]
    assert pos.tolist() == [15, 0, 1, 2, 0, 1]
    assert kv.tolist() == [6, 3, 7, 5]
    pos0, slots0, _ = oracle.advance([5, 0, 7, 3], [0, 1, 4, 4, 6])
    assert pos0.tolist() == slots0.tolist()


def test_speculative_loop_with_rejections_equals_whole_prompt():
    """Draft rows after the true ones are appended, attended and then rejected by
    the fold; the next pass's geometry (from committed_len) rewrites their slots.
    Rows of the true sequence must see exactly what the single 37-row pass saw."""
    wl = W.make_config(1)
    whole = _oracle_run(wl)
    st = wl.step
    junk_k, junk_v, junk_q = st.k[::-1].copy(), st.v[::-1].copy(), st.q[::-1].copy()
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
    c = np.zeros(1, np.int32)
    schedule = [(1, 3), (4, 0), (2, 5), (3, 2), (7, 1), (1, 4), (8, 3), (5, 0), (6, 2)]
    assert sum(a for a, _ in schedule) == 37
    got = {}
    j = 0
    for accept, drafts in schedule:
        t0 = int(c[0])
        n = accept + drafts
        indptr = np.array([0, n], np.int32)
        pos, slots, kv = oracle.advance(c, indptr)
        idx = np.arange(t0, t0 + accept)
        jj = np.arange(j, j + drafts) % 37
        j += drafts
        p = W.Pass(indptr=indptr, positions=pos, slots=slots, kv_len=kv, fold=np.array([accept], np.int32),
                   k=np.concatenate([st.k[idx], junk_k[jj]]), v=np.concatenate([st.v[idx], junk_v[jj]]),
                   q=np.concatenate([st.q[idx], junk_q[jj]]))
        r = oracle.step(pool, c, p, wl.H_q, wl.theta, wl.sm_scale)
        assert r["status"] == 0
        for i in range(accept):
            got[t0 + i] = (r["O"][i], r["LSE"][i])
        c = r["committed"]
    assert int(c[0]) == 37
    for t in range(37):
        assert np.array_equal(got[t][0], whole["O"][t]) and np.array_equal(got[t][1], whole["LSE"][t])
    K1, V1 = pool.lane_kv(0, 37)
    K0, V0 = whole["pool"].lane_kv(0, 37)
    assert np.array_equal(K1, K0) and np.array_equal(V1, V0)


def test_run_ahead_positions_are_offset_slots():
    ra = W.make_run_ahead(3, H_kv=1, G=2, d=16, P=4, num_lanes=6, passes=3, max_prompt=20)
    c = np.diff(ra.prefix.indptr).astype(np.int32) if ra.prefix is not None else np.zeros(ra.num_lanes, np.int32)
    pos, slots, kv = oracle.advance(c, ra.indptr, ra.pos_offset)
    for lane in range(ra.num_lanes):
        r0, r1 = ra.indptr[lane], ra.indptr[lane + 1]
        assert np.array_equal(pos[r0:r1] - slots[r0:r1], np.full(r1 - r0, ra.pos_offset[lane]))
        assert kv[lane] == c[lane] + (r1 - r0)
        if r1 > r0:
            assert slots[r1 - 1] == kv[lane] - 1


# ----------------------------------------------------------------------------- attention mass

def _oracle_mass(wl, res):
    st = wl.step
    return oracle.attn_mass(res["pool"], st.indptr, st.positions, st.slots, st.kv_len, st.q, wl.H_q, wl.theta,
                            wl.sm_scale, wl.mask_bits, wl.mask_word_offset)


@pytest.mark.parametrize("seed,P,G,d", [(0, 1, 2, 16), (2, 4, 4, 8), (3, 16, 2, 16), (5, 16, 1, 32)])
def test_attn_mass_matches_bruteforce(seed, P, G, d):
    wl = W.make_random(seed, H_kv=2, G=G, d=d, P=P, num_lanes=5, max_rows=20, max_ctx=40)
    res = _oracle_run(wl)
    mass = _oracle_mass(wl, res)
    ref = _bf_run(wl)
    want = np.zeros_like(mass)
    for lane, entries in enumerate(ref["mass"]):
        base = int(wl.page_indptr[lane]) * wl.P
        for (g, j), v in entries.items():
            want[g, base + j] += v
    assert np.max(np.abs(mass - want)) <= 1e-12


def test_attn_mass_sums_to_reading_pairs():
    # each (row, query head) that reads any slot spreads exactly one unit of mass
    for seed in range(4):
        wl = W.make_random(40 + seed, H_kv=2, G=4, d=16, P=8, num_lanes=6, max_rows=24, max_ctx=60)
        res = _oracle_run(wl)
        mass = _oracle_mass(wl, res)
        pairs = int(np.isfinite(res["LSE"]).sum())
        assert abs(mass.sum() - pairs) <= 1e-9 * max(pairs, 1)
        assert np.all(mass >= 0)


def test_attn_mass_zero_query_is_uniform():
    wl = W.make_config(1)
    wl.step.q[:] = 0
    res = _oracle_run(wl)
    mass = _oracle_mass(wl, res)
    G = wl.H_q // wl.H_kv
    # row r reads slots 0..r with probability 1/(r+1) each, for each of the G heads of a group
    want = np.array([G * sum(1.0 / (r + 1) for r in range(j, 37)) for j in range(37)])
    base = int(wl.page_indptr[0]) * wl.P
    for g in range(wl.H_kv):
        np.testing.assert_allclose(mass[g, base:base + 37], want, rtol=1e-13, atol=0)
        assert np.all(mass[g, base + 37:] == 0)


# ----------------------------------------------------------------------------- projection-site LoRA

def test_lora_matches_bruteforce():
    ip = np.array([0, 2, 2, 5, 6], dtype=np.int32)
    lw = W.make_lora(7, ip, d_in=8, d_out=6, rank=3, num_adapters=3, none_frac=0.0)
    lw.adapter[:] = [2, 0, 1, -1]
    out, exact, st = oracle.lora(lw.x, lw.y, lw.adapter, ip, lw.a, lw.b, lw.scale)
    bits, ex = bf.lora(lw.x.tolist(), lw.y.tolist(), lw.adapter, ip, lw.a.tolist(), lw.b.tolist(),
                       [float(s) for s in lw.scale])
    assert st == 0
    assert out.tolist() == bits
    assert np.max(np.abs(exact - np.array(ex))) <= 1e-12
    assert np.array_equal(out[5], lw.y[5])  # lane 3 has no adapter


def test_lora_zero_b_and_out_of_range_id_keep_y():
    ip = np.array([0, 3, 7], dtype=np.int32)
    lw = W.make_lora(3, ip, d_in=16, d_out=8, rank=4, num_adapters=2, none_frac=0.0)
    lw.adapter[:] = [0, 5]
    lw.b[0] = 0
    out, _, st = oracle.lora(lw.x, lw.y, lw.adapter, ip, lw.a, lw.b, lw.scale)
    assert np.array_equal(out, lw.y) and st == oracle.ST_ADAPTER


def test_lora_rank_one_closed_form():
    # A = e_j (selects x[:, j]), B = a column c: out = y + s * c * x_j, element by element
    ip = np.array([0, 4], dtype=np.int32)
    lw = W.make_lora(5, ip, d_in=12, d_out=10, rank=1, num_adapters=1, none_frac=0.0)
    j = 7
    lw.a[:] = 0
    lw.a[0, 0, j] = 0x3F80  # 1.0
    out, exact, _ = oracle.lora(lw.x, lw.y, lw.adapter, ip, lw.a, lw.b, lw.scale)
    c = oracle.bf16_to_f64(lw.b[0, :, 0])
    xj = oracle.bf16_to_f64(lw.x[:, j])
    want = oracle.bf16_to_f64(lw.y) + float(lw.scale[0]) * np.outer(xj, c)
    assert np.array_equal(exact, want)
    assert np.array_equal(out, oracle.f64_to_bf16(want))


def test_ia3_matches_exact_rounding_and_closed_forms():
    ip = np.array([0, 3, 3, 7, 9], dtype=np.int32)
    rng = np.random.default_rng(11)
    y = W.bf16_bits_from_f32(rng.standard_normal((9, 16)).astype(np.float32))
    scale = W.bf16_bits_from_f32(rng.uniform(0.1, 3.0, (2, 16)).astype(np.float32))
    adapter = np.array([1, 0, -1, 0], dtype=np.int32)
    out, st = oracle.ia3(y, adapter, ip, scale)
    assert st == 0
    for lane in range(4):
        for r in range(ip[lane], ip[lane + 1]):
            for c in range(16):
                k = adapter[lane]
                want = int(y[r, c]) if k < 0 else bf.bf16_round_exact(bf.bf16_value(y[r, c]) * bf.bf16_value(scale[k, c]))
                assert int(out[r, c]) == want
    ones = np.full((1, 16), 0x3F80, np.uint16)          # 1.0: y unchanged, bit for bit
    assert np.array_equal(oracle.ia3(y, np.zeros(4, np.int32), ip, ones)[0], y)
    twos = np.full((1, 16), 0x4000, np.uint16)          # 2.0: exponent + 1
    o2, _ = oracle.ia3(y, np.zeros(4, np.int32), ip, twos)
    nz = (y & 0x7FFF) != 0
    assert np.array_equal(o2[nz], (y[nz] + 0x80).astype(np.uint16))
    _, st = oracle.ia3(y, np.array([0, 0, 5, 0], np.int32), ip, ones)
    assert st == oracle.ST_ADAPTER


# ---- score-driven eviction (TOVA step): selection and bitmaps

def test_order_key_sorts_like_the_floats():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=200).astype(np.float32) * 10.0 ** rng.integers(-30, 30, size=200),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45], dtype=np.float32)]).astype(np.float32)
    keys = oracle.order_key(x)
    by_key = x[np.argsort(keys, kind="stable")]
    # equal floats may only differ as -0.0 / +0.0, which the key orders -0 < +0
    assert np.array_equal(by_key, np.sort(x, kind="stable"))
    assert oracle.order_key(np.float32(-0.0)) < oracle.order_key(np.float32(0.0))


def _keep_by_rank(keys, cand, k):
    """Brute force: a candidate is kept iff fewer than k candidates beat it
    (larger key, or equal key at a lower slot)."""
    keep = np.zeros(len(keys), dtype=bool)
    for j in np.nonzero(cand)[0]:
        rank = sum(1 for i in np.nonzero(cand)[0] if keys[i] > keys[j] or (keys[i] == keys[j] and i < j))
        keep[j] = rank < k
    return keep


@pytest.mark.parametrize("seed", range(6))
def test_tova_keep_matches_rank_definition(seed):
    rng = np.random.default_rng(100 + seed)
    P, H, L = 8, int(rng.integers(1, 4)), 4
    pages = rng.integers(1, 6, size=L)
    page_indptr = np.concatenate([[0], np.cumsum(pages)])
    S = int(page_indptr[-1]) * P
    # few distinct levels, so equal keys are common
    mass = (rng.integers(0, 4, size=(H, S)) * 0.25).astype(np.float32)
    committed = np.array([rng.integers(0, pages[l] * P + 1) for l in range(L)])
    budget = rng.integers(-1, 40, size=L)
    prev_limit = np.array([rng.integers(0, c + 1) for c in committed])
    prev_keep = [rng.random(c) < 0.6 for c in committed]
    for pk in (None, prev_keep):
        got = oracle.tova_keep(mass, page_indptr, P, committed, budget, pk, prev_limit)
        for lane in range(L):
            c = int(committed[lane])
            keys = oracle.order_key(mass[:, page_indptr[lane] * P:page_indptr[lane] * P + c].sum(axis=0, dtype=np.float32))
            cand = np.ones(c, dtype=bool)
            if pk is not None:
                cand[:prev_limit[lane]] = pk[lane][:prev_limit[lane]]
            k = min(max(int(budget[lane]), 0), int(cand.sum()))
            assert np.array_equal(got[lane], _keep_by_rank(keys, cand, k)), (seed, lane)


def test_tova_keep_special_cases():
    P = 8
    page_indptr = np.array([0, 2])
    mass = np.zeros((2, 16), dtype=np.float32)
    mass[0, :10] = [3, 1, 4, 1, 5, 9, 2, 6, 5, 3]
    mass[1, :10] = [0, 0, 0, 0, 0, 0, 0, 0, 0, 1]        # head sums: [3,1,4,1,5,9,2,6,5,4]
    c = np.array([10])
    # top 3 by score: 9 (slot 5), 6 (slot 7), then the two 5s -> the lower slot 4
    keep = oracle.tova_keep(mass, page_indptr, P, c, [3])[0]
    assert np.nonzero(keep)[0].tolist() == [4, 5, 7]
    assert oracle.tova_keep(mass, page_indptr, P, c, [0])[0].sum() == 0
    assert oracle.tova_keep(mass, page_indptr, P, c, [10])[0].all()
    assert oracle.tova_keep(mass, page_indptr, P, c, [99])[0].all()
    # equal scores everywhere: the lowest slots
    flat = np.ones((1, 16), dtype=np.float32)
    assert np.nonzero(oracle.tova_keep(flat, page_indptr, P, c, [4])[0])[0].tolist() == [0, 1, 2, 3]
    # a slot dropped earlier stays dropped, however large its score
    pk = [np.array([1, 1, 1, 1, 1, 0, 1, 1, 1, 1], dtype=bool)]
    keep = oracle.tova_keep(mass, page_indptr, P, c, [3], pk, [8])[0]
    assert not keep[5]
    assert np.nonzero(keep)[0].tolist() == [4, 7, 8]   # scores 6 (slot 7), then 5s at slots 4 and 8
    # slots at or past prev_limit are candidates even without a keep bit
    pk0 = [np.zeros(10, dtype=bool)]
    assert np.nonzero(oracle.tova_keep(mass, page_indptr, P, c, [5], pk0, [8])[0])[0].tolist() == [8, 9]


def test_tova_mask_hand_worked_and_causal_when_all_kept():
    # one lane: 5 old slots, keep {0, 3}; three new rows at slots 5, 6, 7; kv_len 8
    keep = [np.array([1, 0, 0, 1, 0], dtype=bool)]
    words, st = oracle.tova_mask(keep, [0, 3], [5, 6, 7], [8], [5], [1])
    assert st == 0
    assert words[0].tolist() == [0b00101001, 0b01101001, 0b11101001]
    # too few words per row for kv_len: flagged
    _, st = oracle.tova_mask(keep, [0, 3], [5, 6, 7], [40], [5], [1])
    assert st == oracle.ST_MASK_SHORT
    # every old slot kept: the bitmap is the slot-order rule attend() applies without a mask
    rng = np.random.default_rng(7)
    c, n = 37, 6
    slots = c + rng.permutation(n)
    kv = c + n
    words, _ = oracle.tova_mask([np.ones(c, dtype=bool)], [0, n], slots, [kv], [c], [2])
    for t in range(n):
        bits = [j for j in range(kv) if (int(words[0][2 * t + (j >> 5)]) >> (j & 31)) & 1]
        A, _ = oracle.allowed_slots(0, t, kv, slots, np.array([0, n]))
        assert bits == list(A)
