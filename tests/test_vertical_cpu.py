"""Vertical batching of a frame (fp_vertical_merge, runner.vertical_groups): a
prefix pass and its continuation on the same lanes merged into one pass (the
reviews' section 5: such a pair can share one dispatch when the order between
them is kept). Pinned on the CPU against the oracle: the merged pass gives bit
for bit the same stored K/V, outputs, LSE and committed lengths as the two
passes in sequence; passes that one pass cannot replace are refused."""

import numpy as np
import pytest

import oracle
import workloads as W


@pytest.fixture(scope="module")
def lib():
    import os

    from ragged_paged_kv_fp_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from ragged_paged_kv_fp_amd import build

        build.build()
    return _lib.load()


def _oracle_passes(wl, passes, committed0):
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
    c = np.zeros(wl.num_lanes, np.int32)
    if wl.prefix is not None:
        p = wl.prefix
        oracle.append(pool, c, p.indptr, p.positions, p.slots, p.k, p.v, wl.theta)
        c, _ = oracle.fold(c, p.indptr, p.fold)
    assert c.tolist() == list(committed0)
    res = []
    for p in passes:
        r = oracle.step(pool, c, p, wl.H_q, wl.theta, wl.sm_scale)
        c = r["committed"]
        res.append(r)
    return pool, res, c


def _committed0(wl):
    c = np.zeros(wl.num_lanes, np.int32)
    if wl.prefix is not None:
        c, _ = oracle.fold(c, wl.prefix.indptr, wl.prefix.fold)
    return c


def _split3(st, rng):
    n = np.diff(st.indptr)
    f1 = np.array([int(rng.integers(0, m + 1)) for m in n])
    A, rest = W.split_pass(st, f1)
    f2 = np.array([int(rng.integers(0, m + 1)) for m in np.diff(rest.indptr)])
    B, C = W.split_pass(rest, f2)
    return [A, B, C]


@pytest.mark.parametrize("wl_kind,seed", [("c1", 0), ("c3", 1), ("c3", 2), ("rand", 3), ("rand", 4), ("c2", 5)])
def test_merged_pass_equals_passes_in_sequence(lib, wl_kind, seed):
    from ragged_paged_kv_fp_amd import runner

    if wl_kind == "c1":
        wl = W.make_config(1)
    elif wl_kind == "rand":
        wl = W.make_random(seed, H_kv=2, G=2, d=16, P=4, num_lanes=5, max_rows=20, max_ctx=30, masked=False,
                           fold_modes=False)
    else:
        wl = W.make_config(int(wl_kind[1]), seed=seed, scale="small")
    rng = np.random.default_rng(seed)
    passes = _split3(wl.step, rng)
    c0 = _committed0(wl)
    groups = runner.vertical_groups(passes, c0, wl.page_indptr, wl.P)
    assert len(groups) == 1, "a prefix chain with fold all must merge into one pass"
    merged = groups[0]["pass"]
    pool_s, seq, c_s = _oracle_passes(wl, passes, c0)
    pool_m, (res_m,), c_m = _oracle_passes(wl, [merged], c0)
    assert np.array_equal(pool_s.k, pool_m.k) and np.array_equal(pool_s.v, pool_m.v)
    assert c_s.tolist() == c_m.tolist()
    assert res_m["status"] == 0 and all(r["status"] == 0 for r in seq)
    for (idx, rows), r in zip(groups[0]["parts"], seq):
        assert np.array_equal(res_m["O"][rows], r["O"]), idx
        assert np.array_equal(res_m["LSE"][rows], r["LSE"]), idx


def _pair(wl, rng):
    n = np.diff(wl.step.indptr)
    return W.split_pass(wl.step, np.array([int(rng.integers(1, m + 1)) if m else 0 for m in n]))


def test_passes_one_pass_cannot_replace_are_refused(lib):
    from ragged_paged_kv_fp_amd import api

    wl = W.make_config(3, seed=7, scale="small")
    c0 = _committed0(wl)
    A, B = _pair(wl, np.random.default_rng(7))
    ok = api.vertical_merge(A, B, c0, wl.page_indptr, wl.P)
    assert ok is not None and ok["indptr"][-1] == A.num_rows + B.num_rows

    def refused(a, b, c=c0):
        return api.vertical_merge(a, b, c, wl.page_indptr, wl.P) is None

    lane = int(np.argmax(np.diff(A.indptr)))
    r0 = int(A.indptr[lane])
    import copy
    # A does not freeze what it wrote: B would not see it as history
    a2 = copy.deepcopy(A); a2.fold = a2.fold.copy(); a2.fold[lane] = 0
    assert refused(a2, B)
    # A's rows are not the slots right after the committed prefix
    a3 = copy.deepcopy(A); a3.slots = a3.slots.copy(); a3.slots[r0] += 1
    assert refused(a3, B)
    # B rewrites a slot A froze
    b4 = copy.deepcopy(B); b4.slots = b4.slots.copy()
    lb = next(l for l in range(B.num_lanes) if B.indptr[l + 1] > B.indptr[l] and A.indptr[l + 1] > A.indptr[l])
    b4.slots[int(B.indptr[lb])] = int(A.slots[int(A.indptr[lb])])
    assert refused(A, b4)
    # B's fold count comes from a device channel: the merged count is not known on the host
    b5 = copy.deepcopy(B); b5.fold = b5.fold.copy(); b5.fold[lb] = W.FOLD_CHANNEL
    assert refused(A, b5)
    # B reads fewer slots than A's rows need
    b6 = copy.deepcopy(B); b6.kv_len = b6.kv_len.copy(); b6.kv_len[lb] = int(c0[lb])
    assert refused(A, b6)
    # a kv_len beyond the lane's pages (the two passes would each flag and clamp it)
    a7 = copy.deepcopy(A); a7.kv_len = a7.kv_len.copy(); a7.kv_len[lane] = 10 ** 6
    assert refused(a7, B)
    # committed lengths other than the ones A starts from
    assert refused(A, B, c0 + 1)


def test_groups_follow_committed_lengths_across_unmergeable_passes(lib):
    """A frame [A, B, X, Y] where X cannot follow B (it rewrites B's frozen
    slots) merges A+B and then X+Y, the latter from the committed lengths A+B
    leave behind."""
    from ragged_paged_kv_fp_amd import runner

    wl = W.make_config(1)
    st = wl.step
    A, rest = W.split_pass(st, [10])
    B, _ = W.split_pass(rest, [27])
    X, Y = W.split_pass(st, [20])  # the same rows again from slot 0: frozen by A+B
    groups = runner.vertical_groups([A, B, X, Y], np.zeros(1, np.int32), wl.page_indptr, wl.P)
    assert [len(g["parts"]) for g in groups] == [2, 1, 1]
