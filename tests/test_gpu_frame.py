"""Frames: several passes submitted back to back over one pool (runner.Frame).

A pass split per lane into a prefix pass (folded all) and its continuation,
run as a two-pass frame, must give the whole pass's results (prefix then
continuation equals the whole prompt, here with both passes in one frame);
the frame captured once in a HIP graph and replayed several times, with
eager work and synchronisations between replays, must reproduce the eager
frame bit for bit.
"""

import numpy as np
import pytest

import parity_util as pu
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_paged_kv_fp_amd import _lib

    _lib.load()


def _split_rows(st, first):
    a, b = [], []
    for lane in range(st.num_lanes):
        r0, r1 = int(st.indptr[lane]), int(st.indptr[lane + 1])
        s = min(max(int(first[lane]), 0), r1 - r0)
        a += list(range(r0, r0 + s))
        b += list(range(r0 + s, r1))
    return np.asarray(a, dtype=np.int64), np.asarray(b, dtype=np.int64)


@pytest.mark.parametrize("cfg,seed", [(1, 0), (3, 2), (3, 5)])
def test_frame_prefix_and_continuation(cfg, seed):
    import torch

    from ragged_paged_kv_fp_amd import runner

    wl = W.make_config(cfg, seed=seed, scale="small" if cfg > 1 else "full")
    st = wl.step
    assert np.all(st.fold == W.FOLD_ALL) and wl.mask_bits is None
    rng = np.random.default_rng(seed)
    n = np.diff(st.indptr)
    first = np.array([int(rng.integers(0, m + 1)) for m in n])
    A, B = W.split_pass(st, first)
    a_rows, b_rows = _split_rows(st, first)
    print(f"frame config {cfg} seed {seed}: rows {st.num_rows} -> {A.num_rows} + {B.num_rows}", flush=True)
    ref = pu.oracle_run(wl)
    ds = runner.DeviceStep(wl)
    ds.run_prefix()
    fr = runner.Frame(ds.pool, [A, B], wl.H_q, wl.theta, wl.sm_scale)
    fr.run()
    torch.cuda.synchronize()
    O = np.zeros((st.num_rows, wl.H_q, wl.d))
    L = np.zeros((st.num_rows, wl.H_q))
    for rows, it in ((a_rows, fr.items[0]), (b_rows, fr.items[1])):
        O[rows] = it["out"].cpu().numpy()
        L[rows] = it["lse"].cpu().numpy()
    pu.compare_arrays(O, L, ref["O"], ref["LSE"])
    ds.geom = fr.items[1]["geom"]
    pu.compare_pool(ds, ref)
    assert ds.pool.committed_len.cpu().numpy().tolist() == ref["committed"].tolist()
    assert int(fr.status.cpu()[0]) == 0
    eager = [(it["out"].clone(), it["lse"].clone(), it["dst"].clone()) for it in fr.items]
    pool0 = ds.pool_t.clone()
    fr.capture()
    for rep in range(4):
        for it in fr.items:  # eager work between replays
            it["out"].zero_()
        fr.replay()
        if rep % 2:
            torch.cuda.synchronize()
        for (o, l, d), it in zip(eager, fr.items):
            assert torch.equal(o, it["out"]) and torch.equal(l, it["lse"]) and torch.equal(d, it["dst"]), rep
        assert torch.equal(pool0, ds.pool_t)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg,seed", [(1, 0), (3, 2), (3, 5), (2, 1)])
def test_vertical_frame_one_pass(cfg, seed):
    """The same split frame with vertical batching: the prefix pass and its
    continuation run as one pass (one append, one attend); outputs equal the
    oracle's whole pass, the stored K/V and committed lengths equal it bit for
    bit, each original pass's readout rows are its default ones, and the
    merged frame replayed from a HIP graph reproduces the eager one."""
    import torch

    from ragged_paged_kv_fp_amd import runner

    wl = W.make_config(cfg, seed=seed, scale="small" if cfg > 1 else "full")
    st = wl.step
    rng = np.random.default_rng(seed)
    first = np.array([int(rng.integers(0, m + 1)) for m in np.diff(st.indptr)])
    A, B = W.split_pass(st, first)
    a_rows, b_rows = _split_rows(st, first)
    ref = pu.oracle_run(wl)
    ds = runner.DeviceStep(wl)
    ds.run_prefix()
    fr = runner.Frame(ds.pool, [A, B], wl.H_q, wl.theta, wl.sm_scale, vertical=True)
    assert len(fr.items) == 1, "prefix + continuation should merge into one pass"
    fr.run()
    torch.cuda.synchronize()
    O = np.zeros((st.num_rows, wl.H_q, wl.d))
    L = np.zeros((st.num_rows, wl.H_q))
    parts = fr.parts()
    for (idx, out, lse), rows in zip(parts, (a_rows, b_rows)):
        O[rows] = out.cpu().numpy()
        L[rows] = lse.cpu().numpy()
    pu.compare_arrays(O, L, ref["O"], ref["LSE"])
    ds.geom = fr.items[0]["geom"]
    pu.compare_pool(ds, ref)
    assert ds.pool.committed_len.cpu().numpy().tolist() == ref["committed"].tolist()
    assert int(fr.status.cpu()[0]) == 0
    for idx, out, _ in parts:
        p = (A, B)[idx]
        ip = np.asarray(p.indptr, np.int64)
        last = (ip[1:] - 1)[np.diff(ip) > 0]
        assert torch.equal(fr.readout_of(idx), out.reshape(out.shape[0], -1)[torch.as_tensor(last, device=out.device)])
    eager = (fr.items[0]["out"].clone(), fr.items[0]["lse"].clone(), fr.items[0]["dst"].clone())
    fr.capture()
    for rep in range(3):
        fr.items[0]["out"].zero_()
        fr.replay()
        torch.cuda.synchronize()
        assert torch.equal(eager[0], fr.items[0]["out"]) and torch.equal(eager[2], fr.items[0]["dst"]), rep
