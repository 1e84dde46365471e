"""GPU parity of the repeating decode loop: fp_advance writes each pass's
geometry from committed_len on the device (no host round trip between passes),
against the oracle's loop that derives the same geometry on the host.

Covers speculative acceptance counts from a device channel (including
out-of-range counts that the fold clamps), idle lanes, position offsets, and
one pass captured in a HIP graph and replayed pass after pass.
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


def _say(*a):
    print(*a, flush=True)


def _run_eager(lp, passes):
    import torch

    rec = []
    for t in range(passes):
        lp.load(t)
        lp.one_pass()
        rec.append(dict(O=lp.out.clone(), LSE=lp.lse.clone(), positions=lp.geom.positions.clone(),
                        slots=lp.geom.slots.clone(), kv_len=lp.geom.kv_len.clone(),
                        committed=lp.pool.committed_len.clone(), dst=lp.dst.clone()))
    torch.cuda.synchronize()
    return rec


def _check_against_oracle(lp, rec, ref):
    ra = lp.ra
    last = ra.indptr[1:][np.diff(ra.indptr) > 0] - 1
    for t, (g, r) in enumerate(zip(rec, ref["passes"])):
        for key in ("positions", "slots", "kv_len", "committed"):
            assert g[key].cpu().numpy().tolist() == r[key].tolist(), f"pass {t}: {key} differs"
        O = g["O"].cpu().numpy().astype(np.float64)
        L = g["LSE"].cpu().numpy().astype(np.float64)
        pu.compare_arrays(O, L, r["O"], r["LSE"])
        out = g["O"].cpu().numpy().reshape(O.shape[0], -1)
        assert np.array_equal(g["dst"].cpu().numpy(), out[last]), f"pass {t}: readout differs"
    K, V = lp.pool_logical()
    assert np.array_equal(V, ref["pool"].v)
    assert pu.ulp_distance(K, ref["pool"].k).max() <= 1
    assert int(lp.status.cpu()[0]) == ref["status"]


@pytest.mark.parametrize("seed,H_kv,G,d,P", [(0, 2, 4, 128, 16), (1, 1, 8, 64, 8), (2, 4, 2, 128, 32),
                                             (3, 8, 4, 128, 16)])
def test_run_ahead_loop_device_geometry(seed, H_kv, G, d, P):
    from ragged_paged_kv_fp_amd import runner

    ra = W.make_run_ahead(seed, H_kv=H_kv, G=G, d=d, P=P, num_lanes=9, passes=6, max_prompt=400)
    _say(f"run-ahead seed {seed}: H_kv={H_kv} G={G} d={d} P={P} rows/pass={int(ra.indptr[-1])}")
    ref = pu.oracle_run_ahead(ra)
    lp = runner.RunAheadLoop(ra)
    rec = _run_eager(lp, ra.passes)
    _check_against_oracle(lp, rec, ref)


def test_run_ahead_graph_replay_matches_eager_and_oracle():
    import torch

    from ragged_paged_kv_fp_amd import runner

    ra = W.make_run_ahead(7, H_kv=2, G=4, d=128, P=16, num_lanes=12, passes=8, max_prompt=600)
    _say(f"graph replay: rows/pass={int(ra.indptr[-1])} passes={ra.passes}")
    ref = pu.oracle_run_ahead(ra)
    eager = runner.RunAheadLoop(ra)
    rec_e = _run_eager(eager, ra.passes)
    lp = runner.RunAheadLoop(ra)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lp.one_pass()
    torch.cuda.synchronize()
    rec = []
    for t in range(ra.passes):
        lp.load(t)
        graph.replay()
        rec.append(dict(O=lp.out.clone(), LSE=lp.lse.clone(), positions=lp.geom.positions.clone(),
                        slots=lp.geom.slots.clone(), kv_len=lp.geom.kv_len.clone(),
                        committed=lp.pool.committed_len.clone(), dst=lp.dst.clone()))
        if t % 3 == 1:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for t, (g, e) in enumerate(zip(rec, rec_e)):
        for key in g:
            assert torch.equal(g[key], e[key]), f"replay {t}: {key} differs from the eager pass"
    _check_against_oracle(lp, rec, ref)
