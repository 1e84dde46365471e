"""fp_attend_noalloc (the entry point for callers that cannot allocate: the
library's static device scratch instead of a caller workspace) against
fp_attend on the same inputs, through the C ABI: bit-identical outputs on two
calls in a row, the second with a smaller pass, and both within the oracle's
tolerance; a pass larger than the scratch is rejected before anything runs."""

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


def _noalloc_matches(wl):
    import torch

    from ragged_paged_kv_fp_amd import api

    print(f"noalloc: {wl.name} lanes={wl.num_lanes} rows={wl.step.num_rows}", flush=True)
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)  # append -> fp_attend (caller workspace) -> fold -> readout
    out = torch.full_like(ds.out, float("nan"))
    lse = torch.full_like(ds.lse, float("nan"))
    status = torch.zeros_like(ds.status)
    api.attend_noalloc(ds.pool, ds.geom, ds.q, wl.H_q, wl.theta, wl.sm_scale, out, status, lse, ds.mask)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == 0 and int(ds.status.cpu()[0]) == ref["status"] == 0
    assert np.array_equal(out.cpu().numpy(), ds.out.cpu().numpy()), "noalloc output differs from fp_attend"
    assert np.array_equal(lse.cpu().numpy(), ds.lse.cpu().numpy()), "noalloc lse differs from fp_attend"
    pu.compare_arrays(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref["O"], ref["LSE"])


def test_noalloc_equals_attend_twice_second_smaller():
    from ragged_paged_kv_fp_amd import api

    big = W.make_config(3, seed=0, scale="small")     # prefill and decode lanes, split merges
    small = W.make_config(1, seed=0)                    # one 37-row lane
    assert big.step.num_rows > small.step.num_rows
    _noalloc_matches(big)
    _noalloc_matches(small)
    # a masked long-context pass too (tile lists live in the scratch as well)
    _noalloc_matches(W.make_config(5, seed=1, scale="small"))
    assert api.attend_noalloc_max_bytes() == 64 << 20


def test_noalloc_rejects_pass_beyond_scratch():
    import torch

    from ragged_paged_kv_fp_amd import api, runner
    from ragged_paged_kv_fp_amd._lib import FP_ERR_WORKSPACE, FpError

    # 300k rows x 32 heads x 128 dims of rotated Q alone is ~2.3 GiB > 64 MiB:
    # only the host plan runs (no kernel is launched on this error)
    wl = W.make_config(2, seed=0, scale="small")
    ds = runner.DeviceStep(wl)
    n = 300_000
    ip = np.array([0, n], np.int32)
    geom = runner.api.Geometry(indptr=torch.tensor(ip, device="cuda"), indptr_host=ip.copy(),
                               positions=ds.geom.positions, slots=ds.geom.slots, kv_len=ds.geom.kv_len[:1],
                               fold=ds.geom.fold[:1])
    ps = runner.api.Pool(kv=ds.pool.kv, num_pages=ds.pool.num_pages, page_size=ds.pool.page_size,
                         num_kv_heads=ds.pool.num_kv_heads, head_dim=ds.pool.head_dim,
                         page_indptr=ds.pool.page_indptr[:2], page_indptr_host=ds.pool.page_indptr_host[:2].copy(),
                         page_ids=ds.pool.page_ids, committed_len=ds.pool.committed_len[:1])
    assert api.attend_workspace_bytes(ps, geom, wl.H_q) > api.attend_noalloc_max_bytes()
    with pytest.raises(FpError) as e:
        api.attend_noalloc(ps, geom, ds.q, wl.H_q, wl.theta, wl.sm_scale, ds.out, ds.status)
    assert e.value.code == FP_ERR_WORKSPACE
