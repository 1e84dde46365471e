"""GPU parity of projection-site LoRA adapters (fp_adapter_lora) against the oracle.

Tolerance, from the arithmetic: the GPU keeps v = A x (fp32 sums of exact
bf16 products) as two bf16 terms hi + lo (16 significant bits, relative error
at most 2^-16) for B v, then forms y + s (B v) in fp32 and rounds to bf16.
Against the exact value e = y + s B (A x) an output element may therefore
differ by half a bf16 unit of the computed value (the final rounding; bf16
has 8 significant bits, so its unit roundoff is 2^-8), plus
2^-16 s (|B| |A x|) (the split of v), plus fp32 rounding (1e-6 of the
magnitudes). Bits that agree with the oracle's correctly rounded output are
counted and reported. Lanes without an adapter keep y bit for bit.
"""

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_paged_kv_fp_amd import _lib

    _lib.load()


def _bits(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def _run(lw, in_place=False):
    import torch

    from ragged_paged_kv_fp_amd import api

    dev = "cuda"
    ip = lw.indptr.astype(np.int32)
    geom = api.Geometry(indptr=torch.from_numpy(ip).to(dev), indptr_host=ip.copy(), positions=None, slots=None,
                        kv_len=None, fold=None)
    lora = api.Lora(a=_bits(lw.a, dev), b=_bits(lw.b, dev), scale=torch.from_numpy(lw.scale).to(dev))
    x = _bits(lw.x, dev)
    y = _bits(lw.y, dev)
    out = y if in_place else torch.full_like(y, 0x7FC0)
    ws = torch.empty(max(api.lora_workspace_bytes(geom, lora), 256), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    api.adapter_lora(geom, lora, torch.from_numpy(lw.adapter).to(dev), x, y, out, ws, status)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), int(status.cpu()[0])


def _check(lw, got, lanes=None):
    adapter = lw.adapter.copy()
    if lanes is not None:
        keep = np.zeros_like(adapter, dtype=bool)
        keep[list(lanes)] = True
        adapter[~keep] = -1
    want, exact, st = oracle.lora(lw.x, lw.y, adapter, lw.indptr, lw.a, lw.b, lw.scale)
    rows = np.concatenate([np.arange(lw.indptr[l], lw.indptr[l + 1]) for l in
                           (range(len(adapter)) if lanes is None else lanes)]).astype(np.int64)
    g, e, wb = got[rows], exact[rows], want[rows]
    gv = oracle.bf16_to_f64(g)
    # |B| |A x| per element, for the bound on the rounding of v
    mag = np.zeros_like(e)
    for lane in (range(len(adapter)) if lanes is None else lanes):
        k = int(lw.adapter[lane])
        r0, r1 = int(lw.indptr[lane]), int(lw.indptr[lane + 1])
        sel = (rows >= r0) & (rows < r1)
        if k < 0 or k >= lw.a.shape[0] or not sel.any():
            assert np.array_equal(got[r0:r1], lw.y[r0:r1]), f"lane {lane} without adapter changed"
            continue
        v = oracle.bf16_to_f64(lw.x[r0:r1]) @ oracle.bf16_to_f64(lw.a[k]).T
        mag[sel] = float(lw.scale[k]) * (np.abs(v) @ np.abs(oracle.bf16_to_f64(lw.b[k])).T)
    top = np.abs(e) + 2.0 ** -16 * mag + 1e-6 * (np.abs(e) + mag)  # largest fp32 value before rounding
    ulp = np.exp2(np.floor(np.log2(np.maximum(top, 2.0 ** -126))) - 7)
    bound = 0.5 * ulp + 2.0 ** -16 * mag + 1e-6 * (np.abs(e) + mag)
    err = np.abs(gv - e)
    assert np.all(np.isfinite(gv))
    assert np.all(err <= bound), f"worst excess {float((err - bound).max())}"
    return float((g == wb).mean()), st


# the last three: d_in steps that do not divide evenly over the four waves
# (some waves with one step or none), and d_out with a partial column block
@pytest.mark.parametrize("rank,d_in,d_out", [(16, 4096, 1024), (32, 512, 4096), (48, 1024, 96), (64, 2048, 512),
                                             (16, 192, 544), (48, 64, 32), (32, 320, 1056)])
def test_lora_small_pass(rank, d_in, d_out):
    wl = W.make_config(3, seed=1, scale="small")
    lw = W.make_lora(rank, wl.step.indptr, d_in=d_in, d_out=d_out, rank=rank, num_adapters=5)
    got, st = _run(lw)
    exact_frac, want_st = _check(lw, got)
    assert st == want_st == 0
    assert exact_frac >= 0.99
    print(f"rank {rank} d_in {d_in} d_out {d_out}: rows {int(lw.indptr[-1])}, bits equal to oracle {exact_frac:.4f}",
          flush=True)


def test_lora_in_place_and_bad_adapter_id():
    wl = W.make_config(4, seed=0, scale="small")
    lw = W.make_lora(9, wl.step.indptr, d_in=1024, d_out=512, rank=16, num_adapters=3)
    lw.adapter[1] = 7          # out of range: flagged, lane keeps y
    lw.adapter[2] = -1
    got, st = _run(lw, in_place=True)
    _, want_st = _check(lw, got)
    assert st == want_st == oracle.ST_ADAPTER
    r0, r1 = int(lw.indptr[1]), int(lw.indptr[2])
    assert np.array_equal(got[r0:r1], lw.y[r0:r1])


def test_lora_full_size_mixed_wave_sampled():
    wl = W.make_config(3, seed=0)
    lw = W.make_lora(4, wl.step.indptr, d_in=4096, d_out=4096, rank=16, num_adapters=8)
    got, st = _run(lw)
    n = np.diff(lw.indptr)
    lanes = [int(np.argmax(n)), 3, 50, 127]   # the longest prefill lane and some decode lanes
    frac, _ = _check(lw, got, lanes)
    print(f"full size: rows {int(lw.indptr[-1])}, sampled lanes {lanes}, bits equal {frac:.4f}", flush=True)
    # every lane without an adapter keeps y exactly
    for lane in np.nonzero(lw.adapter < 0)[0]:
        r0, r1 = int(lw.indptr[lane]), int(lw.indptr[lane + 1])
        assert np.array_equal(got[r0:r1], lw.y[r0:r1])


def test_ia3_bit_exact():
    import torch

    from ragged_paged_kv_fp_amd import api

    wl = W.make_config(3, seed=0)
    ip = wl.step.indptr.astype(np.int32)
    N, d_out = int(ip[-1]), 1024
    rng = np.random.default_rng(3)
    y = W.bf16_bits_from_f32(rng.standard_normal((N, d_out)).astype(np.float32))
    scale = W.bf16_bits_from_f32(rng.uniform(0.25, 4.0, (6, d_out)).astype(np.float32))
    adapter = rng.integers(-1, 6, size=len(ip) - 1).astype(np.int32)
    adapter[5] = 9  # out of range: flagged, lane keeps y
    want, want_st = oracle.ia3(y, adapter, ip, scale)
    dev = "cuda"
    geom = api.Geometry(indptr=torch.from_numpy(ip).to(dev), indptr_host=ip.copy(), positions=None, slots=None,
                        kv_len=None, fold=None)
    for in_place in (False, True):
        yt = _bits(y, dev)
        out = yt if in_place else torch.full_like(yt, 0x7FC0)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        api.adapter_ia3(geom, _bits(scale, dev), torch.from_numpy(adapter).to(dev), yt, out, status)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"in_place={in_place}"
        assert int(status.cpu()[0]) == want_st == oracle.ST_ADAPTER


def test_lora_and_ia3_at_the_lane_limit():
    """4096 lanes (the library's limit), mostly empty or one row with a few
    long ones: every thread of the plan scans four lanes and the item list
    comes from the binary search over the lanes' starts."""
    rng = np.random.default_rng(11)
    L = 4096
    n = rng.choice([0, 0, 1, 1, 1, 2, 5], size=L)
    n[rng.choice(L, 6, replace=False)] = rng.integers(33, 200, size=6)
    ip = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    lw = W.make_lora(12, ip, d_in=256, d_out=128, rank=32, num_adapters=7)
    got, st = _run(lw)
    exact_frac, want_st = _check(lw, got)
    assert st == want_st == 0
    assert exact_frac >= 0.99
    want, want_st = oracle.ia3(lw.y, lw.adapter, ip, lw.b[:, :, 0].copy())
    import torch

    from ragged_paged_kv_fp_amd import api

    dev = "cuda"
    geom = api.Geometry(indptr=torch.from_numpy(ip).to(dev), indptr_host=ip.copy(), positions=None, slots=None,
                        kv_len=None, fold=None)
    out = torch.full_like(_bits(lw.y, dev), 0x7FC0)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    api.adapter_ia3(geom, _bits(lw.b[:, :, 0].copy(), dev), torch.from_numpy(lw.adapter).to(dev), _bits(lw.y, dev),
                    out, status)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)
    assert int(status.cpu()[0]) == want_st == 0
