"""Shared helpers of the GPU parity tests: run a workload on the HIP path and
on the oracle, then compare what the step produced.

Tolerances: attention outputs max-abs <= 1e-2 and relative L2 <= 5e-3 against
the fp64 oracle (bf16 inputs, fp32 accumulation); LSE abs <= 1e-2; slot
writes, page indexing, fold lengths, readout gathers and status bits exact.
Rotated K is compared bit for bit too: both sides round the same fp64
rotation once to nearest-even bf16 (the kernel with device sin/cos, the oracle
with numpy's), and fp64 sin/cos that differ in the last fp64 place could only
change a bf16 rounding that sits within 2^-45 of a tie.
"""

from __future__ import annotations

import numpy as np

import oracle

MAX_ABS = 1e-2
REL_L2 = 5e-3
LSE_ABS = 1e-2


def oracle_run(wl, fill=0, lanes=None, rows=None):
    """Oracle state after the prefix pass and the step (optionally on a lane/row sample)."""
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids, fill_bits=fill)
    c = np.zeros(wl.num_lanes, np.int32)
    if wl.prefix is not None:
        p = wl.prefix
        oracle.append(pool, c, p.indptr, p.positions, p.slots, p.k, p.v, wl.theta, lanes=lanes)
        c, _ = oracle.fold(c, p.indptr, p.fold)
    st = wl.step
    s_app = oracle.append(pool, c, st.indptr, st.positions, st.slots, st.k, st.v, wl.theta, lanes=lanes)
    O, LSE, s_att = oracle.attend(pool, st.indptr, st.positions, st.slots, st.kv_len, st.q, wl.H_q, wl.theta,
                                  wl.sm_scale, wl.mask_bits, wl.mask_word_offset, rows=rows)
    c1, s_fold = oracle.fold(c, st.indptr, st.fold, wl.channel)
    rl = oracle.readout_rows(st.indptr, wl.readout_rows)
    _, s_ro = oracle.readout(np.zeros((st.num_rows, 1)), st.num_rows, rl)  # status only: rows out of range
    return dict(pool=pool, O=O, LSE=LSE, committed=c1, readout_rows=rl, status=s_app | s_att | s_fold | s_ro,
                rows=rows)


def gpu_run(wl, fill=0, split=None, device="cuda"):
    import torch

    from ragged_paged_kv_fp_amd import runner

    ds = runner.DeviceStep(wl, device=device, fill_bits=fill, split=split)
    ds.run_prefix()
    torch.cuda.synchronize()
    ds.status.zero_()
    ds.step()
    torch.cuda.synchronize()
    return ds


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units between two bit patterns (sign-magnitude to a monotone integer line)."""
    def line(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(line(a_bits) - line(b_bits))


def compare_pool(ds, ref, lanes=None):
    """V and rotated K bit-exact; on a lane sample only the sampled lanes' pages count."""
    K, V = ds.pool_logical()
    pk, pv = ref["pool"].k, ref["pool"].v
    if lanes is not None:
        wl = ds.wl
        pages = np.concatenate([wl.page_ids[wl.page_indptr[l]:wl.page_indptr[l + 1]] for l in lanes])
        K, V, pk, pv = K[pages], V[pages], pk[pages], pv[pages]
    assert np.array_equal(V, pv), "V payload or slot placement differs"
    d = ulp_distance(K, pk)
    assert d.max() == 0, f"rotated K differs in {int((d > 0).sum())} elements (up to {d.max()} ulp)"
    return 1.0


def compare_outputs(ds, ref):
    O = ds.out.cpu().numpy().astype(np.float64)
    L = ds.lse.cpu().numpy().astype(np.float64)
    rows = ref["rows"]
    if rows is not None:
        O, L = O[rows], L[rows]
    return compare_arrays(O, L, ref["O"], ref["LSE"])


def compare_arrays(O, L, R, RL):
    """Attention output O / LSE L (float64 arrays from the device) against the oracle's R / RL."""
    assert np.all(np.isfinite(O)), "non-finite output"
    err = float(np.abs(O - R).max()) if O.size else 0.0
    nref = float(np.linalg.norm(R))
    rel = float(np.linalg.norm(O - R) / nref) if nref > 0 else float(np.linalg.norm(O - R))
    assert err <= MAX_ABS, f"max-abs {err}"
    assert rel <= REL_L2, f"rel-L2 {rel}"
    fin = np.isfinite(RL)
    assert np.array_equal(np.isfinite(L), fin), "LSE -inf pattern differs"
    lerr = float(np.abs(L[fin] - RL[fin]).max()) if fin.any() else 0.0
    assert lerr <= LSE_ABS, f"LSE abs {lerr}"
    return err, rel


def compare_step(ds, ref, lanes=None):
    """Everything exact except the floating-point tolerances above."""
    exact_k = compare_pool(ds, ref, lanes)
    err, rel = compare_outputs(ds, ref)
    assert ds.pool.committed_len.cpu().numpy().tolist() == ref["committed"].tolist(), "fold lengths differ"
    assert int(ds.status.cpu()[0]) == ref["status"], f"status {int(ds.status.cpu()[0])} != {ref['status']}"
    rl = ref["readout_rows"]
    out = ds.out.cpu().numpy().reshape(ds.out.shape[0], int(np.prod(ds.out.shape[1:])))  # also for a pass of 0 rows
    dst = ds.dst.cpu().numpy()
    assert dst.shape[0] == len(rl)
    ok = (rl >= 0) & (rl < out.shape[0])
    want = np.zeros_like(dst)
    want[ok] = out[rl[ok]]  # a row outside the pass reads as zeros
    assert np.array_equal(dst, want), "readout gather differs"
    return dict(max_abs=err, rel_l2=rel, k_exact=exact_k)


def oracle_run_ahead(ra):
    """The oracle's repeating decode loop: geometry from committed lengths each pass."""
    pool = oracle.Pool(ra.num_pages, ra.P, ra.H_kv, ra.d, ra.page_indptr, ra.page_ids)
    L = ra.num_lanes
    c = np.zeros(L, np.int32)
    if ra.prefix is not None:
        p = ra.prefix
        oracle.append(pool, c, p.indptr, p.positions, p.slots, p.k, p.v, ra.theta)
        c, _ = oracle.fold(c, p.indptr, p.fold)
    fold = np.full(L, oracle.FOLD_CHANNEL)
    passes, status = [], 0
    for t in range(ra.passes):
        pos, slots, kv = oracle.advance(c, ra.indptr, ra.pos_offset)
        s1 = oracle.append(pool, c, ra.indptr, pos, slots, ra.k[t], ra.v[t], ra.theta)
        O, LSE, s2 = oracle.attend(pool, ra.indptr, pos, slots, kv, ra.q[t], ra.H_q, ra.theta, ra.sm_scale)
        c, s3 = oracle.fold(c, ra.indptr, fold, ra.accept[t])
        passes.append(dict(O=O, LSE=LSE, positions=pos, slots=slots, kv_len=kv, committed=c))
        status |= s1 | s2 | s3
    return dict(pool=pool, passes=passes, committed=c, status=status, rows=None)
