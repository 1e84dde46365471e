"""GPU parity of the score-driven eviction step (fp_tova_mask) against the oracle.

The selection is integer work decided on fp32 keys: both sides sum each slot's
mass over the KV heads in head order in fp32 (the oracle's tova_scores), so the
kept sets and the bitmaps must match bit for bit. The masses fed to both sides
are the same fp32 arrays: synthetic ones (with many equal scores, and with
random ones whose head sums round), and, in the loop test, the mass the GPU's
own fp_attn_mass produced for the pass before.
"""

import numpy as np
import pytest

import oracle
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


def _pack(bits: np.ndarray, nwords: int) -> np.ndarray:
    words = np.zeros(nwords, dtype=np.uint32)
    for j in np.nonzero(bits)[0]:
        words[j >> 5] |= np.uint32(1 << (int(j) & 31))
    return words


def _dev(a, torch, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype=dtype, device="cuda")


CASES = [
    # seed, P, H, lanes, largest pages per lane, quantized masses, with prev_keep
    (0, 16, 8, 6, 40, True, False),
    (1, 8, 4, 5, 30, False, True),
    (2, 32, 2, 7, 12, True, True),
    (3, 16, 8, 3, 2100, False, True),   # a lane longer than the LDS key cache (32768 slots)
]


@pytest.mark.parametrize("seed,P,H,L,maxpages,quant,with_prev", CASES)
def test_tova_select_and_rows_match_oracle(seed, P, H, L, maxpages, quant, with_prev):
    import torch

    from ragged_paged_kv_fp_amd import api

    rng = np.random.default_rng(1000 + seed)
    pages = rng.integers(1, maxpages + 1, size=L)
    if maxpages > 1000:
        pages[0] = maxpages          # the long lane
    page_indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    cap = pages * P
    S = int(page_indptr[-1]) * P
    committed = np.array([rng.integers(0, c + 1) for c in cap], dtype=np.int32)
    committed[0] = min(cap[0], max(committed[0], cap[0] - 40))
    committed[-1] = 0                # a lane with no old slots
    if quant:
        mass = (rng.integers(0, 5, size=(H, S)) * 0.125).astype(np.float32)
    else:
        mass = rng.random((H, S), dtype=np.float32) * np.float32(0.3)
    budget = np.array([rng.integers(-1, c + 3) for c in committed], dtype=np.int32)
    budget[1 % L] = 0
    # next pass: n_l rows at fresh slots c .. c+n-1 (permuted), reading c + n slots
    n = np.array([min(int(rng.integers(0, 5)), int(cap[l] - committed[l])) for l in range(L)])
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    slots = np.concatenate([committed[l] + rng.permutation(n[l]) for l in range(L)]).astype(np.int32)
    kv_len = (committed + n).astype(np.int32)
    wpr = np.array([(kv + 31) // 32 + int(rng.integers(0, 2)) for kv in kv_len])
    wpr[2 % L] = 0                   # a lane without bitmap words keeps the causal rule
    if L > 3 and kv_len[3] > 32:
        wpr[3] = 1                   # too few words: flagged
    span = wpr * n
    mask_off = np.concatenate([[0], np.cumsum(span)]).astype(np.int64)
    keep_words = (cap + 31) // 32
    keep_off = np.concatenate([[0], np.cumsum(keep_words)]).astype(np.int64)
    prev_limit = np.array([rng.integers(0, c + 1) for c in committed], dtype=np.int32)
    prev_bits = [rng.random(int(c)) < 0.7 for c in committed]
    prev_words = np.concatenate([_pack(prev_bits[l], int(keep_words[l])) for l in range(L)])
    _say(f"tova case seed={seed} P={P} H={H} lanes={L} capacity={cap.tolist()} committed={committed.tolist()}")

    kv_dummy = torch.zeros(8, dtype=torch.int16, device="cuda")
    pool = api.Pool(kv=kv_dummy, num_pages=int(page_indptr[-1]), page_size=P, num_kv_heads=H, head_dim=128,
                    page_indptr=_dev(page_indptr, torch, torch.int32), page_indptr_host=page_indptr.copy(),
                    page_ids=_dev(np.arange(page_indptr[-1], dtype=np.int32), torch, torch.int32),
                    committed_len=_dev(committed, torch, torch.int32))
    geom = api.Geometry(indptr=_dev(indptr, torch, torch.int32), indptr_host=indptr.copy(),
                        positions=_dev(slots, torch, torch.int32), slots=_dev(slots, torch, torch.int32),
                        kv_len=_dev(kv_len, torch, torch.int32),
                        fold=_dev(np.full(L, -1, np.int32), torch, torch.int32))
    mask_t = torch.full((max(int(mask_off[-1]), 1),), -1, dtype=torch.int32, device="cuda")
    mask = api.Mask(bits=mask_t, word_offset=_dev(mask_off, torch, torch.int64), word_offset_host=mask_off.copy())
    keep_t = torch.full((int(keep_off[-1]),), -1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    prev_t = _dev(prev_words.view(np.int32), torch, torch.int32) if with_prev else None
    plim_t = _dev(prev_limit, torch, torch.int32) if with_prev else None
    api.tova_mask(pool, geom, _dev(mass, torch, torch.float32), _dev(budget, torch, torch.int32),
                  _dev(keep_off, torch, torch.int64), keep_t, mask, status, prev_t, plim_t)
    torch.cuda.synchronize()
    got_keep = keep_t.cpu().numpy().view(np.uint32)
    got_mask = mask_t.cpu().numpy().view(np.uint32)

    keep = oracle.tova_keep(mass, page_indptr, P, committed, budget, prev_bits if with_prev else None, prev_limit)
    for l in range(L):
        nw = (int(committed[l]) + 31) // 32
        want = _pack(keep[l], nw)
        assert np.array_equal(got_keep[keep_off[l]:keep_off[l] + nw], want), f"keep words of lane {l}"
    words, st = oracle.tova_mask(keep, indptr, slots, kv_len, committed, wpr)
    for l in range(L):
        if span[l] == 0:
            continue
        assert np.array_equal(got_mask[mask_off[l]:mask_off[l + 1]], words[l]), f"bitmap of lane {l}"
    assert int(status.cpu()[0]) == st


def test_tova_loop_drives_the_next_pass():
    """Pass 1 on the GPU (a random pass of prefill, decode and verify lanes,
    causal and bitmap, with spare pages), its attention mass, the eviction step with half of each lane's slots as the
    budget, then pass 2 attending under the produced bitmaps: the bitmaps match
    the oracle's selection on the GPU's mass, and pass 2's attention matches
    the oracle's on the same bitmaps."""
    import torch

    from ragged_paged_kv_fp_amd import api

    wl = W.make_random(3, H_kv=2, G=4, d=128, P=16, num_lanes=6, max_rows=80, max_ctx=600, masked=True,
                       fold_modes=False, extra_pages=3)
    ds = pu.gpu_run(wl)  # prefix, then append -> attend -> fold -> readout
    S = int(wl.page_indptr[-1]) * wl.P
    mass_t = torch.zeros((wl.H_kv, S), dtype=torch.float32, device="cuda")
    api.attn_mass(ds.pool, ds.geom, wl.H_q, ds.lse, ds.workspace, mass_t, ds.mask, ds.split)
    torch.cuda.synchronize()
    committed = ds.pool.committed_len.cpu().numpy().astype(np.int32)
    cap = np.diff(wl.page_indptr) * wl.P
    rng = np.random.default_rng(11)
    L = wl.num_lanes
    n = np.array([min(3, int(cap[l] - committed[l])) for l in range(L)])
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    slots = np.concatenate([committed[l] + np.arange(n[l]) for l in range(L)]).astype(np.int32)
    positions = slots + 5
    kv_len = (committed + n).astype(np.int32)
    wpr = (kv_len + 31) // 32
    mask_off = np.concatenate([[0], np.cumsum(wpr * n)]).astype(np.int64)
    keep_off = np.concatenate([[0], np.cumsum((cap + 31) // 32)]).astype(np.int64)
    budget = (committed // 2).astype(np.int32)
    _say(f"tova loop: lanes={L} committed={committed.tolist()} budget={budget.tolist()}")
    geom2 = api.Geometry(indptr=_dev(indptr, torch, torch.int32), indptr_host=indptr.copy(),
                         positions=_dev(positions, torch, torch.int32), slots=_dev(slots, torch, torch.int32),
                         kv_len=_dev(kv_len, torch, torch.int32),
                         fold=_dev(np.full(L, -1, np.int32), torch, torch.int32))
    mask_t = torch.zeros((int(mask_off[-1]),), dtype=torch.int32, device="cuda")
    mask2 = api.Mask(bits=mask_t, word_offset=_dev(mask_off, torch, torch.int64), word_offset_host=mask_off.copy())
    keep_t = torch.zeros((int(keep_off[-1]),), dtype=torch.int32, device="cuda")
    st2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.tova_mask(ds.pool, geom2, mass_t, _dev(budget, torch, torch.int32), _dev(keep_off, torch, torch.int64),
                  keep_t, mask2, st2)
    N2 = int(indptr[-1])
    k2 = W.bf16_bits_from_f32(rng.normal(size=(N2, wl.H_kv, wl.d)).astype(np.float32))
    v2 = W.bf16_bits_from_f32(rng.normal(size=(N2, wl.H_kv, wl.d)).astype(np.float32))
    q2 = W.bf16_bits_from_f32(rng.normal(size=(N2, wl.H_q, wl.d)).astype(np.float32))
    as_dev = lambda a: _dev(a.view(np.int16), torch, torch.int16)  # noqa: E731
    api.append_kv(ds.pool, geom2, as_dev(k2), as_dev(v2), wl.theta, st2)
    out2 = torch.zeros((N2, wl.H_q, wl.d), dtype=torch.float32, device="cuda")
    lse2 = torch.zeros((N2, wl.H_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(api.attend_workspace_bytes(ds.pool, geom2, wl.H_q, mask2), 256), dtype=torch.uint8,
                     device="cuda")
    api.attend(ds.pool, geom2, as_dev(q2), wl.H_q, wl.theta, wl.sm_scale, out2, ws, st2, lse=lse2, mask=mask2)
    torch.cuda.synchronize()
    assert int(st2.cpu()[0]) == 0
    gpu_bits = mask_t.cpu().numpy().view(np.uint32)

    mass = mass_t.cpu().numpy()
    keep = oracle.tova_keep(mass, wl.page_indptr, wl.P, committed, budget)
    for l in range(L):
        assert int(keep[l].sum()) == min(int(budget[l]), int(committed[l]))
    words, st = oracle.tova_mask(keep, indptr, slots, kv_len, committed, wpr)
    assert st == 0
    assert np.array_equal(gpu_bits, np.concatenate(words)), "bitmaps differ from the oracle's selection"
    # pass 2 against the oracle, on the oracle's own pool after pass 1 and the fold
    ref = pu.oracle_run(wl)
    c_ref = np.asarray(ref["committed"], dtype=np.int32)
    assert np.array_equal(c_ref, committed)
    oracle.append(ref["pool"], c_ref, indptr, positions, slots, k2, v2, wl.theta)
    O, LSE, s = oracle.attend(ref["pool"], indptr, positions, slots, kv_len, q2, wl.H_q, wl.theta, wl.sm_scale,
                              gpu_bits, mask_off)
    assert s == 0
    err, rel = pu.compare_arrays(out2.cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64), O,
                                 LSE)
    _say(f"tova loop pass 2: max-abs {err:.2e} rel-L2 {rel:.2e}")
