"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small copies of the five workload configurations and random geometries run
whole on both sides; the full-size configurations run whole on the GPU and
are checked on sampled lanes and rows. Invariants: page-pool permutation,
NaN-poisoned pool, prefix/suffix split, all-causal bitmap vs folding,
determinism, decode split size. Error paths set status bits and suppress writes.
"""

import numpy as np
import pytest

import oracle
import parity_util as pu
import workloads as W

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_paged_kv_fp_amd import _lib

    _lib.load()


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config_small(cfg, seed):
    wl = W.make_config(cfg, seed=seed, scale="small" if cfg > 1 else "full")
    _say(f"config {cfg} seed {seed}: lanes={wl.num_lanes} rows={wl.step.num_rows}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    r = pu.compare_step(ds, ref)
    _say(r)


@pytest.mark.parametrize("seed,H_kv,G,d,P", [
    (0, 2, 2, 64, 16), (1, 1, 4, 128, 8), (2, 2, 8, 64, 32), (3, 4, 1, 128, 16),
    (4, 2, 4, 128, 32), (5, 1, 2, 64, 8), (6, 3, 4, 128, 16), (7, 2, 8, 128, 8),
])
def test_random_geometry(seed, H_kv, G, d, P):
    wl = W.make_random(seed, H_kv=H_kv, G=G, d=d, P=P, num_lanes=7, max_rows=90, max_ctx=400)
    _say(f"random seed {seed}: H_kv={H_kv} G={G} d={d} P={P} rows={wl.step.num_rows}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    _say(pu.compare_step(ds, ref))


def test_maximum_lanes():
    """4096 lanes, the plan's limit (each plan thread then classifies four
    lanes): decode, verify, prefill and empty lanes, causal and bitmap lanes,
    every fold mode, against the oracle."""
    wl = W.make_random(71, H_kv=1, G=2, d=64, P=8, num_lanes=4096, max_rows=24, max_ctx=60, extra_pages=4)
    n = np.diff(wl.step.indptr)
    _say(f"maximum lanes: lanes={wl.num_lanes} rows={wl.step.num_rows} decode-class={int(((n > 0) & (n * 2 <= 32)).sum())} "
         f"prefill-class={int((n * 2 > 32).sum())} empty={int((n == 0).sum())}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    _say(pu.compare_step(ds, ref))


HOLE_BITS = 0x3FC0  # bf16 1.5: what a slot no pass wrote holds (finite, as the step requires below kv_len)


@pytest.mark.parametrize("seed,H_kv,G,d,P,kinds,masked", [
    (0, 2, 2, 64, 16, None, True), (1, 1, 4, 128, 8, [2, 2, 1, 0], True), (2, 2, 8, 64, 32, [1, 1, 2, 0], True),
    (3, 4, 1, 128, 16, [2, 1, 0], True), (4, 2, 4, 128, 32, [0, 0, 1, 1, 2], False),
    (5, 1, 2, 64, 8, None, False), (6, 8, 4, 128, 16, [2, 2, 2, 1, 0, 0], True), (7, 2, 8, 128, 8, [2, 1], True),
    (8, 2, 4, 128, 16, [2, 2, 2, 2], False), (9, 2, 4, 128, 16, [1, 1, 1, 1, 0, 0, 0, 0], True),
])
def test_explicit_slot_geometry(seed, H_kv, G, d, P, kinds, masked):
    """Rows naming their slots (State geometry, for algorithms that manage KV
    slots directly): permuted and gapped slots, prefix slots above the frozen
    count rewritten, kv_len below some rows' slots, holes below kv_len holding
    the pool's fill; decode-, verify- and prefill-class lanes, causal and bitmap."""
    wl = W.make_explicit(seed, H_kv=H_kv, G=G, d=d, P=P, num_lanes=len(kinds) if kinds else 7, max_rows=120,
                         max_ctx=500, masked=masked, kinds=kinds)
    n = np.diff(wl.step.indptr)
    _say(f"explicit seed {seed}: H_kv={H_kv} G={G} d={d} P={P} rows={wl.step.num_rows} "
         f"decode-class={int(((n > 0) & (n * G <= 32)).sum())} prefill-class={int((n * G > 32).sum())}")
    ref = pu.oracle_run(wl, fill=HOLE_BITS)
    ds = pu.gpu_run(wl, fill=HOLE_BITS)
    _say(pu.compare_step(ds, ref))


@pytest.mark.parametrize("seed,H_kv,d,P,rows", [
    (40, 2, 64, 8, 2300), (41, 3, 128, 16, 4500), (42, 2, 128, 32, 9000), (43, 1, 64, 32, 17000),
    (44, 8, 128, 16, 17000),
])
def test_append_row_groups(seed, H_kv, d, P, rows):
    """The KV write of passes large enough that one workgroup takes 2, 4, 8 or
    16 consecutive rows: contiguous runs from any page offset and across
    pages, single rows, reversed and gapped runs, rows at frozen or
    out-of-range slots, lanes of 1 to 300 rows. The whole pool (holes keep the
    fill) and the status bits equal the oracle's append."""
    import torch

    wl = W.make_append_mix(seed, H_kv=H_kv, d=d, P=P, rows=rows)
    st = wl.step
    _say(f"append mix seed {seed}: H_kv={H_kv} d={d} P={P} rows={st.num_rows} lanes={st.num_lanes}")
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids, fill_bits=HOLE_BITS)
    c = np.zeros(wl.num_lanes, np.int32)
    p = wl.prefix
    assert oracle.append(pool, c, p.indptr, p.positions, p.slots, p.k, p.v, wl.theta) == 0
    c, _ = oracle.fold(c, p.indptr, p.fold)
    status = oracle.append(pool, c, st.indptr, st.positions, st.slots, st.k, st.v, wl.theta)
    assert status == oracle.ST_SLOT_RANGE | oracle.ST_FROZEN  # both refusals occur in every case

    from ragged_paged_kv_fp_amd import runner

    ds = runner.DeviceStep(wl, device="cuda", fill_bits=HOLE_BITS)
    ds.run_prefix()
    torch.cuda.synchronize()
    assert int(ds.status.cpu()[0]) == 0
    ds.append()
    torch.cuda.synchronize()
    assert int(ds.status.cpu()[0]) == status
    pu.compare_pool(ds, dict(pool=pool))


@pytest.mark.parametrize("seed,L,kv,window,sinks,P", [(0, 4, 32768, 1024, 4, 16), (1, 3, 30001, 1000, 3, 32),
                                                       (2, 5, 5000, 77, 0, 8)])
def test_window_decode_lanes_walk_tile_lists(seed, L, kv, window, sinks, P):
    """Masked decode lanes read only the tiles their bitmap touches (Docs,
    Attention masks: sliding window with attention sinks): at kv_len 32768 a
    window of 1024 plus 4 sinks is 33 of 1024 tiles. The slots in between are
    holes the prefix never wrote; the result equals the oracle's."""
    wl = W.make_window_decode(seed, L=L, kv=kv, window=window, sinks=sinks, H_q=16, H_kv=4, d=128, P=P)
    _say(f"window decode seed {seed}: lanes={L} kv={kv} window={window} sinks={sinks} P={P}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    _say(pu.compare_step(ds, ref))


@pytest.mark.parametrize("split", [64, 512])
def test_empty_splits_leave_no_partials(split):
    """Masked decode lanes whose tile lists fall in a few KV splits: the other
    splits of each (lane, KV head) hold no tile, write only max -inf and sum
    0, and the merge gives them weight 0 without reading their partial
    output. The workspace starts as NaN bytes, so any partial output the
    merge read without it having been written would show."""
    import torch

    from ragged_paged_kv_fp_amd import runner

    wl = W.make_window_decode(2, L=5, kv=5000, window=77, sinks=2, H_q=16, H_kv=4, d=128, P=8)
    _say(f"window decode with empty splits: split={split}")
    ref = pu.oracle_run(wl)
    ds = runner.DeviceStep(wl, device="cuda", split=split)
    ds.run_prefix()
    torch.cuda.synchronize()
    ds.workspace.fill_(0xFF)
    ds.status.zero_()
    ds.step()
    torch.cuda.synchronize()
    _say(pu.compare_step(ds, ref))


def _hazard_bits(wl):
    """fp_check_hazards on the GPU and oracle.hazards, both after the prefix pass and its fold."""
    import torch

    from ragged_paged_kv_fp_amd import api, runner

    ds = runner.DeviceStep(wl)
    ds.run_prefix()
    torch.cuda.synchronize()
    ws = torch.empty(api.hazard_workspace_bytes(ds.pool), dtype=torch.uint8, device=ds.device)
    st = torch.zeros(1, dtype=torch.int32, device=ds.device)
    api.check_hazards(ds.pool, ds.geom, ws, st)
    torch.cuda.synchronize()
    pool = oracle.Pool(wl.num_pages, wl.P, wl.H_kv, wl.d, wl.page_indptr, wl.page_ids)
    c = np.zeros(wl.num_lanes, np.int32)
    if wl.prefix is not None:
        c, _ = oracle.fold(c, wl.prefix.indptr, wl.prefix.fold)
    assert ds.pool.committed_len.cpu().numpy().tolist() == c.tolist()
    return int(st.cpu()[0]), oracle.hazards(pool, c, wl.step.indptr, wl.step.slots, wl.step.kv_len)


def test_hazard_check_matches_oracle():
    """Eq. (4) (reviews, section 5) conflicts between lanes, and cells written twice:
    the GPU check and the oracle agree bit for bit on valid passes (no bits) and
    on passes with planted conflicts (the bits they expect)."""
    DUP, SH = oracle.ST_DUP_WRITE, oracle.ST_SHARED_CELL
    for wl in (W.make_explicit(11, num_lanes=6), W.make_config(3, seed=2, scale="small"),
               W.make_random(12, num_lanes=6)):
        got, want = _hazard_bits(wl)
        assert got == want == 0, (wl.name, got, want)
    # a duplicate slot within one lane
    wl = W.make_explicit(13, num_lanes=6, kinds=[2, 1, 0, 2, 1, 0])
    st = wl.step
    lane = next(l for l in range(wl.num_lanes) if st.indptr[l + 1] - st.indptr[l] >= 2)
    st.slots = st.slots.copy()
    st.slots[st.indptr[lane] + 1] = st.slots[st.indptr[lane]]
    got, want = _hazard_bits(wl)
    assert want & DUP and got == want, (got, want)
    # lane b's first page replaced by the page lane a writes into: b reads a's fresh cell
    wl = W.make_config(3, seed=3, scale="small")
    st = wl.step
    n = np.diff(st.indptr)
    a = int(np.argmax(n))
    b = next(l for l in range(wl.num_lanes) if l != a and st.kv_len[l] >= wl.P)
    s_a = int(st.slots[st.indptr[a]])
    wl.page_ids = wl.page_ids.copy()
    wl.page_ids[wl.page_indptr[b]] = wl.page_ids[wl.page_indptr[a] + s_a // wl.P]
    got, want = _hazard_bits(wl)
    assert want & SH and got == want, (got, want)
    # two lanes whose rows write one cell
    wl = W.make_config(2, seed=6, scale="small")
    st = wl.step
    wl.page_ids = wl.page_ids.copy()
    last1 = (int(st.slots[1]) // wl.P)
    last0 = (int(st.slots[0]) // wl.P)
    st.slots = st.slots.copy()
    st.slots[1] = last1 * wl.P + int(st.slots[0]) % wl.P
    st.kv_len = st.kv_len.copy()
    st.kv_len[1] = max(int(st.kv_len[1]), int(st.slots[1]) + 1)
    wl.page_ids[wl.page_indptr[1] + last1] = wl.page_ids[wl.page_indptr[0] + last0]
    got, want = _hazard_bits(wl)
    assert want == DUP | SH and got == want, (got, want)


def test_page_permutation_bit_identical_with_nan_decoys():
    wl = W.make_random(21, H_kv=2, G=4, d=128, P=16, num_lanes=6, max_rows=70, max_ctx=300, extra_pages=9)
    a = pu.gpu_run(wl, fill=NAN_BF16)
    rng = np.random.default_rng(3)
    wl.page_ids = rng.permutation(wl.num_pages)[: len(wl.page_ids)].astype(np.int32)
    b = pu.gpu_run(wl, fill=NAN_BF16)
    assert np.array_equal(a.out.cpu().numpy(), b.out.cpu().numpy())
    assert np.array_equal(a.lse.cpu().numpy(), b.lse.cpu().numpy())
    ref = pu.oracle_run(wl, fill=NAN_BF16)
    pu.compare_step(b, ref)


def test_poisoned_pool_outputs_finite_and_equal():
    wl = W.make_config(2, seed=4, scale="small")
    a = pu.gpu_run(wl, fill=0)
    b = pu.gpu_run(wl, fill=NAN_BF16)
    oa, ob = a.out.cpu().numpy(), b.out.cpu().numpy()
    assert np.all(np.isfinite(ob)) and np.array_equal(oa, ob)
    wl3 = W.make_config(3, seed=4, scale="small")
    a3, b3 = pu.gpu_run(wl3, fill=0), pu.gpu_run(wl3, fill=NAN_BF16)
    assert np.array_equal(a3.out.cpu().numpy(), b3.out.cpu().numpy())


def test_prefix_then_continuation_equals_whole_prompt():
    import torch

    from ragged_paged_kv_fp_amd import api, runner

    wl = W.make_config(1)
    whole = pu.gpu_run(wl)
    K0, V0 = whole.pool_logical()
    O0 = whole.out.cpu().numpy()
    st = wl.step
    for split in (1, 5, 16, 31, 32, 33, 36):
        ds = runner.DeviceStep(wl)
        ds.run_prefix()
        pre = W.Pass(indptr=np.array([0, split], np.int32), positions=st.positions[:split], slots=st.slots[:split],
                     kv_len=np.array([split], np.int32), fold=np.array([W.FOLD_ALL], np.int32),
                     k=st.k[:split], v=st.v[:split], q=st.q[:split])
        post = W.Pass(indptr=np.array([0, 37 - split], np.int32), positions=st.positions[split:],
                      slots=st.slots[split:], kv_len=np.array([37], np.int32),
                      fold=np.array([W.FOLD_ALL], np.int32), k=st.k[split:], v=st.v[split:], q=st.q[split:])
        outs = []
        for p in (pre, post):
            g = runner._geometry(p, ds.device)
            k, v, q = runner._bits16(p.k, ds.device), runner._bits16(p.v, ds.device), runner._bits16(p.q, ds.device)
            out = torch.zeros((p.num_rows, wl.H_q, wl.d), dtype=torch.float32, device=ds.device)
            ws = torch.empty(max(256, api.attend_workspace_bytes(ds.pool, g, wl.H_q)), dtype=torch.uint8,
                             device=ds.device)
            api.append_kv(ds.pool, g, k, v, wl.theta, ds.status)
            api.attend(ds.pool, g, q, wl.H_q, wl.theta, wl.sm_scale, out, ws, ds.status)
            api.fold(ds.pool, g, ds.status)
            outs.append(out)
        torch.cuda.synchronize()
        K1, V1 = ds.pool_logical()
        assert np.array_equal(K0, K1) and np.array_equal(V0, V1), f"pool bytes differ at split {split}"
        O1 = torch.cat(outs).cpu().numpy()
        assert np.abs(O1 - O0).max() <= pu.MAX_ABS
        assert int(ds.pool.committed_len.cpu()[0]) == 37 and int(ds.status.cpu()[0]) == 0


def test_all_causal_bitmap_equals_folding():
    wl = W.make_config(3, seed=1, scale="small")
    base = pu.gpu_run(wl)
    st = wl.step
    offs = [0]
    words = []
    for lane in range(wl.num_lanes):
        n = int(st.indptr[lane + 1] - st.indptr[lane])
        kvl = int(st.kv_len[lane])
        wpr = -(-kvl // 32)
        j = np.arange(wpr * 32)
        for r in range(int(st.indptr[lane]), int(st.indptr[lane + 1])):
            allowed = (j <= st.slots[r]) & (j < kvl)
            words.append((allowed.reshape(wpr, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(1))
        offs.append(offs[-1] + n * wpr)
    wl.mask_bits = np.concatenate(words).astype(np.uint32)
    wl.mask_word_offset = np.array(offs, np.int64)
    masked = pu.gpu_run(wl)
    assert np.array_equal(base.out.cpu().numpy(), masked.out.cpu().numpy())
    assert np.array_equal(base.lse.cpu().numpy(), masked.lse.cpu().numpy())


def test_run_to_run_deterministic():
    wl = W.make_config(4, seed=2, scale="small")
    a, b = pu.gpu_run(wl), pu.gpu_run(wl)
    assert np.array_equal(a.out.cpu().numpy(), b.out.cpu().numpy())
    assert np.array_equal(a.lse.cpu().numpy(), b.lse.cpu().numpy())


@pytest.mark.parametrize("split", [32, 64, 256, 4096])
def test_decode_split_size_invariance(split):
    wl = W.make_config(2, seed=5, scale="small")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl, split=split)
    pu.compare_step(ds, ref)


@pytest.mark.parametrize("seed,split", [(91, 32), (82, 96)])
def test_merge_over_many_splits(seed, split):
    """Decode and verify lanes of up to 6000 slots at 32- and 96-slot splits:
    up to about 190 splits per (lane, KV head), so the merge takes its split
    statistics in more than one chunk of 128; bitmap lanes among them leave
    empty splits that the merge must skip in every chunk."""
    wl = W.make_random(seed, H_kv=2, G=4, d=128, P=16, num_lanes=8, max_rows=9, max_ctx=6000, masked=True)
    n = np.diff(wl.step.indptr)
    cap = np.diff(wl.page_indptr) * wl.P
    _say(f"many splits seed {seed} split {split}: most splits {int((cap[n > 0] + split - 1).max() // split)}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl, split=split)
    _say(pu.compare_step(ds, ref))


def test_plan_mismatch_emits_no_attention_work():
    """Launches are sized from the host copies of the offset arrays; when the
    device indptr disagrees (here: one row more in the last lane, or a row
    moved between lanes so a decode lane turns into a prefill lane), the plan
    sets FP_ST_PLAN_MISMATCH and emits no work item, so fp_attend leaves out
    and lse untouched instead of indexing past what was sized."""
    import torch

    wl = W.make_config(3, seed=1, scale="small")
    ds = pu.gpu_run(wl)
    assert int(ds.status.cpu()[0]) == 0
    ip = wl.step.indptr.astype(np.int32)
    n = np.diff(ip)
    variants = []
    bigger = ip.copy()
    bigger[-1] += 1
    variants.append(bigger)
    dec = next(l for l in range(wl.num_lanes - 1) if n[l] == 1 and n[l + 1] > 1)
    moved = ip.copy()
    moved[dec + 1] += 1  # lane dec takes a row of lane dec + 1: 2 rows x 4 heads, still decode class...
    moved[dec + 1] += 8  # ...and 8 more: 10 rows x 4 heads = 40 columns, a prefill lane
    assert moved[dec + 1] < moved[dec + 2]
    variants.append(moved)
    for v in variants:
        ds.geom.indptr = torch.from_numpy(v).to(ds.device)  # the host copy keeps the original offsets
        ds.out.fill_(float("nan"))
        ds.lse.fill_(7.0)
        ds.status.zero_()
        ds.attend()
        torch.cuda.synchronize()
        from ragged_paged_kv_fp_amd._lib import FP_ST_PLAN_MISMATCH

        assert int(ds.status.cpu()[0]) & FP_ST_PLAN_MISMATCH
        assert torch.isnan(ds.out).all() and bool((ds.lse == 7.0).all())


def test_error_paths_set_status_and_suppress_writes():
    wl = W.make_config(1)
    st = wl.step
    st.slots = st.slots.copy()
    st.slots[3] = 48      # beyond 3 pages x 16
    st.slots[4] = -5
    st.kv_len = np.array([60], np.int32)   # beyond capacity: clamped
    st.fold = np.array([50], np.int32)     # literal beyond rows: clamped
    ref = pu.oracle_run(wl, fill=0x1234)
    ds = pu.gpu_run(wl, fill=0x1234)
    want = oracle.ST_SLOT_RANGE | oracle.ST_KVLEN | oracle.ST_FOLD_CLAMP
    assert ref["status"] == want
    pu.compare_step(ds, ref)


def test_frozen_slot_writes_are_suppressed():
    import torch

    wl = W.make_config(4, seed=0, scale="small")
    ds = pu.gpu_run(wl, fill=0x1234)
    # replay the append with sign-flipped K/V without resetting committed_len:
    # folded slots are frozen now and must keep their values, the rest take the new ones
    K0, V0 = ds.pool_logical()
    c = ds.pool.committed_len.cpu().numpy()
    ds.status.zero_()
    ds.k ^= torch.tensor(-0x8000, dtype=torch.int16, device=ds.k.device)
    ds.v ^= torch.tensor(-0x8000, dtype=torch.int16, device=ds.v.device)
    ds.append()
    torch.cuda.synchronize()
    assert int(ds.status.cpu()[0]) == oracle.ST_FROZEN
    K1, V1 = ds.pool_logical()
    st = wl.step
    n_frozen = n_new = 0
    for lane in range(wl.num_lanes):
        for r in range(int(st.indptr[lane]), int(st.indptr[lane + 1])):
            s_ = int(st.slots[r])
            pg = int(wl.page_ids[wl.page_indptr[lane] + s_ // wl.P])
            off = s_ % wl.P
            if s_ < c[lane]:
                n_frozen += 1
                assert np.array_equal(V1[pg, :, off], V0[pg, :, off]) and np.array_equal(K1[pg, :, off], K0[pg, :, off])
            else:
                n_new += 1
                assert np.array_equal(V1[pg, :, off], st.v[r] ^ 0x8000)
    assert n_frozen > 0 and n_new > 0


def test_channel_fold_out_of_range_clamped():
    wl = W.make_config(4, seed=1, scale="small")
    wl.channel = wl.channel.copy()
    verify = [i for i, f in enumerate(wl.step.fold) if f == W.FOLD_CHANNEL]
    wl.channel[verify[0]] = 99
    wl.channel[verify[-1]] = -3
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    assert ref["status"] == oracle.ST_FOLD_CLAMP
    pu.compare_step(ds, ref)


def _fold_readout_case(case):
    if case == "channel_clamp":
        wl = W.make_config(4, seed=2, scale="small")
        wl.channel = wl.channel.copy()
        verify = [i for i, f in enumerate(wl.step.fold) if f == W.FOLD_CHANNEL]
        wl.channel[verify[0]] = 99
        wl.channel[verify[-1]] = -3
        return wl
    if case == "row_list":
        wl = W.make_random(41, H_kv=2, G=4, d=128, P=16, num_lanes=300, max_rows=12, max_ctx=90)
        n = wl.step.num_rows
        wl.readout_rows = np.concatenate([np.arange(n - 1, -1, -7), [-1, n, 0]]).astype(np.int32)
        return wl
    return W.make_config(2, seed=3, scale="small")  # default readout, one row per lane


@pytest.mark.parametrize("case", ["channel_clamp", "row_list", "default"])
def test_fold_readout_one_launch_matches_two(case):
    # fp_fold_readout must leave committed_len, the readout rows and the status
    # word exactly as fp_fold followed by fp_readout does (and as the oracle says).
    import torch

    wl = _fold_readout_case(case)
    _say(f"fold+readout {case}: lanes={wl.num_lanes} rows={wl.step.num_rows}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)  # the step ends in fp_fold_readout
    pu.compare_step(ds, ref)
    one = (ds.pool.committed_len.cpu().clone(), ds.dst.cpu().clone(), int(ds.status.cpu()[0]))
    ds.reset()
    ds.status.zero_()
    ds.dst.fill_(float("nan"))
    torch.cuda.synchronize()
    ds.fold()
    ds.readout()
    torch.cuda.synchronize()
    assert torch.equal(ds.pool.committed_len.cpu(), one[0])
    assert np.array_equal(ds.dst.cpu().numpy().view(np.uint32), one[1].numpy().view(np.uint32))
    assert int(ds.status.cpu()[0]) == one[2]
    if case == "row_list":
        assert one[2] & oracle.ST_READOUT_RANGE
    if case == "channel_clamp":
        assert one[2] & oracle.ST_FOLD_CLAMP


def test_readout_into_unaligned_rows():
    # a destination 4 bytes off 16-byte alignment takes the scalar copy and
    # still receives every row exactly
    import torch

    from ragged_paged_kv_fp_amd import api

    wl = W.make_config(4, seed=3, scale="small")
    ds = pu.gpu_run(wl)
    want = ds.dst.cpu().numpy().copy()
    n, e = ds.dst.shape
    raw = torch.full((n * e + 1,), float("nan"), dtype=torch.float32, device=ds.dst.device)
    dst = raw[1:].view(n, e)
    assert dst.data_ptr() % 16 == 4
    ds.status.zero_()
    api.readout(ds.geom, ds.out, dst, ds.status, ds.readout_rows)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert int(ds.status.cpu()[0]) == 0


def test_pass_without_rows():
    # lanes with cached history and no new rows: append and attend have
    # nothing to do, the fold clamps the channel count and the literal count to
    # the lanes' zero rows (status 8) and the default readout lists no row
    wl = W.make_empty_pass(5)
    _say(f"empty pass: lanes={wl.num_lanes} rows={wl.step.num_rows}")
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    pu.compare_step(ds, ref)
    assert ref["status"] == oracle.ST_FOLD_CLAMP and ds.dst.shape[0] == 0


def test_empty_rows_and_mask_short():
    wl = W.make_random(33, H_kv=2, G=4, d=128, P=16, num_lanes=6, max_rows=60, max_ctx=200)
    # an all-zero bitmap lane: every row empty -> O = 0, LSE = -inf
    for lane in range(wl.num_lanes):
        o0, o1 = int(wl.mask_word_offset[lane]), int(wl.mask_word_offset[lane + 1])
        if o1 > o0:
            wl.mask_bits = wl.mask_bits.copy()
            wl.mask_bits[o0:o1] = 0
            break
    ref = pu.oracle_run(wl)
    ds = pu.gpu_run(wl)
    pu.compare_step(ds, ref)


# ------------------------------------------------------------------ full-size configurations, sampled

def _sample(wl, n_lanes, rows_per_lane, seed):
    rng = np.random.default_rng(seed)
    st = wl.step
    nonempty = [l for l in range(wl.num_lanes) if st.indptr[l + 1] > st.indptr[l]]
    lanes = sorted(rng.choice(nonempty, size=min(n_lanes, len(nonempty)), replace=False).tolist())
    rows = []
    for l in lanes:
        r0, r1 = int(st.indptr[l]), int(st.indptr[l + 1])
        pick = {r0, r1 - 1} | set(rng.integers(r0, r1, size=min(rows_per_lane, r1 - r0)).tolist())
        rows.extend(sorted(pick))
    return lanes, np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("cfg,n_lanes,rows_per_lane", [(2, 8, 1), (3, 6, 6), (4, 10, 8), (5, 3, 5)])
def test_full_size_sampled(cfg, n_lanes, rows_per_lane):
    wl = W.make_config(cfg, seed=0, scale="full")
    _say(f"full config {cfg}: lanes={wl.num_lanes} rows={wl.step.num_rows} pages={wl.num_pages}")
    ds = pu.gpu_run(wl)
    lanes, rows = _sample(wl, n_lanes, rows_per_lane, seed=cfg)
    # prefill lanes of config 3 are the expensive, MFMA-bound part: make sure some are sampled
    if cfg == 3:
        pre = [l for l in range(wl.num_lanes) if wl.step.indptr[l + 1] - wl.step.indptr[l] > 1][:2]
        extra = []
        for l in pre:
            r0, r1 = int(wl.step.indptr[l]), int(wl.step.indptr[l + 1])
            extra += [r0, (r0 + r1) // 2, r1 - 1]
        lanes = sorted(set(lanes) | set(pre))
        rows = np.array(sorted(set(rows.tolist()) | set(extra)), dtype=np.int64)
    ref = pu.oracle_run(wl, lanes=lanes, rows=rows)
    pu.compare_pool(ds, ref, lanes=lanes)
    err, rel = pu.compare_outputs(ds, ref)
    assert ds.pool.committed_len.cpu().numpy().tolist() == ref["committed"].tolist()
    assert int(ds.status.cpu()[0]) == 0 and ref["status"] == 0
    rl = ref["readout_rows"]
    out = ds.out.cpu().numpy().reshape(ds.out.shape[0], -1)
    assert np.array_equal(ds.dst.cpu().numpy(), out[rl])
    # properties that hold at any size: finite outputs; single-head rows are convex combinations of V
    assert np.all(np.isfinite(ds.out.cpu().numpy()))
    _say(dict(max_abs=err, rel_l2=rel, lanes=len(lanes), rows=len(rows)))
