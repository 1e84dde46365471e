"""CPU-side checks of the C ABI library: it loads, exports every function
include/fp.h declares, its host-only accounting matches Eqs. (1)/(2) and the
oracle, and bad arguments are rejected with the documented codes before
anything is enqueued (no GPU call is made by these tests)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp.h")


@pytest.fixture(scope="module")
def lib():
    from ragged_paged_kv_fp_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from ragged_paged_kv_fp_amd import build

        build.build()
    return _lib.load()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    from ragged_paged_kv_fp_amd import _lib

    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert b"gfx950" in lib.fp_version()


def test_header_constants_match_binding_and_oracle():
    from ragged_paged_kv_fp_amd import _lib

    src = open(HEADER).read()
    consts = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(FP_\w+)\s+\(?(-?\d+)\)?", src)}
    for name, val in consts.items():
        assert getattr(_lib, name) == val, name
    assert consts["FP_ST_SLOT_RANGE"] == oracle.ST_SLOT_RANGE
    assert consts["FP_ST_FROZEN"] == oracle.ST_FROZEN
    assert consts["FP_ST_KVLEN"] == oracle.ST_KVLEN
    assert consts["FP_ST_FOLD_CLAMP"] == oracle.ST_FOLD_CLAMP
    assert consts["FP_ST_READOUT_RANGE"] == oracle.ST_READOUT_RANGE
    assert consts["FP_ST_MASK_SHORT"] == oracle.ST_MASK_SHORT
    assert consts["FP_ST_PAGE_RANGE"] == oracle.ST_PAGE_RANGE
    assert consts["FP_ST_ADAPTER"] == oracle.ST_ADAPTER
    assert consts["FP_ST_DUP_WRITE"] == oracle.ST_DUP_WRITE
    assert consts["FP_ST_SHARED_CELL"] == oracle.ST_SHARED_CELL
    assert consts["FP_FOLD_ALL"] == oracle.FOLD_ALL and consts["FP_FOLD_CHANNEL"] == oracle.FOLD_CHANNEL


def test_accounting_matches_eq1_eq2(lib):
    assert lib.fp_kv_bytes(32, 8, 128, 1, 2) == 131072
    assert lib.fp_kv_bytes(32, 8, 128, 8192, 2) == 1 << 30
    for P in (8, 16, 32):
        assert lib.fp_page_bytes(P, 8, 128) == oracle.kv_bytes(1, 8, 128, P, 2)
        for T in range(0, 65537):
            assert lib.fp_pages_for(T, P) == oracle.pages_for(T, P)
            assert lib.fp_page_waste(T, P) == oracle.page_waste(T, P)
    assert lib.fp_pages_for(37, 16) == 3 and lib.fp_page_waste(37, 16) == 11


# ------------------------------------------------------------------ host validation

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _structs(L=2, rows=(3, 1), pages=(1, 2), P=16, H=2, d=64):
    from ragged_paged_kv_fp_amd import _lib

    keep = []
    ip = np.array([0] + list(np.cumsum(rows)), np.int32)
    pp = np.array([0] + list(np.cumsum(pages)), np.int32)
    keep += [ip, pp]
    g = _lib.FpGeometry(L, int(ip[-1]), FAKE, ip.ctypes.data, FAKE, FAKE, FAKE, FAKE)
    p = _lib.FpKvPool(FAKE, int(pp[-1]), P, H, d, FAKE, pp.ctypes.data, FAKE, FAKE)
    return g, p, keep


def _ws(lib, p, g, hq=4, m=None, t=None):
    return lib.fp_attend_workspace_bytes(ctypes.byref(p), ctypes.byref(g), m, hq, t)


def test_workspace_query_is_host_only_and_sized(lib):
    g, p, keep = _structs()
    n = _ws(lib, p, g)
    assert n > 0
    # two decode lanes (3*2 and 1*2 row-heads <= 32): items = H * ceil(cap/512) each; q copy = N*Hq*d*2
    assert n >= 4 * 4 * 64 * 2


@pytest.mark.parametrize("mut,code", [
    ("page_size=12", -3), ("head_dim=96", -3), ("num_kv_heads=0", -2), ("num_pages=0", -2),
    ("hq=5", -2), ("hq=6", -3), ("hq=32", -3), ("num_lanes=0", -2), ("num_rows=7", -2), ("kv=0", -1),
])
def test_bad_arguments_rejected(lib, mut, code):
    g, p, keep = _structs()
    hq = 4
    k, v = mut.split("=")
    v = int(v)
    if k == "hq":
        hq = v
    elif hasattr(p, k) and k not in ("num_rows", "num_lanes"):
        setattr(p, k, v)
    else:
        setattr(g, k, v)
    assert _ws(lib, p, g, hq=hq) == code


def test_lane_limit(lib):
    """4096 lanes (the plan's limit) are accepted; 4097 are refused before
    anything is enqueued."""
    for L, ok in ((4096, True), (4097, False)):
        g, p, keep = _structs(L=L, rows=[1] * L, pages=[1] * L)
        n = _ws(lib, p, g)
        assert (n > 0) if ok else (n == -3), (L, n)


def test_workspace_too_small_and_null_pointers(lib):
    g, p, keep = _structs()
    st = ctypes.c_int32(0)
    rc = lib.fp_attend(ctypes.byref(p), ctypes.byref(g), FAKE, 4, 10000.0, 0.125, None, FAKE, None, FAKE, 16, None,
                       ctypes.addressof(st), None)
    assert rc == -4
    # out must be 16-byte aligned like Q (the kernels store it in 16-byte vectors)
    rc = lib.fp_attend(ctypes.byref(p), ctypes.byref(g), FAKE, 4, 10000.0, 0.125, None, FAKE + 4, None, FAKE, 1 << 30,
                       None, ctypes.addressof(st), None)
    assert rc == -3
    rc = lib.fp_attend(ctypes.byref(p), ctypes.byref(g), None, 4, 10000.0, 0.125, None, FAKE, None, FAKE, 1 << 30,
                       None, ctypes.addressof(st), None)
    assert rc == -1
    assert lib.fp_append_kv(None, ctypes.byref(g), FAKE, FAKE, 1e4, ctypes.addressof(st), None) == -1
    assert lib.fp_append_kv(ctypes.byref(p), ctypes.byref(g), None, FAKE, 1e4, ctypes.addressof(st), None) == -1
    assert lib.fp_append_kv(ctypes.byref(p), ctypes.byref(g), FAKE, FAKE, 1e4, None, None) == -1
    assert lib.fp_fold(ctypes.byref(p), ctypes.byref(g), None, None, None) == -1


def test_mask_and_tuning_validation(lib):
    from ragged_paged_kv_fp_amd import _lib

    g, p, keep = _structs(rows=(3, 1))
    wo = np.array([0, 7, 7], np.int64)  # 7 words over 3 rows: not a whole number per row
    m = _lib.FpMask(FAKE, FAKE, wo.ctypes.data)
    assert _ws(lib, p, g, m=ctypes.byref(m)) == -2
    wo2 = np.array([0, 6, 8], np.int64)
    m2 = _lib.FpMask(FAKE, FAKE, wo2.ctypes.data)
    assert _ws(lib, p, g, m=ctypes.byref(m2)) > 0
    t = _lib.FpTuning()
    t.decode_split_slots = 48
    assert _ws(lib, p, g, t=ctypes.byref(t)) == -2
    t.decode_split_slots = 64
    assert _ws(lib, p, g, t=ctypes.byref(t)) > 0
    t.reserved[2] = 1
    assert _ws(lib, p, g, t=ctypes.byref(t)) == -2


def test_readout_default_count_checked(lib):
    g, p, keep = _structs(L=3, rows=(3, 0, 2), pages=(1, 1, 1))
    st = ctypes.c_int32(0)
    assert lib.fp_readout(ctypes.byref(g), FAKE, 8, None, 3, FAKE, ctypes.addressof(st), None) == -2
    assert lib.fp_readout(ctypes.byref(g), FAKE, 8, None, 2, FAKE, None, None) == -1
    # the one-launch fold+readout runs both calls' checks before enqueueing anything
    assert lib.fp_fold_readout(ctypes.byref(p), ctypes.byref(g), None, FAKE, 8, None, 3, FAKE,
                               ctypes.addressof(st), None) == -2
    assert lib.fp_fold_readout(ctypes.byref(p), ctypes.byref(g), None, FAKE, 8, None, 2, FAKE, None, None) == -1
    assert lib.fp_fold_readout(None, ctypes.byref(g), None, FAKE, 8, None, 2, FAKE, ctypes.addressof(st), None) == -1
    assert lib.fp_fold_readout(ctypes.byref(p), ctypes.byref(g), None, None, 8, None, 2, FAKE,
                               ctypes.addressof(st), None) == -1


def test_attn_mass_and_advance_validation(lib):
    g, p, keep = _structs()
    st = ctypes.c_int32(0)
    # mass: lse, workspace and output are required; the workspace must hold the rotated Q
    assert lib.fp_attn_mass(ctypes.byref(p), ctypes.byref(g), 4, None, None, FAKE, 1 << 20, None, FAKE, None) == -1
    assert lib.fp_attn_mass(ctypes.byref(p), ctypes.byref(g), 4, None, FAKE, FAKE, 1 << 20, None, None, None) == -1
    assert lib.fp_attn_mass(ctypes.byref(p), ctypes.byref(g), 4, None, FAKE, FAKE, 16, None, FAKE, None) == -4
    assert lib.fp_attn_mass(ctypes.byref(p), ctypes.byref(g), 5, None, FAKE, FAKE, 1 << 20, None, FAKE, None) == -2
    # advance: outputs and the pool's committed lengths are required; the host offsets must be consistent
    assert lib.fp_advance(ctypes.byref(p), ctypes.byref(g), None, FAKE, FAKE, None, None) == -1
    assert lib.fp_advance(ctypes.byref(p), ctypes.byref(g), None, None, FAKE, FAKE, None) == -1
    g.num_rows = 9
    assert lib.fp_advance(ctypes.byref(p), ctypes.byref(g), None, FAKE, FAKE, FAKE, None) == -2


@pytest.mark.parametrize("mut,code", [
    ("rank=8", -3), ("rank=80", -3), ("rank=24", -3), ("d_in=96", -3), ("d_out=48", -3),
    ("num_adapters=0", -2), ("d_in=0", -2), ("workspace=16", -4), ("status=0", -1), ("x=0", -1),
])
def test_lora_validation(lib, mut, code):
    from ragged_paged_kv_fp_amd import _lib

    g, p, keep = _structs()
    lo = _lib.FpLora(3, 16, 256, 128, FAKE, FAKE, FAKE)
    ws, status, x = 1 << 20, FAKE, FAKE
    k, v = mut.split("=")
    v = int(v)
    if k == "workspace":
        ws = v
    elif k == "status":
        status = None
    elif k == "x":
        x = None
    else:
        setattr(lo, k, v)
    rc = lib.fp_adapter_lora(ctypes.byref(g), ctypes.byref(lo), FAKE, x, FAKE, FAKE, FAKE, ws, status, None)
    assert rc == code


def test_lora_workspace_size(lib):
    from ragged_paged_kv_fp_amd import _lib

    g, p, keep = _structs(L=3, rows=(70, 0, 5), pages=(1, 1, 1))
    for rank, rp in ((16, 32), (48, 64), (64, 64)):
        lo = _lib.FpLora(2, rank, 256, 128, FAKE, FAKE, FAKE)
        n = lib.fp_lora_workspace_bytes(ctypes.byref(g), ctypes.byref(lo))
        items = 3 + 1  # ceil(70/32) + ceil(5/32)
        want = -(-(2 * 2 * 75 * rp) // 256) * 256 + -(-(16 * items) // 256) * 256
        assert n == want, (rank, n, want)


def test_ia3_validation(lib):
    g, p, keep = _structs()
    st = FAKE
    assert lib.fp_adapter_ia3(ctypes.byref(g), 2, 12, FAKE, FAKE, FAKE, FAKE, st, None) == -3
    assert lib.fp_adapter_ia3(ctypes.byref(g), 0, 64, FAKE, FAKE, FAKE, FAKE, st, None) == -2
    assert lib.fp_adapter_ia3(ctypes.byref(g), 2, 64, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.fp_adapter_ia3(ctypes.byref(g), 2, 64, None, FAKE, FAKE, FAKE, st, None) == -1
    g.num_rows = 9
    assert lib.fp_adapter_ia3(ctypes.byref(g), 2, 64, FAKE, FAKE, FAKE, FAKE, st, None) == -2


def test_noalloc_validation_before_any_device_call(lib):
    g, p, keep = _structs()
    st = ctypes.c_int32(0)
    call = lambda g_, hq=4, status=ctypes.addressof(st), q=FAKE: lib.fp_attend_noalloc(  # noqa: E731
        ctypes.byref(p), ctypes.byref(g_), q, hq, 1e4, 0.125, None, FAKE, None, None, status, None)
    assert call(g, status=None) == -1
    assert call(g, q=None) == -1
    assert call(g, hq=5) == -2
    assert lib.fp_attend_noalloc_max_bytes() == 64 << 20
    # a pass whose workspace exceeds the scratch (rotated Q of 300k rows alone) is refused
    big, pb, keep2 = _structs(L=1, rows=(300000,), pages=(1,))
    assert _ws(lib, pb, big) > lib.fp_attend_noalloc_max_bytes()
    assert lib.fp_attend_noalloc(ctypes.byref(pb), ctypes.byref(big), FAKE, 4, 1e4, 0.125, None, FAKE, None, None,
                                 ctypes.addressof(st), None) == -4


def test_hazard_check_validation(lib):
    g, p, keep = _structs(P=16)
    st = ctypes.c_int32(0)
    need = lib.fp_hazard_workspace_bytes(ctypes.byref(p))
    assert need == 3 * 4 * p.num_pages * 16
    assert lib.fp_check_hazards(ctypes.byref(p), ctypes.byref(g), FAKE, need - 1, ctypes.addressof(st), None) == -4
    assert lib.fp_check_hazards(ctypes.byref(p), ctypes.byref(g), None, need, ctypes.addressof(st), None) == -1
    assert lib.fp_check_hazards(ctypes.byref(p), ctypes.byref(g), FAKE, need, None, None) == -1
    p.page_size = 12
    assert lib.fp_hazard_workspace_bytes(ctypes.byref(p)) == -3


def test_stale_library_is_refused(lib, tmp_path):
    """The binding compares the library's compiled-in source hash with the tree's:
    the built library matches, and a changed source makes the check raise."""
    from ragged_paged_kv_fp_amd import _lib, build

    _lib.check_fresh(lib)  # the library under test was built from these sources
    changed = []
    for src in build.DEPS:
        dst = tmp_path / os.path.basename(src)
        data = open(src, "rb").read()
        if src.endswith("fp_decode.h"):
            data += b"\n// edited\n"
        dst.write_bytes(data)
        changed.append(str(dst))
    with pytest.raises(_lib.StaleLibraryError):
        _lib.check_fresh(lib, changed)
    same = [str(tmp_path / ("same_" + os.path.basename(s))) for s in build.DEPS]
    for src, dst in zip(build.DEPS, same):
        open(dst, "wb").write(open(src, "rb").read())
    with pytest.raises(_lib.StaleLibraryError):  # file names are part of the hash
        _lib.check_fresh(lib, same)


def test_tova_mask_validation(lib):
    g, p, keep = _structs()
    st = ctypes.c_int32(0)
    wo = np.array([0, 3, 3], np.int64)  # lane 0: 3 rows x 1 word, lane 1 keeps the causal rule

    def call(mass=FAKE, budget=FAKE, prev=None, plim=None, koff=FAKE, kept=FAKE, bits=FAKE, woh=wo.ctypes.data,
             status=ctypes.addressof(st)):
        return lib.fp_tova_mask(ctypes.byref(p), ctypes.byref(g), mass, budget, prev, plim, koff, kept, bits, FAKE,
                                woh, status, None)

    for kw in ("mass", "budget", "koff", "kept", "bits", "woh", "status"):
        assert call(**{kw: None}) == -1, kw
    assert call(prev=FAKE) == -1  # prev_keep without prev_limit
    bad = np.array([0, 2, 2], np.int64)  # 2 words over 3 rows
    assert call(woh=bad.ctypes.data) == -2
    p.page_size = 12
    assert call() == -3
