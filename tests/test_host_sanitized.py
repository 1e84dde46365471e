"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libfp_hostsan.so is libfp.so with its host code built with -fsanitize=address
and -fsanitize=undefined (device code untouched). A child process preloads
clang's ASan runtime, loads it through the binding and drives every host-only
path: argument validation and its error codes, the shape-only launch plans of
the configurations, random, explicit-slot and windowed-decode passes, the
hazard and no-allocation entry points' checks, frame merging and the Eq. (1)/(2)
accounting. A memory error or undefined behaviour aborts the child with a
sanitizer report; no GPU call is made.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import ctypes, sys
import numpy as np
sys.path[:0] = [ROOT, ROOT + "/tests"]
import workloads as W
from ragged_paged_kv_fp_amd import _lib, build, api, runner

lib = _lib.load(build.ASAN_LIB)
FAKE = 0x10000


def structs(wl):
    st = wl.step
    ip = st.indptr.astype(np.int32).copy()
    pp = wl.page_indptr.astype(np.int32).copy()
    g = _lib.FpGeometry(st.num_lanes, int(ip[-1]), FAKE, ip.ctypes.data, FAKE, FAKE, FAKE, FAKE)
    p = _lib.FpKvPool(FAKE, wl.num_pages, wl.P, wl.H_kv, wl.d, FAKE, pp.ctypes.data, FAKE, FAKE)
    m = None
    keep = [ip, pp]
    if wl.mask_bits is not None and wl.mask_bits.size:
        wo = wl.mask_word_offset.astype(np.int64).copy()
        keep.append(wo)
        m = _lib.FpMask(FAKE, FAKE, wo.ctypes.data)
    return g, p, m, keep


wls = [W.make_config(c, seed=1, scale="small") for c in (2, 3, 4, 5)] + [W.make_config(1)]
wls += [W.make_random(s) for s in range(4)] + [W.make_explicit(s) for s in range(4)]
wls += [W.make_window_decode(0, L=4, kv=4096, window=256)]
total = 0
for wl in wls:
    g, p, m, keep = structs(wl)
    for split in (None, 32, 512, 4096):
        t = None
        if split:
            t = _lib.FpTuning()
            t.decode_split_slots = split
        n = lib.fp_attend_workspace_bytes(ctypes.byref(p), ctypes.byref(g), ctypes.byref(m) if m else None, wl.H_q,
                                          ctypes.byref(t) if t else None)
        assert n > 0, (wl.name, split, n)
        total += n
    st = ctypes.c_int32(0)
    # validation failures return before any device call
    assert lib.fp_attend(ctypes.byref(p), ctypes.byref(g), FAKE, wl.H_q, 1e4, 0.1, None, FAKE, None, FAKE, 16, None,
                         ctypes.addressof(st), None) in (-4, 0)
    assert lib.fp_attend_noalloc(ctypes.byref(p), ctypes.byref(g), None, wl.H_q, 1e4, 0.1, None, FAKE, None, None,
                                 ctypes.addressof(st), None) in (-1, 0)
    assert lib.fp_check_hazards(ctypes.byref(p), ctypes.byref(g), FAKE, 1, ctypes.addressof(st), None) == -4
    assert lib.fp_hazard_workspace_bytes(ctypes.byref(p)) == 12 * wl.num_pages * wl.P
    assert lib.fp_attend_workspace_bytes(ctypes.byref(p), ctypes.byref(g), None, wl.H_q + 1, None) in (-2, -3)
    bad = _lib.FpKvPool(FAKE, wl.num_pages, 12, wl.H_kv, wl.d, FAKE, keep[1].ctypes.data, FAKE, FAKE)
    assert lib.fp_attend_workspace_bytes(ctypes.byref(bad), ctypes.byref(g), None, wl.H_q, None) == -3
# frame merging on split passes
for c in (1, 3):
    wl = W.make_config(c, seed=2, scale="small" if c > 1 else "full")
    rng = np.random.default_rng(c)
    A, B = W.split_pass(wl.step, [int(rng.integers(0, n + 1)) for n in np.diff(wl.step.indptr)])
    c0 = np.zeros(wl.num_lanes, np.int32)
    if wl.prefix is not None:
        c0 = np.diff(wl.prefix.indptr).astype(np.int32)
    assert api.vertical_merge(A, B, c0, wl.page_indptr, wl.P) is not None
    assert api.vertical_merge(A, B, c0 + 1, wl.page_indptr, wl.P) is None
    assert len(runner.vertical_groups([A, B], c0, wl.page_indptr, wl.P)) == 1
for T in range(0, 5000, 7):
    for P in (1, 8, 16, 32):
        assert lib.fp_page_waste(T, P) == P * (-(-T // P)) - T
assert lib.fp_kv_bytes(32, 8, 128, 8192, 2) == 1 << 30
print("host paths ok", total)
'''.replace("ROOT", repr(ROOT))


def test_host_code_under_address_and_ub_sanitizers():
    from ragged_paged_kv_fp_amd import _lib, build

    fresh = False
    if os.path.exists(build.ASAN_LIB):
        import ctypes

        probe = subprocess.run([sys.executable, "-c", "import ctypes,sys; l=ctypes.CDLL(sys.argv[1]); "
                                "l.fp_source_hash.restype=ctypes.c_char_p; print(l.fp_source_hash().decode())",
                                build.ASAN_LIB], capture_output=True, text=True,
                               env=dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(),
                                        ASAN_OPTIONS="detect_leaks=0"))
        fresh = probe.returncode == 0 and probe.stdout.strip() == build.source_hash()
    if not fresh:
        build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0 and "host paths ok" in res.stdout, out[-4000:]
