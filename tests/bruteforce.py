"""Independent dense brute force of the ForwardPass attention step, pure Python.

Used only to pin the paged fp64 oracle on tiny inputs. It shares no code with
the oracle: no page table (a lane's KV is a dict slot -> vectors), RoPE as a
complex multiplication, bf16 rounding by exact rational arithmetic, attention
by the textbook formula with explicit loops.
"""

from __future__ import annotations

import cmath
import math
import struct
from fractions import Fraction


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def bf16_round_exact(x: float) -> int:
    """Nearest-even bf16 of a finite double, decided in exact rational arithmetic."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    a = Fraction(abs(x))
    # bf16 normal numbers: (1 + m/128) * 2^(e-127), e in 1..254
    e = math.floor(math.log2(abs(x)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < -126 or e > 127:
        raise ValueError("outside the bf16 normal range")
    ulp = Fraction(2) ** (e - 7)
    lo = (a // ulp) * ulp
    hi = lo + ulp
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:  # tie: even significand
        r = lo if (lo / ulp) % 2 == 0 else hi
    f = float(r)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert u & 0xFFFF == 0
    return sign | (u >> 16)


def rope_complex(vec, pos, theta):
    """Rotate pairs as complex numbers z_i = x[2i] + i x[2i+1] times exp(i pos w_i)."""
    d = len(vec)
    out = [0.0] * d
    for i in range(d // 2):
        w = float(theta) ** (-2.0 * i / d)
        z = complex(vec[2 * i], vec[2 * i + 1]) * cmath.exp(1j * (pos * w))
        out[2 * i], out[2 * i + 1] = z.real, z.imag
    return out


def run(wl_arrays, *, H_q, H_kv, d, theta, sm_scale, cap, prefix=None, committed0=None, hole_bits=None):
    """Dense brute force of one pass.

    wl_arrays: dict with indptr, positions, slots, kv_len, fold, k, v, q (lists / numpy),
    optional mask (per global row: set of slots, or None for causal), channel.
    cap: per-lane capacity in slots. prefix: same dict shape for a pre-pass (append, then its fold).
    hole_bits: bf16 bit pattern every never-written slot holds (K and V alike);
    None means no row may read such a slot.
    Returns dict(O, LSE, committed, store, mass) with O[row][head] lists and
    mass[lane][(kv head, slot)] the summed attention probability of the slot.
    """
    L = len(wl_arrays["indptr"]) - 1
    store = [dict() for _ in range(L)]
    committed = list(committed0) if committed0 is not None else [0] * L

    def do_append(p):
        for lane in range(L):
            for r in range(int(p["indptr"][lane]), int(p["indptr"][lane + 1])):
                s = int(p["slots"][r])
                if s < 0 or s >= cap[lane] or s < committed[lane]:
                    continue
                ks, vs = [], []
                for h in range(H_kv):
                    kv = [bf16_value(b) for b in p["k"][r][h]]
                    rot = rope_complex(kv, int(p["positions"][r]), theta)
                    ks.append([bf16_value(bf16_round_exact(t)) for t in rot])
                    vs.append([bf16_value(b) for b in p["v"][r][h]])
                store[lane][s] = (ks, vs)

    def do_fold(p, channel):
        for lane in range(L):
            n = int(p["indptr"][lane + 1]) - int(p["indptr"][lane])
            f = int(p["fold"][lane])
            if f == -1:
                k = n
            elif f == -2:
                k = 0 if channel is None else int(channel[lane])
            elif f >= 0:
                k = f
            else:
                k = 0
            committed[lane] += min(max(k, 0), n)

    if prefix is not None:
        do_append(prefix)
        do_fold(prefix, None)

    def slot_kv(lane, j):
        if j in store[lane]:
            return store[lane][j]
        if hole_bits is None:
            raise KeyError(f"lane {lane} reads slot {j}, which was never written")
        hv = [bf16_value(hole_bits)] * d
        return [hv] * H_kv, [hv] * H_kv

    w = wl_arrays
    do_append(w)
    G = H_q // H_kv
    N = int(w["indptr"][-1])
    O = [[[0.0] * d for _ in range(H_q)] for _ in range(N)]
    LSE = [[-math.inf] * H_q for _ in range(N)]
    masks = w.get("mask")
    mass = [dict() for _ in range(L)]  # lane -> {(kv head, slot): summed probability}
    for lane in range(L):
        eff = min(max(int(w["kv_len"][lane]), 0), cap[lane])
        for r in range(int(w["indptr"][lane]), int(w["indptr"][lane + 1])):
            if masks is not None and masks[r] is not None:
                allowed = sorted(j for j in masks[r] if j < eff)
            else:
                allowed = list(range(min(eff, int(w["slots"][r]) + 1)))
            if not allowed:
                continue
            for hq in range(H_q):
                g = hq // G
                qv = rope_complex([bf16_value(b) for b in w["q"][r][hq]], int(w["positions"][r]), theta)
                scores = []
                for j in allowed:
                    kj = slot_kv(lane, j)[0][g]
                    scores.append(sum(a * b for a, b in zip(qv, kj)) * sm_scale)
                m = max(scores)
                ps = [math.exp(s - m) for s in scores]
                tot = sum(ps)
                for p_, j in zip(ps, allowed):
                    mass[lane][(g, j)] = mass[lane].get((g, j), 0.0) + p_ / tot
                acc = [0.0] * d
                for p_, j in zip(ps, allowed):
                    vj = slot_kv(lane, j)[1][g]
                    for t in range(d):
                        acc[t] += p_ * vj[t]
                O[r][hq] = [a / tot for a in acc]
                LSE[r][hq] = m + math.log(tot)
    do_fold(w, w.get("channel"))
    return dict(O=O, LSE=LSE, committed=committed, store=store, mass=mass)


def lora(x, y, adapter, indptr, a, b, scale):
    """Adapter output by explicit loops: out[r][i] = bf16(y + s * sum_j b[i][j] * sum_t a[j][t] x[t]).
    Arguments are nested lists of bf16 bit patterns (scale: floats). Returns (bits, exact)."""
    bits = [list(row) for row in y]
    exact = [[bf16_value(v) for v in row] for row in y]
    for lane in range(len(indptr) - 1):
        k = int(adapter[lane])
        if k < 0 or k >= len(a):
            continue
        for r in range(int(indptr[lane]), int(indptr[lane + 1])):
            xv = [bf16_value(t) for t in x[r]]
            v = [sum(bf16_value(a[k][j][t]) * xv[t] for t in range(len(xv))) for j in range(len(a[k]))]
            for i in range(len(y[r])):
                e = bf16_value(y[r][i]) + scale[k] * sum(bf16_value(b[k][i][j]) * v[j] for j in range(len(v)))
                exact[r][i] = e
                bits[r][i] = bf16_round_exact(e)
    return bits, exact
