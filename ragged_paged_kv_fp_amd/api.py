"""Thin Python binding of the C ABI: argument marshalling only.

Each function takes torch tensors that live on the GPU (plus numpy host copies
of the offset arrays the library plans launches from), passes their addresses
to libfp.so and raises FpError on a negative return code. Every step of the
computation runs in the library's HIP kernels; nothing here computes.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import FpError, FpGeometry, FpKvPool, FpLora, FpMask, FpTuning


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _hptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _dev_check(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclass
class Pool:
    """One attention layer of the paged pool (page layout documented in include/fp.h)."""

    kv: torch.Tensor              # uint16/bfloat16 [num_pages][2*H*P*d] (any shape, contiguous)
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    page_indptr: torch.Tensor     # int32 [L+1] device
    page_indptr_host: np.ndarray  # int32 [L+1]
    page_ids: torch.Tensor        # int32 device
    committed_len: torch.Tensor   # int32 [L] device

    def struct(self) -> FpKvPool:
        self.page_indptr_host = np.ascontiguousarray(self.page_indptr_host, dtype=np.int32)
        return FpKvPool(_ptr(self.kv), self.num_pages, self.page_size, self.num_kv_heads, self.head_dim,
                        _ptr(self.page_indptr), _hptr(self.page_indptr_host), _ptr(self.page_ids),
                        _ptr(self.committed_len))


@dataclass
class Geometry:
    """StateGeometry of one pass: rows of lane l are [indptr[l], indptr[l+1])."""

    indptr: torch.Tensor          # int32 [L+1] device
    indptr_host: np.ndarray       # int32 [L+1]
    positions: torch.Tensor       # int32 [N]
    slots: torch.Tensor           # int32 [N]
    kv_len: torch.Tensor          # int32 [L]
    fold: torch.Tensor            # int32 [L]

    @property
    def num_lanes(self) -> int:
        return int(self.indptr_host.shape[0] - 1)

    @property
    def num_rows(self) -> int:
        return int(self.indptr_host[-1])

    def struct(self) -> FpGeometry:
        self.indptr_host = np.ascontiguousarray(self.indptr_host, dtype=np.int32)
        return FpGeometry(self.num_lanes, self.num_rows, _ptr(self.indptr), _hptr(self.indptr_host),
                          _ptr(self.positions), _ptr(self.slots), _ptr(self.kv_len), _ptr(self.fold))


@dataclass
class Mask:
    bits: torch.Tensor                # int32/uint32 words, device
    word_offset: torch.Tensor         # int64 [L+1] device
    word_offset_host: np.ndarray      # int64 [L+1]

    def struct(self) -> FpMask:
        self.word_offset_host = np.ascontiguousarray(self.word_offset_host, dtype=np.int64)
        return FpMask(_ptr(self.bits), _ptr(self.word_offset), _hptr(self.word_offset_host))


def _tuning(split: Optional[int], events=None):
    if split is None and events is None:
        return None
    t = FpTuning()
    t.decode_split_slots = int(split or 0)
    if events is not None:
        t.attn_begin, t.attn_end = int(events[0]), int(events[1])
        if len(events) > 2:  # (begin, end, prefill_end, merge_end)
            t.prefill_end, t.merge_end = int(events[2]), int(events[3])
    return ctypes.byref(t)


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        raise FpError(fn, rc)
    return rc


def append_kv(pool: Pool, geom: Geometry, k: torch.Tensor, v: torch.Tensor, rope_theta: float,
              status: torch.Tensor, stream=None) -> None:
    """fp_append_kv: RoPE K at positions, write K/V into each row's slot."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    _check("fp_append_kv", lib.fp_append_kv(ctypes.byref(ps), ctypes.byref(gs), _ptr(k), _ptr(v),
                                            float(rope_theta), _ptr(status), _stream(stream)))


def attend_workspace_bytes(pool: Pool, geom: Geometry, num_q_heads: int, mask: Optional[Mask] = None,
                           split: Optional[int] = None) -> int:
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    ms = mask.struct() if mask is not None else None
    return _check("fp_attend_workspace_bytes",
                  lib.fp_attend_workspace_bytes(ctypes.byref(ps), ctypes.byref(gs),
                                                ctypes.byref(ms) if ms is not None else None,
                                                int(num_q_heads), _tuning(split)))


def attend(pool: Pool, geom: Geometry, q: torch.Tensor, num_q_heads: int, rope_theta: float, sm_scale: float,
           out: torch.Tensor, workspace: torch.Tensor, status: torch.Tensor, lse: Optional[torch.Tensor] = None,
           mask: Optional[Mask] = None, split: Optional[int] = None, stream=None, events=None) -> None:
    """fp_attend: attention of every row over its lane's kv_len slots (causal or bitmap).

    events: optional raw hipEvent_t handles (begin, end) recorded around the attention kernels, or
    (begin, end, prefill_end, merge_end) to also split prefill from decode and time the split merge.
    """
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    ms = mask.struct() if mask is not None else None
    _check("fp_attend", lib.fp_attend(ctypes.byref(ps), ctypes.byref(gs), _ptr(q), int(num_q_heads),
                                      float(rope_theta), float(sm_scale),
                                      ctypes.byref(ms) if ms is not None else None,
                                      _ptr(out), _ptr(lse), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _tuning(split, events),
                                      _ptr(status), _stream(stream)))


def attend_noalloc(pool: Pool, geom: Geometry, q: torch.Tensor, num_q_heads: int, rope_theta: float,
                   sm_scale: float, out: torch.Tensor, status: torch.Tensor, lse: Optional[torch.Tensor] = None,
                   mask: Optional[Mask] = None, split: Optional[int] = None, stream=None, events=None) -> None:
    """fp_attend_noalloc: fp_attend on the library's static device scratch (no workspace argument)."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    ms = mask.struct() if mask is not None else None
    _check("fp_attend_noalloc", lib.fp_attend_noalloc(ctypes.byref(ps), ctypes.byref(gs), _ptr(q), int(num_q_heads),
                                                      float(rope_theta), float(sm_scale),
                                                      ctypes.byref(ms) if ms is not None else None,
                                                      _ptr(out), _ptr(lse), _tuning(split, events), _ptr(status),
                                                      _stream(stream)))


def attend_noalloc_max_bytes() -> int:
    return int(_lib.load().fp_attend_noalloc_max_bytes())


def hazard_workspace_bytes(pool: Pool) -> int:
    lib = _lib.load()
    ps = pool.struct()
    return _check("fp_hazard_workspace_bytes", lib.fp_hazard_workspace_bytes(ctypes.byref(ps)))


def check_hazards(pool: Pool, geom: Geometry, workspace: torch.Tensor, status: torch.Tensor, stream=None) -> None:
    """fp_check_hazards: Eq. (4) write/read conflicts of the pass's lanes (debug; before append_kv)."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    _check("fp_check_hazards", lib.fp_check_hazards(ctypes.byref(ps), ctypes.byref(gs), _ptr(workspace),
                                                    workspace.numel() * workspace.element_size(), _ptr(status),
                                                    _stream(stream)))


def fold(pool: Pool, geom: Geometry, status: torch.Tensor, channel: Optional[torch.Tensor] = None,
         stream=None) -> None:
    """fp_fold: committed_len += none | all | literal | channel count, clamped."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    _check("fp_fold", lib.fp_fold(ctypes.byref(ps), ctypes.byref(gs), _ptr(channel), _ptr(status),
                                  _stream(stream)))


def readout(geom: Geometry, out: torch.Tensor, dst: torch.Tensor, status: torch.Tensor,
            rows: Optional[torch.Tensor] = None, stream=None) -> None:
    """fp_readout: gather the chosen rows of out (default: last row of each lane)."""
    lib = _lib.load()
    gs = geom.struct()
    row_elems = int(out.numel() // max(1, geom.num_rows)) if geom.num_rows else int(dst.shape[-1])
    num = int(dst.shape[0])
    _check("fp_readout", lib.fp_readout(ctypes.byref(gs), _ptr(out), row_elems, _ptr(rows), num, _ptr(dst),
                                        _ptr(status), _stream(stream)))


def fold_readout(pool: Pool, geom: Geometry, out: torch.Tensor, dst: torch.Tensor, status: torch.Tensor,
                 channel: Optional[torch.Tensor] = None, rows: Optional[torch.Tensor] = None, stream=None) -> None:
    """fp_fold_readout: fold() then readout() of the same pass, in one launch."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    row_elems = int(out.numel() // max(1, geom.num_rows)) if geom.num_rows else int(dst.shape[-1])
    num = int(dst.shape[0])
    _check("fp_fold_readout", lib.fp_fold_readout(ctypes.byref(ps), ctypes.byref(gs), _ptr(channel), _ptr(out),
                                                  row_elems, _ptr(rows), num, _ptr(dst), _ptr(status),
                                                  _stream(stream)))


def attn_mass(pool: Pool, geom: Geometry, num_q_heads: int, lse: torch.Tensor, workspace: torch.Tensor,
              slot_mass: torch.Tensor, mask: Optional[Mask] = None, split: Optional[int] = None,
              stream=None) -> None:
    """fp_attn_mass: add each slot's attention mass of the pass (per KV head) into
    slot_mass [H_kv][page_indptr[L] * P]; call after attend() with the same
    pool, geom, mask, split and workspace."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    ms = mask.struct() if mask is not None else None
    _check("fp_attn_mass", lib.fp_attn_mass(ctypes.byref(ps), ctypes.byref(gs), int(num_q_heads),
                                            ctypes.byref(ms) if ms is not None else None, _ptr(lse),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _tuning(split), _ptr(slot_mass), _stream(stream)))


def tova_mask(pool: Pool, geom: Geometry, slot_mass: torch.Tensor, budget: torch.Tensor,
              keep_word_offset: torch.Tensor, keep: torch.Tensor, mask: Mask, status: torch.Tensor,
              prev_keep: Optional[torch.Tensor] = None, prev_limit: Optional[torch.Tensor] = None,
              stream=None) -> None:
    """fp_tova_mask: per lane keep the budget old slots (below committed_len) with
    the largest attention mass summed over KV heads, then write the pass's row
    bitmaps into mask.bits (kept old slots + the pass's own slots by slot order)."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    ms = mask.struct()
    _check("fp_tova_mask", lib.fp_tova_mask(ctypes.byref(ps), ctypes.byref(gs), _ptr(slot_mass), _ptr(budget),
                                            _ptr(prev_keep), _ptr(prev_limit), _ptr(keep_word_offset), _ptr(keep),
                                            ms.bits, ms.word_offset, ms.word_offset_host, _ptr(status),
                                            _stream(stream)))


@dataclass
class Lora:
    """Adapters of one projection site: A [n][rank][d_in], B [n][d_out][rank] (bf16), scale [n] (fp32)."""

    a: torch.Tensor
    b: torch.Tensor
    scale: torch.Tensor

    def struct(self) -> FpLora:
        n, r, d_in = self.a.shape
        return FpLora(int(n), int(r), int(d_in), int(self.b.shape[1]), _ptr(self.a), _ptr(self.b), _ptr(self.scale))


def lora_workspace_bytes(geom: Geometry, lora: Lora) -> int:
    lib = _lib.load()
    gs, ls = geom.struct(), lora.struct()
    return _check("fp_lora_workspace_bytes", lib.fp_lora_workspace_bytes(ctypes.byref(gs), ctypes.byref(ls)))


def adapter_lora(geom: Geometry, lora: Lora, adapter: torch.Tensor, x: torch.Tensor, y: torch.Tensor,
                 out: torch.Tensor, workspace: torch.Tensor, status: torch.Tensor, stream=None) -> None:
    """fp_adapter_lora: out = bf16(y + s_k B_k (A_k x)) per lane's adapter k (y kept where k < 0)."""
    lib = _lib.load()
    gs, ls = geom.struct(), lora.struct()
    _check("fp_adapter_lora", lib.fp_adapter_lora(ctypes.byref(gs), ctypes.byref(ls), _ptr(adapter), _ptr(x),
                                                  _ptr(y), _ptr(out), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(), _ptr(status),
                                                  _stream(stream)))


def adapter_ia3(geom: Geometry, scale: torch.Tensor, adapter: torch.Tensor, y: torch.Tensor, out: torch.Tensor,
                status: torch.Tensor, stream=None) -> None:
    """fp_adapter_ia3: out = bf16(y * scale[k]) per lane's adapter k (y kept where k < 0); scale [n][d_out] bf16."""
    lib = _lib.load()
    gs = geom.struct()
    n, d_out = scale.shape
    _check("fp_adapter_ia3", lib.fp_adapter_ia3(ctypes.byref(gs), int(n), int(d_out), _ptr(scale), _ptr(adapter),
                                                _ptr(y), _ptr(out), _ptr(status), _stream(stream)))


def advance(pool: Pool, geom: Geometry, pos_offset: Optional[torch.Tensor] = None, stream=None) -> None:
    """fp_advance: write geom's positions / slots / kv_len on the device from the
    pool's committed lengths (rows appended after the frozen prefix)."""
    lib = _lib.load()
    ps, gs = pool.struct(), geom.struct()
    _check("fp_advance", lib.fp_advance(ctypes.byref(ps), ctypes.byref(gs), _ptr(pos_offset), _ptr(geom.positions),
                                        _ptr(geom.slots), _ptr(geom.kv_len), _stream(stream)))


def vertical_merge(a, b, committed: np.ndarray, page_indptr_host: np.ndarray, page_size: int):
    """fp_vertical_merge on host copies of two consecutive passes a, b (objects
    with indptr, slots, kv_len, fold as numpy int32 arrays). Returns None when
    one pass cannot do what a then b do, else a dict with the merged pass's
    indptr, kv_len, fold and the row maps src_row, row_of_a, row_of_b."""
    lib = _lib.load()
    L = int(len(a.indptr) - 1)
    i32 = lambda x: np.ascontiguousarray(x, dtype=np.int32)  # noqa: E731
    ia, sa, ka, fa = i32(a.indptr), i32(a.slots), i32(a.kv_len), i32(a.fold)
    ib, sb, kb, fb = i32(b.indptr), i32(b.slots), i32(b.kv_len), i32(b.fold)
    c, pp = i32(committed), i32(page_indptr_host)
    NA, NB = int(ia[-1]), int(ib[-1])
    out = dict(indptr=np.zeros(L + 1, np.int32), src_row=np.zeros(max(NA + NB, 1), np.int32),
               row_of_a=np.zeros(max(NA, 1), np.int32), row_of_b=np.zeros(max(NB, 1), np.int32),
               kv_len=np.zeros(L, np.int32), fold=np.zeros(L, np.int32))
    rc = lib.fp_vertical_merge(L, _hptr(ia), _hptr(sa), _hptr(ka), _hptr(fa), _hptr(ib), _hptr(sb), _hptr(kb),
                               _hptr(fb), _hptr(c), _hptr(pp), int(page_size), _hptr(out["indptr"]),
                               _hptr(out["src_row"]), _hptr(out["row_of_a"]), _hptr(out["row_of_b"]),
                               _hptr(out["kv_len"]), _hptr(out["fold"]))
    if rc == 1:
        return None
    _check("fp_vertical_merge", rc)
    out["src_row"], out["row_of_a"], out["row_of_b"] = out["src_row"][:NA + NB], out["row_of_a"][:NA], out["row_of_b"][:NB]
    return out


def kv_bytes(L: int, H_kv: int, d: int, T: int, b: int) -> int:
    return int(_lib.load().fp_kv_bytes(L, H_kv, d, T, b))


def pages_for(T: int, P: int) -> int:
    return int(_lib.load().fp_pages_for(T, P))


def page_waste(T: int, P: int) -> int:
    return int(_lib.load().fp_page_waste(T, P))


def page_bytes(P: int, H_kv: int, d: int) -> int:
    return int(_lib.load().fp_page_bytes(P, H_kv, d))


def version() -> str:
    return _lib.load().fp_version().decode()
