"""Device buffers for one pass and the ABI calls in order.

Uploads a host-side description of a pass (offset arrays, slots, positions,
bf16 bit patterns, page table, masks, channel) into caller-owned torch
tensors and issues append -> attend -> fold + readout (one launch) on one
stream; fold() and readout() remain for callers that want them apart.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import api


def _dev(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def _bits16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def _geometry(p, device) -> api.Geometry:
    return api.Geometry(indptr=_dev(p.indptr.astype(np.int32), device), indptr_host=p.indptr.astype(np.int32).copy(),
                        positions=_dev(p.positions.astype(np.int32), device),
                        slots=_dev(p.slots.astype(np.int32), device),
                        kv_len=_dev(p.kv_len.astype(np.int32), device), fold=_dev(p.fold.astype(np.int32), device))


class DeviceStep:
    """Owns the device tensors of one workload (a prefix pass plus the step)."""

    def __init__(self, wl, device="cuda", fill_bits: int = 0, split: Optional[int] = None, with_lse: bool = True):
        self.wl = wl
        self.device = torch.device(device)
        self.split = split
        dev = self.device
        page_elems = 2 * wl.H_kv * wl.P * wl.d
        fill = int(np.array([fill_bits], dtype=np.uint16).view(np.int16)[0])
        self.pool_t = torch.full((wl.num_pages, page_elems), fill, dtype=torch.int16, device=dev)
        L = wl.num_lanes
        self.pool = api.Pool(kv=self.pool_t, num_pages=wl.num_pages, page_size=wl.P, num_kv_heads=wl.H_kv,
                             head_dim=wl.d, page_indptr=_dev(wl.page_indptr.astype(np.int32), dev),
                             page_indptr_host=wl.page_indptr.astype(np.int32).copy(),
                             page_ids=_dev(wl.page_ids.astype(np.int32), dev),
                             committed_len=torch.zeros(L, dtype=torch.int32, device=dev))
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.prefix_geom = _geometry(wl.prefix, dev) if wl.prefix is not None else None
        if wl.prefix is not None:
            self.prefix_k = _bits16(wl.prefix.k, dev)
            self.prefix_v = _bits16(wl.prefix.v, dev)
        st = wl.step
        self.geom = _geometry(st, dev)
        self.k = _bits16(st.k, dev)
        self.v = _bits16(st.v, dev)
        self.q = _bits16(st.q, dev)
        N = st.num_rows
        self.out = torch.zeros((N, wl.H_q, wl.d), dtype=torch.float32, device=dev)
        self.lse = torch.zeros((N, wl.H_q), dtype=torch.float32, device=dev) if with_lse else None
        self.mask = None
        if wl.mask_bits is not None and wl.mask_bits.size > 0:  # all spans empty: every lane causal
            self.mask = api.Mask(bits=_dev(wl.mask_bits.view(np.int32), dev),
                                 word_offset=_dev(wl.mask_word_offset.astype(np.int64), dev),
                                 word_offset_host=wl.mask_word_offset.astype(np.int64).copy())
        self.channel = _dev(wl.channel.astype(np.int32), dev) if wl.channel is not None else None
        self.readout_rows = _dev(wl.readout_rows.astype(np.int32), dev) if wl.readout_rows is not None else None
        if wl.readout_rows is not None:
            nro = len(wl.readout_rows)
        else:
            nro = int((np.diff(st.indptr) > 0).sum())
        self.dst = torch.zeros((nro, wl.H_q * wl.d), dtype=torch.float32, device=dev)
        ws = api.attend_workspace_bytes(self.pool, self.geom, wl.H_q, self.mask, split)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.committed0 = None

    # ------------------------------------------------------------------ passes
    def run_prefix(self) -> None:
        """Append the cached prefix of every lane and fold it (untimed set-up)."""
        wl = self.wl
        if self.prefix_geom is not None:
            api.append_kv(self.pool, self.prefix_geom, self.prefix_k, self.prefix_v, wl.theta, self.status)
            api.fold(self.pool, self.prefix_geom, self.status)
        self.committed0 = self.pool.committed_len.clone()

    def reset(self) -> None:
        """Restore committed_len to its post-prefix value so the step can be replayed."""
        self.pool.committed_len.copy_(self.committed0)

    def append(self, stream=None):
        api.append_kv(self.pool, self.geom, self.k, self.v, self.wl.theta, self.status, stream)

    def attend(self, stream=None, split=None, events=None):
        wl = self.wl
        api.attend(self.pool, self.geom, self.q, wl.H_q, wl.theta, wl.sm_scale, self.out, self.workspace,
                   self.status, self.lse, self.mask, self.split if split is None else split, stream, events)

    def fold(self, stream=None):
        api.fold(self.pool, self.geom, self.status, self.channel, stream)

    def readout(self, stream=None):
        api.readout(self.geom, self.out, self.dst, self.status, self.readout_rows, stream)

    def finish(self, stream=None):
        """fold() and readout() of the pass, in one launch."""
        api.fold_readout(self.pool, self.geom, self.out, self.dst, self.status, self.channel, self.readout_rows,
                         stream)

    def step(self, stream=None, events=None) -> None:
        self.append(stream)
        self.attend(stream, events=events)
        self.finish(stream)

    # ------------------------------------------------------------------ views
    def pool_logical(self):
        """Pool as (K [pages][H][P][d], V [pages][H][P][d]) uint16 numpy arrays (V un-transposed)."""
        wl = self.wl
        raw = self.pool_t.cpu().numpy().view(np.uint16).reshape(wl.num_pages, 2, wl.H_kv, -1)
        K = raw[:, 0].reshape(wl.num_pages, wl.H_kv, wl.P, wl.d)
        V = raw[:, 1].reshape(wl.num_pages, wl.H_kv, wl.d, wl.P).transpose(0, 1, 3, 2)
        return K, V


class RunAheadLoop:
    """Device buffers of a repeating decode loop (pass shape fixed, geometry from
    committed_len): per pass advance -> append -> attend -> fold(channel) ->
    readout, all on one stream with no host round trip between passes.

    Inputs of pass t are uploaded up front (k[t], v[t], q[t], accept[t]); the
    pass itself reads the static buffers k, v, q, channel, so a caller may
    capture one pass in a HIP graph and feed it by copying into them.
    """

    def __init__(self, ra, device="cuda", split: Optional[int] = None):
        self.ra = ra
        self.device = dev = torch.device(device)
        self.split = split
        L, N = ra.num_lanes, int(ra.indptr[-1])
        self.pool_t = torch.zeros((ra.num_pages, 2 * ra.H_kv * ra.P * ra.d), dtype=torch.int16, device=dev)
        self.pool = api.Pool(kv=self.pool_t, num_pages=ra.num_pages, page_size=ra.P, num_kv_heads=ra.H_kv,
                             head_dim=ra.d, page_indptr=_dev(ra.page_indptr.astype(np.int32), dev),
                             page_indptr_host=ra.page_indptr.astype(np.int32).copy(),
                             page_ids=_dev(ra.page_ids.astype(np.int32), dev),
                             committed_len=torch.zeros(L, dtype=torch.int32, device=dev))
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.geom = api.Geometry(indptr=_dev(ra.indptr.astype(np.int32), dev),
                                 indptr_host=ra.indptr.astype(np.int32).copy(),
                                 positions=torch.zeros(N, dtype=torch.int32, device=dev),
                                 slots=torch.zeros(N, dtype=torch.int32, device=dev),
                                 kv_len=torch.zeros(L, dtype=torch.int32, device=dev),
                                 fold=torch.full((L,), -2, dtype=torch.int32, device=dev))
        self.pos_offset = _dev(ra.pos_offset.astype(np.int32), dev)
        self.ks = [_bits16(x, dev) for x in ra.k]
        self.vs = [_bits16(x, dev) for x in ra.v]
        self.qs = [_bits16(x, dev) for x in ra.q]
        self.accepts = [_dev(a.astype(np.int32), dev) for a in ra.accept]
        self.k = torch.empty_like(self.ks[0]) if ra.passes else None
        self.v = torch.empty_like(self.vs[0]) if ra.passes else None
        self.q = torch.empty_like(self.qs[0]) if ra.passes else None
        self.channel = torch.zeros(L, dtype=torch.int32, device=dev)
        self.out = torch.zeros((N, ra.H_q, ra.d), dtype=torch.float32, device=dev)
        self.lse = torch.zeros((N, ra.H_q), dtype=torch.float32, device=dev)
        nro = int((np.diff(ra.indptr) > 0).sum())
        self.dst = torch.zeros((nro, ra.H_q * ra.d), dtype=torch.float32, device=dev)
        ws = api.attend_workspace_bytes(self.pool, self.geom, ra.H_q, None, split)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        if ra.prefix is not None:
            p = ra.prefix
            g = _geometry(p, dev)
            api.append_kv(self.pool, g, _bits16(p.k, dev), _bits16(p.v, dev), ra.theta, self.status)
            api.fold(self.pool, g, self.status)

    def load(self, t: int, stream=None) -> None:
        """Copy pass t's inputs into the static buffers (stream-ordered)."""
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            self.k.copy_(self.ks[t], non_blocking=True)
            self.v.copy_(self.vs[t], non_blocking=True)
            self.q.copy_(self.qs[t], non_blocking=True)
            self.channel.copy_(self.accepts[t], non_blocking=True)

    def one_pass(self, stream=None) -> None:
        ra = self.ra
        api.advance(self.pool, self.geom, self.pos_offset, stream)
        api.append_kv(self.pool, self.geom, self.k, self.v, ra.theta, self.status, stream)
        api.attend(self.pool, self.geom, self.q, ra.H_q, ra.theta, ra.sm_scale, self.out, self.workspace,
                   self.status, self.lse, None, self.split, stream)
        api.fold_readout(self.pool, self.geom, self.out, self.dst, self.status, self.channel, None, stream)

    def pool_logical(self):
        ra = self.ra
        raw = self.pool_t.cpu().numpy().view(np.uint16).reshape(ra.num_pages, 2, ra.H_kv, -1)
        K = raw[:, 0].reshape(ra.num_pages, ra.H_kv, ra.P, ra.d)
        V = raw[:, 1].reshape(ra.num_pages, ra.H_kv, ra.d, ra.P).transpose(0, 1, 3, 2)
        return K, V


class _Rows:
    """Host description of one pass (the fields the ABI calls take)."""

    def __init__(self, indptr, positions, slots, kv_len, fold, k, v, q):
        self.indptr, self.positions, self.slots = indptr, positions, slots
        self.kv_len, self.fold, self.k, self.v, self.q = kv_len, fold, k, v, q

    @property
    def num_lanes(self) -> int:
        return int(self.indptr.shape[0] - 1)

    @property
    def num_rows(self) -> int:
        return int(self.indptr[-1])


def _committed_after(c: np.ndarray, p) -> Optional[np.ndarray]:
    """Committed lengths after pass p's fold, when they follow from its host
    arrays (all or a literal count; a channel count is only known on the device)."""
    n = np.diff(p.indptr).astype(np.int64)
    f = np.asarray(p.fold, dtype=np.int64)
    if np.any(f < -1):
        return None
    k = np.where(f == -1, n, np.clip(f, 0, n))
    return (c.astype(np.int64) + k).astype(np.int32)


def vertical_groups(passes, committed0: np.ndarray, page_indptr_host: np.ndarray, page_size: int):
    """Vertical batching of a frame (the reviews' section 5: a prefix forward
    and its continuation combined into one dispatch, order kept inside it):
    consecutive passes are merged greedily for as long as fp_vertical_merge
    finds the merged pass equivalent. Returns a list of groups, each a dict
    with the pass to run ('pass') and, per original pass of the group, its
    index and the merged rows of its rows ('parts': [(index, rows)])."""
    groups = []
    c_next = np.asarray(committed0, dtype=np.int32)  # committed lengths before the next group (None: unknown)
    cur, c_cur = None, None
    for idx, p in enumerate(passes):
        if cur is not None and c_cur is not None:
            m = api.vertical_merge(cur["pass"], p, c_cur, page_indptr_host, page_size)
            if m is not None:
                a = cur["pass"]
                pick = lambda x, y: np.concatenate([x, y])[m["src_row"]]  # noqa: E731
                cur["pass"] = _Rows(m["indptr"], pick(a.positions, p.positions), pick(a.slots, p.slots), m["kv_len"],
                                    m["fold"], pick(a.k, p.k), pick(a.v, p.v), pick(a.q, p.q))
                cur["parts"] = [(i, m["row_of_a"][rows]) for i, rows in cur["parts"]] + [(idx, m["row_of_b"])]
                continue
        if cur is not None:
            groups.append(cur)
            c_next = None if c_cur is None else _committed_after(c_cur, cur["pass"])
        cur = {"pass": _Rows(np.asarray(p.indptr, np.int32), p.positions, p.slots, p.kv_len, p.fold, p.k, p.v, p.q),
               "parts": [(idx, np.arange(p.num_rows, dtype=np.int32))]}
        c_cur = c_next
    if cur is not None:
        groups.append(cur)
    return groups


class Frame:
    """Several passes over one pool submitted back to back (Pie's submit_frame:
    passes in consecutive scheduler waves, in order), each pass being the four
    ABI calls with its own geometry, inputs and outputs.

    With vertical=True, consecutive passes that one pass can replace exactly
    (fp_vertical_merge: a prefix and its continuation on the same lanes) are
    merged first, so the frame issues one append and one attend for them; the
    readout rows of every original pass are gathered by the merged pass's
    explicit readout list, and parts()/readout_of() map the merged outputs
    back to the original passes.

    run() enqueues the whole frame eagerly; capture() records it once into a
    HIP graph and replay() then submits it with one launch from the host. The
    frame restores the committed lengths it started from first, so it can be
    replayed; that restore is a device-to-device copy, not a memset.
    """

    def __init__(self, pool: api.Pool, passes, H_q: int, theta: float, sm_scale: float, device="cuda",
                 vertical: bool = False):
        self.pool = pool
        self.H_q, self.theta, self.sm_scale = H_q, float(theta), float(sm_scale)
        dev = torch.device(device)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.committed0 = pool.committed_len.clone()
        if vertical:
            groups = vertical_groups(passes, self.committed0.cpu().numpy(), pool.page_indptr_host, pool.page_size)
        else:
            groups = [{"pass": p, "parts": [(i, np.arange(p.num_rows, dtype=np.int32))]} for i, p in enumerate(passes)]
        self.items = []
        for grp in groups:
            p = grp["pass"]
            g = _geometry(p, dev)
            N = p.num_rows
            it = dict(geom=g, k=_bits16(p.k, dev), v=_bits16(p.v, dev), q=_bits16(p.q, dev),
                      out=torch.zeros((N, H_q, pool.head_dim), dtype=torch.float32, device=dev),
                      lse=torch.zeros((N, H_q), dtype=torch.float32, device=dev), parts=grp["parts"])
            # readout: every original pass's default rows (the last row of each lane it has rows in)
            rl, spans = [], []
            for idx, rows in grp["parts"]:
                ip = np.asarray(passes[idx].indptr, dtype=np.int64)
                last = (ip[1:] - 1)[np.diff(ip) > 0]
                spans.append((idx, len(rl), len(rl) + len(last)))
                rl.extend(rows[last].tolist())
            it["readout_rows"] = None if len(grp["parts"]) == 1 else _dev(np.asarray(rl, np.int32), dev)
            it["spans"] = spans
            it["dst"] = torch.zeros((max(len(rl), 1), H_q * pool.head_dim), dtype=torch.float32, device=dev)
            it["nro"] = len(rl)
            ws = api.attend_workspace_bytes(pool, g, H_q)
            it["ws"] = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
            self.items.append(it)
        self.graph = None

    def run(self) -> None:
        self.pool.committed_len.copy_(self.committed0)
        for it in self.items:
            g = it["geom"]
            api.append_kv(self.pool, g, it["k"], it["v"], self.theta, self.status)
            api.attend(self.pool, g, it["q"], self.H_q, self.theta, self.sm_scale, it["out"], it["ws"], self.status,
                       it["lse"])
            api.fold_readout(self.pool, g, it["out"], it["dst"][:it["nro"]], self.status, None, it["readout_rows"])

    def parts(self):
        """(original pass index, its rows' out, its rows' lse) for every original pass, in frame order."""
        res = []
        for it in self.items:
            for idx, rows in it["parts"]:
                r = torch.from_numpy(rows.astype(np.int64)).to(it["out"].device)
                res.append((idx, it["out"][r], it["lse"][r]))
        return sorted(res, key=lambda x: x[0])

    def readout_of(self, idx: int) -> torch.Tensor:
        """The readout rows of original pass idx (its default: last row of each lane with rows)."""
        for it in self.items:
            for j, lo, hi in it["spans"]:
                if j == idx:
                    return it["dst"][lo:hi]
        raise KeyError(idx)

    def capture(self) -> None:
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        torch.cuda.synchronize()

    def replay(self) -> None:
        self.graph.replay()
