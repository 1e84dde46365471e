// fp_prefill.h - ragged prefill attention (lanes with more rows x GQA heads than one MFMA N block).
//
// One workgroup of eight waves per (lane, KV head, block of 256/G rows): wave w
// owns query head g*G + w%G for 32 rows of the block, so every K/V tile the
// workgroup stages in LDS feeds all G query heads of the KV head (GQA sharing).
// Tiles of 32 slots are read from HBM once per workgroup into a four-stage
// LDS ring laid out so the MFMA fragment reads are free of bank conflicts:
//   K   [32 slots][D]   rows padded by 16 bytes
//   V^T [D][32 slots]   rows padded by 16 bytes
// (the padding staggers the rows a quarter-wave reads across all LDS banks, and
// keeps every fragment of a lane at a constant offset from one base address).
// Scores use S^T = K * Q^T and O^T += V^T * P^T on v_mfma_f32_32x32x16_bf16
// (the same register mapping as the 32-column decode path), with the online
// softmax rescaling O only when a column's running max grows by more than 2^8.
//
// The tile loop is unrolled by the ring depth, so every LDS stage address is a
// constant, and it is specialised for the two kinds of lane: causal lanes walk
// tiles 0..T-1 and mask only the tiles that cross a row's causal limit; masked
// lanes walk the row block's tile list (written by summary_kernel: the tiles
// with any allowed slot, tagged when all slots are allowed) and carry each
// row's mask word through LDS with the tile.
#pragma once

#include <type_traits>

#include "fp_kernels.h"

namespace fpk {

constexpr int kPreWaves = 8;
constexpr int kPreThreads = 64 * kPreWaves;
constexpr int kPreStages = 4;          // LDS ring depth (the loop is unrolled by the same count)
constexpr float kRescaleSlack = 8.0f;  // log2 units: p stays below 2^8 between rescales

template <int D>
struct PreLds {
    static constexpr int KC = D / 8;              // 16-byte chunks per K row
    static constexpr int KROW = D * 2 + 16;       // padded K row (bytes)
    static constexpr int VROW = 32 * 2 + 16;      // padded V^T row (bytes)
    static constexpr int K_BYTES = 32 * KROW;
    static constexpr int V_BYTES = D * VROW;
    static constexpr int MW_OFF = K_BYTES + V_BYTES;  // mask words of the block's rows (masked lanes)
    static constexpr int STAGE = MW_OFF + 4 * 256;
};

// What this thread brings in for one tile: a 16-byte K chunk and V^T chunk and,
// on masked lanes, the mask word of its own query row, all for the shared LDS
// stage (the word goes through LDS too, so no loaded value outlives its ring slot).
struct PreStage {
    uint4 k, v;
    uint32_t mw;
};

// Physical pages of the K and V^T chunks this thread moves for one tile (loaded
// one pipeline step before the data, so waiting for them never waits for the
// data loads still in flight behind them).
struct PrePages {
    int k, v;
};

// Per-thread constants of the tile copy. A tile is 32 slots and a page holds
// P in {8, 16, 32} slots, so a tile starts on a page boundary and the chunk a
// thread moves sits at the same offset inside the same page of every tile:
// only the page id changes from tile to tile.
template <int D>
struct PreCopy {
    const char *kp, *vp;  // chunk address inside physical page 0
    uint32_t pbytes;      // bytes per physical page
    int last_page;        // highest physical page id in the pool
    int kpg, vpg;         // page of the chunk within the tile's pages
    int tshift;           // log2(pages per tile)
    int lastpg;           // last working-set page holding a slot below kv_len
    int k_lds, v_lds;     // LDS byte offsets of the chunk in a stage
    int mw_lds;           // LDS byte offset of the row's mask word
    int ts;               // the tile holding slot kv_len (its tail slots are not part of the sequence)
    uint32_t vmk[4];      // V^T chunk mask for tile ts: the words of slots below kv_len
};

template <int D>
__device__ __forceinline__ PreCopy<D> pre_copy(const KvView &kv, int rloc) {
    constexpr int KC = PreLds<D>::KC;
    const int tid = threadIdx.x;
    PreCopy<D> c;
    const int rk = (tid % (32 * KC)) / KC, ck = tid % KC;          // K: slot rk, 16-byte chunk ck
    const int dv = (tid % (4 * D)) >> 2, cv = tid & 3;             // V^T: row dv, slots 8cv..8cv+7
    const char *base = reinterpret_cast<const char *>(kv.kbase);
    c.kp = base + 2 * (((int64_t)kv.g * kv.P + (rk & kv.pmask)) * D + 8 * ck);
    c.vp = base + 2 * (kv.vblock + (int64_t)kv.g * D * kv.P + (int64_t)dv * kv.P + ((8 * cv) & kv.pmask));
    c.pbytes = (uint32_t)(2 * kv.page_elems);
    c.last_page = kv.last_page;
    c.kpg = rk >> kv.pshift;
    c.vpg = (8 * cv) >> kv.pshift;
    c.tshift = 5 - kv.pshift;
    c.lastpg = kv.eff > 0 ? (kv.eff - 1) >> kv.pshift : 0;
    c.k_lds = rk * PreLds<D>::KROW + 16 * ck;
    c.v_lds = PreLds<D>::K_BYTES + dv * PreLds<D>::VROW + 16 * cv;
    c.mw_lds = PreLds<D>::MW_OFF + 4 * rloc;
    c.ts = kv.eff >> 5;
    const int nv = (kv.eff & 31) - 8 * cv;  // valid slots of the V^T chunk in tile ts
#pragma unroll
    for (int q = 0; q < 4; ++q) c.vmk[q] = nv >= 2 * q + 2 ? 0xFFFFFFFFu : (nv >= 2 * q + 1 ? 0x0000FFFFu : 0u);
    return c;
}

template <int D>
__device__ __forceinline__ void pre_pages(const KvView &kv, const PreCopy<D> &c, int t, PrePages &pp) {
    const int base = t << c.tshift;
    pp.k = kv.pids[min(base + c.kpg, c.lastpg)];
    pp.v = kv.pids[min(base + c.vpg, c.lastpg)];
}

// Every load here is unconditional and nothing is done to the loaded values
// until they are stored to LDS two steps later, so the compiler can count
// outstanding loads exactly and wait for one tile's data without draining
// later prefetches. K of slots at or past kv_len is never zeroed: those slots
// only occur in tiles whose scores go through the per-slot select, which drops them.
template <int D, bool MASKED>
__device__ __forceinline__ void pre_data(const PreCopy<D> &c, int t, const PrePages &pp, PreStage &st,
                                         const uint32_t *mrow, int wpr) {
    if constexpr (MASKED) st.mw = mrow[t < wpr ? t : 0];
    const uint32_t pk = (uint32_t)min(max(pp.k, 0), c.last_page);
    const uint32_t pv = (uint32_t)min(max(pp.v, 0), c.last_page);
    st.k = *reinterpret_cast<const uint4 *>(c.kp + (uint64_t)pk * c.pbytes);
    st.v = *reinterpret_cast<const uint4 *>(c.vp + (uint64_t)pv * c.pbytes);
}

// Stores tile t's chunks into an LDS stage. V^T entries of slots at or past
// kv_len are zeroed (p = 0 times a stale NaN would still be NaN); only tile ts
// has such entries. Every thread stores: with fewer chunks than threads (head
// dim 64) two threads write the same bytes, and all lanes of a row write the
// same mask word, so no store needs a lane condition.
template <int D, bool MASKED>
__device__ __forceinline__ void pre_store(const PreCopy<D> &c, const PreStage &st, char *stage, int t) {
    *reinterpret_cast<uint4 *>(stage + c.k_lds) = st.k;
    uint4 v = st.v;
    if (t == c.ts) v = make_uint4(v.x & c.vmk[0], v.y & c.vmk[1], v.z & c.vmk[2], v.w & c.vmk[3]);  // uniform
    *reinterpret_cast<uint4 *>(stage + c.v_lds) = v;
    if constexpr (MASKED) *reinterpret_cast<uint32_t *>(stage + c.mw_lds) = st.mw;
}

template <int D>
struct PreWave {
    uint4 qf[D / 16];
    f32x16 o[D / 32];
    float m, l;
};

// S^T = K * Q^T for the staged tile: the eight K fragments of a lane sit at
// constant offsets from one address, read first, then one accumulator chain.
template <int D>
__device__ __forceinline__ f32x16 pre_qk(const char *stage, const PreWave<D> &w) {
    const int ln = lane_id(), h = ln >> 5, n = ln & 31;
    const char *krow = stage + kslot_of_row(n) * PreLds<D>::KROW + h * D;
    uint4 kf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const uint4 *>(krow + 16 * s);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc = mfma32(kf[s], w.qf[s], acc);
    return acc;
}

// Softmax prologue of one tile: drop the slots a column may not see (unless
// the whole tile is allowed), take the column max over both lane halves and
// rescale O and l when it grew by more than 2^kRescaleSlack. The running max
// starts at -FLT_MAX, not -inf, so p = exp2(s - m) needs no special case for a
// column that has seen no valid slot yet (a dropped score is -inf, p = 0).
template <int D>
__device__ __forceinline__ void pre_prologue(f32x16 &s, bool full, uint32_t vbits, PreWave<D> &w) {
    const int h = lane_id() >> 5;
    if (!full) {
        const uint32_t vb = vbits >> (8 * h);  // register i holds tile slot 16(i/8) + 8h + i%8
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = 16 * (i >> 3) + (i & 7);
            const uint32_t keep = (uint32_t)((int32_t)(vb << (31 - k)) >> 31);  // all ones if allowed
            s[i] = __uint_as_float((__float_as_uint(s[i]) & keep) | (0xFF800000u & ~keep));
        }
    }
    float mt = fmaxf(s[0], s[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mt = fmaxf(fmaxf(mt, s[i]), s[i + 1]);
    {
        // the two lane halves hold the two halves of the column's 32 slots
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const bool grow = mt > w.m + kRescaleSlack;
    if (__any(grow)) {
        const float m_new = grow ? mt : w.m;
        const float alpha = __builtin_amdgcn_exp2f(w.m - m_new);
        w.l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] *= alpha;
        w.m = m_new;
    }
}

// Main block of one pipeline step, free of branches and cut into segments
// the scheduler keeps in order (it reorders only inside one): after the K and
// V^T fragment reads, each segment issues one MFMA of the next tile's QK^T
// chain together with the exp2 / bf16 packing of two weights of the current
// tile, so the VALU work runs while the dependent MFMA chain waits on itself;
// the P*V MFMAs of the first weight half join the chain's later segments, and
// the second half shares its segments with the tile copy (list entry and page
// ids, LDS store, prefetch loads: copy(k) is called for k = 0, 1, 2). The
// denominator sums the same bf16 weights the numerator uses.
template <int D, class Copy>
__device__ __forceinline__ void pre_main(const char *stc, const char *stn, const f32x16 &sc, f32x16 &sn,
                                         PreWave<D> &w, Copy &&copy) {
    constexpr int NQK = D / 16;          // QK^T MFMAs of the chain
    constexpr int NDB = D / 32;          // 32-row blocks of O^T
    constexpr int PPS = 8 / NQK;         // weight pairs packed per chain segment
    static_assert(NQK >= 2 * NDB && 8 % NQK == 0, "segment plan");
    const int ln = lane_id(), h = ln >> 5, n = ln & 31;
    const char *krow = stn + kslot_of_row(n) * PreLds<D>::KROW + h * D;
    const char *vrow = stc + PreLds<D>::K_BYTES + n * PreLds<D>::VROW + 16 * h;
    uint4 kf[NQK], vf[NDB][2];
#pragma unroll
    for (int s = 0; s < NQK; ++s) kf[s] = *reinterpret_cast<const uint4 *>(krow + 16 * s);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        vf[db][0] = *reinterpret_cast<const uint4 *>(vrow + 32 * db * PreLds<D>::VROW);
        vf[db][1] = *reinterpret_cast<const uint4 *>(vrow + 32 * db * PreLds<D>::VROW + 32);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pk[8];
    f32x16 acc = {};
    uint4 pb0 = {};
#pragma unroll
    for (int s = 0; s < NQK; ++s) {
        acc = mfma32(kf[s], w.qf[s], acc);
#pragma unroll
        for (int u = 0; u < PPS; ++u) {
            const int q = s * PPS + u;
            pk[q] = pack_bf16x2(__builtin_amdgcn_exp2f(sc[2 * q] - w.m), __builtin_amdgcn_exp2f(sc[2 * q + 1] - w.m));
        }
        if (s == NQK - NDB - 1) pb0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        if (s >= NQK - NDB) {
            const int db = s - (NQK - NDB);
            w.o[db] = mfma32(vf[db][0], pb0, w.o[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    sn = acc;
    const uint4 pb1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        w.o[db] = mfma32(vf[db][1], pb1, w.o[db]);
#pragma unroll
        for (int q = db * (8 / NDB); q < (db + 1) * (8 / NDB); ++q)
            w.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[q]),
                                                  __builtin_bit_cast(bf16x2, 0x3F803F80u), w.l, false);
        if (db < 3) copy(db);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NDB < 3) {
#pragma unroll
        for (int k = NDB; k < 3; ++k) copy(k);
    }
}

// Allowed slots of tile j0 for this lane's column as a 32-bit mask.
__device__ __forceinline__ uint32_t tile_bits(int j0, int lim, bool masked, uint32_t mw) {
    const int rem = lim - j0;
    const uint32_t lm = rem >= 32 ? 0xFFFFFFFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
    return masked ? (mw & lm) : lm;
}

// Keeps an index in a vector register, so a load through it is a vector
// memory load (ordered with the tile loads) rather than a scalar one.
__device__ __forceinline__ int in_vgpr(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int K>
using StepK = std::integral_constant<int, K>;

// Prefill body for one work item; MASKED selects the masked-lane walk.
template <int D, int G, bool MASKED>
__device__ __forceinline__ void prefill_item(const AttnArgs &a, int4 it, char (*s_tile)[PreLds<D>::STAGE],
                                             int *s_lmax) {
    const int lane = it.x, g = it.y, rstart = it.z, nr = it.w;
    const int wv = threadIdx.x / kWave;
    const int ln = lane_id(), n = ln & 31, h = ln >> 5;
    const int rsub = wv / G;
    const int head = g * G + (wv % G);
    const int rloc = 32 * rsub + n;                 // row within the item
    const bool colv = rloc < nr;
    const int r0 = a.indptr[lane];
    const int nrows = a.indptr[lane + 1] - r0;
    const int64_t row = r0 + rstart + (colv ? rloc : 0);
    int cap;
    KvView kv = make_view(a, lane, g, &cap);
    kv.vblock = (int64_t)a.H * a.P * D;

    PreWave<D> w;
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.qrot + (row * a.Hq + head) * D + h * (D / 2));
#pragma unroll
        for (int s = 0; s < D / 16; ++s) w.qf[s] = colv ? src[s] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] = f32x16{};
        w.m = -__FLT_MAX__;
        w.l = 0.0f;
    }
    // Mask-word pointers are always valid so their loads need no branch.
    const uint32_t *mrow = reinterpret_cast<const uint32_t *>(a.indptr);
    int wpr = 1;
    const int32_t *lst = nullptr;  // masked lanes: [count, entries...] of this row block
    int T;                         // tiles this workgroup visits
    if constexpr (MASKED) {
        wpr = (int)((a.mask_off[lane + 1] - a.mask_off[lane]) / nrows);
        mrow = a.mask_bits + a.mask_off[lane] + (int64_t)(rstart + (colv ? rloc : 0)) * wpr;
        const LaneInfo li = a.lane_info[lane];
        lst = a.summary + li.sum_off + (int64_t)(rstart / prefill_rows(G)) * li.sum_stride;
        T = li.sum_off >= 0 ? __builtin_amdgcn_readfirstlane(lst[0]) : 0;
    }
    const int lim = !colv ? 0 : (MASKED ? kv.eff : min(a.slots[row] + 1, kv.eff));
    const int lmin_w = __builtin_amdgcn_readfirstlane(-wave_max_i(colv ? -lim : -0x7FFFFFFF));  // valid columns
    // Let the Q loads land before the pipeline starts: otherwise the first use
    // of Q inside the loop carries a wait for every load in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if constexpr (!MASKED) {
        const int lmax_w = __builtin_amdgcn_readfirstlane(wave_max_i(lim));
        if (ln == 0) s_lmax[wv] = lmax_w;
        __syncthreads();
        int lwg = 0;
#pragma unroll
        for (int v = 0; v < kPreWaves; ++v) lwg = max(lwg, s_lmax[v]);
        T = (__builtin_amdgcn_readfirstlane(lwg) + 31) >> 5;
    }

    if (T > 0) {  // workgroup-uniform
        // Software pipeline over the tile sequence; at step i: the softmax and
        // P*V of tile i run while the QK^T MFMAs of tile i+1 are issued (its K
        // sits in the next LDS stage), tile i+2 moves from registers to LDS,
        // tiles i+3 and i+4 are in flight from HBM, and the page ids of tile
        // i+5 are read. Tile j lives in LDS stage j % 4. Steps past the end of
        // the sequence repeat its last tile, so every load is unconditional;
        // tiles past a wave's last row (the end of the causal diagonal) are
        // computed like the others with every slot dropped.
        const PreCopy<D> cp = pre_copy<D>(kv, rloc);
        // masked lanes: list entries of steps i..i+5, and the load of step i+6
        int q0 = 0, q1 = 0, q2 = 0, q3 = 0, q4 = 0, q5 = 0, lv = 0;
        auto entry = [&](int i) { return lst[1 + min(i, T - 1)]; };
        auto tile_at = [&](int i, int qe) {  // tile of step i
            if constexpr (MASKED) return qe & 0x7FFFFFFF;
            else return min(i, T - 1);
        };
        if constexpr (MASKED) {
            q0 = __builtin_amdgcn_readfirstlane(entry(0));
            q1 = __builtin_amdgcn_readfirstlane(entry(1));
            q2 = __builtin_amdgcn_readfirstlane(entry(2));
            q3 = __builtin_amdgcn_readfirstlane(entry(3));
            q4 = __builtin_amdgcn_readfirstlane(entry(4));
            q5 = __builtin_amdgcn_readfirstlane(entry(5));
            lv = lst[in_vgpr(1 + min(6, T - 1))];
        }
        PreStage ringA, ringB;
        PrePages pgA, pgB;
        pre_pages<D>(kv, cp, tile_at(0, q0), pgA);
        pre_pages<D>(kv, cp, tile_at(1, q1), pgB);
        pre_data<D, MASKED>(cp, tile_at(0, q0), pgA, ringA, mrow, wpr);
        pre_data<D, MASKED>(cp, tile_at(1, q1), pgB, ringB, mrow, wpr);
        pre_pages<D>(kv, cp, tile_at(2, q2), pgA);
        pre_pages<D>(kv, cp, tile_at(3, q3), pgB);
        pre_store<D, MASKED>(cp, ringA, s_tile[0], tile_at(0, q0));
        pre_store<D, MASKED>(cp, ringB, s_tile[1], tile_at(1, q1));
        pre_data<D, MASKED>(cp, tile_at(2, q2), pgA, ringA, mrow, wpr);
        pre_data<D, MASKED>(cp, tile_at(3, q3), pgB, ringB, mrow, wpr);
        pre_pages<D>(kv, cp, tile_at(4, q4), pgA);
        __syncthreads();

        f32x16 sA = pre_qk<D>(s_tile[0], w), sB = {};
        auto step = [&](auto kc, int i) {
            constexpr int K = decltype(kc)::value;
            char *stc = s_tile[K];
            char *stn = s_tile[(K + 1) % kPreStages];
            char *sts = s_tile[(K + 2) % kPreStages];
            f32x16 &sc = (K & 1) ? sB : sA;
            f32x16 &sn = (K & 1) ? sA : sB;
            PreStage &ring = (K & 1) ? ringB : ringA;
            PrePages &pgc = (K & 1) ? pgB : pgA;  // page ids of tile i+4 (read one step ago)
            PrePages &pgn = (K & 1) ? pgA : pgB;  // receives the page ids of tile i+5
            int q6 = 0;
            if constexpr (MASKED) q6 = __builtin_amdgcn_readfirstlane(lv);
            const int tc = tile_at(i, q0), t2 = tile_at(i + 2, q2), t4 = tile_at(i + 4, q4),
                      t5 = tile_at(i + 5, q5);
            {
                const int j0 = 32 * tc;
                bool full;
                uint32_t bits = 0u;
                if constexpr (MASKED) {
                    full = q0 < 0 && j0 + 32 <= kv.eff;  // bit 31: every slot allowed for every row
                    if (!full) bits = tile_bits(j0, lim, true, *reinterpret_cast<const uint32_t *>(stc + cp.mw_lds));
                } else {
                    full = j0 + 32 <= lmin_w;
                    if (!full) bits = tile_bits(j0, lim, false, 0u);
                }
                pre_prologue<D>(sc, full, bits, w);
            }
            pre_main<D>(stc, stn, sc, sn, w, [&](int k) {
                if (k == 0) {
                    // list entry and page ids first: the data loads then wait
                    // only on loads issued one step earlier, never the newest
                    if constexpr (MASKED) lv = lst[in_vgpr(1 + min(i + 7, T - 1))];
                    pre_pages<D>(kv, cp, t5, pgn);
                }
                if (k == 1) pre_store<D, MASKED>(cp, ring, sts, t2);
                if (k == 2) pre_data<D, MASKED>(cp, t4, pgc, ring, mrow, wpr);
            });
            __syncthreads();
            if constexpr (MASKED) {
                q0 = q1;
                q1 = q2;
                q2 = q3;
                q3 = q4;
                q4 = q5;
                q5 = q6;
            }
        };
        for (int i = 0;; i += kPreStages) {
            step(StepK<0>{}, i);
            if (i + 1 >= T) break;
            step(StepK<1>{}, i + 1);
            if (i + 2 >= T) break;
            step(StepK<2>{}, i + 2);
            if (i + 3 >= T) break;
            step(StepK<3>{}, i + 3);
            if (i + 4 >= T) break;
        }
    }

    if (!colv) return;
    const float l_tot = w.l + __shfl_xor(w.l, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float *orow = a.out + (row * a.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<float4 *>(orow + 32 * db + 8 * i4 + 4 * h) =
                make_float4(w.o[db][4 * i4] * inv, w.o[db][4 * i4 + 1] * inv, w.o[db][4 * i4 + 2] * inv,
                            w.o[db][4 * i4 + 3] * inv);
    if (a.lse && h == 0)
        a.lse[row * a.Hq + head] = l_tot > 0.0f ? (w.m + __log2f(l_tot)) * 0.69314718055994531f : kNegInf;
}

// Prefill: one workgroup of eight waves per (lane, KV head, block of 256/G
// rows); wave w owns query head g*G + w%G for the 32 rows at 32*(w/G).
template <int D, int G>
__global__ void __launch_bounds__(kPreThreads) prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char s_tile[kPreStages][PreLds<D>::STAGE];
    __shared__ int s_lmax[kPreWaves];
    const int4 it = a.pre_items[blockIdx.x];
    if (it.x < 0) return;
    const bool masked = a.mask_off && a.mask_off[it.x + 1] > a.mask_off[it.x];  // workgroup-uniform
    if (masked) prefill_item<D, G, true>(a, it, s_tile, s_lmax);
    else prefill_item<D, G, false>(a, it, s_tile, s_lmax);
}

}  // namespace fpk
