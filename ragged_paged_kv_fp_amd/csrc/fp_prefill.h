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
constexpr float kNoSlot = -0x1p100f;   // a tile max below this: the column may read no slot of the tile
constexpr uint32_t kBiasOut = 0xFE80FE80u;  // two bf16 -2^126: the bias of a slot a row may not read

template <int D>
struct PreLds {
    static constexpr int KC = D / 8;              // 16-byte chunks per K row
    static constexpr int KROW = D * 2 + 16;       // padded K row (bytes)
    static constexpr int VROW = 32 * 2 + 16;      // padded V^T row (bytes)
    static constexpr int K_BYTES = 32 * KROW;
    static constexpr int V_BYTES = D * VROW;
    static constexpr int MW_OFF = K_BYTES + V_BYTES;  // mask words of the block's rows (masked lanes)
    static constexpr int STAGE = MW_OFF + 4 * 256;
    // the keep-mask table sits at the start of LDS, so a lane's table address
    // is 8 x the mask nibble with no base added
    static constexpr int LUT_OFF = 0;                   // [16][2] uint32: bf16 keep masks of a mask nibble
    static constexpr int AOP_OFF = LUT_OFF + 16 * 8;     // [2][64] uint4: A operands of the bias MFMAs
    static constexpr int RING_OFF = AOP_OFF + 2 * 64 * 16;
    static constexpr int TOTAL = RING_OFF + kPreStages * STAGE;
};

// What this thread brings in for one tile: a 16-byte K chunk and V^T chunk and,
// on masked lanes, the mask word of its own query row, all for the shared LDS
// stage (the word goes through LDS too, so no loaded value outlives its ring slot).
struct PreStage {
    uint4 k, v;
    uint32_t mw;
};

// Keeps an index in a vector register, so a load through it is a vector
// memory load (ordered with the tile loads) rather than a scalar one.
__device__ __forceinline__ int in_vgpr(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Physical pages of the K and V^T chunks a wave moves for one tile (loaded
// one pipeline step before the data, so waiting for them never waits for the
// data loads still in flight behind them). Each is one wave-uniform id, held
// in a vector register only while its load is in flight.
struct PrePages {
    int k, v;
};

// Per-thread constants of the tile copy. A tile is 32 slots and a page holds
// P in {8, 16, 32} slots, so a tile starts on a page boundary and the chunk a
// thread moves sits at the same offset inside the same page of every tile:
// only the page id changes from tile to tile. The chunks are dealt out so that
// all 64 chunks of a wave lie in one page: K by slot (a wave holds 64/KC
// consecutive slots, at most 8), V^T page by page (a page's D x P block is D*P/8
// >= 64 chunks, chunk e holding row e / (P/8), slots 8 (e % (P/8)) .. + 7). The
// address of a chunk is then a wave-uniform page base plus a per-thread 32-bit
// offset, and only the base is recomputed per tile, in scalar registers.
template <int D>
struct PreCopy {
    const char *base;     // pool
    uint32_t koff, voff;  // byte offsets of the thread's chunks inside a physical page
    uint32_t pbytes;      // bytes per physical page
    int last_page;        // highest physical page id in the pool
    int kpg, vpg;         // page of the wave's chunks within the tile's pages (wave-uniform)
    int tshift;           // log2(pages per tile)
    int lastpg;           // last working-set page holding a slot below kv_len
    int k_lds, v_lds;     // LDS byte offsets of the chunks in a stage
    int mw_lds;           // LDS byte offset of the row's mask word
    int ts;               // the tile holding slot kv_len (its tail slots are not part of the sequence)
    int vnv;              // slots of this thread's V^T chunk below kv_len in tile ts
};

template <int D>
__device__ __forceinline__ PreCopy<D> pre_copy(const KvView &kv, int rloc) {
    constexpr int KC = PreLds<D>::KC;
    const int tid = threadIdx.x;
    PreCopy<D> c;
    const int rk = (tid % (32 * KC)) / KC, ck = tid % KC;  // K: slot rk, 16-byte chunk ck
    const int cvi = tid % (4 * D);                         // V^T chunk of the tile
    const int vsh = kv.pshift - 3;                         // log2(chunks per V^T row of a page)
    const int pgv = cvi >> (__builtin_ctz(D) + vsh);       // page of the chunk within the tile
    const int e = cvi & ((D << vsh) - 1);
    const int dv = e >> vsh, slot0 = pgv * kv.P + 8 * (e & ((1 << vsh) - 1));
    c.base = reinterpret_cast<const char *>(kv.kbase);
    c.koff = (uint32_t)(2 * (((int64_t)kv.g * kv.P + (rk & kv.pmask)) * D + 8 * ck));
    c.voff = (uint32_t)(2 * (kv.vblock + (int64_t)kv.g * D * kv.P + (int64_t)dv * kv.P + (slot0 & kv.pmask)));
    c.pbytes = (uint32_t)(2 * kv.page_elems);
    c.last_page = kv.last_page;
    c.kpg = __builtin_amdgcn_readfirstlane(rk >> kv.pshift);
    c.vpg = __builtin_amdgcn_readfirstlane(pgv);
    c.tshift = 5 - kv.pshift;
    c.lastpg = kv.eff > 0 ? (kv.eff - 1) >> kv.pshift : 0;
    c.k_lds = rk * PreLds<D>::KROW + 16 * ck;
    c.v_lds = PreLds<D>::K_BYTES + dv * PreLds<D>::VROW + 2 * slot0;
    c.mw_lds = PreLds<D>::MW_OFF + 4 * rloc;
    c.ts = kv.eff >> 5;
    c.vnv = (kv.eff & 31) - slot0;
    return c;
}

template <int D>
__device__ __forceinline__ void pre_pages(const KvView &kv, const PreCopy<D> &c, int t, PrePages &pp) {
    const int base = t << c.tshift;
    pp.k = kv.pids[in_vgpr(min(base + c.kpg, c.lastpg))];
    pp.v = kv.pids[in_vgpr(min(base + c.vpg, c.lastpg))];
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
    const uint32_t pk = (uint32_t)min(max(__builtin_amdgcn_readfirstlane(pp.k), 0), c.last_page);
    const uint32_t pv = (uint32_t)min(max(__builtin_amdgcn_readfirstlane(pp.v), 0), c.last_page);
    st.k = *reinterpret_cast<const uint4 *>(c.base + (uint64_t)pk * c.pbytes + c.koff);
    st.v = *reinterpret_cast<const uint4 *>(c.base + (uint64_t)pv * c.pbytes + c.voff);
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
    if (t == c.ts) {  // workgroup-uniform: keep the chunk's slots below kv_len
        uint32_t mk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) mk[q] = c.vnv >= 2 * q + 2 ? 0xFFFFFFFFu : (c.vnv >= 2 * q + 1 ? 0x0000FFFFu : 0u);
        v = make_uint4(v.x & mk[0], v.y & mk[1], v.z & mk[2], v.w & mk[3]);
    }
    *reinterpret_cast<uint4 *>(stage + c.v_lds) = v;
    if constexpr (MASKED) *reinterpret_cast<uint32_t *>(stage + c.mw_lds) = st.mw;
}

template <int D>
struct PreWave {
    uint4 qf[D / 16];
    f32x16 o[D / 32];
    float m, l;      // running max (log2 units, always a bf16 value) and denominator
    uint32_t negm2;  // -m as two bf16 halves (exact: m is bf16-representable), the bias operand
    bool seen;       // the column has had an allowed slot
};

__device__ __forceinline__ float bf16_round(float x) { return __uint_as_float(pack_bf16x2(x, x) << 16); }

__device__ __forceinline__ uint32_t neg_m2(float m) {
    const uint32_t hb = __float_as_uint(-m) >> 16;
    return hb | (hb << 16);
}

// The score shift and the mask enter the QK^T accumulation as extra MFMAs,
// so the softmax needs neither a subtraction nor a per-slot select:
//  * RowBias (causal lanes): one rank-1 MFMA, A[m][k] = (k == 0), B[0][n] = -m_n,
//    adds -m to every slot of the column.
//  * MaskBias (masked lanes): two MFMAs over the 32 tile slots whose A operand
//    is the slot permutation of the score rows (row m holds slot
//    kslot_of_row(m), so A[m][k] = (kslot_of_row(m) == k)) and whose B operand
//    holds -m for a slot the row may read and -2^126 for one it may not. The
//    B operand is built from the row's mask bytes, a nibble at a time,
//    through a 16-entry table of bf16 keep masks in LDS (128 bytes: the
//    entries sit in distinct banks, so the lanes' lookups never conflict).
// A score the row may not read then sits near -2^126 and its weight is 0; the
// column max of a tile therefore covers allowed slots only. Slots at or past
// kv_len can hold stale K (even NaN), so the one tile that crosses kv_len
// still drops them with a select.
struct RowBias {
    static constexpr int kDone = 0;  // tail segment after which the scores are complete
    uint32_t a0, negm2;
    __device__ __forceinline__ void fetch() {}
    __device__ __forceinline__ void load(int) {}
    __device__ __forceinline__ void build() {}
    __device__ __forceinline__ f32x16 apply(f32x16 acc, int k) const {
        return k == 0 ? mfma32(make_uint4(a0, 0u, 0u, 0u), make_uint4(negm2, 0u, 0u, 0u), acc) : acc;
    }
};

// The two MFMAs of MaskBias run one after the other through one operand set
// (load(k), build(), apply(acc, k)), which keeps eight registers free.
struct MaskBias {
    static constexpr int kDone = 1;  // tail segment after which the scores are complete
    const char *lut;     // the keep-mask table (LDS)
    const char *aop;     // the A operands (LDS)
    const uint32_t *mw;  // the row's mask word for the tile (LDS)
    uint32_t lm;         // slots of the tile below kv_len (wave-uniform)
    uint32_t fullm;      // all ones when every row may read every slot of the tile (wave-uniform)
    uint32_t bits;       // slots of the tile the lane's row may read
    uint32_t negm2;
    uint4 a, b;
    // issued together with the tile's fragment reads, consumed by load(0)
    __device__ __forceinline__ void fetch() { bits = *mw; }
    __device__ __forceinline__ void load(int k) {
        const int ln = lane_id(), kg = ln >> 5;
        // B lane (n, kg) of MFMA k holds slots 16k + 8kg .. 16k + 8kg + 7: after
        // the shift by 8kg they are bits 16k .. 16k + 7
        if (k == 0) bits = ((bits & lm) | fullm) >> (8 * kg);
        const uint2 lo = *reinterpret_cast<const uint2 *>(lut + 8 * ((bits >> (16 * k)) & 15u));
        const uint2 hi = *reinterpret_cast<const uint2 *>(lut + 8 * ((bits >> (16 * k + 4)) & 15u));
        b = make_uint4(lo.x, lo.y, hi.x, hi.y);
        a = *reinterpret_cast<const uint4 *>(aop + 1024 * k + 16 * ln);
    }
    __device__ __forceinline__ void build() { b = make_uint4(bfi(b.x), bfi(b.y), bfi(b.z), bfi(b.w)); }
    __device__ __forceinline__ uint32_t bfi(uint32_t keep) const { return (keep & negm2) | (~keep & kBiasOut); }
    __device__ __forceinline__ f32x16 apply(f32x16 acc, int) const { return mfma32(a, b, acc); }
};

// Fills the keep-mask table (entry e, a nibble: word q keeps bf16 half 0 if
// bit 2q of e is set and half 1 if bit 2q+1 is) and the A operands of MaskBias.
template <int D>
__device__ __forceinline__ void fill_bias_tables(char *lds) {
    for (int wi = threadIdx.x; wi < 16 * 2; wi += kPreThreads) {
        const int e = wi >> 1, q = wi & 1;
        const uint32_t v = (((e >> (2 * q)) & 1) ? 0x0000FFFFu : 0u) | (((e >> (2 * q + 1)) & 1) ? 0xFFFF0000u : 0u);
        reinterpret_cast<uint32_t *>(lds + PreLds<D>::LUT_OFF)[wi] = v;
    }
    for (int t = threadIdx.x; t < 2 * 64; t += kPreThreads) {
        const int which = t >> 6, ln = t & 63, m = ln & 31, kg = ln >> 5;
        const int j = kslot_of_row(m) - 16 * which - 8 * kg;  // position of the 1 in this lane's 8 k's
        uint32_t r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = (j == 2 * q ? 0x00003F80u : 0u) | (j == 2 * q + 1 ? 0x3F800000u : 0u);
        reinterpret_cast<uint4 *>(lds + PreLds<D>::AOP_OFF)[t] = make_uint4(r[0], r[1], r[2], r[3]);
    }
}

// S^T = K * Q^T (+ bias) for the staged tile: the K fragments of a lane sit at
// constant offsets from one address, read first, then one accumulator chain.
template <int D, class Bias>
__device__ __forceinline__ f32x16 pre_qk(const char *stage, const PreWave<D> &w, Bias &bias) {
    const int ln = lane_id(), h = ln >> 5, n = ln & 31;
    const char *krow = stage + kslot_of_row(n) * PreLds<D>::KROW + h * D;
    uint4 kf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const uint4 *>(krow + 16 * s);
    bias.fetch();
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc = mfma32(kf[s], w.qf[s], acc);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        bias.load(k);
        bias.build();
        acc = bias.apply(acc, k);
    }
    return acc;
}

// Softmax prologue of one tile, in two parts. pre_max: the scores arrive as
// s - m (the shift was added by the bias MFMA); with sel, slots outside vbits
// are first set to -inf; returns the column max over both lane halves.
// pre_rescale: the running max moves (rounded to bf16, so -m stays exact in
// the next bias) the first time the column sees an allowed slot and whenever
// the max grows by more than 2^kRescaleSlack, rescaling O and l and
// re-shifting the scores. It must follow every P*V and denominator update of
// the previous tile.
__device__ __forceinline__ float pre_max(f32x16 &s, bool sel, uint32_t vbits) {
    const int h = lane_id() >> 5;
    if (sel) {
        const uint32_t vb = vbits >> (8 * h);  // register i holds tile slot 16(i/8) + 8h + i%8
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = 16 * (i >> 3) + (i & 7);
            const uint32_t keep = (uint32_t)((int32_t)(vb << (31 - k)) >> 31);  // all ones if allowed
            s[i] = __uint_as_float((__float_as_uint(s[i]) & keep) | (0xFF800000u & ~keep));
        }
    }
    // a tree of three-input maxima keeps the dependent chain short
    auto mx3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
    float mt = fmaxf(mx3(mx3(s[0], s[1], s[2]), mx3(s[3], s[4], s[5]), mx3(s[6], s[7], s[8])),
                     mx3(mx3(s[9], s[10], s[11]), mx3(s[12], s[13], s[14]), s[15]));
    // the two lane halves hold the two halves of the column's 32 slots
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

template <int D>
__device__ __forceinline__ void pre_rescale(f32x16 &s, float mt, PreWave<D> &w) {
    const bool valid = mt > kNoSlot;
    const bool grow = valid && (!w.seen || mt > kRescaleSlack);
    if (__any(grow)) {
        const float m_new = grow ? bf16_round(w.m + mt) : w.m;
        const float delta = m_new - w.m;
        const float alpha = w.seen ? __builtin_amdgcn_exp2f(-delta) : 1.0f;
        w.l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] -= delta;
        w.m = m_new;
        w.negm2 = neg_m2(m_new);
        w.seen = w.seen || valid;
    }
}

// Main block of one pipeline step, free of branches and cut into segments
// the scheduler keeps in order (it reorders only inside one): after the K and
// first V^T fragment reads, each segment issues one MFMA of the next tile's QK^T
// chain together with the exp2 / bf16 packing of two weights of the current
// tile, so the VALU work runs while the dependent MFMA chain waits on itself;
// the P*V MFMAs of the first weight half join the chain's later segments, the
// bias MFMAs close the chain, and the second half of P*V shares its segments
// with the tile copy (list entry and page ids, LDS store, prefetch loads:
// copy(k) is called for k = 0, 1, 2). The denominator sums the same bf16
// weights the numerator uses.
template <int D, class Bias, class Copy, class Next>
__device__ __forceinline__ void pre_main(const char *stc, const char *stn, const f32x16 &sc, f32x16 &sn,
                                         PreWave<D> &w, Bias &bias, Copy &&copy, Next &&next) {
    constexpr int NQK = D / 16;          // QK^T MFMAs of the chain
    constexpr int NDB = D / 32;          // 32-row blocks of O^T
    constexpr int PPS = 8 / NQK;         // weight pairs packed per chain segment
    static_assert(NQK >= 2 * NDB && 8 % NQK == 0 && NDB >= 2, "segment plan");
    const int ln = lane_id(), h = ln >> 5, n = ln & 31;
    const char *krow = stn + kslot_of_row(n) * PreLds<D>::KROW + h * D;
    const char *vrow = stc + PreLds<D>::K_BYTES + n * PreLds<D>::VROW + 16 * h;
    uint4 kf[NQK], vf[NDB][2];
#pragma unroll
    for (int s = 0; s < NQK; ++s) kf[s] = *reinterpret_cast<const uint4 *>(krow + 16 * s);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vf[db][0] = *reinterpret_cast<const uint4 *>(vrow + 32 * db * PreLds<D>::VROW);
    bias.fetch();
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
            pk[q] = pack_bf16x2(__builtin_amdgcn_exp2f(sc[2 * q]), __builtin_amdgcn_exp2f(sc[2 * q + 1]));
        }
        if (s == NQK - NDB - 1) pb0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        if (s >= NQK - NDB) {
            const int db = s - (NQK - NDB);
            w.o[db] = mfma32(vf[db][0], pb0, w.o[db]);
        }
        if (s == NQK / 2) {
            // the second V^T half takes the registers of the K fragments the
            // chain has consumed by now
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                vf[db][1] = *reinterpret_cast<const uint4 *>(vrow + 32 * db * PreLds<D>::VROW + 32);
        }
        if (s == NQK - 1) bias.load(0);  // the K fragments are all consumed now
        __builtin_amdgcn_sched_barrier(0);
    }
    const uint4 pb1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        w.o[db] = mfma32(vf[db][1], pb1, w.o[db]);
        // the bias MFMAs close the chain with the first P*V of the tail (both
        // kinds of lane add -m last, so an all-allowed bitmap reproduces the
        // causal path bit for bit); then the next tile's scores are complete
        // and its max is taken here, the dependent VALU chain overlapping the
        // P*V MFMAs still in flight
        if (db == 0) {
            bias.build();
            acc = bias.apply(acc, 0);
            bias.load(1);
        }
        if (db == 1 && Bias::kDone >= 1) {
            bias.build();
            acc = bias.apply(acc, 1);
        }
        if (db == (Bias::kDone + 1 < NDB - 1 ? Bias::kDone + 1 : NDB - 1)) {
            sn = acc;
            next(0);
        }
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
    next(1);
}

// Allowed slots of tile j0 for this lane's column as a 32-bit mask.
__device__ __forceinline__ uint32_t tile_bits(int j0, int lim, bool masked, uint32_t mw) {
    const int rem = lim - j0;
    const uint32_t lm = rem >= 32 ? 0xFFFFFFFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
    return masked ? (mw & lm) : lm;
}

template <int K>
using StepK = std::integral_constant<int, K>;

// Prefill body for one work item; MASKED selects the masked-lane walk.
template <int D, int G, bool MASKED>
__device__ __forceinline__ void prefill_item(const AttnArgs &a, int4 it, char *lds, int *s_lmax) {
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
    auto stage = [&](int k) { return lds + PreLds<D>::RING_OFF + k * PreLds<D>::STAGE; };

    PreWave<D> w;
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.qrot + (row * a.Hq + head) * D + h * (D / 2));
#pragma unroll
        for (int s = 0; s < D / 16; ++s) w.qf[s] = colv ? src[s] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] = f32x16{};
        w.m = 0.0f;
        w.negm2 = neg_m2(0.0f);
        w.l = 0.0f;
        w.seen = false;
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
        fill_bias_tables<D>(lds);
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
        pre_store<D, MASKED>(cp, ringA, stage(0), tile_at(0, q0));
        pre_store<D, MASKED>(cp, ringB, stage(1), tile_at(1, q1));
        pre_data<D, MASKED>(cp, tile_at(2, q2), pgA, ringA, mrow, wpr);
        pre_data<D, MASKED>(cp, tile_at(3, q3), pgB, ringB, mrow, wpr);
        pre_pages<D>(kv, cp, tile_at(4, q4), pgA);
        __syncthreads();

        // Bias operands of the tile of step i (staged in stage st): its
        // allowed slots per row, and -m as it stands now.
        auto make_bias = [&](int i, int qe, const char *st) {
            if constexpr (MASKED) {
                MaskBias b;
                b.lut = lds + PreLds<D>::LUT_OFF;
                b.aop = lds + PreLds<D>::AOP_OFF;
                const int j0 = 32 * tile_at(i, qe);
                // bit 31 of the entry: every slot allowed for every row
                b.fullm = qe < 0 && j0 + 32 <= kv.eff ? 0xFFFFFFFFu : 0u;
                b.lm = tile_bits(j0, kv.eff, false, 0u);
                b.mw = reinterpret_cast<const uint32_t *>(st + cp.mw_lds);
                b.negm2 = w.negm2;
                return b;
            } else {
                RowBias b;
                b.a0 = h == 0 ? 0x00003F80u : 0u;
                b.negm2 = w.negm2;
                return b;
            }
        };
        // Softmax prologue of the tile of step i: slots are dropped by a select
        // only where the bias cannot do it (stale K past kv_len) or, on causal
        // lanes, where the tile crosses a row's causal limit.
        auto tile_max = [&](int i, int qe, f32x16 &s) {
            const int t = tile_at(i, qe);
            int j0 = 32 * t;
            bool sel;
            if constexpr (MASKED) sel = t == cp.ts;
            else sel = j0 + 32 > lmin_w;
            // the selected tile's start stays opaque, so the compiler computes
            // its drop masks where they are used instead of keeping them live
            // across the loop
            asm volatile("" : "+s"(j0));
            return pre_max(s, sel, sel ? tile_bits(j0, MASKED ? kv.eff : lim, false, 0u) : 0u);
        };
        auto b0 = make_bias(0, q0, stage(0));
        f32x16 sA = pre_qk<D>(stage(0), w, b0), sB = {};
        pre_rescale<D>(sA, tile_max(0, q0, sA), w);
        auto step = [&](auto kc, int i) {
            constexpr int K = decltype(kc)::value;
            char *stc = stage(K);
            char *stn = stage((K + 1) % kPreStages);
            char *sts = stage((K + 2) % kPreStages);
            f32x16 &sc = (K & 1) ? sB : sA;
            f32x16 &sn = (K & 1) ? sA : sB;
            PreStage &ring = (K & 1) ? ringB : ringA;
            PrePages &pgc = (K & 1) ? pgB : pgA;  // page ids of tile i+4 (read one step ago)
            PrePages &pgn = (K & 1) ? pgA : pgB;  // receives the page ids of tile i+5
            int q6 = 0;
            if constexpr (MASKED) q6 = __builtin_amdgcn_readfirstlane(lv);
            const int t2 = tile_at(i + 2, q2), t4 = tile_at(i + 4, q4), t5 = tile_at(i + 5, q5);
            auto bias = make_bias(i + 1, q1, stn);
            float mt_next = 0.0f;
            pre_main<D>(stc, stn, sc, sn, w, bias, [&](int k) {
                if (k == 0) {
                    // list entry and page ids first: the data loads then wait
                    // only on loads issued one step earlier, never the newest
                    if constexpr (MASKED) lv = lst[in_vgpr(1 + min(i + 7, T - 1))];
                    pre_pages<D>(kv, cp, t5, pgn);
                }
                if (k == 1) pre_store<D, MASKED>(cp, ring, sts, t2);
                if (k == 2) pre_data<D, MASKED>(cp, t4, pgc, ring, mrow, wpr);
            }, [&](int part) {
                if (i + 1 < T) {  // workgroup-uniform
                    if (part == 0) mt_next = tile_max(i + 1, q1, sn);
                    else pre_rescale<D>(sn, mt_next, w);
                }
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
        // Whole groups of four steps in a loop whose only exit is at its
        // bottom, then the remaining steps: exits in the middle of the loop
        // body would be merged into one block that also leads back to the
        // loop header, and the loads in flight on that path would then be
        // waited for at the top of every group.
        const int T4 = T & ~(kPreStages - 1);
        for (int i = 0; i < T4; i += kPreStages) {
            step(StepK<0>{}, i);
            step(StepK<1>{}, i + 1);
            step(StepK<2>{}, i + 2);
            step(StepK<3>{}, i + 3);
        }
        if (T4 < T) {
            step(StepK<0>{}, T4);
            if (T4 + 1 < T) {
                step(StepK<1>{}, T4 + 1);
                if (T4 + 2 < T) step(StepK<2>{}, T4 + 2);
            }
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
    __shared__ __attribute__((aligned(16))) char s_lds[PreLds<D>::TOTAL];
    __shared__ int s_lmax[kPreWaves];
    const int4 it = a.pre_items[blockIdx.x];
    if (it.x < 0) return;
    const bool masked = a.mask_off && a.mask_off[it.x + 1] > a.mask_off[it.x];  // workgroup-uniform
    if (masked) prefill_item<D, G, true>(a, it, s_lds, s_lmax);
    else prefill_item<D, G, false>(a, it, s_lds, s_lmax);
}

}  // namespace fpk
