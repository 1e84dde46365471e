// fp_prefill.h - ragged prefill attention (lanes with more rows x GQA heads than one MFMA N block).
//
// One workgroup of eight waves per (lane, KV head, block of 256/G rows): wave w
// owns query head g*G + w%G for 32 rows of the block, so every K/V tile the
// workgroup stages in LDS feeds all G query heads of the KV head (GQA sharing).
// Tiles of 32 slots are read from HBM once per workgroup into a three-stage
// LDS ring laid out so the MFMA fragment reads are free of bank conflicts:
//   K   [32 slots][D]   rows padded by 16 bytes
//   V^T [D][32 slots]   rows padded by 16 bytes
// (the padding staggers the rows a quarter-wave reads across all LDS banks, and
// keeps every fragment of a lane at a constant offset from one base address).
// Scores use S^T = K * Q^T and O^T += V^T * P^T on v_mfma_f32_32x32x16_bf16
// (the same register mapping as the 32-column decode path), with the online
// softmax rescaling O only when a column's running max grows by more than 2^8.
#pragma once

#include "fp_kernels.h"

namespace fpk {

constexpr int kPreWaves = 8;
constexpr int kPreThreads = 64 * kPreWaves;
constexpr float kRescaleSlack = 8.0f;  // log2 units: p stays below 2^8 between rescales
constexpr int kPreSumWords = 1024;     // summary words per kind staged in LDS: capacity <= 1M slots

template <int D>
struct PreLds {
    static constexpr int KC = D / 8;              // 16-byte chunks per K row
    static constexpr int KROW = D * 2 + 16;       // padded K row (bytes)
    static constexpr int VROW = 32 * 2 + 16;      // padded V^T row (bytes)
    static constexpr int K_BYTES = 32 * KROW;
    static constexpr int V_BYTES = D * VROW;
    static constexpr int STAGE = K_BYTES + V_BYTES;
};

// What this thread brings in for one tile: a 16-byte K chunk and V^T chunk for
// the shared LDS stage and the mask word of its own query column.
template <int D>
struct PreStage {
    uint4 k, v;
    uint32_t mw;
};

// Physical pages of the K and V^T chunks this thread moves for tile t (loaded
// one pipeline step before the data, so waiting for them never waits for the
// data loads still in flight behind them).
struct PrePages {
    int k, v;
};

template <int D>
__device__ __forceinline__ void pre_pages(const KvView &kv, int t, PrePages &pp) {
    constexpr int KC = PreLds<D>::KC;
    const int tid = threadIdx.x;
    t = t < 0 ? 0 : t;
    const int j0 = 32 * t;
    const int sk = j0 + (tid % (32 * KC)) / KC;
    const int sv = j0 + 8 * (tid & 3);
    pp.k = kv.pids[(sk < kv.eff ? sk : 0) / kv.P];
    pp.v = kv.pids[(sv < kv.eff ? sv : 0) / kv.P];
}

// Every load here is unconditional (out-of-range slots read a valid address and
// are zeroed afterwards; tiles past the sequence fetch tile 0 and are never
// used), so the compiler can count outstanding loads exactly and wait for one
// tile's data without draining the later prefetches.
template <int D>
__device__ __forceinline__ void pre_data(const KvView &kv, int t, const PrePages &pp, PreStage<D> &st,
                                         const uint32_t *mrow, int64_t wpr) {
    constexpr int KC = PreLds<D>::KC;
    const int tid = threadIdx.x;
    t = t < 0 ? 0 : t;
    const int j0 = 32 * t;
    st.mw = mrow[t < wpr ? t : 0];  // mrow points at valid memory for every lane
    {
        const int s = j0 + (tid % (32 * KC)) / KC, c = tid % KC;
        const bool ok = (tid < 32 * KC) && s < kv.eff;
        const int sc = ok ? s : 0;
        const int64_t page = (int64_t)min(max(pp.k, 0), kv.last_page);
        const uint4 v = *reinterpret_cast<const uint4 *>(kv.kbase + page * kv.page_elems +
                                                         ((int64_t)kv.g * kv.P + (sc % kv.P)) * D + 8 * c);
        st.k = ok ? v : make_uint4(0, 0, 0, 0);
    }
    {
        const int d = (tid % (4 * D)) >> 2, cc = tid & 3;
        const int s8 = j0 + 8 * cc;
        const bool ok = (tid < 4 * D) && s8 < kv.eff;
        const int sc = ok ? s8 : 0;
        const int64_t page = (int64_t)min(max(pp.v, 0), kv.last_page);
        const uint16_t *src = kv.kbase + page * kv.page_elems + kv.vblock + (int64_t)kv.g * D * kv.P +
                              (int64_t)d * kv.P + (sc % kv.P);
        const uint4 v = *reinterpret_cast<const uint4 *>(src);
        // slots at or past kv_len must not reach P*V (0 * NaN is NaN)
        const int nv = ok ? kv.eff - s8 : 0;
        uint32_t mk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) mk[q] = (2 * q + 1 < nv) ? 0xFFFFFFFFu : ((2 * q < nv) ? 0x0000FFFFu : 0u);
        st.v = make_uint4(v.x & mk[0], v.y & mk[1], v.z & mk[2], v.w & mk[3]);
    }
}

template <int D>
__device__ __forceinline__ void pre_store(const PreStage<D> &st, char *stage) {
    constexpr int KC = PreLds<D>::KC;
    const int tid = threadIdx.x;
    if (tid < 32 * KC) {
        const int s = tid / KC, c = tid % KC;
        *reinterpret_cast<uint4 *>(stage + s * PreLds<D>::KROW + 16 * c) = st.k;
    }
    if (tid < D * 4) {
        const int d = tid >> 2, cc = tid & 3;
        *reinterpret_cast<uint4 *>(stage + PreLds<D>::K_BYTES + d * PreLds<D>::VROW + 16 * cc) = st.v;
    }
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

// Softmax of one tile's scores (valid-slot bits per lane, or all valid) and
// O^T += V^T * P^T from the staged tile.
template <int D>
__device__ __forceinline__ void pre_pv(const char *stage, const f32x16 &sacc, bool full, uint32_t vbits,
                                       PreWave<D> &w) {
    const int ln = lane_id(), h = ln >> 5, n = ln & 31;
    // V^T fragments do not depend on P: issue their reads before the softmax
    const char *vrow = stage + PreLds<D>::K_BYTES + n * PreLds<D>::VROW + 16 * h;
    uint4 vf[D / 32][2];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        vf[db][0] = *reinterpret_cast<const uint4 *>(vrow + 32 * db * PreLds<D>::VROW);
        vf[db][1] = *reinterpret_cast<const uint4 *>(vrow + 32 * db * PreLds<D>::VROW + 32);
    }
    float sv[16];
    float mt = kNegInf;
    if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sv[i] = sacc[i];
            mt = fmaxf(mt, sv[i]);
        }
    } else {
        const uint32_t vb = vbits >> (8 * h);  // register i holds tile slot 16(i/8) + 8h + i%8
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sv[i] = ((vb >> (16 * (i >> 3) + (i & 7))) & 1u) ? sacc[i] : kNegInf;
            mt = fmaxf(mt, sv[i]);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = mt > w.m + kRescaleSlack;
    if (__any(grow)) {
        const float m_new = grow ? mt : w.m;
        const float alpha = (w.m == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(w.m - m_new);
        w.l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] *= alpha;
        w.m = m_new;
    }
    const float m_use = (w.m == kNegInf) ? 0.0f : w.m;
    float ps = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float p0 = __builtin_amdgcn_exp2f(sv[2 * q] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(sv[2 * q + 1] - m_use);
        ps += p0 + p1;
        pk[q] = pack_bf16x2(p0, p1);
    }
    w.l += ps;
    const uint4 pb0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    const uint4 pb1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        w.o[db] = mfma32(vf[db][0], pb0, w.o[db]);
        w.o[db] = mfma32(vf[db][1], pb1, w.o[db]);
    }
}

// Allowed slots of tile j0 for this lane's column as a 32-bit mask.
__device__ __forceinline__ uint32_t tile_bits(int j0, int lim, bool masked, uint32_t mw) {
    const int rem = lim - j0;
    const uint32_t lm = rem >= 32 ? 0xFFFFFFFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
    return masked ? (mw & lm) : lm;
}

// Tiles a workgroup visits: 0..T-1 under the causal rule, or the tiles whose
// summary bit is set for a masked lane (all threads walk the same sequence).
struct TileSeq {
    const uint32_t *any;  // summary words staged in LDS; nullptr: dense
    int T, wi;
    uint32_t bits;
};

__device__ __forceinline__ int seq_next(TileSeq &q, int cur) {
    if (!q.any) return (cur + 1 < q.T) ? cur + 1 : -1;
    for (;;) {
        if (q.bits) {
            const int b = __builtin_ctz(q.bits);
            q.bits &= q.bits - 1u;
            const int t = 32 * q.wi + b;
            return t < q.T ? t : -1;
        }
        ++q.wi;
        if (32 * q.wi >= q.T) return -1;
        q.bits = __builtin_amdgcn_readfirstlane(q.any[q.wi]);
    }
}

// Prefill: one workgroup of eight waves per (lane, KV head, block of 256/G
// rows); wave w owns query head g*G + w%G for the 32 rows at 32*(w/G).
template <int D, int G>
__global__ void __launch_bounds__(kPreThreads) prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char s_tile[3][PreLds<D>::STAGE];
    __shared__ int s_lmax[kPreWaves];
    __shared__ uint32_t s_sum[2][kPreSumWords];  // the row block's summary words: any, all

    const int4 it = a.pre_items[blockIdx.x];
    if (it.x < 0) return;
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
        w.m = kNegInf;
        w.l = 0.0f;
    }
    const bool masked = a.mask_off && a.mask_off[lane + 1] > a.mask_off[lane];
    // Mask-word pointers are always valid so their loads need no branch: a
    // causal lane reads a harmless word of indptr and ignores it.
    const uint32_t *mrow = reinterpret_cast<const uint32_t *>(a.indptr);
    int64_t wpr = 1;
    if (masked) {
        wpr = (a.mask_off[lane + 1] - a.mask_off[lane]) / nrows;
        mrow = a.mask_bits + a.mask_off[lane] + (int64_t)(rstart + (colv ? rloc : 0)) * wpr;
    }
    const int lim = !colv ? 0 : (masked ? kv.eff : min(a.slots[row] + 1, kv.eff));
    const int lmax_w = __builtin_amdgcn_readfirstlane(wave_max_i(lim));
    const int lmin_w = __builtin_amdgcn_readfirstlane(-wave_max_i(colv ? -lim : -0x7FFFFFFF));  // valid columns
    // Let the Q loads land before the pipeline starts: otherwise the first use
    // of Q inside the loop carries a wait for every load in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (ln == 0) s_lmax[wv] = lmax_w;
    __syncthreads();
    int lwg = 0;
#pragma unroll
    for (int v = 0; v < kPreWaves; ++v) lwg = max(lwg, s_lmax[v]);
    lwg = __builtin_amdgcn_readfirstlane(lwg);

    TileSeq seq;
    seq.T = (lwg + 31) >> 5;
    seq.any = nullptr;
    seq.wi = 0;
    seq.bits = 0;
    if (masked) {  // workgroup-uniform
        const LaneInfo li = a.lane_info[lane];
        const uint32_t *gs = a.summary + li.sum_off + (int64_t)(rstart / prefill_rows(G)) * 2 * li.sum_wpb;
        const int nw = min(li.sum_wpb, kPreSumWords);
        for (int i = threadIdx.x; i < nw; i += kPreThreads) {
            s_sum[0][i] = gs[i];
            s_sum[1][i] = gs[li.sum_wpb + i];
        }
        __syncthreads();
        seq.any = s_sum[0];
        seq.bits = seq.T > 0 ? __builtin_amdgcn_readfirstlane(seq.any[0]) : 0u;
    }
    const uint32_t *allw = s_sum[1];

    // Software pipeline over the tile sequence t0, t1, t2, ...: while the
    // softmax and P*V of tile t0 run, the QK^T MFMAs of t1 are already issued
    // (its K sits in the next LDS stage), t2 and t3 are in flight from HBM in
    // registers (ring), and the page ids of t4 are being read. Three LDS stages
    // rotate; the loop is unrolled twice so no register holding in-flight data
    // is copied, and every global load in the loop is unconditional.
    int st = 0;
    int t0 = seq_next(seq, -1);
    int t1 = t0 >= 0 ? seq_next(seq, t0) : -1;
    int t2 = t1 >= 0 ? seq_next(seq, t1) : -1;
    int t3 = t2 >= 0 ? seq_next(seq, t2) : -1;
    int t4 = t3 >= 0 ? seq_next(seq, t3) : -1;
    PreStage<D> ringA, ringB;
    PrePages pgA, pgB;
    uint32_t mw0 = 0u, mw1 = 0u;
    if (t0 >= 0) {  // workgroup-uniform
        pre_pages<D>(kv, t0, pgA);
        pre_pages<D>(kv, t1, pgB);
        pre_data<D>(kv, t0, pgA, ringA, mrow, wpr);
        pre_data<D>(kv, t1, pgB, ringB, mrow, wpr);
        pre_pages<D>(kv, t2, pgA);
        pre_pages<D>(kv, t3, pgB);
        pre_store<D>(ringA, s_tile[0]);
        mw0 = ringA.mw;
        pre_store<D>(ringB, s_tile[1]);
        mw1 = ringB.mw;
        pre_data<D>(kv, t2, pgA, ringA, mrow, wpr);
        pre_data<D>(kv, t3, pgB, ringB, mrow, wpr);
        pre_pages<D>(kv, t4, pgA);
    }
    __syncthreads();

    auto active = [&](int t) { return t >= 0 && 32 * t < lmax_w; };
    auto finish = [&](int t, const f32x16 &sacc, uint32_t mw, int stage) {
        const int j0 = 32 * t;
        const bool full = masked ? (((allw[t >> 5] >> (t & 31)) & 1u) && j0 + 32 <= kv.eff) : (j0 + 32 <= lmin_w);
        pre_pv<D>(s_tile[stage], sacc, full, full ? 0u : tile_bits(j0, lim, masked, mw), w);
    };
    f32x16 sA = {}, sB = {};
    if (active(t0)) sA = pre_qk<D>(s_tile[0], w);
    while (t0 >= 0) {
        const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
        if (active(t1)) sB = pre_qk<D>(s_tile[st1], w);
        if (active(t0)) finish(t0, sA, mw0, st);
        // page ids first: the data loads below then wait only on page ids
        // read one step earlier, never on the newest loads
        const int t5 = t4 >= 0 ? seq_next(seq, t4) : -1;
        pre_pages<D>(kv, t5, pgB);
        pre_store<D>(ringA, s_tile[st2]);  // tile t2
        const uint32_t mw2 = ringA.mw;
        pre_data<D>(kv, t4, pgA, ringA, mrow, wpr);
        __syncthreads();
        st = st1;
        if (t1 < 0) break;

        const int su1 = st == 2 ? 0 : st + 1, su2 = su1 == 2 ? 0 : su1 + 1;
        if (active(t2)) sA = pre_qk<D>(s_tile[su1], w);
        if (active(t1)) finish(t1, sB, mw1, st);
        const int t6 = t5 >= 0 ? seq_next(seq, t5) : -1;
        pre_pages<D>(kv, t6, pgA);
        pre_store<D>(ringB, s_tile[su2]);  // tile t3
        const uint32_t mw3 = ringB.mw;
        pre_data<D>(kv, t5, pgB, ringB, mrow, wpr);
        __syncthreads();
        st = su1;
        if (t2 < 0) break;
        t0 = t2;
        t1 = t3;
        t2 = t4;
        t3 = t5;
        t4 = t6;
        mw0 = mw2;
        mw1 = mw3;
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

}  // namespace fpk
