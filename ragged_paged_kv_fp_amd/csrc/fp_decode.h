// fp_decode.h - split-KV decode attention (lanes whose rows x GQA heads fit one MFMA N block).
//
// One workgroup of four waves per (lane, KV head, KV split). The waves take
// every fourth 32-slot tile of the split; each keeps the next tile's K/V in a
// second register set while it computes the current one, with the page ids
// fetched one tile further ahead. At the end the waves combine through LDS,
// and a lane read in several splits is combined by merge_kernel.
//
// Two MFMA shapes:
//   NC = 16 : v_mfma_f32_16x16x32_bf16, up to 16 query row-heads per lane
//   NC = 32 : v_mfma_f32_32x32x16_bf16, up to 32 (e.g. 8 draft rows x 4 heads)
#pragma once

#include <type_traits>

#include "fp_kernels.h"

namespace fpk {

typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Waves per decode workgroup: four for the 16-column kernel (two workgroups per
// CU at two waves per SIMD); two for the 32-column kernel, whose registers allow
// one wave per SIMD, so that two items still run side by side on each CU and one
// item's start and end overlap the other's streaming.
template <int NC>
constexpr int dec_waves() { return NC == 32 ? 2 : 4; }
constexpr int kLdsRow = 68;  // padded row of 64 floats: rows land on different LDS banks

// A tile's K/V as loaded from the pool. The K rows are read as whole
// contiguous 1 KB runs of the pages (every load instruction covers complete
// cache lines, so the loads can be non-temporal) and staged through a small
// per-wave LDS buffer into the MFMA fragment layout; the V^T fragments are
// already contiguous runs and are loaded directly.
template <int D>
struct KvFrags {
    uint4 k[D / 16];  // raw K: run u holds tile rows u*(512/D) .. of this lane's 16-byte column
    uint4 v[D / 16];
};

struct TilePages {
    int kp;          // lane l: physical page of the tile's (l & 3)-th page (raw K runs)
    int64_t v0, v1;  // physical pages of this lane's V^T fragments
};

// Keep bf16 elements [0, nv) of an 8-element fragment (slots at or past kv_len
// must not reach P*V, since 0 * NaN is NaN).
__device__ __forceinline__ uint4 keep_first(uint4 v, int nv) {
    uint32_t mk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mk[q] = (2 * q + 1 < nv) ? 0xFFFFFFFFu : ((2 * q < nv) ? 0x0000FFFFu : 0u);
    return make_uint4(v.x & mk[0], v.y & mk[1], v.z & mk[2], v.w & mk[3]);
}

// Physical pages for the tile at j0: the tile's pages for the raw K runs (one
// per lane, indexed by lane & 3) and the pages of this lane's V^T slot groups
// (slot groups at or past kv_len read the lane's first page instead: every
// load stays branch-free and in bounds).
template <int NC>
__device__ __forceinline__ TilePages tile_pages(const KvView &kv, int j0) {
    const int l = lane_id();
    int vg0, vg1;
    if (NC == 16) {
        vg0 = j0 + 8 * (l >> 4);
        vg1 = vg0;
    } else {
        vg0 = j0 + 8 * (l >> 5);
        vg1 = vg0 + 16;
    }
    TilePages tp;
    const int lastpg = kv.eff > 0 ? (kv.eff - 1) >> kv.pshift : 0;
    tp.kp = (int)page_of(kv, min((j0 >> kv.pshift) + (l & 3), lastpg));
    tp.v0 = page_of(kv, (vg0 < kv.eff ? vg0 : 0) >> kv.pshift);
    tp.v1 = NC == 32 ? page_of(kv, (vg1 < kv.eff ? vg1 : 0) >> kv.pshift) : tp.v0;
    return tp;
}

// Raw K runs and V^T fragments of the tile at j0 (all loads non-temporal: the
// decode pass reads every KV byte once).
//  K: run u covers tile rows u*(512/D) .. u*(512/D) + 512/D - 1, lane l takes
//     row u*(512/D) + l/(D/8), 16-byte column l % (D/8); a run never crosses a
//     page (P >= 8 >= 512/D rows), so its page is one wave-uniform value.
//  V^T rows of the O^T = V^T * P^T operand:
//  NC=16: lane (q = l/16, m = l%16): V^T row d = 16 db + m, slots 8q .. 8q+7.
//  NC=32: lane (h = l/32, n = l%32): V^T row d = 32 db + n, slots 16 t + 8h .. +7.
template <int D, int NC>
__device__ __forceinline__ void tile_load(const KvView &kv, int j0, const TilePages &tp, KvFrags<D> &f) {
    constexpr int RPR = 512 / D;  // tile rows per run
    constexpr int LPR = D / 8;    // lanes per row
    const int l = lane_id();
    const int64_t kcol = (int64_t)kv.g * kv.P * D + 8 * (l % LPR);
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
        const int r = u * RPR + l / LPR;
        const int64_t page = __builtin_amdgcn_readlane(tp.kp, (u * RPR) >> kv.pshift);
        f.k[u] = load_nt(kv.kbase + page * kv.page_elems + kcol + (int64_t)(r & kv.pmask) * D);
    }
    const int64_t vbase = kv.vblock + (int64_t)kv.g * D * kv.P;
    if (NC == 16) {
        const int m = l & 15, q = l >> 4;
        const int vg = j0 + 8 * q;
        const int vc = vg < kv.eff ? vg : 0;
        const uint16_t *vb = kv.kbase + tp.v0 * kv.page_elems + vbase + (vc & kv.pmask);
        const int nv = vg < kv.eff ? kv.eff - vg : 0;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
            f.v[db] = keep_first(load_nt(vb + (int64_t)(16 * db + m) * kv.P), nv);
    } else {
        const int n = l & 31, h = l >> 5;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            const int vs = j0 + 16 * t2 + 8 * h;
            const int vc = vs < kv.eff ? vs : 0;
            const uint16_t *vb = kv.kbase + (t2 ? tp.v1 : tp.v0) * kv.page_elems + vbase + (vc & kv.pmask);
            const int nv = vs < kv.eff ? kv.eff - vs : 0;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                f.v[2 * db + t2] = keep_first(load_nt(vb + (int64_t)(32 * db + n) * kv.P), nv);
        }
    }
}

// Per-wave K staging buffer: 32 tile rows of D bf16, rows padded by 16 bytes.
template <int D>
struct DecLds {
    static constexpr int KROW = 2 * D + 16;
    static constexpr int BYTES = 32 * KROW;
};

// Writes the raw K runs to the wave's buffer and reads back the K operand
// fragments of S^T = K * Q^T (rows as the MFMA shape expects them):
//  NC=16: lane (q, m): K row 8(m/4) + 4b + m%4 of M-block b, d in [q D/4, (q+1) D/4).
//  NC=32: lane (h, n): K row kslot_of_row(n), d in [h D/2, (h+1) D/2).
// Slots at or past kv_len keep whatever the pool holds: their scores are
// dropped by the softmax select.
template <int D, int NC>
__device__ __forceinline__ void stage_k(const KvFrags<D> &f, char *buf, uint4 (&kf)[D / 16]) {
    constexpr int RPR = 512 / D, LPR = D / 8, KROW = DecLds<D>::KROW;
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
        *reinterpret_cast<uint4 *>(buf + (u * RPR + l / LPR) * KROW + 16 * (l % LPR)) = f.k[u];
    if (NC == 16) {
        constexpr int KS = D / 32;
        const int m = l & 15, q = l >> 4;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const char *row = buf + (8 * (m >> 2) + 4 * b + (m & 3)) * KROW + q * (D / 2);
#pragma unroll
            for (int s = 0; s < KS; ++s) kf[b * KS + s] = *reinterpret_cast<const uint4 *>(row + 16 * s);
        }
    } else {
        const int n = l & 31, h = l >> 5;
        const char *row = buf + kslot_of_row(n) * KROW + h * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const uint4 *>(row + 16 * s);
    }
}

template <int D, int NC>
struct DecState {
    static constexpr int QF = (NC == 16) ? D / 32 : D / 16;   // Q^T fragments per lane
    static constexpr int OB = (NC == 16) ? D / 16 : D / 32;   // O^T accumulator blocks
    using Acc = typename std::conditional<NC == 16, f32x4, f32x16>::type;
    uint4 qf[QF];
    Acc o[OB];
    float m, l;
};

__device__ __forceinline__ void softmax_update(float mt, float &m_run, float &m_use, float &alpha) {
    const float m_new = fmaxf(m_run, mt);
    m_use = (m_new == kNegInf) ? 0.0f : m_new;
    alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
}

template <int D>
__device__ __forceinline__ void tile_compute(const KvFrags<D> &f, char *kbuf, int j0, int lim, uint32_t mw,
                                             bool masked, DecState<D, 16> &w) {
    constexpr int KS = D / 32;
    const int q = lane_id() >> 4;
    uint4 kf[D / 16];
    stage_k<D, 16>(f, kbuf, kf);
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        s0 = mfma16(kf[s], w.qf[s], s0);
        s1 = mfma16(kf[KS + s], w.qf[s], s1);
    }
    float sv[8];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int so = 8 * q + j;
        bool ok = (j0 + so) < lim;
        if (masked) ok = ok && ((mw >> so) & 1u);
        sv[j] = ok ? (j < 4 ? s0[j] : s1[j - 4]) : kNegInf;
        mt = fmaxf(mt, sv[j]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    float m_use, alpha;
    softmax_update(mt, w.m, m_use, alpha);
    float ps = 0.0f;
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(sv[2 * j] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(sv[2 * j + 1] - m_use);
        ps += p0 + p1;
        pk[j] = pack_bf16x2(p0, p1);
    }
    w.l = w.l * alpha + ps;
    const uint4 pb = make_uint4(pk[0], pk[1], pk[2], pk[3]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        w.o[db] *= alpha;
        w.o[db] = mfma16(f.v[db], pb, w.o[db]);
    }
}

template <int D>
__device__ __forceinline__ void tile_compute(const KvFrags<D> &f, char *kbuf, int j0, int lim, uint32_t mw,
                                             bool masked, DecState<D, 32> &w) {
    const int h = lane_id() >> 5;
    uint4 kf[D / 16];
    stage_k<D, 32>(f, kbuf, kf);
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sacc = mfma32(kf[s], w.qf[s], sacc);
    float sv[16];
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int so = 16 * (i >> 3) + 8 * h + (i & 7);
        bool ok = (j0 + so) < lim;
        if (masked) ok = ok && ((mw >> so) & 1u);
        sv[i] = ok ? sacc[i] : kNegInf;
        mt = fmaxf(mt, sv[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    float m_use, alpha;
    softmax_update(mt, w.m, m_use, alpha);
    float ps = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float p0 = __builtin_amdgcn_exp2f(sv[2 * q] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(sv[2 * q + 1] - m_use);
        ps += p0 + p1;
        pk[q] = pack_bf16x2(p0, p1);
    }
    w.l = w.l * alpha + ps;
    const uint4 pb0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    const uint4 pb1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        w.o[db] *= alpha;
        w.o[db] = mfma32(f.v[2 * db], pb0, w.o[db]);
        w.o[db] = mfma32(f.v[2 * db + 1], pb1, w.o[db]);
    }
}

// Write this wave's accumulator values whose d falls in [64c, 64c+64), scaled, into LDS row `col`.
template <int D, int NC>
__device__ __forceinline__ void stage_o(const DecState<D, NC> &w, int c, float scale, float *row) {
    const int l = lane_id();
    if (NC == 16) {
        const int q = l >> 4;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            if (db / 4 != c) continue;
            const float4 v = make_float4(w.o[db][0] * scale, w.o[db][1] * scale, w.o[db][2] * scale, w.o[db][3] * scale);
            *reinterpret_cast<float4 *>(row + 16 * (db - 4 * c) + 4 * q) = v;
        }
    } else {
        const int h = l >> 5;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            if (db / 2 != c) continue;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const float4 v = make_float4(w.o[db][4 * i4] * scale, w.o[db][4 * i4 + 1] * scale,
                                             w.o[db][4 * i4 + 2] * scale, w.o[db][4 * i4 + 3] * scale);
                *reinterpret_cast<float4 *>(row + 32 * (db - 2 * c) + 8 * i4 + 4 * h) = v;
            }
        }
    }
}

// LDS of one decode workgroup. The K staging buffers (used by the tile loop)
// and the output combine rows (used after it, past a barrier) share storage.
template <int D, int NC>
struct DecShared {
    static constexpr int W = dec_waves<NC>();
    float ml[W][2][32];
    float fin[2][32];
    union __attribute__((aligned(16))) {  // 16-byte LDS accesses
        float o[W][NC][kLdsRow];
        char k[W][DecLds<D>::BYTES];
    } u;
    int steps[W];  // tile steps of each wave (masked launch)
};

// One work item (lane, KV head, KV split): every barrier inside is reached by
// all threads of the workgroup.
template <int D, int NC, bool MASKED>
__device__ __forceinline__ void decode_item(const AttnArgs &a, const int4 it, DecShared<D, NC> &sh) {
    auto &s_ml = sh.ml;
    auto &s_fin = sh.fin;
    auto &s_o = sh.u.o;
    auto &s_k = sh.u.k;
    constexpr int kDecWaves = dec_waves<NC>(), kDecThreads = 64 * kDecWaves;
    const int lane = it.x, g = it.y, s0 = it.z, s1 = it.w;
    const LaneInfo li = a.lane_info[lane];
    const int r0 = a.indptr[lane];
    const int nrows = a.indptr[lane + 1] - r0;
    const int ncols = nrows * a.G;
    const int wv = threadIdx.x / kWave, l = lane_id();
    const int col = (NC == 16) ? (l & 15) : (l & 31);
    const int part = (NC == 16) ? (l >> 4) : (l >> 5);
    const bool colv = col < ncols;
    const int64_t row = r0 + (colv ? col / a.G : 0);
    const int head = g * a.G + (colv ? col % a.G : 0);
    int cap;
    KvView kv = make_view(a, lane, g, &cap);
    kv.vblock = (int64_t)a.H * a.P * D;

    DecState<D, NC> w;
    {
        constexpr int QF = DecState<D, NC>::QF;
        const uint4 *src = reinterpret_cast<const uint4 *>(a.qrot + (row * a.Hq + head) * D + part * (D / (NC == 16 ? 4 : 2)));
#pragma unroll
        for (int s = 0; s < QF; ++s) w.qf[s] = colv ? src[s] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < DecState<D, NC>::OB; ++b) w.o[b] = typename DecState<D, NC>::Acc{};
        w.m = kNegInf;
        w.l = 0.0f;
    }
    constexpr bool masked = MASKED;  // a masked lane (the launch holds only those) walks its tile list
    const uint32_t *mrow = nullptr;
    int64_t wpr = 0;
    if constexpr (MASKED) {
        wpr = (a.mask_off[lane + 1] - a.mask_off[lane]) / nrows;
        mrow = a.mask_bits + a.mask_off[lane] + (colv ? (col / a.G) : 0) * wpr;
    }
    const int lim = !colv ? 0 : (masked ? kv.eff : min(a.slots[row] + 1, kv.eff));
    // Tiles of this wave: without a tile list, every kDecWaves-th 32-slot tile
    // of the split below the wave's furthest limit; with one (a masked lane,
    // built by summary_kernel: only the tiles where some row of the lane may
    // read a slot), every kDecWaves-th entry of the split's share of the list,
    // each lane of the wave holding one entry.
    constexpr int kStep = 32 * kDecWaves;
    const int first = s0 + 32 * wv;
    int nsteps;
    uint32_t ent = 0;
    if constexpr (MASKED) {
        const int32_t *lst = a.summary + li.sum_off;
        const int p0 = s0 >> 5, p1 = (s1 + 31) >> 5;
        const int pl = min(p0 + wv + kDecWaves * l, li.sum_stride - 2);  // stays inside the record
        ent = (uint32_t)lst[1 + pl];
        const int cnt = __builtin_amdgcn_readfirstlane(min(lst[0], p1));
        nsteps = cnt > p0 + wv ? (cnt - p0 - wv + kDecWaves - 1) / kDecWaves : 0;
    } else {
        const int jend = __builtin_amdgcn_readfirstlane(min(s1, wave_max_i(lim)));
        nsteps = first < jend ? (jend - 1 - first) / kStep + 1 : 0;
    }

    // ---- stream this wave's tiles. While tile i is computed, tile i+1 is in
    // flight and the page ids of tile i+2 are being read; a step past the
    // wave's last maps to its last tile (a cache hit), so every load is
    // unconditional and the compiler's memory waits only cover the data
    // actually needed.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // Q (and the list entries) have landed before the pipeline starts
    // the pipeline over steps 0..ilast, the tile of step i starting at slot jof(i)
    auto stream_tiles = [&](int ilast, auto jof) {
        auto mword = [&](int j0) { return (masked && colv && (j0 >> 5) < wpr) ? mrow[j0 >> 5] : 0u; };
        int i = 0;
        KvFrags<D> fa, fb;
        TilePages pa = tile_pages<NC>(kv, jof(0));
        TilePages pb = tile_pages<NC>(kv, jof(1));
        tile_load<D, NC>(kv, jof(0), pa, fa);
        pa = tile_pages<NC>(kv, jof(2));
        for (;;) {
            tile_load<D, NC>(kv, jof(i + 1), pb, fb);
            pb = tile_pages<NC>(kv, jof(i + 3));
            const int j0 = jof(i);
            tile_compute<D>(fa, s_k[wv], j0, lim, mword(j0), masked, w);
            if (i + 1 > ilast) break;
            tile_load<D, NC>(kv, jof(i + 2), pa, fa);
            pa = tile_pages<NC>(kv, jof(i + 4));
            const int j1 = jof(i + 1);
            tile_compute<D>(fb, s_k[wv], j1, lim, mword(j1), masked, w);
            if (i + 2 > ilast) break;
            i += 2;
        }
    };
    if (nsteps > 0) {  // wave-uniform
        const int ilast = nsteps - 1;
        if constexpr (MASKED) {
            stream_tiles(ilast, [&](int i) {
                return 32 * (int)(__builtin_amdgcn_readlane(ent, i < ilast ? i : ilast) & 0x7FFFFFFFu);
            });
        } else {
            stream_tiles(ilast, [&](int i) { return first + kStep * (i < ilast ? i : ilast); });
        }
    }

    // ---- combine the four waves through LDS
    float lsum = w.l;
    if (NC == 16) lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (part == 0) {
        s_ml[wv][0][col] = w.m;
        s_ml[wv][1][col] = lsum;
    }
    if constexpr (MASKED) {
        if (l == 0) sh.steps[wv] = nsteps;
    }
    __syncthreads();
    const bool single = li.nsplit <= 1;
    const int64_t pidx = (int64_t)li.dec_off + (int64_t)g * li.nsplit + s0 / a.split;  // (lane, KV head, split)
    // A masked lane's split whose share of the tile list is empty for every
    // wave (most splits of a windowed lane) leaves only its statistics: max
    // -inf and sum 0, which give it weight 0 in the merge, so its partial
    // output is neither written nor read. (Unmasked kernels keep one path:
    // this branch there changed how the compiler schedules the first tile.)
    if constexpr (MASKED) {
        int steps = 0;
#pragma unroll
        for (int v = 0; v < kDecWaves; ++v) steps += sh.steps[v];
        if (!single && steps == 0) {  // workgroup-uniform
            for (int n = threadIdx.x; n < ncols; n += kDecThreads) {
                a.part_ml[pidx * 64 + n] = kNegInf;
                a.part_ml[pidx * 64 + 32 + n] = 0.0f;
            }
            return;
        }
    }
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) M = fmaxf(M, s_ml[v][0][col]);
    const float scale = (M == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(w.m - M);
    if (wv == 0 && part == 0) {
        float L = 0.0f;
#pragma unroll
        for (int v = 0; v < kDecWaves; ++v)
            L += (M == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(s_ml[v][0][col] - M) * s_ml[v][1][col];
        s_fin[0][col] = M;
        s_fin[1][col] = L;
    }
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        stage_o<D, NC>(w, c, scale, &s_o[wv][col][0]);
        __syncthreads();
        // four consecutive dims per thread: 16-byte LDS reads and stores
        for (int e = threadIdx.x; e < NC * 16; e += kDecThreads) {
            const int n = e >> 4, dl = 4 * (e & 15);
            if (n >= ncols) continue;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int v = 0; v < kDecWaves; ++v) {
                const float4 x = *reinterpret_cast<const float4 *>(&s_o[v][n][dl]);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
            }
            const float Lt = s_fin[1][n];
            if (single) {
                const int64_t orow = r0 + n / a.G;
                const int ohead = g * a.G + n % a.G;
                const float4 o = Lt > 0.0f ? make_float4(acc.x / Lt, acc.y / Lt, acc.z / Lt, acc.w / Lt)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4 *>(&a.out[(orow * a.Hq + ohead) * D + 64 * c + dl]) = o;
                if (c == 0 && dl == 0 && a.lse)
                    a.lse[orow * a.Hq + ohead] = Lt > 0.0f ? (s_fin[0][n] + __log2f(Lt)) * 0.69314718055994531f : kNegInf;
            } else {
                *reinterpret_cast<float4 *>(&a.part_o[(pidx * a.ncols_max + n) * D + 64 * c + dl]) = acc;
                if (c == 0 && dl == 0) {
                    a.part_ml[pidx * 64 + n] = s_fin[0][n];
                    a.part_ml[pidx * 64 + 32 + n] = Lt;
                }
            }
        }
        __syncthreads();
    }
}

// One workgroup per work item of the launch's list (the decode items of the
// pass's unmasked lanes, or of its masked lanes). The hardware dispatcher
// starts workgroups in launch order as others finish, so the long items at
// the head of the list go first and the short partial splits set the tail.
template <int D, int NC, bool MASKED>
__global__ void __launch_bounds__(64 * dec_waves<NC>(), NC == 16 ? 2 : 1) decode_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) DecShared<D, NC> sh;
    const int4 it = a.dec_list[blockIdx.x];
    if (it.x >= 0) decode_item<D, NC, MASKED>(a, it, sh);
}

// Combine the KV splits of one (decode lane, KV head), all its query
// columns at once: a workgroup of kMergeThreads. Every split's (max, sum) of
// every column goes to LDS at once, and each thread issues the loads of its
// first kMergeBatch splits' partial outputs before waiting on anything, so
// the work is two memory round trips deep rather than one per step. Then the
// column maxima and denominators are read from LDS and every thread
// accumulates four float4 output groups over the splits.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxSplits = 128;  // splits whose statistics fit the LDS arrays at once
constexpr int kMergeBatch = 4;        // splits of partial outputs in flight per thread

template <int D>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(AttnArgs a) {
    __shared__ float s_m[kMergeMaxSplits][32], s_l[kMergeMaxSplits][32];
    __shared__ float s_M[32], s_den[32];
    const int lane = blockIdx.x, g = blockIdx.y;
    const LaneInfo li = a.lane_info[lane];
    if (li.dec_off < 0 || li.nsplit <= 1) return;  // workgroup-uniform
    const int r0 = a.indptr[lane];
    const int ncols = (a.indptr[lane + 1] - r0) * a.G;
    const int64_t first = (int64_t)li.dec_off + (int64_t)g * li.nsplit;
    const int ns = li.nsplit;
    const int tid = threadIdx.x;
    const float *ml = a.part_ml + first * 64;
    constexpr int D4 = D / 4;
    const int n4 = ncols * D4;                              // float4 groups of the lane's outputs
    const int64_t ostride4 = (int64_t)a.ncols_max * D4;     // float4 groups per split of partial outputs
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o) + first * ostride4;
    // partial outputs of the first kMergeBatch splits: issued before any wait
    float4 pre[kMergeBatch][4];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e4 = tid + kMergeThreads * k;
            pre[b][k] = (b < ns && e4 < n4) ? po[b * ostride4 + e4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    // per-column maximum and denominator over every split, kMergeMaxSplits at a time
    float M = kNegInf, den = 0.0f;
    for (int c0 = 0; c0 < ns; c0 += kMergeMaxSplits) {
        const int cn = min(kMergeMaxSplits, ns - c0);
        __syncthreads();
        for (int e = tid; e < cn * 32; e += kMergeThreads) {
            const int sp = e >> 5, cc = e & 31;
            s_m[sp][cc] = ml[(c0 + sp) * 64 + cc];
            s_l[sp][cc] = ml[(c0 + sp) * 64 + 32 + cc];
        }
        __syncthreads();
        if (tid < 32) {
            float Mc = M;
            for (int sp = 0; sp < cn; ++sp) Mc = fmaxf(Mc, s_m[sp][tid]);
            if (Mc != kNegInf) {
                den = M == kNegInf ? 0.0f : den * __builtin_amdgcn_exp2f(M - Mc);
                for (int sp = 0; sp < cn; ++sp) den += __builtin_amdgcn_exp2f(s_m[sp][tid] - Mc) * s_l[sp][tid];
            }
            M = Mc;
        }
    }
    if (tid < 32) {
        s_M[tid] = M;
        s_den[tid] = den;
    }
    // weighted sum of the partial outputs; a refilled slot takes the split
    // kMergeBatch further on, so kMergeBatch splits stay in flight
    float4 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < ns; c0 += kMergeMaxSplits) {
        const int cn = min(kMergeMaxSplits, ns - c0);
        if (ns > kMergeMaxSplits) {  // LDS holds the last chunk's maxima: bring this chunk's back
            __syncthreads();
            for (int e = tid; e < cn * 32; e += kMergeThreads) s_m[e >> 5][e & 31] = ml[(c0 + (e >> 5)) * 64 + (e & 31)];
        }
        __syncthreads();
        for (int b0 = 0; b0 < cn; b0 += kMergeBatch) {
#pragma unroll
            for (int b = 0; b < kMergeBatch; ++b) {
                const int sp = c0 + b0 + b;
                if (sp >= ns) break;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e4 = tid + kMergeThreads * k;
                    if (e4 >= n4) continue;
                    const int n = e4 / D4;
                    const float Mn = s_M[n];
                    const float w = Mn == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(s_m[b0 + b][n] - Mn);
                    if (w != 0.0f) {  // a split of weight 0 may have left no partial output
                        const float4 v = pre[b][k];
                        acc[k].x += w * v.x;
                        acc[k].y += w * v.y;
                        acc[k].z += w * v.z;
                        acc[k].w += w * v.w;
                    }
                }
                const int nx = sp + kMergeBatch;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e4 = tid + kMergeThreads * k;
                    // splits of this chunk whose column max is -inf are not loaded
                    if (nx < ns && e4 < n4 && (nx >= c0 + cn || s_m[nx - c0][e4 / D4] != kNegInf))
                        pre[b][k] = po[nx * ostride4 + e4];
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e4 = tid + kMergeThreads * k;
        if (e4 >= n4) continue;
        const int n = e4 / D4, d4 = e4 - n * D4;
        const float dn = s_den[n];
        const float inv = dn > 0.0f ? 1.0f / dn : 0.0f;
        const int64_t orow = r0 + n / a.G;
        const int ohead = g * a.G + n % a.G;
        *reinterpret_cast<float4 *>(a.out + (orow * a.Hq + ohead) * D + 4 * d4) =
            make_float4(acc[k].x * inv, acc[k].y * inv, acc[k].z * inv, acc[k].w * inv);
    }
    if (tid < ncols && a.lse) {
        const float dn = s_den[tid];
        const int64_t orow = r0 + tid / a.G;
        const int ohead = g * a.G + tid % a.G;
        a.lse[orow * a.Hq + ohead] = dn > 0.0f ? (s_M[tid] + __log2f(dn)) * 0.69314718055994531f : kNegInf;
    }
}

}  // namespace fpk
