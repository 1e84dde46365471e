// fp_stats.h - attention statistics of a pass: the mass each KV slot received.
//
// For lane l, KV head g and slot j below the lane's (clamped) kv_len:
//   mass[g][j] += sum over the lane's rows r and the G query heads h of g of
//                 p(r, h, j) = 2^(s(r,h,j) - lse2(r,h)) if row r may read slot j, else 0
// where s is the log2-scaled score fp_attend used (rotated, prescaled bf16 Q
// from its workspace times the pool's K) and lse2 its log-sum-exp in base 2.
// Each row's probabilities therefore sum to one over its allowed slots, the
// same normalisation as the attention output.
//
// One workgroup of four waves per (lane, KV head, chunk of eight 32-slot
// tiles). The chunk's K is staged once in LDS (rows padded by 16 bytes, as in
// the prefill kernel, so fragment reads are free of bank conflicts); the waves
// then stream the lane's (32-row block, query head) pairs: a pair's Q
// fragments are loaded once and serve all eight tiles, each tile computing
// S^T = K * Q^T with the prefill kernel's slot permutation (lane half h holds
// slots 8h..8h+7 and 16+8h..16+8h+7 of its column) and adding p to per-lane,
// per-slot sums held in registers. Before that, the workgroup marks in LDS
// the row blocks that may read any slot of the chunk (every row's mask words
// or causal limit loaded at once), so the waves skip the other pairs without
// waiting on memory for each. A pair with no allowed slot in the chunk is
// skipped by the whole wave; otherwise all eight tiles are computed (dropped
// slots add zero), so the MFMA chain of one tile overlaps the exponentials of
// the one before. At the end the 32 columns of a
// wave are summed in registers (DPP and a row swap), the four waves through LDS, and one
// thread per slot adds the total to the output: a single owner per output
// word and a fixed summation order, so the result does not depend on
// scheduling.
#pragma once

#include "fp_kernels.h"

namespace fpk {

constexpr int kMassWaves = 4;
constexpr int kMassTiles = 8;  // 32-slot tiles per workgroup
constexpr int kMassMaxBlocks = 4096;  // row blocks a lane may have for the LDS skip flags

struct MassArgs {
    const uint16_t *pool;
    int64_t page_elems;
    int num_pages, P, H, G, Hq;
    const int32_t *page_indptr, *page_ids;
    const int32_t *indptr, *slots, *kv_len;
    const uint16_t *qrot;             // [N][Hq][D] rotated, prescaled bf16 (fp_attend's workspace)
    const float *lse;                 // [N][Hq] natural-log LSE from fp_attend
    const uint32_t *mask_bits;        // nullable
    const int64_t *mask_off;          // nullable
    float *mass;                      // [H][stride]
    int64_t stride;                   // page_indptr[L] * P
    int chunks;                       // chunks of the largest working set
    int L;                            // lanes
};

// Sum over the 32 lanes of each lane half, in registers: two quad swaps, the
// half-row and row mirrors (every lane of a 16-lane row then holds the row's
// sum), and one swap of 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float half_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D>
struct MassLds {
    static constexpr int KROW = 2 * D + 16;
    static constexpr int K_BYTES = 32 * kMassTiles * KROW;
};

template <int D>
__global__ void __launch_bounds__(64 * kMassWaves) mass_kernel(MassArgs a) {
    __shared__ __attribute__((aligned(16))) char s_k[MassLds<D>::K_BYTES];
    __shared__ float s_sum[kMassWaves][32 * kMassTiles];
    __shared__ uint8_t s_live[kMassMaxBlocks];  // row block may read a slot of the chunk
    constexpr int KROW = MassLds<D>::KROW;
    constexpr int KC = D / 8;  // 16-byte chunks per K row
    // Workgroups go to the XCDs round robin by launch index; index i runs on
    // XCD i % 8. Each XCD takes (lane, KV head) pairs x, x + 8, ... one after
    // the other with all their chunks, so the workgroups resident on an XCD
    // at one time mostly share one pair's Q, which then stays in that XCD's L2.
    const int xcd = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
    const int pair = kXcds * (kx / a.chunks) + xcd;
    if (pair >= a.L * a.H) return;
    const int lane = pair / a.H, g = pair % a.H;
    const int p0 = a.page_indptr[lane];
    const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
    const int eff = clamp_kv(a.kv_len[lane], cap);
    const int r0 = a.indptr[lane], n = a.indptr[lane + 1] - r0;
    const int c0 = 32 * kMassTiles * (kx % a.chunks);  // first slot of the chunk
    if (n <= 0 || n * a.G <= 32 || c0 >= eff) return;  // workgroup-uniform; decode-class lanes below
    const int ntl = min(kMassTiles, (eff - c0 + 31) >> 5);  // tiles of the chunk below kv_len
    const int wv = threadIdx.x / kWave, ln = lane_id(), nn = ln & 31, h = ln >> 5;
    const int pshift = __builtin_ctz(a.P);

    // Stage the chunk's K: page ids, then every data load, then every store,
    // all unconditional, so the workgroup waits for memory once (a condition
    // would let the compiler sink each load next to its store). Rows at or
    // past kv_len load the lane's last row below it again (a cache hit); their
    // scores are dropped.
    {
        constexpr int PER = 32 * kMassTiles * KC / (64 * kMassWaves);
        int pid[PER];
        uint4 stg[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int slot = min(c0 + (int)(threadIdx.x + u * 64 * kMassWaves) / KC, eff - 1);
            pid[u] = a.page_ids[p0 + (slot >> pshift)];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = threadIdx.x + u * 64 * kMassWaves;
            const int slot = min(c0 + e / KC, eff - 1), ck = e % KC;
            const int64_t phys = min(max(pid[u], 0), a.num_pages - 1);
            stg[u] = *reinterpret_cast<const uint4 *>(
                a.pool + phys * a.page_elems + ((int64_t)g * a.P + (slot & (a.P - 1))) * D + 8 * ck);
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = threadIdx.x + u * 64 * kMassWaves;
            *reinterpret_cast<uint4 *>(s_k + (e / KC) * KROW + 16 * (e % KC)) = stg[u];
        }
    }
    __syncthreads();

    const bool masked = a.mask_off && a.mask_off[lane + 1] > a.mask_off[lane];
    const int wpr = masked ? (int)((a.mask_off[lane + 1] - a.mask_off[lane]) / n) : 0;
    const int t0 = c0 >> 5;  // first tile of the chunk in the lane
    const int nrb = (n + 31) >> 5;
    const bool flags = nrb <= kMassMaxBlocks;  // workgroup-uniform; otherwise every pair is tried
    if (flags) {
        for (int b = threadIdx.x; b < nrb; b += 64 * kMassWaves) s_live[b] = 0;
        __syncthreads();
        const int rem = eff - c0;
        for (int r = threadIdx.x; r < n; r += 64 * kMassWaves) {
            bool live;
            if (masked) {
                const uint32_t *mw = a.mask_bits + a.mask_off[lane] + (int64_t)r * wpr;
                uint32_t any = 0u;
                for (int t = 0; t < ntl && t0 + t < wpr; ++t) {
                    const int q = rem - 32 * t;
                    any |= mw[t0 + t] & (q >= 32 ? 0xFFFFFFFFu : ((1u << q) - 1u));
                }
                live = any != 0u;
            } else {
                live = a.slots[r0 + r] + 1 > c0;
            }
            if (live) s_live[r >> 5] = 1;  // every writer stores the same value
        }
        __syncthreads();
    }
    const int items = ((n + 31) >> 5) * a.G;
    constexpr float kLog2e = 1.4426950408889634f;
    // Step s of the QK^T chain takes head-dimension elements 16s + 8kg ..
    // 16s + 8kg + 7 for lane group kg (= h) on both operands, so each Q load
    // instruction reads 32 contiguous bytes of every row it touches rather
    // than two 16-byte pieces half a row apart.
    const char *krow = s_k + kslot_of_row(nn) * KROW + 16 * h;

    float msum[kMassTiles][16];
#pragma unroll
    for (int t = 0; t < kMassTiles; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) msum[t][i] = 0.0f;

    for (int it = wv; it < items; it += kMassWaves) {
        const int rb = it / a.G, head = g * a.G + it % a.G;
        if (flags && !s_live[rb]) continue;  // workgroup-uniform
        const int rl = 32 * rb + nn;  // row within the lane (this lane's column)
        const bool valid = rl < n;
        const int64_t row = r0 + (valid ? rl : 0);
        const float lse2 = valid ? a.lse[row * a.Hq + head] * kLog2e : kNegInf;
        const bool live = valid && lse2 > kNegInf;
        // allowed slots of each tile of the chunk for this column
        uint32_t bits[kMassTiles];
        if (masked) {
            const uint32_t *mw = a.mask_bits + a.mask_off[lane] + (int64_t)(valid ? rl : 0) * wpr;
#pragma unroll
            for (int t = 0; t < kMassTiles; ++t) bits[t] = (live && t < ntl && t0 + t < wpr) ? mw[t0 + t] : 0u;
        } else {
            const int lim = live ? a.slots[row] + 1 - c0 : 0;  // causal: slots at or below the row's own
#pragma unroll
            for (int t = 0; t < kMassTiles; ++t) {
                const int r = lim - 32 * t;
                bits[t] = r >= 32 ? 0xFFFFFFFFu : (r <= 0 ? 0u : ((1u << r) - 1u));
            }
        }
        {
            const int rem = eff - c0;  // slots below kv_len from the chunk start
#pragma unroll
            for (int t = 0; t < kMassTiles; ++t) {
                const int r = rem - 32 * t;
                bits[t] &= r >= 32 ? 0xFFFFFFFFu : (r <= 0 ? 0u : ((1u << r) - 1u));
            }
        }
        uint32_t any = 0u;
#pragma unroll
        for (int t = 0; t < kMassTiles; ++t) any |= bits[t];
        if (!__any(any != 0u)) continue;  // wave-uniform
        uint4 qf[D / 16];
        {
            const uint16_t *qsrc = a.qrot + (row * a.Hq + head) * D + 8 * h;
#pragma unroll
            for (int s = 0; s < D / 16; ++s)  // row is clamped to the lane's first
                qf[s] = *reinterpret_cast<const uint4 *>(qsrc + 16 * s);
            if (!valid) {
#pragma unroll
                for (int s = 0; s < D / 16; ++s) qf[s] = make_uint4(0, 0, 0, 0);
            }
        }
        // -lse2 enters the accumulation as one more MFMA, its two bf16 terms
        // (hi + lo, 16 significant bits) in rows 0 and 1 of B against ones in
        // columns 0 and 1 of A, so no subtraction per score is needed
        uint4 bias_a, bias_b;
        {
            const float nl = live ? -lse2 : 0.0f;
            const uint32_t hi = pack_bf16x2(nl, nl) & 0xFFFFu;
            const float rest = nl - __uint_as_float(hi << 16);
            const uint32_t lo = pack_bf16x2(rest, rest) & 0xFFFFu;
            bias_a = make_uint4(h == 0 ? 0x3F803F80u : 0u, 0u, 0u, 0u);
            bias_b = make_uint4(h == 0 ? (hi | (lo << 16)) : 0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int t = 0; t < kMassTiles; ++t) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
                acc = mfma32(*reinterpret_cast<const uint4 *>(krow + t * 32 * KROW + 32 * s), qf[s], acc);
            acc = mfma32(bias_a, bias_b, acc);
            // register i holds tile slot 16(i/8) + 8h + i%8 of this column;
            // a dropped slot's weight is cleared by a sign-extended bit mask
            const uint32_t hb = bits[t] >> (8 * h);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = 16 * (i >> 3) + (i & 7);
                uint32_t keep;  // all ones if slot k is allowed (kept opaque: a select would take three instructions)
                asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(hb), "i"(k));
                msum[t][i] += __uint_as_float(__float_as_uint(__builtin_amdgcn_exp2f(acc[i])) & keep);
            }
        }
    }
    // sum the 32 columns of each lane half; lane (nn = 0, h) then holds the
    // wave's totals of its 16 slots of every tile
#pragma unroll
    for (int t = 0; t < kMassTiles; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float v = half_sum(msum[t][i]);
            if (nn == 0) s_sum[wv][32 * t + 16 * (i >> 3) + 8 * h + (i & 7)] = v;
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < 32 * ntl; j += 64 * kMassWaves) {
        if (c0 + j >= eff) continue;
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < kMassWaves; ++w) tot += s_sum[w][j];
        a.mass[(int64_t)g * a.stride + (int64_t)p0 * a.P + c0 + j] += tot;
    }
}

// Decode-class lanes (rows x G <= 32): all the lane's (row, query head)
// pairs fit in the 32 columns of one MFMA block, so each wave loads its Q
// once and streams kMassWaveTiles consecutive K tiles from memory (the next
// tile's K runs load while the current one computes),
// reducing each tile's 32 columns in registers and adding the 32 slot totals
// to the output (one writer per word). Column c is row c / G, query head
// g * G + c % G.
constexpr int kMassWaveTiles = 8;  // 2, 4, 8 and 16 measured: 8 (and 2) about 4 % faster than 4 on the decode wave

template <int D>
__global__ void __launch_bounds__(64 * kMassWaves) mass_decode_kernel(MassArgs a) {
    __shared__ __attribute__((aligned(16))) char s_k[kMassWaves][DecLds<D>::BYTES];
    const int lane = blockIdx.x / a.H, g = blockIdx.x % a.H;
    const int r0 = a.indptr[lane], n = a.indptr[lane + 1] - r0;
    if (n <= 0 || n * a.G > 32) return;  // workgroup-uniform; other lanes take the chunked kernel
    const int p0 = a.page_indptr[lane];
    const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
    const int eff = clamp_kv(a.kv_len[lane], cap);
    const int wv = threadIdx.x / kWave, ln = lane_id(), nn = ln & 31, h = ln >> 5;
    const int tb = kMassWaveTiles * (kMassWaves * blockIdx.y + wv);  // first tile of this wave
    if (32 * tb >= eff) return;  // wave-uniform: no barrier follows
    const int pshift = __builtin_ctz(a.P);
    const bool valid = nn < n * a.G;
    const int rl = valid ? nn / a.G : 0;
    const int64_t row = r0 + rl;
    const int head = g * a.G + (valid ? nn % a.G : 0);
    const float lse2 = valid ? a.lse[row * a.Hq + head] * 1.4426950408889634f : kNegInf;
    const bool live = valid && lse2 > kNegInf;
    const bool masked = a.mask_off && a.mask_off[lane + 1] > a.mask_off[lane];
    const int wpr = masked ? (int)((a.mask_off[lane + 1] - a.mask_off[lane]) / n) : 0;
    const int lim = a.slots[row] + 1;  // causal limit of this column's row
    const uint32_t *mwp = masked ? a.mask_bits + a.mask_off[lane] + (int64_t)rl * wpr
                                 : reinterpret_cast<const uint32_t *>(a.indptr);
    uint4 qf[D / 16];
    {
        const uint4 *qsrc = reinterpret_cast<const uint4 *>(a.qrot + (row * a.Hq + head) * D + h * (D / 2));
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[s] = qsrc[s];
        if (!valid) {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) qf[s] = make_uint4(0, 0, 0, 0);
        }
    }
    // K arrives as whole 1 KB runs of the pages (every load instruction covers
    // complete cache lines, like the decode kernel's K) and passes through the
    // wave's LDS buffer into the MFMA fragment layout: lane (n, h) then holds
    // tile row kslot_of_row(n), half h of the head dimension. Lane l keeps the
    // physical page of the tile's (l & 3)-th page; rows at or past kv_len read
    // the lane's last page (their scores are dropped).
    constexpr int RPR = 512 / D, LPR = D / 8;  // tile rows per run, lanes per row
    const int lastpg = (eff - 1) >> pshift;
    auto tile_kp = [&](int u) {
        const int pg = min((32 * (tb + u) >> pshift) + (ln & 3), lastpg);
        return min(max(a.page_ids[p0 + pg], 0), a.num_pages - 1);
    };
    const int64_t kcol = (int64_t)g * a.P * D + 8 * (ln % LPR);
    auto kload = [&](int kp, KvFrags<D> &f) {
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const int r = u * RPR + ln / LPR;
            const int64_t page = __builtin_amdgcn_readlane(kp, (u * RPR) >> pshift);
            f.k[u] = load_nt(a.pool + page * a.page_elems + kcol + (int64_t)(r & (a.P - 1)) * D);
        }
    };
    const uint32_t mm = masked ? 0xFFFFFFFFu : 0u;
    uint32_t mw_next = mwp[masked ? min(tb, wpr - 1) : 0];  // mask word of the wave's first tile
    int kp[2];
    kp[0] = tile_kp(0);
    kp[1] = tile_kp(min(1, kMassWaveTiles - 1));
    KvFrags<D> kb[2];
    kload(kp[0], kb[0]);
    kp[0] = tile_kp(min(2, kMassWaveTiles - 1));
#pragma unroll
    for (int u = 0; u < kMassWaveTiles; ++u) {
        const int j0 = 32 * (tb + u);
        if (j0 >= eff) break;  // wave-uniform
        if (u + 1 < kMassWaveTiles) {
            kload(kp[(u + 1) & 1], kb[(u + 1) & 1]);
            kp[(u + 1) & 1] = tile_kp(min(u + 3, kMassWaveTiles - 1));
        }
        uint4 kf[D / 16];
        stage_k<D, 32>(kb[u & 1], s_k[wv], kf);
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) acc = mfma32(kf[s], qf[s], acc);
        // allowed slots of the tile for this column: the row's mask word
        // (loaded a tile ahead) on masked lanes, the causal limit on the
        // others; both enter through masks so the word is used on every path
        // (a load used only behind a branch would be sunk into it and waited
        // for right there)
        const uint32_t mwv = mw_next;
        mw_next = mwp[masked ? min((j0 >> 5) + 1, wpr - 1) : 0];
        const int rl_ = lim - j0, rk = eff - j0;
        const uint32_t lm = rl_ >= 32 ? 0xFFFFFFFFu : (rl_ <= 0 ? 0u : ((1u << rl_) - 1u));
        const uint32_t km = rk >= 32 ? 0xFFFFFFFFu : ((1u << rk) - 1u);
        const uint32_t wm = (!masked || (j0 >> 5) < wpr) ? mwv : 0u;
        uint32_t bits = (wm | ~mm) & (lm | mm) & km;
        bits = live ? bits : 0u;
        // register i holds tile slot 16(i/8) + 8h + i%8 of this column
        const uint32_t hb = bits >> (8 * h);
        float mine = 0.0f;  // lane nn < 16 of half h keeps the total of register nn
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = 16 * (i >> 3) + (i & 7);
            const float p = ((hb >> k) & 1u) ? __builtin_amdgcn_exp2f(acc[i] - lse2) : 0.0f;
            const float tot = half_sum(p);
            mine = nn == i ? tot : mine;
        }
        if (nn < 16) {
            const int slot = j0 + 16 * (nn >> 3) + 8 * h + (nn & 7);
            if (slot < eff) a.mass[(int64_t)g * a.stride + (int64_t)p0 * a.P + slot] += mine;
        }
    }
}

}  // namespace fpk
