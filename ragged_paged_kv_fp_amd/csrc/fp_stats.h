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
// One workgroup of four waves per (lane, KV head, 32-slot tile): the tile's K
// stays in registers as the A operand of S^T = K * Q^T (the prefill kernel's
// slot permutation, so lane half h holds slots 8h..8h+7 and 16+8h..16+8h+7 of
// its column), and the waves stream the lane's (32-row block, query head)
// pairs, accumulating p per slot in registers. A pair with no allowed slot in
// the tile is skipped by the whole wave. The 32 columns of a wave are summed
// with butterfly shuffles, the four waves through LDS, and one thread per
// slot adds the total to the output: a single owner per output word, so the
// result does not depend on scheduling.
#pragma once

#include "fp_kernels.h"

namespace fpk {

constexpr int kMassWaves = 4;

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
    int tiles;                        // 32-slot tiles of the largest working set
};

template <int D>
__global__ void __launch_bounds__(64 * kMassWaves) mass_kernel(MassArgs a) {
    __shared__ float s_sum[kMassWaves][32];
    const int lane = blockIdx.x / a.H, g = blockIdx.x % a.H;
    const int p0 = a.page_indptr[lane];
    const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
    const int eff = clamp_kv(a.kv_len[lane], cap);
    const int r0 = a.indptr[lane], n = a.indptr[lane + 1] - r0;
    if (n <= 0 || eff <= 0) return;  // workgroup-uniform
    const int wv = threadIdx.x / kWave, ln = lane_id(), nn = ln & 31, h = ln >> 5;
    const int pshift = __builtin_ctz(a.P);
    const int lastpg = (eff - 1) >> pshift;
    const bool masked = a.mask_off && a.mask_off[lane + 1] > a.mask_off[lane];
    const int wpr = masked ? (int)((a.mask_off[lane + 1] - a.mask_off[lane]) / n) : 0;
    const int nrb = (n + 31) >> 5;
    const int items = nrb * a.G;
    constexpr float kLog2e = 1.4426950408889634f;

    for (int t = blockIdx.y; t < a.tiles; t += gridDim.y) {
        const int j0 = 32 * t;
        if (j0 >= eff) break;  // workgroup-uniform
        // K rows of the tile as the A operand; slots past the working set read
        // the last page that holds a slot below kv_len (their scores are dropped)
        uint4 kf[D / 16];
        {
            const int srow = j0 + kslot_of_row(nn);
            const int pg = min(srow >> pshift, lastpg);
            const int64_t phys = min(max(a.page_ids[p0 + pg], 0), a.num_pages - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(
                a.pool + phys * a.page_elems + ((int64_t)g * a.P + (srow & (a.P - 1))) * D + h * (D / 2));
#pragma unroll
            for (int s = 0; s < D / 16; ++s) kf[s] = src[s];
        }
        float msum[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) msum[i] = 0.0f;

        for (int it = wv; it < items; it += kMassWaves) {
            const int rb = it / a.G, head = g * a.G + it % a.G;
            const int rl = 32 * rb + nn;  // row within the lane (the lane's column)
            const bool valid = rl < n;
            const int64_t row = r0 + (valid ? rl : 0);
            const float lse2 = valid ? a.lse[row * a.Hq + head] * kLog2e : kNegInf;
            // slots of the tile this column may read, as a 32-bit mask
            uint32_t bits = 0u;
            if (valid && lse2 > kNegInf) {
                const int rem = eff - j0;
                uint32_t lm = rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
                if (masked) {
                    bits = t < wpr ? a.mask_bits[a.mask_off[lane] + (int64_t)rl * wpr + t] : 0u;
                } else {
                    const int lim = a.slots[row] + 1 - j0;  // causal: slots at or below the row's own
                    bits = lim >= 32 ? 0xFFFFFFFFu : (lim <= 0 ? 0u : ((1u << lim) - 1u));
                }
                bits &= lm;
            }
            if (!__any(bits != 0u)) continue;  // wave-uniform
            const uint4 *qsrc = reinterpret_cast<const uint4 *>(a.qrot + (row * a.Hq + head) * D + h * (D / 2));
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < D / 16; ++s) acc = mfma32(kf[s], valid ? qsrc[s] : make_uint4(0, 0, 0, 0), acc);
            // register i holds tile slot 16(i/8) + 8h + i%8 of this column
            const uint32_t hb = bits >> (8 * h);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = 16 * (i >> 3) + (i & 7);
                const bool keep = (hb >> k) & 1u;
                msum[i] += keep ? __builtin_amdgcn_exp2f(acc[i] - lse2) : 0.0f;
            }
        }
        // sum the 32 columns of each lane half: lane (nn = 0, h) then holds
        // the wave's totals of its 16 slots
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v = msum[i];
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off);
            msum[i] = v;
        }
        if (nn == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s_sum[wv][16 * (i >> 3) + 8 * h + (i & 7)] = msum[i];
        }
        __syncthreads();
        if (threadIdx.x < 32 && j0 + (int)threadIdx.x < eff) {
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < kMassWaves; ++w) tot += s_sum[w][threadIdx.x];
            float *dst = a.mass + (int64_t)g * a.stride + (int64_t)p0 * a.P + j0 + threadIdx.x;
            *dst += tot;
        }
        __syncthreads();
    }
}

}  // namespace fpk
