// fp_evict.h - score-driven KV eviction on the device (fp_tova_mask).
//
// The Docs' Attention masks section names attention-based eviction (TOVA) as
// something per-row bitmaps express, and the review's section 7 has the
// forward pass hand back the attention scores such a policy needs. This step
// closes the loop on the GPU: from the attention mass of earlier passes
// (fp_attn_mass) it picks, per lane, the old slots to keep and writes the next
// pass's row bitmaps, with no host round trip.
//
//  tova_select_kernel: one workgroup per lane. The score of old slot j (below
//    the lane's committed length) is the fp32 sum of its mass over the KV heads
//    in head order; scores compare by their total-order key (order_key). The
//    budget-th largest candidate key T is found by a radix select (four 8-bit
//    digits, most significant first, one LDS histogram per digit); the lane
//    then keeps every candidate above T and the lowest-slot candidates equal
//    to T until the budget is met, found with a block-wide scan in slot order.
//    The keys of a lane with up to kTovaLdsKeys old slots are computed once
//    into LDS (coalesced reads of the mass); a longer lane recomputes them from
//    the mass on every pass over its slots. Either way the step needs no workspace.
//  tova_rows_kernel: one workgroup per row of the pass, one thread per mask
//    word: kept old slots, plus the pass's own slots up to the row's slot.
#pragma once

#include "fp_kernels.h"

namespace fpk {

struct TovaArgs {
    const float *mass;  // [H][S]
    int64_t S;
    int H, P, L;
    const int32_t *page_indptr, *committed, *budget, *prev_limit;
    const uint32_t *prev_keep;
    const int64_t *keep_off;
    uint32_t *keep;
};

constexpr int kTovaThreads = kPlanThreads;  // the block scan below is written for this size
constexpr int kTovaLdsKeys = 32768;         // old slots whose keys a lane keeps in LDS (128 KiB)

// Total order of fp32 values as uint32 keys: negatives below positives, a
// positive-sign NaN above +inf.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Bits [0, n) of a word set, n clamped to [0, 32].
__device__ __forceinline__ uint32_t low_bits(int n) {
    return n <= 0 ? 0u : (n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u));
}

__global__ void __launch_bounds__(kTovaThreads) tova_select_kernel(TovaArgs a) {
    __shared__ uint32_t s_key[kTovaLdsKeys];
    __shared__ int s_hist[256];
    __shared__ int s_w[kTovaThreads / kWave];
    __shared__ int s_sel[2];  // digit found, remaining count
    const int l = blockIdx.x, tid = threadIdx.x;
    const int cap = (a.page_indptr[l + 1] - a.page_indptr[l]) * a.P;
    const int c = clamp_kv(a.committed[l], cap);
    const int64_t base = (int64_t)a.page_indptr[l] * a.P;
    const uint32_t *pk = a.prev_keep ? a.prev_keep + a.keep_off[l] : nullptr;
    const int plim = pk ? clamp_kv(a.prev_limit[l], c) : 0;
    uint32_t *kw = a.keep + a.keep_off[l];
    const int nwords = (c + 31) >> 5;
    // candidates of word w (slots 32w .. 32w+31 below c)
    auto cand_word = [&](int w) {
        const uint32_t inside = low_bits(c - 32 * w);
        if (!pk) return inside;
        const uint32_t fresh = ~low_bits(plim - 32 * w);  // at or past prev_limit
        return inside & (pk[w] | fresh);
    };
    auto key_of = [&](int j) {
        float s = 0.0f;
        for (int g = 0; g < a.H; ++g) s += a.mass[(int64_t)g * a.S + base + j];
        return order_key(s);
    };
    const bool in_lds = c <= kTovaLdsKeys;  // workgroup-uniform
    if (in_lds) {
#pragma unroll 4
        for (int j = tid; j < c; j += kTovaThreads) s_key[j] = key_of(j);
    }
    auto key_at = [&](int j) { return in_lds ? s_key[j] : key_of(j); };

    // candidates, and the budget clamped to them
    int nc = 0;
    for (int w = tid; w < nwords; w += kTovaThreads) nc += __popc(cand_word(w));
    int ncand;
    block_excl_scan(nc, s_w, &ncand);
    const int k = min(max(a.budget[l], 0), ncand);
    if (k == ncand || k == 0) {  // workgroup-uniform: every candidate or none
        for (int w = tid; w < nwords; w += kTovaThreads) kw[w] = k ? cand_word(w) : 0u;
        return;
    }

    // radix select of the k-th largest candidate key
    uint32_t prefix = 0, pmask = 0;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += kTovaThreads) s_hist[b] = 0;
        __syncthreads();
        for (int w = tid; w < nwords; w += kTovaThreads) {
            uint32_t cw = cand_word(w);
            while (cw) {
                const int b = __builtin_ctz(cw);
                cw &= cw - 1;
                const uint32_t key = key_at(32 * w + b);
                if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
            }
        }
        __syncthreads();
        if (tid == 0) {
            int acc = 0, d = 255;
            for (; d > 0; --d) {
                if (acc + s_hist[d] >= rem) break;
                acc += s_hist[d];
            }
            s_sel[0] = d;
            s_sel[1] = rem - acc;
        }
        __syncthreads();
        prefix |= (uint32_t)s_sel[0] << shift;
        pmask |= 255u << shift;
        rem = s_sel[1];
        __syncthreads();
    }
    // keep keys above the threshold, and the first `rem` equal ones in slot order
    const uint32_t T = prefix;
    int taken = 0;  // equal keys kept by earlier chunks of words
    for (int w0 = 0; w0 < nwords; w0 += kTovaThreads) {
        const int w = w0 + tid;
        uint32_t gt = 0, eq = 0;
        if (w < nwords) {
            uint32_t cw = cand_word(w);
            while (cw) {
                const int b = __builtin_ctz(cw);
                cw &= cw - 1;
                const uint32_t key = key_at(32 * w + b);
                gt |= (key > T ? 1u : 0u) << b;
                eq |= (key == T ? 1u : 0u) << b;
            }
        }
        int tot;
        const int before = taken + block_excl_scan(__popc(eq), s_w, &tot);
        int allow = min(max(rem - before, 0), __popc(eq));
        uint32_t kept = 0;
        while (allow > 0) {  // the lowest `allow` equal slots of the word
            const uint32_t lowest = eq & (~eq + 1u);
            kept |= lowest;
            eq ^= lowest;
            --allow;
        }
        if (w < nwords) kw[w] = gt | kept;
        taken += tot;
    }
}

struct TovaRowArgs {
    const int32_t *indptr, *slots, *kv_len, *committed, *page_indptr;
    int L, P;
    const uint32_t *keep;
    const int64_t *keep_off, *mask_off;
    uint32_t *mask;
    int32_t *status;
};

__global__ void __launch_bounds__(256) tova_rows_kernel(TovaRowArgs a) {
    const int64_t row = blockIdx.x;
    const int l = find_lane(a.indptr, a.L, row);
    const int r0 = a.indptr[l], n = a.indptr[l + 1] - r0;
    const int64_t span = a.mask_off[l + 1] - a.mask_off[l];
    if (span <= 0 || n <= 0) return;  // a lane without bitmap words keeps the causal rule
    const int wpr = (int)(span / n);
    const int cap = (a.page_indptr[l + 1] - a.page_indptr[l]) * a.P;
    const int c = clamp_kv(a.committed[l], cap);
    const int kv = clamp_kv(a.kv_len[l], cap);
    if ((int64_t)wpr * 32 < kv && threadIdx.x == 0 && row == r0) atomicOr(a.status, FP_ST_MASK_SHORT);
    const int lim = min(kv, a.slots[row] + 1);  // new slots up to the row's own
    const uint32_t *kw = a.keep + a.keep_off[l];
    uint32_t *out = a.mask + a.mask_off[l] + (int64_t)(row - r0) * wpr;
    const int kwords = (c + 31) >> 5;
    for (int w = threadIdx.x; w < wpr; w += blockDim.x) {
        const int j0 = 32 * w;
        const uint32_t old = low_bits(c - j0);
        const uint32_t kept = (w < kwords ? kw[w] : 0u) & old & low_bits(kv - j0);
        const uint32_t fresh = low_bits(lim - j0) & ~old;
        out[w] = kept | fresh;
    }
}

}  // namespace fpk
