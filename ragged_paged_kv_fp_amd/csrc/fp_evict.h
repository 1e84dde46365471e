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
//    digits, most significant first; per digit, each wave counts into its own
//    LDS histogram, since the keys of one lane crowd into few bins and shared
//    bins would serialise the atomics, and the copies are summed); the lane
//    then keeps every candidate above T and the lowest-slot candidates equal
//    to T until the budget is met, found with a block-wide scan in slot order.
//    The keys of a lane with up to kTovaLdsKeys old slots are computed once
//    into LDS (coalesced reads of the mass), and every pass over them sweeps
//    the slots with a stride of one per thread; a longer lane recomputes its
//    keys from the mass on every pass. Either way the step needs no workspace.
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

// Inclusive prefix sum over threads 0..255 of the workgroup (every thread of
// the workgroup calls it; threads from 256 on contribute 0).
__device__ __forceinline__ int scan256(int v, int *s_w) {
    const int ln = lane_id(), wv = threadIdx.x / kWave;
    int x = threadIdx.x < 256 ? v : 0;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (ln >= o) x += y;
    }
    if (ln == kWave - 1 && wv < 4) s_w[wv] = x;
    __syncthreads();
    for (int w = 0; w < 4; ++w) x += (w < wv && wv < 4) ? s_w[w] : 0;
    __syncthreads();
    return x;
}

__global__ void __launch_bounds__(kTovaThreads) tova_select_kernel(TovaArgs a) {
    constexpr int PER = kTovaLdsKeys / kTovaThreads;  // slots per thread on the LDS path
    constexpr int NW = kTovaLdsKeys / 32;
    __shared__ uint32_t s_key[kTovaLdsKeys];
    __shared__ uint32_t s_cw[NW];  // candidate words (LDS path)
    __shared__ uint32_t s_gw[NW];  // words of the kept keys above the threshold (LDS path)
    __shared__ int s_hist[kTovaThreads / kWave][256];
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
    // the sum over heads in head order; four heads' loads in flight at a time
    auto key_of = [&](int j) {
        const float *m = a.mass + base + j;
        float s = 0.0f;
        int g = 0;
        for (; g + 4 <= a.H; g += 4) {
            const float v0 = m[(int64_t)g * a.S], v1 = m[(int64_t)(g + 1) * a.S];
            const float v2 = m[(int64_t)(g + 2) * a.S], v3 = m[(int64_t)(g + 3) * a.S];
            s += v0;
            s += v1;
            s += v2;
            s += v3;
        }
        for (; g < a.H; ++g) s += m[(int64_t)g * a.S];
        return order_key(s);
    };
    // LDS path: thread tid owns slots tid + 1024 u, so every LDS access below
    // is a stride-1 sweep across the workgroup (no bank conflicts) and the
    // slots' loads are independent of each other
    const bool in_lds = c <= kTovaLdsKeys;  // workgroup-uniform
    if (in_lds) {
        float acc[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[u] = 0.0f;
        for (int g = 0; g < a.H; ++g) {
            const float *mg = a.mass + (int64_t)g * a.S + base;
            float v[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int j = tid + u * kTovaThreads;
                v[u] = j < c ? mg[j] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < PER; ++u) acc[u] += v[u];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int j = tid + u * kTovaThreads;
            if (j < c) s_key[j] = order_key(acc[u]);
        }
        for (int w = tid; w < nwords; w += kTovaThreads) s_cw[w] = cand_word(w);
    }
    auto cand_bit = [&](int j) { return (s_cw[j >> 5] >> (j & 31)) & 1u; };

    // candidates, and the budget clamped to them
    int nc = 0;
    for (int w = tid; w < nwords; w += kTovaThreads) nc += __popc(cand_word(w));
    int ncand;
    block_excl_scan(nc, s_w, &ncand);  // its barriers also publish the LDS keys and words
    const int k = min(max(a.budget[l], 0), ncand);
    if (k == ncand || k == 0) {  // workgroup-uniform: every candidate or none
        for (int w = tid; w < nwords; w += kTovaThreads) kw[w] = k ? cand_word(w) : 0u;
        return;
    }

    // radix select of the k-th largest candidate key
    uint32_t prefix = 0, pmask = 0;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = tid; b < (kTovaThreads / kWave) * 256; b += kTovaThreads) (&s_hist[0][0])[b] = 0;
        __syncthreads();
        int *hist = s_hist[tid / kWave];
        if (in_lds) {
            // Lanes whose keys share the digit add once: the masses of a lane
            // mostly share their sign and exponent, so in the first pass nearly
            // every lane of a wave hits one bin, and an atomic per lane would
            // serialise on it. A group of fewer than 8 lanes ends the
            // aggregation; the rest (diverse digits) add one by one.
#pragma unroll 4
            for (int u = 0; u < PER; ++u) {
                const int j = tid + u * kTovaThreads;
                bool has = false;
                uint32_t d = 0;
                if (j < c && cand_bit(j)) {
                    const uint32_t key = s_key[j];
                    has = (key & pmask) == prefix;
                    d = (key >> shift) & 255u;
                }
                uint64_t todo = __ballot(has);
                while (todo) {  // wave-uniform
                    const int leader = __builtin_ctzll(todo);
                    const uint32_t dl = __shfl(d, leader);
                    const uint64_t same = __ballot(has && d == dl) & todo;
                    if (__popcll(same) < 8) {
                        if (has && ((todo >> lane_id()) & 1ull)) atomicAdd(&hist[d], 1);
                        break;
                    }
                    if (lane_id() == leader) atomicAdd(&hist[dl], (int)__popcll(same));
                    todo &= ~same;
                }
            }
        } else {
            for (int w = tid; w < nwords; w += kTovaThreads) {
                uint32_t cw = cand_word(w);
                while (cw) {
                    const int b = __builtin_ctz(cw);
                    cw &= cw - 1;
                    const uint32_t key = key_of(32 * w + b);
                    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
                }
            }
        }
        __syncthreads();
        // digit d: thread 255 - d sums the wave copies of bin d; a scan over the
        // threads counts the keys of the digits above d and d itself
        int cnt = 0;
        if (tid < 256)
            for (int v = 0; v < kTovaThreads / kWave; ++v) cnt += s_hist[v][255 - tid];
        const int incl = scan256(cnt, s_w);
        if (tid < 256 && incl >= rem && incl - cnt < rem) {
            s_sel[0] = 255 - tid;
            s_sel[1] = rem - (incl - cnt);
        }
        __syncthreads();
        prefix |= (uint32_t)s_sel[0] << shift;
        pmask |= 255u << shift;
        rem = s_sel[1];
        __syncthreads();
    }
    // keep keys above the threshold, and the first `rem` equal ones in slot order
    const uint32_t T = prefix;
    if (in_lds) {
        // words of the keys above T and equal to T: the 32 slots of word
        // (tid >> 5) + 32 u sit in one half of a wave, so a ballot assembles them
        uint32_t *s_ew = reinterpret_cast<uint32_t *>(&s_hist[0][0]);
        const int wv = tid / kWave;
#pragma unroll 8
        for (int u = 0; u < PER; ++u) {
            const int j = tid + u * kTovaThreads;
            const bool cd = j < c && cand_bit(j);
            const uint32_t key = cd ? s_key[j] : 0u;
            const uint64_t bg = __ballot(cd && key > T), be = __ballot(cd && key == T);
            if (lane_id() == 0) {
                const int w = 2 * wv + 32 * u;
                s_gw[w] = (uint32_t)bg;
                s_gw[w + 1] = (uint32_t)(bg >> 32);
                s_ew[w] = (uint32_t)be;
                s_ew[w + 1] = (uint32_t)(be >> 32);
            }
        }
        __syncthreads();
        const uint32_t eq0 = tid < nwords ? s_ew[tid] : 0u;
        int tot;
        const int before = block_excl_scan(__popc(eq0), s_w, &tot);
        int allow = min(max(rem - before, 0), __popc(eq0));
        uint32_t eq = eq0, kept = 0;
        while (allow > 0) {  // the lowest `allow` equal slots of the word
            const uint32_t lowest = eq & (~eq + 1u);
            kept |= lowest;
            eq ^= lowest;
            --allow;
        }
        if (tid < nwords) kw[tid] = s_gw[tid] | kept;
        return;
    }
    int taken = 0;  // equal keys kept by earlier chunks of words
    for (int w0 = 0; w0 < nwords; w0 += kTovaThreads) {
        const int w = w0 + tid;
        uint32_t gt = 0, eq = 0;
        if (w < nwords) {
            uint32_t cw = cand_word(w);
            while (cw) {
                const int b = __builtin_ctz(cw);
                cw &= cw - 1;
                const uint32_t key = key_of(32 * w + b);
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
