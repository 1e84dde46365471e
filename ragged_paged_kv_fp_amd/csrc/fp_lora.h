// fp_lora.h - projection-site LoRA adapters: out = bf16(y + s_k * B_k (A_k x))
// for the rows of every lane whose adapter id k is set, in two launches.
//
// shrink: one workgroup of four waves per (lane, 32-row block). V^T = A_k X^T
//   on v_mfma_f32_16x16x32_bf16 (16-row rank blocks of A_k as the A operand,
//   the block's x rows as two 16-row B operands), the d_in sum split over the
//   four waves and reduced through LDS; V (rank values per row) goes to the workspace as two bf16
//   terms, hi = bf16(v) and lo = bf16(v - hi), which carry 16 significant bits.
// expand: one workgroup of four waves per (lane, 32-row block, 512 output
//   columns). Out^T = B_k V^T (B_k rows as the A operand: contiguous rank
//   vectors; V rows as the B operand, hi and lo terms in two MFMAs); the
//   scaled products pass through LDS so that y is read and out written as
//   whole 256-byte row runs, y + s_k * (B_k v) in fp32 rounded to bf16.
// Lanes without an adapter keep y bit for bit (copied unless out is y).
// A plan kernel first lists the (lane, 32-row block) work items in the
// workspace with the block's first row, row count and adapter id, so both
// launches cover exactly the pass's row blocks and a workgroup needs one
// dependent load before its data loads.
#pragma once

#include "fp_kernels.h"

namespace fpk {

constexpr int kLoraWaves = 4;
constexpr int kLoraCols = 32 * kLoraWaves;  // output columns per expand workgroup

struct LoraArgs {
    const int32_t *indptr;
    int L;
    const int32_t *adapter;
    int n_ad, r, rp, d_in, d_out;  // rp: rank padded to a multiple of 32 (workspace row stride)
    const uint16_t *x, *y;
    uint16_t *out;
    const uint16_t *a, *b;
    const float *scale;
    uint16_t *v;                   // workspace bf16 [2][N][rp]: hi terms, then lo terms
    int64_t N;
    const int4 *items;             // workspace: (lane, first row, rows, adapter id) per work item, lane -1 past the list
    int n_items;                   // work items the host counted from its copy of indptr
    int32_t *status;
    bool in_place;
};

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return (uint16_t)(pack_bf16x2(f, f) & 0xFFFFu); }

constexpr int kLoraPlanThreads = 1024;

// One workgroup: items in lane order, a lane of n rows giving ceil(n/32)
// blocks. A saturating scan gives every lane its first item in LDS; then each
// thread writes items i, i + 1024, ... after finding the lane of item i by a
// binary search over those starts (so no thread writes a long lane's items
// one by one). If the device offsets disagree with the host's count, the list
// is cut (or padded with lane -1) to the host's length and
// FP_ST_PLAN_MISMATCH set.
__global__ void __launch_bounds__(kLoraPlanThreads) lora_plan_kernel(const int32_t *indptr, int L,
                                                                       const int32_t *adapter, int4 *items,
                                                                       int n_items, int32_t *status) {
    __shared__ int s_tot[kLoraPlanThreads];
    __shared__ int s_start[kMaxLanes];
    constexpr int PER = kMaxLanes / kLoraPlanThreads;  // lanes per thread
    const int t = threadIdx.x;
    int cnt[PER], mine = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int l = t * PER + u;
        const int n = l < L ? indptr[l + 1] - indptr[l] : 0;
        cnt[u] = n > 0 ? min((n + 31) >> 5, n_items) : 0;
        mine = min(mine + cnt[u], n_items);
    }
    // inclusive scan saturating at n_items: no sum can overflow and every
    // start below stays in [0, n_items]
    s_tot[t] = mine;
    __syncthreads();
    for (int off = 1; off < kLoraPlanThreads; off <<= 1) {
        const int v = t >= off ? s_tot[t - off] : 0;
        __syncthreads();
        s_tot[t] = min(s_tot[t] + v, n_items);
        __syncthreads();
    }
    int base = s_tot[t] - mine;
    const int total = s_tot[kLoraPlanThreads - 1];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        s_start[t * PER + u] = base;
        base = min(base + cnt[u], n_items);
    }
    __syncthreads();
    // the lane of item i < total is the last lane starting at or before i
    // (an empty lane starts where the next one does, so it is never the last)
    for (int i = t; i < n_items; i += kLoraPlanThreads) {
        if (i >= total) {
            items[i] = make_int4(-1, 0, 0, -1);
            continue;
        }
        int lo = 0, hi = L - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_start[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const int r0 = indptr[lo], row0 = r0 + 32 * (i - s_start[lo]);
        items[i] = make_int4(lo, row0, min(32, indptr[lo + 1] - row0), adapter[lo]);
    }
    if (t == 0 && total != n_items) atomicOr(status, FP_ST_PLAN_MISMATCH);
}

// Shrink: V^T = A_k X^T on v_mfma_f32_16x16x32_bf16, one 16-row rank block of
// A_k per MFMA A operand (every lane of the operand holds a real rank row, so
// no load is spent on padding) and the block's x rows as two 16-row B
// operands; each load instruction reads 64 contiguous bytes of 16 rows. RB is
// the rank in blocks of 16.
template <int RB>
__global__ void __launch_bounds__(64 * kLoraWaves) lora_shrink_kernel(LoraArgs a) {
    __shared__ float s_part[kLoraWaves][16 * RB][33];
    const int4 item = a.items[blockIdx.x];
    const int row0 = item.y, nr = item.z, k = item.w;
    if (item.x < 0 || nr <= 0) return;  // workgroup-uniform
    if (k < 0 || k >= a.n_ad) return;   // the expand pass handles these lanes
    const int wv = threadIdx.x / kWave, ln = lane_id(), n16 = ln & 15, kg = ln >> 4;
    // B operands: rows n16 and 16 + n16 of the block (rows past it repeat the
    // block's last row; their V columns are never stored); A operands: rank
    // rows 16 rb + n16. Lane group kg holds the 8 columns at 8 kg of a 32-wide step.
    const uint16_t *xrow[2];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) xrow[rh] = a.x + (int64_t)(row0 + min(16 * rh + n16, nr - 1)) * a.d_in + 8 * kg;
    const uint16_t *arow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) arow[rb] = a.a + ((int64_t)k * a.r + 16 * rb + n16) * a.d_in + 8 * kg;
    f32x4 acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] = acc[rb][1] = f32x4{};
    // pairs of 32-wide steps (64 columns: one 128-byte line of each row) dealt
    // round robin: wave wv takes pairs wv, wv + 4, ..., so each line of x is
    // read whole by one wave in two consecutive loads
    const int steps = 2 * max(0, (a.d_in / 64 - wv + kLoraWaves - 1) / kLoraWaves);
    auto col = [&](int st) { return 64 * (wv + kLoraWaves * (st >> 1)) + 32 * (st & 1); };
    // groups of GS 32-wide steps in a ring of NB register buffers: NB - 1
    // groups' loads are in flight while a group's MFMAs run (every load is
    // unconditional, the group index clamped to the last, so the compiler
    // counts outstanding loads exactly)
    constexpr int GS = 2, NB = RB <= 2 ? 4 : 3;  // fewer buffers for the larger ranks (registers)
    struct Grp {
        uint4 x[GS][2], a[GS][RB];
    };
    auto load = [&](int g, Grp &b) {
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            const int kk = col(GS * g + j);
#pragma unroll
            for (int rh = 0; rh < 2; ++rh) b.x[j][rh] = *reinterpret_cast<const uint4 *>(xrow[rh] + kk);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) b.a[j][rb] = *reinterpret_cast<const uint4 *>(arow[rb] + kk);
        }
    };
    auto compute = [&](const Grp &b) {
#pragma unroll
        for (int j = 0; j < GS; ++j)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int rh = 0; rh < 2; ++rh) acc[rb][rh] = mfma16(b.a[j][rb], b.x[j][rh], acc[rb][rh]);
    };
    const int groups = steps / GS;
    if (groups > 0) {  // workgroup-uniform
        // the scheduling barriers keep the groups' loads in issue order, so
        // the wait before a group's MFMAs leaves the later groups in flight
        Grp b[NB];
#pragma unroll
        for (int u = 0; u < NB - 1; ++u) {
            load(min(u, groups - 1), b[u]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int g = 0; g < groups; g += NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                load(min(g + u + NB - 1, groups - 1), b[(u + NB - 1) % NB]);
                __builtin_amdgcn_sched_barrier(0);
                if (g + u < groups) compute(b[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    for (int st = GS * groups; st < steps; ++st) {  // a step left over from the groups (none while GS is 2)
        Grp t;
        const int kk = col(st);
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) t.x[0][rh] = *reinterpret_cast<const uint4 *>(xrow[rh] + kk);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) t.a[0][rb] = *reinterpret_cast<const uint4 *>(arow[rb] + kk);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int rh = 0; rh < 2; ++rh) acc[rb][rh] = mfma16(t.a[0][rb], t.x[0][rh], acc[rb][rh]);
    }
    // register i of lane (n16, kg) holds V^T[16 rb + 4 kg + i][16 rh + n16]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int rh = 0; rh < 2; ++rh)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_part[wv][16 * rb + 4 * kg + i][16 * rh + n16] = acc[rb][rh][i];
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 16 * RB; e += 64 * kLoraWaves) {
        const int row = e / (16 * RB), m = e % (16 * RB);
        if (row >= nr) continue;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kLoraWaves; ++w) sum += s_part[w][m][row];
        const uint16_t hi = f32_to_bf16_bits(sum);
        const int64_t at = (int64_t)(row0 + row) * a.rp + m;
        a.v[at] = hi;
        a.v[a.N * a.rp + at] = f32_to_bf16_bits(sum - __uint_as_float((uint32_t)hi << 16));
    }
}

// Expand: one workgroup per (item, kLoraBlocks blocks of 128 output
// columns). Every load of the workgroup (V's hi and lo terms once, then y and
// the B_k rows of all its column blocks) is issued before the first MFMA, so
// the workgroup waits for memory about once; the blocks then go through the
// LDS transpose one after the other. RS is the rank in 16-wide steps.
constexpr int kLoraBlocks = 4;

template <int RS>
__global__ void __launch_bounds__(64 * kLoraWaves) lora_expand_kernel(LoraArgs a) {
    __shared__ __attribute__((aligned(16))) float s_d[32][kLoraCols + 4];  // s_k * (B_k v), [row][column]
    const int4 item = a.items[blockIdx.x];
    const int row0 = item.y, nr = item.z, k = item.w;
    if (item.x < 0 || nr <= 0) return;  // workgroup-uniform
    const bool bad = k >= a.n_ad;
    const bool none = k < 0 || bad;
    if (bad && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(a.status, FP_ST_ADAPTER);
    if (none && a.in_place) return;
    const int cw = kLoraCols * kLoraBlocks * blockIdx.y;  // the workgroup's first output column
    // each thread: 16 consecutive columns of one row per block, so a row's
    // 256 bytes are read and written by eight neighbouring threads (loads
    // from a valid row and column even where nothing is written)
    const int rr = threadIdx.x >> 3, cs = 16 * (threadIdx.x & 7);
    const bool rok = rr < nr;
    uint4 y[kLoraBlocks][2];
#pragma unroll
    for (int cb = 0; cb < kLoraBlocks; ++cb) {
        const int col = cw + kLoraCols * cb + cs;
        const int64_t at = (int64_t)(row0 + (rok ? rr : 0)) * a.d_out + (col < a.d_out ? col : 0);
        y[cb][0] = *reinterpret_cast<const uint4 *>(a.y + at);
        y[cb][1] = *reinterpret_cast<const uint4 *>(a.y + at + 8);
    }
    const int wv = threadIdx.x / kWave, ln = lane_id(), nn = ln & 31, h = ln >> 5;
    uint4 vh[RS], vl[RS], bf[kLoraBlocks][RS];
    float sc = 0.0f;
    if (!none) {  // workgroup-uniform
        const bool rv = nn < nr;
        const uint16_t *vrow = a.v + (int64_t)(row0 + (rv ? nn : 0)) * a.rp + 8 * h;
        const uint32_t vm = rv ? 0xFFFFFFFFu : 0u;  // rows past the block enter as zeros
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const uint4 hv = *reinterpret_cast<const uint4 *>(vrow + 16 * s);
            const uint4 lv = *reinterpret_cast<const uint4 *>(vrow + a.N * a.rp + 16 * s);
            vh[s] = make_uint4(hv.x & vm, hv.y & vm, hv.z & vm, hv.w & vm);
            vl[s] = make_uint4(lv.x & vm, lv.y & vm, lv.z & vm, lv.w & vm);
        }
#pragma unroll
        for (int cb = 0; cb < kLoraBlocks; ++cb) {
            const int c = min(cw + kLoraCols * cb + 32 * wv + nn, a.d_out - 1);  // this lane's B_k row
            const uint16_t *brow = a.b + ((int64_t)k * a.d_out + c) * a.r + 8 * h;
#pragma unroll
            for (int s = 0; s < RS; ++s) bf[cb][s] = *reinterpret_cast<const uint4 *>(brow + 16 * s);
        }
        sc = a.scale[k];
    }
#pragma unroll
    for (int cb = 0; cb < kLoraBlocks; ++cb) {
        const int cbw = cw + kLoraCols * cb;  // the block's first column
        if (cbw >= a.d_out) break;          // workgroup-uniform
        if (!none) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < RS; ++s) {
                acc = mfma32(bf[cb][s], vh[s], acc);
                acc = mfma32(bf[cb][s], vl[s], acc);
            }
            if (cb > 0) __syncthreads();  // the previous block's reads of s_d are done
            // register i of lane (n, h): column 8(i/4) + 4h + i%4 of row n
#pragma unroll
            for (int i = 0; i < 16; ++i) s_d[nn][32 * wv + 8 * (i >> 2) + 4 * h + (i & 3)] = sc * acc[i];
            __syncthreads();
        }
        const int col = cbw + cs;
        if (!rok || col >= a.d_out) continue;
        const int64_t at = (int64_t)(row0 + rr) * a.d_out + col;
        if (none) {
            *reinterpret_cast<uint4 *>(a.out + at) = y[cb][0];
            *reinterpret_cast<uint4 *>(a.out + at + 8) = y[cb][1];
            continue;
        }
        const float *d = &s_d[rr][cs];
        auto mix = [&](uint32_t w, int j) {  // two bf16 of y plus two deltas, rounded to bf16
            return pack_bf16x2(__uint_as_float(w << 16) + d[j], __uint_as_float(w & 0xFFFF0000u) + d[j + 1]);
        };
        const uint4 y0 = y[cb][0], y1 = y[cb][1];
        *reinterpret_cast<uint4 *>(a.out + at) = make_uint4(mix(y0.x, 0), mix(y0.y, 2), mix(y0.z, 4), mix(y0.w, 6));
        *reinterpret_cast<uint4 *>(a.out + at + 8) =
            make_uint4(mix(y1.x, 8), mix(y1.y, 10), mix(y1.z, 12), mix(y1.w, 14));
    }
}

// IA3: one workgroup per row (its lane found once, from uniform addresses),
// each thread taking 8 output columns per round; y * scale in fp32 is exact,
// so one rounding to bf16.
constexpr int kIa3Threads = 256;

__global__ void __launch_bounds__(kIa3Threads) ia3_kernel(const int32_t *indptr, int L, const int32_t *adapter, int n_ad,
                                                          int d_out, const uint16_t *scale, const uint16_t *y,
                                                          uint16_t *out, int32_t *status) {
    const int64_t row = blockIdx.x;
    const int lane = find_lane(indptr, L, row);
    const int k = adapter[lane];
    const bool none = k < 0 || k >= n_ad;
    if (k >= n_ad && threadIdx.x == 0 && row == indptr[lane]) atomicOr(status, FP_ST_ADAPTER);
    if (none && out == y) return;  // workgroup-uniform
    auto mul = [](uint32_t a, uint32_t b) {
        return pack_bf16x2(__uint_as_float(a << 16) * __uint_as_float(b << 16),
                           __uint_as_float(a & 0xFFFF0000u) * __uint_as_float(b & 0xFFFF0000u));
    };
    const uint16_t *yr = y + row * d_out;
    uint16_t *orow = out + row * d_out;
    const uint16_t *sr = scale + (int64_t)(none ? 0 : k) * d_out;
    for (int c = 8 * threadIdx.x; c < d_out; c += 8 * kIa3Threads) {
        const uint4 yv = *reinterpret_cast<const uint4 *>(yr + c);
        if (none) {
            *reinterpret_cast<uint4 *>(orow + c) = yv;
            continue;
        }
        const uint4 sv = *reinterpret_cast<const uint4 *>(sr + c);
        *reinterpret_cast<uint4 *>(orow + c) =
            make_uint4(mul(yv.x, sv.x), mul(yv.y, sv.y), mul(yv.z, sv.z), mul(yv.w, sv.w));
    }
}

}  // namespace fpk
