// fp_lora.h - projection-site LoRA adapters: out = bf16(y + s_k * B_k (A_k x))
// for the rows of every lane whose adapter id k is set, in two launches.
//
// shrink: one workgroup of four waves per (lane, 32-row block). V^T = A_k X^T
//   on v_mfma_f32_32x32x16_bf16 (A_k rows as the A operand, the block's x rows
//   as the B operand), the d_in sum split over the four waves and reduced
//   through LDS; V (rank values per row) goes to the workspace as two bf16
//   terms, hi = bf16(v) and lo = bf16(v - hi), which carry 16 significant bits.
// expand: one workgroup of four waves per (lane, 32-row block, 128 output
//   columns). Out^T = B_k V^T (B_k rows as the A operand: contiguous rank
//   vectors; V rows as the B operand, hi and lo terms in two MFMAs); the
//   scaled products pass through LDS so that y is read and out written as
//   whole 256-byte row runs, y + s_k * (B_k v) in fp32 rounded to bf16.
// Lanes without an adapter keep y bit for bit (copied unless out is y).
// A plan kernel first lists the (lane, 32-row block) work items in the
// workspace, so both launches cover exactly the pass's row blocks.
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
    const int2 *items;             // workspace: (lane, row block) per work item, lane -1 past the list
    int n_items;                   // work items the host counted from its copy of indptr
    int32_t *status;
    bool in_place;
};

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return (uint16_t)(pack_bf16x2(f, f) & 0xFFFFu); }

constexpr int kLoraPlanThreads = 1024;

// One workgroup: items in lane order, a lane of n rows giving ceil(n/32)
// blocks. If the device offsets disagree with the host's count, the list is
// cut (or padded with lane -1) to the host's length and FP_ST_PLAN_MISMATCH set.
__global__ void __launch_bounds__(kLoraPlanThreads) lora_plan_kernel(const int32_t *indptr, int L, int2 *items,
                                                                       int n_items, int32_t *status) {
    __shared__ int s_tot[kLoraPlanThreads];
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
        for (int b = 0; b < cnt[u] && base + b < n_items; ++b) items[base + b] = make_int2(t * PER + u, b);
        base += cnt[u];
    }
    for (int i = total + t; i < n_items; i += kLoraPlanThreads) items[i] = make_int2(-1, 0);
    if (t == 0 && total != n_items) atomicOr(status, FP_ST_PLAN_MISMATCH);
}

template <int MB>
__global__ void __launch_bounds__(64 * kLoraWaves) lora_shrink_kernel(LoraArgs a) {
    __shared__ float s_part[kLoraWaves][MB][32][33];
    const int2 item = a.items[blockIdx.x];
    const int lane = item.x, rb = item.y;
    if (lane < 0) return;  // workgroup-uniform
    const int r0 = a.indptr[lane], n = a.indptr[lane + 1] - r0;
    if (32 * rb >= n) return;
    const int k = a.adapter[lane];
    if (k < 0 || k >= a.n_ad) return;  // the expand pass handles these lanes
    const int wv = threadIdx.x / kWave, ln = lane_id(), nn = ln & 31, h = ln >> 5;
    const int rowl = 32 * rb + nn;
    const bool rv = rowl < n;
    const uint16_t *xrow = a.x + (int64_t)(r0 + (rv ? rowl : 0)) * a.d_in + 8 * h;
    const uint16_t *arow[MB];
    bool av[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = 32 * mb + nn;
        av[mb] = m < a.r;
        arow[mb] = a.a + ((int64_t)k * a.r + (av[mb] ? m : 0)) * a.d_in + 8 * h;
    }
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
    const int steps = a.d_in / (16 * kLoraWaves);
    const int kb = wv * steps * 16;  // this wave's share of d_in
    // groups of four 16-wide steps in two register buffers: the next group's
    // loads are in flight while the current group's MFMAs run
    constexpr int GS = 4;
    struct Grp {
        uint4 x[GS], a[MB][GS];
    };
    auto load = [&](int g, Grp &b) {
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            const int kk = kb + 16 * (GS * g + j);
            b.x[j] = *reinterpret_cast<const uint4 *>(xrow + kk);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) b.a[mb][j] = *reinterpret_cast<const uint4 *>(arow[mb] + kk);
        }
    };
    auto compute = [&](const Grp &b) {
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            const uint4 xf = rv ? b.x[j] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32(av[mb] ? b.a[mb][j] : make_uint4(0, 0, 0, 0), xf, acc[mb]);
        }
    };
    const int groups = steps / GS;
    Grp b0, b1;
    int g = 0;
    if (groups > 0) load(0, b0);
    for (; g + 1 < groups; g += 2) {
        load(g + 1, b1);
        compute(b0);
        if (g + 2 < groups) load(g + 2, b0);
        compute(b1);
    }
    if (g < groups) compute(b0);
    for (int st = GS * groups; st < steps; ++st) {  // the last steps of a d_in that is not a multiple of 256
        const int kk = kb + 16 * st;
        const uint4 xf = rv ? *reinterpret_cast<const uint4 *>(xrow + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const uint4 af = *reinterpret_cast<const uint4 *>(arow[mb] + kk);
            acc[mb] = mfma32(av[mb] ? af : make_uint4(0, 0, 0, 0), xf, acc[mb]);
        }
    }
    // register i of lane (n, h) holds V^T[8(i/4) + 4h + i%4 (+32 mb)][n]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s_part[wv][mb][8 * (i >> 2) + 4 * h + (i & 3)][nn] = acc[mb][i];
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 32 * MB; e += 64 * kLoraWaves) {
        const int row = e / (32 * MB), m = e % (32 * MB);
        if (32 * rb + row >= n) continue;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kLoraWaves; ++w) sum += s_part[w][m >> 5][m & 31][row];
        const uint16_t hi = f32_to_bf16_bits(sum);
        const int64_t at = (int64_t)(r0 + 32 * rb + row) * a.rp + m;
        a.v[at] = hi;
        a.v[a.N * a.rp + at] = f32_to_bf16_bits(sum - __uint_as_float((uint32_t)hi << 16));
    }
}

__global__ void __launch_bounds__(64 * kLoraWaves) lora_expand_kernel(LoraArgs a) {
    __shared__ __attribute__((aligned(16))) float s_d[32][kLoraCols + 4];  // s_k * (B_k v), [row][column]
    const int2 item = a.items[blockIdx.x];
    const int lane = item.x, rb = item.y;
    if (lane < 0) return;  // workgroup-uniform
    const int r0 = a.indptr[lane], n = a.indptr[lane + 1] - r0;
    if (32 * rb >= n) return;
    const int k = a.adapter[lane];
    const bool bad = k >= a.n_ad;
    const bool none = k < 0 || bad;
    if (bad && blockIdx.y == 0 && rb == 0 && threadIdx.x == 0) atomicOr(a.status, FP_ST_ADAPTER);
    if (none && a.in_place) return;
    const int cw = kLoraCols * blockIdx.y;  // the workgroup's first output column
    if (!none) {
        const int wv = threadIdx.x / kWave, ln = lane_id(), nn = ln & 31, h = ln >> 5;
        const int c0 = cw + 32 * wv;  // this wave's 32 output columns
        const int rowl = 32 * rb + nn;
        const bool rv = rowl < n;
        const int64_t row = r0 + (rv ? rowl : 0);
        f32x16 acc = {};
        if (c0 < a.d_out) {  // wave-uniform
            const uint16_t *brow = a.b + ((int64_t)k * a.d_out + c0 + nn) * a.r + 8 * h;
            const uint16_t *vrow = a.v + row * a.rp + 8 * h;
            const int64_t lo = a.N * a.rp;
            for (int s = 0; s < a.r / 16; ++s) {
                const uint4 bf = *reinterpret_cast<const uint4 *>(brow + 16 * s);
                uint4 vh = *reinterpret_cast<const uint4 *>(vrow + 16 * s);
                uint4 vl = *reinterpret_cast<const uint4 *>(vrow + lo + 16 * s);
                if (!rv) vh = vl = make_uint4(0, 0, 0, 0);
                acc = mfma32(bf, vh, acc);
                acc = mfma32(bf, vl, acc);
            }
        }
        const float sc = a.scale[k];
        // register i of lane (n, h): column 8(i/4) + 4h + i%4 of row n
#pragma unroll
        for (int i = 0; i < 16; ++i) s_d[nn][32 * wv + 8 * (i >> 2) + 4 * h + (i & 3)] = sc * acc[i];
        __syncthreads();
    }
    // each thread: 16 consecutive columns of one row, so a row's 256 bytes
    // are read and written by eight neighbouring threads
    const int rr = threadIdx.x >> 3, cs = 16 * (threadIdx.x & 7);
    const int col = cw + cs;
    if (32 * rb + rr >= n || col >= a.d_out) return;
    const int64_t at = (int64_t)(r0 + 32 * rb + rr) * a.d_out + col;
    const uint4 y0 = *reinterpret_cast<const uint4 *>(a.y + at);
    const uint4 y1 = *reinterpret_cast<const uint4 *>(a.y + at + 8);
    if (none) {
        *reinterpret_cast<uint4 *>(a.out + at) = y0;
        *reinterpret_cast<uint4 *>(a.out + at + 8) = y1;
        return;
    }
    const float *d = &s_d[rr][cs];
    auto mix = [&](uint32_t w, int j) {  // two bf16 of y plus two deltas, rounded to bf16
        return pack_bf16x2(__uint_as_float(w << 16) + d[j], __uint_as_float(w & 0xFFFF0000u) + d[j + 1]);
    };
    *reinterpret_cast<uint4 *>(a.out + at) = make_uint4(mix(y0.x, 0), mix(y0.y, 2), mix(y0.z, 4), mix(y0.w, 6));
    *reinterpret_cast<uint4 *>(a.out + at + 8) =
        make_uint4(mix(y1.x, 8), mix(y1.y, 10), mix(y1.z, 12), mix(y1.w, 14));
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
