// fp_kernels.h - HIP kernels of the ForwardPass attention step (gfx950).
//
// Pool page layout (bf16): K block [H][P][D] then V block [H][D][P] (V transposed),
// so that both MFMA operands of S^T = K*Q^T and O^T = V^T*P^T load as 16-byte
// vectors straight from the page, with no LDS transpose.
#pragma once

#include "fp_device.h"
#include "../../include/fp.h"

namespace fpk {

// Per-lane plan record written by the plan (plan_kernel).
struct LaneInfo {
    int dec_off;   // first decode work item of the lane, -1 if the lane is not a decode lane
    int nsplit;    // decode KV splits of the lane (items per KV head)
    int sum_off;     // first word of the lane's tile lists, -1 if the lane has none
    int sum_stride;  // words per row-block tile list: a count, then one entry per KV tile
};

// ============================================================================ append

__device__ __forceinline__ void rotate_pair_f64(double x0, double x1, double c, double s, double *y0, double *y1) {
#pragma clang fp contract(off)
    *y0 = x0 * c - x1 * s;
    *y1 = x0 * s + x1 * c;
}

struct AppendArgs {
    uint16_t *pool;
    int64_t page_elems;
    int num_pages, P, H;
    const int32_t *page_indptr, *page_ids, *committed;
    const int32_t *indptr;
    int L;
    int64_t N;
    const int32_t *positions, *slots;
    const uint16_t *k, *v;
    int32_t *status;
    int rshift;  // log2 of the rows per workgroup (<= kAppendRows)
    RopeFreqs freqs;
};

constexpr int kAppendRows = 16;        // most consecutive rows one append workgroup writes
constexpr int kBatch = 8;              // 16-byte loads a thread of the row kernels issues before using them
constexpr int kAppendVBytes = 16640;   // LDS staging V: 16 rows x (4 heads x 128 dims + 8 padding) bf16

// log2 of the rows per workgroup of the row-grouped kernels (append, Q
// rotation): many rows share a workgroup when there are enough rows to fill
// the chip, one row per workgroup for a short pass.
__host__ __forceinline__ int row_group_shift(int64_t N, int max_rows) {
    int s = 0;
    while ((1 << s) < max_rows && N / (2LL << s) >= 1024) ++s;
    return s;
}

// One 16-byte chunk of a head row (four RoPE pairs) rotated in fp64 by the
// pairs' (cos, sin) and rounded once to nearest-even bf16.
__device__ __forceinline__ uint4 rotate_chunk(uint4 x, const double2 *cs) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        double y0, y1;
        rotate_pair_f64((double)bf16_lo(w[q]), (double)bf16_hi(w[q]), cs[q].x, cs[q].y, &y0, &y1);
        w[q] = f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One 16-byte chunk of a query row (four RoPE pairs) rotated in fp32 by the
// pairs' prescaled (cos, sin) and rounded to nearest-even bf16. The query is
// rounded to bf16 for the MFMA in any case; fp32 changes that rounding only
// where the fp64 product lies within a few fp32 ulps of a bf16 rounding
// boundary, and then by one bf16 ulp.
__device__ __forceinline__ uint4 rotate_chunk_f32(uint4 x, const float2 *cs) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float x0 = bf16_lo(w[q]), x1 = bf16_hi(w[q]);
        const float2 r = cs[q];
        w[q] = pack_bf16x2(fmaf(x0, r.x, -x1 * r.y), fmaf(x0, r.y, x1 * r.x));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One workgroup per 2^rshift consecutive rows. Workgroups are dealt to the 8
// XCDs in turn, so block b takes row group (b mod 8) * ceil-share + b / 8:
// each XCD gets a contiguous run of groups, and neighbouring groups, which
// write the two halves of V^T rows when a page holds more slots than a group
// has rows, merge their writes in one L2 instead of sending two partial
// writes of each line to HBM.
//  1. Side by side: wave 0 validates the rows (lane, slot, freeze, page),
//     finding the lanes of the group's first and last rows with a 32-way
//     search per half wave (one round of loads per factor of 32 lanes) and
//     each row's lane between those two; the other waves put the fp64
//     (cos, sin) of every (row, RoPE pair) in LDS, shared by the row's KV
//     heads. (Issuing the first K and V loads before this was slower.)
//  2. K: one thread per 16-byte chunk (four pairs) of a (row, head) row, chunk
//     index fastest, so a wave reads and writes whole 256-byte head rows.
//  3. V goes through LDS a group of heads at a time (16-byte loads), rows
//     padded by 16 bytes, then is stored into the V^T block. Eight rows at
//     consecutive slots filling an aligned 8-slot segment of one page (most
//     of a prefill chunk) are a full segment: per (head, dim) column a thread
//     gathers its eight values from LDS and writes them with one 16-byte
//     store. The other rows (decode rows, chunk ends, scattered slots) are
//     stored per element with the row index fastest, so a wave's 2-byte
//     stores still cover consecutive bytes of V^T rows.
template <int D>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
    constexpr int PAIRS = D / 2, C8 = D / 8, CSH = D == 128 ? 4 : 3;
    __shared__ int64_t s_base[kAppendRows];  // element offset of the row's page, -1: row not written
    __shared__ int s_off[kAppendRows];
    // The angle table serves the K rotation and the V staging buffer the V
    // transpose after it (a barrier between), so they share LDS: at about
    // 17 KB a workgroup, enough workgroups stay resident per compute unit for
    // a 20,000-row pass to run in one round.
    constexpr int kCsBytes = kAppendRows * PAIRS * (int)sizeof(double2);
    __shared__ __attribute__((aligned(16))) char s_u[kCsBytes > kAppendVBytes ? kCsBytes : kAppendVBytes];
    double2 *s_cs = reinterpret_cast<double2 *>(s_u);
    uint16_t *s_v = reinterpret_cast<uint16_t *>(s_u);
    __shared__ int s_seg[kAppendRows / 8];  // first row of each full segment
    __shared__ int s_erow[kAppendRows];     // rows stored per element
    __shared__ int s_nseg, s_nerow;
    const int R = 1 << a.rshift;
    const int nb = gridDim.x, per = nb >> 3, rem = nb & 7, xcd = blockIdx.x & 7;
    const int grp = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (blockIdx.x >> 3);
    const int64_t r0 = (int64_t)grp << a.rshift;
    const int nr = (int)(a.N - r0 < R ? a.N - r0 : R);
    const int tid = threadIdx.x;
    const int H = a.H;
    const int nk = nr * H * C8;                                          // K chunks
    const int hg = max(1, min(H, (kAppendVBytes / 2 - 8 * R) / (R * D)));  // V heads per round
    // 16-byte chunks of K (e < nk) and of V's head round h0 (e < nr * hn * C8), kBatch per thread
    auto load_k = [&](int e0, uint4 (&x)[kBatch]) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + 256 * u;
            const int rh = e >> CSH;  // (row - r0) * H + head: the row's K rows are contiguous
            x[u] = e < nk ? *reinterpret_cast<const uint4 *>(a.k + (r0 * H + rh) * D + 8 * (e & (C8 - 1)))
                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_v = [&](int e0, int h0, int hn, uint4 (&x)[kBatch]) {
        const int nv = nr * hn * C8;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + 256 * u;
            const int c = e & (C8 - 1), rh = e >> CSH;
            const int j = rh / hn, hh = rh - j * hn;
            x[u] = e < nv ? *reinterpret_cast<const uint4 *>(a.v + (r0 + j) * H * D + (int64_t)(h0 + hh) * D + 8 * c)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    if (tid < kWave) {
        // lanes of the group's first row (half wave 0) and last row (half wave 1):
        // largest lane l with indptr[l] <= row, probing 32 evenly spaced lanes
        // of the remaining range per round (the probes that hold are a prefix)
        const int half = tid >> 5, q = tid & 31;
        const int64_t target = half ? r0 + nr - 1 : r0;
        const int slot = tid < nr ? a.slots[r0 + tid] : 0;
        int lo = 0, hi = a.L;  // answer in [lo, hi)
        while (__ballot(hi - lo > 1)) {
            const bool busy = hi - lo > 1;
            const int step = (hi - lo + 31) >> 5;
            const int pr = lo + q * step;
            const uint64_t b = __ballot(busy && pr < hi && (int64_t)a.indptr[pr] <= target);
            if (busy) {
                // the probe at lo holds when indptr is ordered; at least 1 keeps
                // [lo, hi) inside the lanes whatever the device copy holds
                const int k = max(1, __popc(half ? (uint32_t)(b >> 32) : (uint32_t)b));
                hi = min(hi, lo + k * step);
                lo += (k - 1) * step;
            }
        }
        const int lane_first = __builtin_amdgcn_readlane(lo, 0), lane_last = __builtin_amdgcn_readlane(lo, 32);
        int64_t base = -1;
        int off = 0;
        if (tid < nr) {
            const int64_t row = r0 + tid;
            int l0 = lane_first, l1 = lane_last + 1;  // the row's lane lies in [l0, l1)
            while (l1 - l0 > 1) {
                const int mid = (l0 + l1) >> 1;
                if ((int64_t)a.indptr[mid] <= row) l0 = mid; else l1 = mid;
            }
            const int lane = l0;
            const int p0 = a.page_indptr[lane];
            const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
            if (slot < 0 || slot >= cap) {
                atomicOr(a.status, FP_ST_SLOT_RANGE);
            } else if (slot < a.committed[lane]) {
                atomicOr(a.status, FP_ST_FROZEN);
            } else {
                const int64_t page = a.page_ids[p0 + slot / a.P];
                if (page < 0 || page >= a.num_pages) {
                    atomicOr(a.status, FP_ST_PAGE_RANGE);
                } else {
                    base = page * a.page_elems;
                    off = slot % a.P;
                }
            }
        }
        if (tid < kAppendRows) {
            s_base[tid] = base;
            s_off[tid] = off;
        }
    } else {
        for (int e = tid - kWave; e < nr * PAIRS; e += blockDim.x - kWave) {
            double c, sn;
            rope_cos_sin(a.positions[r0 + (e / PAIRS)], a.freqs.w[e % PAIRS], &c, &sn);
            s_cs[e] = make_double2(c, sn);
        }
    }
    __syncthreads();
    if (tid < 64) {  // V^T store lists, by the first wave (read after the V staging barrier)
        // A run starts at a valid row that does not continue the previous
        // row's slot in the same page, or that begins an aligned segment; a
        // run of 8 rows is then a full segment.
        const int j = tid;
        const bool valid = j < kAppendRows && s_base[j] >= 0;
        const bool start = valid && (j == 0 || s_base[j - 1] != s_base[j] || s_off[j - 1] + 1 != s_off[j] ||
                                     (s_off[j] & 7) == 0);
        const uint64_t starts = __ballot(start);
        const uint64_t breaks = starts | __ballot(!valid);  // rows past the group are not valid
        const bool seg = start && __builtin_ctzll(breaks >> (j + 1)) == 7;  // j < 16: a break above it exists
        const uint64_t segs = __ballot(seg);
        uint32_t in_seg = 0;
        for (uint64_t f = segs; f; f &= f - 1) in_seg |= 0xffu << __builtin_ctzll(f);
        const bool el = valid && !((in_seg >> j) & 1);
        const uint64_t els = __ballot(el);
        if (seg) s_seg[__popcll(segs & ((1ull << j) - 1ull))] = j;
        if (el) s_erow[__popcll(els & ((1ull << j) - 1ull))] = j;
        if (tid == 0) {
            s_nseg = __popcll(segs);
            s_nerow = __popcll(els);
        }
    }
    // K chunks kBatch at a time per thread: all loads of a batch are issued
    // before the first rotation, so a thread keeps kBatch loads in flight
    for (int e0 = tid; e0 < nk; e0 += kBatch * 256) {
        uint4 xk[kBatch];
        load_k(e0, xk);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + 256 * u;
            if (e >= nk) break;
            const int c = e & (C8 - 1), rh = e >> CSH;
            const int j = rh / H, h = rh - j * H;
            const int64_t base = s_base[j];
            if (base >= 0)
                *reinterpret_cast<uint4 *>(a.pool + base + ((int64_t)h * a.P + s_off[j]) * D + 8 * c) =
                    rotate_chunk(xk[u], &s_cs[j * PAIRS + 4 * c]);
        }
    }
    const int64_t vblock = (int64_t)H * a.P * D;  // V block [H][D][P] follows the K block
    __syncthreads();  // every K rotation has read the angle table before V overwrites it
    for (int h0 = 0; h0 < H; h0 += hg) {
        const int hn = min(hg, H - h0);
        const int rs = hn * D + 8;  // LDS row stride (elements): 16 bytes of padding per row
        const int nv = nr * hn * C8;
        for (int e0 = tid; e0 < nv; e0 += kBatch * 256) {
            uint4 xv[kBatch];
            load_v(e0, h0, hn, xv);
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = e0 + 256 * u;
                if (e >= nv) break;
                const int c = e & (C8 - 1), rh = e >> CSH;
                const int j = rh / hn, hh = rh - j * hn;
                *reinterpret_cast<uint4 *>(&s_v[j * rs + hh * D + 8 * c]) = xv[u];
            }
        }
        __syncthreads();
        const int nseg = s_nseg, ne = s_nerow;
        for (int col = tid; col < hn * D; col += blockDim.x) {  // col = hh * D + d
            const int64_t vrow = vblock + ((int64_t)h0 * D + col) * a.P;  // V^T row (h0 + hh, d) in a page
            for (int q = 0; q < nseg; ++q) {
                const int j = s_seg[q];
                const uint16_t *src = &s_v[j * rs + col];
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (uint32_t)src[2 * i * rs] | ((uint32_t)src[(2 * i + 1) * rs] << 16);
                *reinterpret_cast<uint4 *>(a.pool + s_base[j] + vrow + s_off[j]) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        if (ne > 0) {
            const int lg = ne == 1 ? 0 : 32 - __builtin_clz(ne - 1);  // the element rows, padded to 2^lg
            for (int e = tid; e < (hn * D) << lg; e += blockDim.x) {
                const int k = e & ((1 << lg) - 1), col = e >> lg;
                if (k < ne) {
                    const int j = s_erow[k];
                    a.pool[s_base[j] + vblock + ((int64_t)h0 * D + col) * a.P + s_off[j]] = s_v[j * rs + col];
                }
            }
        }
        __syncthreads();
    }
}

// ============================================================================ hazards

// Write/read conflicts of one pass (the reviews' Eq. (4): what one lane writes
// must not be read or written by another lane), on KV cells (physical page,
// offset). Three words per cell: how many rows write it this pass, and the
// smallest and largest lane that does. A cell written twice sets
// FP_ST_DUP_WRITE; a cell whose writers are not all the lane that writes or
// reads it sets FP_ST_SHARED_CELL. Debug path: four small launches.
struct HazardArgs {
    const int32_t *indptr, *slots, *kv_len, *page_indptr, *page_ids, *committed;
    int L, num_pages, P;
    int64_t N, cells;
    int32_t *cnt, *lmin, *lmax;  // [cells] each
    int32_t *status;
};

__global__ void __launch_bounds__(256) hazard_init_kernel(HazardArgs a) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < a.cells; c += (int64_t)gridDim.x * blockDim.x) {
        a.cnt[c] = 0;
        a.lmin[c] = 0x7FFFFFFF;
        a.lmax[c] = -1;
    }
}

// Cell row `row` writes this pass (the write fp_append_kv performs), or -1 if
// that write is suppressed; *lane_out gets the row's lane.
__device__ __forceinline__ int64_t hazard_write_cell(const HazardArgs &a, int64_t row, int *lane_out) {
    const int lane = find_lane(a.indptr, a.L, row);
    *lane_out = lane;
    const int slot = a.slots[row];
    const int p0 = a.page_indptr[lane];
    const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
    if (slot < 0 || slot >= cap || slot < a.committed[lane]) return -1;
    const int page = a.page_ids[p0 + slot / a.P];
    if (page < 0 || page >= a.num_pages) return -1;
    return (int64_t)page * a.P + slot % a.P;
}

__global__ void __launch_bounds__(256) hazard_mark_kernel(HazardArgs a) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.N) return;
    int lane;
    const int64_t c = hazard_write_cell(a, row, &lane);
    if (c < 0) return;
    atomicAdd(&a.cnt[c], 1);
    atomicMin(&a.lmin[c], lane);
    atomicMax(&a.lmax[c], lane);
}

__global__ void __launch_bounds__(256) hazard_rows_kernel(HazardArgs a) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.N) return;
    int lane;
    const int64_t c = hazard_write_cell(a, row, &lane);
    if (c < 0) return;
    int bits = 0;
    if (a.cnt[c] > 1) bits |= FP_ST_DUP_WRITE;
    if (a.lmin[c] != a.lmax[c]) bits |= FP_ST_SHARED_CELL;
    if (bits) atomicOr(a.status, bits);
}

// Block (x, lane): slots [256 x, 256 x + 256) of the lane that it reads.
__global__ void __launch_bounds__(256) hazard_reads_kernel(HazardArgs a) {
    const int lane = blockIdx.y;
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    const int p0 = a.page_indptr[lane];
    const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
    if (j >= clamp_kv(a.kv_len[lane], cap)) return;
    const int page = a.page_ids[p0 + j / a.P];
    if (page < 0 || page >= a.num_pages) return;
    const int64_t c = (int64_t)page * a.P + j % a.P;
    if (a.cnt[c] > 0 && (a.lmin[c] != lane || a.lmax[c] != lane)) atomicOr(a.status, FP_ST_SHARED_CELL);
}

// ============================================================================ fold

// Lane l = 256 b + t of workgroup b: committed_len += its fold count.
__device__ __forceinline__ void fold_body(const int32_t *indptr, const int32_t *fold, const int32_t *channel,
                                          int32_t *committed, int L, int32_t *status, int b) {
    const int l = b * blockDim.x + threadIdx.x;
    if (l >= L) return;
    const int n = indptr[l + 1] - indptr[l];
    const int f = fold[l];
    int k;
    bool clamped = false;
    if (f == FP_FOLD_ALL) {
        k = n;
    } else if (f == FP_FOLD_CHANNEL) {
        if (channel) k = channel[l];
        else { k = 0; clamped = true; }
    } else if (f >= 0) {
        k = f;
    } else {
        k = 0;
        clamped = true;
    }
    if (k < 0) { k = 0; clamped = true; }
    if (k > n) { k = n; clamped = true; }
    committed[l] += k;
    if (clamped) atomicOr(status, FP_ST_FOLD_CLAMP);
}

__global__ void __launch_bounds__(256) fold_kernel(const int32_t *indptr, const int32_t *fold, const int32_t *channel,
                                                    int32_t *committed, int L, int32_t *status) {
    fold_body(indptr, fold, channel, committed, L, status, (int)blockIdx.x);
}

// ============================================================================ advance

// Geometry of the next pass from the committed lengths: thread t < L writes
// kv_len of lane t, thread t < N writes row t's slot and position.
__global__ void __launch_bounds__(256) advance_kernel(const int32_t *indptr, const int32_t *committed,
                                                       const int32_t *pos_offset, int L, int N,
                                                       int32_t *positions, int32_t *slots, int32_t *kv_len) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < L) kv_len[t] = committed[t] + (indptr[t + 1] - indptr[t]);
    if (t < N) {
        const int lane = find_lane(indptr, L, t);
        const int slot = committed[lane] + (t - indptr[lane]);
        slots[t] = slot;
        positions[t] = slot + (pos_offset ? pos_offset[lane] : 0);
    }
}

// ============================================================================ readout

// Block b copies one readout row: rows[b] if a list is given, else the last row
// of lane b (its destination index counts the non-empty lanes before it).
__device__ __forceinline__ void readout_body(const int32_t *indptr, int L, int64_t N, const float *out,
                                             int row_elems, const int32_t *rows, int num_readout, float *dst,
                                             int32_t *status, int b) {
    __shared__ int s_cnt[256 / kWave];
    int64_t src, di;
    if (rows) {
        di = b;
        src = rows[b];
        if (src < 0 || src >= N) {
            src = -1;
            if (threadIdx.x == 0) atomicOr(status, FP_ST_READOUT_RANGE);
        }
    } else {
        const int n = indptr[b + 1] - indptr[b];
        if (n <= 0) return;
        int cnt = 0;
        for (int j = threadIdx.x; j < b; j += blockDim.x) cnt += (indptr[j + 1] > indptr[j]) ? 1 : 0;
        for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
        if (lane_id() == 0) s_cnt[threadIdx.x / kWave] = cnt;
        __syncthreads();
        int tot = 0;
        for (int w = 0; w < (int)(blockDim.x / kWave); ++w) tot += s_cnt[w];
        di = tot;
        if (di >= num_readout) return;  // device offsets disagree with the host count
        src = indptr[b + 1] - 1;
        if (src >= N) {
            src = -1;
            if (threadIdx.x == 0) atomicOr(status, FP_ST_READOUT_RANGE);
        }
    }
    float *d = dst + di * (int64_t)row_elems;
    if (src < 0) {
        for (int e = threadIdx.x; e < row_elems; e += blockDim.x) d[e] = 0.0f;
        return;
    }
    const float *s = out + src * (int64_t)row_elems;
    if ((row_elems & 3) == 0 && ((reinterpret_cast<uintptr_t>(s) | reinterpret_cast<uintptr_t>(d)) & 15) == 0) {
        const float4 *s4 = reinterpret_cast<const float4 *>(s);
        float4 *d4 = reinterpret_cast<float4 *>(d);
        for (int e = threadIdx.x; e < (row_elems >> 2); e += blockDim.x) d4[e] = s4[e];
    } else {
        for (int e = threadIdx.x; e < row_elems; e += blockDim.x) d[e] = s[e];
    }
}

__global__ void __launch_bounds__(256) readout_kernel(const int32_t *indptr, int L, int64_t N, const float *out,
                                                       int row_elems, const int32_t *rows, int num_readout, float *dst,
                                                       int32_t *status) {
    readout_body(indptr, L, N, out, row_elems, rows, num_readout, dst, status, (int)blockIdx.x);
}

// Fold and readout in one launch: the first fold_blocks workgroups fold, the
// rest copy readout rows. The two touch disjoint memory (committed lengths
// against the output rows), so their order inside the launch does not matter.
__global__ void __launch_bounds__(256) fold_readout_kernel(const int32_t *indptr, const int32_t *fold,
                                                            const int32_t *channel, int32_t *committed, int L,
                                                            int fold_blocks, int64_t N, const float *out,
                                                            int row_elems, const int32_t *rows, int num_readout,
                                                            float *dst, int32_t *status) {
    const int b = (int)blockIdx.x;
    if (b < fold_blocks)
        fold_body(indptr, fold, channel, committed, L, status, b);
    else
        readout_body(indptr, L, N, out, row_elems, rows, num_readout, dst, status, b - fold_blocks);
}

// ============================================================================ Q rotation

struct RopeQArgs {
    const uint16_t *q;
    uint16_t *qrot;
    const int32_t *positions;
    int64_t N;
    int Hq;
    double qscale;  // sm_scale * log2(e): scores come out in base-2 units
    int rshift;     // log2 of the rows per workgroup (<= kQRows)
    RopeFreqs freqs;
};

constexpr int kQRows = 16;  // most rows one Q-rotation workgroup handles

// One workgroup per 2^rshift rows: the (cos, sin) of every (row, pair),
// computed in fp64, prescaled by qscale and rounded to fp32, go to LDS (all
// query heads of a row share them), then one thread per 16-byte chunk (four
// pairs) of a (row, head) row rotates it in fp32 and rounds it to bf16
// (rotate_chunk_f32); consecutive threads take consecutive chunks, so
// a wave reads and writes whole head rows. Output: the rotated, prescaled Q in
// bf16, same [N][Hq][D] layout as q.
template <int D>
__device__ __forceinline__ void rope_q_body(const RopeQArgs &a, int block) {
    constexpr int PAIRS = D / 2, C8 = D / 8, CSH = D == 128 ? 4 : 3;
    __shared__ float2 s_cs[kQRows * PAIRS];
    const int R = 1 << a.rshift;
    const int64_t r0 = (int64_t)block << a.rshift;
    const int nr = (int)(a.N - r0 < R ? a.N - r0 : R);
    for (int e = threadIdx.x; e < nr * PAIRS; e += blockDim.x) {
        double c, sn;
        rope_cos_sin(a.positions[r0 + (e / PAIRS)], a.freqs.w[e % PAIRS], &c, &sn);
        s_cs[e] = make_float2((float)(c * a.qscale), (float)(sn * a.qscale));
    }
    __syncthreads();
    const int Hq = a.Hq;
    const int nq = nr * Hq * C8;
    const int nt = blockDim.x;
    for (int e0 = threadIdx.x; e0 < nq; e0 += kBatch * nt) {
        uint4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + nt * u;
            x[u] = e < nq ? *reinterpret_cast<const uint4 *>(a.q + (r0 * Hq + (e >> CSH)) * D + 8 * (e & (C8 - 1)))
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + nt * u;
            if (e >= nq) break;
            const int c = e & (C8 - 1), rh = e >> CSH;
            const int j = rh / Hq;
            *reinterpret_cast<uint4 *>(a.qrot + (r0 * Hq + rh) * D + 8 * c) = rotate_chunk_f32(x[u], &s_cs[j * PAIRS + 4 * c]);
        }
    }
}

// ============================================================================ plan

constexpr int kXcds = 8;  // accelerator complex dies: workgroups go to them round robin by launch index
constexpr int kPlanThreads = 1024;
constexpr int kMaxLanes = 4096;
constexpr int kDecodeCols = 32;  // query row-heads one decode wave holds (MFMA N)
constexpr int kPreCols = 256;    // query row-heads per prefill workgroup (8 waves x 32 columns)

// Rows of one prefill work item: all GQA heads of those rows fill the workgroup.
__host__ __device__ __forceinline__ int prefill_rows(int G) { return kPreCols / G; }

constexpr int kLastBuckets = 129;  // last-split lengths in 32-slot tiles, 0..128 (splits up to 4096 slots)
constexpr int kDecodeCols16 = 16;  // passes whose decode lanes have at most this many row-heads run the 16-column kernel

struct PlanArgs {
    const int32_t *indptr, *page_indptr, *kv_len;
    const int64_t *mask_off;  // nullable
    int L, H, G, P, split;
    int64_t n_dec_host[2];  // decode items of the unmasked lanes, of the masked lanes
    int64_t n_pre_host, sum_host, N_host;
    int ncols_host;
    int merge_host;     // the host allotted split-merge buffers
    LaneInfo *lane_info;
    int4 *dec_items;   // unmasked lanes' items, then masked lanes': {lane, kv head, first slot, end slot}
    int4 *pre_items;   // {lane, kv head, first local row, rows}
    int32_t *status;
};

struct LaneCounts {
    int dec, pre, sum, nsplit, nrb, stride, ncols, cls;  // cls: 1 for a masked decode lane
};

__device__ __forceinline__ LaneCounts lane_counts(const PlanArgs &a, int l, int32_t *st) {
    LaneCounts r = {0, 0, 0, 0, 0, 0, 0, 0};
    const int n = a.indptr[l + 1] - a.indptr[l];
    const int cap = (a.page_indptr[l + 1] - a.page_indptr[l]) * a.P;
    const int kv = a.kv_len[l];
    if (kv < 0 || kv > cap) *st |= FP_ST_KVLEN;
    if (n <= 0) return r;
    const bool masked = a.mask_off && a.mask_off[l + 1] > a.mask_off[l];
    if (masked) {
        const int64_t wpr = (a.mask_off[l + 1] - a.mask_off[l]) / n;
        if (32 * wpr < (int64_t)clamp_kv(kv, cap)) *st |= FP_ST_MASK_SHORT;
    }
    if (n * a.G <= kDecodeCols) {
        r.nsplit = cap > 0 ? (cap + a.split - 1) / a.split : 1;
        r.dec = a.H * r.nsplit;
        r.ncols = n * a.G;
        if (masked) {  // one tile list for the lane (all its rows); its items go to the masked launch
            r.stride = (cap + 31) / 32 + 1;
            r.sum = r.stride;
            r.cls = 1;
        }
    } else {
        r.nrb = (n + prefill_rows(a.G) - 1) / prefill_rows(a.G);
        r.pre = a.H * r.nrb;
        if (masked) {
            r.stride = (cap + 31) / 32 + 1;
            r.sum = r.nrb * r.stride;
        }
    }
    return r;
}

__device__ __forceinline__ int upper_lane(const int *offs, int L, int idx) {
    int lo = 0, hi = L;  // largest l in [0, L) with offs[l] <= idx
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= idx) lo = mid; else hi = mid;
    }
    return lo;
}

// Inclusive prefix sum over the 64 lanes of a wave in registers (DPP): within
// each 16-lane row by shifts of 1, 2, 4 and 8 lanes, then each row's total
// carried into the rows after it by broadcasts of lanes 15 and 31. A lane whose
// source lies outside its row, or a row the step does not write, adds 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Exclusive prefix sums over the workgroup's threads (in thread order) of K
// values at once, in place; tot[k] gets the sum of all. One pair of barriers
// for all K: each wave scans its values in registers and leaves its totals in
// s_w (K ints per wave); then lanes 0..15 of every wave read the 16 wave
// totals of a value and scan them the same way, and each wave takes its
// offset and the grand total from that scan by lane reads.
template <int K>
__device__ __forceinline__ void block_excl_scan_n(int (&v)[K], int (&tot)[K], int *s_w) {
    constexpr int NW = kPlanThreads / kWave;
    static_assert(NW <= 16, "the wave totals are scanned within one 16-lane row");
    const int ln = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    int x[K];
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] = wave_incl_scan(v[k]);
    if (ln == kWave - 1) {
#pragma unroll
        for (int k = 0; k < K; ++k) s_w[k * NW + wv] = x[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int inc = wave_incl_scan(ln < NW ? s_w[k * NW + ln] : 0);
        const int before = wv > 0 ? __builtin_amdgcn_readlane(inc, wv - 1) : 0;
        tot[k] = __builtin_amdgcn_readlane(inc, NW - 1);
        v[k] = before + x[k] - v[k];
    }
    __syncthreads();
}

// Exclusive prefix sum of one value per thread; *total gets the sum of all.
// s_w: one int per wave.
__device__ __forceinline__ int block_excl_scan(int v, int *s_w, int *total) {
    int vv[1] = {v}, tt[1];
    block_excl_scan_n<1>(vv, tt, s_w);
    *total = tt[0];
    return vv[0];
}

// Single workgroup: per-lane classification (decode if all rows x GQA heads fit
// one MFMA tile, prefill otherwise), prefix offsets, and the work-item lists.
// The decode list holds the items of the unmasked decode lanes, then those of
// the masked ones (a launch each: masked lanes walk tile lists); within each
// part, first every split but each (lane, KV head)'s last, then the last
// splits (the partial ones) ordered by the slots they read, longest first, so
// that the long items are dispatched first and the shortest set the tail. Split outputs are stored by (lane, KV head, split): lane_info's
// dec_off counts every decode item of the lanes before, in lane order.
__device__ __forceinline__ void plan_body(const PlanArgs &a) {
    __shared__ int s_pre[kMaxLanes + 1];    // prefill items before lane l
    __shared__ int s_full[2][kMaxLanes + 1];  // non-last decode items of part c (unmasked, masked) before lane l
    __shared__ int s_lane_at[2][kMaxLanes];   // part c's decode lanes by the length of their last split, longest first
    __shared__ int s_hist[2][kLastBuckets];   // decode lanes of part c per last-split bucket, then bucket offsets
    __shared__ int s_nsplit[kMaxLanes];       // decode splits of lane l
    __shared__ int s_cap[kMaxLanes];          // slot capacity of lane l
    __shared__ int s_w[7 * (kPlanThreads / kWave)];
    __shared__ int s_bad;
    const int tid = threadIdx.x;
    if (tid == 0) s_bad = 0;
    for (int e = tid; e < 2 * kLastBuckets; e += kPlanThreads) s_hist[e / kLastBuckets][e % kLastBuckets] = 0;
    const int per = (a.L + kPlanThreads - 1) / kPlanThreads;
    const int l0 = tid * per, l1 = min(a.L, l0 + per);
    // bucket of a decode lane's last split by the slots it reads there, in
    // 32-slot tiles: 0 for the longest
    auto last_key = [&](int l, const LaneCounts &c) {
        const int cap = (a.page_indptr[l + 1] - a.page_indptr[l]) * a.P;
        const int rem = clamp_kv(a.kv_len[l], cap) - (c.nsplit - 1) * a.split;
        const int t = rem <= 0 ? 0 : (min(rem, a.split) + 31) >> 5;
        return (kLastBuckets - 1) - min(t, kLastBuckets - 1);
    };
    // A thread keeps its first lane's counts and key in registers for the
    // later passes (with at most 1024 lanes, its only lane); further lanes are
    // read again. Split counts and capacities go to LDS for the item lists.
    LaneCounts c0 = {0, 0, 0, 0, 0, 0, 0, 0};
    int key0 = 0;
    int32_t st = 0, dummy = 0;
    auto counts_of = [&](int l) { return l == l0 ? c0 : lane_counts(a, l, &dummy); };
    auto key_of = [&](int l, const LaneCounts &c) { return l == l0 ? key0 : last_key(l, c); };
    int td = 0, tp = 0, ts = 0, tc = 0, tf0 = 0, tf1 = 0, tn0 = 0, tn1 = 0;
    for (int l = l0; l < l1; ++l) {
        const LaneCounts c = lane_counts(a, l, &st);
        const int key = last_key(l, c);
        if (l == l0) {
            c0 = c;
            key0 = key;
        }
        s_nsplit[l] = c.nsplit;
        s_cap[l] = (a.page_indptr[l + 1] - a.page_indptr[l]) * a.P;
        td += c.dec; tp += c.pre; ts += c.sum;
        if (c.dec) {
            if (c.cls == 0) { tf0 += c.dec - a.H; tn0 += 1; }
            else { tf1 += c.dec - a.H; tn1 += 1; }
        }
        tc = max(tc, c.ncols);
        if (c.nsplit > 1 && !a.merge_host) tc = kDecodeCols + 1;  // forces the mismatch path
    }
    if (st) atomicOr(a.status, st);
    int sc[7] = {td, tp, ts, tf0, tf1, tn0, tn1}, tot[7];
    block_excl_scan_n<7>(sc, tot, s_w);  // its barriers also order s_bad's initialisation
    if (tc > a.ncols_host) atomicOr(&s_bad, 1);
    int od = sc[0], op = sc[1], os = sc[2], of0 = sc[3], of1 = sc[4], on0 = sc[5], on1 = sc[6];
    const int Td = tot[0], Tp = tot[1], Ts = tot[2], Tf0 = tot[3], Tf1 = tot[4], Tn0 = tot[5], Tn1 = tot[6];
    for (int l = l0; l < l1; ++l) {
        const LaneCounts c = counts_of(l);
        s_pre[l] = op;
        s_full[0][l] = of0;
        s_full[1][l] = of1;
        if (c.dec) atomicAdd(&s_hist[c.cls][key_of(l, c)], 1);
        LaneInfo li;
        li.dec_off = c.dec ? od : -1;
        li.nsplit = c.nsplit;
        li.sum_off = c.sum ? os : -1;
        li.sum_stride = c.stride;
        a.lane_info[l] = li;
        od += c.dec; op += c.pre; os += c.sum;
        if (c.dec) {
            if (c.cls == 0) { of0 += c.dec - a.H; on0 += 1; }
            else { of1 += c.dec - a.H; on1 += 1; }
        }
    }
    const int n0 = Tf0 + a.H * Tn0, n1 = Tf1 + a.H * Tn1;  // decode items of each part
    __syncthreads();  // the histograms are complete
    if (tid < 2 * kWave) {  // bucket offsets, longest last splits first: wave c scans part c's buckets
        static_assert(kLastBuckets <= 3 * kWave, "three buckets per lane");
        const int c = tid / kWave, b0 = 3 * lane_id();
        int cnt[3], sum = 0;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            cnt[j] = b0 + j < kLastBuckets ? s_hist[c][b0 + j] : 0;
            sum += cnt[j];
        }
        int acc = wave_incl_scan(sum) - sum;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (b0 + j < kLastBuckets) s_hist[c][b0 + j] = acc;
            acc += cnt[j];
        }
    }
    __syncthreads();
    for (int l = l0; l < l1; ++l) {
        const LaneCounts c = counts_of(l);
        if (c.dec) s_lane_at[c.cls][atomicAdd(&s_hist[c.cls][key_of(l, c)], 1)] = l;
    }
    if (tid == 0) {
        s_pre[a.L] = Tp;
        s_full[0][a.L] = Tf0;
        s_full[1][a.L] = Tf1;
        // Launch grids and workspace were sized from the host copies; device
        // offsets that disagree would index past them, so no work is emitted.
        if (n0 != a.n_dec_host[0] || n1 != a.n_dec_host[1] || Td != n0 + n1 || Tp != a.n_pre_host ||
            Ts != a.sum_host || (int64_t)a.indptr[a.L] != a.N_host)
            atomicOr(&s_bad, 1);
    }
    __syncthreads();
    const bool bad = s_bad != 0;
    if (bad) {
        for (int l = tid; l < a.L; l += kPlanThreads) a.lane_info[l] = LaneInfo{-1, 0, -1, 0};
        if (tid == 0) atomicOr(a.status, FP_ST_PLAN_MISMATCH);
    }
    const int64_t n_dec = a.n_dec_host[0] + a.n_dec_host[1];
    for (int64_t idx = tid; idx < n_dec; idx += kPlanThreads) {
        int4 it = make_int4(-1, 0, 0, 0);
        if (!bad) {
            const int cls = idx < n0 ? 0 : 1;
            const int local = (int)idx - (cls ? n0 : 0);
            const int tf = cls ? Tf1 : Tf0;
            int l, g, sp;
            if (local < tf) {
                // a non-last split: the largest lane whose first such item is at or before local
                l = upper_lane(s_full[cls], a.L, local);
                const int j = local - s_full[cls][l];
                const int ns = s_nsplit[l];
                g = j / (ns - 1);
                sp = j - g * (ns - 1);
            } else {
                // last splits: lanes by the length of their last split, longest first
                const int j = local - tf;
                l = s_lane_at[cls][j / a.H];
                g = j % a.H;
                sp = s_nsplit[l] - 1;
            }
            const int cap = s_cap[l];
            it = make_int4(l, g, sp * a.split, min((sp + 1) * a.split, cap));
        }
        a.dec_items[idx] = it;
    }
    const int tot_p = bad ? 0 : Tp;
    for (int64_t idx = tid; idx < a.n_pre_host; idx += kPlanThreads) {
        int4 it = make_int4(-1, 0, 0, 0);
        if (idx < tot_p) {
            const int l = upper_lane(s_pre, a.L, (int)idx);
            const int local = (int)idx - s_pre[l];
            const int n = a.indptr[l + 1] - a.indptr[l];
            // KV head fastest: consecutive items go to different XCDs, and the
            // row blocks of one (lane, KV head) land on the same XCD and L2.
            // Last row blocks first: under the causal rule they read the most slots.
            const int RB = prefill_rows(a.G);
            const int nrb = (n + RB - 1) / RB;
            const int rb = nrb - 1 - local / a.H, g = local % a.H;
            it = make_int4(l, g, rb * RB, min(RB, n - rb * RB));
        }
        a.pre_items[idx] = it;
    }
}

// The plan: one workgroup.
__global__ void __launch_bounds__(kPlanThreads) plan_kernel(PlanArgs pa) { plan_body(pa); }

// Q rotation: a launch of its own with small workgroups, so that many of them
// (each with its own loads in flight) share a compute unit; the plan's large
// LDS footprint would allow one per compute unit.
constexpr int kRopeThreads = 256;

template <int D>
__global__ void __launch_bounds__(kRopeThreads) rope_q_kernel(RopeQArgs ra) { rope_q_body<D>(ra, (int)blockIdx.x); }

// The plan and the Q rotation in one launch, for passes whose rotation needs
// at most about four workgroups per compute unit (decode and verify waves):
// workgroup 0 plans, workgroup 1 + b rotates row group b on the other compute
// units while the plan, the longer of the two, runs. One launch and its gap
// fewer; the rotation workgroups carry the plan's block size and LDS, which
// matters only when there are many.
constexpr int kPrepMaxRopeBlocks = 1023;

template <int D>
__global__ void __launch_bounds__(kPlanThreads) prep_kernel(PlanArgs pa, RopeQArgs ra) {
    if (blockIdx.x == 0) plan_body(pa);
    else rope_q_body<D>(ra, (int)blockIdx.x - 1);
}

// ============================================================================ mask summary

struct SummaryArgs {
    int64_t n_pre;  // prefill items (a multiple of H: each lane's come in groups of its KV heads)
    int L, H;
    const int4 *pre_items;
    const LaneInfo *lane_info;
    const int32_t *indptr, *page_indptr, *kv_len;
    const uint32_t *bits;
    const int64_t *mask_off;
    int P, G;
    int32_t *summary;
};

// Tile list of one row block of a masked prefill lane (the rows of one prefill
// work item), or of all rows of a masked decode lane: the 32-slot KV tiles
// below kv_len in which some row of the block
// has an allowed slot, in increasing order, each entry tagged in bit 31 when
// every row of the block may read every slot of the tile. Record layout:
// [count, entry 0, entry 1, ...]. The prefill kernel walks this list, so
// tiles with no allowed slot are never loaded. The plan lists a lane's prefill
// items with the KV head fastest, so the KV-head-0 items, one per row block,
// are items 0, H, 2H, ...: workgroup b < n_pre / H takes item b * H, and the
// workgroups after them take the masked decode lanes.
constexpr int kSumThreads = 1024;  // one thread per tile of up to 32768 slots: one pass over the rows

__global__ void __launch_bounds__(kSumThreads) summary_kernel(SummaryArgs a) {
    __shared__ int s_wc[kSumThreads / kWave];
    int l, rstart, nr;
    LaneInfo li;
    int32_t *rec;
    const int64_t n_blocks = a.n_pre / a.H;
    if ((int64_t)blockIdx.x < n_blocks) {  // a row block of a masked prefill lane (its KV head 0 item)
        const int4 it = a.pre_items[(int64_t)blockIdx.x * a.H];
        if (it.x < 0 || it.y != 0) return;
        l = it.x;
        li = a.lane_info[l];
        if (li.sum_off < 0) return;
        rstart = it.z;
        nr = it.w;
        rec = a.summary + li.sum_off + (int64_t)(rstart / prefill_rows(a.G)) * li.sum_stride;
    } else {  // a masked decode lane: one list over all its rows
        l = (int)(blockIdx.x - n_blocks);
        if (l >= a.L) return;
        li = a.lane_info[l];
        if (li.sum_off < 0 || li.dec_off < 0) return;
        rstart = 0;
        nr = a.indptr[l + 1] - a.indptr[l];
        rec = a.summary + li.sum_off;
    }
    const int nl = a.indptr[l + 1] - a.indptr[l];
    const int64_t wpr = (a.mask_off[l + 1] - a.mask_off[l]) / nl;
    const int cap = (a.page_indptr[l + 1] - a.page_indptr[l]) * a.P;
    const int eff = clamp_kv(a.kv_len[l], cap);
    const uint32_t *rb = a.bits + a.mask_off[l] + (int64_t)rstart * wpr;
    // tiles holding slots below kv_len whose mask word exists (a short row reads 0 beyond its words)
    const int ntiles = (int)min((int64_t)((eff + 31) >> 5), wpr);
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    int running = 0;
    for (int t0 = 0; t0 < ntiles; t0 += kSumThreads) {
        const int t = t0 + (int)threadIdx.x;
        const bool inr = t < ntiles;
        uint32_t any = 0, all = ~0u;
        if (inr) {
            int r = 0;
            for (; r + 16 <= nr; r += 16) {  // 16 rows' words in flight per thread
                uint32_t w16[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) w16[u] = rb[(int64_t)(r + u) * wpr + t];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    any |= w16[u];
                    all &= w16[u];
                }
            }
            for (; r < nr; ++r) {
                const uint32_t w = rb[(int64_t)r * wpr + t];
                any |= w;
                all &= w;
            }
        }
        const uint32_t valid = !inr ? 0u : ((32 * t + 32 <= eff) ? ~0u : ((1u << (eff - 32 * t)) - 1u));
        const bool anyb = inr && (any & valid);
        const bool allb = inr && ((all | ~valid) == ~0u);
        const uint64_t ba = __ballot(anyb);
        if (lane == 0) s_wc[wv] = __popcll(ba);
        __syncthreads();
        int before = running, total = 0;
#pragma unroll
        for (int v = 0; v < kSumThreads / kWave; ++v) {
            before += v < wv ? s_wc[v] : 0;
            total += s_wc[v];
        }
        if (anyb) rec[1 + before + __popcll(ba & ((1ull << lane) - 1ull))] = t | (allb ? (int)0x80000000u : 0);
        running += total;
        __syncthreads();
    }
    if (threadIdx.x == 0) rec[0] = running;
}

// ============================================================================ attention

struct AttnArgs {
    const uint16_t *pool;
    int64_t page_elems;
    int num_pages, P, H, G, Hq;
    const int32_t *page_indptr, *page_ids;
    const int32_t *indptr, *slots, *kv_len;
    const uint16_t *qrot;             // [N][Hq][D] rotated, prescaled bf16
    const uint32_t *mask_bits;        // nullable
    const int64_t *mask_off;          // nullable
    float *out, *lse;                 // lse nullable
    const int4 *dec_items, *pre_items;
    const int4 *dec_list;             // the decode items of one launch (one column class)
    const LaneInfo *lane_info;
    float *part_o;                    // [items][ncols_max][D] unnormalized split outputs
    float *part_ml;                   // [items][2][32] split max (base 2) and sum
    int ncols_max;
    int split;                        // decode KV slots per work item
    const int32_t *summary;           // row-block tile lists of masked prefill lanes
};

// Per-wave view of one (lane, KV head): where its slots live and how far rows may read.
struct KvView {
    const uint16_t *kbase;   // pool
    const int32_t *pids;     // page_ids + page_indptr[lane]
    int64_t page_elems;
    int64_t vblock;          // element offset of the V block in a page
    int P, pshift, pmask;    // page size (a power of two), log2 and P - 1
    int g, H, eff, last_page;
};

// Physical page of working-set page j; an id outside the pool reads the nearest valid page.
__device__ __forceinline__ int64_t page_of(const KvView &kv, int j) {
    const int p = kv.pids[j];
    return (int64_t)min(max(p, 0), kv.last_page);
}

__device__ __forceinline__ KvView make_view(const AttnArgs &a, int lane, int g, int *cap_out) {
    KvView kv;
    const int p0 = a.page_indptr[lane];
    const int cap = (a.page_indptr[lane + 1] - p0) * a.P;
    kv.kbase = a.pool;
    kv.pids = a.page_ids + p0;
    kv.page_elems = a.page_elems;
    kv.P = a.P;
    kv.pshift = __builtin_ctz(a.P);
    kv.pmask = a.P - 1;
    kv.g = g;
    kv.H = a.H;
    kv.eff = clamp_kv(a.kv_len[lane], cap);
    kv.last_page = a.num_pages - 1;
    *cap_out = cap;
    return kv;
}

}  // namespace fpk

#include "fp_decode.h"
#include "fp_prefill.h"
#include "fp_stats.h"
#include "fp_lora.h"
#include "fp_evict.h"
