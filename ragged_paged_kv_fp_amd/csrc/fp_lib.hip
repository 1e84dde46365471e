// fp_lib.hip - host side of the C ABI declared in include/fp.h.
//
// Host work is limited to argument checks, shape-only planning from the
// *_host copies of the offset arrays (how many work items to launch, how big
// the workspace is) and kernel launches on the caller's stream. All per-lane
// decisions that depend on device data (kv_len, slots, committed_len, channel
// counts, mask bits) are taken by the kernels.
#include "fp_kernels.h"

#include <algorithm>
#include <functional>
#include <math.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

// The library's own device scratch (fp_attend_noalloc): 64 MiB per device,
// file scope, held until the process ends. Host code must use the address
// hipGetSymbolAddress returns for the current device, never this name.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using namespace fpk;

// Decode split sizes the default plan chooses from, largest first: the largest
// that still gives every resident decode workgroup slot on the device about
// two work items. Longer splits pay the per-item start (page ids, then the
// first KV loads: two dependent memory round trips) and the split merge
// fewer times; too few items leave compute units idle at the end.
constexpr int kSplitChoices[] = {4096, 2048, 1024, 512};
constexpr double kItemsPerSlot = 1.7;

// Compute units of the current device, queried once per device.
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

int check_pool(const fp_kv_pool *p) {
    if (!p || !p->kv || !p->page_indptr || !p->page_indptr_host || !p->page_ids || !p->committed_len) return FP_ERR_NULL;
    if (!aligned16(p->kv)) return FP_ERR_UNSUPPORTED;
    if (p->num_pages < 1 || p->num_kv_heads < 1) return FP_ERR_SHAPE;
    if (p->page_size != 8 && p->page_size != 16 && p->page_size != 32) return FP_ERR_UNSUPPORTED;
    if (p->head_dim != 64 && p->head_dim != 128) return FP_ERR_UNSUPPORTED;
    return FP_OK;
}

int check_geom(const fp_geometry *g, const fp_kv_pool *p) {
    if (!g || !g->indptr || !g->indptr_host || !g->kv_len || !g->fold) return FP_ERR_NULL;
    if (g->num_lanes < 1 || g->num_rows < 0) return FP_ERR_SHAPE;
    if (g->num_rows > 0 && (!g->positions || !g->slots)) return FP_ERR_NULL;
    const int32_t *ip = g->indptr_host;
    if (ip[0] != 0 || ip[g->num_lanes] != g->num_rows) return FP_ERR_SHAPE;
    for (int l = 0; l < g->num_lanes; ++l)
        if (ip[l + 1] < ip[l]) return FP_ERR_SHAPE;
    if (p) {
        const int32_t *pp = p->page_indptr_host;
        if (pp[0] != 0) return FP_ERR_SHAPE;
        for (int l = 0; l < g->num_lanes; ++l) {
            if (pp[l + 1] < pp[l]) return FP_ERR_SHAPE;
            if ((int64_t)(pp[l + 1] - pp[l]) * p->page_size > (int64_t)INT32_MAX / 2) return FP_ERR_UNSUPPORTED;
        }
    }
    return FP_OK;
}

int check_mask(const fp_mask *m, const fp_geometry *g) {
    if (!m) return FP_OK;
    if (!m->bits || !m->word_offset || !m->word_offset_host) return FP_ERR_NULL;
    const int64_t *wo = m->word_offset_host;
    for (int l = 0; l < g->num_lanes; ++l) {
        const int64_t span = wo[l + 1] - wo[l];
        const int n = g->indptr_host[l + 1] - g->indptr_host[l];
        if (span < 0) return FP_ERR_SHAPE;
        if (span > 0 && (n == 0 || span % n != 0)) return FP_ERR_SHAPE;
    }
    return FP_OK;
}

struct Plan {
    int L = 0, H = 0, G = 0, Hq = 0, D = 0, P = 0, split = 0, ncols_max = 1;
    int64_t N = 0, n_dec = 0, n_dec_cls[2] = {0, 0}, n_pre = 0, sum_words = 0;
    bool merge = false, summaries = false, dec_lists = false, wide = false;
    size_t off_lane = 0, off_dec = 0, off_pre = 0, off_qrot = 0, off_po = 0, off_pml = 0, off_sum = 0;
    size_t total = 0;
};

// Workgroups of a kernel resident on the device at once (occupancy query,
// cached per device and kernel).
template <class Kernel>
int resident_blocks(Kernel kernel, int threads) {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1) nb = 1;
        cached[dev] = nb * device_cus();
    }
    return cached[dev];
}

// A second look at the split for unmasked decode passes: an estimate of when
// the last decode item ends, by list scheduling in the plan's dispatch order
// (every split but each lane's last, all of one size, then the last splits
// longest first), each item taken by the first resident workgroup that frees
// up. An item costs its 32-slot tiles (by capacity) plus a start of
// kItemStartTiles tiles: page ids and the first K/V loads before it streams,
// fitted to split sweeps on MI355X. The KV heads of a lane give H equal copies
// of each of its items in a row, so m = resident workgroups / H slots taking
// one copy each give the same schedule. With few items per slot this is where
// the split matters: the longest items set the end. The plan takes a smaller
// split from kSplitRefine only when the estimate is kRefineGain below the
// first choice's, which keeps the first choice wherever the two are close.
constexpr int kSplitRefine[] = {3072, 1536, 1024, 512};
constexpr double kItemStartTiles = 6.0;
constexpr double kRefineGain = 0.9;
constexpr int kRefineSlots = 2048;  // most slots the estimate keeps (more are folded in)

// Stack use stays near 12 KB: a last split is at most 128 tiles (splits are at
// most 4096 slots), and a slot's load, a sum of tile counts, is exact in float.
double decode_makespan(const fp_kv_pool *pool, const fp_geometry *geom, int G, int split, int m) {
    uint8_t lasts[kMaxLanes];  // the last split of each decode lane, in tiles
    float load[kRefineSlots];
    int nl = 0;
    int64_t nfull = 0;
    for (int l = 0; l < geom->num_lanes; ++l) {
        const int n = geom->indptr_host[l + 1] - geom->indptr_host[l];
        if (n <= 0 || n * G > kDecodeCols) continue;
        const int cap = (pool->page_indptr_host[l + 1] - pool->page_indptr_host[l]) * pool->page_size;
        const int ns = cap > 0 ? (cap + split - 1) / split : 1;
        nfull += ns - 1;
        lasts[nl++] = (uint8_t)(cap > 0 ? (cap - (ns - 1) * split + 31) / 32 : 0);
    }
    std::sort(lasts, lasts + nl, std::greater<uint8_t>());
    m = std::max(1, std::min(m, kRefineSlots));
    const float cf = (float)(kItemStartTiles + split / 32);
    const int64_t per = nfull / m, rem = nfull % m;
    float end = 0.0f;
    for (int i = 0; i < m; ++i) {
        load[i] = (float)(per + (i < rem ? 1 : 0)) * cf;
        end = std::max(end, load[i]);
    }
    std::make_heap(load, load + m, std::greater<float>());  // min-heap: the slot that frees up first
    for (int i = 0; i < nl; ++i) {
        std::pop_heap(load, load + m, std::greater<float>());
        load[m - 1] += (float)kItemStartTiles + lasts[i];
        end = std::max(end, load[m - 1]);
        std::push_heap(load, load + m, std::greater<float>());
    }
    return end;
}

// Shape-only plan: mirrors lane_counts() of the device plan from the host copies.
int make_plan(const fp_kv_pool *pool, const fp_geometry *geom, const fp_mask *mask, int32_t Hq,
              const fp_tuning *tun, Plan *pl) {
    int rc = check_pool(pool);
    if (rc) return rc;
    if ((rc = check_geom(geom, pool))) return rc;
    if ((rc = check_mask(mask, geom))) return rc;
    if (Hq < 1 || Hq % pool->num_kv_heads) return FP_ERR_SHAPE;
    const int G = Hq / pool->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return FP_ERR_UNSUPPORTED;
    if (geom->num_lanes > kMaxLanes) return FP_ERR_UNSUPPORTED;
    int split = 0;
    if (tun) {
        for (int i = 0; i < 7; ++i)
            if (tun->reserved[i]) return FP_ERR_SHAPE;
        if (tun->decode_split_slots) {
            if (tun->decode_split_slots < 32 || tun->decode_split_slots % 32) return FP_ERR_SHAPE;
            split = tun->decode_split_slots;
        }
    }
    if (split == 0) {
        // decode workgroups resident at once, for the kernel the pass will run
        // (the 32-column kernel as soon as one decode lane has more than 16
        // query row-heads)
        bool wide = false;  // (Plan::wide, known before the loop below fills it)
        bool dec_masked = false;
        for (int l = 0; l < geom->num_lanes; ++l) {
            const int n = geom->indptr_host[l + 1] - geom->indptr_host[l];
            if (n * G > kDecodeCols16 && n * G <= kDecodeCols) wide = true;
            if (n > 0 && n * G <= kDecodeCols && mask && mask->word_offset_host[l + 1] > mask->word_offset_host[l])
                dec_masked = true;
        }
        const int resident = wide ? resident_blocks(decode_kernel<128, 32, false>, 64 * dec_waves<32>())
                                  : resident_blocks(decode_kernel<128, 16, false>, 64 * dec_waves<16>());
        // counted in four-wave workgroups: a two-wave workgroup streams an item
        // at half the rate, so it counts as half a slot
        const double slots = resident * ((wide ? dec_waves<32>() : dec_waves<16>()) / 4.0);
        for (const int cand : kSplitChoices) {
            split = cand;
            int64_t items = 0;
            for (int l = 0; l < geom->num_lanes; ++l) {
                const int n = geom->indptr_host[l + 1] - geom->indptr_host[l];
                const int cap = (pool->page_indptr_host[l + 1] - pool->page_indptr_host[l]) * pool->page_size;
                if (n > 0 && n * G <= kDecodeCols) items += (int64_t)pool->num_kv_heads * (cap > 0 ? (cap + cand - 1) / cand : 1);
            }
            if ((double)items >= kItemsPerSlot * slots) break;
        }
        // masked decode items cost their tile lists, not their slot ranges: no estimate for them
        if (!dec_masked) {
            const int m = std::max(1, resident / pool->num_kv_heads);
            const double first = decode_makespan(pool, geom, G, split, m);
            double best = first;
            int pick = split;
            for (const int cand : kSplitRefine) {
                if (cand >= split) continue;
                const double e = decode_makespan(pool, geom, G, cand, m);
                if (e < best) {
                    best = e;
                    pick = cand;
                }
            }
            if (best < kRefineGain * first) split = pick;
        }
    }
    Plan p;
    p.L = geom->num_lanes;
    p.H = pool->num_kv_heads;
    p.G = G;
    p.Hq = Hq;
    p.D = pool->head_dim;
    p.P = pool->page_size;
    p.split = split;
    p.N = geom->num_rows;
    for (int l = 0; l < p.L; ++l) {
        const int n = geom->indptr_host[l + 1] - geom->indptr_host[l];
        const int cap = (pool->page_indptr_host[l + 1] - pool->page_indptr_host[l]) * p.P;
        if (n <= 0) continue;
        const bool masked = mask && mask->word_offset_host[l + 1] > mask->word_offset_host[l];
        if (n * G <= kDecodeCols) {
            const int nsplit = cap > 0 ? (cap + split - 1) / split : 1;
            p.n_dec += (int64_t)p.H * nsplit;
            p.n_dec_cls[masked ? 1 : 0] += (int64_t)p.H * nsplit;
            if (n * G > kDecodeCols16) p.wide = true;
            if (nsplit > 1) p.merge = true;
            if (n * G > p.ncols_max) p.ncols_max = n * G;
            if (masked) {
                p.sum_words += (cap + 31) / 32 + 1;
                p.summaries = true;
                p.dec_lists = true;
            }
        } else {
            const int nrb = (n + prefill_rows(G) - 1) / prefill_rows(G);
            p.n_pre += (int64_t)p.H * nrb;
            if (masked) {
                p.sum_words += (int64_t)nrb * ((cap + 31) / 32 + 1);
                p.summaries = true;
            }
        }
    }
    if (p.n_dec > INT32_MAX / 2 || p.n_pre > INT32_MAX / 2 || p.sum_words > INT32_MAX / 2) return FP_ERR_UNSUPPORTED;
    // the rotated Q comes first: its place depends only on the rows and heads,
    // so fp_attn_mass finds it whatever tuning or mask the plan had
    size_t off = 0;
    p.off_qrot = off; off = align256(off + sizeof(uint16_t) * (size_t)p.N * Hq * p.D);
    p.off_lane = off; off = align256(off + sizeof(LaneInfo) * (size_t)p.L);
    p.off_dec = off;  off = align256(off + sizeof(int4) * (size_t)p.n_dec);
    p.off_pre = off;  off = align256(off + sizeof(int4) * (size_t)p.n_pre);
    p.off_po = off;   off = align256(off + (p.merge ? sizeof(float) * (size_t)p.n_dec * p.ncols_max * p.D : 0));
    p.off_pml = off;  off = align256(off + (p.merge ? sizeof(float) * (size_t)p.n_dec * 64 : 0));
    p.off_sum = off;  off = align256(off + sizeof(uint32_t) * (size_t)p.sum_words);
    p.total = off;
    *pl = p;
    return FP_OK;
}

// w_i = theta^(-2i/d) in fp64, the RoPE frequency of pair (2i, 2i+1).
RopeFreqs rope_freqs(float theta, int d) {
    RopeFreqs f;
    for (int i = 0; i < kMaxPairs; ++i) f.w[i] = i < d / 2 ? pow((double)theta, -2.0 * (double)i / (double)d) : 0.0;
    return f;
}

inline int launch_ok() { return hipGetLastError() == hipSuccess ? FP_OK : FP_ERR_HIP; }

template <int D, int G>
void launch_prefill(const AttnArgs &a, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL((prefill_kernel<D, G>), dim3((unsigned)n), dim3(kPreThreads), 0, s, a);
}

template <int D>
void launch_prefill_g(const AttnArgs &a, int G, int64_t n, hipStream_t s) {
    switch (G) {
        case 1: launch_prefill<D, 1>(a, n, s); break;
        case 2: launch_prefill<D, 2>(a, n, s); break;
        case 4: launch_prefill<D, 4>(a, n, s); break;
        default: launch_prefill<D, 8>(a, n, s); break;
    }
}

// Scratch memory of fp_attend_noalloc: the workspace fp_attend would take
// from the caller (rotated Q, plan records, work lists, split partials, tile
// lists), held by the library on every device it runs on until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// kernels get the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in scratch_dev.

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices] = {};

// Device address of this device's scratch array (FP_ERR_HIP if the lookup fails).
int scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FP_ERR_HIP;
        scratch_dev[dev] = ptr;
    }
    *out = scratch_dev[dev];
    return FP_OK;
}

// fp_attend on a given workspace (the caller's, or the library's static scratch).
int attend_impl(const fp_kv_pool *pool, const fp_geometry *geom, const void *q, int32_t num_q_heads, float rope_theta,
                float sm_scale, const fp_mask *mask, float *out, float *lse, void *workspace, size_t workspace_bytes,
                const fp_tuning *tuning, int32_t *status, hipStream_t stream) {
    Plan p;
    int rc = make_plan(pool, geom, mask, num_q_heads, tuning, &p);
    if (rc) return rc;
    if (!status) return FP_ERR_NULL;
    if (p.N == 0) return FP_OK;
    if (!q || !out) return FP_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return FP_ERR_UNSUPPORTED;
    if (!workspace) return FP_ERR_NULL;
    if (workspace_bytes < p.total) return FP_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    LaneInfo *lane_info = reinterpret_cast<LaneInfo *>(ws + p.off_lane);
    int4 *dec_items = reinterpret_cast<int4 *>(ws + p.off_dec);
    int4 *pre_items = reinterpret_cast<int4 *>(ws + p.off_pre);
    uint16_t *qrot = reinterpret_cast<uint16_t *>(ws + p.off_qrot);

    PlanArgs pa;
    pa.indptr = geom->indptr;
    pa.page_indptr = pool->page_indptr;
    pa.kv_len = geom->kv_len;
    pa.mask_off = mask ? mask->word_offset : nullptr;
    pa.L = p.L; pa.H = p.H; pa.G = p.G; pa.P = p.P; pa.split = p.split;
    pa.n_dec_host[0] = p.n_dec_cls[0];
    pa.n_dec_host[1] = p.n_dec_cls[1];
    pa.n_pre_host = p.n_pre;
    pa.sum_host = p.sum_words;
    pa.N_host = p.N;
    pa.ncols_host = p.ncols_max;
    pa.merge_host = p.merge ? 1 : 0;
    pa.lane_info = lane_info;
    pa.dec_items = dec_items;
    pa.pre_items = pre_items;
    pa.status = status;

    RopeQArgs ra;
    ra.q = static_cast<const uint16_t *>(q);
    ra.qrot = qrot;
    ra.positions = geom->positions;
    ra.N = p.N;
    ra.Hq = p.Hq;
    ra.qscale = (double)sm_scale * 1.4426950408889634;  // log2(e)
    ra.freqs = rope_freqs(rope_theta, p.D);
    ra.rshift = row_group_shift(p.N, kQRows);
    const int64_t rblocks = (p.N + (1 << ra.rshift) - 1) >> ra.rshift;
    if (rblocks <= kPrepMaxRopeBlocks) {  // plan and Q rotation in one launch
        const dim3 pgrid((unsigned)(1 + rblocks));
        if (p.D == 128) hipLaunchKernelGGL(prep_kernel<128>, pgrid, dim3(kPlanThreads), 0, stream, pa, ra);
        else hipLaunchKernelGGL(prep_kernel<64>, pgrid, dim3(kPlanThreads), 0, stream, pa, ra);
        if ((rc = launch_ok())) return rc;
    } else {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, pa);
        if ((rc = launch_ok())) return rc;
        const dim3 rgrid((unsigned)rblocks);
        if (p.D == 128) hipLaunchKernelGGL(rope_q_kernel<128>, rgrid, dim3(kRopeThreads), 0, stream, ra);
        else hipLaunchKernelGGL(rope_q_kernel<64>, rgrid, dim3(kRopeThreads), 0, stream, ra);
        if ((rc = launch_ok())) return rc;
    }

    AttnArgs a;
    a.pool = static_cast<const uint16_t *>(pool->kv);
    a.num_pages = pool->num_pages;
    a.P = p.P; a.H = p.H; a.G = p.G; a.Hq = p.Hq;
    a.page_elems = 2LL * p.H * p.P * p.D;
    a.page_indptr = pool->page_indptr;
    a.page_ids = pool->page_ids;
    a.indptr = geom->indptr;
    a.slots = geom->slots;
    a.kv_len = geom->kv_len;
    a.qrot = qrot;
    a.mask_bits = mask ? mask->bits : nullptr;
    a.mask_off = mask ? mask->word_offset : nullptr;
    a.out = out;
    a.lse = lse;
    a.dec_items = dec_items;
    a.pre_items = pre_items;
    a.lane_info = lane_info;
    a.part_o = p.merge ? reinterpret_cast<float *>(ws + p.off_po) : nullptr;
    a.part_ml = p.merge ? reinterpret_cast<float *>(ws + p.off_pml) : nullptr;
    a.ncols_max = p.ncols_max;
    a.split = p.split;
    a.summary = reinterpret_cast<const int32_t *>(ws + p.off_sum);

    if (p.summaries) {
        SummaryArgs sa;
        sa.n_pre = p.n_pre;
        sa.L = p.L;
        sa.H = p.H;
        sa.pre_items = pre_items;
        sa.lane_info = lane_info;
        sa.indptr = geom->indptr;
        sa.page_indptr = pool->page_indptr;
        sa.kv_len = geom->kv_len;
        sa.bits = mask->bits;
        sa.mask_off = mask->word_offset;
        sa.P = p.P;
        sa.G = p.G;
        sa.summary = reinterpret_cast<int32_t *>(ws + p.off_sum);
        hipLaunchKernelGGL(summary_kernel, dim3((unsigned)(p.n_pre / p.H + (p.dec_lists ? p.L : 0))), dim3(kSumThreads),
                           0, stream, sa);
        if ((rc = launch_ok())) return rc;
    }
    if (tuning && tuning->attn_begin && hipEventRecord(tuning->attn_begin, stream) != hipSuccess) return FP_ERR_HIP;
    if (p.n_pre) {
        if (p.D == 128) launch_prefill_g<128>(a, p.G, p.n_pre, stream);
        else launch_prefill_g<64>(a, p.G, p.n_pre, stream);
        if ((rc = launch_ok())) return rc;
    }
    if (tuning && tuning->prefill_end && hipEventRecord(tuning->prefill_end, stream) != hipSuccess) return FP_ERR_HIP;
    // decode: the 16-column kernel (two waves per SIMD) when every decode lane
    // has at most 16 query row-heads, else the 32-column kernel for all of
    // them (two launches of different widths would each pay their own start
    // and tail, one after the other); the unmasked lanes' items in one
    // launch, the masked lanes' (which walk tile lists) in a second
    for (int part = 0; part < 2; ++part) {
        const int64_t n = p.n_dec_cls[part];
        if (n == 0) continue;
        AttnArgs ac = a;
        ac.dec_list = dec_items + (part ? p.n_dec_cls[0] : 0);
        const dim3 grid((unsigned)n), block(64 * (p.wide ? dec_waves<32>() : dec_waves<16>()));
        if (p.D == 128) {
            if (!p.wide) {
                if (part == 0) hipLaunchKernelGGL((decode_kernel<128, 16, false>), grid, block, 0, stream, ac);
                else hipLaunchKernelGGL((decode_kernel<128, 16, true>), grid, block, 0, stream, ac);
            } else {
                if (part == 0) hipLaunchKernelGGL((decode_kernel<128, 32, false>), grid, block, 0, stream, ac);
                else hipLaunchKernelGGL((decode_kernel<128, 32, true>), grid, block, 0, stream, ac);
            }
        } else {
            if (!p.wide) {
                if (part == 0) hipLaunchKernelGGL((decode_kernel<64, 16, false>), grid, block, 0, stream, ac);
                else hipLaunchKernelGGL((decode_kernel<64, 16, true>), grid, block, 0, stream, ac);
            } else {
                if (part == 0) hipLaunchKernelGGL((decode_kernel<64, 32, false>), grid, block, 0, stream, ac);
                else hipLaunchKernelGGL((decode_kernel<64, 32, true>), grid, block, 0, stream, ac);
            }
        }
        if ((rc = launch_ok())) return rc;
    }
    if (tuning && tuning->attn_end && hipEventRecord(tuning->attn_end, stream) != hipSuccess) return FP_ERR_HIP;
    if (p.merge) {
        const dim3 grid(p.L, p.H);
        if (p.D == 128) hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, stream, a);
        else hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, stream, a);
        if ((rc = launch_ok())) return rc;
    }
    if (tuning && tuning->merge_end && hipEventRecord(tuning->merge_end, stream) != hipSuccess) return FP_ERR_HIP;
    return FP_OK;
}

}  // namespace

extern "C" {

int fp_append_kv(const fp_kv_pool *pool, const fp_geometry *geom, const void *k, const void *v, float rope_theta,
                 int32_t *status, hipStream_t stream) {
    int rc = check_pool(pool);
    if (rc) return rc;
    if ((rc = check_geom(geom, pool))) return rc;
    if (!status) return FP_ERR_NULL;
    if (geom->num_rows == 0) return FP_OK;
    if (!k || !v) return FP_ERR_NULL;
    if (!aligned16(k) || !aligned16(v)) return FP_ERR_UNSUPPORTED;
    AppendArgs a;
    a.pool = static_cast<uint16_t *>(pool->kv);
    a.num_pages = pool->num_pages;
    a.P = pool->page_size;
    a.H = pool->num_kv_heads;
    a.page_elems = 2LL * a.H * a.P * pool->head_dim;
    a.page_indptr = pool->page_indptr;
    a.page_ids = pool->page_ids;
    a.committed = pool->committed_len;
    a.indptr = geom->indptr;
    a.L = geom->num_lanes;
    a.N = geom->num_rows;
    a.positions = geom->positions;
    a.slots = geom->slots;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.status = status;
    a.freqs = rope_freqs(rope_theta, pool->head_dim);
    a.rshift = row_group_shift(a.N, kAppendRows);
    const dim3 grid((unsigned)((a.N + (1 << a.rshift) - 1) >> a.rshift));
    if (pool->head_dim == 128) hipLaunchKernelGGL(append_kernel<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(append_kernel<64>, grid, dim3(256), 0, stream, a);
    return launch_ok();
}

int64_t fp_attend_workspace_bytes(const fp_kv_pool *pool, const fp_geometry *geom, const fp_mask *mask,
                                  int32_t num_q_heads, const fp_tuning *tuning) {
    Plan p;
    const int rc = make_plan(pool, geom, mask, num_q_heads, tuning, &p);
    if (rc) return rc;
    return (int64_t)p.total;
}

int fp_attend(const fp_kv_pool *pool, const fp_geometry *geom, const void *q, int32_t num_q_heads, float rope_theta,
              float sm_scale, const fp_mask *mask, float *out, float *lse, void *workspace, size_t workspace_bytes,
              const fp_tuning *tuning, int32_t *status, hipStream_t stream) {
    return attend_impl(pool, geom, q, num_q_heads, rope_theta, sm_scale, mask, out, lse, workspace, workspace_bytes,
                       tuning, status, stream);
}

int fp_attend_noalloc(const fp_kv_pool *pool, const fp_geometry *geom, const void *q, int32_t num_q_heads,
                      float rope_theta, float sm_scale, const fp_mask *mask, float *out, float *lse,
                      const fp_tuning *tuning, int32_t *status, hipStream_t stream) {
    Plan p;
    int rc = make_plan(pool, geom, mask, num_q_heads, tuning, &p);
    if (rc) return rc;
    if (!status) return FP_ERR_NULL;
    if (p.N == 0) return FP_OK;
    if (!q || !out) return FP_ERR_NULL;
    if (p.total > kScratchBytes) return FP_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((rc = scratch_ptr(&ws))) return rc;
    return attend_impl(pool, geom, q, num_q_heads, rope_theta, sm_scale, mask, out, lse, ws, kScratchBytes, tuning,
                       status, stream);
}

int64_t fp_attend_noalloc_max_bytes(void) { return (int64_t)kScratchBytes; }

int64_t fp_hazard_workspace_bytes(const fp_kv_pool *pool) {
    const int rc = check_pool(pool);
    if (rc) return rc;
    return (int64_t)3 * sizeof(int32_t) * pool->num_pages * pool->page_size;
}

int fp_check_hazards(const fp_kv_pool *pool, const fp_geometry *geom, void *workspace, size_t workspace_bytes,
                     int32_t *status, hipStream_t stream) {
    int rc = check_pool(pool);
    if (rc) return rc;
    if ((rc = check_geom(geom, pool))) return rc;
    if (geom->num_lanes > 65535) return FP_ERR_UNSUPPORTED;
    if (!status || !workspace) return FP_ERR_NULL;
    const int64_t cells = (int64_t)pool->num_pages * pool->page_size;
    if ((int64_t)workspace_bytes < fp_hazard_workspace_bytes(pool)) return FP_ERR_WORKSPACE;
    HazardArgs a;
    a.indptr = geom->indptr;
    a.slots = geom->slots;
    a.kv_len = geom->kv_len;
    a.page_indptr = pool->page_indptr;
    a.page_ids = pool->page_ids;
    a.committed = pool->committed_len;
    a.L = geom->num_lanes;
    a.num_pages = pool->num_pages;
    a.P = pool->page_size;
    a.N = geom->num_rows;
    a.cells = cells;
    a.cnt = static_cast<int32_t *>(workspace);
    a.lmin = a.cnt + cells;
    a.lmax = a.lmin + cells;
    a.status = status;
    int max_cap = 0;
    for (int l = 0; l < a.L; ++l)
        max_cap = std::max(max_cap, (pool->page_indptr_host[l + 1] - pool->page_indptr_host[l]) * a.P);
    const int64_t init_blocks = std::min<int64_t>((cells + 255) / 256, 4096);
    hipLaunchKernelGGL(hazard_init_kernel, dim3((unsigned)init_blocks), dim3(256), 0, stream, a);
    if ((rc = launch_ok())) return rc;
    if (a.N > 0) {
        const unsigned rb = (unsigned)((a.N + 255) / 256);
        hipLaunchKernelGGL(hazard_mark_kernel, dim3(rb), dim3(256), 0, stream, a);
        if ((rc = launch_ok())) return rc;
        hipLaunchKernelGGL(hazard_rows_kernel, dim3(rb), dim3(256), 0, stream, a);
        if ((rc = launch_ok())) return rc;
        if (max_cap > 0) {
            hipLaunchKernelGGL(hazard_reads_kernel, dim3((unsigned)((max_cap + 255) / 256), (unsigned)a.L), dim3(256), 0,
                               stream, a);
            if ((rc = launch_ok())) return rc;
        }
    }
    return FP_OK;
}

// Checks of a fold call; on success *blocks is its workgroup count.
static int fold_check(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *status, unsigned *blocks) {
    if (!pool || !pool->committed_len) return FP_ERR_NULL;
    if (!geom || !geom->indptr || !geom->fold || !geom->indptr_host) return FP_ERR_NULL;
    if (!status) return FP_ERR_NULL;
    if (geom->num_lanes < 1) return FP_ERR_SHAPE;
    *blocks = (unsigned)((geom->num_lanes + 255) / 256);
    return FP_OK;
}

// Checks of a readout call; on success *blocks is its workgroup count (zero
// when there is nothing to copy).
static int readout_check(const fp_geometry *geom, const float *out, int32_t row_elems, const int32_t *rows,
                         int32_t num_readout, const float *dst, const int32_t *status, unsigned *blocks) {
    if (!geom || !geom->indptr || !geom->indptr_host) return FP_ERR_NULL;
    if (geom->num_lanes < 1 || row_elems < 1 || num_readout < 0) return FP_ERR_SHAPE;
    if (!status) return FP_ERR_NULL;
    const int L = geom->num_lanes;
    const int32_t *ip = geom->indptr_host;
    if (ip[0] != 0 || ip[L] != geom->num_rows) return FP_ERR_SHAPE;
    if (!rows) {
        int nonempty = 0;
        for (int l = 0; l < L; ++l) {
            if (ip[l + 1] < ip[l]) return FP_ERR_SHAPE;
            nonempty += ip[l + 1] > ip[l];
        }
        if (nonempty != num_readout) return FP_ERR_SHAPE;
    }
    *blocks = 0;
    if (num_readout == 0) return FP_OK;
    if (!out || !dst) return FP_ERR_NULL;
    *blocks = rows ? (unsigned)num_readout : (unsigned)L;
    return FP_OK;
}

int fp_fold(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *channel, int32_t *status,
            hipStream_t stream) {
    unsigned fb = 0;
    int rc = fold_check(pool, geom, status, &fb);
    if (rc) return rc;
    hipLaunchKernelGGL(fold_kernel, dim3(fb), dim3(256), 0, stream, geom->indptr, geom->fold, channel,
                       pool->committed_len, geom->num_lanes, status);
    return launch_ok();
}

int fp_readout(const fp_geometry *geom, const float *out, int32_t row_elems, const int32_t *rows, int32_t num_readout,
               float *dst, int32_t *status, hipStream_t stream) {
    unsigned rb = 0;
    int rc = readout_check(geom, out, row_elems, rows, num_readout, dst, status, &rb);
    if (rc) return rc;
    if (rb == 0) return FP_OK;
    hipLaunchKernelGGL(readout_kernel, dim3(rb), dim3(256), 0, stream, geom->indptr, geom->num_lanes,
                       (int64_t)geom->num_rows, out, row_elems, rows, num_readout, dst, status);
    return launch_ok();
}

int fp_fold_readout(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *channel, const float *out,
                    int32_t row_elems, const int32_t *rows, int32_t num_readout, float *dst, int32_t *status,
                    hipStream_t stream) {
    unsigned fb = 0, rb = 0;
    int rc = fold_check(pool, geom, status, &fb);
    if (rc) return rc;
    if ((rc = readout_check(geom, out, row_elems, rows, num_readout, dst, status, &rb))) return rc;
    hipLaunchKernelGGL(fold_readout_kernel, dim3(fb + rb), dim3(256), 0, stream, geom->indptr, geom->fold, channel,
                       pool->committed_len, geom->num_lanes, (int)fb, (int64_t)geom->num_rows, out, row_elems, rows,
                       num_readout, dst, status);
    return launch_ok();
}

int fp_attn_mass(const fp_kv_pool *pool, const fp_geometry *geom, int32_t num_q_heads, const fp_mask *mask,
                 const float *lse, const void *workspace, size_t workspace_bytes, const fp_tuning *tuning,
                 float *slot_mass, hipStream_t stream) {
    Plan p;
    int rc = make_plan(pool, geom, mask, num_q_heads, tuning, &p);
    if (rc) return rc;
    if (p.N == 0) return FP_OK;
    if (!lse || !workspace || !slot_mass) return FP_ERR_NULL;
    if (workspace_bytes < sizeof(uint16_t) * (size_t)p.N * p.Hq * p.D) return FP_ERR_WORKSPACE;  // the rotated Q
    const int32_t *pp = pool->page_indptr_host;
    int max_pages = 0;
    for (int l = 0; l < p.L; ++l) max_pages = std::max(max_pages, pp[l + 1] - pp[l]);
    const int64_t chunks = ((int64_t)max_pages * p.P + 32 * kMassTiles - 1) / (32 * kMassTiles);
    if (chunks == 0) return FP_OK;
    if (chunks > 65535) return FP_ERR_UNSUPPORTED;
    MassArgs m;
    m.pool = static_cast<const uint16_t *>(pool->kv);
    m.page_elems = 2LL * p.H * p.P * p.D;
    m.num_pages = pool->num_pages;
    m.P = p.P; m.H = p.H; m.G = p.G; m.Hq = p.Hq;
    m.page_indptr = pool->page_indptr;
    m.page_ids = pool->page_ids;
    m.indptr = geom->indptr;
    m.slots = geom->slots;
    m.kv_len = geom->kv_len;
    m.qrot = reinterpret_cast<const uint16_t *>(static_cast<const char *>(workspace) + p.off_qrot);
    m.lse = lse;
    m.mask_bits = mask ? mask->bits : nullptr;
    m.mask_off = mask ? mask->word_offset : nullptr;
    m.mass = slot_mass;
    m.stride = (int64_t)pp[p.L] * p.P;
    m.chunks = (int)chunks;
    m.L = p.L;
    // lanes with rows x G <= 32 go to the decode-class kernel, the others to the chunked one
    bool any_dec = false, any_pre = false;
    for (int l = 0; l < p.L; ++l) {
        const int n = geom->indptr_host[l + 1] - geom->indptr_host[l];
        if (n > 0 && n * p.G <= 32) any_dec = true;
        if (n * p.G > 32) any_pre = true;
    }
    const dim3 block(64 * kMassWaves);
    if (any_pre) {
        const int64_t rounds = ((int64_t)p.L * p.H + kXcds - 1) / kXcds;  // pairs per XCD
        const dim3 grid((unsigned)(kXcds * rounds * chunks));
        if (p.D == 128) hipLaunchKernelGGL(mass_kernel<128>, grid, block, 0, stream, m);
        else hipLaunchKernelGGL(mass_kernel<64>, grid, block, 0, stream, m);
        if ((rc = launch_ok())) return rc;
    }
    if (any_dec) {
        const int64_t tiles = ((int64_t)max_pages * p.P + 31) / 32;
        const int64_t per_wg = (int64_t)kMassWaves * kMassWaveTiles;
        const dim3 grid((unsigned)(p.L * p.H), (unsigned)((tiles + per_wg - 1) / per_wg));
        if (p.D == 128) hipLaunchKernelGGL(mass_decode_kernel<128>, grid, block, 0, stream, m);
        else hipLaunchKernelGGL(mass_decode_kernel<64>, grid, block, 0, stream, m);
        if ((rc = launch_ok())) return rc;
    }
    return FP_OK;
}

namespace {
// (lane, 32-row block) work items of a pass, from the host copy of indptr
int64_t lora_items(const fp_geometry *geom) {
    int64_t t = 0;
    for (int l = 0; l < geom->num_lanes; ++l) {
        const int n = geom->indptr_host[l + 1] - geom->indptr_host[l];
        if (n > 0) t += (n + 31) / 32;
    }
    return t;
}
}  // namespace

int64_t fp_lora_workspace_bytes(const fp_geometry *geom, const fp_lora *lora) {
    if (!geom || !lora || !geom->indptr_host) return FP_ERR_NULL;
    if (geom->num_rows < 0 || geom->num_lanes < 1 || lora->rank < 1) return FP_ERR_SHAPE;
    const int rp = (lora->rank + 31) / 32 * 32;
    return (int64_t)(align256(2 * sizeof(uint16_t) * (size_t)geom->num_rows * rp) +
                     align256(sizeof(int4) * (size_t)lora_items(geom)));
}

int fp_adapter_lora(const fp_geometry *geom, const fp_lora *lora, const int32_t *adapter, const void *x,
                    const void *y, void *out, void *workspace, size_t workspace_bytes, int32_t *status,
                    hipStream_t stream) {
    if (!geom || !lora || !geom->indptr || !geom->indptr_host || !status) return FP_ERR_NULL;
    if (geom->num_lanes < 1 || geom->num_lanes > kMaxLanes || geom->num_rows < 0) return FP_ERR_SHAPE;
    const int32_t *ip = geom->indptr_host;
    if (ip[0] != 0 || ip[geom->num_lanes] != geom->num_rows) return FP_ERR_SHAPE;
    for (int l = 0; l < geom->num_lanes; ++l)
        if (ip[l + 1] < ip[l]) return FP_ERR_SHAPE;
    if (lora->num_adapters < 1 || lora->d_in < 1 || lora->d_out < 1) return FP_ERR_SHAPE;
    if (lora->rank % 16 || lora->rank < 16 || lora->rank > 64 || lora->d_in % 64 || lora->d_out % 32 ||
        (int64_t)lora->d_out > (int64_t)65535 * kLoraCols * kLoraBlocks)
        return FP_ERR_UNSUPPORTED;
    if (geom->num_rows == 0) return FP_OK;
    if (!adapter || !x || !y || !out || !lora->a || !lora->b || !lora->scale || !workspace) return FP_ERR_NULL;
    if ((int64_t)workspace_bytes < fp_lora_workspace_bytes(geom, lora)) return FP_ERR_WORKSPACE;
    LoraArgs a;
    a.indptr = geom->indptr;
    a.L = geom->num_lanes;
    a.adapter = adapter;
    a.n_ad = lora->num_adapters;
    a.r = lora->rank;
    a.rp = (lora->rank + 31) / 32 * 32;
    a.d_in = lora->d_in;
    a.d_out = lora->d_out;
    a.x = static_cast<const uint16_t *>(x);
    a.y = static_cast<const uint16_t *>(y);
    a.out = static_cast<uint16_t *>(out);
    a.a = static_cast<const uint16_t *>(lora->a);
    a.b = static_cast<const uint16_t *>(lora->b);
    a.scale = lora->scale;
    const int64_t n_items = lora_items(geom);
    if (n_items > INT32_MAX / 2) return FP_ERR_UNSUPPORTED;
    a.v = static_cast<uint16_t *>(workspace);
    a.N = geom->num_rows;
    int4 *items = reinterpret_cast<int4 *>(static_cast<char *>(workspace) +
                                           align256(2 * sizeof(uint16_t) * (size_t)geom->num_rows * a.rp));
    a.items = items;
    a.n_items = (int)n_items;
    a.status = status;
    a.in_place = out == y;
    hipLaunchKernelGGL(lora_plan_kernel, dim3(1), dim3(kLoraPlanThreads), 0, stream, geom->indptr, a.L, adapter,
                       items, a.n_items, status);
    int rc = launch_ok();
    if (rc) return rc;
    const dim3 block(64 * kLoraWaves);
    const dim3 grid((unsigned)n_items);
    switch (a.r / 16) {
        case 1: hipLaunchKernelGGL(lora_shrink_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(lora_shrink_kernel<2>, grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(lora_shrink_kernel<3>, grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL(lora_shrink_kernel<4>, grid, block, 0, stream, a); break;
    }
    if ((rc = launch_ok())) return rc;
    const dim3 egrid((unsigned)n_items, (unsigned)((a.d_out + kLoraCols * kLoraBlocks - 1) / (kLoraCols * kLoraBlocks)));
    switch (a.r / 16) {
        case 1: hipLaunchKernelGGL(lora_expand_kernel<1>, egrid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(lora_expand_kernel<2>, egrid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(lora_expand_kernel<3>, egrid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL(lora_expand_kernel<4>, egrid, block, 0, stream, a); break;
    }
    return launch_ok();
}

int fp_adapter_ia3(const fp_geometry *geom, int32_t num_adapters, int32_t d_out, const void *scale,
                   const int32_t *adapter, const void *y, void *out, int32_t *status, hipStream_t stream) {
    if (!geom || !geom->indptr || !geom->indptr_host || !status) return FP_ERR_NULL;
    if (geom->num_lanes < 1 || geom->num_rows < 0 || num_adapters < 1 || d_out < 1) return FP_ERR_SHAPE;
    if (d_out % 8) return FP_ERR_UNSUPPORTED;
    const int32_t *ip = geom->indptr_host;
    if (ip[0] != 0 || ip[geom->num_lanes] != geom->num_rows) return FP_ERR_SHAPE;
    for (int l = 0; l < geom->num_lanes; ++l)
        if (ip[l + 1] < ip[l]) return FP_ERR_SHAPE;
    if (geom->num_rows == 0) return FP_OK;
    if (!scale || !adapter || !y || !out) return FP_ERR_NULL;
    hipLaunchKernelGGL(ia3_kernel, dim3((unsigned)geom->num_rows), dim3(kIa3Threads), 0, stream, geom->indptr,
                       geom->num_lanes, adapter, num_adapters, d_out, static_cast<const uint16_t *>(scale),
                       static_cast<const uint16_t *>(y), static_cast<uint16_t *>(out), status);
    return launch_ok();
}

int fp_tova_mask(const fp_kv_pool *pool, const fp_geometry *geom, const float *slot_mass, const int32_t *budget,
                 const uint32_t *prev_keep, const int32_t *prev_limit, const int64_t *keep_word_offset,
                 uint32_t *keep, uint32_t *mask_bits, const int64_t *mask_word_offset,
                 const int64_t *mask_word_offset_host, int32_t *status, hipStream_t stream) {
    int rc = check_pool(pool);
    if (rc) return rc;
    if ((rc = check_geom(geom, pool))) return rc;
    if (!slot_mass || !budget || !keep_word_offset || !keep || !mask_bits || !mask_word_offset ||
        !mask_word_offset_host || !status)
        return FP_ERR_NULL;
    if (prev_keep && !prev_limit) return FP_ERR_NULL;
    const fp_mask m{mask_bits, mask_word_offset, mask_word_offset_host};
    if ((rc = check_mask(&m, geom))) return rc;
    const int L = geom->num_lanes;
    TovaArgs ta{};
    ta.mass = slot_mass;
    ta.S = (int64_t)pool->page_indptr_host[L] * pool->page_size;
    ta.H = pool->num_kv_heads;
    ta.P = pool->page_size;
    ta.L = L;
    ta.page_indptr = pool->page_indptr;
    ta.committed = pool->committed_len;
    ta.budget = budget;
    ta.prev_limit = prev_limit;
    ta.prev_keep = prev_keep;
    ta.keep_off = keep_word_offset;
    ta.keep = keep;
    hipLaunchKernelGGL(tova_select_kernel, dim3((unsigned)L), dim3(kTovaThreads), 0, stream, ta);
    if ((rc = launch_ok())) return rc;
    if (geom->num_rows == 0) return FP_OK;
    TovaRowArgs ra{};
    ra.indptr = geom->indptr;
    ra.slots = geom->slots;
    ra.kv_len = geom->kv_len;
    ra.committed = pool->committed_len;
    ra.page_indptr = pool->page_indptr;
    ra.L = L;
    ra.P = pool->page_size;
    ra.keep = keep;
    ra.keep_off = keep_word_offset;
    ra.mask_off = mask_word_offset;
    ra.mask = mask_bits;
    ra.status = status;
    hipLaunchKernelGGL(tova_rows_kernel, dim3((unsigned)geom->num_rows), dim3(256), 0, stream, ra);
    return launch_ok();
}

int fp_advance(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *pos_offset, int32_t *positions,
               int32_t *slots, int32_t *kv_len, hipStream_t stream) {
    if (!pool || !pool->committed_len) return FP_ERR_NULL;
    if (!geom || !geom->indptr || !geom->indptr_host || !kv_len) return FP_ERR_NULL;
    if (geom->num_lanes < 1 || geom->num_rows < 0) return FP_ERR_SHAPE;
    const int32_t *ip = geom->indptr_host;
    if (ip[0] != 0 || ip[geom->num_lanes] != geom->num_rows) return FP_ERR_SHAPE;
    for (int l = 0; l < geom->num_lanes; ++l)
        if (ip[l + 1] < ip[l]) return FP_ERR_SHAPE;
    if (geom->num_rows > 0 && (!positions || !slots)) return FP_ERR_NULL;
    const int n = geom->num_lanes > geom->num_rows ? geom->num_lanes : geom->num_rows;
    hipLaunchKernelGGL(advance_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, geom->indptr,
                       pool->committed_len, pos_offset, geom->num_lanes, geom->num_rows, positions, slots, kv_len);
    return launch_ok();
}

int fp_vertical_merge(int32_t L, const int32_t *indptr_a, const int32_t *slots_a, const int32_t *kv_len_a,
                      const int32_t *fold_a, const int32_t *indptr_b, const int32_t *slots_b,
                      const int32_t *kv_len_b, const int32_t *fold_b, const int32_t *committed,
                      const int32_t *page_indptr_host, int32_t page_size, int32_t *indptr_m, int32_t *src_row,
                      int32_t *row_of_a, int32_t *row_of_b, int32_t *kv_len_m, int32_t *fold_m) {
    if (!indptr_a || !indptr_b || !kv_len_a || !kv_len_b || !fold_a || !fold_b || !committed || !page_indptr_host ||
        !indptr_m || !src_row || !row_of_a || !row_of_b || !kv_len_m || !fold_m)
        return FP_ERR_NULL;
    if (L < 1 || page_size < 1 || indptr_a[0] != 0 || indptr_b[0] != 0) return FP_ERR_SHAPE;
    for (int l = 0; l < L; ++l)
        if (indptr_a[l + 1] < indptr_a[l] || indptr_b[l + 1] < indptr_b[l]) return FP_ERR_SHAPE;
    const int32_t NA = indptr_a[L], NB = indptr_b[L];
    if ((NA > 0 && !slots_a) || (NB > 0 && !slots_b)) return FP_ERR_NULL;
    // eligibility first: nothing is written unless every lane qualifies
    for (int l = 0; l < L; ++l) {
        const int a0 = indptr_a[l], na = indptr_a[l + 1] - a0;
        const int b0 = indptr_b[l], nb = indptr_b[l + 1] - b0;
        const int64_t c = committed[l];
        const int64_t cap = (int64_t)(page_indptr_host[l + 1] - page_indptr_host[l]) * page_size;
        if (kv_len_a[l] < 0 || kv_len_a[l] > cap || kv_len_b[l] < 0 || kv_len_b[l] > cap) return 1;
        if (!(fold_a[l] == FP_FOLD_ALL || fold_a[l] == na)) return 1;
        if (!(fold_b[l] == FP_FOLD_ALL || (fold_b[l] >= 0 && fold_b[l] <= nb))) return 1;
        for (int i = 0; i < na; ++i)
            if (slots_a[a0 + i] != c + i) return 1;
        if (na > 0 && kv_len_a[l] < c + na) return 1;
        if (nb > 0 && na > 0 && kv_len_b[l] < c + na) return 1;
        for (int i = 0; i < nb; ++i)
            if (slots_b[b0 + i] < c + na) return 1;
    }
    indptr_m[0] = 0;
    for (int l = 0; l < L; ++l) {
        const int a0 = indptr_a[l], na = indptr_a[l + 1] - a0;
        const int b0 = indptr_b[l], nb = indptr_b[l + 1] - b0;
        int m = indptr_m[l];
        for (int i = 0; i < na; ++i, ++m) {
            src_row[m] = a0 + i;
            row_of_a[a0 + i] = m;
        }
        for (int i = 0; i < nb; ++i, ++m) {
            src_row[m] = NA + b0 + i;
            row_of_b[b0 + i] = m;
        }
        indptr_m[l + 1] = m;
        kv_len_m[l] = nb > 0 ? kv_len_b[l] : kv_len_a[l];
        fold_m[l] = fold_b[l] == FP_FOLD_ALL ? FP_FOLD_ALL : na + fold_b[l];
    }
    return FP_OK;
}

uint64_t fp_kv_bytes(int32_t L, int32_t H_kv, int32_t d, uint64_t T, int32_t b) {
    return 2ull * (uint64_t)L * (uint64_t)H_kv * (uint64_t)d * T * (uint64_t)b;
}

uint64_t fp_pages_for(uint64_t T, int32_t P) { return P > 0 ? (T + (uint64_t)P - 1) / (uint64_t)P : 0; }

uint64_t fp_page_waste(uint64_t T, int32_t P) { return P > 0 ? fp_pages_for(T, P) * (uint64_t)P - T : 0; }

uint64_t fp_page_bytes(int32_t P, int32_t H_kv, int32_t d) { return 2ull * (uint64_t)H_kv * (uint64_t)P * (uint64_t)d * 2ull; }

const char *fp_version(void) { return "ragged_paged_kv_fp_amd 0.2 (gfx950)"; }

#ifndef FP_SOURCE_HASH
#define FP_SOURCE_HASH "unknown"
#endif
const char *fp_source_hash(void) { return FP_SOURCE_HASH; }

}  // extern "C"
