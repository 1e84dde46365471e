// fp_peaks.hip - two microbenchmarks of the device the step runs on, so that
// roofline fractions can be stated against measured peaks beside the vendor
// figures: a read-only HBM stream and a bf16 MFMA loop. Measurement code
// only (libfp_peaks.so, loaded by the benchmark); the step never uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread

// Workgroup b reads the contiguous chunk [b * chunk, (b + 1) * chunk) of the
// buffer in 16-byte non-temporal loads, kReadUnroll of them in flight per
// thread, and folds them with XOR; the fold is stored only where it equals a
// value it cannot take for the buffer's contents, so no load is dead.
__global__ void __launch_bounds__(kReadThreads) read_stream_kernel(const u32x4 *src, int64_t chunk16, int64_t n16,
                                                                   uint32_t never, uint32_t *sink) {
    const int64_t begin = (int64_t)blockIdx.x * chunk16;
    const int64_t end = begin + chunk16 < n16 ? begin + chunk16 : n16;
    uint32_t acc = 0;
    int64_t i = begin + threadIdx.x;
    for (; i + (kReadUnroll - 1) * kReadThreads < end; i += kReadUnroll * kReadThreads) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kReadThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += kReadThreads) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never) sink[threadIdx.x] = acc;
}

constexpr int kChains = 4;  // independent accumulators per wave: the MFMA pipe never waits on a result

// Every wave issues iters x kChains v_mfma_f32_32x32x16_bf16 on register
// operands (32*32*16*2 flop each) and stores a sum of its results only where
// it equals a value the chains cannot produce.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float never, float *sink) {
    const uint32_t t = threadIdx.x;
    u32x4 ua = {0x3F803F80u ^ t, 0x3F003F00u, 0x3E803E80u, 0x3F803F00u};
    u32x4 ub = {0x3F003F80u, 0x3E803F80u ^ (t << 16), 0x3F803E80u, 0x3F003F00u};
    const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
    f32x16 c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][15];
    if (s == never) sink[t] = s;
}

}  // namespace

extern "C" {

// One read pass over `bytes` (a multiple of 16) of device memory at `buf`, in
// `blocks` workgroups of contiguous chunks. sink: >= 256 uint32 of device memory.
int fp_peak_read(const void *buf, int64_t bytes, int32_t blocks, void *sink, hipStream_t stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 || blocks < 1) return -1;
    const int64_t n16 = bytes / 16;
    const int64_t chunk16 = (n16 + blocks - 1) / blocks;
    hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), chunk16, n16, 0xA5A5A5A5u, static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// `blocks` workgroups of four waves, each wave issuing iters * 4 bf16 MFMAs of
// 32768 flop. sink: >= 256 floats of device memory.
int fp_peak_mfma(int32_t iters, int32_t blocks, void *sink, hipStream_t stream) {
    if (!sink || iters < 1 || blocks < 1) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, -1234.5f,
                       static_cast<float *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Flop of one fp_peak_mfma launch.
double fp_peak_mfma_flop(int32_t iters, int32_t blocks) {
    return (double)blocks * 4.0 * (double)iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

}  // extern "C"
