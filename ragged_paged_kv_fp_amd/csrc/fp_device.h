// fp_device.h - device helpers shared by the kernels of the ForwardPass attention step.
// gfx950 (CDNA4) only: 64-lane waves, bf16 MFMA 32x32x16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fpk {

constexpr int kWave = 64;
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt encoding: vmcnt(0), other counters unconstrained
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// 16-byte load marked non-temporal: data read once per pass (the decode KV
// stream) bypasses the cache reuse policy, which lets HBM reads run closer to
// peak.
__device__ __forceinline__ uint4 load_nt(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Nearest-even bf16 of a double in one rounding, the general path: truncate
// to float (toward zero), set the last float bit if anything was dropped
// (round-to-odd), then round that float to bf16 nearest-even. Float keeps
// enough extra bits for the two steps to equal one correct rounding.
__device__ __forceinline__ uint32_t f64_to_bf16_slow(double x) {
    float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if ((double)f != x) u |= 1u;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Nearest-even bf16 of a double in one rounding. When the double's exponent
// lies in bf16's normal range, rounding its 52-bit significand to 7 bits at
// bit 45 (adding 2^44 - 1 plus the kept last bit) is that rounding, a carry
// into the exponent included (up to infinity); the exponent is then rebiased
// from 1023 to 127. Zeros, bf16 subnormals, infinities and NaN take the
// general path.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t e = (uint32_t)(b >> 52) & 0x7FFu;
    if (e - 897u > 1150u - 897u) return f64_to_bf16_slow(x);
    const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
    const uint32_t r = (uint32_t)((mag + 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45);  // exponent | 7 bits
    return (r - (896u << 7)) | ((uint32_t)(b >> 48) & 0x8000u);
}

constexpr int kMaxPairs = 64;  // head_dim / 2 for head_dim <= 128

// Frequencies of the RoPE pairs, w_i = theta^(-2i/d), filled on the host in fp64.
struct RopeFreqs {
    double w[kMaxPairs];
};

// cos and sin of the rotation angle pos * w_i of RoPE pair i, in fp64.
__device__ __forceinline__ void rope_cos_sin(int pos, double w, double *c, double *s) {
    sincos((double)pos * w, s, c);
}

// Largest lane l with indptr[l] <= row (rows of lane l are [indptr[l], indptr[l+1])).
__device__ __forceinline__ int find_lane(const int32_t *indptr, int num_lanes, int64_t row) {
    int lo = 0, hi = num_lanes;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)indptr[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ int clamp_kv(int kv, int cap) { return kv < 0 ? 0 : (kv > cap ? cap : kv); }

// Row of the 32-row K operand that holds tile slot pi(m). Chosen so that, after
// S^T = K * Q^T, lane half h holds the scores of tile slots 8h..8h+7 in
// accumulator registers 0..7 and 16+8h..16+8h+7 in registers 8..15: exactly
// the B-operand layout the P*V product needs, so P never moves between lanes.
__device__ __forceinline__ int kslot_of_row(int m) {
    return 16 * ((m >> 3) >> 1) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> two bf16 (nearest-even) in one register, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int wave_max_i(int v) {
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

}  // namespace fpk
