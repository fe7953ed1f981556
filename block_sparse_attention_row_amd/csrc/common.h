// Device-side helpers shared by the gfx950 kernels of libsparse_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

constexpr int kTokensPerBlock = 64;
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;   // log2 headroom before the online-softmax max is moved

// bf16 <-> fp32 as raw 16-bit patterns (bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even, two values packed in one dword
// (a in the low half).  NaN inputs do not occur on these paths.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    ua += 0x7fffu + ((ua >> 16) & 1u);
    ub += 0x7fffu + ((ub >> 16) & 1u);
    return (ua >> 16) | (ub & 0xffff0000u);
}

template <typename T> struct DType;
template <> struct DType<float> { static constexpr int code = 0; };
template <> struct DType<__bf16> { static constexpr int code = 1; };

// Integer wave sums and scans through DPP lane moves.
template <int CTRL> __device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int s) {
    s += dppi<0xB1>(s);
    s += dppi<0x4E>(s);
    s += dppi<0x141>(s);
    s += dppi<0x140>(s);
    return __builtin_amdgcn_readlane(s, 0) + __builtin_amdgcn_readlane(s, 16) + __builtin_amdgcn_readlane(s, 32) +
           __builtin_amdgcn_readlane(s, 48);
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
    v += dppi<0x111>(v);
    v += dppi<0x112>(v);
    v += dppi<0x114>(v);
    v += dppi<0x118>(v);
    const int q0 = __builtin_amdgcn_readlane(v, 15), q1 = __builtin_amdgcn_readlane(v, 31),
              q2 = __builtin_amdgcn_readlane(v, 47);
    const int row16 = lane >> 4;
    return v + (row16 >= 1 ? q0 : 0) + (row16 >= 2 ? q1 : 0) + (row16 >= 3 ? q2 : 0);
}

// Wave-wide reductions over 64 lanes (results in every lane).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// DPP lane moves within 16-lane rows (no LDS round trip); lanes without a source read 0.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppWaveShl1 = 0x130;  // lane l takes lane l + 1 (whole wave)
constexpr int kDppWaveShr1 = 0x138;  // lane l takes lane l - 1 (whole wave)
// ds_swizzle bit mode within 32-lane groups (and 0x1f, or 0, xor 31): lane l takes 31 - l
constexpr int kSwizzleXor31 = (31 << 10) | 0x1f;

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Max / sum over the whole wave, returned uniformly (reduced per row with DPP, then
// the four row results read out with v_readlane).
__device__ __forceinline__ float wave_max_u(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum_u(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
    v += dpp<kDppShr1>(v);
    v += dpp<kDppShr2>(v);
    v += dpp<kDppShr4>(v);
    v += dpp<kDppShr8>(v);
    const float r0 = lane_value(v, 15), r1 = lane_value(v, 31), r2 = lane_value(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
}

template <int CTRL> __device__ __forceinline__ uint32_t dppu(uint32_t v, uint32_t fill) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, 0xF, 0xF, false);
}
// Unsigned min / max over the wave, returned uniformly.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dppu<kDppXor1>(v, v));
    v = min(v, dppu<kDppXor2>(v, v));
    v = min(v, dppu<kDppHalfMirror>(v, v));
    v = min(v, dppu<kDppMirror>(v, v));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32_u(uint32_t v) {
    v = max(v, dppu<kDppXor1>(v, v));
    v = max(v, dppu<kDppXor2>(v, v));
    v = max(v, dppu<kDppHalfMirror>(v, v));
    v = max(v, dppu<kDppMirror>(v, v));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

// Combine each lane with its partner l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bijective mapping of a flat work index so that the workgroups the hardware
// sends to one XCD (dispatch is round-robin over the 8 XCDs) receive a
// contiguous range of work items: neighbouring rows then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
    constexpr int64_t kXcd = 8;
    const int64_t x = bid % kXcd, k = bid / kXcd;
    const int64_t per = n / kXcd, rem = n % kXcd;
    return x * per + (x < rem ? x : rem) + k;
}

// Like xcd_remap, but the work items are dealt to the XCDs in runs of C consecutive
// items, round-robin: every XCD still works on neighbouring items at any moment
// (they share its L2), while items whose cost drifts along the index (heads with
// different thresholds) spread evenly over the XCDs.  Items past the last whole
// round of runs fall back to xcd_remap.  A bijection on [0, n).
template <int64_t C> __device__ __forceinline__ int64_t xcd_chunk_remap(int64_t bid, int64_t n) {
    constexpr int64_t kXcd = 8;
    const int64_t full = n / (kXcd * C) * (kXcd * C);
    if (bid >= full) return full + xcd_remap(bid - full, n - full);
    const int64_t x = bid % kXcd, k = bid / kXcd;
    return (k / C) * (kXcd * C) + x * C + k % C;
}

// (1, 1) in bf16, for row sums with v_dot2_f32_bf16
#define kOnes2 ((bf16x2){(__bf16)1.0f, (__bf16)1.0f})

// Exclusive prefix over the 1024 threads (thread order) and the total.
__device__ __forceinline__ int32_t block_scan32(int32_t v, int32_t *lds16, int32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    __syncthreads();
    if (lane == 63) lds16[wave] = incl;
    __syncthreads();
    int32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const int32_t x = lds16[w];
        before += w < wave ? x : 0;
        tot += x;
    }
    total = tot;
    return before + incl - v;
}

}  // namespace sattn
