// Device helpers shared by the gfx950 kernels: element loads with widening to
// fp32, bf16 rounding for stores, the log-decay conversion and wave-level
// reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace wkv7 {

using bf16_t = uint16_t;  // bf16 bit pattern
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// Read-only global memory viewed through the constant address space: a load
// from it at a wave-uniform address becomes a scalar (SMEM) load into SGPRs.
template <typename T> using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const T* p) { return (cptr<T>)(p); }

__device__ __forceinline__ void ld8u(cptr<float> p, int64_t i, float* o) {
    #pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = p[i + c];
}
__device__ __forceinline__ void ld8u(cptr<bf16_t> p, int64_t i, float* o) {
    cptr<uint32_t> q = (cptr<uint32_t>)(p + i);
    #pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t x = q[c];
        o[2 * c] = __uint_as_float(x << 16);
        o[2 * c + 1] = __uint_as_float(x & 0xffff0000u);
    }
}

template <typename T> using gptr = const __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> as_global(const T* p) { return (gptr<T>)(p); }

// Widen one element.
__device__ __forceinline__ float ld1(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld1(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// Load 4 consecutive elements starting at p + i (i a multiple of 4, 16-byte
// aligned base), widened to fp32.
__device__ __forceinline__ void ld4(const float* p, int64_t i, float* o) {
    float4 x = *reinterpret_cast<const float4*>(p + i);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
}
__device__ __forceinline__ void ld4(const bf16_t* p, int64_t i, float* o) {
    uint2 x = *reinterpret_cast<const uint2*>(p + i);
    o[0] = __uint_as_float(x.x << 16); o[1] = __uint_as_float(x.x & 0xffff0000u);
    o[2] = __uint_as_float(x.y << 16); o[3] = __uint_as_float(x.y & 0xffff0000u);
}
// 8 consecutive elements (i a multiple of 8).
__device__ __forceinline__ void ld8(const float* p, int64_t i, float* o) {
    ld4(p, i, o); ld4(p, i + 4, o + 4);
}
__device__ __forceinline__ void ld8(const bf16_t* p, int64_t i, float* o) {
    uint4 x = *reinterpret_cast<const uint4*>(p + i);
    o[0] = __uint_as_float(x.x << 16); o[1] = __uint_as_float(x.x & 0xffff0000u);
    o[2] = __uint_as_float(x.y << 16); o[3] = __uint_as_float(x.y & 0xffff0000u);
    o[4] = __uint_as_float(x.z << 16); o[5] = __uint_as_float(x.z & 0xffff0000u);
    o[6] = __uint_as_float(x.w << 16); o[7] = __uint_as_float(x.w & 0xffff0000u);
}

__device__ __forceinline__ void st1(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st1(bf16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }

// decay = exp(-exp(x)) for the log-decay input mode, via the hardware exp2.
__device__ __forceinline__ float decay_from_logneglog(float x) {
    float e = __builtin_amdgcn_exp2f(x * kLog2e);
    return __builtin_amdgcn_exp2f(-e * kLog2e);
}
// log2(decay) for both modes.
__device__ __forceinline__ float log2_decay(float x, bool logneglog) {
    if (logneglog) return -__builtin_amdgcn_exp2f(x * kLog2e) * kLog2e;
    return __builtin_amdgcn_logf(x);
}

// 1 / max(|k|, 1e-12) from the sum of squares |k|^2: the scale of the
// normalised key kk = k / max(|k|, 1e-12) (L2 normalisation with a floor).
__device__ __forceinline__ float inv_key_norm(float sumsq) {
    return 1.f / fmaxf(__builtin_sqrtf(sumsq), 1e-12f);
}

// Make the compiler materialise x here (inserting any wait for the load
// that produced it at this point rather than at a later first use).
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(uint32_t& x) { asm volatile("" : "+v"(x)); }

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum16(float x) {
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppRowHalfMirror>(x);
    x += dpp<kDppRowMirror>(x);
    return x;
}

}  // namespace wkv7
