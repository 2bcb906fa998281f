// Shared by the two passes of the D = 128 two-pass form (wkv7_twopass128.hip:
// the per-chunk matrices on bf16 matrix cores; wkv7_twopass128_scan.hip: the
// chunk recurrence on fp16 matrix cores): chunk geometry, the layout of the
// workspace record that pass 1 writes and pass 2 reads, and small device helpers.
#pragma once

#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace tp128 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int L = 32;          // chunk length
constexpr int DK = 128;        // head size
constexpr int DV = 32;         // value rows per pass-2 workgroup
constexpr int NSLICE = DK / DV;
constexpr int PT = 40;         // 16-bit pitch of [*][L] operands (LDS)

// Workspace record of one (b, h, chunk).  Every operand is a single fp16 value (the
// recurrence's matrix-core type; fp16's 11-bit significand keeps a single W, Q, Bh,
// E or P operand inside the error budget where bf16 needed hi + lo pairs for Q, E
// and P, at half the bytes).  Blocks of 1 KB hold one fp16x8 operand per lane (lane l at byte 16 l).
// Per key pair kp (keys 32 kp .. 32 kp + 31), block:
//   0, 1   W   as the A operand of W (m = token of block tb, k = key), tb = 0, 1
//   2, 3   Q   same layout as W
//   4, 5   Bh  as the A operand of Bh^T (m = key of tile 2 kp + u, k = token), u = 0, 1
//   6, 7   E   same layout as Bh
// then P (A operand, m = token of block tb, k = token), tb = 0, 1; d[128] fp32;
// bonus[32] fp32.
constexpr int WS_BLK = 1024;
constexpr int WS_KP = 8 * WS_BLK;
constexpr int BLK_W = 0, BLK_Q = 2, BLK_BH = 4, BLK_E = 6;
constexpr int WS_P = 4 * WS_KP;
constexpr int WS_D = WS_P + 2 * WS_BLK;
constexpr int WS_BON = WS_D + DK * 4;
constexpr int WS_CHUNK = 35584;
static_assert(WS_BON + L * 4 <= WS_CHUNK && WS_CHUNK % 256 == 0 && WS_CHUNK - 256 < WS_BON + L * 4,
              "workspace record");

// Position of index k of a 32-deep contraction block in its pair-interleaved
// storage: position 8 q + 4 e + r holds index 16 e + 4 q + r.
__host__ __device__ constexpr int pairpos(int k) {
    return 32 * (k >> 5) + 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3);
}

template <typename T> __device__ __forceinline__ T lds(const char* base, int byte_off) {
    return *reinterpret_cast<const T*>(base + byte_off);
}
template <typename T> __device__ __forceinline__ void sts(char* base, int byte_off, T v) {
    *reinterpret_cast<T*>(base + byte_off) = v;
}
__device__ __forceinline__ f32x4 ld_f32x4(const char* p) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    return f32x4{x.x, x.y, x.z, x.w};
}
__device__ __forceinline__ uint32_t dpp_u32_xor1(uint32_t x) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppQuadXor1, 0xF, 0xF, false));
}

// fp16 conversions (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
    f16x2 v = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16lo_f32(uint32_t p) {
    return static_cast<float>(__builtin_bit_cast(f16x2, p)[0]);
}
__device__ __forceinline__ float f16hi_f32(uint32_t p) {
    return static_cast<float>(__builtin_bit_cast(f16x2, p)[1]);
}
// Two C-layout tiles (lane values 4 each) as one 32-deep fp16 operand.
__device__ __forceinline__ f16x8 to_f16x8(const f32x4 c0, const f32x4 c1) {
    return __builtin_bit_cast(f16x8, make_uint4(pack_f16(c0[0], c0[1]), pack_f16(c0[2], c0[3]),
                                                pack_f16(c1[0], c1[1]), pack_f16(c1[2], c1[3])));
}

__device__ __forceinline__ f16x8 cat16(uint2 a, uint2 b) {
    return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// x = hi + lo, both fp16 (x - hi is exact in fp32).
__device__ __forceinline__ void split2h(float x, float y, uint32_t& hi, uint32_t& lo) {
    hi = pack_f16(x, y);
    lo = pack_f16(x - f16lo_f32(hi), y - f16hi_f32(hi));
}

constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, int(n), kRsrcWord3);
}

// Chunk descriptor: tokens [c0, c0 + L) of sequence bb, clipped at T (the rest reads 0).
__device__ __forceinline__ rsrc_t chunk_rsrc(const char* base, int64_t tok0, int c0, int T, uint32_t stride) {
    const int nv = max(0, min(T - c0, L));
    const int64_t t0 = nv > 0 ? tok0 + c0 : 0;
    return make_rsrc(base + t0 * stride, uint32_t(nv) * stride);
}

// Arguments of pass 2.
struct ScanArgs {
    const void* v;
    const float* s0;
    float* s1;
    void* y;
    const char* ws;
    // Chunks cb .. ce - 1 from state s0 (or zero) to s1 (or not written); the record
    // of chunk c of (b, h) is record b h * nrec + c - cb of the workspace.
    int T, H, H_kv, BH, cb, ce, nrec;
    float y_scale;
};

// Enqueues pass 2 for the inputs' and y's element types (fp32 when the flag is
// set, else bf16) and the epilogue option.
hipError_t launch_scan128(const ScanArgs& g, bool in_f32, bool y_f32, bool epi, hipStream_t stream);

}  // namespace tp128
}  // namespace wkv7
