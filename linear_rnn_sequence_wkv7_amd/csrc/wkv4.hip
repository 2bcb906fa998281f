// RWKV-4 WKV operator on gfx950 (SSM note "RWKV: state-space based sequence
// model", time-mixing section):
//
//   wkv_t = (a_{t-1} + e^{u + k_t} v_t) / (b_{t-1} + e^{u + k_t}),
//   a_t = e^{-w} a_{t-1} + e^{k_t} v_t,  b_t = e^{-w} b_{t-1} + e^{k_t}
//
// per batch b and channel c.  e^k overflows fp32 for k > 88, so a and b are
// kept with a shared exponent: a = A 2^P, b = B 2^P (P in log2 units), and
// every addition rescales both terms to the larger exponent (the usual
// log-sum-exp scaling): adding e^x v to (A, B, P) gives P' = max(P, x),
// A' = A 2^(P - P') + v 2^(x - P'), B' likewise.  The ratio is then computed
// from scaled terms that never exceed 1.
//
// The recurrence is linear in (a, b) with a scalar decay per channel, so it
// runs chunk-parallel in three launches over chunks of 64 tokens:
//   1. every (b, chunk, c) reduces its chunk from a zero state (local state);
//   2. one thread per (b, c) scans the chunks: incoming state of chunk j =
//      the previous incoming state decayed by the chunk length, merged with the
//      previous chunk's local state; the last merge is the final state;
//   3. every (b, chunk, c) reruns its chunk from its incoming state and writes y.
// Inputs are read twice (steps 1 and 3), y once; one thread per channel, so
// each wave's loads of a token row are 64 consecutive channels.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

constexpr int CL = 64;        // chunk length (tokens)
constexpr int NT4 = 256;      // threads per workgroup (channels)
constexpr float kNegBig = -1e38f;   // exponent of the zero state

struct Wkv4Args {
    const float* w;      // [C] decay rate
    const float* u;      // [C] bonus
    const void *k, *v;   // [B, T, C]
    void* y;             // [B, T, C]
    const float* s0;     // [B, 3, C] (A, B, P natural-log units) or null
    float* s1;           // [B, 3, C] or null
    float* ws;           // [B, nch, 3, C]
    int B, T, C, nch;
};

struct Scaled {
    float A, Bd, P;   // a = A 2^P, b = Bd 2^P (P in log2 units)
};

// (A, B, P) + e^x (v, 1), x in log2 units.
__device__ __forceinline__ Scaled add_term(Scaled s, float x, float v) {
    const float p = fmaxf(s.P, x);
    const float e1 = __builtin_amdgcn_exp2f(s.P - p), e2 = __builtin_amdgcn_exp2f(x - p);
    return Scaled{fmaf(e1, s.A, e2 * v), fmaf(e1, s.Bd, e2), p};
}

// Merge two states (sums of both).
__device__ __forceinline__ Scaled merge(Scaled s, Scaled t) {
    const float p = fmaxf(s.P, t.P);
    const float e1 = __builtin_amdgcn_exp2f(s.P - p), e2 = __builtin_amdgcn_exp2f(t.P - p);
    return Scaled{fmaf(e1, s.A, e2 * t.A), fmaf(e1, s.Bd, e2 * t.Bd), p};
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, range-checked

// Buffer descriptor over tokens [t0, t0 + n) of sequence b: loads past it read 0.
__device__ __forceinline__ rsrc_t chunk_rsrc(const void* base, int64_t elem0, int n, int C, int esize) {
    const char* p = static_cast<const char*>(base) + elem0 * esize;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, n * C * esize, kRsrcWord3);
}
__device__ __forceinline__ float buf_ld(rsrc_t r, uint32_t off, const bf16_t*) {
    return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
}
__device__ __forceinline__ float buf_ld(rsrc_t r, uint32_t off, const float*) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// The chunk's values of channel c: unconditional loads (all issued before any use).
template <typename Tin>
__device__ __forceinline__ void load_chunk_row(const Tin* p, int64_t elem0, int n, int C, int c, float* out) {
    const rsrc_t r = chunk_rsrc(p, elem0, n, C, int(sizeof(Tin)));
    #pragma unroll
    for (int i = 0; i < CL; ++i) out[i] = buf_ld(r, uint32_t((i * C + c) * int(sizeof(Tin))), p);
}

// Step 1: local state of chunk j from zero.
template <typename Tin>
__global__ __launch_bounds__(NT4) void wkv4_local_kernel(Wkv4Args g) {
    const int c = blockIdx.x * NT4 + threadIdx.x;
    const int j = blockIdx.y, bb = blockIdx.z;
    if (c >= g.C) return;
    const int t0 = j * CL, n = min(CL, g.T - t0);
    const Tin* kp = static_cast<const Tin*>(g.k);
    const Tin* vp = static_cast<const Tin*>(g.v);
    const int64_t elem0 = (int64_t(bb) * g.T + t0) * g.C;
    const float w2 = g.w[c] * kLog2e;
    float kk[CL], vv[CL];
    load_chunk_row(kp, elem0, n, g.C, c, kk);
    load_chunk_row(vp, elem0, n, g.C, c, vv);
    Scaled s{0.f, 0.f, kNegBig};
    auto step = [&](int i) {
        s.P -= w2;
        s = add_term(s, kk[i] * kLog2e, vv[i]);
    };
    if (n == CL) {
        #pragma unroll
        for (int i = 0; i < CL; ++i) step(i);
    } else {
        #pragma unroll
        for (int i = 0; i < CL; ++i)
            if (i < n) step(i);
    }
    float* o = g.ws + ((int64_t(bb) * g.nch + j) * 3) * g.C + c;
    o[0] = s.A;
    o[g.C] = s.Bd;
    o[2 * g.C] = s.P;
}

// Step 2: incoming state of every chunk (in place of its local state); the final state.
__global__ __launch_bounds__(NT4) void wkv4_scan_kernel(Wkv4Args g) {
    const int c = blockIdx.x * NT4 + threadIdx.x;
    const int bb = blockIdx.y;
    if (c >= g.C) return;
    const float w2 = g.w[c] * kLog2e;
    Scaled cur{0.f, 0.f, kNegBig};
    if (g.s0) {
        const float* s = g.s0 + int64_t(bb) * 3 * g.C + c;
        cur = Scaled{s[0], s[g.C], s[2 * g.C] * kLog2e};
    }
    // Chunks in groups of 16: the group's local states are loaded before the
    // first merge, so the loads overlap instead of forming a chain.
    constexpr int G = 16;
    for (int j0 = 0; j0 < g.nch; j0 += G) {
        Scaled loc[G];
        #pragma unroll
        for (int q = 0; q < G; ++q) {
            const int j = min(j0 + q, g.nch - 1);
            const float* o = g.ws + ((int64_t(bb) * g.nch + j) * 3) * g.C + c;
            loc[q] = Scaled{o[0], o[g.C], o[2 * g.C]};
        }
        #pragma unroll
        for (int q = 0; q < G; ++q) {
            const int j = j0 + q;
            if (j < g.nch) {
                float* o = g.ws + ((int64_t(bb) * g.nch + j) * 3) * g.C + c;
                o[0] = cur.A;
                o[g.C] = cur.Bd;
                o[2 * g.C] = cur.P;
                const int n = min(CL, g.T - j * CL);
                cur.P -= w2 * float(n);
                cur = merge(cur, loc[q]);
            }
        }
    }
    if (g.s1) {
        float* s = g.s1 + int64_t(bb) * 3 * g.C + c;
        s[0] = cur.A;
        s[g.C] = cur.Bd;
        s[2 * g.C] = cur.P * (1.f / kLog2e);
    }
}

// Step 3: outputs of chunk j from its incoming state.
template <typename Tin, typename Ty>
__global__ __launch_bounds__(NT4) void wkv4_out_kernel(Wkv4Args g) {
    const int c = blockIdx.x * NT4 + threadIdx.x;
    const int j = blockIdx.y, bb = blockIdx.z;
    if (c >= g.C) return;
    const int t0 = j * CL, n = min(CL, g.T - t0);
    const Tin* kp = static_cast<const Tin*>(g.k);
    const Tin* vp = static_cast<const Tin*>(g.v);
    Ty* yp = static_cast<Ty*>(g.y);
    const int64_t elem0 = (int64_t(bb) * g.T + t0) * g.C;
    const int64_t base = elem0 + c;
    const float w2 = g.w[c] * kLog2e, u2 = g.u[c] * kLog2e;
    float kk[CL], vv[CL];
    load_chunk_row(kp, elem0, n, g.C, c, kk);
    load_chunk_row(vp, elem0, n, g.C, c, vv);
    const float* o = g.ws + ((int64_t(bb) * g.nch + j) * 3) * g.C + c;
    Scaled s{o[0], o[g.C], o[2 * g.C]};
    auto step = [&](int i) {
        const float x = kk[i] * kLog2e;
        // wkv = (a + e^{u+k} v) / (b + e^{u+k}) from the state before this token.
        const Scaled q = add_term(s, u2 + x, vv[i]);
        st1(yp, base + int64_t(i) * g.C, q.A * __builtin_amdgcn_rcpf(q.Bd));
        s.P -= w2;
        s = add_term(s, x, vv[i]);
    };
    if (n == CL) {
        #pragma unroll
        for (int i = 0; i < CL; ++i) step(i);
    } else {
        #pragma unroll
        for (int i = 0; i < CL; ++i)
            if (i < n) step(i);
    }
}

template <typename Tin, typename Ty>
hipError_t launch_t(const Wkv4Args& g, hipStream_t stream) {
    const dim3 blk(NT4);
    const unsigned cb = unsigned((g.C + NT4 - 1) / NT4);
    hipLaunchKernelGGL(wkv4_local_kernel<Tin>, dim3(cb, unsigned(g.nch), unsigned(g.B)), blk, 0, stream, g);
    hipLaunchKernelGGL(wkv4_scan_kernel, dim3(cb, unsigned(g.B)), blk, 0, stream, g);
    hipLaunchKernelGGL((wkv4_out_kernel<Tin, Ty>), dim3(cb, unsigned(g.nch), unsigned(g.B)), blk, 0, stream, g);
    return hipGetLastError();
}

}  // namespace

int64_t wkv4_workspace_bytes_internal(int B, int T, int C) {
    const int64_t nch = (int64_t(T) + CL - 1) / CL;
    return int64_t(B) * nch * 3 * C * 4;
}

hipError_t launch_wkv4(const Wkv4Params& p, hipStream_t stream) {
    Wkv4Args g{p.w, p.u, p.k, p.v, p.y, p.s0, p.s1, static_cast<float*>(p.ws), p.B, p.T, p.C,
               int((p.T + CL - 1) / CL)};
    if (p.T == 0) {   // state_out <- state_in (or the zero state)
        if (!p.s1) return hipSuccess;
        g.nch = 0;
        hipLaunchKernelGGL(wkv4_scan_kernel, dim3(unsigned((p.C + NT4 - 1) / NT4), unsigned(p.B)), dim3(NT4), 0,
                           stream, g);
        return hipGetLastError();
    }
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? launch_t<bf16_t, bf16_t>(g, stream) : launch_t<bf16_t, float>(g, stream);
    return p.y_dtype == WKV7_BF16 ? launch_t<float, bf16_t>(g, stream) : launch_t<float, float>(g, stream);
}

}  // namespace wkv7
