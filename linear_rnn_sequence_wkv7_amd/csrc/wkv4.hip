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
// from scaled terms that never exceed 1.  A full chunk whose k (and u) span
// less than 2^100, with w >= 0, instead scales all its terms by one exponent
// per pass, the largest that pass meets, so that a token costs one exp2 and no
// rescaling; other chunks keep the running exponent.
//
// The recurrence is linear in (a, b) with a scalar decay per channel, so it
// runs chunk-parallel over chunks of 64 tokens in a single pass with a
// look-back: every workgroup takes one (batch, chunk, 256-channel block),
// loads its k and v once into registers and
//   1. reduces its chunk from a zero state and publishes that local state;
//   2. per channel, walks back over the preceding chunks: one that has
//      published its inclusive state (everything up to its end) ends the walk,
//      one that has only published its local state is merged in and the walk
//      goes on; the merged sum, decayed to this chunk's start (plus state_in
//      when the walk passes the first chunk), is the incoming state;
//   3. publishes its inclusive state and reruns its chunk from the incoming
//      state, writing y from the registers.
// k and v are read once, y written once.  No fences: every published value is
// written and read with a device-scope atomic (kept out of the XCD-private L2
// caches) and is ready when it no longer holds the not-ready pattern that a
// first small kernel writes over the whole state area; a release/acquire pair
// per chunk would write back or invalidate an XCD's whole L2 each time.
// Workgroups take their chunk from a ticket counter in the order they start,
// chunk-major, so a thread only waits for chunks whose workgroups are already
// running; each wait is also bounded (past the bound the chunk's outputs are
// NaN, never a hang; each wait that gives up is counted in the workspace, and
// wkv4_wait_status reports the count after the call).  One thread per channel,
// so each wave's loads of a token row are 64 consecutive channels.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

constexpr int CL = 64;        // chunk length (tokens)
constexpr int NT4 = 256;      // threads per workgroup (channels)
constexpr float kNegBig = -1e38f;   // exponent of the zero state
constexpr float kFixedRange = 100.f; // log2 range of one chunk's terms under one exponent
constexpr float kMaxU2 = 60.f;       // largest u log2(e) for 2^u2 as a factor

struct Wkv4Args {
    const float* w;      // [C] decay rate
    const float* u;      // [C] bonus
    const void *k, *v;   // [B, T, C]
    void* y;             // [B, T, C]
    const float* s0;     // [B, 3, C] (A, B, P natural-log units) or null
    float* s1;           // [B, 3, C] or null
    float* ws;           // [B, nch, 3, C] local states, then the inclusive ones likewise
    int* ticket;         // chunk ticket counter; ticket[1]: waits that gave up
    int B, T, C, nch;
    int spin_max;        // polls before a wait gives up
};

struct Scaled {
    float A, Bd, P;   // a = A 2^P, b = Bd 2^P (P in log2 units)
};

// The two rescaling factors 2^(a - max(a, b)) and 2^(b - max(a, b)): one of them is
// 2^0 = 1, so one exp2 of -|a - b| gives both.
__device__ __forceinline__ void rescale2(float a, float b, float& ea, float& eb, float& p) {
    const float d = b - a;
    const float e = __builtin_amdgcn_exp2f(-fabsf(d));
    const bool b_larger = d > 0.f;
    ea = b_larger ? e : 1.f;
    eb = b_larger ? 1.f : e;
    p = b_larger ? b : a;
}

// (A, B, P) + e^x (v, 1), x in log2 units.
__device__ __forceinline__ Scaled add_term(Scaled s, float x, float v) {
    float e1, e2, p;
    rescale2(s.P, x, e1, e2, p);
    return Scaled{fmaf(e1, s.A, e2 * v), fmaf(e1, s.Bd, e2), p};
}

// Merge two states (sums of both).
__device__ __forceinline__ Scaled merge(Scaled s, Scaled t) {
    float e1, e2, p;
    rescale2(s.P, t.P, e1, e2, p);
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

// With no tokens: the final state is the initial state (or the zero state).
__global__ __launch_bounds__(NT4) void wkv4_copy_state_kernel(Wkv4Args g) {
    const int c = blockIdx.x * NT4 + threadIdx.x, bb = blockIdx.y;
    if (c >= g.C) return;
    float* s1 = g.s1 + int64_t(bb) * 3 * g.C + c;
    if (g.s0) {
        const float* s0 = g.s0 + int64_t(bb) * 3 * g.C + c;
        const float A = s0[0], Bd = s0[g.C], P = s0[2 * g.C];
        s1[0] = A;
        s1[g.C] = Bd;
        s1[2 * g.C] = P;
    } else {
        s1[0] = 0.f;
        s1[g.C] = 0.f;
        s1[2 * g.C] = kNegBig * (1.f / kLog2e);
    }
}

constexpr uint32_t kNotReady = 0x7fbadbadu;   // a NaN pattern the arithmetic here does not produce
constexpr int kSpinMax = 1 << 18;              // default bound of one wait (tens of ms)

// Mark every state not ready and reset the ticket counter and the count of
// waits that gave up.
__global__ __launch_bounds__(256) void wkv4_reset_kernel(uint32_t* __restrict__ st, int64_t n, int* ticket) {
    if (blockIdx.x == 0 && threadIdx.x < 2) ticket[threadIdx.x] = 0;
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256)
        st[e] = kNotReady;
}

__device__ __forceinline__ void publish(float* p, int C, Scaled s) {
    __hip_atomic_store(p, s.A, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + C, s.Bd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 2 * C, s.P, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ready_read(const float* p, int C, Scaled& s) {
    s.A = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.Bd = __hip_atomic_load(p + C, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.P = __hip_atomic_load(p + 2 * C, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __float_as_uint(s.A) != kNotReady && __float_as_uint(s.Bd) != kNotReady &&
           __float_as_uint(s.P) != kNotReady;
}

template <typename Tin, typename Ty>
__global__ __launch_bounds__(NT4) void wkv4_onepass_kernel(Wkv4Args g) {
    __shared__ int s_ticket;
    const int tid = threadIdx.x;
    if (tid == 0) s_ticket = atomicAdd(g.ticket, 1);
    __syncthreads();
    const int ncb = (g.C + NT4 - 1) / NT4;
    const int per_j = ncb * g.B;
    const int j = s_ticket / per_j, rem = s_ticket - j * per_j;
    const int bb = rem / ncb, cb = rem - bb * ncb;
    const int c = cb * NT4 + tid;
    if (c >= g.C) return;   // no barrier below
    const int t0 = j * CL, n = min(CL, g.T - t0);
    const Tin* kp = static_cast<const Tin*>(g.k);
    const Tin* vp = static_cast<const Tin*>(g.v);
    Ty* yp = static_cast<Ty*>(g.y);
    const int64_t elem0 = (int64_t(bb) * g.T + t0) * g.C;
    const float w2 = g.w[c] * kLog2e, u2 = g.u[c] * kLog2e;
    float kk[CL], vv[CL];
    load_chunk_row(kp, elem0, n, g.C, c, kk);
    load_chunk_row(vp, elem0, n, g.C, c, vv);

    // 1. Local state, published.
    // Largest and smallest k of a full chunk: the fixed exponent of both passes.
    float mx = 0.f, mn = 0.f;
    if (n == CL) {
        mx = kk[0];
        mn = kk[0];
        #pragma unroll
        for (int i = 1; i < CL; ++i) {
            mx = fmaxf(mx, kk[i]);
            mn = fminf(mn, kk[i]);
        }
        mx *= kLog2e;
        mn *= kLog2e;
    }
    const float dw = __builtin_amdgcn_exp2f(-w2);
    Scaled loc{0.f, 0.f, kNegBig};
    auto step = [&](int i) {
        loc.P -= w2;
        loc = add_term(loc, kk[i] * kLog2e, vv[i]);
    };
    if (n == CL) {
        // Every token's term within 2^-100 of the largest, and no growth (w < 0 would
        // let the sums outgrow the fixed exponent).
        if (mn >= mx - kFixedRange && w2 >= 0.f) {
            float A = 0.f, Bd = 0.f;
            #pragma unroll
            for (int i = 0; i < CL; ++i) {
                const float ex = __builtin_amdgcn_exp2f(fmaf(kk[i], kLog2e, -mx));
                A = fmaf(A, dw, ex * vv[i]);
                Bd = fmaf(Bd, dw, ex);
            }
            loc = Scaled{A, Bd, mx};
        } else {
            #pragma unroll
            for (int i = 0; i < CL; ++i) step(i);
        }
    } else {
        #pragma unroll
        for (int i = 0; i < CL; ++i)
            if (i < n) step(i);
    }
    float* const loc_ws = g.ws + c;
    float* const inc_ws = g.ws + int64_t(g.B) * g.nch * 3 * g.C + c;
    auto row = [&](int k) { return (int64_t(bb) * g.nch + k) * 3 * g.C; };
    publish(loc_ws + row(j), g.C, loc);

    // 2. Look back: the incoming state at the start of chunk j (the end of chunk j - 1).
    Scaled in{0.f, 0.f, kNegBig};
    bool complete = false;   // an inclusive state was reached
    for (int k = j - 1; k >= 0 && !complete; --k) {
        Scaled x;
        for (int it = 0;; ++it) {
            if (ready_read(inc_ws + row(k), g.C, x)) {
                complete = true;
                break;
            }
            if (ready_read(loc_ws + row(k), g.C, x)) break;
            if (it >= g.spin_max) {   // bounded: give up with NaN outputs from here on, never hang
                x = Scaled{__uint_as_float(0x7fc00000u), __uint_as_float(0x7fc00000u), 0.f};
                __hip_atomic_fetch_add(g.ticket + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                complete = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        x.P -= w2 * float((j - 1 - k) * CL);   // full chunks k + 1 .. j - 1 lie in between
        in = merge(x, in);
    }
    if (!complete && g.s0) {
        const float* s0 = g.s0 + int64_t(bb) * 3 * g.C + c;
        Scaled x{s0[0], s0[g.C], s0[2 * g.C] * kLog2e};
        x.P -= w2 * float(t0);
        in = merge(x, in);
    }

    // 3. Inclusive state, published; then the outputs from the incoming state.
    Scaled inc = in;
    inc.P -= w2 * float(n);
    inc = merge(inc, loc);
    publish(inc_ws + row(j), g.C, inc);
    if (j == g.nch - 1 && g.s1) {
        float* s1 = g.s1 + int64_t(bb) * 3 * g.C + c;
        s1[0] = inc.A;
        s1[g.C] = inc.Bd;
        s1[2 * g.C] = inc.P * (1.f / kLog2e);
    }
    const int64_t base = elem0 + c;
    Scaled st = in;
    auto out = [&](int i) {
        const float x = kk[i] * kLog2e;
        // wkv = (a + e^{u+k} v) / (b + e^{u+k}) from the state before this token.
        const Scaled q = add_term(st, u2 + x, vv[i]);
        st1(yp, base + int64_t(i) * g.C, q.A * __builtin_amdgcn_rcpf(q.Bd));
        st.P -= w2;
        st = add_term(st, x, vv[i]);
    };
    if (n == CL) {
        // With all of k in registers the output pass can scale every term by one
        // exponent R, the largest it meets (the incoming state's, and e^k and
        // e^{u+k} over the chunk): then a token costs one exp2 and no rescaling.
        // Lanes where some token's own terms would fall more than 2^-100 below R
        // (so that the sums could lose their leading terms to underflow), or where
        // 2^u2 would be huge, or the state grows (w < 0), keep the running-exponent form.
        const float R = fmaxf(in.P, mx + fmaxf(u2, 0.f));
        if (mn + fminf(u2, 0.f) >= R - kFixedRange && u2 <= kMaxU2 && w2 >= 0.f) {
            const float cu = __builtin_amdgcn_exp2f(u2);
            const float sc = __builtin_amdgcn_exp2f(in.P - R), nR = -R;
            float A = in.A * sc, Bd = in.Bd * sc;
            #pragma unroll
            for (int i = 0; i < CL; ++i) {
                const float ex = __builtin_amdgcn_exp2f(fmaf(kk[i], kLog2e, nR));   // e^k / 2^R
                const float eu = ex * cu;                                           // e^{u+k} / 2^R
                st1(yp, base + int64_t(i) * g.C, fmaf(eu, vv[i], A) * __builtin_amdgcn_rcpf(Bd + eu));
                A = fmaf(A, dw, ex * vv[i]);
                Bd = fmaf(Bd, dw, ex);
            }
        } else {
            #pragma unroll
            for (int i = 0; i < CL; ++i) out(i);
        }
    } else {
        #pragma unroll
        for (int i = 0; i < CL; ++i)
            if (i < n) out(i);
    }
}

template <typename Tin, typename Ty>
hipError_t launch_t(const Wkv4Args& g, hipStream_t stream) {
    const int64_t ncb = (g.C + NT4 - 1) / NT4;
    const int64_t nst = 2 * int64_t(g.B) * g.nch * 3 * g.C;
    const int64_t rb = (nst + 255) / 256;
    hipLaunchKernelGGL(wkv4_reset_kernel, dim3(unsigned(rb < 8192 ? rb : 8192)), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(g.ws), nst, g.ticket);
    hipLaunchKernelGGL((wkv4_onepass_kernel<Tin, Ty>), dim3(unsigned(ncb * g.nch * g.B)), dim3(NT4), 0, stream, g);
    return hipGetLastError();
}

}  // namespace

// Layout: local states [B][nch][3][C], inclusive states likewise, then 256 bytes
// holding the ticket counter and the count of waits that gave up; 0 when there is
// nothing to compute.
int64_t wkv4_workspace_bytes_internal(int B, int T, int C) {
    const int64_t nch = (int64_t(T) + CL - 1) / CL;
    if (int64_t(B) * nch * C == 0) return 0;
    return ((2 * int64_t(B) * nch * 3 * C * 4 + 255) & ~int64_t(255)) + 256;
}

int64_t wkv4_wait_counter_offset(int B, int T, int C) {
    return wkv4_workspace_bytes_internal(B, T, C) - 256 + 4;
}

hipError_t launch_wkv4(const Wkv4Params& p, hipStream_t stream) {
    const int nch = int((p.T + CL - 1) / CL);
    const int64_t states = (2 * int64_t(p.B) * nch * 3 * p.C * 4 + 255) & ~int64_t(255);
    Wkv4Args g{p.w, p.u, p.k, p.v, p.y, p.s0, p.s1, static_cast<float*>(p.ws),
               reinterpret_cast<int*>(static_cast<char*>(p.ws) + states), p.B, p.T, p.C, nch,
               p.spin_limit > 0 ? p.spin_limit : kSpinMax};
    if (p.T == 0) {   // state_out <- state_in (or the zero state)
        if (!p.s1) return hipSuccess;
        hipLaunchKernelGGL(wkv4_copy_state_kernel, dim3(unsigned((p.C + NT4 - 1) / NT4), unsigned(p.B)), dim3(NT4),
                           0, stream, g);
        return hipGetLastError();
    }
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? launch_t<bf16_t, bf16_t>(g, stream) : launch_t<bf16_t, float>(g, stream);
    return p.y_dtype == WKV7_BF16 ? launch_t<float, bf16_t>(g, stream) : launch_t<float, float>(g, stream);
}

}  // namespace wkv7
