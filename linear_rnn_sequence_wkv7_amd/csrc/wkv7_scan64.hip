// Token-by-token scan of the WKV-7 recurrence for head size D = 64 on gfx950.
//
//   sa_t = S_{t-1} a_t;  S_t = S_{t-1} diag(w_t) + sa_t b_t^T + v_t k_t^T;  y_t = S_t r_t
//
// (generalised delta rule: wiki note "RWKV-7 Goose: Expressive Dynamic State
// Evolution", full state update; readout after the update as in the
// youngju.dev RWKV-7 article's time-mix pseudocode.)
//
// Mapping: one 256-thread workgroup per (b, h); wave q owns the 16 value rows
// [16 q, 16 q + 16).  Rows evolve independently given the token's key-side
// vectors, so the four waves never exchange data and the kernel has no LDS and
// no barrier.  Within a wave, lane l = 16 rb + cb holds the 4 x 4 block of S at
// rows 16 q + 4 rb + (0..3) and key columns 4 cb + (0..3): every 16-lane DPP row
// of the wave holds 4 whole rows, so both per-token dot products are sums over
// the 16 lanes of a DPP row (DPP adds, no LDS):
//   - S a (the removal projection, needed by every lane for its 4 rows): an
//     all-reduce, 4 DPP adds per value;
//   - S r (the readout, needed once per row): a reduce-scatter that leaves row
//     4 rb + (cb >> 2) in lane cb, 11 instructions for the 4 values.
// A lane reads 4 consecutive elements of r, w, k, a, b (its columns) and of v
// (its rows) per token with one vector load each, prefetched PF tokens ahead
// into a register ring; the removal projection of token t + 1 is formed right
// after the update of token t, so its reduction overlaps that token's readout.
//
// Kernel vectors from k (KK): the a slot carries alpha and b is not read.
// With kk = k / n, n = max(|k|, 1e-12), (S a) b^T = -(S k)(k alpha)^T / n^2:
// the projection is formed with k, |k|^2 is summed over the DPP row alongside
// it, and the update adds (-(S k) / n^2) (k alpha)_j and v (k (1 - decay +
// alpha))_j.  Masked tokens (mask byte 0) run as the identity token: r, k, a,
// b = 0 and decay 1 leave the state bit for bit and give y = 0.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

constexpr int D = 64;
constexpr int NTHR = 256;   // four waves
// Tokens of loads in flight ahead of the one in use (the ring holds PF tokens).
template <typename Tin> constexpr int kPF = sizeof(Tin) == 2 ? 8 : 4;
constexpr int kPFMax = 8;
constexpr int kDppRowRor8 = 0x128;   // row_ror:8 (lane cb reads lane cb ^ 8 of its row)

struct Args {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    const uint8_t* mask;
    void* y;
    float* s1;
    int T, H, H_kv;
    float y_scale;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer descriptor over [base, base + bytes) (wave-uniform): loads at offsets past
// the end return zeros without touching memory.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, int(n), 0x00020000);
}

// 4 consecutive elements, raw: buffer descriptor, the lane's byte offset and the
// token's (wave-uniform) byte offset.
template <typename Tin> struct Raw4;
template <> struct Raw4<bf16_t> {
    uint2 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t d = e < 2 ? x.x : x.y;
        return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
    }
};
template <> struct Raw4<float> {
    uint4 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        return __uint_as_float(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w);
    }
};

// One token's loads for one lane (raw) and the values the update uses (decoded).
template <typename Tin> struct TokRaw {
    Raw4<Tin> r, w, k, a, b, v;
    uint32_t m;
};
struct Tok {
    float r[4], dec[4], k[4], a[4], b[4], v[4];
};

template <typename Ty> __device__ __forceinline__ void store_out(rsrc_t r, uint32_t voff, uint32_t soff, float x);
template <> __device__ __forceinline__ void store_out<float>(rsrc_t r, uint32_t voff, uint32_t soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}
template <> __device__ __forceinline__ void store_out<bf16_t>(rsrc_t r, uint32_t voff, uint32_t soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, voff, soff, 0);
}

__device__ __forceinline__ float ror8(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowRor8, 0xF, 0xF, false));
}

// Reduce-scatter of p[0..3] (rows 0..3 of the lane's block) over the 16 lanes
// of a DPP row: lane cb ends with the row-(cb >> 2) sum.
__device__ __forceinline__ float reduce_scatter4(const float (&p)[4], int cb) {
    const bool lo = cb < 8;                 // keeps rows 0, 1 (partner cb ^ 8 keeps 2, 3)
    const float u0 = (lo ? p[0] : p[2]) + ror8(lo ? p[2] : p[0]);
    const float u1 = (lo ? p[1] : p[3]) + ror8(lo ? p[3] : p[1]);
    const bool lo2 = (cb & 7) < 4;          // partner 7 - (cb & 7) in the same half-row
    float z = (lo2 ? u0 : u1) + dpp<kDppRowHalfMirror>(lo2 ? u1 : u0);
    z += dpp<kDppQuadXor1>(z);
    z += dpp<kDppQuadXor2>(z);
    return z;
}

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
__global__ __launch_bounds__(NTHR)
void scan64_kernel(Args g) {
    const int T = g.T, H = g.H, H_kv = g.H_kv;
    const int q = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int l = threadIdx.x & 63, rb = l >> 4, cb = l & 15;
    const int bh = blockIdx.x;
    const int bb = bh / H, h = bh - bb * H, hk = h / (H / H_kv);
    const int row0 = 16 * q + 4 * rb, col0 = 4 * cb;

    // Each input is read through a descriptor over this (b, h)'s T tokens (token
    // t at byte t * step, the lane's elements at its own offset); the host makes
    // sure that the offsets of T + PF + 1 tokens fit in 32 bits.
    constexpr uint32_t SI = sizeof(Tin), SY = sizeof(Ty);
    const int64_t base_q = (int64_t(bb) * T * H + h) * D, base_kv = (int64_t(bb) * T * H_kv + hk) * D;
    const uint32_t step_q = uint32_t(H) * D * SI, step_kv = uint32_t(H_kv) * D * SI;
    const uint32_t nq = uint32_t(T) * step_q, nkv = uint32_t(T) * step_kv;
    const rsrc_t Rr = make_rsrc(static_cast<const char*>(g.r) + base_q * SI, nq);
    const rsrc_t Rw = make_rsrc(static_cast<const char*>(g.w) + base_q * SI, nq);
    const rsrc_t Ra = make_rsrc(static_cast<const char*>(g.a) + base_q * SI, nq);
    const rsrc_t Rb = make_rsrc(KK ? g.a : static_cast<const char*>(g.b) + base_q * SI, KK ? 0u : nq);
    const rsrc_t Rk = make_rsrc(static_cast<const char*>(g.k) + base_kv * SI, nkv);
    const rsrc_t Rv = make_rsrc(static_cast<const char*>(g.v) + base_kv * SI, nkv);
    const rsrc_t Rm = make_rsrc(MASK ? g.mask + int64_t(bb) * T : g.r, MASK ? uint32_t(T) : 0u);
    const uint32_t ocol = uint32_t(col0) * SI, orow = uint32_t(row0) * SI;

    float S[4][4];
    const int64_t sbase = int64_t(bh) * D * D;
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (g.s0) {
            const float4 x = *reinterpret_cast<const float4*>(g.s0 + sbase + int64_t(row0 + i) * D + col0);
            S[i][0] = x.x; S[i][1] = x.y; S[i][2] = x.z; S[i][3] = x.w;
        } else {
            S[i][0] = S[i][1] = S[i][2] = S[i][3] = 0.f;
        }
    }
    float rk[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI) {
        const float4 x = *reinterpret_cast<const float4*>(g.r_k + h * D + col0);
        rk[0] = x.x; rk[1] = x.y; rk[2] = x.z; rk[3] = x.w;
    }

    // Loads of token t (zeros past the last token: never used).
    auto load = [&](int t, TokRaw<Tin>& x) {
        const uint32_t oq = uint32_t(t) * step_q, okv = uint32_t(t) * step_kv;
        x.r.load(Rr, ocol, oq);
        x.w.load(Rw, ocol, oq);
        x.a.load(Ra, ocol, oq);
        if constexpr (!KK) x.b.load(Rb, ocol, oq);
        x.k.load(Rk, ocol, okv);
        x.v.load(Rv, orow, okv);
        if constexpr (MASK) x.m = __builtin_amdgcn_raw_buffer_load_b8(Rm, 0, uint32_t(t), 0);
    };
    // Decoded token: decay from w, the identity token if masked, and with KK the
    // operands formed from k and alpha (b_j -> k_j alpha_j, k_j -> k_j (1 - w_j + alpha_j);
    // the projection is formed with k and scaled by -1/n^2 after the reduction).
    auto decode = [&](const TokRaw<Tin>& x, Tok& o) {
        const bool keep = !MASK || x.m != 0;
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float dec = LOGW ? decay_from_logneglog(x.w.get(e)) : x.w.get(e);
            const float kk = x.k.get(e), al = x.a.get(e);
            o.r[e] = keep ? x.r.get(e) : 0.f;
            o.dec[e] = keep ? dec : 1.f;
            o.k[e] = keep ? (KK ? kk * (1.f - dec + al) : kk) : 0.f;
            o.a[e] = keep ? (KK ? kk : al) : 0.f;
            o.b[e] = keep ? (KK ? kk * al : x.b.get(e)) : 0.f;
            o.v[e] = keep ? x.v.get(e) : 0.f;
        }
    };
    // Removal projection of token `o` for the lane's 4 rows, summed over the DPP row
    // (every lane gets the sums).
    auto projection = [&](const Tok& o, float (&sa)[4]) {
        float ss = 0.f;
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s = S[i][0] * o.a[0];
            s = fmaf(S[i][1], o.a[1], s);
            s = fmaf(S[i][2], o.a[2], s);
            sa[i] = fmaf(S[i][3], o.a[3], s);
        }
        if constexpr (KK) {
            ss = o.a[0] * o.a[0];
            ss = fmaf(o.a[1], o.a[1], ss);
            ss = fmaf(o.a[2], o.a[2], ss);
            ss = fmaf(o.a[3], o.a[3], ss);
        }
        #pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = sum16(sa[i]);
        if constexpr (KK) {
            const float inv = inv_key_norm(sum16(ss));
            const float c2 = -inv * inv;
            #pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] *= c2;
        }
    };

    const uint32_t step_y = uint32_t(H) * D * SY;
    const rsrc_t Ry = make_rsrc(static_cast<char*>(g.y) + base_q * SY, uint32_t(T) * step_y);
    const uint32_t oy = uint32_t(row0 + (cb >> 2)) * SY;
    const bool ylane = (cb & 3) == 0;

    // Ring of raw loads: slot (t mod PF) holds token t until it is decoded.  Each
    // token's loads are issued together (not interleaved with other tokens'), so
    // that the wait for the oldest token leaves the younger ones in flight.
    constexpr int PF = kPF<Tin>;
    TokRaw<Tin> ring[PF];
    #pragma unroll
    for (int s = 0; s < PF; ++s) {
        load(s, ring[s]);
        __builtin_amdgcn_sched_barrier(0);
    }
    Tok ta, tb;
    decode(ring[0], ta);
    load(PF, ring[0]);
    float sa[4];
    projection(ta, sa);

    // One token: S_t from S_{t-1} (token t decoded in cur), y_t, and the projection
    // of token t + 1 (decoded into nxt from its ring slot, which then takes the
    // loads of token t + 1 + PF).
    auto step = [&](const int t, TokRaw<Tin>& slot, const Tok& cur, Tok& nxt) {
        decode(slot, nxt);                 // token t + 1 (unused at t = T - 1)
        // The decoded values are materialised here, so the slot's registers are free
        // for its next loads: the loop then needs no register copies of loads in
        // flight (a copy waits for its load, at the loop's back edge).
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            settle(nxt.r[e]); settle(nxt.dec[e]); settle(nxt.k[e]);
            settle(nxt.a[e]); settle(nxt.b[e]); settle(nxt.v[e]);
        }
        load(t + 1 + PF, slot);
        float yp4[4];
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            float y = 0.f;
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                float s = S[i][e] * cur.dec[e];
                s = fmaf(sa[i], cur.b[e], s);
                s = fmaf(cur.v[i], cur.k[e], s);
                S[i][e] = s;
                y = fmaf(s, cur.r[e], y);
            }
            yp4[i] = y;
        }
        projection(nxt, sa);
        float yv = reduce_scatter4(yp4, cb) * g.y_scale;
        if constexpr (EPI) {
            float bon = 0.f;
            #pragma unroll
            for (int e = 0; e < 4; ++e) bon = fmaf(cur.r[e] * cur.k[e], rk[e], bon);
            bon = sum16(bon);
            // v of the lane's output row 4 rb + (cb >> 2), by two bit selects.
            const bool b4 = cb & 4, b8 = cb & 8;
            const float v01 = b4 ? cur.v[1] : cur.v[0], v23 = b4 ? cur.v[3] : cur.v[2];
            yv = fmaf(bon, b8 ? v23 : v01, yv);
        }
        if (ylane) store_out<Ty>(Ry, oy, uint32_t(t) * step_y, yv);
    };
    // Unrolled by PF (ring slots known at compile time), the decoded tokens
    // alternating between ta and tb (no copies).
    static_assert(PF % 2 == 0, "even ring");
    int t = 0;
    for (; t + PF <= T; t += PF) {
        #pragma unroll
        for (int s = 0; s < PF; s += 2) {
            step(t + s, ring[(s + 1) % PF], ta, tb);
            step(t + s + 1, ring[(s + 2) % PF], tb, ta);
        }
    }
    #pragma unroll
    for (int s = 0; s < PF - 1; ++s) {
        if (t + s >= T) break;
        if (s & 1) step(t + s, ring[(s + 1) % PF], tb, ta);
        else step(t + s, ring[(s + 1) % PF], ta, tb);
    }

    if (g.s1) {
        #pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<float4*>(g.s1 + sbase + int64_t(row0 + i) * D + col0) =
                make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
    }
}

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
hipError_t launch_t(const Params& p, hipStream_t stream) {
    Args g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.mask, p.y, p.s1, p.T, p.H, p.H_kv, p.y_scale};
    hipLaunchKernelGGL((scan64_kernel<Tin, Ty, LOGW, EPI, KK, MASK>), dim3(unsigned(p.B) * unsigned(p.H)), dim3(NTHR), 0,
                       stream, g);
    return hipGetLastError();
}

template <typename Tin, typename Ty, bool KK, bool MASK>
hipError_t dispatch_epi(const Params& p, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_t<Tin, Ty, true, true, KK, MASK>(p, s) : launch_t<Tin, Ty, true, false, KK, MASK>(p, s);
    return epi ? launch_t<Tin, Ty, false, true, KK, MASK>(p, s) : launch_t<Tin, Ty, false, false, KK, MASK>(p, s);
}

template <typename Tin, typename Ty, bool KK>
hipError_t dispatch_mask(const Params& p, hipStream_t s) {
    return p.mask ? dispatch_epi<Tin, Ty, KK, true>(p, s) : dispatch_epi<Tin, Ty, KK, false>(p, s);
}

template <typename Tin, typename Ty>
hipError_t dispatch_modes(const Params& p, hipStream_t s) {
    return p.ab_mode == WKV7_AB_FROM_K ? dispatch_mask<Tin, Ty, true>(p, s) : dispatch_mask<Tin, Ty, false>(p, s);
}

}  // namespace

bool scan64_fits(const Params& p) {
    // Byte offsets of T + PF + 1 tokens (PF <= kPFMax) of the widest per-token row (r, w, a, b or y
    // at 4 bytes per element) fit the 32-bit buffer offsets.
    return p.D == D && p.T >= 1 && (int64_t(p.T) + kPFMax + 1) * p.H * D * 4 < (int64_t(1) << 32);
}

hipError_t launch_scan64(const Params& p, hipStream_t stream) {
    if (!scan64_fits(p)) return hipErrorInvalidValue;
    // The grid's work-items must fit in 32 bits.
    if (int64_t(p.B) * p.H * NTHR > int64_t(0xffffffffu)) return hipErrorInvalidConfiguration;
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<bf16_t, bf16_t>(p, stream) : dispatch_modes<bf16_t, float>(p, stream);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<float, bf16_t>(p, stream) : dispatch_modes<float, float>(p, stream);
}

}  // namespace wkv7
