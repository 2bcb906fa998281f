// Token-by-token scan of the WKV-7 recurrence for head sizes D = 64 and 128 on gfx950.
//
//   sa_t = S_{t-1} a_t;  S_t = S_{t-1} diag(w_t) + sa_t b_t^T + v_t k_t^T;  y_t = S_t r_t
//
// (generalised delta rule: wiki note "RWKV-7 Goose: Expressive Dynamic State
// Evolution", full state update; readout after the update as in the
// youngju.dev RWKV-7 article's time-mix pseudocode.)
//
// Mapping: a lane holds an R x C block of S (C = D / 16 key columns; R = 4
// rows at D = 64, 2 at D = 128), so every 16-lane DPP row of a wave holds R
// whole rows and a wave 4 R rows; D / (4 R) waves (one wave per SIMD: four per
// workgroup, D / (16 R) workgroups per (b, h), 1 at D = 64 and 4 at D = 128)
// cover a head.  Rows evolve independently given the token's key-side vectors,
// so the waves never exchange data and the kernel has no LDS and no barrier.
// Lane l = 16 rb + cb of wave u of the head holds rows 4 R u + R rb + (0..R-1)
// and key columns C cb + (0..C-1); both per-token dot products are sums over
// the 16 lanes of a DPP row (DPP adds, no LDS):
//   - S a (the removal projection, needed by every lane for its R rows): an
//     all-reduce, 4 DPP adds per value;
//   - S r (the readout, needed once per row): a reduce-scatter that leaves row
//     R rb + cb / (16 / R) in lane cb (11 instructions for 4 rows, 6 for 2).
// A lane reads C consecutive elements of r, w, k, a, b (its columns) and R of v
// (its rows) per token with one or two vector loads each, prefetched PF tokens ahead
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

// Tokens of loads in flight ahead of the one in use (the ring holds PF tokens,
// sized to the registers of the raw loads).
template <int D, typename Tin> constexpr int kPF = (D == 64 ? 8 : 4) / int(sizeof(Tin) / 2);
constexpr int kPFMax = 8;
constexpr int kDppRowRor8 = 0x128;   // row_ror:8 (lane cb reads lane cb ^ 8 of its row)

struct Args {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    const uint8_t* mask;
    void* y;
    float* s1;
    int T, H, H_kv, BH;
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

// N consecutive elements, raw: buffer descriptor, the lane's byte offset and the
// token's (wave-uniform) byte offset.
template <typename Tin, int N> struct RawN;
template <> struct RawN<bf16_t, 2> {
    uint32_t x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    __device__ __forceinline__ float get(int e) const {
        return e ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    }
};
template <> struct RawN<float, 2> {
    uint2 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const { return __uint_as_float(e ? x.y : x.x); }
};
template <> struct RawN<bf16_t, 4> {
    uint2 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t d = e < 2 ? x.x : x.y;
        return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
    }
};
template <> struct RawN<bf16_t, 8> {
    uint4 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t d = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
        return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
    }
};
template <> struct RawN<float, 4> {
    uint4 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        return __uint_as_float(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w);
    }
};
template <> struct RawN<float, 8> {
    uint4 x[2];
    __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        x[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
        x[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        const uint4& u = x[e >> 2];
        return __uint_as_float((e & 3) == 0 ? u.x : (e & 3) == 1 ? u.y : (e & 3) == 2 ? u.z : u.w);
    }
};

// One token's loads for one lane (raw) and the values the update uses (decoded).
template <typename Tin, int C, int R> struct TokRaw {
    RawN<Tin, C> r, w, k, a, b;
    RawN<Tin, R> v;
    uint32_t m;
};
template <int C, int R> struct Tok {
    float r[C], dec[C], k[C], a[C], b[C], v[R];
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

// Reduce-scatter of p[0..R-1] (rows 0..R-1 of the lane's block) over the 16
// lanes of a DPP row: lane cb ends with the sum of row cb / (16 / R).
__device__ __forceinline__ float reduce_scatter(const float (&p)[2], int cb) {
    const bool lo = cb < 8;                 // keeps row 0 (partner cb ^ 8 keeps row 1)
    float z = (lo ? p[0] : p[1]) + ror8(lo ? p[1] : p[0]);
    z += dpp<kDppRowHalfMirror>(z);
    z += dpp<kDppQuadXor1>(z);
    z += dpp<kDppQuadXor2>(z);
    return z;
}
__device__ __forceinline__ float reduce_scatter(const float (&p)[4], int cb) {
    const bool lo = cb < 8;                 // keeps rows 0, 1 (partner cb ^ 8 keeps 2, 3)
    const float u0 = (lo ? p[0] : p[2]) + ror8(lo ? p[2] : p[0]);
    const float u1 = (lo ? p[1] : p[3]) + ror8(lo ? p[3] : p[1]);
    const bool lo2 = (cb & 7) < 4;          // partner 7 - (cb & 7) in the same half-row
    float z = (lo2 ? u0 : u1) + dpp<kDppRowHalfMirror>(lo2 ? u1 : u0);
    z += dpp<kDppQuadXor1>(z);
    z += dpp<kDppQuadXor2>(z);
    return z;
}

template <int D, typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
__global__ __launch_bounds__(256)
void scan_dpp_kernel(Args g) {
    constexpr int C = D / 16;               // key columns per lane
    constexpr int R = D == 64 ? 4 : 2;      // value rows per lane
    constexpr int NSL = D / (16 * R);       // workgroups per (b, h)
    const int T = g.T, H = g.H, H_kv = g.H_kv;
    const int q = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int l = threadIdx.x & 63, rb = l >> 4, cb = l & 15;
    // Workgroup -> (b, h, slice); with several slices per (b, h) their ids are 8
    // apart (one XCD under round-robin dispatch, so their input reads meet in one L2).
    const int gid = blockIdx.x;
    const int bh = NSL == 1 ? gid : (gid & 7) + 8 * (gid / (8 * NSL));
    const int slice = NSL == 1 ? 0 : (gid >> 3) % NSL;
    if (bh >= g.BH) return;
    const int bb = bh / H, h = bh - bb * H, hk = h / (H / H_kv);
    const int row0 = 4 * R * (4 * slice + q) + R * rb, col0 = C * cb;

    // Each input is read through a descriptor that starts at token t_base of this
    // (b, h) (token t at byte (t - t_base) * step, the lane's elements at its own
    // offset) and ends after token T - 1; t_base moves forward by PF tokens per loop
    // iteration, so the 32-bit offsets cover at most 2 PF + 1 tokens whatever T
    // (the host checks that they fit).
    constexpr uint32_t SI = sizeof(Tin), SY = sizeof(Ty);
    const int64_t base_q = (int64_t(bb) * T * H + h) * D, base_kv = (int64_t(bb) * T * H_kv + hk) * D;
    const uint32_t step_q = uint32_t(H) * D * SI, step_kv = uint32_t(H_kv) * D * SI;
    const uint32_t step_y = uint32_t(H) * D * SY;
    const char* r0 = static_cast<const char*>(g.r) + base_q * SI;
    const char* w0 = static_cast<const char*>(g.w) + base_q * SI;
    const char* a0 = static_cast<const char*>(g.a) + base_q * SI;
    const char* b0 = KK ? a0 : static_cast<const char*>(g.b) + base_q * SI;
    const char* k0 = static_cast<const char*>(g.k) + base_kv * SI;
    const char* v0 = static_cast<const char*>(g.v) + base_kv * SI;
    const char* m0 = MASK ? reinterpret_cast<const char*>(g.mask) + int64_t(bb) * T : r0;
    char* y0 = static_cast<char*>(g.y) + base_q * SY;
    rsrc_t Rr, Rw, Ra, Rb, Rk, Rv, Rm, Ry;
    int t_base = 0;
    auto rebase = [&](int t0) {
        t_base = t0;
        const int64_t left = T - t0;
        auto bytes = [&](uint32_t step) { return uint32_t(min(left * step, int64_t(0xffffffffu))); };
        Rr = make_rsrc(r0 + int64_t(t0) * step_q, bytes(step_q));
        Rw = make_rsrc(w0 + int64_t(t0) * step_q, bytes(step_q));
        Ra = make_rsrc(a0 + int64_t(t0) * step_q, bytes(step_q));
        Rb = make_rsrc(b0 + int64_t(t0) * step_q, KK ? 0u : bytes(step_q));
        Rk = make_rsrc(k0 + int64_t(t0) * step_kv, bytes(step_kv));
        Rv = make_rsrc(v0 + int64_t(t0) * step_kv, bytes(step_kv));
        Rm = make_rsrc(m0 + t0, MASK ? bytes(1) : 0u);
        Ry = make_rsrc(y0 + int64_t(t0) * step_y, bytes(step_y));
    };
    rebase(0);
    const uint32_t ocol = uint32_t(col0) * SI, orow = uint32_t(row0) * SI;

    float S[R][C];
    const int64_t sbase = int64_t(bh) * D * D;
    #pragma unroll
    for (int i = 0; i < R; ++i)
        #pragma unroll
        for (int e = 0; e < C; e += 4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (g.s0) x = *reinterpret_cast<const float4*>(g.s0 + sbase + int64_t(row0 + i) * D + col0 + e);
            S[i][e] = x.x; S[i][e + 1] = x.y; S[i][e + 2] = x.z; S[i][e + 3] = x.w;
        }
    float rk[C];
    #pragma unroll
    for (int e = 0; e < C; e += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (EPI) x = *reinterpret_cast<const float4*>(g.r_k + h * D + col0 + e);
        rk[e] = x.x; rk[e + 1] = x.y; rk[e + 2] = x.z; rk[e + 3] = x.w;
    }

    // Loads of token t (zeros past the last token: never used).
    auto load = [&](int t, TokRaw<Tin, C, R>& x) {
        const uint32_t oq = uint32_t(t - t_base) * step_q, okv = uint32_t(t - t_base) * step_kv;
        x.r.load(Rr, ocol, oq);
        x.w.load(Rw, ocol, oq);
        x.a.load(Ra, ocol, oq);
        if constexpr (!KK) x.b.load(Rb, ocol, oq);
        x.k.load(Rk, ocol, okv);
        x.v.load(Rv, orow, okv);
        if constexpr (MASK) x.m = __builtin_amdgcn_raw_buffer_load_b8(Rm, 0, uint32_t(t - t_base), 0);
    };
    // Decoded token: decay from w, the identity token if masked, and with KK the
    // operands formed from k and alpha (b_j -> k_j alpha_j, k_j -> k_j (1 - w_j + alpha_j);
    // the projection is formed with k and scaled by -1/n^2 after the reduction).
    auto decode = [&](const TokRaw<Tin, C, R>& x, Tok<C, R>& o) {
        const bool keep = !MASK || x.m != 0;
        #pragma unroll
        for (int e = 0; e < C; ++e) {
            const float dec = LOGW ? decay_from_logneglog(x.w.get(e)) : x.w.get(e);
            const float kk = x.k.get(e), al = x.a.get(e);
            o.r[e] = keep ? x.r.get(e) : 0.f;
            o.dec[e] = keep ? dec : 1.f;
            o.k[e] = keep ? (KK ? kk * (1.f - dec + al) : kk) : 0.f;
            o.a[e] = keep ? (KK ? kk : al) : 0.f;
            o.b[e] = keep ? (KK ? kk * al : x.b.get(e)) : 0.f;
        }
        #pragma unroll
        for (int i = 0; i < R; ++i) o.v[i] = keep ? x.v.get(i) : 0.f;
    };
    // Removal projection of token `o` for the lane's 4 rows, summed over the DPP row
    // (every lane gets the sums).
    auto projection = [&](const Tok<C, R>& o, float (&sa)[R]) {
        #pragma unroll
        for (int i = 0; i < R; ++i) {
            float s = S[i][0] * o.a[0];
            #pragma unroll
            for (int e = 1; e < C; ++e) s = fmaf(S[i][e], o.a[e], s);
            sa[i] = s;
        }
        float ss = 0.f;
        if constexpr (KK) {
            ss = o.a[0] * o.a[0];
            #pragma unroll
            for (int e = 1; e < C; ++e) ss = fmaf(o.a[e], o.a[e], ss);
        }
        #pragma unroll
        for (int i = 0; i < R; ++i) sa[i] = sum16(sa[i]);
        if constexpr (KK) {
            const float inv = inv_key_norm(sum16(ss));
            const float c2 = -inv * inv;
            #pragma unroll
            for (int i = 0; i < R; ++i) sa[i] *= c2;
        }
    };

    const uint32_t oy = uint32_t(row0 + cb / (16 / R)) * SY;
    const bool ylane = cb % (16 / R) == 0;

    // Ring of raw loads: slot (t mod PF) holds token t until it is decoded.  Each
    // token's loads are issued together (not interleaved with other tokens'), so
    // that the wait for the oldest token leaves the younger ones in flight.
    constexpr int PF = kPF<D, Tin>;
    TokRaw<Tin, C, R> ring[PF];
    #pragma unroll
    for (int s = 0; s < PF; ++s) {
        load(s, ring[s]);
        __builtin_amdgcn_sched_barrier(0);
    }
    Tok<C, R> ta, tb;
    decode(ring[0], ta);
    load(PF, ring[0]);
    float sa[R];
    projection(ta, sa);

    // One token: S_t from S_{t-1} (token t decoded in cur), y_t, and the projection
    // of token t + 1 (decoded into nxt from its ring slot, which then takes the
    // loads of token t + 1 + PF).
    auto step = [&](const int t, TokRaw<Tin, C, R>& slot, const Tok<C, R>& cur, Tok<C, R>& nxt) {
        decode(slot, nxt);                 // token t + 1 (unused at t = T - 1)
        // The decoded values are materialised here, so the slot's registers are free
        // for its next loads: the loop then needs no register copies of loads in
        // flight (a copy waits for its load, at the loop's back edge).
        #pragma unroll
        for (int e = 0; e < C; ++e) {
            settle(nxt.r[e]); settle(nxt.dec[e]); settle(nxt.k[e]); settle(nxt.a[e]); settle(nxt.b[e]);
        }
        #pragma unroll
        for (int i = 0; i < R; ++i) settle(nxt.v[i]);
        load(t + 1 + PF, slot);
        float yp[R];
        #pragma unroll
        for (int i = 0; i < R; ++i) {
            float y = 0.f;
            #pragma unroll
            for (int e = 0; e < C; ++e) {
                float s = S[i][e] * cur.dec[e];
                s = fmaf(sa[i], cur.b[e], s);
                s = fmaf(cur.v[i], cur.k[e], s);
                S[i][e] = s;
                y = fmaf(s, cur.r[e], y);
            }
            yp[i] = y;
        }
        projection(nxt, sa);
        float yv = reduce_scatter(yp, cb) * g.y_scale;
        if constexpr (EPI) {
            float bon = 0.f;
            #pragma unroll
            for (int e = 0; e < C; ++e) bon = fmaf(cur.r[e] * cur.k[e], rk[e], bon);
            bon = sum16(bon);
            // v of the lane's output row, by bit selects.
            const bool b4 = cb & 4, b8 = cb & 8;
            float vo;
            if constexpr (R == 4) vo = b8 ? (b4 ? cur.v[3] : cur.v[2]) : (b4 ? cur.v[1] : cur.v[0]);
            else vo = b8 ? cur.v[1] : cur.v[0];
            yv = fmaf(bon, vo, yv);
        }
        if (ylane) store_out<Ty>(Ry, oy, uint32_t(t - t_base) * step_y, yv);
    };
    // Unrolled by PF (ring slots known at compile time), the decoded tokens
    // alternating between ta and tb (no copies).
    static_assert(PF % 2 == 0, "even ring");
    int t = 0;
    for (; t + PF <= T; t += PF) {
        rebase(t);
        #pragma unroll
        for (int s = 0; s < PF; s += 2) {
            step(t + s, ring[(s + 1) % PF], ta, tb);
            step(t + s + 1, ring[(s + 2) % PF], tb, ta);
        }
    }
    rebase(t);
    #pragma unroll
    for (int s = 0; s < PF - 1; ++s) {
        if (t + s >= T) break;
        if (s & 1) step(t + s, ring[(s + 1) % PF], tb, ta);
        else step(t + s, ring[(s + 1) % PF], ta, tb);
    }

    if (g.s1) {
        #pragma unroll
        for (int i = 0; i < R; ++i)
            #pragma unroll
            for (int e = 0; e < C; e += 4)
                *reinterpret_cast<float4*>(g.s1 + sbase + int64_t(row0 + i) * D + col0 + e) =
                    make_float4(S[i][e], S[i][e + 1], S[i][e + 2], S[i][e + 3]);
    }
}

template <int D, typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
hipError_t launch_t(const Params& p, hipStream_t stream) {
    const int bh = p.B * p.H;
    Args g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.mask, p.y, p.s1, p.T, p.H, p.H_kv, bh, p.y_scale};
    // D = 64: one workgroup per (b, h); D = 128: 4 per (b, h), in groups of 8 (b, h).
    const unsigned grid = D == 64 ? unsigned(bh) : unsigned((bh + 7) / 8) * 32u;
    hipLaunchKernelGGL((scan_dpp_kernel<D, Tin, Ty, LOGW, EPI, KK, MASK>), dim3(grid), dim3(256), 0, stream, g);
    return hipGetLastError();
}

template <int D, typename Tin, typename Ty, bool KK, bool MASK>
hipError_t dispatch_epi(const Params& p, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_t<D, Tin, Ty, true, true, KK, MASK>(p, s) : launch_t<D, Tin, Ty, true, false, KK, MASK>(p, s);
    return epi ? launch_t<D, Tin, Ty, false, true, KK, MASK>(p, s) : launch_t<D, Tin, Ty, false, false, KK, MASK>(p, s);
}

template <int D, typename Tin, typename Ty, bool KK>
hipError_t dispatch_mask(const Params& p, hipStream_t s) {
    return p.mask ? dispatch_epi<D, Tin, Ty, KK, true>(p, s) : dispatch_epi<D, Tin, Ty, KK, false>(p, s);
}

template <int D, typename Tin, typename Ty>
hipError_t dispatch_modes(const Params& p, hipStream_t s) {
    return p.ab_mode == WKV7_AB_FROM_K ? dispatch_mask<D, Tin, Ty, true>(p, s) : dispatch_mask<D, Tin, Ty, false>(p, s);
}

template <int D>
hipError_t dispatch_types(const Params& p, hipStream_t s) {
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<D, bf16_t, bf16_t>(p, s) : dispatch_modes<D, bf16_t, float>(p, s);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<D, float, bf16_t>(p, s) : dispatch_modes<D, float, float>(p, s);
}

}  // namespace

bool scan_fits(const Params& p) {
    // D = 64 or 128, the byte offsets of 2 PF + 1 tokens (PF <= kPFMax) of the
    // widest per-token row (r, w, a, b or y at 4 bytes per element) fit the 32-bit
    // buffer offsets, and the grid's work-items fit in 32 bits.
    return (p.D == 64 || p.D == 128) && p.T >= 1 &&
           int64_t(2 * kPFMax + 1) * p.H * p.D * 4 < (int64_t(1) << 32) &&
           (int64_t(p.B) * p.H + 7) / 8 * 8 * (p.D == 64 ? 1 : 4) * 256 <= int64_t(0xffffffffu);
}

hipError_t launch_scan(const Params& p, hipStream_t stream) {
    if (!scan_fits(p)) return hipErrorInvalidValue;
    return p.D == 64 ? dispatch_types<64>(p, stream) : dispatch_types<128>(p, stream);
}

}  // namespace wkv7
