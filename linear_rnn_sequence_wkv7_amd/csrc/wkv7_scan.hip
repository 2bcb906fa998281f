// Token-by-token scan of the WKV-7 recurrence on gfx950: the dispatch of the
// scan algorithm, and its earlier form, kept for the calls the DPP-row scan
// (wkv7_scan_dpp.hip) does not take (rows so wide that the byte offsets of a few
// tokens overflow 32 bits, or grids beyond 2^32 work-items).
//
//   sa_t = S_{t-1} a_t;  S_t = S_{t-1} diag(w_t) + sa_t b_t^T + v_t k_t^T;  y_t = S_t r_t
//
// (generalised delta rule: wiki note "RWKV-7 Goose: Expressive Dynamic State
// Evolution", full state update; readout after the update as in the
// youngju.dev RWKV-7 article's time-mix pseudocode.)
//
// Mapping: one workgroup per (b, h).  Wave q owns the key columns
// [q*CS, (q+1)*CS); lane l owns value rows l and (for D = 128) l + 64, so a
// lane keeps RPL*CS state floats in VGPRs for the whole sequence.  The
// per-token vectors a, w, b, k, r restricted to a wave's columns are
// wave-uniform: they are loaded with scalar loads and used as SGPR operands,
// so every VALU instruction of the update reads one broadcast value for free.
// The removal projection S a is a sum over all D columns, i.e. over the
// NW = D/CS waves: each wave writes its partial to LDS, one barrier per token
// separates writes from reads (double-buffered), and every wave adds the NW
// partials of its rows.  Readout partials S r go to an LDS ring of TY tokens
// and are reduced, scaled, given the hxa07D bonus term and stored (coalesced)
// once every TY tokens.
//
// Kernel vectors from k (KK): the a slot carries alpha and b is not read.
// With kk = k / n, n = max(|k|, 1e-12), the removal term is
// (S a) b^T = -(S k)(k alpha)^T / n^2, so each wave reduces S k (not S a) and
// the partial |k|^2 of its columns through the same LDS exchange, and the
// update adds (-(S k) / n^2) (k alpha)_j and v (k (1 - decay + alpha))_j.
// Masked tokens (mask byte 0) run as the identity update: r, k, a, b = 0 and
// decay 1 leave the state bit for bit and give y = 0.  Lane i of a wave holds
// the mask byte of token t0 + i of the current ring block.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

struct ScanArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    const uint8_t* mask;
    void* y;
    float* s1;
    int B, T, H, H_kv;
    float y_scale;
};

template <int D> struct ScanShape;
template <> struct ScanShape<64> { static constexpr int CS = 8, TY = 16; };
template <> struct ScanShape<128> { static constexpr int CS = 8, TY = 4; };

// Raw (undecoded) per-token vector slice of one wave: CS = 8 columns of
// a, w, b, k, r as bf16 pairs or fp32, held in SGPRs.
template <typename Tin> struct RawSlice;
template <> struct RawSlice<bf16_t> {
    uint32_t a[4], w[4], b[4], k[4], r[4];
    template <bool LOAD_B>
    __device__ __forceinline__ void load(cptr<bf16_t> ap, cptr<bf16_t> wp, cptr<bf16_t> bp,
                                         cptr<bf16_t> kp, cptr<bf16_t> rp, int64_t oq, int64_t okv) {
        #pragma unroll
        for (int c = 0; c < 4; ++c) {
            a[c] = ((cptr<uint32_t>)(ap + oq))[c];
            w[c] = ((cptr<uint32_t>)(wp + oq))[c];
            b[c] = LOAD_B ? ((cptr<uint32_t>)(bp + oq))[c] : 0u;
            k[c] = ((cptr<uint32_t>)(kp + okv))[c];
            r[c] = ((cptr<uint32_t>)(rp + oq))[c];
        }
    }
    // The identity token: a, b, k, r = 0 and decay 1 (w = 1, or -inf in the log-decay mode).
    template <bool LOGW> __device__ __forceinline__ void make_identity() {
        #pragma unroll
        for (int c = 0; c < 4; ++c) {
            a[c] = 0u; b[c] = 0u; k[c] = 0u; r[c] = 0u;
            w[c] = LOGW ? 0xff80ff80u : 0x3f803f80u;
        }
    }
    static __device__ __forceinline__ float get(const uint32_t* x, int c) {
        return (c & 1) ? __uint_as_float(x[c >> 1] & 0xffff0000u) : __uint_as_float(x[c >> 1] << 16);
    }
    __device__ __forceinline__ float A(int c) const { return get(a, c); }
    __device__ __forceinline__ float W(int c) const { return get(w, c); }
    __device__ __forceinline__ float Bv(int c) const { return get(b, c); }
    __device__ __forceinline__ float K(int c) const { return get(k, c); }
    __device__ __forceinline__ float R(int c) const { return get(r, c); }
};
template <> struct RawSlice<float> {
    float a[8], w[8], b[8], k[8], r[8];
    template <bool LOAD_B>
    __device__ __forceinline__ void load(cptr<float> ap, cptr<float> wp, cptr<float> bp,
                                         cptr<float> kp, cptr<float> rp, int64_t oq, int64_t okv) {
        #pragma unroll
        for (int c = 0; c < 8; ++c) {
            a[c] = ap[oq + c]; w[c] = wp[oq + c]; b[c] = LOAD_B ? bp[oq + c] : 0.f;
            k[c] = kp[okv + c]; r[c] = rp[oq + c];
        }
    }
    template <bool LOGW> __device__ __forceinline__ void make_identity() {
        #pragma unroll
        for (int c = 0; c < 8; ++c) {
            a[c] = 0.f; b[c] = 0.f; k[c] = 0.f; r[c] = 0.f;
            w[c] = LOGW ? -__builtin_inff() : 1.f;
        }
    }
    __device__ __forceinline__ float A(int c) const { return a[c]; }
    __device__ __forceinline__ float W(int c) const { return w[c]; }
    __device__ __forceinline__ float Bv(int c) const { return b[c]; }
    __device__ __forceinline__ float K(int c) const { return k[c]; }
    __device__ __forceinline__ float R(int c) const { return r[c]; }
};

template <int D, typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
__global__ __launch_bounds__((D / ScanShape<D>::CS) * 64)
void scan_kernel(ScanArgs g) {
    constexpr int CS = ScanShape<D>::CS;
    static_assert(CS == 8, "a wave slice is 8 columns");
    constexpr int TY = ScanShape<D>::TY;
    constexpr int NW = D / CS;
    constexpr int RPL = D / 64;
    constexpr int NT = NW * 64;
    // L2 prefetch of the per-token vectors: 64-byte lines per token per vector.
    constexpr int LINES_PER_VEC = D * int(sizeof(Tin)) / 64;
    constexpr int PF_LINES = TY * 6 * LINES_PER_VEC;       // r, w, k, v, a, b for TY tokens

    constexpr int VPT = (TY * D + NT - 1) / NT;            // v values staged per thread per block

    __shared__ float red[2][NW][D];
    __shared__ float ybuf[TY][NW][D];
    __shared__ float vbuf[TY][D];
    __shared__ float bonus_buf[TY][NW];
    __shared__ float ksq_buf[2][NW];       // per-wave |k|^2 partials (KK)

    // Wave-uniform reads of the per-token vectors go through the scalar path.
    const cptr<Tin> rp = as_const(static_cast<const Tin*>(g.r));
    const cptr<Tin> wp = as_const(static_cast<const Tin*>(g.w));
    const cptr<Tin> kp = as_const(static_cast<const Tin*>(g.k));
    const cptr<Tin> ap = as_const(static_cast<const Tin*>(g.a));
    const cptr<Tin> bp = as_const(static_cast<const Tin*>(g.b));
    const Tin* __restrict__ vp = static_cast<const Tin*>(g.v);
    Ty* __restrict__ yp = static_cast<Ty*>(g.y);

    const int T = g.T, H = g.H, H_kv = g.H_kv;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x;
    const int bb = bh / H, h = bh - bb * H;
    const int hk = h / (H / H_kv);
    const int c0 = q * CS;

    // Row/column bases (token 0).
    const int64_t base_q = (int64_t(bb) * T * H + h) * D;      // r, w, a, b, y
    const int64_t base_kv = (int64_t(bb) * T * H_kv + hk) * D; // k, v
    const int64_t step_q = int64_t(H) * D, step_kv = int64_t(H_kv) * D;

    float S[RPL][CS];
    const int64_t sbase = int64_t(bh) * D * D;
    #pragma unroll
    for (int p = 0; p < RPL; ++p) {
        const int row = lane + 64 * p;
        if (g.s0) {
            #pragma unroll
            for (int c = 0; c < CS; c += 4) {
                float4 x = *reinterpret_cast<const float4*>(g.s0 + sbase + int64_t(row) * D + c0 + c);
                S[p][c] = x.x; S[p][c + 1] = x.y; S[p][c + 2] = x.z; S[p][c + 3] = x.w;
            }
        } else {
            #pragma unroll
            for (int c = 0; c < CS; ++c) S[p][c] = 0.f;
        }
    }

    #pragma unroll
    for (int p = 0; p < RPL; ++p) {
        #pragma unroll
        for (int c = 0; c < CS; ++c) settle(S[p][c]);
    }

    float rk[CS];
    if constexpr (EPI) {
        #pragma unroll
        for (int c = 0; c < CS; ++c) rk[c] = g.r_k ? g.r_k[h * D + c0 + c] : 0.f;
    }

    // Touch every 64-byte line of the six input rows for tokens [tb, tb + TY)
    // so that the scalar loads of those tokens hit L2.  The loaded words are
    // folded into `sink` one ring block later, which keeps the loads alive
    // without waiting on them early.  Thread -> (vector, token, line) is fixed;
    // ids past the last line and tokens past the end are clamped to valid
    // addresses (a repeated touch is harmless), so there are no branches.
    static_assert(PF_LINES <= NT, "one prefetch line per thread");
    const int64_t total_q = int64_t(g.B) * T * H * D, total_kv = int64_t(g.B) * T * H_kv * D;
    gptr<uint32_t> pf_base;
    int64_t pf_off, pf_step, pf_last;
    {
        const int id = min(int(threadIdx.x), PF_LINES - 1);
        const int line = id % LINES_PER_VEC;
        const int vec = (id / LINES_PER_VEC) % 6;
        const int s_tok = id / (LINES_PER_VEC * 6);
        // b is not read (and may be null) when the kernel vectors come from k: touch a again.
        const void* src = vec == 0 ? g.r : vec == 1 ? g.w : vec == 2 ? g.k : vec == 3 ? g.v : vec == 4 || KK ? g.a : g.b;
        const bool kvv = (vec == 2 || vec == 3);
        pf_base = as_global(static_cast<const uint32_t*>(src));
        pf_step = kvv ? step_kv : step_q;
        pf_off = (kvv ? base_kv : base_q) + s_tok * pf_step + line * (64 / int(sizeof(Tin)));
        pf_last = (kvv ? total_kv : total_q) - 1;
    }
    uint32_t pf = 0, sink = 0;
    auto prefetch = [&](int tb) {
        const int64_t e = min(pf_off + tb * pf_step, pf_last);
        pf = pf_base[e * int64_t(sizeof(Tin)) / 4];
    };
    prefetch(0);
    prefetch(TY);

    // v for the TY tokens of a ring block is staged in LDS as fp32.
    float vstage[VPT];
    int64_t voff[VPT];
    #pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int e = min(int(threadIdx.x) + u * NT, TY * D - 1);
        voff[u] = base_kv + (e / D) * step_kv + (e % D);
    }
    auto load_v = [&](int tb) {
        #pragma unroll
        for (int u = 0; u < VPT; ++u) vstage[u] = ld1(vp, min(voff[u] + tb * step_kv, total_kv - 1));
    };
    auto store_v = [&]() {
        #pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = threadIdx.x + u * NT;
            if (e < TY * D) vbuf[e / D][e % D] = vstage[u];
        }
    };
    // Mask bytes of a ring block: lane i holds token tb + i's (1 without a mask).
    const int64_t mbase = int64_t(bb) * T;
    auto load_mask = [&](int tb) -> uint32_t {
        return MASK ? uint32_t(g.mask[mbase + min(tb + lane, T - 1)]) : 1u;
    };
    uint32_t mnext = load_mask(0), mcur = 0;
    load_v(0);
    store_v();
    mcur = mnext;
    __syncthreads();

    int t0 = 0;  // first token of the current ring block
    // One token.  `cur` holds this token's vector slice; the next token's is
    // loaded into `nxt` while this token's update runs.
    auto step = [&](const int t, const RawSlice<Tin>& in, RawSlice<Tin>& nxt) {
        const int buf = t & 1;
        RawSlice<Tin> cur = in;
        if constexpr (MASK) {
            if (__builtin_amdgcn_readlane(int(mcur), t - t0) == 0) cur.template make_identity<LOGW>();
        }
        // Partial removal projection over this wave's columns (S k for KK).
        #pragma unroll
        for (int p = 0; p < RPL; ++p) {
            float s0 = 0.f, s1 = 0.f;
            #pragma unroll
            for (int c = 0; c < CS; c += 2) {
                s0 = fmaf(S[p][c], KK ? cur.K(c) : cur.A(c), s0);
                s1 = fmaf(S[p][c + 1], KK ? cur.K(c + 1) : cur.A(c + 1), s1);
            }
            red[buf][q][lane + 64 * p] = s0 + s1;
        }
        if constexpr (KK) {
            if (lane == 0) {
                float ss = 0.f;
                #pragma unroll
                for (int c = 0; c < CS; ++c) ss = fmaf(cur.K(c), cur.K(c), ss);
                ksq_buf[buf][q] = ss;
            }
        }
        __syncthreads();
        float sa[RPL], vrow[RPL];
        #pragma unroll
        for (int p = 0; p < RPL; ++p) {
            float acc = 0.f;
            #pragma unroll
            for (int qq = 0; qq < NW; ++qq) acc += red[buf][qq][lane + 64 * p];
            sa[p] = acc;
            vrow[p] = vbuf[t - t0][lane + 64 * p];
            settle(vrow[p]);
            settle(sa[p]);
        }
        // KK: sa holds S k; the removal coefficient of (k alpha)_j is -(S k) / n^2.
        if constexpr (KK) {
            float ss = 0.f;
            #pragma unroll
            for (int qq = 0; qq < NW; ++qq) ss += ksq_buf[buf][qq];
            const float inv = inv_key_norm(ss);
            const float c2 = -inv * inv;
            #pragma unroll
            for (int p = 0; p < RPL; ++p) sa[p] *= c2;
        }
        // Issue the next token's scalar loads only after the LDS reads above
        // have been waited on (SMEM and LDS share one wait counter), so they
        // stay in flight during this token's update.
        __builtin_amdgcn_sched_barrier(0);
        const int tn = (t + 1 < T) ? t + 1 : t;
        nxt.template load<!KK>(ap, wp, bp, kp, rp, base_q + tn * step_q + c0, base_kv + tn * step_kv + c0);

        // State update (in place: S*w, then + sa*b, then + v*k) and partial readout.
        #pragma unroll
        for (int p = 0; p < RPL; ++p) {
            float y0 = 0.f, y1 = 0.f;
            #pragma unroll
            for (int c = 0; c < CS; ++c) {
                const float wc = LOGW ? decay_from_logneglog(cur.W(c)) : cur.W(c);
                // KK: b_j -> (k alpha)_j (sa already carries -1/n^2), k_j -> k_j (1 - w_j + alpha_j).
                const float bc = KK ? cur.K(c) * cur.A(c) : cur.Bv(c);
                const float kc = KK ? cur.K(c) * (1.f - wc + cur.A(c)) : cur.K(c);
                float s = S[p][c] * wc;
                s = fmaf(sa[p], bc, s);
                s = fmaf(vrow[p], kc, s);
                S[p][c] = s;
                if (c & 1) y1 = fmaf(s, cur.R(c), y1); else y0 = fmaf(s, cur.R(c), y0);
            }
            ybuf[t - t0][q][lane + 64 * p] = y0 + y1;
        }
        if constexpr (EPI) {
            if (lane == 0) {
                float bsum = 0.f;
                #pragma unroll
                for (int c = 0; c < CS; ++c) {
                    float kc = cur.K(c);
                    if constexpr (KK) {
                        const float wc = LOGW ? decay_from_logneglog(cur.W(c)) : cur.W(c);
                        kc *= 1.f - wc + cur.A(c);
                    }
                    bsum = fmaf(cur.R(c) * kc, rk[c], bsum);
                }
                bonus_buf[t - t0][q] = bsum;
            }
        }
        // End of a ring block: reduce and store y, stage the next block's v,
        // and prefetch the block after next into L2.
        if (t - t0 == TY - 1 || t == T - 1) {
            __syncthreads();
            load_v(t + 1);
            mnext = load_mask(t + 1);
            const int nsteps = t - t0 + 1;
            for (int e = threadIdx.x; e < nsteps * D; e += NT) {
                const int s = e / D, i = e - s * D;
                float acc = 0.f;
                #pragma unroll
                for (int qq = 0; qq < NW; ++qq) acc += ybuf[s][qq][i];
                acc *= g.y_scale;
                if constexpr (EPI) {
                    float bsum = 0.f;
                    #pragma unroll
                    for (int qq = 0; qq < NW; ++qq) bsum += bonus_buf[s][qq];
                    acc = fmaf(bsum, vbuf[s][i], acc);
                }
                st1(yp, base_q + (t0 + s) * step_q + i, acc);
            }
            // Every wave finished reading vbuf (barrier above) and this thread's
            // epilogue reads of it are done; the next token's barrier publishes it.
            __syncthreads();
            store_v();
            mcur = mnext;
            // Issued last so that no wait in the ring block below covers them.
            sink ^= pf;
            prefetch(t0 + 2 * TY);
            t0 = t + 1;
        }
    };

    // Two tokens per iteration with the slices swapping roles (no SGPR copies).
    RawSlice<Tin> sl0, sl1;
    sl0.template load<!KK>(ap, wp, bp, kp, rp, base_q + c0, base_kv + c0);
    int t = 0;
    for (; t + 1 < T; t += 2) {
        step(t, sl0, sl1);
        step(t + 1, sl1, sl0);
    }
    if (t < T) step(t, sl0, sl1);

    if (g.s1) {
        #pragma unroll
        for (int p = 0; p < RPL; ++p) {
            const int row = lane + 64 * p;
            #pragma unroll
            for (int c = 0; c < CS; c += 4) {
                float4 x = make_float4(S[p][c], S[p][c + 1], S[p][c + 2], S[p][c + 3]);
                *reinterpret_cast<float4*>(g.s1 + sbase + int64_t(row) * D + c0 + c) = x;
            }
        }
    }
    // Never true for valid inputs (T >= 1 leaves t0 == T); keeps the prefetch loads live.
    if (g.s1 && t0 != T && sink == 0x9e3779b9u) g.s1[0] = 0.f;
}

template <int D, typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
hipError_t launch_scan_t(const Params& p, hipStream_t stream) {
    ScanArgs g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.mask, p.y, p.s1, p.B, p.T, p.H, p.H_kv, p.y_scale};
    dim3 grid(unsigned(p.B) * unsigned(p.H));
    dim3 block((D / ScanShape<D>::CS) * 64);
    hipLaunchKernelGGL((scan_kernel<D, Tin, Ty, LOGW, EPI, KK, MASK>), grid, block, 0, stream, g);
    return hipGetLastError();
}

template <int D, typename Tin, typename Ty, bool KK, bool MASK>
hipError_t dispatch_epi(const Params& p, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_scan_t<D, Tin, Ty, true, true, KK, MASK>(p, s) : launch_scan_t<D, Tin, Ty, true, false, KK, MASK>(p, s);
    return epi ? launch_scan_t<D, Tin, Ty, false, true, KK, MASK>(p, s) : launch_scan_t<D, Tin, Ty, false, false, KK, MASK>(p, s);
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

hipError_t launch_scan(const Params& p, hipStream_t stream) {
    if (scan_dpp_fits(p)) return launch_scan_dpp(p, stream);
    return p.D == 64 ? dispatch_types<64>(p, stream) : dispatch_types<128>(p, stream);
}

}  // namespace wkv7
