// One decode token per sequence: the WKV-7 update and readout with T = 1,
// streaming every (b, h) state through HBM exactly once (read state_in,
// write state_out).  RNN-mode inference keeps only this state per head
// (104case.com RWKV translation, RNN-like sequential decoding; youngju.dev
// RWKV-7 article, inference mode), so this kernel is bound by HBM bandwidth:
// 2 * D*D*4 bytes of state per head against 9*D*D flops.
//
// Mapping: one wave per (b, h), four heads per 256-thread workgroup.  The
// wave reads the row-major D x D state with 16-byte loads so that each load
// instruction covers 4 rows x 64 contiguous columns (1 KiB, fully coalesced):
// lane l = 16*rl + cq holds columns [4cq, 4cq+4) (and [64+4cq, 64+4cq+4) for
// D = 128) of rows 4*it + rl.  Row sums (S a for the removal term, S r for the
// readout) are a per-lane partial plus a 16-lane DPP all-reduce.  For D = 128
// the rows are processed in four batches of 32 to bound register use.
//
// With the kernel vectors formed from k (KK), the key norm is one more 16-lane
// sum; a masked token becomes the identity update (r, k, a, b = 0, decay 1),
// which leaves the state bit for bit and gives y = 0.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

struct DecodeArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    const uint8_t* mask;
    void* y;
    float* s1;
    int B, H, H_kv;
    float y_scale;
};

template <int D, typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
__global__ __launch_bounds__(256)
void decode_kernel(DecodeArgs g) {
    constexpr int CPL = D / 16;          // columns per lane (two groups of 4 for D = 128)
    constexpr int NG = CPL / 4;          // column groups of 4
    constexpr int NIT = D / 4;           // row iterations (4 rows each)
    constexpr int NB = (D == 64) ? 16 : 8;  // row iterations per batch
    constexpr int NBATCH = NIT / NB;

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t bh = int64_t(blockIdx.x) * 4 + wave;
    if (bh >= int64_t(g.B) * g.H) return;
    const int bb = int(bh / g.H), h = int(bh - int64_t(bb) * g.H);
    const int hk = h / (g.H / g.H_kv);
    const int rl = lane >> 4, cq = lane & 15;

    const Tin* __restrict__ rp = static_cast<const Tin*>(g.r);
    const Tin* __restrict__ wp = static_cast<const Tin*>(g.w);
    const Tin* __restrict__ kp = static_cast<const Tin*>(g.k);
    const Tin* __restrict__ vp = static_cast<const Tin*>(g.v);
    const Tin* __restrict__ ap = static_cast<const Tin*>(g.a);
    const Tin* __restrict__ bp = static_cast<const Tin*>(g.b);

    const int64_t oq = (int64_t(bb) * g.H + h) * D;        // T == 1
    const int64_t okv = (int64_t(bb) * g.H_kv + hk) * D;

    // This lane's columns of the per-token vectors.
    float av[CPL], wv[CPL], bv[CPL], kv[CPL], rv[CPL];
    #pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int col = 64 * gi + 4 * cq;
        ld4(ap, oq + col, av + 4 * gi);
        ld4(wp, oq + col, wv + 4 * gi);
        if constexpr (!KK) ld4(bp, oq + col, bv + 4 * gi);
        ld4(kp, okv + col, kv + 4 * gi);
        ld4(rp, oq + col, rv + 4 * gi);
    }
    if constexpr (LOGW) {
        #pragma unroll
        for (int c = 0; c < CPL; ++c) wv[c] = decay_from_logneglog(wv[c]);
    }
    if constexpr (KK) {
        // av holds alpha: kk = k / max(|k|, 1e-12), a = -kk, b = kk alpha, k <- k (1 - decay + alpha).
        float ss = 0.f;
        #pragma unroll
        for (int c = 0; c < CPL; ++c) ss = fmaf(kv[c], kv[c], ss);
        const float inv = inv_key_norm(sum16(ss));
        #pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float kk = kv[c] * inv, al = av[c];
            av[c] = -kk;
            bv[c] = kk * al;
            kv[c] *= 1.f - wv[c] + al;
        }
    }
    if (MASK && g.mask[bb] == 0) {   // T == 1: mask[b][0]
        #pragma unroll
        for (int c = 0; c < CPL; ++c) { av[c] = 0.f; bv[c] = 0.f; kv[c] = 0.f; rv[c] = 0.f; wv[c] = 1.f; }
    }
    // v: lane j holds v_j (and v_{64+j}); rows fetch theirs with a lane shuffle.
    float vl[D / 64];
    #pragma unroll
    for (int p = 0; p < D / 64; ++p) vl[p] = ld1(vp, okv + lane + 64 * p);

    float bonus = 0.f;
    if constexpr (EPI) {
        float part = 0.f;
        #pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            float rk4[4];
            ld4(g.r_k, int64_t(h) * D + 64 * gi + 4 * cq, rk4);
            #pragma unroll
            for (int c = 0; c < 4; ++c) part = fmaf(rv[4 * gi + c] * kv[4 * gi + c], rk4[c], part);
        }
        bonus = sum16(part);
    }

    const float* __restrict__ sin = g.s0 ? g.s0 + bh * D * D : nullptr;
    float* __restrict__ sout = g.s1 + bh * D * D;
    float ykeep[NIT / 16];
    #pragma unroll
    for (int i = 0; i < NIT / 16; ++i) ykeep[i] = 0.f;

    #pragma unroll
    for (int batch = 0; batch < NBATCH; ++batch) {
        float S[NB][CPL];
        // Load: iteration it covers rows 4*it .. 4*it+3; lane offset 16 B * lane within each 64-column half.
        #pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int row = 4 * (batch * NB + j) + rl;
            #pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (sin) {
                    const f32x4 x = __builtin_nontemporal_load(
                        reinterpret_cast<const f32x4*>(sin + int64_t(row) * D + 64 * gi + 4 * cq));
                    S[j][4 * gi] = x.x; S[j][4 * gi + 1] = x.y; S[j][4 * gi + 2] = x.z; S[j][4 * gi + 3] = x.w;
                } else {
                    S[j][4 * gi] = S[j][4 * gi + 1] = S[j][4 * gi + 2] = S[j][4 * gi + 3] = 0.f;
                }
            }
        }
        #pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int it = batch * NB + j;
            const int row = 4 * it + rl;
            float p0 = 0.f, p1 = 0.f;
            #pragma unroll
            for (int c = 0; c < CPL; c += 2) {
                p0 = fmaf(S[j][c], av[c], p0);
                p1 = fmaf(S[j][c + 1], av[c + 1], p1);
            }
            const float sa = sum16(p0 + p1);
            const float vi = __shfl(vl[(4 * it) / 64], row & 63);
            float y0 = 0.f, y1 = 0.f;
            #pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float s = fmaf(S[j][c], wv[c], sa * bv[c]);
                s = fmaf(vi, kv[c], s);
                S[j][c] = s;
                if (c & 1) y1 = fmaf(s, rv[c], y1); else y0 = fmaf(s, rv[c], y0);
            }
            float yi = sum16(y0 + y1) * g.y_scale;
            if constexpr (EPI) yi = fmaf(bonus, vi, yi);
            if ((it & 15) == cq) ykeep[it >> 4] = yi;
        }
        #pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int row = 4 * (batch * NB + j) + rl;
            #pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                f32x4 x = {S[j][4 * gi], S[j][4 * gi + 1], S[j][4 * gi + 2], S[j][4 * gi + 3]};
                __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(sout + int64_t(row) * D + 64 * gi + 4 * cq));
            }
        }
    }
    // Lane (rl, cq) holds y for rows 4*(cq + 16*m) + rl.
    Ty* __restrict__ yp = static_cast<Ty*>(g.y);
    #pragma unroll
    for (int m = 0; m < NIT / 16; ++m) st1(yp, oq + 4 * (cq + 16 * m) + rl, ykeep[m]);
}

template <int D, typename Tin, typename Ty, bool LOGW, bool EPI, bool KK, bool MASK>
hipError_t launch_t(const Params& p, hipStream_t stream) {
    DecodeArgs g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.mask, p.y, p.s1, p.B, p.H, p.H_kv, p.y_scale};
    const int64_t heads = int64_t(p.B) * p.H;
    dim3 grid(unsigned((heads + 3) / 4));
    hipLaunchKernelGGL((decode_kernel<D, Tin, Ty, LOGW, EPI, KK, MASK>), grid, dim3(256), 0, stream, g);
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

// T == 0: state_out <- state_in, or zeros.
__global__ __launch_bounds__(256) void state_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst, int64_t n4) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_decode(const Params& p, hipStream_t stream) {
    return p.D == 64 ? dispatch_types<64>(p, stream) : dispatch_types<128>(p, stream);
}

hipError_t launch_state_copy(const Params& p, hipStream_t stream) {
    const int64_t n4 = int64_t(p.B) * p.H * p.D * p.D / 4;
    if (p.s0 == p.s1) return hipSuccess;
    const int64_t blocks = (n4 + 255) / 256;
    dim3 grid(unsigned(blocks < 65536 ? blocks : 65536));
    hipLaunchKernelGGL(state_copy_kernel, grid, dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(p.s0), reinterpret_cast<float4*>(p.s1), n4);
    return hipGetLastError();
}

}  // namespace wkv7
