// Chunk-parallel WKV-7 forward on gfx950 bf16 matrix cores (fp32 accumulation).
//
// The pages say only that the WKV operation parallelises over chunks
// (youngju.dev RWKV-7 article, Q&A 5).  The algebra used here follows from
// unrolling the update S_t = S_{t-1}(diag(w_t) + a_t b_t^T) + v_t k_t^T (wiki
// note "RWKV-7 Goose", generalised delta rule) over a chunk of L = 64 tokens
// starting from S0.  With g_t = sum_{s<=t} log2 w_s (per key column j),
// E(t, s) = 2^(g_t - g_s), and sa_t = S_{t-1} a_t:
//
//   A_ab[t,s] = sum_j a_tj b_sj 2^(g_{t-1,j} - g_sj)   (s < t)    A_ak likewise with k
//   A_rb[t,s] = sum_j r_tj b_sj 2^(g_tj - g_sj)        (s <= t)   A_rk likewise with k
//   SA  = (I - A_ab)^-1 (At S0^T + A_ak V)        At_t = a_t 2^(g_{t-1})
//   Y   = Rt S0^T + A_rb SA + A_rk V              Rt_t = r_t 2^(g_t)
//   S_L = S0 diag(2^g_L) + SA^T Bh + V^T Kh       Bh_s = b_s 2^(g_L - g_s), Kh likewise
//
// All matrix products run on v_mfma_f32_16x16x{16,32}_bf16.  Operands that
// decide the result to within the tolerance are split into bf16 hi + lo parts
// (x = hi + lo to ~16 mantissa bits) and multiplied term by term: the scaled r
// and k that form A_rk / A_rb, A_rk and A_ak themselves, the state in its
// products, K-hat, the removal projections RHS / SA, and v itself when the
// inputs are fp32 (bf16 inputs are exact as bf16).  The state itself is
// carried in fp32 registers and its decay 2^g_L is applied elementwise.
//
// Mapping: one 256-thread workgroup per (b, h); wave w owns value rows
// i in [16w, 16w+16).  Everything that depends on the state -- RHS, the
// blocked triangular solve for SA, Y and the new state -- stays in that
// wave's registers: the fp32 C layout of a 16x16 MFMA result is exactly the B
// operand layout of a 16x16x16 MFMA, and the state is kept transposed
// (S^T tiles: lane = value row, registers = key columns) so that it is the B
// operand of At S0^T and Rt S0^T directly.  Only quantities that do not
// depend on the state (decay prefix, scaled operands, the four L x L
// matrices, the inverses of the diagonal 16 x 16 blocks of I - A_ab) are
// built cooperatively in LDS, with barriers between those phases.
//
// Domain: the per-column decay product over one chunk must stay above 2^-126
// (2^(-g) is formed explicitly); the hxa07D decay parameterisation keeps
// w >= exp(-exp(-0.5)) = 0.545, i.e. |g_L| <= 56.  A ragged last chunk is
// padded with identity tokens (w = 1, a = b = k = v = r = 0).
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int L = 64;          // chunk length
constexpr int DH = 64;         // head size handled by this kernel
constexpr int NTHR = 256;
constexpr int P72 = 72;        // bf16 pitch of the 64 x 64 operand matrices (144 B rows)
constexpr int MAT = 64 * P72 * 2;
constexpr int PD = 20;         // pitch of the 16 x 16 diagonal blocks
constexpr int PG = 68;         // fp32 pitch of the decay-prefix scratch

// LDS map (bytes).  Region 1 holds B~, K~ during P1..P2 and A_ab, A_rb and the
// fp32 diagonal blocks of A_ab afterwards; region 2 holds the prefix scratch
// during P1 and A_ak, A_rk afterwards.
constexpr int OFF_AT = 0;
constexpr int OFF_RTH = OFF_AT + MAT;
constexpr int OFF_RTL = OFF_RTH + MAT;
constexpr int OFF_VT = OFF_RTL + MAT;      // V^T  [i][s]
constexpr int OFF_BHT = OFF_VT + MAT;      // Bh^T [j][s]
constexpr int OFF_KHTH = OFF_BHT + MAT;    // Kh^T [j][s] hi / lo
constexpr int OFF_KHTL = OFF_KHTH + MAT;
constexpr int OFF_R1 = OFF_KHTL + MAT;
constexpr int OFF_BT = OFF_R1;             // B~ [s][j]
constexpr int OFF_KTH = OFF_R1 + MAT;      // K~ [s][j] hi / lo
constexpr int OFF_KTL = OFF_R1 + 2 * MAT;
constexpr int OFF_AAB = OFF_R1;            // A_ab [t][s] bf16
constexpr int OFF_ARB = OFF_R1 + MAT;      // A_rb [t][s] bf16
constexpr int OFF_ADIAG = OFF_R1 + 2 * MAT;  // fp32 [4][16][PD] diagonal blocks of A_ab
constexpr int OFF_R2 = OFF_R1 + 3 * MAT;
constexpr int OFF_G = OFF_R2;              // fp32 [64][PG] decay prefix
constexpr int OFF_TOT = OFF_R2 + 64 * PG * 4;  // fp32 [4][64] segment totals
constexpr int OFF_AKH = OFF_R2;            // A_ak [t][s] hi / lo
constexpr int OFF_AKL = OFF_R2 + MAT;
constexpr int OFF_RKH = OFF_R2 + 2 * MAT;  // A_rk [t][s] hi / lo
constexpr int OFF_RKL = OFF_R2 + 3 * MAT;
constexpr int OFF_DINV = OFF_R2 + 4 * MAT;   // bf16 [4][16][PD] inverses of diagonal blocks
constexpr int OFF_GL = OFF_DINV + 4 * 16 * PD * 2;
constexpr int OFF_BONUS = OFF_GL + 256;
constexpr int OFF_VTL = OFF_BONUS + 256;   // V^T lo part (fp32 inputs only)
constexpr int SMEM_BF16 = OFF_VTL;
constexpr int SMEM_F32 = OFF_VTL + MAT;
static_assert(4 * 16 * PD * 4 <= MAT, "diagonal blocks fit");
static_assert(64 * PG * 4 + 1024 <= 2 * MAT, "prefix scratch fits");
static_assert(SMEM_F32 <= 160 * 1024, "LDS budget");

struct ChunkArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    void* y;
    float* s1;
    int T, H, H_kv;
    float y_scale;
};

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    bf16x2 v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// x = hi + lo with hi, lo bf16 (pairs packed into one dword each).
__device__ __forceinline__ void split2(float x, float y, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(x, y);
    lo = pack_bf16(x - lo_f32(hi), y - hi_f32(hi));
}

// C-layout fp32 tile (4 consecutive k) -> 16x16x16 B operand, hi and lo parts.
__device__ __forceinline__ void to_operand(const f32x4 c, s16x4& hi, s16x4& lo) {
    uint32_t h0, l0, h1, l1;
    split2(c[0], c[1], h0, l0);
    split2(c[2], c[3], h1, l1);
    hi = __builtin_bit_cast(s16x4, make_uint2(h0, h1));
    lo = __builtin_bit_cast(s16x4, make_uint2(l0, l1));
}

template <typename T> __device__ __forceinline__ T lds(const char* base, int byte_off) {
    return *reinterpret_cast<const T*>(base + byte_off);
}
template <typename T> __device__ __forceinline__ void sts(char* base, int byte_off, T v) {
    *reinterpret_cast<T*>(base + byte_off) = v;
}

// One token row (16 consecutive elements) of an input tensor, undecoded.
template <typename Tin> struct Row16;
template <> struct Row16<bf16_t> {
    uint4 x[2];
    __device__ __forceinline__ void load(const bf16_t* p, bool ok) {
        if (ok) {
            x[0] = reinterpret_cast<const uint4*>(p)[0];
            x[1] = reinterpret_cast<const uint4*>(p)[1];
        } else {
            x[0] = x[1] = make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ float get(int e) const {
        const uint4& u = x[e >> 3];
        const uint32_t d = (e & 6) == 0 ? u.x : (e & 6) == 2 ? u.y : (e & 6) == 4 ? u.z : u.w;
        return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
    }
};
template <> struct Row16<float> {
    float4 x[4];
    __device__ __forceinline__ void load(const float* p, bool ok) {
        #pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = ok ? reinterpret_cast<const float4*>(p)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ float get(int e) const {
        const float4& u = x[e >> 2];
        return (e & 3) == 0 ? u.x : (e & 3) == 1 ? u.y : (e & 3) == 2 ? u.z : u.w;
    }
};

template <typename Tin, typename Ty, bool LOGW, bool EPI>
__global__ __launch_bounds__(NTHR)
void chunked_kernel(ChunkArgs g) {
    constexpr bool VSPLIT = sizeof(Tin) == 4;   // fp32 v is not exact in bf16
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;
    const int H = g.H, T = g.T;
    const int bh = blockIdx.x;
    const int bb = bh / H, h = bh - bb * H;
    const int hk = h / (H / g.H_kv);
    const int64_t step_q = int64_t(H) * DH, step_kv = int64_t(g.H_kv) * DH;
    const int64_t base_q = (int64_t(bb) * T * H + h) * DH;
    const int64_t base_kv = (int64_t(bb) * T * g.H_kv + hk) * DH;
    const Tin* rp = static_cast<const Tin*>(g.r);
    const Tin* wp = static_cast<const Tin*>(g.w);
    const Tin* kp = static_cast<const Tin*>(g.k);
    const Tin* vp = static_cast<const Tin*>(g.v);
    const Tin* ap = static_cast<const Tin*>(g.a);
    const Tin* bp = static_cast<const Tin*>(g.b);
    Ty* yp = static_cast<Ty*>(g.y);

    // State, transposed: ST[jt][r] = S[i = 16w + lr][j = 16jt + 4lq + r].
    f32x4 ST[4];
    const int i_row = 16 * w + lr;
    const int64_t sbase = int64_t(bh) * DH * DH + int64_t(i_row) * DH;
    #pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        if (g.s0) {
            const float4 x = *reinterpret_cast<const float4*>(g.s0 + sbase + 16 * jt + 4 * lq);
            ST[jt] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            ST[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // P1 thread mapping: token row t1 = tid / 4, columns [16 q1, 16 q1 + 16).
    const int t1 = tid >> 2, q1 = tid & 3;
    float rk16[16];
    if constexpr (EPI) {
        #pragma unroll
        for (int e = 0; e < 16; ++e) rk16[e] = g.r_k[h * DH + 16 * q1 + e];
    }
    Row16<Tin> rr, ww, kk, vv, aa, bbv;
    auto load_rows = [&](int c0) {
        const int t = c0 + t1;
        const bool ok = t < T;
        const int tt = ok ? t : 0;
        rr.load(rp + base_q + tt * step_q + 16 * q1, ok);
        ww.load(wp + base_q + tt * step_q + 16 * q1, ok);
        kk.load(kp + base_kv + tt * step_kv + 16 * q1, ok);
        vv.load(vp + base_kv + tt * step_kv + 16 * q1, ok);
        aa.load(ap + base_q + tt * step_q + 16 * q1, ok);
        bbv.load(bp + base_q + tt * step_q + 16 * q1, ok);
    };
    load_rows(0);

    const int nchunks = (T + L - 1) / L;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = ch * L;
        const bool tok_ok = c0 + t1 < T;
        // ---------------- P1: decay prefix and scaled operands ----------------
        float lw[16];
        #pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float x = ww.get(e);
            lw[e] = !tok_ok ? 0.f : LOGW ? -__builtin_amdgcn_exp2f(x * kLog2e) * kLog2e : __builtin_amdgcn_logf(x);
        }
        {
            char* G = smem + OFF_G;
            #pragma unroll
            for (int e = 0; e < 16; e += 4)
                sts<float4>(G, (t1 * PG + 16 * q1 + e) * 4, make_float4(lw[e], lw[e + 1], lw[e + 2], lw[e + 3]));
        }
        __syncthreads();
        {
            // Column prefix: thread (j, segment p) scans tokens [16p, 16p + 16).
            const int j = tid & 63, p = tid >> 6;
            char* G = smem + OFF_G;
            float pre[16];
            float run = 0.f;
            #pragma unroll
            for (int e = 0; e < 16; ++e) {
                run += lds<float>(G, ((16 * p + e) * PG + j) * 4);
                pre[e] = run;
            }
            sts<float>(smem + OFF_TOT, (p * 64 + j) * 4, run);
            __syncthreads();
            float off = 0.f;
            for (int pp = 0; pp < p; ++pp) off += lds<float>(smem + OFF_TOT, (pp * 64 + j) * 4);
            #pragma unroll
            for (int e = 0; e < 16; ++e) sts<float>(G, ((16 * p + e) * PG + j) * 4, pre[e] + off);
        }
        __syncthreads();
        float bonus_part = 0.f;
        {
            const char* G = smem + OFF_G;
            uint32_t at[8], rth[8], rtl[8], bt[8], kth[8], ktl[8];
            #pragma unroll
            for (int e = 0; e < 16; e += 2) {
                float E[2], Ep[2], Ei[2], Eh[2];
                #pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int j = 16 * q1 + e + u;
                    const float gt = lds<float>(G, (t1 * PG + j) * 4);
                    const float gp = t1 > 0 ? lds<float>(G, ((t1 - 1) * PG + j) * 4) : 0.f;
                    const float gl = lds<float>(G, (63 * PG + j) * 4);
                    E[u] = __builtin_amdgcn_exp2f(gt);
                    Ep[u] = __builtin_amdgcn_exp2f(gp);
                    Ei[u] = __builtin_amdgcn_exp2f(-gt);
                    Eh[u] = __builtin_amdgcn_exp2f(gl - gt);
                }
                const float a0 = aa.get(e), a1 = aa.get(e + 1);
                const float r0 = rr.get(e), r1 = rr.get(e + 1);
                const float b0 = bbv.get(e), b1 = bbv.get(e + 1);
                const float k0 = kk.get(e), k1 = kk.get(e + 1);
                at[e / 2] = pack_bf16(a0 * Ep[0], a1 * Ep[1]);
                split2(r0 * E[0], r1 * E[1], rth[e / 2], rtl[e / 2]);
                bt[e / 2] = pack_bf16(b0 * Ei[0], b1 * Ei[1]);
                split2(k0 * Ei[0], k1 * Ei[1], kth[e / 2], ktl[e / 2]);
                // Transposed operands: V^T, Bh^T, Kh^T (hi/lo), element by element.
                const float bh0 = b0 * Eh[0], bh1 = b1 * Eh[1];
                uint32_t khh, khl;
                split2(k0 * Eh[0], k1 * Eh[1], khh, khl);
                const int j0 = 16 * q1 + e;
                uint32_t vpk, vpl;
                split2(vv.get(e), vv.get(e + 1), vpk, vpl);
                if constexpr (VSPLIT) {
                    sts<uint16_t>(smem + OFF_VTL, ((j0) * P72 + t1) * 2, uint16_t(vpl));
                    sts<uint16_t>(smem + OFF_VTL, ((j0 + 1) * P72 + t1) * 2, uint16_t(vpl >> 16));
                }
                const uint32_t bhp = pack_bf16(bh0, bh1);
                sts<uint16_t>(smem + OFF_VT, ((j0) * P72 + t1) * 2, uint16_t(vpk));
                sts<uint16_t>(smem + OFF_VT, ((j0 + 1) * P72 + t1) * 2, uint16_t(vpk >> 16));
                sts<uint16_t>(smem + OFF_BHT, ((j0) * P72 + t1) * 2, uint16_t(bhp));
                sts<uint16_t>(smem + OFF_BHT, ((j0 + 1) * P72 + t1) * 2, uint16_t(bhp >> 16));
                sts<uint16_t>(smem + OFF_KHTH, ((j0) * P72 + t1) * 2, uint16_t(khh));
                sts<uint16_t>(smem + OFF_KHTH, ((j0 + 1) * P72 + t1) * 2, uint16_t(khh >> 16));
                sts<uint16_t>(smem + OFF_KHTL, ((j0) * P72 + t1) * 2, uint16_t(khl));
                sts<uint16_t>(smem + OFF_KHTL, ((j0 + 1) * P72 + t1) * 2, uint16_t(khl >> 16));
                if constexpr (EPI) bonus_part += r0 * k0 * rk16[e] + r1 * k1 * rk16[e + 1];
            }
            const int ro = (t1 * P72 + 16 * q1) * 2;
            sts<uint4>(smem + OFF_AT, ro, make_uint4(at[0], at[1], at[2], at[3]));
            sts<uint4>(smem + OFF_AT, ro + 16, make_uint4(at[4], at[5], at[6], at[7]));
            sts<uint4>(smem + OFF_RTH, ro, make_uint4(rth[0], rth[1], rth[2], rth[3]));
            sts<uint4>(smem + OFF_RTH, ro + 16, make_uint4(rth[4], rth[5], rth[6], rth[7]));
            sts<uint4>(smem + OFF_RTL, ro, make_uint4(rtl[0], rtl[1], rtl[2], rtl[3]));
            sts<uint4>(smem + OFF_RTL, ro + 16, make_uint4(rtl[4], rtl[5], rtl[6], rtl[7]));
            if (t1 == 63) {
                #pragma unroll
                for (int e = 0; e < 16; ++e)
                    sts<float>(smem + OFF_GL, (16 * q1 + e) * 4, lds<float>(G, (63 * PG + 16 * q1 + e) * 4));
            }
            // Region 1 (B~, K~) is not read before the next barrier by anyone
            // but the prefix scratch lives in region 2, so these stores are safe now.
            sts<uint4>(smem + OFF_BT, ro, make_uint4(bt[0], bt[1], bt[2], bt[3]));
            sts<uint4>(smem + OFF_BT, ro + 16, make_uint4(bt[4], bt[5], bt[6], bt[7]));
            sts<uint4>(smem + OFF_KTH, ro, make_uint4(kth[0], kth[1], kth[2], kth[3]));
            sts<uint4>(smem + OFF_KTH, ro + 16, make_uint4(kth[4], kth[5], kth[6], kth[7]));
            sts<uint4>(smem + OFF_KTL, ro, make_uint4(ktl[0], ktl[1], ktl[2], ktl[3]));
            sts<uint4>(smem + OFF_KTL, ro + 16, make_uint4(ktl[4], ktl[5], ktl[6], ktl[7]));
        }
        if constexpr (EPI) {
            // The four threads of a token row are one quad.
            bonus_part += dpp<kDppQuadXor1>(bonus_part);
            bonus_part += dpp<kDppQuadXor2>(bonus_part);
            if (q1 == 0) sts<float>(smem + OFF_BONUS, t1 * 4, bonus_part);
        }
        // Next chunk's rows: in flight during P2..P7.
        if (ch + 1 < nchunks) load_rows(c0 + L);
        __syncthreads();

        // ---------------- P2: the four L x L matrices ----------------
        // Tile list (tb, sb), sb <= tb; wave w takes tiles w, w + 4, w + 8.
        // Each tile is computed as C'[s][t] = Y[s] . X[t] so that a lane holds
        // 4 consecutive s of one t: a row-major [t][s] store of 4 elements.
        f32x4 acc_ab[3], acc_ak[3], acc_rb[3], acc_rk[3];
        int tile_tb[3], tile_sb[3];
        #pragma unroll
        for (int n = 0; n < 3; ++n) {
            const int id = w + 4 * n;
            int tb = 0, sb = 0;
            // id -> (tb, sb) over the lower triangle in row order.
            tb = id >= 6 ? 3 : id >= 3 ? 2 : id >= 1 ? 1 : 0;
            sb = id - (tb * (tb + 1)) / 2;
            tile_tb[n] = tb; tile_sb[n] = sb;
            acc_ab[n] = acc_ak[n] = acc_rb[n] = acc_rk[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (id < 10) {
                #pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    const int ya = ((16 * sb + lr) * P72 + 32 * kq + 8 * lq) * 2;  // Y row s
                    const int xb = ((16 * tb + lr) * P72 + 32 * kq + 8 * lq) * 2;  // X row t
                    const bf16x8 Bt8 = lds<bf16x8>(smem + OFF_BT, ya);
                    const bf16x8 Kh8 = lds<bf16x8>(smem + OFF_KTH, ya);
                    const bf16x8 Kl8 = lds<bf16x8>(smem + OFF_KTL, ya);
                    const bf16x8 At8 = lds<bf16x8>(smem + OFF_AT, xb);
                    const bf16x8 Rh8 = lds<bf16x8>(smem + OFF_RTH, xb);
                    const bf16x8 Rl8 = lds<bf16x8>(smem + OFF_RTL, xb);
                    acc_ab[n] = mfma32(Bt8, At8, acc_ab[n]);
                    acc_ak[n] = mfma32(Kh8, At8, acc_ak[n]);
                    acc_ak[n] = mfma32(Kl8, At8, acc_ak[n]);
                    acc_rb[n] = mfma32(Bt8, Rh8, acc_rb[n]);
                    acc_rb[n] = mfma32(Bt8, Rl8, acc_rb[n]);
                    acc_rk[n] = mfma32(Kh8, Rh8, acc_rk[n]);
                    acc_rk[n] = mfma32(Kh8, Rl8, acc_rk[n]);
                    acc_rk[n] = mfma32(Kl8, Rh8, acc_rk[n]);
                }
            }
        }
        __syncthreads();   // every wave has read B~ / K~ (region 1) and the prefix scratch is dead
        #pragma unroll
        for (int n = 0; n < 3; ++n) {
            const int id = w + 4 * n;
            if (id < 10) {
                const int tb = tile_tb[n], sb = tile_sb[n];
                const int t = 16 * tb + lr;            // C' column
                const int s0 = 16 * sb + 4 * lq;       // C' rows s0 .. s0 + 3
                f32x4 ab = acc_ab[n], ak = acc_ak[n], rb = acc_rb[n], rkk = acc_rk[n];
                if (tb == sb) {
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int sl = 4 * lq + r;
                        if (sl >= lr) { ab[r] = 0.f; ak[r] = 0.f; }
                        if (sl > lr) { rb[r] = 0.f; rkk[r] = 0.f; }
                    }
                    // fp32 copy of the diagonal block for the exact inverse.
                    sts<float4>(smem + OFF_ADIAG, ((tb * 16 + lr) * PD + 4 * lq) * 4,
                                make_float4(ab[0], ab[1], ab[2], ab[3]));
                }
                const int o = (t * P72 + s0) * 2;
                sts<uint2>(smem + OFF_AAB, o, make_uint2(pack_bf16(ab[0], ab[1]), pack_bf16(ab[2], ab[3])));
                sts<uint2>(smem + OFF_ARB, o, make_uint2(pack_bf16(rb[0], rb[1]), pack_bf16(rb[2], rb[3])));
                uint32_t h0, l0, h1, l1;
                split2(ak[0], ak[1], h0, l0); split2(ak[2], ak[3], h1, l1);
                sts<uint2>(smem + OFF_AKH, o, make_uint2(h0, h1));
                sts<uint2>(smem + OFF_AKL, o, make_uint2(l0, l1));
                split2(rkk[0], rkk[1], h0, l0); split2(rkk[2], rkk[3], h1, l1);
                sts<uint2>(smem + OFF_RKH, o, make_uint2(h0, h1));
                sts<uint2>(smem + OFF_RKL, o, make_uint2(l0, l1));
            }
        }
        {
            // Zero the upper tiles (t-block 0, s-block 1) and (2, 3) of A_ak and A_rk,
            // which the 32-deep products of P4/P6 read.
            const int tile = tid >> 6, m = (tid >> 5) & 1, rw = (tid & 31) >> 1, half = tid & 1;
            const int offs[4] = {OFF_AKH, OFF_AKL, OFF_RKH, OFF_RKL};
            const int tb = m ? 2 : 0, sb = tb + 1;
            sts<uint4>(smem + offs[tile], ((16 * tb + rw) * P72 + 16 * sb + 8 * half) * 2, make_uint4(0, 0, 0, 0));
        }
        __syncthreads();

        // ---------------- P3: inverses of the diagonal blocks of I - A_ab ----------------
        if (l < 16) {
            const int c = l;
            float x[16];
            #pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = (t == c) ? 1.f : 0.f;
                #pragma unroll
                for (int s = 0; s < t; ++s) acc = fmaf(lds<float>(smem + OFF_ADIAG, ((w * 16 + t) * PD + s) * 4), x[s], acc);
                x[t] = acc;
            }
            #pragma unroll
            for (int t = 0; t < 16; ++t)
                sts<uint16_t>(smem + OFF_DINV, ((w * 16 + t) * PD + c) * 2, __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[t])));
        }
        __syncthreads();

        // ---------------- P4: RHS = At S0^T + A_ak V for this wave's value rows ----------------
        // State as 16x16x16 B operands (k = key column j = 16 jt + 4 lq + r, n = value row).
        s16x4 Sh[4], Sl[4];
        #pragma unroll
        for (int jt = 0; jt < 4; ++jt) to_operand(ST[jt], Sh[jt], Sl[jt]);
        // V^T as 16x16x32 B operands (k = token s = 32 kq + 8 lq + e, n = value row).
        bf16x8 VB[2], VBl[2];
        #pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            VB[kq] = lds<bf16x8>(smem + OFF_VT, (i_row * P72 + 32 * kq + 8 * lq) * 2);
            if constexpr (VSPLIT) VBl[kq] = lds<bf16x8>(smem + OFF_VTL, (i_row * P72 + 32 * kq + 8 * lq) * 2);
        }
        f32x4 RHS[4];
        #pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const s16x4 A4 = lds<s16x4>(smem + OFF_AT, ((16 * tb + lr) * P72 + 16 * jt + 4 * lq) * 2);
                acc = mfma16(A4, Sh[jt], acc);
                acc = mfma16(A4, Sl[jt], acc);
            }
            #pragma unroll
            for (int kq = 0; kq <= tb / 2; ++kq) {
                const int o = ((16 * tb + lr) * P72 + 32 * kq + 8 * lq) * 2;
                const bf16x8 Ah8 = lds<bf16x8>(smem + OFF_AKH, o);
                acc = mfma32(Ah8, VB[kq], acc);
                acc = mfma32(lds<bf16x8>(smem + OFF_AKL, o), VB[kq], acc);
                if constexpr (VSPLIT) acc = mfma32(Ah8, VBl[kq], acc);
            }
            RHS[tb] = acc;
        }

        // ---------------- P5: SA = (I - A_ab)^-1 RHS, blocked forward substitution ----------------
        f32x4 SA[4];
        s16x4 SAh[4], SAl[4];
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            f32x4 x = RHS[ib];
            #pragma unroll
            for (int jb = 0; jb < ib; ++jb) {
                const s16x4 A4 = lds<s16x4>(smem + OFF_AAB, ((16 * ib + lr) * P72 + 16 * jb + 4 * lq) * 2);
                x = mfma16(A4, SAh[jb], x);
                x = mfma16(A4, SAl[jb], x);
            }
            s16x4 xh, xl;
            to_operand(x, xh, xl);
            const s16x4 D4 = lds<s16x4>(smem + OFF_DINV, ((16 * ib + lr) * PD + 4 * lq) * 2);
            f32x4 sa = {0.f, 0.f, 0.f, 0.f};
            sa = mfma16(D4, xh, sa);
            sa = mfma16(D4, xl, sa);
            SA[ib] = sa;
            to_operand(sa, SAh[ib], SAl[ib]);
        }

        // ---------------- P6: Y = Rt S0^T + A_rb SA + A_rk V ----------------
        #pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int o = ((16 * tb + lr) * P72 + 16 * jt + 4 * lq) * 2;
                const s16x4 Rh4 = lds<s16x4>(smem + OFF_RTH, o);
                const s16x4 Rl4 = lds<s16x4>(smem + OFF_RTL, o);
                acc = mfma16(Rh4, Sh[jt], acc);
                acc = mfma16(Rh4, Sl[jt], acc);
                acc = mfma16(Rl4, Sh[jt], acc);
            }
            #pragma unroll
            for (int sb = 0; sb <= tb; ++sb) {
                const s16x4 A4 = lds<s16x4>(smem + OFF_ARB, ((16 * tb + lr) * P72 + 16 * sb + 4 * lq) * 2);
                acc = mfma16(A4, SAh[sb], acc);
                acc = mfma16(A4, SAl[sb], acc);
            }
            #pragma unroll
            for (int kq = 0; kq <= tb / 2; ++kq) {
                const int o = ((16 * tb + lr) * P72 + 32 * kq + 8 * lq) * 2;
                const bf16x8 Rh8 = lds<bf16x8>(smem + OFF_RKH, o);
                acc = mfma32(Rh8, VB[kq], acc);
                acc = mfma32(lds<bf16x8>(smem + OFF_RKL, o), VB[kq], acc);
                if constexpr (VSPLIT) acc = mfma32(Rh8, VBl[kq], acc);
            }
            // acc[r] = Y[t = 16 tb + 4 lq + r][i_row]
            const int tl0 = 16 * tb + 4 * lq;
            float vtr[4], bon[4];
            if constexpr (EPI) {
                const uint2 vraw = lds<uint2>(smem + OFF_VT, (i_row * P72 + tl0) * 2);
                vtr[0] = lo_f32(vraw.x); vtr[1] = hi_f32(vraw.x); vtr[2] = lo_f32(vraw.y); vtr[3] = hi_f32(vraw.y);
                if constexpr (VSPLIT) {
                    const uint2 vlo = lds<uint2>(smem + OFF_VTL, (i_row * P72 + tl0) * 2);
                    vtr[0] += lo_f32(vlo.x); vtr[1] += hi_f32(vlo.x); vtr[2] += lo_f32(vlo.y); vtr[3] += hi_f32(vlo.y);
                }
                const float4 bq = lds<float4>(smem + OFF_BONUS, tl0 * 4);
                bon[0] = bq.x; bon[1] = bq.y; bon[2] = bq.z; bon[3] = bq.w;
            }
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = c0 + tl0 + r;
                float yv = acc[r] * g.y_scale;
                if constexpr (EPI) yv = fmaf(bon[r], vtr[r], yv);
                if (t < T) st1(yp, base_q + t * step_q + i_row, yv);
            }
        }

        // ---------------- P7: S_L^T = 2^g_L S0^T + Bh^T SA + Kh^T V ----------------
        #pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const float4 gl4 = lds<float4>(smem + OFF_GL, (16 * jt + 4 * lq) * 4);
            f32x4 acc = ST[jt];
            acc[0] *= __builtin_amdgcn_exp2f(gl4.x);
            acc[1] *= __builtin_amdgcn_exp2f(gl4.y);
            acc[2] *= __builtin_amdgcn_exp2f(gl4.z);
            acc[3] *= __builtin_amdgcn_exp2f(gl4.w);
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const s16x4 B4 = lds<s16x4>(smem + OFF_BHT, ((16 * jt + lr) * P72 + 16 * tb + 4 * lq) * 2);
                acc = mfma16(B4, SAh[tb], acc);
                acc = mfma16(B4, SAl[tb], acc);
            }
            #pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                const int o = ((16 * jt + lr) * P72 + 32 * kq + 8 * lq) * 2;
                const bf16x8 Kh8 = lds<bf16x8>(smem + OFF_KHTH, o);
                acc = mfma32(Kh8, VB[kq], acc);
                acc = mfma32(lds<bf16x8>(smem + OFF_KHTL, o), VB[kq], acc);
                if constexpr (VSPLIT) acc = mfma32(Kh8, VBl[kq], acc);
            }
            ST[jt] = acc;
        }
        __syncthreads();   // all LDS operands of this chunk consumed before P1 rewrites them
    }

    if (g.s1) {
        #pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            *reinterpret_cast<float4*>(g.s1 + sbase + 16 * jt + 4 * lq) = make_float4(ST[jt][0], ST[jt][1], ST[jt][2], ST[jt][3]);
    }
}

template <typename Tin, typename Ty, bool LOGW, bool EPI>
hipError_t launch_t(const Params& p, hipStream_t stream) {
    ChunkArgs g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.y, p.s1, p.T, p.H, p.H_kv, p.y_scale};
    auto kern = chunked_kernel<Tin, Ty, LOGW, EPI>;
    constexpr int smem = sizeof(Tin) == 4 ? SMEM_F32 : SMEM_BF16;
    static bool attr_set = false;   // per template instance; idempotent if raced
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(p.B) * unsigned(p.H)), dim3(NTHR), smem, stream, g);
    return hipGetLastError();
}

template <typename Tin, typename Ty>
hipError_t dispatch_modes(const Params& p, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_t<Tin, Ty, true, true>(p, s) : launch_t<Tin, Ty, true, false>(p, s);
    return epi ? launch_t<Tin, Ty, false, true>(p, s) : launch_t<Tin, Ty, false, false>(p, s);
}

}  // namespace

hipError_t launch_chunked(const Params& p, hipStream_t stream) {
    if (p.D != DH || p.chunk_len != L) return hipErrorInvalidValue;
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<bf16_t, bf16_t>(p, stream) : dispatch_modes<bf16_t, float>(p, stream);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<float, bf16_t>(p, stream) : dispatch_modes<float, float>(p, stream);
}

}  // namespace wkv7
