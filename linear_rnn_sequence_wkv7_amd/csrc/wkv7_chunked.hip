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
// All matrix products run on v_mfma_f32_16x16x32_bf16.  Operands that decide
// the result to within the tolerance are split into bf16 hi + lo parts
// (x = hi + lo to ~16 mantissa bits) and multiplied term by term: the scaled r
// and k that form A_rk / A_rb, A_rk and A_ak themselves, the state in its
// products, K-hat, the removal projections RHS / SA, and v itself when the
// inputs are fp32 (bf16 inputs are exact as bf16).  The state itself is
// carried in fp32 registers and its decay 2^g_L is applied elementwise.
//
// Mapping: one 512-thread workgroup (8 waves) per (b, h).  Waves w and w + 4
// share the value rows i in [16 (w mod 4), +16) ("strip"); each keeps half of
// the strip's state in registers, transposed (S^T tiles: lane = value row,
// registers = 4 consecutive key columns), which is exactly the C layout of a
// 16x16 MFMA result and the B-operand layout of a 16-deep product.  Two such
// 16-deep products are fused into one 32-deep MFMA: the matrices that are
// multiplied against register-resident operands (At, Rt, Bt, Kt along the key
// axis; A_ab, A_rb, Bh^T along the token axis) are stored in LDS with that
// axis interleaved in pairs of 16-blocks (position 32 p + 8 q + 4 e + r holds
// index 16 (2 p + e) + 4 q + r), so one 16-byte read gives the A operand of a
// pair.  A single 16-deep product against a split operand x = hi + lo is fused
// the same way: A = [a, a], B = [hi, lo].  The halves of the strip's state are
// exchanged once per chunk through LDS.  Only quantities that do not depend
// on the state (decay prefix, scaled operands, the four L x L matrices, the
// inverses of the diagonal 16 x 16 blocks of I - A_ab) are built
// cooperatively, with barriers between those phases.
//
// Every MFMA accumulator chain uses that one opcode: on gfx950, feeding the
// result of one MFMA opcode into another as its accumulator gave wrong values
// whenever the two issued close together (the compiler's wait states did not
// cover it), so a single 16-deep term is padded to 32 with zeros instead.
//
// Kernel vectors from k (KK): the a slot carries alpha and b is not read; per
// token kk = k / n with n = max(|k|, 1e-12), a = -kk, b = kk alpha and
// k' = k (1 - decay + alpha) (the hxa07D article's preparation before its
// kernel call, section 8).  The eight row threads of a token hold its 64 keys,
// so they form |k|^2 by an 8-lane sum and publish 1 / n in LDS.  The column
// threads, one chunk ahead, form k' and k alpha 2^(g_L - g) without it, and
// scale their Bh^T by 1 / n after the row phase of the chunk, so both layouts
// use the same 1 / n.  Row threads also read the decay row for k'.
//
// Global memory is read and written through buffer descriptors that cover
// the valid tokens of one chunk of one sequence: tokens past the end read as
// zero (identity tokens: a = b = k = v = r = 0; w is set to 1 explicitly) and
// their y stores are dropped by the range check.
//
// Domain: the per-column decay product over one chunk must stay above 2^-126
// (2^(-g) is formed explicitly); the hxa07D decay parameterisation keeps
// w >= exp(-exp(-0.5)) = 0.545, i.e. |g_L| <= 56.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int L = 64;          // chunk length
constexpr int DH = 64;         // head size handled by this kernel
constexpr int NTHR = 512;      // 8 waves: two per value strip
constexpr int P72 = 72;        // bf16 pitch of the 64 x 64 operand matrices (144 B rows)
constexpr int MAT = 64 * P72 * 2;
constexpr int PD = 20;         // pitch of the 16 x 16 diagonal blocks
constexpr int PE = 68;         // fp32 pitch of the decay tables

// LDS map (bytes).  Region 1 holds B~, K~ during P1b..P2 and A_ab, A_rb
// afterwards; region 2 holds the decay tables 2^g, 2^-g of the next chunk from
// P5 on (written after every wave has left P4) until P1b, and A_ak, A_rk from
// P2 to P4.
// Pair-interleaved axis (see above): At, Rt, Bt, Kt (key axis), A_ab, A_rb,
// Bh^T (token axis).  Natural order: A_ak, A_rk, Kh^T, V^T.
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
constexpr int OFF_R2 = OFF_R1 + 3 * MAT;
constexpr int OFF_E = OFF_R2;              // fp32 [64][PE] 2^g
constexpr int OFF_EI = OFF_R2 + 64 * PE * 4;   // fp32 [64][PE] 2^-g
constexpr int OFF_AKH = OFF_R2;            // A_ak [t][s] hi / lo
constexpr int OFF_AKL = OFF_R2 + MAT;
constexpr int OFF_RKH = OFF_R2 + 2 * MAT;  // A_rk [t][s] hi / lo
constexpr int OFF_RKL = OFF_R2 + 3 * MAT;
constexpr int OFF_DINV = OFF_R2 + 4 * MAT;   // bf16 [4][16][PD] inverses of diagonal blocks
constexpr int OFF_EL = OFF_DINV + 4 * 16 * PD * 2;   // fp32 [64] 2^g_L
constexpr int OFF_BONUS = OFF_EL + 256;    // fp32 [64] hxa07D bonus coefficient per token
constexpr int OFF_XS = OFF_BONUS + 256;    // state halves exchanged by the two waves of a strip
constexpr int XS_BYTES = 4 * 2 * 2 * 64 * 16;   // [strip][half][hi/lo][lane] 16 B
constexpr int OFF_TOT = OFF_XS + XS_BYTES; // fp32 [8][64] column-segment totals (own slot: written during P5)
constexpr int OFF_RK = OFF_TOT + 8 * 64 * 4;  // fp32 [64] r_k of this head (epilogue)
constexpr int OFF_INVN = OFF_RK + 64 * 4;     // fp32 [64] 1 / max(|k_t|, 1e-12) of the chunk's tokens (KK)
constexpr int OFF_VTL = OFF_INVN + 64 * 4;    // V^T lo part (fp32 inputs only)
constexpr int SMEM_BF16 = OFF_VTL;
constexpr int SMEM_F32 = OFF_VTL + MAT;
static_assert(2 * 64 * PE * 4 <= 4 * MAT, "decay tables fit");
static_assert(SMEM_F32 <= 160 * 1024, "LDS budget");

// Position of index k (0..63) on a pair-interleaved axis.
__host__ __device__ constexpr int pairpos(int k) {
    return 32 * (k >> 5) + 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3);
}
static_assert(pairpos(0) == 0 && pairpos(16) == 4 && pairpos(4) == 8 && pairpos(20) == 12 && pairpos(35) == 35 &&
              pairpos(51) == 39 && pairpos(63) == 63, "pair interleave");

struct ChunkArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    const uint8_t* mask;
    void* y;
    float* s1;
    int T, H, H_kv;
    float y_scale;
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(s16x4 a, s16x4 b) {
    return __builtin_bit_cast(bf16x8, s16x8(__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)));
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

// C-layout fp32 tile (4 consecutive k) -> 16-deep B operand, hi and lo parts.
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

// Raw buffer descriptor over [base, base + bytes); word 3 selects the 32-bit
// data format that gfx9-family raw buffer accesses need.  Accesses at byte
// offsets >= bytes read zero / are dropped.  Offsets are always passed in the
// VGPR operand (soffset 0), which the range check covers.
// The arguments are wave-uniform; reading them through readfirstlane keeps the
// descriptor in SGPRs (a descriptor in VGPRs costs a waterfall loop per access).
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, int(n), kRsrcWord3);
}

template <typename T> struct Buf;
template <> struct Buf<bf16_t> {
    // One element as fp32 bits.
    static __device__ __forceinline__ uint32_t load1(rsrc_t r, uint32_t off) {
        return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16;
    }
    static __device__ __forceinline__ void store1(rsrc_t r, uint32_t off, float x) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, off, 0, 0);
    }
};
template <> struct Buf<float> {
    static __device__ __forceinline__ uint32_t load1(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    static __device__ __forceinline__ void store1(rsrc_t r, uint32_t off, float x) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
    }
};

// 8 consecutive elements of one token row, undecoded (row threads).
template <typename Tin> struct Row8;
template <> struct Row8<bf16_t> {
    uint4 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    __device__ __forceinline__ void keep_if(bool keep) {
        x.x = keep ? x.x : 0u; x.y = keep ? x.y : 0u; x.z = keep ? x.z : 0u; x.w = keep ? x.w : 0u;
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t d = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
        return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
    }
};
template <> struct Row8<float> {
    uint4 x[2];
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        x[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        x[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
    }
    __device__ __forceinline__ void keep_if(bool keep) {
        #pragma unroll
        for (int i = 0; i < 2; ++i) {
            x[i].x = keep ? x[i].x : 0u; x[i].y = keep ? x[i].y : 0u;
            x[i].z = keep ? x[i].z : 0u; x[i].w = keep ? x[i].w : 0u;
        }
    }
    __device__ __forceinline__ float get(int e) const {
        const uint4& u = x[e >> 2];
        return __uint_as_float((e & 3) == 0 ? u.x : (e & 3) == 1 ? u.y : (e & 3) == 2 ? u.z : u.w);
    }
};

template <int V> struct IC { static constexpr int value = V; };

// Token tiles of Y computed by the wave of half hf: {0, 3} and {1, 2}, which
// balances the triangular products A_rk V and A_rb SA between the two halves.
__host__ __device__ constexpr int ytile(int hf, int u) { return hf ? 1 + u : 3 * u; }

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool MASK, bool KK>
__global__ __launch_bounds__(NTHR)
void chunked_kernel(ChunkArgs g) {
    constexpr bool VSPLIT = sizeof(Tin) == 4;   // fp32 v is not exact in bf16
    constexpr uint32_t SI = sizeof(Tin), SY = sizeof(Ty);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, known wave-uniform
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
    const int strip = w & 3, hf = w >> 2;      // value rows [16 strip, 16 strip + 16); half of the work
    const int H = g.H, T = g.T;
    const int bh = blockIdx.x;
    const int bb = bh / H, h = bh - bb * H;
    const int hk = h / (H / g.H_kv);
    // Bytes per token of the [B, T, H(_kv), D] tensors, and the first token of this sequence.
    const uint32_t stq = uint32_t(H) * DH * SI, stkv = uint32_t(g.H_kv) * DH * SI, sty = uint32_t(H) * DH * SY;
    const int64_t tok0 = int64_t(bb) * T;
    const char* rp = static_cast<const char*>(g.r);
    const char* wp = static_cast<const char*>(g.w);
    const char* kp = static_cast<const char*>(g.k);
    const char* vp = static_cast<const char*>(g.v);
    const char* ap = static_cast<const char*>(g.a);
    const char* bp = static_cast<const char*>(g.b);
    char* yp = static_cast<char*>(g.y);

    // This wave's half of its strip's state, transposed:
    // ST[u][r] = S[i = 16 strip + lr][j = 16 (2 hf + u) + 4 lq + r].
    f32x4 ST[2];
    const int i_row = 16 * strip + lr;
    const int64_t sbase = int64_t(bh) * DH * DH + int64_t(i_row) * DH;
    #pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int jt = 2 * hf + u;
        if (g.s0) {
            const float4 x = *reinterpret_cast<const float4*>(g.s0 + sbase + 16 * jt + 4 * lq);
            ST[u] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            ST[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // Column threads (P1a): key column jc = l, tokens [8 w, 8 w + 8).
    // Row threads (P1b): token tr = tid / 8, key columns [8 qr, 8 qr + 8).
    const int jc = l, pc = w;
    const int tr = tid >> 3, qr = tid & 7;
    // The epilogue's r_k row goes to LDS (read where used: in registers for the
    // whole kernel it would push the fp32-input variants past the register file).
    if constexpr (EPI) {
        if (tid < DH) reinterpret_cast<float*>(smem + OFF_RK)[tid] = g.r_k[h * DH + tid];
    }
    // Chunk-relative byte offsets (the descriptors move with the chunk), kept as
    // per-lane values in VGPRs: the column threads' 8 tokens (fp32 inputs, whose
    // rows take twice the registers, keep the first and add the token stride at
    // each load), the row threads' token, and the first of each 4-token group of
    // a lane's y elements (the others added where stored).
    constexpr int NCO = VSPLIT ? 1 : 8;
    uint32_t col_q[NCO], col_kv[NCO], y_off[2];
    #pragma unroll
    for (int e = 0; e < NCO; ++e) {
        col_q[e] = uint32_t(8 * pc + e) * stq + uint32_t(h * DH + jc) * SI;
        col_kv[e] = uint32_t(8 * pc + e) * stkv + uint32_t(hk * DH + jc) * SI;
        asm volatile("" : "+v"(col_q[e]));
        asm volatile("" : "+v"(col_kv[e]));
    }
    #pragma unroll
    for (int u = 0; u < 2; ++u) {
        y_off[u] = uint32_t(16 * ytile(hf, u) + 4 * lq) * sty + uint32_t(h * DH + i_row) * SY;
        asm volatile("" : "+v"(y_off[u]));
    }
    const uint32_t row_q = uint32_t(tr) * stq + uint32_t(h * DH + 8 * qr) * SI;
    const uint32_t row_kv = uint32_t(tr) * stkv + uint32_t(hk * DH + 8 * qr) * SI;

    uint32_t cw[8], cb[8], ck[8], cv[8];
    // Row loads; KK: rb holds the decay input row w (b is not read).
    Row8<Tin> rr, ra, rb, rkv;
    // Mask bytes (1 without a mask): lane l of a column wave holds token 8 pc + (l & 7)'s,
    // a row thread its token's.  Masked tokens become identity tokens (zeros, decay 1).
    const char* mp = reinterpret_cast<const char*>(g.mask);
    uint32_t cm = 1u, rm = 1u;
    // Columns of a chunk (for its P1a) and rows (for its P1b) load separately.
    auto chunk_rsrc = [&](int c0, const char* base, uint32_t stride) {
        const int nv = max(0, min(T - c0, L));   // valid tokens (0 past the end: every load reads zero)
        const int64_t t0 = nv > 0 ? tok0 + c0 : 0;
        return make_rsrc(base + t0 * stride, uint32_t(nv) * stride);
    };
    auto load_cols = [&](int c0) {
        // KK: the b slot of the column loads carries alpha (the a input); b is not read.
        const rsrc_t Rw = chunk_rsrc(c0, wp, stq), Rb = chunk_rsrc(c0, KK ? ap : bp, stq);
        const rsrc_t Rk = chunk_rsrc(c0, kp, stkv), Rv = chunk_rsrc(c0, vp, stkv);
        if constexpr (MASK) cm = __builtin_amdgcn_raw_buffer_load_b8(chunk_rsrc(c0, mp, 1u), uint32_t(8 * pc + (l & 7)), 0, 0);
        uint32_t oq[8], okv[8];
        if constexpr (VSPLIT) {
            uint32_t q0 = col_q[0], kv0 = col_kv[0];
            asm volatile("" : "+v"(q0), "+v"(kv0));   // formed here, not kept per token
            #pragma unroll
            for (int e = 0; e < 8; ++e) {
                oq[e] = q0 + uint32_t(e) * stq;
                okv[e] = kv0 + uint32_t(e) * stkv;
            }
        } else {
            #pragma unroll
            for (int e = 0; e < 8; ++e) {
                oq[e] = col_q[e];
                okv[e] = col_kv[e];
            }
        }
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
            cw[e] = Buf<Tin>::load1(Rw, oq[e]);
            cb[e] = Buf<Tin>::load1(Rb, oq[e]);
            ck[e] = Buf<Tin>::load1(Rk, okv[e]);
            cv[e] = Buf<Tin>::load1(Rv, okv[e]);
        }
    };
    auto load_rows = [&](int c0) {
        rr.load(chunk_rsrc(c0, rp, stq), row_q);
        ra.load(chunk_rsrc(c0, ap, stq), row_q);
        rb.load(chunk_rsrc(c0, KK ? wp : bp, stq), row_q);
        rkv.load(chunk_rsrc(c0, kp, stkv), row_kv);
        if constexpr (MASK) rm = __builtin_amdgcn_raw_buffer_load_b8(chunk_rsrc(c0, mp, 1u), uint32_t(tr), 0, 0);
    };
    load_cols(0);
    load_rows(0);

    // Lane offset of the 32-deep operand pattern inside a 64 x 64 bf16 matrix:
    // row lr, k = 8 lq .. 8 lq + 7.
    const int op32 = (lr * P72 + 8 * lq) * 2;
    // 16-deep operand of 16-block jb on a pair-interleaved axis: row lr, 4 elements.
    auto op_single = [&](int row0, int jb) { return ((row0 + lr) * P72 + 32 * (jb >> 1) + 8 * lq + 4 * (jb & 1)) * 2; };
    const int xs_own = ((strip * 2 + hf) * 2 * 64 + l) * 16;
    const int xs_oth = ((strip * 2 + (1 - hf)) * 2 * 64 + l) * 16;

    // ---------------- P1a: decay prefix down each key column ----------------
    // Runs one chunk ahead: the prefix of chunk c + 1 during P5 of chunk c, its
    // tables after the barrier that follows P5.  Decay mode: running products of
    // w, 2^-g as a reciprocal; log-decay mode: running sums of log2 w =
    // -exp(x) log2(e), then exp2.  The outputs that P6 / P7 of chunk c still read
    // from LDS (Kh^T, V^T, Bh^T, 2^g_L) stay in registers (d_*) until chunk c + 1
    // begins.
    float pre[8];
    uint32_t d_bh4[4], d_khh[4], d_khl[4], d_vh[4], d_vl[4];
    float d_bhf[KK ? 8 : 1];   // KK: Bh^T column values before their 1 / n
    float d_EL = 0.f;
    auto p1a_prefix = [&](int c0) {
        float run = LOGW ? 0.f : 1.f;
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = __uint_as_float(cw[e]);
            // Wave-uniform; w = 1 past the end and for masked tokens, whose b and k are zeroed.
            const bool ok = c0 + 8 * pc + e < T && (!MASK || __builtin_amdgcn_readlane(int(cm), e) != 0);
            float dec;   // this token's decay (KK: the k (1 - decay + alpha) factor)
            if constexpr (LOGW) {
                const float lw = -__builtin_amdgcn_exp2f(x * kLog2e) * kLog2e;
                run += ok ? lw : 0.f;
                dec = KK ? __builtin_amdgcn_exp2f(lw) : 0.f;
            } else {
                run *= ok ? x : 1.f;
                dec = x;
            }
            if constexpr (MASK) {
                cb[e] = ok ? cb[e] : 0u;
                ck[e] = ok ? ck[e] : 0u;
            }
            pre[e] = run;
            if constexpr (KK) {
                // b without its 1 / n (applied to Bh^T after the row phase), k' = k (1 - decay + alpha).
                const float kv = __uint_as_float(ck[e]), al = __uint_as_float(cb[e]);
                cb[e] = __float_as_uint(kv * al);
                ck[e] = __float_as_uint(kv * (1.f - dec + al));
            }
        }
        sts<float>(smem + OFF_TOT, (pc * 64 + jc) * 4, run);
    };
    auto p1a_tables = [&]() {
        float off = LOGW ? 0.f : 1.f, total = off;
        #pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const float tp = lds<float>(smem + OFF_TOT, (pp * 64 + jc) * 4);
            if constexpr (LOGW) {
                off += pp < pc ? tp : 0.f;
                total += tp;
            } else {
                off *= pp < pc ? tp : 1.f;
                total *= tp;
            }
        }
        const float EL = LOGW ? __builtin_amdgcn_exp2f(total) : total;
        d_EL = EL;
        #pragma unroll
        for (int e = 0; e < 8; e += 2) {
            float Eh[2];
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                float E, Ei;
                if constexpr (LOGW) {
                    const float gv = pre[e + u] + off;
                    E = __builtin_amdgcn_exp2f(gv);
                    Ei = __builtin_amdgcn_exp2f(-gv);
                } else {
                    E = pre[e + u] * off;
                    Ei = __builtin_amdgcn_rcpf(E);
                }
                sts<float>(smem + OFF_E, ((8 * pc + e + u) * PE + jc) * 4, E);
                sts<float>(smem + OFF_EI, ((8 * pc + e + u) * PE + jc) * 4, Ei);
                Eh[u] = EL * Ei;
            }
            const float b0 = __uint_as_float(cb[e]), b1 = __uint_as_float(cb[e + 1]);
            const float k0 = __uint_as_float(ck[e]), k1 = __uint_as_float(ck[e + 1]);
            if constexpr (KK) {
                d_bhf[e] = b0 * Eh[0];
                d_bhf[e + 1] = b1 * Eh[1];
            } else {
                d_bh4[e / 2] = pack_bf16(b0 * Eh[0], b1 * Eh[1]);
            }
            split2(k0 * Eh[0], k1 * Eh[1], d_khh[e / 2], d_khl[e / 2]);
            if constexpr (VSPLIT) {
                split2(__uint_as_float(cv[e]), __uint_as_float(cv[e + 1]), d_vh[e / 2], d_vl[e / 2]);
            } else {
                d_vh[e / 2] = (cv[e] >> 16) | (cv[e + 1] & 0xffff0000u);   // bf16 bits as they are
            }
        }
    };
    auto p1a_store = [&]() {
        if (pc == 0) sts<float>(smem + OFF_EL, jc * 4, d_EL);
        const int o = (jc * P72 + 8 * pc) * 2;
        sts<uint4>(smem + OFF_KHTH, o, make_uint4(d_khh[0], d_khh[1], d_khh[2], d_khh[3]));
        sts<uint4>(smem + OFF_KHTL, o, make_uint4(d_khl[0], d_khl[1], d_khl[2], d_khl[3]));
        sts<uint4>(smem + OFF_VT, o, make_uint4(d_vh[0], d_vh[1], d_vh[2], d_vh[3]));
        if constexpr (VSPLIT) sts<uint4>(smem + OFF_VTL, o, make_uint4(d_vl[0], d_vl[1], d_vl[2], d_vl[3]));
        // Bh^T on the pair-interleaved token axis: tokens 8 pc + (0..3) and 8 pc + (4..7).
        const int ob = (jc * P72 + pairpos(8 * pc)) * 2;
        if constexpr (!KK) {
            sts<uint2>(smem + OFF_BHT, ob, make_uint2(d_bh4[0], d_bh4[1]));
            sts<uint2>(smem + OFF_BHT, ob + 16, make_uint2(d_bh4[2], d_bh4[3]));
        }
    };
    // KK: Bh^T of the chunk once its row phase has published 1 / n per token.
    auto store_bh_kk = [&]() {
        const float4 n0 = lds<float4>(smem + OFF_INVN, 32 * pc), n1 = lds<float4>(smem + OFF_INVN, 32 * pc + 16);
        const float invn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
        uint32_t bh4[4];
        #pragma unroll
        for (int e = 0; e < 8; e += 2) bh4[e / 2] = pack_bf16(d_bhf[e] * invn[e], d_bhf[e + 1] * invn[e + 1]);
        const int ob = (jc * P72 + pairpos(8 * pc)) * 2;
        sts<uint2>(smem + OFF_BHT, ob, make_uint2(bh4[0], bh4[1]));
        sts<uint2>(smem + OFF_BHT, ob + 16, make_uint2(bh4[2], bh4[3]));
    };
    p1a_prefix(0);
    __syncthreads();
    p1a_tables();
    __syncthreads();

    const int nchunks = (T + L - 1) / L;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = ch * L;
        // Own state half as the B operand of the key pair hf (hi / lo); published for the partner.
        bf16x8 SoH, SoL;
        {
            s16x4 h0, l0, h1, l1;
            to_operand(ST[0], h0, l0);
            to_operand(ST[1], h1, l1);
            SoH = cat(h0, h1);
            SoL = cat(l0, l1);
            sts<bf16x8>(smem + OFF_XS, xs_own, SoH);
            sts<bf16x8>(smem + OFF_XS, xs_own + 64 * 16, SoL);
        }
        p1a_store();

        // ---------------- P1b: row-major scaled operands ----------------
        if constexpr (MASK) {
            const bool keep = rm != 0;
            rr.keep_if(keep); ra.keep_if(keep); rb.keep_if(keep); rkv.keep_if(keep);
        }
        {
            float E[8], Ei[8], Ep[8];
            const int oe = (tr * PE + 8 * qr) * 4;
            const float4 e0 = lds<float4>(smem + OFF_E, oe), e1 = lds<float4>(smem + OFF_E, oe + 16);
            const float4 i0 = lds<float4>(smem + OFF_EI, oe), i1 = lds<float4>(smem + OFF_EI, oe + 16);
            E[0] = e0.x; E[1] = e0.y; E[2] = e0.z; E[3] = e0.w; E[4] = e1.x; E[5] = e1.y; E[6] = e1.z; E[7] = e1.w;
            Ei[0] = i0.x; Ei[1] = i0.y; Ei[2] = i0.z; Ei[3] = i0.w; Ei[4] = i1.x; Ei[5] = i1.y; Ei[6] = i1.z; Ei[7] = i1.w;
            if (tr > 0) {
                const float4 p0 = lds<float4>(smem + OFF_E, oe - PE * 4), p1 = lds<float4>(smem + OFF_E, oe - PE * 4 + 16);
                Ep[0] = p0.x; Ep[1] = p0.y; Ep[2] = p0.z; Ep[3] = p0.w; Ep[4] = p1.x; Ep[5] = p1.y; Ep[6] = p1.z; Ep[7] = p1.w;
            } else {
                #pragma unroll
                for (int e = 0; e < 8; ++e) Ep[e] = 1.f;
            }
            uint32_t at[4], rth[4], rtl[4], bt[4], kth[4], ktl[4];
            float bonus_part = 0.f;
            float rk8[8];
            if constexpr (EPI) {
                const float4 q0 = lds<float4>(smem + OFF_RK, 32 * qr), q1 = lds<float4>(smem + OFF_RK, 32 * qr + 16);
                rk8[0] = q0.x; rk8[1] = q0.y; rk8[2] = q0.z; rk8[3] = q0.w;
                rk8[4] = q1.x; rk8[5] = q1.y; rk8[6] = q1.z; rk8[7] = q1.w;
            }
            // KK: 1 / n of this token from its 64 keys, held by the 8 row threads of the
            // token (lanes 8 m .. 8 m + 7 of one wave); published for the column threads.
            float invn = 0.f;
            if constexpr (KK) {
                float ss = 0.f;
                #pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(rkv.get(e), rkv.get(e), ss);
                ss += dpp<kDppQuadXor1>(ss);
                ss += dpp<kDppQuadXor2>(ss);
                ss += dpp<kDppRowHalfMirror>(ss);
                invn = inv_key_norm(ss);
                if (qr == 0) sts<float>(smem + OFF_INVN, tr * 4, invn);
            }
            #pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float r0 = rr.get(e), r1 = rr.get(e + 1);
                float a0, a1, b0, b1, k0, k1;
                if constexpr (KK) {
                    // a = -k / n, b = k alpha / n, k' = k (1 - decay + alpha); ra holds alpha, rb the w row.
                    const float kr0 = rkv.get(e), kr1 = rkv.get(e + 1);
                    const float al0 = ra.get(e), al1 = ra.get(e + 1);
                    const float d0 = LOGW ? decay_from_logneglog(rb.get(e)) : rb.get(e);
                    const float d1 = LOGW ? decay_from_logneglog(rb.get(e + 1)) : rb.get(e + 1);
                    a0 = -kr0 * invn; a1 = -kr1 * invn;
                    b0 = kr0 * al0 * invn; b1 = kr1 * al1 * invn;
                    k0 = kr0 * (1.f - d0 + al0); k1 = kr1 * (1.f - d1 + al1);
                } else {
                    a0 = ra.get(e); a1 = ra.get(e + 1);
                    b0 = rb.get(e); b1 = rb.get(e + 1);
                    k0 = rkv.get(e); k1 = rkv.get(e + 1);
                }
                at[e / 2] = pack_bf16(a0 * Ep[e], a1 * Ep[e + 1]);
                split2(r0 * E[e], r1 * E[e + 1], rth[e / 2], rtl[e / 2]);
                bt[e / 2] = pack_bf16(b0 * Ei[e], b1 * Ei[e + 1]);
                split2(k0 * Ei[e], k1 * Ei[e + 1], kth[e / 2], ktl[e / 2]);
                if constexpr (EPI) bonus_part += r0 * k0 * rk8[e] + r1 * k1 * rk8[e + 1];
            }
            // Pair-interleaved key axis: columns 8 qr + (0..3) and 8 qr + (4..7).
            const int o = (tr * P72 + pairpos(8 * qr)) * 2;
            sts<uint2>(smem + OFF_AT, o, make_uint2(at[0], at[1]));
            sts<uint2>(smem + OFF_AT, o + 16, make_uint2(at[2], at[3]));
            sts<uint2>(smem + OFF_RTH, o, make_uint2(rth[0], rth[1]));
            sts<uint2>(smem + OFF_RTH, o + 16, make_uint2(rth[2], rth[3]));
            sts<uint2>(smem + OFF_RTL, o, make_uint2(rtl[0], rtl[1]));
            sts<uint2>(smem + OFF_RTL, o + 16, make_uint2(rtl[2], rtl[3]));
            sts<uint2>(smem + OFF_BT, o, make_uint2(bt[0], bt[1]));
            sts<uint2>(smem + OFF_BT, o + 16, make_uint2(bt[2], bt[3]));
            sts<uint2>(smem + OFF_KTH, o, make_uint2(kth[0], kth[1]));
            sts<uint2>(smem + OFF_KTH, o + 16, make_uint2(kth[2], kth[3]));
            sts<uint2>(smem + OFF_KTL, o, make_uint2(ktl[0], ktl[1]));
            sts<uint2>(smem + OFF_KTL, o + 16, make_uint2(ktl[2], ktl[3]));
            if constexpr (EPI) {
                // The eight threads of a token row are lanes 8m .. 8m + 7 of one wave.
                bonus_part += dpp<kDppQuadXor1>(bonus_part);
                bonus_part += dpp<kDppQuadXor2>(bonus_part);
                bonus_part += dpp<kDppRowHalfMirror>(bonus_part);
                if (qr == 0) sts<float>(smem + OFF_BONUS, tr * 4, bonus_part);
            }
        }
        load_rows(c0 + L);   // next chunk's rows, for its P1b
        __syncthreads();
        if constexpr (KK) store_bh_kk();   // read in P7, after the barriers to come

        // ---------------- P2: the four L x L matrices; inverses of the diagonal blocks ----------------
        // Tile ids 0..9 list (tb, sb), sb <= tb, in row order.  Waves 0..3 take the
        // off-diagonal tiles {1, 3}, {4, 6}, {7}, {8} (all four matrices, sharing the
        // B~ / K~ reads) and A_ak, A_rb, A_rk of diagonal tile (strip, strip); waves
        // 4..7 take only A_ab of that diagonal tile, whose block inverse is the serial
        // part of this phase.  Each tile is C'[s][t] = Y[s] . X[t], so a lane holds 4
        // consecutive s of one t: a row-major [t][s] store of 4 elements.
        auto tile_tb = [](int id) { return id >= 6 ? 3 : id >= 3 ? 2 : id >= 1 ? 1 : 0; };
        auto tile_id = [&](int n) {
            return hf ? (n == 0 ? strip * (strip + 3) / 2 : -1)
                      : (n == 0 ? min(1 + 3 * strip, 8) : (strip < 2 ? 3 + 3 * strip : -1));
        };
        f32x4 Aab[3], Aak[3], Arb[3], Ark[3];
        f32x4 Nsw = {0.f, 0.f, 0.f, 0.f};   // diagonal block N of A_ab in C layout (waves 4..7)
        #pragma unroll
        for (int n = 0; n < 3; ++n) Aab[n] = Aak[n] = Arb[n] = Ark[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto tile_products = [&](int n, int tb, int sb, bool ab, bool rest, bool swapped) {
            #pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                const int ya = (16 * sb * P72 + 32 * kq) * 2 + op32;
                const int xb = (16 * tb * P72 + 32 * kq) * 2 + op32;
                const bf16x8 Bt8 = lds<bf16x8>(smem + OFF_BT, ya);
                const bf16x8 At8 = lds<bf16x8>(smem + OFF_AT, xb);
                if (ab) Aab[n] = mfma32(Bt8, At8, Aab[n]);
                if (swapped) Nsw = mfma32(At8, Bt8, Nsw);   // same block, operands swapped
                if (rest) {
                    const bf16x8 Kh8 = lds<bf16x8>(smem + OFF_KTH, ya);
                    const bf16x8 Kl8 = lds<bf16x8>(smem + OFF_KTL, ya);
                    const bf16x8 Rh8 = lds<bf16x8>(smem + OFF_RTH, xb);
                    const bf16x8 Rl8 = lds<bf16x8>(smem + OFF_RTL, xb);
                    Aak[n] = mfma32(Kh8, At8, Aak[n]);
                    Aak[n] = mfma32(Kl8, At8, Aak[n]);
                    Arb[n] = mfma32(Bt8, Rh8, Arb[n]);
                    Arb[n] = mfma32(Bt8, Rl8, Arb[n]);
                    Ark[n] = mfma32(Kh8, Rh8, Ark[n]);
                    Ark[n] = mfma32(Kh8, Rl8, Ark[n]);
                    Ark[n] = mfma32(Kl8, Rh8, Ark[n]);
                }
            }
        };
        if (!hf) {
            #pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int id = tile_id(n);
                const int tb = tile_tb(id), sb = id - (tile_tb(id) * (tile_tb(id) + 1)) / 2;
                if (id >= 0) tile_products(n, tb, sb, true, true, false);
            }
            tile_products(2, strip, strip, false, true, false);
        } else {
            tile_products(0, strip, strip, true, false, true);
        }
        // Next chunk's columns (for its prefix after P4); waves 4..7 issue them ahead
        // of the inverse chain.
        load_cols(c0 + L);
        if (hf) {
            // N = block `strip` of A_ab is strictly lower triangular, so N^16 = 0 and
            // (I - N)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8); the factors are
            // polynomials in N and commute.  A C-layout tile of M is the B operand of M
            // and the A operand of M^T, so the products use tiles of both orientations:
            // Aab[0] is C(N^T) (lane: t = lr, s = 4 lq + r), Nsw is C(N) (s = lr, t = 4 lq + r).
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const s16x4 z4 = {0, 0, 0, 0};
            // prod(C(X^T), C(Y)) = C(X Y), operands split hi + lo: [xh, xl].[yh, yh] + [xh, 0].[yl, 0].
            auto prod = [&](const f32x4 xt, const f32x4 y) {
                s16x4 xh, xl, yh, yl;
                to_operand(xt, xh, xl);
                to_operand(y, yh, yl);
                const f32x4 c = mfma32(cat(xh, xl), cat(yh, yh), zero);
                return mfma32(cat(xh, z4), cat(yl, z4), c);
            };
            f32x4 Nn, Nt, I4;
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                Nt[r] = 4 * lq + r >= lr ? 0.f : Aab[0][r];
                Nn[r] = lr >= 4 * lq + r ? 0.f : Nsw[r];
                I4[r] = (4 * lq + r == lr) ? 1.f : 0.f;
            }
            const f32x4 N2 = prod(Nt, Nn), N2t = prod(Nn, Nt);
            const f32x4 N4 = prod(N2t, N2), N4t = prod(N2, N2t);
            const f32x4 N8 = prod(N4t, N4);
            const f32x4 Gt = prod(N2 + I4, Nt + I4);       // C((F1 F2)^T) = C(F2^T F1^T)
            const f32x4 G4t = prod(N4 + I4, Gt);           // C(F4^T F2^T F1^T)
            const f32x4 Dt = prod(N8 + I4, G4t);           // C(D^T): lane holds D[lr][4 lq + r]
            sts<uint2>(smem + OFF_DINV, ((strip * 16 + lr) * PD + 4 * lq) * 2,
                       make_uint2(pack_bf16(Dt[0], Dt[1]), pack_bf16(Dt[2], Dt[3])));
        }
        __syncthreads();   // B~ / K~ (region 1) and the decay tables (region 2) are dead now
        // Row-major [t][s] stores of one tile: A_ab / A_rb bf16 on the pair-interleaved
        // token axis, A_ak / A_rk hi / lo in natural order.
        auto store_ab = [&](int tb, int sb, char* dst, f32x4 c) {
            sts<uint2>(dst, ((16 * tb + lr) * P72 + pairpos(16 * sb + 4 * lq)) * 2,
                       make_uint2(pack_bf16(c[0], c[1]), pack_bf16(c[2], c[3])));
        };
        auto store_hl = [&](int tb, int sb, int off_h, int off_l, f32x4 c) {
            uint32_t h0, l0, h1, l1;
            split2(c[0], c[1], h0, l0);
            split2(c[2], c[3], h1, l1);
            const int o = ((16 * tb + lr) * P72 + 16 * sb + 4 * lq) * 2;
            sts<uint2>(smem + off_h, o, make_uint2(h0, h1));
            sts<uint2>(smem + off_l, o, make_uint2(l0, l1));
        };
        // Diagonal tiles: A_ab, A_ak strictly lower (s < t); A_rb, A_rk lower with diagonal (s <= t).
        auto mask = [&](f32x4 c, bool strict) {
            #pragma unroll
            for (int r = 0; r < 4; ++r) c[r] = 4 * lq + r >= lr + (strict ? 0 : 1) ? 0.f : c[r];
            return c;
        };
        if (!hf) {
            #pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int id = tile_id(n);
                if (id >= 0) {   // off-diagonal
                    const int tb = tile_tb(id), sb = id - (tile_tb(id) * (tile_tb(id) + 1)) / 2;
                    store_ab(tb, sb, smem + OFF_AAB, Aab[n]);
                    store_ab(tb, sb, smem + OFF_ARB, Arb[n]);
                    store_hl(tb, sb, OFF_AKH, OFF_AKL, Aak[n]);
                    store_hl(tb, sb, OFF_RKH, OFF_RKL, Ark[n]);
                }
            }
            store_ab(strip, strip, smem + OFF_ARB, mask(Arb[2], false));
            store_hl(strip, strip, OFF_AKH, OFF_AKL, mask(Aak[2], true));
            store_hl(strip, strip, OFF_RKH, OFF_RKL, mask(Ark[2], false));
        } else {
            store_ab(strip, strip, smem + OFF_AAB, mask(Aab[0], true));
        }
        if (tid < 256) {
            // Zero the upper tiles (t-block 0, s-block 1) and (2, 3) of A_ak and A_rk,
            // which the 32-deep products of P4 read.
            const int mat = tid >> 6, m = (tid >> 5) & 1, rw = (tid & 31) >> 1, half = tid & 1;
            const int base = mat == 0 ? OFF_AKH : mat == 1 ? OFF_AKL : mat == 2 ? OFF_RKH : OFF_RKL;
            const int tb = m ? 2 : 0, sb = tb + 1;
            sts<uint4>(smem + base, ((16 * tb + rw) * P72 + 16 * sb + 8 * half) * 2, make_uint4(0, 0, 0, 0));
        }
        __syncthreads();   // everything P4..P7 read from LDS is in place

        // ---------------- P4: RHS = At S0^T + A_ak V (whole strip), Y's SA-free part ----------------
        // State operands: key pair hf from this wave's registers (own), pair 1 - hf from the partner.
        const bf16x8 SxH = lds<bf16x8>(smem + OFF_XS, xs_oth);
        const bf16x8 SxL = lds<bf16x8>(smem + OFF_XS, xs_oth + 64 * 16);
        const int po = 32 * hf, px = 32 * (1 - hf);   // column of the own / other key pair
        // V^T as 32-deep B operands (k = token s = 32 kq + 8 lq + e, n = value row).
        bf16x8 VB[2], VBl[2];
        #pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            VB[kq] = lds<bf16x8>(smem + OFF_VT, (16 * strip * P72 + 32 * kq) * 2 + op32);
            if constexpr (VSPLIT) VBl[kq] = lds<bf16x8>(smem + OFF_VTL, (16 * strip * P72 + 32 * kq) * 2 + op32);
        }
        f32x4 RHS[4];
        #pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ro = (16 * tb * P72) * 2 + op32;
            const bf16x8 Ao = lds<bf16x8>(smem + OFF_AT, ro + po * 2);
            const bf16x8 Ax = lds<bf16x8>(smem + OFF_AT, ro + px * 2);
            acc = mfma32(Ao, SoH, acc);
            acc = mfma32(Ao, SoL, acc);
            acc = mfma32(Ax, SxH, acc);
            acc = mfma32(Ax, SxL, acc);
            #pragma unroll
            for (int kq = 0; kq <= tb / 2; ++kq) {
                const int o = (16 * tb * P72 + 32 * kq) * 2 + op32;
                const bf16x8 Ah8 = lds<bf16x8>(smem + OFF_AKH, o);
                acc = mfma32(Ah8, VB[kq], acc);
                acc = mfma32(lds<bf16x8>(smem + OFF_AKL, o), VB[kq], acc);
                if constexpr (VSPLIT) acc = mfma32(Ah8, VBl[kq], acc);
            }
            RHS[tb] = acc;
        }

        f32x4 Yacc[2];
        #pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tb = ytile(hf, u);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ro = (16 * tb * P72) * 2 + op32;
            const bf16x8 Rho = lds<bf16x8>(smem + OFF_RTH, ro + po * 2);
            const bf16x8 Rlo = lds<bf16x8>(smem + OFF_RTL, ro + po * 2);
            const bf16x8 Rhx = lds<bf16x8>(smem + OFF_RTH, ro + px * 2);
            const bf16x8 Rlx = lds<bf16x8>(smem + OFF_RTL, ro + px * 2);
            acc = mfma32(Rho, SoH, acc);
            acc = mfma32(Rho, SoL, acc);
            acc = mfma32(Rlo, SoH, acc);
            acc = mfma32(Rhx, SxH, acc);
            acc = mfma32(Rhx, SxL, acc);
            acc = mfma32(Rlx, SxH, acc);
            #pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                if (kq <= tb / 2) {
                    const int o = (16 * tb * P72 + 32 * kq) * 2 + op32;
                    const bf16x8 Rh8 = lds<bf16x8>(smem + OFF_RKH, o);
                    acc = mfma32(Rh8, VB[kq], acc);
                    acc = mfma32(lds<bf16x8>(smem + OFF_RKL, o), VB[kq], acc);
                    if constexpr (VSPLIT) acc = mfma32(Rh8, VBl[kq], acc);
                }
            }
            Yacc[u] = acc;
        }

        p1a_prefix(c0 + L);

        // ---------------- P5: SA = (I - A_ab)^-1 RHS, blocked forward substitution ----------------
        s16x4 SAh[4], SAl[4];
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            f32x4 x = RHS[ib];
            if (ib >= 2) {   // 16-blocks 0 and 1 as one pair
                const bf16x8 A8 = lds<bf16x8>(smem + OFF_AAB, (16 * ib * P72) * 2 + op32);
                x = mfma32(A8, cat(SAh[0], SAh[1]), x);
                x = mfma32(A8, cat(SAl[0], SAl[1]), x);
            }
            if (ib == 1 || ib == 3) {   // the remaining single 16-block ib - 1
                const s16x4 A4 = lds<s16x4>(smem + OFF_AAB, op_single(16 * ib, ib - 1));
                x = mfma32(cat(A4, A4), cat(SAh[ib - 1], SAl[ib - 1]), x);
            }
            s16x4 xh, xl;
            to_operand(x, xh, xl);
            const s16x4 D4 = lds<s16x4>(smem + OFF_DINV, ((16 * ib + lr) * PD + 4 * lq) * 2);
            const f32x4 sa = mfma32(cat(D4, D4), cat(xh, xl), f32x4{0.f, 0.f, 0.f, 0.f});
            to_operand(sa, SAh[ib], SAl[ib]);
        }
        const bf16x8 SPh[2] = {cat(SAh[0], SAh[1]), cat(SAh[2], SAh[3])};
        const bf16x8 SPl[2] = {cat(SAl[0], SAl[1]), cat(SAl[2], SAl[3])};

        __syncthreads();   // next chunk's column totals visible; every wave is past P4 (region 2 free)
        p1a_tables();

        // ---------------- P6: Y += A_rb SA on token tiles ytile(hf, 0..1); epilogue; store ----------------
        {
            const int nv = max(0, min(T - c0, L));
            const rsrc_t Ry = make_rsrc(yp + (tok0 + c0) * sty, uint32_t(nv) * sty);
            auto p6 = [&](auto HFC) {
                constexpr int HF = decltype(HFC)::value;
                #pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int tb = ytile(HF, u);
                    f32x4 acc = Yacc[u];
                    #pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        if (2 * p + 1 <= tb) {
                            const bf16x8 A8 = lds<bf16x8>(smem + OFF_ARB, (16 * tb * P72 + 32 * p) * 2 + op32);
                            acc = mfma32(A8, SPh[p], acc);
                            acc = mfma32(A8, SPl[p], acc);
                        }
                    }
                    if ((tb & 1) == 0) {   // diagonal block tb, not covered by a pair
                        const s16x4 A4 = lds<s16x4>(smem + OFF_ARB, op_single(16 * tb, tb));
                        acc = mfma32(cat(A4, A4), cat(SAh[tb], SAl[tb]), acc);
                    }
                    // acc[r] = Y[t = 16 tb + 4 lq + r][i_row]
                    const int tl0 = 16 * tb + 4 * lq;
                    float vtr[4] = {0.f, 0.f, 0.f, 0.f}, bon[4] = {0.f, 0.f, 0.f, 0.f};
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
                    uint32_t yo = y_off[u];
                    asm volatile("" : "+v"(yo));   // formed here, not kept per element for the whole loop
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float yv = acc[r] * g.y_scale;
                        if constexpr (EPI) yv = fmaf(bon[r], vtr[r], yv);
                        Buf<Ty>::store1(Ry, yo + uint32_t(r) * sty, yv);
                    }
                }
            };
            if (hf == 0) p6(IC<0>{}); else p6(IC<1>{});
        }

        // ---------------- P7: S_L^T = 2^g_L S0^T + Bh^T SA + Kh^T V, key tiles 2 hf, 2 hf + 1 ----------------
        #pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int jt = 2 * hf + u;
            const float4 el4 = lds<float4>(smem + OFF_EL, (16 * jt + 4 * lq) * 4);
            f32x4 acc = ST[u];
            acc[0] *= el4.x; acc[1] *= el4.y; acc[2] *= el4.z; acc[3] *= el4.w;
            #pragma unroll
            for (int p = 0; p < 2; ++p) {
                const bf16x8 B8 = lds<bf16x8>(smem + OFF_BHT, (16 * jt * P72 + 32 * p) * 2 + op32);
                acc = mfma32(B8, SPh[p], acc);
                acc = mfma32(B8, SPl[p], acc);
            }
            #pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                const int o = (16 * jt * P72 + 32 * kq) * 2 + op32;
                const bf16x8 Kh8 = lds<bf16x8>(smem + OFF_KHTH, o);
                acc = mfma32(Kh8, VB[kq], acc);
                acc = mfma32(lds<bf16x8>(smem + OFF_KHTL, o), VB[kq], acc);
                if constexpr (VSPLIT) acc = mfma32(Kh8, VBl[kq], acc);
            }
            ST[u] = acc;
        }
        __syncthreads();   // all LDS operands of this chunk consumed before P1 rewrites them
    }

    if (g.s1) {
        #pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<float4*>(g.s1 + sbase + 16 * (2 * hf + u) + 4 * lq) =
                make_float4(ST[u][0], ST[u][1], ST[u][2], ST[u][3]);
    }
}

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool MASK, bool KK>
hipError_t launch_t(const Params& p, hipStream_t stream) {
    ChunkArgs g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.mask, p.y, p.s1, p.T, p.H, p.H_kv, p.y_scale};
    auto kern = chunked_kernel<Tin, Ty, LOGW, EPI, MASK, KK>;
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

template <typename Tin, typename Ty, bool MASK, bool KK>
hipError_t dispatch_epi(const Params& p, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_t<Tin, Ty, true, true, MASK, KK>(p, s) : launch_t<Tin, Ty, true, false, MASK, KK>(p, s);
    return epi ? launch_t<Tin, Ty, false, true, MASK, KK>(p, s) : launch_t<Tin, Ty, false, false, MASK, KK>(p, s);
}

template <typename Tin, typename Ty, bool KK>
hipError_t dispatch_mask(const Params& p, hipStream_t s) {
    return p.mask ? dispatch_epi<Tin, Ty, true, KK>(p, s) : dispatch_epi<Tin, Ty, false, KK>(p, s);
}

template <typename Tin, typename Ty>
hipError_t dispatch_modes(const Params& p, hipStream_t s) {
    return p.ab_mode == WKV7_AB_FROM_K ? dispatch_mask<Tin, Ty, true>(p, s) : dispatch_mask<Tin, Ty, false>(p, s);
}

}  // namespace

hipError_t launch_chunked(const Params& p, hipStream_t stream) {
    if (p.D != DH || p.chunk_len != L) return hipErrorInvalidValue;
    // Byte offsets inside one chunk's descriptor are 32-bit.
    if (int64_t(L) * p.H * DH * 4 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<bf16_t, bf16_t>(p, stream) : dispatch_modes<bf16_t, float>(p, stream);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<float, bf16_t>(p, stream) : dispatch_modes<float, float>(p, stream);
}

}  // namespace wkv7
