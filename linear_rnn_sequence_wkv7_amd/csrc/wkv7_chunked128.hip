// Chunk-parallel WKV-7 forward for head size D = 128 on gfx950 bf16 matrix
// cores (fp32 accumulation).
//
// Same chunk algebra as the D = 64 kernel (unrolling S_t = S_{t-1}(diag(w_t) +
// a_t b_t^T) + v_t k_t^T over a chunk; wiki note "RWKV-7 Goose", generalised
// delta rule; the pages only say the operation parallelises over chunks,
// youngju.dev RWKV-7 article, Q&A 5), with g_t = sum_{s<=t} log2 w_s per key:
//
//   A_ab[t,s] = sum_j a_tj b_sj 2^(g_{t-1,j} - g_sj)   (s < t)    A_ak likewise with k
//   A_rb[t,s] = sum_j r_tj b_sj 2^(g_tj - g_sj)        (s <= t)   A_rk likewise with k
//   SA  = (I - A_ab)^-1 (At S0^T + A_ak V)        At_t = a_t 2^(g_{t-1})
//   Y   = Rt S0^T + A_rb SA + A_rk V              Rt_t = r_t 2^(g_t)
//   S_L = S0 diag(2^g_L) + SA^T Bh + V^T Kh       Bh_s = b_s 2^(g_L - g_s), Kh likewise
//
// Shape choices for D = 128: chunks of L = 32 tokens (the L x D operand
// matrices of a 64-token chunk would not fit in LDS), and four workgroups per
// (b, h), each owning 32 of the 128 value rows.  Rows of S evolve
// independently given the chunk's key-side matrices, so the four workgroups
// never communicate; each builds the state-independent matrices itself.  The
// four slices of one (b, h) get workgroup ids 8 apart, i.e. the same XCD under
// round-robin dispatch, so their reads of the same inputs meet in one L2.
//
// Inside a workgroup (8 waves): wave w keeps the state tiles of value strip
// w & 1 (16 rows) and key pair w >> 1 (32 keys) in registers, transposed
// (C layout of a 16x16 MFMA result = B operand of a 16-deep product); the
// pairs are published once per chunk through LDS, and every wave builds the
// full removal projection of its strip from them.  As in the D = 64 kernel,
// operands that decide the result are split into bf16 hi + lo parts, matrices
// multiplied against register operands are stored with the contraction axis
// pair-interleaved (position 32 p + 8 q + 4 e + r holds 16 (2 p + e) + 4 q + r),
// every accumulator chain uses the single 16x16x32 opcode, and global memory
// goes through per-chunk buffer descriptors (tokens past the end read as zero,
// their stores are dropped).
// Kernel vectors from k (KK) as in the D = 64 kernel: the a slot carries alpha,
// b is not read; the 16 row threads of a token form 1 / n, n = max(|k|, 1e-12),
// and publish it in LDS; the column threads form k' = k (1 - decay + alpha) and
// k alpha one chunk ahead and scale their Bh^T by 1 / n after the row phase
// (the hxa07D article's preparation before its kernel call, section 8).
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int L = 32;          // chunk length
constexpr int DK = 128;        // head size (keys and values)
constexpr int DV = 32;         // value rows per workgroup
constexpr int NSLICE = DK / DV;
constexpr int NTHR = 512;      // 8 waves
constexpr int PK = 136;        // bf16 pitch of [L][DK] token-major operands (272 B rows)
constexpr int PT = 40;         // bf16 pitch of [*][L] operands (80 B rows)
constexpr int MATK = L * PK * 2;
constexpr int MATT = DK * PT * 2;
constexpr int MATV = DV * PT * 2;   // [32][L]: V^T of the slice, and each L x L matrix
constexpr int PE = 132;        // fp32 pitch of the decay tables
constexpr int PD = 20;         // pitch of the 16 x 16 inverse blocks

// LDS map (bytes).  Region 1 holds B~, K~ during P1b..P2 and the six L x L
// matrices afterwards.  Key axis pair-interleaved: At, Rt, Bt, Kt; token axis
// pair-interleaved: A_ab, A_rb, Bh^T; natural: A_ak, A_rk, Kh^T, V^T.
constexpr int OFF_AT = 0;
constexpr int OFF_RTH = OFF_AT + MATK;
constexpr int OFF_RTL = OFF_RTH + MATK;
constexpr int OFF_R1 = OFF_RTL + MATK;
constexpr int OFF_BT = OFF_R1;
constexpr int OFF_KTH = OFF_R1 + MATK;
constexpr int OFF_KTL = OFF_R1 + 2 * MATK;
constexpr int OFF_AAB = OFF_R1;
constexpr int OFF_ARB = OFF_R1 + MATV;
constexpr int OFF_AKH = OFF_R1 + 2 * MATV;
constexpr int OFF_AKL = OFF_R1 + 3 * MATV;
constexpr int OFF_RKH = OFF_R1 + 4 * MATV;
constexpr int OFF_RKL = OFF_R1 + 5 * MATV;
constexpr int OFF_BHT = OFF_R1 + 3 * MATK;   // Bh^T [j][s]
constexpr int OFF_KHTH = OFF_BHT + MATT;     // Kh^T [j][s] hi / lo
constexpr int OFF_KHTL = OFF_KHTH + MATT;
constexpr int OFF_VT = OFF_KHTL + MATT;      // V^T [i][s], this slice's 32 value rows
constexpr int OFF_E = OFF_VT + MATV;         // fp32 [L][PE] 2^g
constexpr int OFF_EI = OFF_E + L * PE * 4;   // fp32 [L][PE] 2^-g
constexpr int OFF_TOT = OFF_EI + L * PE * 4; // fp32 [4][DK] column-segment totals
constexpr int OFF_DINV = OFF_TOT + 4 * DK * 4;      // bf16 [2][16][PD]
constexpr int OFF_EL = OFF_DINV + 2 * 16 * PD * 2;  // fp32 [DK] 2^g_L
constexpr int OFF_BONUS = OFF_EL + DK * 4;          // fp32 [L]
constexpr int OFF_XS = OFF_BONUS + L * 4;           // [strip][pair][hi/lo][lane] 16 B
constexpr int XS_BYTES = 2 * 4 * 2 * 64 * 16;
constexpr int OFF_INVN = OFF_XS + XS_BYTES;         // fp32 [L] 1 / max(|k_t|, 1e-12) of the chunk (KK)
constexpr int OFF_VTL = OFF_INVN + L * 4;           // V^T lo part (fp32 inputs only)
constexpr int SMEM_BF16 = OFF_VTL;
constexpr int SMEM_F32 = OFF_VTL + MATV;
static_assert(6 * MATV <= 3 * MATK, "L x L matrices fit region 1");
static_assert(SMEM_F32 <= 160 * 1024, "LDS budget");
static_assert(OFF_E % 16 == 0 && OFF_XS % 16 == 0 && OFF_VTL % 16 == 0, "alignment");

__host__ __device__ constexpr int pairpos(int k) {
    return 32 * (k >> 5) + 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3);
}

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
__device__ __forceinline__ void split2(float x, float y, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(x, y);
    lo = pack_bf16(x - lo_f32(hi), y - hi_f32(hi));
}
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

// Raw buffer descriptor over [base, base + bytes) (32-bit data format word of
// the gfx9 family); the arguments are wave-uniform and read through
// readfirstlane so that the descriptor stays in SGPRs.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;   // above every descriptor size used here
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, int(n), kRsrcWord3);
}

template <typename T> struct Buf;
template <> struct Buf<bf16_t> {
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

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool MASK, bool KK>
__global__ __launch_bounds__(NTHR)
void chunked128_kernel(Args g) {
    constexpr bool VSPLIT = sizeof(Tin) == 4;
    constexpr uint32_t SI = sizeof(Tin), SY = sizeof(Ty);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // Workgroup -> (b, h, value slice q); the 4 slices of a (b, h) are 8 ids apart.
    const int gid = blockIdx.x;
    const int q = (gid >> 3) & (NSLICE - 1);
    const int bh = (gid & 7) + 8 * (gid >> 5);
    if (bh >= g.BH) return;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
    const int sg = w & 1, kp = w >> 1;          // value strip of the slice, key pair
    const int H = g.H, T = g.T;
    const int bb = bh / H, h = bh - bb * H;
    const int hk = h / (H / g.H_kv);
    const uint32_t stq = uint32_t(H) * DK * SI, stkv = uint32_t(g.H_kv) * DK * SI, sty = uint32_t(H) * DK * SY;
    const int64_t tok0 = int64_t(bb) * T;
    const char* rp = static_cast<const char*>(g.r);
    const char* wp = static_cast<const char*>(g.w);
    const char* kp_ = static_cast<const char*>(g.k);
    const char* vp = static_cast<const char*>(g.v);
    const char* ap = static_cast<const char*>(g.a);
    const char* bp = static_cast<const char*>(g.b);
    char* yp = static_cast<char*>(g.y);

    // State tiles: ST[u][r] = S[i_row][16 (2 kp + u) + 4 lq + r], i_row = 32 q + 16 sg + lr.
    const int i_loc = 16 * sg + lr, i_row = DV * q + i_loc;
    const int64_t sbase = int64_t(bh) * DK * DK + int64_t(i_row) * DK;
    f32x4 ST[2];
    #pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (g.s0) {
            const float4 x = *reinterpret_cast<const float4*>(g.s0 + sbase + 16 * (2 * kp + u) + 4 * lq);
            ST[u] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            ST[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // Column threads (P1a): key column jc, tokens [8 pc, 8 pc + 8); threads with
    // jc < 32 also carry value column 32 q + jc.  Row threads (P1b): token tr,
    // key columns [8 qr, 8 qr + 8).
    // Row-thread lanes: 8 key groups x 2 tokens per 16-lane LDS pass, which keeps the
    // 8-byte operand stores free of bank conflicts at this pitch; lanes l and l ^ 32
    // share a token.
    const int jc = tid & (DK - 1), pc = tid >> 7;
    const int tr = 4 * w + ((l >> 3) & 3), qr = (l & 7) | ((l >> 5) << 3);
    float rk8[8];
    if constexpr (EPI) {
        #pragma unroll
        for (int e = 0; e < 8; ++e) rk8[e] = g.r_k[h * DK + 8 * qr + e];
    }
    uint32_t col_q[8], col_kv[8], col_v[8], y_off[4];
    #pragma unroll
    for (int e = 0; e < 8; ++e) {
        col_q[e] = uint32_t(8 * pc + e) * stq + uint32_t(h * DK + jc) * SI;
        col_kv[e] = uint32_t(8 * pc + e) * stkv + uint32_t(hk * DK + jc) * SI;
        col_v[e] = jc < DV ? uint32_t(8 * pc + e) * stkv + uint32_t(hk * DK + DV * q + jc) * SI : kOutOfRange;
        asm volatile("" : "+v"(col_q[e]));
        asm volatile("" : "+v"(col_kv[e]));
        asm volatile("" : "+v"(col_v[e]));
    }
    #pragma unroll
    for (int r = 0; r < 4; ++r) {   // Y tile kp (waves with kp < 2)
        y_off[r] = uint32_t(16 * (kp & 1) + 4 * lq + r) * sty + uint32_t(h * DK + i_row) * SY;
        asm volatile("" : "+v"(y_off[r]));
    }
    const uint32_t row_q = uint32_t(tr) * stq + uint32_t(h * DK + 8 * qr) * SI;
    const uint32_t row_kv = uint32_t(tr) * stkv + uint32_t(hk * DK + 8 * qr) * SI;

    uint32_t cw[8], cb[8], ck[8], cv[8];
    // Row loads; KK: rb holds the decay input row w (b is not read).
    Row8<Tin> rr, ra, rb, rkv;
    // Mask bytes (1 without a mask): lane l of a column wave holds token 8 pc + (l & 7)'s,
    // a row thread its token's.  Masked tokens become identity tokens (zeros, decay 1).
    const char* mp = reinterpret_cast<const char*>(g.mask);
    uint32_t cm = 1u, rm = 1u;
    // Columns of a chunk (for its P1a) and rows (for its P1b) load separately: the
    // next chunk's columns are requested at the start of a chunk, its rows after P1b.
    auto chunk_rsrc = [&](int c0, const char* base, uint32_t stride) {
        const int nv = max(0, min(T - c0, L));
        const int64_t t0 = nv > 0 ? tok0 + c0 : 0;
        return make_rsrc(base + t0 * stride, uint32_t(nv) * stride);
    };
    auto load_cols = [&](int c0) {
        // KK: the b slot of the column loads carries alpha (the a input); b is not read.
        const rsrc_t Rw = chunk_rsrc(c0, wp, stq), Rb = chunk_rsrc(c0, KK ? ap : bp, stq);
        const rsrc_t Rk = chunk_rsrc(c0, kp_, stkv), Rv = chunk_rsrc(c0, vp, stkv);
        if constexpr (MASK) cm = __builtin_amdgcn_raw_buffer_load_b8(chunk_rsrc(c0, mp, 1u), uint32_t(8 * pc + (l & 7)), 0, 0);
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
            cw[e] = Buf<Tin>::load1(Rw, col_q[e]);
            cb[e] = Buf<Tin>::load1(Rb, col_q[e]);
            ck[e] = Buf<Tin>::load1(Rk, col_kv[e]);
            cv[e] = Buf<Tin>::load1(Rv, col_v[e]);
        }
    };
    auto load_rows = [&](int c0) {
        rr.load(chunk_rsrc(c0, rp, stq), row_q);
        ra.load(chunk_rsrc(c0, ap, stq), row_q);
        rb.load(chunk_rsrc(c0, KK ? wp : bp, stq), row_q);
        rkv.load(chunk_rsrc(c0, kp_, stkv), row_kv);
        if constexpr (MASK) rm = __builtin_amdgcn_raw_buffer_load_b8(chunk_rsrc(c0, mp, 1u), uint32_t(tr), 0, 0);
    };
    load_cols(0);
    load_rows(0);

    const int opK = (lr * PK + 8 * lq) * 2;   // 32-deep operand: row lr, k = 8 lq .. 8 lq + 7 ([L][DK])
    const int opT = (lr * PT + 8 * lq) * 2;   // same on the [*][L] matrices
    const int xs_own = ((sg * 4 + kp) * 2 * 64 + l) * 16;

    // ---------------- P1a: decay prefix down each key column ----------------
    // Runs one chunk ahead: the prefix of chunk c + 1 during P2 of chunk c, its
    // tables after P2's first barrier.  The 2^g / 2^-g tables and the segment
    // totals have LDS of their own; the outputs P4..P7 of chunk c still read
    // (Kh^T, V^T, Bh^T, 2^g_L) stay in registers (d_*) until chunk c + 1 begins.
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
        sts<float>(smem + OFF_TOT, (pc * DK + jc) * 4, run);
    };
    auto p1a_tables = [&]() {
        float off = LOGW ? 0.f : 1.f, total = off;
        #pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            const float tp = lds<float>(smem + OFF_TOT, (pp * DK + jc) * 4);
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
                d_vh[e / 2] = (cv[e] >> 16) | (cv[e + 1] & 0xffff0000u);
            }
        }
    };
    auto p1a_store = [&]() {
        if (pc == 0) sts<float>(smem + OFF_EL, jc * 4, d_EL);
        const int o = (jc * PT + 8 * pc) * 2;
        sts<uint4>(smem + OFF_KHTH, o, make_uint4(d_khh[0], d_khh[1], d_khh[2], d_khh[3]));
        sts<uint4>(smem + OFF_KHTL, o, make_uint4(d_khl[0], d_khl[1], d_khl[2], d_khl[3]));
        const int ob = (jc * PT + pairpos(8 * pc)) * 2;
        if constexpr (!KK) {
            sts<uint2>(smem + OFF_BHT, ob, make_uint2(d_bh4[0], d_bh4[1]));
            sts<uint2>(smem + OFF_BHT, ob + 16, make_uint2(d_bh4[2], d_bh4[3]));
        }
        if (jc < DV) {
            sts<uint4>(smem + OFF_VT, o, make_uint4(d_vh[0], d_vh[1], d_vh[2], d_vh[3]));
            if constexpr (VSPLIT) sts<uint4>(smem + OFF_VTL, o, make_uint4(d_vl[0], d_vl[1], d_vl[2], d_vl[3]));
        }
    };
    // KK: Bh^T of the chunk once its row phase has published 1 / n per token.
    auto store_bh_kk = [&]() {
        const float4 n0 = lds<float4>(smem + OFF_INVN, 32 * pc), n1 = lds<float4>(smem + OFF_INVN, 32 * pc + 16);
        const float invn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
        uint32_t bh4[4];
        #pragma unroll
        for (int e = 0; e < 8; e += 2) bh4[e / 2] = pack_bf16(d_bhf[e] * invn[e], d_bhf[e + 1] * invn[e + 1]);
        const int ob = (jc * PT + pairpos(8 * pc)) * 2;
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
        {
            s16x4 h0, l0, h1, l1;
            to_operand(ST[0], h0, l0);
            to_operand(ST[1], h1, l1);
            sts<bf16x8>(smem + OFF_XS, xs_own, cat(h0, h1));
            sts<bf16x8>(smem + OFF_XS, xs_own + 64 * 16, cat(l0, l1));
        }
        p1a_store();
        load_cols(c0 + L);

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
            // KK: 1 / n of this token from its 128 keys, held by its 16 row threads (8
            // consecutive lanes and the same 8 lanes + 32); published for the column threads.
            float invn = 0.f;
            if constexpr (KK) {
                float ss = 0.f;
                #pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(rkv.get(e), rkv.get(e), ss);
                ss += dpp<kDppQuadXor1>(ss);
                ss += dpp<kDppQuadXor2>(ss);
                ss += dpp<kDppRowHalfMirror>(ss);
                ss += __shfl_xor(ss, 32);
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
            const int o = (tr * PK + pairpos(8 * qr)) * 2;
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
                // The 16 threads of a token row: 8 consecutive lanes and the same 8 lanes + 32.
                bonus_part += dpp<kDppQuadXor1>(bonus_part);
                bonus_part += dpp<kDppQuadXor2>(bonus_part);
                bonus_part += dpp<kDppRowHalfMirror>(bonus_part);
                bonus_part += __shfl_xor(bonus_part, 32);
                if (qr == 0) sts<float>(smem + OFF_BONUS, tr * 4, bonus_part);
            }
        }
        load_rows(c0 + L);
        __syncthreads();
        if constexpr (KK) store_bh_kk();   // read in P7, after the barriers to come

        // ---------------- P2: the four L x L matrices; inverses of the diagonal blocks ----------------
        // Units (tile, group) of tiles 0 = (0,0), 1 = (1,0), 2 = (1,1) and groups
        // 0 = A_ab, A_ak; 1 = A_rb, A_rk: waves 0..5 take (0,0) (2,0) (0,1) (2,1)
        // (1,1) (1,0), so that waves 0 and 1, which own the diagonal blocks of A_ab
        // and form their inverses, sit on different SIMDs.  Waves 6, 7 clear tiles.
        const int ptile = w < 4 ? 2 * (w & 1) : 1, pgrp = w < 4 ? (w >> 1) : (w == 4 ? 1 : 0);
        const int ptb = ptile >= 1 ? 1 : 0, psb = ptile == 2 ? 1 : 0;
        const bool pdiag = pgrp == 0 && ptb == psb && w < 6;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
        if (pdiag) {
            // Diagonal unit: A_ab and its swapped form first, so that the inverse chain
            // can overlap the A_ak products.
            f32x4 Nsw = acc0;   // C(N): the block with operands swapped
            #pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const int xb = (16 * ptb * PK + 32 * kq) * 2 + opK;
                const bf16x8 Bt8 = lds<bf16x8>(smem + OFF_BT, xb);
                const bf16x8 At8 = lds<bf16x8>(smem + OFF_AT, xb);
                acc0 = mfma32(Bt8, At8, acc0);
                Nsw = mfma32(At8, Bt8, Nsw);
            }
            #pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const int xb = (16 * ptb * PK + 32 * kq) * 2 + opK;
                const bf16x8 At8 = lds<bf16x8>(smem + OFF_AT, xb);
                acc1 = mfma32(lds<bf16x8>(smem + OFF_KTH, xb), At8, acc1);
                acc1 = mfma32(lds<bf16x8>(smem + OFF_KTL, xb), At8, acc1);
            }
            // (I - N)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) for the strictly lower block N;
            // acc0 is C(N^T) (t = lr, s = 4 lq + r), Nsw is C(N) (s = lr, t = 4 lq + r).
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const s16x4 z4 = {0, 0, 0, 0};
            auto prod = [&](const f32x4 xt, const f32x4 y) {   // C(X^T), C(Y) -> C(X Y)
                s16x4 xh, xl, yh, yl;
                to_operand(xt, xh, xl);
                to_operand(y, yh, yl);
                const f32x4 c = mfma32(cat(xh, xl), cat(yh, yh), zero);
                return mfma32(cat(xh, z4), cat(yl, z4), c);
            };
            f32x4 Nn, Nt, I4;
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                Nt[r] = 4 * lq + r >= lr ? 0.f : acc0[r];
                Nn[r] = lr >= 4 * lq + r ? 0.f : Nsw[r];
                I4[r] = (4 * lq + r == lr) ? 1.f : 0.f;
            }
            const f32x4 N2 = prod(Nt, Nn), N2t = prod(Nn, Nt);
            const f32x4 N4 = prod(N2t, N2), N4t = prod(N2, N2t);
            const f32x4 N8 = prod(N4t, N4);
            const f32x4 Gt = prod(N2 + I4, Nt + I4);
            const f32x4 G4t = prod(N4 + I4, Gt);
            const f32x4 Dt = prod(N8 + I4, G4t);           // lane holds D[lr][4 lq + r]
            sts<uint2>(smem + OFF_DINV, ((ptb * 16 + lr) * PD + 4 * lq) * 2,
                       make_uint2(pack_bf16(Dt[0], Dt[1]), pack_bf16(Dt[2], Dt[3])));
        } else if (w < 6) {
            #pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const int ya = (16 * psb * PK + 32 * kq) * 2 + opK;
                const int xb = (16 * ptb * PK + 32 * kq) * 2 + opK;
                const bf16x8 Bt8 = lds<bf16x8>(smem + OFF_BT, ya);
                const bf16x8 Kh8 = lds<bf16x8>(smem + OFF_KTH, ya);
                const bf16x8 Kl8 = lds<bf16x8>(smem + OFF_KTL, ya);
                if (pgrp == 0) {
                    const bf16x8 At8 = lds<bf16x8>(smem + OFF_AT, xb);
                    acc0 = mfma32(Bt8, At8, acc0);
                    acc1 = mfma32(Kh8, At8, acc1);
                    acc1 = mfma32(Kl8, At8, acc1);
                } else {
                    const bf16x8 Rh8 = lds<bf16x8>(smem + OFF_RTH, xb);
                    const bf16x8 Rl8 = lds<bf16x8>(smem + OFF_RTL, xb);
                    acc0 = mfma32(Bt8, Rh8, acc0);
                    acc0 = mfma32(Bt8, Rl8, acc0);
                    acc1 = mfma32(Kh8, Rh8, acc1);
                    acc1 = mfma32(Kh8, Rl8, acc1);
                    acc1 = mfma32(Kl8, Rh8, acc1);
                }
            }
        }
        p1a_prefix(c0 + L);
        __syncthreads();   // B~ / K~ (region 1) are dead now; next chunk's column totals visible
        p1a_tables();
        if (w < 6) {
            f32x4 c0v = acc0, c1v = acc1;
            if (ptb == psb) {
                const int lim = lr + pgrp;   // group 0 strictly lower, group 1 with the diagonal
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool z = 4 * lq + r >= lim;
                    c0v[r] = z ? 0.f : c0v[r];
                    c1v[r] = z ? 0.f : c1v[r];
                }
            }
            const int orow = (16 * ptb + lr) * PT;
            sts<uint2>(smem + (pgrp == 0 ? OFF_AAB : OFF_ARB), (orow + pairpos(16 * psb + 4 * lq)) * 2,
                       make_uint2(pack_bf16(c0v[0], c0v[1]), pack_bf16(c0v[2], c0v[3])));
            uint32_t h0, l0, h1, l1;
            split2(c1v[0], c1v[1], h0, l0);
            split2(c1v[2], c1v[3], h1, l1);
            const int o = (orow + 16 * psb + 4 * lq) * 2;
            sts<uint2>(smem + (pgrp == 0 ? OFF_AKH : OFF_RKH), o, make_uint2(h0, h1));
            sts<uint2>(smem + (pgrp == 0 ? OFF_AKL : OFF_RKL), o, make_uint2(l0, l1));
        } else {
            // Zero the upper tile (t-block 0, s-block 1) of A_ak and A_rk, read by the
            // 32-deep products of P4.
            const int t2 = tid - 384;
            const int mat = t2 >> 5, rw = (t2 & 31) >> 1, half = t2 & 1;
            const int base = mat == 0 ? OFF_AKH : mat == 1 ? OFF_AKL : mat == 2 ? OFF_RKH : OFF_RKL;
            sts<uint4>(smem + base, (rw * PT + 16 + 8 * half) * 2, make_uint4(0, 0, 0, 0));
        }
        __syncthreads();   // everything P4..P7 read from LDS is in place

        // ---------------- P4: RHS = At S0^T + A_ak V (strip sg), Y's SA-free part ----------------
        bf16x8 Sh[4], Sl[4];
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int xs = ((sg * 4 + p) * 2 * 64 + l) * 16;
            Sh[p] = lds<bf16x8>(smem + OFF_XS, xs);
            Sl[p] = lds<bf16x8>(smem + OFF_XS, xs + 64 * 16);
        }
        const bf16x8 VB = lds<bf16x8>(smem + OFF_VT, 16 * sg * PT * 2 + opT);
        bf16x8 VBl;
        if constexpr (VSPLIT) VBl = lds<bf16x8>(smem + OFF_VTL, 16 * sg * PT * 2 + opT);
        f32x4 RHS[2];
        #pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int p = 0; p < 4; ++p) {
                const bf16x8 A8 = lds<bf16x8>(smem + OFF_AT, (16 * tb * PK + 32 * p) * 2 + opK);
                acc = mfma32(A8, Sh[p], acc);
                acc = mfma32(A8, Sl[p], acc);
            }
            const int o = 16 * tb * PT * 2 + opT;
            const bf16x8 Ah8 = lds<bf16x8>(smem + OFF_AKH, o);
            acc = mfma32(Ah8, VB, acc);
            acc = mfma32(lds<bf16x8>(smem + OFF_AKL, o), VB, acc);
            if constexpr (VSPLIT) acc = mfma32(Ah8, VBl, acc);
            RHS[tb] = acc;
        }
        f32x4 Yacc = {0.f, 0.f, 0.f, 0.f};
        if (kp < 2) {   // token tile kp of Y for this strip
            const int tb = kp;
            #pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int o = (16 * tb * PK + 32 * p) * 2 + opK;
                const bf16x8 Rh8 = lds<bf16x8>(smem + OFF_RTH, o);
                const bf16x8 Rl8 = lds<bf16x8>(smem + OFF_RTL, o);
                Yacc = mfma32(Rh8, Sh[p], Yacc);
                Yacc = mfma32(Rh8, Sl[p], Yacc);
                Yacc = mfma32(Rl8, Sh[p], Yacc);
            }
            const int o = 16 * tb * PT * 2 + opT;
            const bf16x8 Rk8 = lds<bf16x8>(smem + OFF_RKH, o);
            Yacc = mfma32(Rk8, VB, Yacc);
            Yacc = mfma32(lds<bf16x8>(smem + OFF_RKL, o), VB, Yacc);
            if constexpr (VSPLIT) Yacc = mfma32(Rk8, VBl, Yacc);
        }

        // ---------------- P5: SA = (I - A_ab)^-1 RHS, two 16-blocks ----------------
        s16x4 SAh[2], SAl[2];
        #pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            f32x4 x = RHS[ib];
            if (ib == 1) {
                const s16x4 A4 = lds<s16x4>(smem + OFF_AAB, ((16 + lr) * PT + 8 * lq) * 2);   // block (1, 0)
                x = mfma32(cat(A4, A4), cat(SAh[0], SAl[0]), x);
            }
            s16x4 xh, xl;
            to_operand(x, xh, xl);
            const s16x4 D4 = lds<s16x4>(smem + OFF_DINV, ((16 * ib + lr) * PD + 4 * lq) * 2);
            const f32x4 sa = mfma32(cat(D4, D4), cat(xh, xl), f32x4{0.f, 0.f, 0.f, 0.f});
            to_operand(sa, SAh[ib], SAl[ib]);
        }
        const bf16x8 SPh = cat(SAh[0], SAh[1]), SPl = cat(SAl[0], SAl[1]);

        // ---------------- P6: Y += A_rb SA on token tile kp (kp < 2); epilogue; store ----------------
        if (kp < 2) {
            const int nv = max(0, min(T - c0, L));
            const rsrc_t Ry = make_rsrc(yp + (tok0 + c0) * sty, uint32_t(nv) * sty);
            auto p6 = [&](auto TBC) {
                constexpr int TB = decltype(TBC)::value;
                f32x4 acc = Yacc;
                if constexpr (TB == 0) {
                    const s16x4 A4 = lds<s16x4>(smem + OFF_ARB, (lr * PT + 8 * lq) * 2);   // block (0, 0)
                    acc = mfma32(cat(A4, A4), cat(SAh[0], SAl[0]), acc);
                } else {
                    const bf16x8 A8 = lds<bf16x8>(smem + OFF_ARB, 16 * PT * 2 + opT);    // blocks (1, 0..1)
                    acc = mfma32(A8, SPh, acc);
                    acc = mfma32(A8, SPl, acc);
                }
                const int tl0 = 16 * TB + 4 * lq;
                float vtr[4] = {0.f, 0.f, 0.f, 0.f}, bon[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (EPI) {
                    const uint2 vraw = lds<uint2>(smem + OFF_VT, (i_loc * PT + tl0) * 2);
                    vtr[0] = lo_f32(vraw.x); vtr[1] = hi_f32(vraw.x); vtr[2] = lo_f32(vraw.y); vtr[3] = hi_f32(vraw.y);
                    if constexpr (VSPLIT) {
                        const uint2 vlo = lds<uint2>(smem + OFF_VTL, (i_loc * PT + tl0) * 2);
                        vtr[0] += lo_f32(vlo.x); vtr[1] += hi_f32(vlo.x); vtr[2] += lo_f32(vlo.y); vtr[3] += hi_f32(vlo.y);
                    }
                    const float4 bq = lds<float4>(smem + OFF_BONUS, tl0 * 4);
                    bon[0] = bq.x; bon[1] = bq.y; bon[2] = bq.z; bon[3] = bq.w;
                }
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float yv = acc[r] * g.y_scale;
                    if constexpr (EPI) yv = fmaf(bon[r], vtr[r], yv);
                    Buf<Ty>::store1(Ry, y_off[r], yv);
                }
            };
            if (kp == 0) p6(IC<0>{}); else p6(IC<1>{});
        }

        // ---------------- P7: S_L^T = 2^g_L S0^T + Bh^T SA + Kh^T V, key tiles 2 kp, 2 kp + 1 ----------------
        #pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int jt = 2 * kp + u;
            const float4 el4 = lds<float4>(smem + OFF_EL, (16 * jt + 4 * lq) * 4);
            f32x4 acc = ST[u];
            acc[0] *= el4.x; acc[1] *= el4.y; acc[2] *= el4.z; acc[3] *= el4.w;
            const int o = 16 * jt * PT * 2 + opT;
            const bf16x8 B8 = lds<bf16x8>(smem + OFF_BHT, o);
            acc = mfma32(B8, SPh, acc);
            acc = mfma32(B8, SPl, acc);
            const bf16x8 Kh8 = lds<bf16x8>(smem + OFF_KHTH, o);
            acc = mfma32(Kh8, VB, acc);
            acc = mfma32(lds<bf16x8>(smem + OFF_KHTL, o), VB, acc);
            if constexpr (VSPLIT) acc = mfma32(Kh8, VBl, acc);
            ST[u] = acc;
        }
        __syncthreads();   // all LDS operands of this chunk consumed before P1 rewrites them
    }

    if (g.s1) {
        #pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<float4*>(g.s1 + sbase + 16 * (2 * kp + u) + 4 * lq) =
                make_float4(ST[u][0], ST[u][1], ST[u][2], ST[u][3]);
    }
}

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool MASK, bool KK>
hipError_t launch_t(const Params& p, hipStream_t stream) {
    const int bh = p.B * p.H;
    Args g{p.r, p.w, p.k, p.v, p.a, p.b, p.s0, p.r_k, p.mask, p.y, p.s1, p.T, p.H, p.H_kv, bh, p.y_scale};
    auto kern = chunked128_kernel<Tin, Ty, LOGW, EPI, MASK, KK>;
    constexpr int smem = sizeof(Tin) == 4 ? SMEM_F32 : SMEM_BF16;
    static bool attr_set = false;   // per template instance; idempotent if raced
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // 32 workgroups per group of 8 (b, h): 8 heads x 4 value slices.
    const unsigned groups = unsigned((bh + 7) / 8);
    hipLaunchKernelGGL(kern, dim3(groups * 32u), dim3(NTHR), smem, stream, g);
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

hipError_t launch_chunked128(const Params& p, hipStream_t stream) {
    if (p.D != DK || p.chunk_len != L) return hipErrorInvalidValue;
    // Byte offsets inside one chunk's descriptor are 32-bit and below the out-of-range marker.
    if (int64_t(L) * p.H * DK * 4 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<bf16_t, bf16_t>(p, stream) : dispatch_modes<bf16_t, float>(p, stream);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<float, bf16_t>(p, stream) : dispatch_modes<float, float>(p, stream);
}

}  // namespace wkv7
