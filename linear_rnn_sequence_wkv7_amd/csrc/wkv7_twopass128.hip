// Two-pass chunked WKV-7 forward for head size D = 128 on gfx950 bf16 matrix
// cores (fp32 accumulation).
//
// The chunk algebra is that of the one-pass kernels (unrolling S_t = S_{t-1}
// (diag(w_t) + a_t b_t^T) + v_t k_t^T over a chunk of L tokens; wiki note
// "RWKV-7 Goose", generalised delta rule; the chunk-parallel reading of the
// youngju.dev RWKV-7 article, Q&A 5):
//
//   SA  = (I - A_ab)^-1 (At S0^T + A_ak V)
//   Y   = Rt S0^T + A_rb SA + A_rk V
//   S_L = S0 diag(2^g_L) + SA^T Bh + V^T Kh
//
// With Dinv = (I - A_ab)^-1 every state-independent product can be formed
// before the recurrence runs:
//
//   W = Dinv At,  U = Dinv A_ak,  Q = Rt + A_rb W,  P = A_rk + A_rb U,  E = Kh + U^T Bh
//   Y   = Q S0^T + P V
//   S_L = S0 diag(d) + (S0 W^T) Bh + V^T E,        d = 2^g_L
//
// Pass 1 (prep) computes W, Q, E, Bh, P, d and the epilogue's per-token
// bonus for every (b, h, chunk) in parallel -- one D = 128 head per chunk, no
// replication across value slices -- and writes them to a caller-provided
// workspace in the exact lane order of the matrix-core operands that pass 2
// loads.  Pass 2 (scan) runs the chunk recurrence: per chunk four products
// against the state and two small ones, with no L x L algebra left on the
// sequential path.  Four workgroups per (b, h) each own 32 value rows; their
// ids are 8 apart, so under round-robin dispatch they share one XCD's L2 and
// the workspace records they all read are fetched from HBM once.
//
// Operand conventions as in the one-pass kernels: bf16 hi + lo splits where
// a rounding would decide the result, 32-deep contraction axes stored
// pair-interleaved (position 8 q + 4 e + r of a 32-block holds index
// 16 e + 4 q + r), and every accumulator chain uses the single 16x16x32
// opcode (never a result of one MFMA opcode as the accumulator of another).
//
// Only pass 1 reads r, w, k, a, b, so both input options live there.  A
// masked token is the identity token (r, k, a, b = 0, decay 1): its rows and
// columns of every per-chunk matrix vanish, so pass 2 adds nothing for it and
// outputs y = 0.  Kernel vectors from k (KK): the a slot carries alpha; each
// row thread reduces |k|^2 over its 8 keys, the 16 threads of a token meet in
// LDS (one extra barrier inside the scaling step), and the operands take
// a = -kk, b = kk alpha and k (1 - decay + alpha) in place of the inputs.
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
constexpr int DK = 128;        // head size
constexpr int DV = 32;         // value rows per pass-2 workgroup
constexpr int NSLICE = DK / DV;
constexpr int PK = 136;        // bf16 pitch of [L][DK] token-major operands
constexpr int PT = 40;         // bf16 pitch of [*][L] operands
constexpr int PD = 20;         // bf16 pitch of a 16 x 16 block
constexpr int MATK = L * PK * 2;
constexpr int MATT = DK * PT * 2;
constexpr int MATL = L * PT * 2;

// Workspace record of one (b, h, chunk).  Blocks of 1 KB hold one bf16x8
// operand per lane (lane l at byte 16 l).  Per key pair kp (keys 32 kp ..
// 32 kp + 31), block:
//   0, 1   W   as the A operand of W (m = token of block tb, k = key), tb = 0, 1
//   2..5   Q   hi (tb = 0, 1), lo (tb = 0, 1), same layout as W
//   6, 7   Bh  as the A operand of Bh^T (m = key of tile 2 kp + u, k = token), u = 0, 1
//   8..11  E   hi (u = 0, 1), lo (u = 0, 1), same layout as Bh
// then P (A operand, m = token of block tb, k = token): hi tb 0, 1, lo tb 0, 1;
// d[128] fp32; bonus[32] fp32.
constexpr int WS_BLK = 1024;
constexpr int WS_KP = 12 * WS_BLK;
constexpr int BLK_W = 0, BLK_QH = 2, BLK_QL = 4, BLK_BH = 6, BLK_EH = 8, BLK_EL = 10;
constexpr int WS_P = 4 * WS_KP;
constexpr int WS_D = WS_P + 4 * WS_BLK;
constexpr int WS_BON = WS_D + DK * 4;
constexpr int WS_CHUNK = 54272;
static_assert(WS_BON + L * 4 <= WS_CHUNK && WS_CHUNK % 256 == 0, "workspace record");

__host__ __device__ constexpr int pairpos(int k) {
    return 32 * (k >> 5) + 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3);
}

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
__device__ __forceinline__ s16x4 to_bf16x4(const f32x4 c) {
    return __builtin_bit_cast(s16x4, make_uint2(pack_bf16(c[0], c[1]), pack_bf16(c[2], c[3])));
}
// hi + lo of two C-layout tiles as one 32-deep operand each.
__device__ __forceinline__ void to_operand2(const f32x4 c0, const f32x4 c1, bf16x8& hi, bf16x8& lo) {
    s16x4 h0, l0, h1, l1;
    to_operand(c0, h0, l0);
    to_operand(c1, h1, l1);
    hi = cat(h0, h1);
    lo = cat(l0, l1);
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
// Inclusive prefix sums over lanes 0..31 and, separately, 32..63, of 8 values per
// lane, step by step across the 8 (a DPP read of a value written by the previous
// instruction would need wait states).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_add8(float (&x)[8]) {
    #pragma unroll
    for (int i = 0; i < 8; ++i)
        x[i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[i]), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ void scan32x8(float (&x)[8]) {
    dpp_add8<0x111, 0xF>(x);   // row_shr:1
    dpp_add8<0x112, 0xF>(x);   // row_shr:2
    dpp_add8<0x114, 0xF>(x);   // row_shr:4
    dpp_add8<0x118, 0xF>(x);   // row_shr:8
    dpp_add8<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3 only: lane 15 (47) of the row below
}

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
    static __device__ __forceinline__ void store1(rsrc_t r, uint32_t off, float x) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, off, 0, 0);
    }
};
template <> struct Buf<float> {
    static __device__ __forceinline__ void store1(rsrc_t r, uint32_t off, float x) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
    }
};

// 8 consecutive elements of one token row.
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

// Token-axis (pair-interleaved) store of one token's 8 values, rows row0 .. row0 + 7,
// packed in pairs in v, into a [row][PT] bf16 matrix.  Lanes l and l ^ 1 hold
// tokens t and t ^ 1: the even lane writes rows row0 .. row0 + 3, the odd lane
// row0 + 4 .. row0 + 7, each a 32-bit pair of the two tokens.
__device__ __forceinline__ void pair_col_store(char* base, int row0, int t, const uint32_t (&v)[4]) {
    uint32_t pv[4];
    #pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = dpp_u32_xor1(v[i]);
    const bool odd = t & 1;
    const int ocol = pairpos(t & ~1);
    #pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
        const int i_e = xx >> 1, i_o = 2 + (xx >> 1);
        const uint32_t own = odd ? v[i_o] : v[i_e];
        const uint32_t oth = odd ? pv[i_o] : pv[i_e];
        const uint32_t own16 = (xx & 1) ? own >> 16 : own & 0xffffu;
        const uint32_t oth16 = (xx & 1) ? oth >> 16 : oth & 0xffffu;
        const uint32_t word = odd ? (oth16 | (own16 << 16)) : (own16 | (oth16 << 16));
        const int row = row0 + (odd ? 4 : 0) + xx;
        sts<uint32_t>(base, (row * PT + ocol) * 2, word);
    }
}

// Chunk descriptor: tokens [c0, c0 + L) of sequence bb, clipped at T (the rest reads 0).
__device__ __forceinline__ rsrc_t chunk_rsrc(const char* base, int64_t tok0, int c0, int T, uint32_t stride) {
    const int nv = max(0, min(T - c0, L));
    const int64_t t0 = nv > 0 ? tok0 + c0 : 0;
    return make_rsrc(base + t0 * stride, uint32_t(nv) * stride);
}

// ============================== pass 1: per-chunk matrices ==============================

// LDS map of pass 1 (bytes).  Token-major operands (key axis pair-interleaved):
// At, Bt, Kt hi / lo, Rt hi / lo.  Key-major (token axis pair-interleaved):
// At^T, Bh^T.  L x L matrices: A_rb [t][s~], A_ak^T hi / lo [s][t~], A_rk hi / lo
// [t][s], Dinv hi / lo [t][s~], U^T hi / lo [s'][s~] (~: pair-interleaved).
constexpr int P_AT = 0;
constexpr int P_BT = P_AT + MATK;
constexpr int P_KTH = P_BT + MATK;
constexpr int P_KTL = P_KTH + MATK;
constexpr int P_RTH = P_KTL + MATK;
constexpr int P_RTL = P_RTH + MATK;
constexpr int P_ATT = P_RTL + MATK;
constexpr int P_BHT = P_ATT + MATT;
constexpr int P_ARB = P_BHT + MATT;
constexpr int P_AKTH = P_ARB + MATL;
constexpr int P_AKTL = P_AKTH + MATL;
constexpr int P_ARKH = P_AKTL + MATL;
constexpr int P_ARKL = P_ARKH + MATL;
constexpr int P_DIH = P_ARKL + MATL;
constexpr int P_DIL = P_DIH + MATL;
constexpr int P_UTH = P_DIL + MATL;
constexpr int P_UTL = P_UTH + MATL;
constexpr int P_D0T = P_UTL + MATL;              // D0^T hi / lo, [16][PD] each
constexpr int P_DL = P_D0T + 2 * 16 * PD * 2;    // fp32 [DK] 2^g_L
constexpr int P_BON = P_DL + DK * 4;             // fp32 [8 waves][L] bonus partials
constexpr int P_KSQ = P_BON + 8 * L * 4;         // fp32 [L][8 waves] |k|^2 partials (KK)
constexpr int SMEM_PREP = P_KSQ + L * 8 * 4;
static_assert(SMEM_PREP <= 160 * 1024, "LDS budget");
static_assert(P_ATT % 16 == 0 && P_ARB % 16 == 0 && P_D0T % 16 == 0 && P_DL % 16 == 0, "alignment");

constexpr int NTHR_PREP = 512;
constexpr int kPrepGrid = 256;   // one persistent workgroup per compute unit of MI355X

struct PrepArgs {
    const void *r, *w, *k, *a, *b;
    const float* r_k;
    const uint8_t* mask;
    char* ws;
    int T, H, H_kv, nch, items;
};

template <typename Tin> struct ItemRows {
    Row8<Tin> r, w, k, a, b;
    float rk[8];
    uint32_t m;   // mask byte of the row's token (1 without a mask, 0 past the end)
};
// (One dword per load instruction suffices: the wait is per instruction.)
__device__ __forceinline__ void settle_row(Row8<bf16_t>& x) { asm volatile("" : "+v"(x.x.x)); }
__device__ __forceinline__ void settle_row(Row8<float>& x) { asm volatile("" : "+v"(x.x[0].x), "+v"(x.x[1].x)); }

template <typename Tin, bool LOGW, bool EPI, bool KK>
__global__ __launch_bounds__(NTHR_PREP)
void prep128_kernel(PrepArgs g) {
    constexpr uint32_t SI = sizeof(Tin);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
    const int H = g.H, T = g.T, nch = g.nch;
    const uint32_t stq = uint32_t(H) * DK * SI, stkv = uint32_t(g.H_kv) * DK * SI;
    // Row threads: token t of the chunk, keys j0 .. j0 + 7.
    const int t = l & 31, j0 = 8 * (2 * w + (l >> 5));

    auto load_item = [&](int item, ItemRows<Tin>& x) {
        const int bh = item / nch, c = item - bh * nch;
        const int bb = bh / H, h = bh - bb * H, hk = h / (H / g.H_kv);
        const int64_t tok0 = int64_t(bb) * T;
        const int c0 = c * L;
        const uint32_t oq = uint32_t(t) * stq + uint32_t(h * DK + j0) * SI;
        const uint32_t okv = uint32_t(t) * stkv + uint32_t(hk * DK + j0) * SI;
        x.r.load(chunk_rsrc(static_cast<const char*>(g.r), tok0, c0, T, stq), oq);
        x.w.load(chunk_rsrc(static_cast<const char*>(g.w), tok0, c0, T, stq), oq);
        x.a.load(chunk_rsrc(static_cast<const char*>(g.a), tok0, c0, T, stq), oq);
        if constexpr (!KK) x.b.load(chunk_rsrc(static_cast<const char*>(g.b), tok0, c0, T, stq), oq);
        x.k.load(chunk_rsrc(static_cast<const char*>(g.k), tok0, c0, T, stkv), okv);
        x.m = g.mask ? uint32_t(__builtin_amdgcn_raw_buffer_load_b8(
                           chunk_rsrc(reinterpret_cast<const char*>(g.mask), tok0, c0, T, 1u), uint32_t(t), 0, 0))
                     : 1u;
        if constexpr (EPI) {
            const float4 u0 = *reinterpret_cast<const float4*>(g.r_k + h * DK + j0);
            const float4 u1 = *reinterpret_cast<const float4*>(g.r_k + h * DK + j0 + 4);
            x.rk[0] = u0.x; x.rk[1] = u0.y; x.rk[2] = u0.z; x.rk[3] = u0.w;
            x.rk[4] = u1.x; x.rk[5] = u1.y; x.rk[6] = u1.z; x.rk[7] = u1.w;
        }
    };

    // 32-deep operand of 16-row block `blk` of a token-major [L][DK] matrix, k-step kq.
    auto opK = [&](int blk, int kq) { return ((16 * blk + lr) * PK + 32 * kq + 8 * lq) * 2; };
    // 32-deep operand of 16-row block `blk` of a [*][PT] matrix (contraction over tokens).
    auto opT = [&](int blk) { return ((16 * blk + lr) * PT + 8 * lq) * 2; };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const s16x4 z4 = {0, 0, 0, 0};

    ItemRows<Tin> cur, nxt;
    auto settle_item = [&](ItemRows<Tin>& x) {
        settle_row(x.r); settle_row(x.w); settle_row(x.k); settle_row(x.a);
        if constexpr (!KK) settle_row(x.b);
        asm volatile("" : "+v"(x.m));
        #pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(x.rk[e]));
    };
    int item = blockIdx.x;
    if (item < g.items) {
        load_item(item, nxt);
        settle_item(nxt);
    }
    for (; item < g.items; item += gridDim.x) {
        cur = nxt;
        const int bh = item / nch, c = item - bh * nch;
        const int c0 = c * L;
        char* rec = g.ws + (int64_t(bh) * nch + c) * WS_CHUNK;

        // ---------------- Q0: decay prefix and the scaled operands (row threads) ----------------
        {
            // Tokens past the end (and masked ones) decay by 1 and carry zeros.
            const bool ok = c0 + t < T && cur.m != 0;
            if (g.mask) {
                cur.r.keep_if(ok); cur.k.keep_if(ok); cur.a.keep_if(ok);
                if constexpr (!KK) cur.b.keep_if(ok);
            }
            if constexpr (KK) {
                // |k|^2 partial over this thread's 8 keys and its partner lane's 8.
                float ss = 0.f;
                #pragma unroll
                for (int x = 0; x < 8; ++x) ss = fmaf(cur.k.get(x), cur.k.get(x), ss);
                ss += __shfl_xor(ss, 32);
                if (l < 32) sts<float>(smem + P_KSQ, (t * 8 + w) * 4, ss);
            }
            // Per key: E = 2^g_t, Ei = 2^-g_t; 2^g_(t-1) is E of the previous token
            // (lane l - 1, 1 at t = 0); d = 2^g_L is E of token 31 (lane 31 / 63) and
            // 2^(g_L - g_t) = d Ei.  Two exp2 per element besides the log-decay.
            float Ex[8], Eix[8], Epx[8], dx[8], gs[8], dec[8];
            #pragma unroll
            for (int x = 0; x < 8; ++x) gs[x] = ok ? log2_decay(cur.w.get(x), LOGW) : 0.f;
            if constexpr (KK) {
                #pragma unroll
                for (int x = 0; x < 8; ++x) dec[x] = LOGW ? __builtin_amdgcn_exp2f(gs[x]) : cur.w.get(x);
            }
            scan32x8(gs);
            #pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float gg = gs[x];
                Ex[x] = __builtin_amdgcn_exp2f(gg);
                Eix[x] = __builtin_amdgcn_exp2f(-gg);
                const float prev = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(Ex[x]), 0x138, 0xF, 0xF, false));   // wave_shr:1
                Epx[x] = t == 0 ? 1.f : prev;
                const float d31 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ex[x]), 31));
                const float d63 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ex[x]), 63));
                dx[x] = l < 32 ? d31 : d63;
            }
            // KK: the token's |k|^2 from the 8 waves' partials.
            float inv = 0.f;
            if constexpr (KK) {
                __syncthreads();
                const float4 s0 = lds<float4>(smem + P_KSQ, t * 32), s1 = lds<float4>(smem + P_KSQ, t * 32 + 16);
                inv = inv_key_norm(((s0.x + s0.y) + (s0.z + s0.w)) + ((s1.x + s1.y) + (s1.z + s1.w)));
            }
            uint32_t at[4], rth[4], rtl[4], bt[4], kth[4], ktl[4], bhat[4];
            float bonus_part = 0.f;
            #pragma unroll
            for (int e = 0; e < 8; e += 2) {
                float Ep[2], E[2], Ei[2], Eh[2];
                #pragma unroll
                for (int u = 0; u < 2; ++u) {
                    E[u] = Ex[e + u];
                    Ep[u] = Epx[e + u];
                    Ei[u] = Eix[e + u];
                    Eh[u] = dx[e + u] * Eix[e + u];
                }
                const float r0 = cur.r.get(e), r1 = cur.r.get(e + 1);
                float k0 = cur.k.get(e), k1 = cur.k.get(e + 1);
                float a0 = cur.a.get(e), a1 = cur.a.get(e + 1);
                float b0, b1;
                if constexpr (KK) {
                    // a holds alpha: b = kk alpha, a = -kk, k <- k (1 - decay + alpha).
                    const float kk0 = k0 * inv, kk1 = k1 * inv;
                    b0 = kk0 * a0; b1 = kk1 * a1;
                    k0 *= 1.f - dec[e] + a0; k1 *= 1.f - dec[e + 1] + a1;
                    a0 = -kk0; a1 = -kk1;
                } else {
                    b0 = cur.b.get(e); b1 = cur.b.get(e + 1);
                }
                at[e / 2] = pack_bf16(a0 * Ep[0], a1 * Ep[1]);
                split2(r0 * E[0], r1 * E[1], rth[e / 2], rtl[e / 2]);
                bt[e / 2] = pack_bf16(b0 * Ei[0], b1 * Ei[1]);
                split2(k0 * Ei[0], k1 * Ei[1], kth[e / 2], ktl[e / 2]);
                bhat[e / 2] = pack_bf16(b0 * Eh[0], b1 * Eh[1]);
                if constexpr (EPI) bonus_part += r0 * k0 * cur.rk[e] + r1 * k1 * cur.rk[e + 1];
            }
            const int o = (t * PK + pairpos(j0)) * 2;
            sts<uint2>(smem + P_AT, o, make_uint2(at[0], at[1]));
            sts<uint2>(smem + P_AT, o + 16, make_uint2(at[2], at[3]));
            sts<uint2>(smem + P_BT, o, make_uint2(bt[0], bt[1]));
            sts<uint2>(smem + P_BT, o + 16, make_uint2(bt[2], bt[3]));
            sts<uint2>(smem + P_KTH, o, make_uint2(kth[0], kth[1]));
            sts<uint2>(smem + P_KTH, o + 16, make_uint2(kth[2], kth[3]));
            sts<uint2>(smem + P_KTL, o, make_uint2(ktl[0], ktl[1]));
            sts<uint2>(smem + P_KTL, o + 16, make_uint2(ktl[2], ktl[3]));
            sts<uint2>(smem + P_RTH, o, make_uint2(rth[0], rth[1]));
            sts<uint2>(smem + P_RTH, o + 16, make_uint2(rth[2], rth[3]));
            sts<uint2>(smem + P_RTL, o, make_uint2(rtl[0], rtl[1]));
            sts<uint2>(smem + P_RTL, o + 16, make_uint2(rtl[2], rtl[3]));
            // Key-major copies of At and Bh.
            pair_col_store(smem + P_ATT, j0, t, at);
            pair_col_store(smem + P_BHT, j0, t, bhat);
            if (t == 0) {
                sts<float4>(smem + P_DL, j0 * 4, make_float4(dx[0], dx[1], dx[2], dx[3]));
                sts<float4>(smem + P_DL, j0 * 4 + 16, make_float4(dx[4], dx[5], dx[6], dx[7]));
            }
            if constexpr (EPI) {
                bonus_part += __shfl_xor(bonus_part, 32);
                if (l < 32) sts<float>(smem + P_BON, (w * L + t) * 4, bonus_part);
            }
        }
        // Next item's rows: this item's are consumed.  (Pinned here so that the loads
        // are not sunk towards their use in the next iteration.)
        if (item + int(gridDim.x) < g.items) load_item(item + gridDim.x, nxt);
        asm volatile("" ::: "memory");
        __syncthreads();

        // ---------------- Q1: the four L x L matrices; Dinv ----------------
        // Tiles (tb, sb) of the lower triangle: 0 = (0,0), 1 = (1,0), 2 = (1,1).
        // prod(C(X^T), C(Y)) = C(X Y), operands split hi + lo.
        auto prod = [&](const f32x4 xt, const f32x4 y) {
            s16x4 xh, xl, yh, yl;
            to_operand(xt, xh, xl);
            to_operand(y, yh, yl);
            const f32x4 cc = mfma32(cat(xh, xl), cat(yh, yh), zero);
            return mfma32(cat(xh, z4), cat(yl, z4), cc);
        };
        f32x4 I4;
        #pragma unroll
        for (int r = 0; r < 4; ++r) I4[r] = (4 * lq + r == lr) ? 1.f : 0.f;
        // (I - N)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) for the strictly lower block
        // N; Nt = C(N^T) (t = lr, s = 4 lq + r), Nn = C(N).  Returns C(D^T).
        auto chain = [&](const f32x4 cab, const f32x4 csw) {
            f32x4 Nn, Nt;
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                Nt[r] = 4 * lq + r >= lr ? 0.f : cab[r];
                Nn[r] = lr >= 4 * lq + r ? 0.f : csw[r];
            }
            const f32x4 N2 = prod(Nt, Nn), N2t = prod(Nn, Nt);
            const f32x4 N4 = prod(N2t, N2), N4t = prod(N2, N2t);
            const f32x4 N8 = prod(N4t, N4);
            const f32x4 Gt = prod(N2 + I4, Nt + I4);
            const f32x4 G4t = prod(N4 + I4, Gt);
            return prod(N8 + I4, G4t);            // lane holds D[lr][4 lq + r]
        };
        auto store_blk = [&](int row0, int col0, const f32x4 v) {
            uint32_t h0, l0, h1, l1;
            split2(v[0], v[1], h0, l0);
            split2(v[2], v[3], h1, l1);
            const int o = ((row0 + lr) * PT + pairpos(col0 + 4 * lq)) * 2;
            sts<uint2>(smem + P_DIH, o, make_uint2(h0, h1));
            sts<uint2>(smem + P_DIL, o, make_uint2(l0, l1));
        };
        // The block inverse of I - A_ab: D0 on wave 0, D1 on wave 1 (the two doubling
        // chains run on different SIMDs), then D10 = D1 A10 D0 on wave 0.
        f32x4 Tm = zero;   // A10 D0 (wave 0), kept across the exchange below
        if (w == 0) {
            // A_ab tiles 0, 1 and block 0 swapped.  C'[s][t] orientation: lane t = lr, s = 4 lq + r.
            f32x4 ab[2] = {zero, zero}, nsw0 = zero;
            #pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const bf16x8 B0 = lds<bf16x8>(smem + P_BT, opK(0, kq));
                const bf16x8 A0 = lds<bf16x8>(smem + P_AT, opK(0, kq)), A1 = lds<bf16x8>(smem + P_AT, opK(1, kq));
                ab[0] = mfma32(B0, A0, ab[0]);
                ab[1] = mfma32(B0, A1, ab[1]);
                nsw0 = mfma32(A0, B0, nsw0);
            }
            const f32x4 Dt0 = chain(ab[0], nsw0);
            // D0^T to LDS (wave-private), hi / lo: D0[lr][4 lq + r] -> row 4 lq + r, column lr.
            {
                uint32_t h0, l0, h1, l1;
                split2(Dt0[0], Dt0[1], h0, l0);
                split2(Dt0[2], Dt0[3], h1, l1);
                const uint16_t hv[4] = {uint16_t(h0), uint16_t(h0 >> 16), uint16_t(h1), uint16_t(h1 >> 16)};
                const uint16_t lv[4] = {uint16_t(l0), uint16_t(l0 >> 16), uint16_t(l1), uint16_t(l1 >> 16)};
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sts<uint16_t>(smem + P_D0T, ((4 * lq + r) * PD + lr) * 2, hv[r]);
                    sts<uint16_t>(smem + P_D0T + 16 * PD * 2, ((4 * lq + r) * PD + lr) * 2, lv[r]);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // T = A10 D0 (C layout: t = 4 lq + r, s = lr).  ab[1] is C(A10^T), i.e. the
            // 16-deep A operand of A10; D0 as the B operand from D0^T rows.
            {
                s16x4 ah, al;
                to_operand(ab[1], ah, al);
                const s16x4 dh = lds<s16x4>(smem + P_D0T, (lr * PD + 4 * lq) * 2);
                const s16x4 dl = lds<s16x4>(smem + P_D0T + 16 * PD * 2, (lr * PD + 4 * lq) * 2);
                Tm = mfma32(cat(ah, ah), cat(dh, dl), zero);
                Tm = mfma32(cat(al, z4), cat(dh, z4), Tm);
            }
            store_blk(0, 0, Dt0);
            store_blk(0, 16, zero);
        } else {
            if (w == 1) {   // D1 from A_ab block 1; C(D1^T) to the U^T area (free until Q2) for wave 0
                f32x4 ab2 = zero, nsw1 = zero;
                #pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const bf16x8 B1 = lds<bf16x8>(smem + P_BT, opK(1, kq)), A1 = lds<bf16x8>(smem + P_AT, opK(1, kq));
                    ab2 = mfma32(B1, A1, ab2);
                    nsw1 = mfma32(A1, B1, nsw1);
                }
                const f32x4 Dt1 = chain(ab2, nsw1);
                sts<float4>(smem + P_UTH, (16 * lq + lr) * 16, make_float4(Dt1[0], Dt1[1], Dt1[2], Dt1[3]));
                store_blk(16, 16, Dt1);
            }
            // Waves 1..3: A_rk; 4..6: A_ak (swapped orientation); 7: all three tiles of A_rb.
            auto tile_tb = [](int n) { return n == 0 ? 0 : 1; };
            auto tile_sb = [](int n) { return n == 2 ? 1 : 0; };
            if (w <= 3) {
                const int n = w - 1, tb = tile_tb(n), sb = tile_sb(n);
                f32x4 acc = zero;
                #pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const bf16x8 Kh8 = lds<bf16x8>(smem + P_KTH, opK(sb, kq)), Kl8 = lds<bf16x8>(smem + P_KTL, opK(sb, kq));
                    const bf16x8 Rh8 = lds<bf16x8>(smem + P_RTH, opK(tb, kq)), Rl8 = lds<bf16x8>(smem + P_RTL, opK(tb, kq));
                    acc = mfma32(Kh8, Rh8, acc);
                    acc = mfma32(Kh8, Rl8, acc);
                    acc = mfma32(Kl8, Rh8, acc);
                }
                // C'[s][t]: lane t = 16 tb + lr, s = 16 sb + 4 lq + r; lower with the diagonal.
                #pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = (tb == sb && 4 * lq + r > lr) ? 0.f : acc[r];
                uint32_t h0, l0, h1, l1;
                split2(acc[0], acc[1], h0, l0);
                split2(acc[2], acc[3], h1, l1);
                const int o = ((16 * tb + lr) * PT + 16 * sb + 4 * lq) * 2;
                sts<uint2>(smem + P_ARKH, o, make_uint2(h0, h1));
                sts<uint2>(smem + P_ARKL, o, make_uint2(l0, l1));
            } else if (w <= 6) {
                const int n = w - 4, tb = tile_tb(n), sb = tile_sb(n);
                f32x4 acc = zero;
                #pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const bf16x8 A8 = lds<bf16x8>(smem + P_AT, opK(tb, kq));
                    acc = mfma32(A8, lds<bf16x8>(smem + P_KTH, opK(sb, kq)), acc);
                    acc = mfma32(A8, lds<bf16x8>(smem + P_KTL, opK(sb, kq)), acc);
                }
                // C[t][s]: lane t = 16 tb + 4 lq + r, s = 16 sb + lr; strictly lower.
                #pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = (tb == sb && 4 * lq + r <= lr) ? 0.f : acc[r];
                uint32_t h0, l0, h1, l1;
                split2(acc[0], acc[1], h0, l0);
                split2(acc[2], acc[3], h1, l1);
                const int o = ((16 * sb + lr) * PT + pairpos(16 * tb + 4 * lq)) * 2;
                sts<uint2>(smem + P_AKTH, o, make_uint2(h0, h1));
                sts<uint2>(smem + P_AKTL, o, make_uint2(l0, l1));
                if (w == 6) {
                    // A_ak^T rows s >= 16 at tokens t < 16 are zero (strictly lower).
                    const int oz = ((16 + lr) * PT + pairpos(4 * lq)) * 2;
                    sts<uint2>(smem + P_AKTH, oz, make_uint2(0, 0));
                    sts<uint2>(smem + P_AKTL, oz, make_uint2(0, 0));
                }
            } else {
                f32x4 acc[3] = {zero, zero, zero};
                #pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const bf16x8 B0 = lds<bf16x8>(smem + P_BT, opK(0, kq)), B1 = lds<bf16x8>(smem + P_BT, opK(1, kq));
                    const bf16x8 R0h = lds<bf16x8>(smem + P_RTH, opK(0, kq)), R0l = lds<bf16x8>(smem + P_RTL, opK(0, kq));
                    const bf16x8 R1h = lds<bf16x8>(smem + P_RTH, opK(1, kq)), R1l = lds<bf16x8>(smem + P_RTL, opK(1, kq));
                    acc[0] = mfma32(B0, R0h, acc[0]);
                    acc[0] = mfma32(B0, R0l, acc[0]);
                    acc[1] = mfma32(B0, R1h, acc[1]);
                    acc[1] = mfma32(B0, R1l, acc[1]);
                    acc[2] = mfma32(B1, R1h, acc[2]);
                    acc[2] = mfma32(B1, R1l, acc[2]);
                }
                #pragma unroll
                for (int n = 0; n < 3; ++n) {
                    const int tb = tile_tb(n), sb = tile_sb(n);
                    f32x4 v = acc[n];
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = (tb == sb && 4 * lq + r > lr) ? 0.f : v[r];
                    sts<uint2>(smem + P_ARB, ((16 * tb + lr) * PT + pairpos(16 * sb + 4 * lq)) * 2,
                               make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])));
                }
                // A_rb row block 0 at s >= 16 is zero.
                sts<uint2>(smem + P_ARB, (lr * PT + pairpos(16 + 4 * lq)) * 2, make_uint2(0, 0));
            }
        }
        __syncthreads();
        if (w == 0) {
            // C(D10^T) = prod(C(T), C(D1^T)) = C(T^T D1^T): lane holds D10[lr][4 lq + r].
            const float4 x = lds<float4>(smem + P_UTH, (16 * lq + lr) * 16);
            store_blk(16, 0, prod(Tm, f32x4{x.x, x.y, x.z, x.w}));
        }
        __syncthreads();

        // ---------------- Q2: U = Dinv A_ak; W and Q for key pair kp, token block tb ----------------
        if (w < 3) {
            // C(U) tile (sb, s'b): lane s = 16 sb + 4 lq + r, s' = 16 s'b + lr.
            const int sb = w == 0 ? 0 : 1, spb = w == 2 ? 1 : 0;
            const bf16x8 Dh = lds<bf16x8>(smem + P_DIH, opT(sb)), Dl = lds<bf16x8>(smem + P_DIL, opT(sb));
            const bf16x8 Kh = lds<bf16x8>(smem + P_AKTH, opT(spb)), Kl = lds<bf16x8>(smem + P_AKTL, opT(spb));
            f32x4 u = mfma32(Dh, Kh, zero);
            u = mfma32(Dh, Kl, u);
            u = mfma32(Dl, Kh, u);
            uint32_t h0, l0, h1, l1;
            split2(u[0], u[1], h0, l0);
            split2(u[2], u[3], h1, l1);
            const int o = ((16 * spb + lr) * PT + pairpos(16 * sb + 4 * lq)) * 2;   // U^T[s'][s~]
            sts<uint2>(smem + P_UTH, o, make_uint2(h0, h1));
            sts<uint2>(smem + P_UTL, o, make_uint2(l0, l1));
        } else if (w == 3) {
            // U^T rows s' >= 16 at s < 16 are zero.
            const int o = ((16 + lr) * PT + pairpos(4 * lq)) * 2;
            sts<uint2>(smem + P_UTH, o, make_uint2(0, 0));
            sts<uint2>(smem + P_UTL, o, make_uint2(0, 0));
        }
        {
            const int kp = w >> 1, tb = w & 1;
            bf16x8 Dh[2], Dl[2], At8[2];
            #pragma unroll
            for (int i = 0; i < 2; ++i) {
                Dh[i] = lds<bf16x8>(smem + P_DIH, opT(i));
                Dl[i] = lds<bf16x8>(smem + P_DIL, opT(i));
                At8[i] = lds<bf16x8>(smem + P_ATT, opT(2 * kp + i));
            }
            // C(W^T) tiles (key tile 2 kp + u, token block tb): lane key 4 lq + r, token lr.
            // (Operands of block tb are loaded again rather than indexed by the
            // wave-dependent tb, which would compile to per-element selects.)
            const bf16x8 DhT = lds<bf16x8>(smem + P_DIH, opT(tb)), DlT = lds<bf16x8>(smem + P_DIL, opT(tb));
            f32x4 wt[2];
            #pragma unroll
            for (int u = 0; u < 2; ++u) wt[u] = mfma32(At8[u], DlT, mfma32(At8[u], DhT, zero));
            {
                const uint4 o4 = make_uint4(pack_bf16(wt[0][0], wt[0][1]), pack_bf16(wt[0][2], wt[0][3]),
                                            pack_bf16(wt[1][0], wt[1][1]), pack_bf16(wt[1][2], wt[1][3]));
                *reinterpret_cast<uint4*>(rec + kp * WS_KP + (BLK_W + tb) * WS_BLK + l * 16) = o4;
            }
            // C(W) tiles (token block sb, key tile 2 kp + u): lane token 4 lq + r, key lr.
            // As A operands they are W^T with the token axis as k.
            s16x4 wh[2][2], wl[2][2];
            #pragma unroll
            for (int sb = 0; sb < 2; ++sb)
                #pragma unroll
                for (int u = 0; u < 2; ++u)
                    to_operand(mfma32(Dl[sb], At8[u], mfma32(Dh[sb], At8[u], zero)), wh[sb][u], wl[sb][u]);
            // C(Q^T) tiles: Q^T = Rt^T + W^T A_rb^T.
            const bf16x8 Ar8 = lds<bf16x8>(smem + P_ARB, opT(tb));
            f32x4 qt[2];
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int orow = ((16 * tb + lr) * PK + pairpos(16 * (2 * kp + u) + 4 * lq)) * 2;
                const uint2 rh = lds<uint2>(smem + P_RTH, orow), rl = lds<uint2>(smem + P_RTL, orow);
                f32x4 acc = {lo_f32(rh.x) + lo_f32(rl.x), hi_f32(rh.x) + hi_f32(rl.x),
                             lo_f32(rh.y) + lo_f32(rl.y), hi_f32(rh.y) + hi_f32(rl.y)};
                acc = mfma32(cat(wh[0][u], wh[1][u]), Ar8, acc);
                acc = mfma32(cat(wl[0][u], wl[1][u]), Ar8, acc);
                qt[u] = acc;
            }
            bf16x8 qh, ql;
            to_operand2(qt[0], qt[1], qh, ql);
            *reinterpret_cast<bf16x8*>(rec + kp * WS_KP + (BLK_QH + tb) * WS_BLK + l * 16) = qh;
            *reinterpret_cast<bf16x8*>(rec + kp * WS_KP + (BLK_QL + tb) * WS_BLK + l * 16) = ql;
        }
        __syncthreads();

        // ---------------- Q3: E = Kh + U^T Bh and Bh for key tile jt; P; d; bonus ----------------
        {
            const int kp = w >> 1, u = w & 1, jt = 2 * kp + u;
            const bf16x8 Bh8 = lds<bf16x8>(smem + P_BHT, opT(jt));
            *reinterpret_cast<bf16x8*>(rec + kp * WS_KP + (BLK_BH + u) * WS_BLK + l * 16) = Bh8;
            const float dj = lds<float>(smem + P_DL, (16 * jt + lr) * 4);
            const int kpos = pairpos(16 * jt + lr);
            f32x4 e[2];
            #pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                f32x4 acc;
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = ((16 * tb + 4 * lq + r) * PK + kpos) * 2;
                    const float kh = bf16_to_f32(lds<uint16_t>(smem + P_KTH, o)) + bf16_to_f32(lds<uint16_t>(smem + P_KTL, o));
                    acc[r] = kh * dj;   // Kh = Kt 2^g_L
                }
                acc = mfma32(lds<bf16x8>(smem + P_UTH, opT(tb)), Bh8, acc);
                acc = mfma32(lds<bf16x8>(smem + P_UTL, opT(tb)), Bh8, acc);
                e[tb] = acc;
            }
            bf16x8 eh, el;
            to_operand2(e[0], e[1], eh, el);
            *reinterpret_cast<bf16x8*>(rec + kp * WS_KP + (BLK_EH + u) * WS_BLK + l * 16) = eh;
            *reinterpret_cast<bf16x8*>(rec + kp * WS_KP + (BLK_EL + u) * WS_BLK + l * 16) = el;
        }
        if (w == 0) {
            // C(P^T) tiles (s'b, tb): P^T = A_rk^T + U^T A_rb^T; lane s' = 16 s'b + 4 lq + r, t = 16 tb + lr.
            f32x4 pt[3];   // (0,0), (0,1), (1,1)
            #pragma unroll
            for (int n = 0; n < 3; ++n) {
                const int spb = n == 2 ? 1 : 0, tb = n == 0 ? 0 : 1;
                const int o = ((16 * tb + lr) * PT + 16 * spb + 4 * lq) * 2;
                const uint2 kh = lds<uint2>(smem + P_ARKH, o), kl = lds<uint2>(smem + P_ARKL, o);
                f32x4 acc = {lo_f32(kh.x) + lo_f32(kl.x), hi_f32(kh.x) + hi_f32(kl.x),
                             lo_f32(kh.y) + lo_f32(kl.y), hi_f32(kh.y) + hi_f32(kl.y)};
                const bf16x8 Ar8 = lds<bf16x8>(smem + P_ARB, opT(tb));
                acc = mfma32(lds<bf16x8>(smem + P_UTH, opT(spb)), Ar8, acc);
                acc = mfma32(lds<bf16x8>(smem + P_UTL, opT(spb)), Ar8, acc);
                pt[n] = acc;
            }
            bf16x8 ph, pl;
            to_operand2(pt[0], zero, ph, pl);
            *reinterpret_cast<bf16x8*>(rec + WS_P + 0 * WS_BLK + l * 16) = ph;
            *reinterpret_cast<bf16x8*>(rec + WS_P + 2 * WS_BLK + l * 16) = pl;
            to_operand2(pt[1], pt[2], ph, pl);
            *reinterpret_cast<bf16x8*>(rec + WS_P + 1 * WS_BLK + l * 16) = ph;
            *reinterpret_cast<bf16x8*>(rec + WS_P + 3 * WS_BLK + l * 16) = pl;
        } else if (w == 1) {
            if (l < 32) *reinterpret_cast<float4*>(rec + WS_D + l * 16) = lds<float4>(smem + P_DL, l * 16);
        } else if (w == 2) {
            if constexpr (EPI) {
                if (l < 32) {
                    float s = 0.f;
                    #pragma unroll
                    for (int v = 0; v < 8; ++v) s += lds<float>(smem + P_BON, (v * L + l) * 4);
                    *reinterpret_cast<float*>(rec + WS_BON + l * 4) = s;
                }
            }
        }
        // Prefetched rows complete here, not across the loop back-edge, where the
        // compiler's wait counting would also wait for this item's stores.
        settle_item(nxt);
        __syncthreads();   // LDS is rewritten by the next item
    }
}


// ============================== pass 2: the chunk recurrence ==============================

// LDS map of pass 2 (bytes): the four waves' partial X and Y tiles, the reduced X
// tiles as bf16 hi / lo operands, and V^T of the slice (two chunk buffers).
constexpr int NTHR_SCAN = 256;
constexpr int S_PART = 0;                          // f32x4 [wave][tile 0..7][lane]
constexpr int S_XOH = S_PART + 4 * 8 * 64 * 16;    // s16x4 [tile 0..3][lane]
constexpr int S_XOL = S_XOH + 4 * 64 * 8;
constexpr int VS_BYTES = DV * PT * 2;
constexpr int S_VS = S_XOL + 4 * 64 * 8;           // bf16 [buffer][DV][PT] V^T hi
constexpr int S_VSL = S_VS + 2 * VS_BYTES;         // lo (fp32 inputs)
constexpr int SMEM_SCAN_BF16 = S_VSL;
constexpr int SMEM_SCAN_F32 = S_VSL + 2 * VS_BYTES;
static_assert(SMEM_SCAN_F32 <= 64 * 1024, "default dynamic LDS limit");

struct ScanArgs {
    const void* v;
    const float* s0;
    float* s1;
    void* y;
    const char* ws;
    int T, H, H_kv, BH, nch;
    float y_scale;
};

// 4 consecutive elements of one token row.
template <typename Tin> struct Row4;
template <> struct Row4<bf16_t> {
    uint2 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t d = e < 2 ? x.x : x.y;
        return (e & 1) ? __uint_as_float(d & 0xffff0000u) : __uint_as_float(d << 16);
    }
};
template <> struct Row4<float> {
    uint4 x;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        return __uint_as_float(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w);
    }
};

// As pair_col_store for 4 rows: the even lane writes row0, row0 + 1, the odd lane
// row0 + 2, row0 + 3.
__device__ __forceinline__ void pair_col_store4(char* base, int row0, int t, const uint32_t (&v)[2]) {
    const uint32_t pv0 = dpp_u32_xor1(v[0]), pv1 = dpp_u32_xor1(v[1]);
    const bool odd = t & 1;
    const int ocol = pairpos(t & ~1);
    const uint32_t own = odd ? v[1] : v[0], oth = odd ? pv1 : pv0;
    #pragma unroll
    for (int xx = 0; xx < 2; ++xx) {
        const uint32_t own16 = xx ? own >> 16 : own & 0xffffu;
        const uint32_t oth16 = xx ? oth >> 16 : oth & 0xffffu;
        const uint32_t word = odd ? (oth16 | (own16 << 16)) : (own16 | (oth16 << 16));
        sts<uint32_t>(base, ((row0 + (odd ? 2 : 0) + xx) * PT + ocol) * 2, word);
    }
}

// One chunk's workspace operands as this wave loads them.
struct Ops {
    bf16x8 W[2], Qh[2], Ql[2], Bh[2], Eh[2], El[2], Ph, Pl;
    f32x4 d[2], bon;
};

template <typename Tin, typename Ty, bool EPI>
__global__ __launch_bounds__(NTHR_SCAN)
void scan128_kernel(ScanArgs g) {
    constexpr bool VSPLIT = sizeof(Tin) == 4;
    constexpr uint32_t SI = sizeof(Tin), SY = sizeof(Ty);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // Workgroup -> (b, h, value slice q); the 4 slices of a (b, h) are 8 ids apart.
    const int gid = blockIdx.x;
    const int q = (gid >> 3) & (NSLICE - 1);
    const int bh = (gid & 7) + 8 * (gid >> 5);
    if (bh >= g.BH) return;
    const int tid = threadIdx.x;
    const int kp = __builtin_amdgcn_readfirstlane(tid >> 6);   // key pair of this wave
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
    const int H = g.H, T = g.T, nch = g.nch;
    const int bb = bh / H, h = bh - bb * H, hk = h / (H / g.H_kv);
    const uint32_t stkv = uint32_t(g.H_kv) * DK * SI, sty = uint32_t(H) * DK * SY;
    const int64_t tok0 = int64_t(bb) * T;
    const char* recs = g.ws + int64_t(bh) * nch * WS_CHUNK;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // State tiles ST[sg][u][r] = S[32 q + 16 sg + lr][16 (2 kp + u) + 4 lq + r]: the
    // C layout of S^T, i.e. B operands of S^T with the key axis as k.
    const int64_t sbase = int64_t(bh) * DK * DK;
    f32x4 ST[2][2];
    #pragma unroll
    for (int sg = 0; sg < 2; ++sg)
        #pragma unroll
        for (int u = 0; u < 2; ++u)
            ST[sg][u] = g.s0 ? ld_f32x4(reinterpret_cast<const char*>(
                                   g.s0 + sbase + int64_t(DV * q + 16 * sg + lr) * DK + 16 * (2 * kp + u) + 4 * lq))
                             : zero;

    // This wave finishes Y tile (token block ty, value strip sy) and X tile 2 ty + sy.
    const int ty = kp >> 1, sy = kp & 1;
    // The next chunk's operands are requested in three groups spread over the
    // chunk (when every wave of the chip issues them at once the memory pipeline
    // backs up and the issuing waves stall): W and Q (first needed), Bh and E,
    // then P, d and the bonus.
    auto load_wq = [&](int c, Ops& o) {
        const char* kb = recs + int64_t(c) * WS_CHUNK + kp * WS_KP + l * 16;
        #pragma unroll
        for (int i = 0; i < 2; ++i) {
            o.W[i] = *reinterpret_cast<const bf16x8*>(kb + (BLK_W + i) * WS_BLK);
            o.Qh[i] = *reinterpret_cast<const bf16x8*>(kb + (BLK_QH + i) * WS_BLK);
            o.Ql[i] = *reinterpret_cast<const bf16x8*>(kb + (BLK_QL + i) * WS_BLK);
        }
    };
    auto load_be = [&](int c, Ops& o) {
        const char* kb = recs + int64_t(c) * WS_CHUNK + kp * WS_KP + l * 16;
        #pragma unroll
        for (int i = 0; i < 2; ++i) {
            o.Bh[i] = *reinterpret_cast<const bf16x8*>(kb + (BLK_BH + i) * WS_BLK);
            o.Eh[i] = *reinterpret_cast<const bf16x8*>(kb + (BLK_EH + i) * WS_BLK);
            o.El[i] = *reinterpret_cast<const bf16x8*>(kb + (BLK_EL + i) * WS_BLK);
        }
    };
    auto load_p = [&](int c, Ops& o) {   // P, d and the bonus
        const char* rec = recs + int64_t(c) * WS_CHUNK;
        o.Ph = *reinterpret_cast<const bf16x8*>(rec + WS_P + ty * WS_BLK + l * 16);
        o.Pl = *reinterpret_cast<const bf16x8*>(rec + WS_P + (2 + ty) * WS_BLK + l * 16);
        #pragma unroll
        for (int i = 0; i < 2; ++i) o.d[i] = ld_f32x4(rec + WS_D + (16 * (2 * kp + i) + 4 * lq) * 4);
        if constexpr (EPI) o.bon = ld_f32x4(rec + WS_BON + (16 * ty + 4 * lq) * 4);
    };
    auto load_ops = [&](int c, Ops& o) {
        load_wq(c, o);
        load_be(c, o);
        load_p(c, o);
    };
    // V of the slice: thread (vt, vg) loads token vt, values 32 q + 4 vg .. + 3.
    const char* vp = static_cast<const char*>(g.v);
    const int vt = tid & 31, vg = tid >> 5;
    Row4<Tin> vrow;
    auto load_v = [&](int c) {
        vrow.load(chunk_rsrc(vp, tok0, c * L, T, stkv), uint32_t(vt) * stkv + uint32_t(hk * DK + DV * q + 4 * vg) * SI);
    };
    auto store_v = [&](int buf) {   // V^T [i][t~] of the slice
        uint32_t vh[2], vl[2];
        #pragma unroll
        for (int e = 0; e < 4; e += 2) {
            if constexpr (VSPLIT) split2(vrow.get(e), vrow.get(e + 1), vh[e / 2], vl[e / 2]);
            else vh[e / 2] = pack_bf16(vrow.get(e), vrow.get(e + 1));
        }
        pair_col_store4(smem + S_VS + buf * VS_BYTES, 4 * vg, vt, vh);
        if constexpr (VSPLIT) pair_col_store4(smem + S_VSL + buf * VS_BYTES, 4 * vg, vt, vl);
    };

    char* yp = static_cast<char*>(g.y);
    // One chunk: operands in `cur`, the next chunk's prefetched into `nxt`.  The
    // loop below alternates two operand sets, so no prefetched register is copied
    // (a copy would wait for the load); each load is waited for at its first use.
    auto chunk = [&](const int c, Ops& cur, Ops& nxt) {
        const int c0 = c * L, buf = c & 1;
        // Next chunk: V rows first (their LDS store closes this iteration), then W, Q.
        // The last iteration loads its own chunk again (unused): unconditional loads
        // keep the compiler's wait counts exact.
        const int cn = min(c + 1, nch - 1);
        load_v(cn);
        load_wq(cn, nxt);
        asm volatile("" ::: "memory");
        // X and Y over this wave's 32 keys: X^T (t x i) = W S^T, Y (t x i) = Q S^T.
        bf16x8 SBh[2], SBl[2];
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg) to_operand2(ST[sg][0], ST[sg][1], SBh[sg], SBl[sg]);
        #pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            #pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                f32x4 xp = mfma32(cur.W[tb], SBh[sg], zero);
                xp = mfma32(cur.W[tb], SBl[sg], xp);
                f32x4 yq = mfma32(cur.Qh[tb], SBh[sg], zero);
                yq = mfma32(cur.Qh[tb], SBl[sg], yq);
                yq = mfma32(cur.Ql[tb], SBh[sg], yq);
                sts<f32x4>(smem + S_PART, ((kp * 8 + 2 * tb + sg) * 64 + l) * 16, xp);
                sts<f32x4>(smem + S_PART, ((kp * 8 + 4 + 2 * tb + sg) * 64 + l) * 16, yq);
            }
        __syncthreads();   // partial tiles and V^T of this chunk visible
        load_be(cn, nxt);
        asm volatile("" ::: "memory");
        // Keep the S diag(d) update below this point (d is among the last operands to
        // arrive; hoisted to the top of the chunk it would wait for them there).
        asm volatile("" : "+v"(ST[0][0]), "+v"(ST[0][1]), "+v"(ST[1][0]), "+v"(ST[1][1]));

        const char* vs = smem + S_VS + buf * VS_BYTES;
        bf16x8 VB[2], VBl[2];
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            VB[sg] = lds<bf16x8>(vs, ((16 * sg + lr) * PT + 8 * lq) * 2);
            if constexpr (VSPLIT) VBl[sg] = lds<bf16x8>(smem + S_VSL + buf * VS_BYTES, ((16 * sg + lr) * PT + 8 * lq) * 2);
        }
        // S <- S diag(d) + V^T E (the X-independent part of the update).
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg)
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 acc = ST[sg][u] * cur.d[u];
                acc = mfma32(cur.Eh[u], VB[sg], acc);
                acc = mfma32(cur.El[u], VB[sg], acc);
                if constexpr (VSPLIT) acc = mfma32(cur.Eh[u], VBl[sg], acc);
                ST[sg][u] = acc;
            }
        // Reduce X tile kp over the four key pairs -> bf16 hi / lo operand tile.
        {
            f32x4 xs = lds<f32x4>(smem + S_PART, (kp * 64 + l) * 16);
            #pragma unroll
            for (int k2 = 1; k2 < 4; ++k2) xs += lds<f32x4>(smem + S_PART, ((k2 * 8 + kp) * 64 + l) * 16);
            s16x4 xh, xl;
            to_operand(xs, xh, xl);
            sts<s16x4>(smem + S_XOH, (kp * 64 + l) * 8, xh);
            sts<s16x4>(smem + S_XOL, (kp * 64 + l) * 8, xl);
        }
        // The last operand group, issued before this chunk's y stores: a wait for a
        // load also waits for every store issued before it.
        load_p(cn, nxt);
        asm volatile("" ::: "memory");
        // Y tile (ty, sy) = sum of partials + P V; epilogue; store.
        {
            f32x4 ys = lds<f32x4>(smem + S_PART, ((4 + kp) * 64 + l) * 16);
            #pragma unroll
            for (int k2 = 1; k2 < 4; ++k2) ys += lds<f32x4>(smem + S_PART, ((k2 * 8 + 4 + kp) * 64 + l) * 16);
            // V of strip sy loaded again rather than indexed by the wave-dependent sy.
            const int ov = ((16 * sy + lr) * PT + 8 * lq) * 2;
            const bf16x8 VBy = lds<bf16x8>(vs, ov);
            ys = mfma32(cur.Ph, VBy, ys);
            ys = mfma32(cur.Pl, VBy, ys);
            if constexpr (VSPLIT) ys = mfma32(cur.Ph, lds<bf16x8>(smem + S_VSL + buf * VS_BYTES, ov), ys);
            const int i_loc = 16 * sy + lr, tl0 = 16 * ty + 4 * lq;
            float vtr[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI) {
                const uint2 vr = lds<uint2>(vs, (i_loc * PT + pairpos(tl0)) * 2);
                vtr[0] = lo_f32(vr.x); vtr[1] = hi_f32(vr.x); vtr[2] = lo_f32(vr.y); vtr[3] = hi_f32(vr.y);
                if constexpr (VSPLIT) {
                    const uint2 vl = lds<uint2>(smem + S_VSL + buf * VS_BYTES, (i_loc * PT + pairpos(tl0)) * 2);
                    vtr[0] += lo_f32(vl.x); vtr[1] += hi_f32(vl.x); vtr[2] += lo_f32(vl.y); vtr[3] += hi_f32(vl.y);
                }
            }
            const int nv = max(0, min(T - c0, L));
            const rsrc_t Ry = make_rsrc(yp + (tok0 + c0) * sty, uint32_t(nv) * sty);
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                float yv = ys[r] * g.y_scale;
                if constexpr (EPI) yv = fmaf(cur.bon[r], vtr[r], yv);
                Buf<Ty>::store1(Ry, uint32_t(tl0 + r) * sty + uint32_t(h * DK + DV * q + i_loc) * SY, yv);
            }
        }
        __syncthreads();   // reduced X tiles visible

        // S <- S + X Bh, X of strip sg as the B operand (k = token, n = value row).
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const bf16x8 xh = cat(lds<s16x4>(smem + S_XOH, (sg * 64 + l) * 8), lds<s16x4>(smem + S_XOH, ((2 + sg) * 64 + l) * 8));
            const bf16x8 xl = cat(lds<s16x4>(smem + S_XOL, (sg * 64 + l) * 8), lds<s16x4>(smem + S_XOL, ((2 + sg) * 64 + l) * 8));
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 acc = mfma32(cur.Bh[u], xh, ST[sg][u]);
                ST[sg][u] = mfma32(cur.Bh[u], xl, acc);
            }
        }
        // V^T of chunk c + 1 into the other buffer (last read during chunk c - 1); the
        // barrier after the next chunk's partial products publishes it.
        store_v(buf ^ 1);
    };
    Ops opa, opb;
    load_v(0);
    load_ops(0, opa);
    store_v(0);
    // The first operand set completes here: its load order would otherwise enter
    // the compiler's wait counts of every loop iteration.
    #pragma unroll
    for (int i = 0; i < 2; ++i) {
        asm volatile("" : "+v"(opa.W[i]), "+v"(opa.Qh[i]), "+v"(opa.Ql[i]), "+v"(opa.Bh[i]), "+v"(opa.Eh[i]), "+v"(opa.El[i]));
        asm volatile("" : "+v"(opa.d[i]));
    }
    asm volatile("" : "+v"(opa.Ph), "+v"(opa.Pl), "+v"(opa.bon));
    int c = 0;
    for (; c + 1 < nch; c += 2) {
        chunk(c, opa, opb);
        chunk(c + 1, opb, opa);
    }
    if (c < nch) chunk(c, opa, opb);

    if (g.s1) {
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg)
            #pragma unroll
            for (int u = 0; u < 2; ++u)
                *reinterpret_cast<float4*>(g.s1 + sbase + int64_t(DV * q + 16 * sg + lr) * DK + 16 * (2 * kp + u) + 4 * lq) =
                    make_float4(ST[sg][u][0], ST[sg][u][1], ST[sg][u][2], ST[sg][u][3]);
    }
}

template <typename Tin, typename Ty, bool LOGW, bool EPI, bool KK>
hipError_t launch_t(const Params& p, void* ws, hipStream_t stream) {
    const int bh = p.B * p.H, nch = (p.T + L - 1) / L;
    const int items = bh * nch;
    PrepArgs pa{p.r, p.w, p.k, p.a, p.b, p.r_k, p.mask, static_cast<char*>(ws), p.T, p.H, p.H_kv, nch, items};
    auto prep = prep128_kernel<Tin, LOGW, EPI, KK>;
    static bool attr_set = false;   // per template instance; idempotent if raced
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_PREP);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // Persistent: one workgroup per compute unit walks the (b, h, chunk) items.
    const int grid1 = items < kPrepGrid ? items : kPrepGrid;
    hipLaunchKernelGGL(prep, dim3(grid1), dim3(NTHR_PREP), SMEM_PREP, stream, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScanArgs sa{p.v, p.s0, p.s1, p.y, static_cast<const char*>(ws), p.T, p.H, p.H_kv, bh, nch, p.y_scale};
    constexpr int smem2 = sizeof(Tin) == 4 ? SMEM_SCAN_F32 : SMEM_SCAN_BF16;
    // 32 workgroups per group of 8 (b, h): 8 heads x 4 value slices.
    const unsigned groups = unsigned((bh + 7) / 8);
    hipLaunchKernelGGL((scan128_kernel<Tin, Ty, EPI>), dim3(groups * 32u), dim3(NTHR_SCAN), smem2, stream, sa);
    return hipGetLastError();
}

template <typename Tin, typename Ty, bool KK>
hipError_t dispatch_epi(const Params& p, void* ws, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_t<Tin, Ty, true, true, KK>(p, ws, s) : launch_t<Tin, Ty, true, false, KK>(p, ws, s);
    return epi ? launch_t<Tin, Ty, false, true, KK>(p, ws, s) : launch_t<Tin, Ty, false, false, KK>(p, ws, s);
}

template <typename Tin, typename Ty>
hipError_t dispatch_modes(const Params& p, void* ws, hipStream_t s) {
    return p.ab_mode == WKV7_AB_FROM_K ? dispatch_epi<Tin, Ty, true>(p, ws, s) : dispatch_epi<Tin, Ty, false>(p, ws, s);
}

}  // namespace

int64_t twopass128_workspace_bytes(int B, int H, int T) {
    return int64_t(B) * H * ((int64_t(T) + L - 1) / L) * WS_CHUNK;
}

hipError_t launch_twopass128(const Params& p, void* ws, hipStream_t stream) {
    if (p.D != DK || p.chunk_len != L) return hipErrorInvalidValue;
    if (int64_t(L) * p.H * DK * 4 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<bf16_t, bf16_t>(p, ws, stream) : dispatch_modes<bf16_t, float>(p, ws, stream);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<float, bf16_t>(p, ws, stream) : dispatch_modes<float, float>(p, ws, stream);
}

}  // namespace wkv7
