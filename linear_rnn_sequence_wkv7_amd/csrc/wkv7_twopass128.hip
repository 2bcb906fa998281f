// Two-pass chunked WKV-7 forward for head size D = 128 on gfx950 matrix cores
// (fp32 accumulation): pass 1 here on bf16 operands, pass 2 in
// wkv7_twopass128_scan.hip on fp16 operands.
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
// workspace, as fp16, in the exact lane order of the matrix-core operands that
// pass 2 loads.  Pass 2 (scan) runs the chunk recurrence: per chunk four products
// against the state and two small ones, with no L x L algebra left on the
// sequential path.  Four workgroups per (b, h) each own 32 value rows; their
// ids are 8 apart, so under round-robin dispatch they share one XCD's L2 and
// the workspace records they all read are fetched from HBM once.
//
// Operand conventions as in the one-pass kernels: bf16 hi + lo splits where
// a rounding would decide the result, 32-deep contraction axes stored
// pair-interleaved (position 8 q + 4 e + r of a 32-block holds index
// 16 e + 4 q + r), and every accumulator chain uses the single 16x16x32 bf16
// opcode (never a result of one MFMA opcode as the accumulator of another; pass
// 2's fp16 opcode lives in its own kernel and source).  The L x L products keep
// bf16 because their scaled operands (b, k times 2^-g) exceed fp16's range.
//
// Only pass 1 reads r, w, k, a, b, so both input options live there.  A
// masked token is the identity token (r, k, a, b = 0, decay 1): its rows and
// columns of every per-chunk matrix vanish, so pass 2 adds nothing for it and
// outputs y = 0.  Kernel vectors from k (KK): the a slot carries alpha; each
// row thread reduces |k|^2 over its 8 keys, the 16 threads of a token meet in
// LDS (one extra barrier inside the scaling step), and the operands take
// a = -kk, b = kk alpha and k (1 - decay + alpha) in place of the inputs.
#include <mutex>

#include "wkv7_twopass128.h"

namespace wkv7 {
namespace tp128 {
namespace {

constexpr int PK = 136;        // bf16 pitch of [L][DK] token-major operands
constexpr int PD = 20;         // bf16 pitch of a 16 x 16 block
constexpr int MATK = L * PK * 2;
constexpr int MATT = DK * PT * 2;
constexpr int MATL = L * PT * 2;

// Workspace record stores: written once here, read once by the recurrence pass.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_rec(char* p, const f16x8 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_rec(char* p, const uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
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
// row0 + 4 .. row0 + 7, each a 32-bit pair of the two tokens (even token low).
// Each lane sends its partner the two words the partner writes, then forms its
// own words with one byte permute each (v_perm_b32: bytes 0..3 of the second
// source, 4..7 of the first; sel[h] takes half h of both words, in the order
// that puts the even token low).
struct PairSel {
    uint32_t sel[2];
    __device__ __forceinline__ explicit PairSel(int t) {
        const bool odd = t & 1;
        sel[0] = odd ? 0x01000504u : 0x05040100u;
        sel[1] = odd ? 0x03020706u : 0x07060302u;
    }
};
__device__ __forceinline__ void pair_col_store(char* base, int row0, int t, const uint32_t (&v)[4], const PairSel& ps) {
    const bool odd = t & 1;
    const int ocol = pairpos(t & ~1);
    #pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t own = odd ? v[2 + k] : v[k];
        const uint32_t oth = dpp_u32_xor1(odd ? v[k] : v[2 + k]);
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = row0 + (odd ? 4 : 0) + 2 * k + h;
            sts<uint32_t>(base, (row * PT + ocol) * 2, __builtin_amdgcn_perm(oth, own, ps.sel[h]));
        }
    }
}


// ============================== pass 1: per-chunk matrices ==============================

// LDS map of pass 1 (bytes).  Token-major operands (key axis pair-interleaved):
// At, Bt, Kt hi / lo, Rt hi / lo.  Key-major (token axis pair-interleaved):
// At^T, Bh^T.  L x L matrices: A_rb [t][s~], A_ak^T hi / lo [s][t~], A_rk hi / lo
// [t][s], Dinv hi / lo [t][s~], U^T hi / lo [s'][s~] (~: pair-interleaved).
// Areas are reused once their contents are dead, so that two workgroups fit
// in one compute unit's LDS: At and Bt are read in the L x L phase only, after
// which their area holds At^T and U^T; Rt is last read in the D10 step (the
// part that Q adds is read into registers there), after which its area holds
// Bh^T; the |k|^2 partials' area holds D1^T for the block inverse.  (At is read
// back by its row threads for the key-major copy; Bh stays in their registers
// until its area is free.)
constexpr int P_AT = 0;
constexpr int P_BT = P_AT + MATK;
constexpr int P_KTH = P_BT + MATK;
constexpr int P_KTL = P_KTH + MATK;
constexpr int P_RTH = P_KTL + MATK;
constexpr int P_RTL = P_RTH + MATK;
constexpr int P_ARB = P_RTL + MATK;
constexpr int P_AKTH = P_ARB + MATL;
constexpr int P_AKTL = P_AKTH + MATL;
constexpr int P_ARKH = P_AKTL + MATL;
constexpr int P_ARKL = P_ARKH + MATL;
constexpr int P_DIH = P_ARKL + MATL;
constexpr int P_DIL = P_DIH + MATL;
constexpr int P_D0T = P_DIL + MATL;              // D0^T hi / lo, [16][PD] each
constexpr int P_DL = P_D0T + 2 * 16 * PD * 2;    // fp32 [DK] 2^g_L
constexpr int P_BON = P_DL + DK * 4;             // fp32 [8 waves][L] bonus partials
constexpr int P_KSQ = P_BON + 8 * L * 4;         // fp32 [L][8 waves] |k|^2 partials (KK)
constexpr int SMEM_PREP = P_KSQ + L * 8 * 4;
// Reused areas.
constexpr int P_ATT = P_AT;                      // from the D10 step on
constexpr int P_UTH = P_ATT + MATT;              // from the U, W, Q phase on
constexpr int P_UTL = P_UTH + MATL;
constexpr int P_BHT = P_RTH;                     // from the U, W, Q phase on
constexpr int P_D1T = P_KSQ;                     // fp32 16 x 16, L x L phase to the D10 step
static_assert(P_UTL + MATL <= P_KTH && P_BHT + MATT <= P_ARB && 16 * 16 * 4 <= L * 8 * 4, "reused areas");
static_assert(2 * SMEM_PREP <= 160 * 1024, "two workgroups per compute unit");
static_assert(P_ATT % 16 == 0 && P_ARB % 16 == 0 && P_D0T % 16 == 0 && P_DL % 16 == 0, "alignment");

constexpr int NTHR_PREP = 512;   // one workgroup per (b, h, chunk) item; two fit in a compute unit

struct PrepArgs {
    const void *r, *w, *k, *a, *b;
    const float* r_k;
    const uint8_t* mask;
    char* ws;
    // Chunks cb .. cb + nwin - 1 of every (b, h): items = B H nwin; the record of
    // (b h, cb + i) is record b h * nrec + i of the workspace.
    int T, H, H_kv, cb, nwin, nrec, items;
};

template <typename Tin> struct ItemRows {
    Row8<Tin> r, w, k, a, b;
    float rk[8];
    uint32_t m;   // mask byte of the row's token (1 without a mask, 0 past the end)
};

template <typename Tin, bool LOGW, bool EPI, bool KK>
__global__ __launch_bounds__(NTHR_PREP) __attribute__((amdgpu_waves_per_eu(4)))
void prep128_kernel(PrepArgs g) {
    constexpr uint32_t SI = sizeof(Tin);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
    const int H = g.H, T = g.T, nwin = g.nwin;
    const uint32_t stq = uint32_t(H) * DK * SI, stkv = uint32_t(g.H_kv) * DK * SI;
    // Row threads: token t of the chunk, keys j0 .. j0 + 7.
    const int t = l & 31, j0 = 8 * (2 * w + (l >> 5));
    const PairSel psel(t);

    // Items run chunk-major and from the last chunk of the window to the first:
    // the pass that follows starts at the first chunk, so the records it reads
    // first are the ones written last, still in the memory-side cache
    // (1.33 against 1.37 ms per step on the hxa07D workload).
    auto item_pos = [&](int item, int& bh, int& cw) {
        const int nbh = g.items / nwin, q = item / nbh;
        bh = item - q * nbh;
        cw = nwin - 1 - q;
    };
    auto load_item = [&](int item, ItemRows<Tin>& x) {
        int bh, c;
        item_pos(item, bh, c);
        c += g.cb;
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

    ItemRows<Tin> cur;
    // One item per workgroup.  (A persistent loop over items with the next item's
    // rows prefetched needs more than the 128 registers that let two workgroups
    // share a compute unit; the other workgroup covers the load latency instead.)
    const int item = blockIdx.x;
    if (item >= g.items) return;
    {
        load_item(item, cur);
        int bh, cw;
        item_pos(item, bh, cw);
        const int c0 = (g.cb + cw) * L;
        char* rec = g.ws + (int64_t(bh) * g.nrec + cw) * WS_CHUNK;

        uint32_t at[4], bhat[4];   // At and Bh of the row thread's token and keys (bf16 pairs)
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
                // Lane 31 of each 32-lane half to the whole half: swizzle in bit mode,
                // source lane ((lane & 0) | 31) ^ 0.
                dx[x] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(Ex[x]), 31 << 5));
            }
            // KK: the token's |k|^2 from the 8 waves' partials.
            float inv = 0.f;
            if constexpr (KK) {
                __syncthreads();
                const float4 s0 = lds<float4>(smem + P_KSQ, t * 32), s1 = lds<float4>(smem + P_KSQ, t * 32 + 16);
                inv = inv_key_norm(((s0.x + s0.y) + (s0.z + s0.w)) + ((s1.x + s1.y) + (s1.z + s1.w)));
            }
            uint32_t rth[4], rtl[4], bt[4], kth[4], ktl[4];
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
            if (t == 0) {
                sts<float4>(smem + P_DL, j0 * 4, make_float4(dx[0], dx[1], dx[2], dx[3]));
                sts<float4>(smem + P_DL, j0 * 4 + 16, make_float4(dx[4], dx[5], dx[6], dx[7]));
            }
            if constexpr (EPI) {
                bonus_part += __shfl_xor(bonus_part, 32);
                if (l < 32) sts<float>(smem + P_BON, (w * L + t) * 4, bonus_part);
            }
        }
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
            if (w == 1) {   // D1 from A_ab block 1; C(D1^T) to LDS for wave 0
                f32x4 ab2 = zero, nsw1 = zero;
                #pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const bf16x8 B1 = lds<bf16x8>(smem + P_BT, opK(1, kq)), A1 = lds<bf16x8>(smem + P_AT, opK(1, kq));
                    ab2 = mfma32(B1, A1, ab2);
                    nsw1 = mfma32(A1, B1, nsw1);
                }
                const f32x4 Dt1 = chain(ab2, nsw1);
                sts<float4>(smem + P_D1T, (16 * lq + lr) * 16, make_float4(Dt1[0], Dt1[1], Dt1[2], Dt1[3]));
                store_blk(16, 16, Dt1);
            }
            // Wave 1 runs the D1 chain only.  A_rk tiles: waves 2, 3, 6; A_ak (swapped
            // orientation): waves 4, 5, 6; A_rb, all three tiles: wave 7.  (Waves w and
            // w + 4 share a SIMD: the partners of the chain waves 0 and 1 stay light.)
            auto tile_tb = [](int n) { return n == 0 ? 0 : 1; };
            auto tile_sb = [](int n) { return n == 2 ? 1 : 0; };
            auto a_rk = [&](int n) {
                const int tb = tile_tb(n), sb = tile_sb(n);
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
            };
            auto a_ak = [&](int n) {
                const int tb = tile_tb(n), sb = tile_sb(n);
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
                if (n == 2) {
                    // A_ak^T rows s >= 16 at tokens t < 16 are zero (strictly lower).
                    const int oz = ((16 + lr) * PT + pairpos(4 * lq)) * 2;
                    sts<uint2>(smem + P_AKTH, oz, make_uint2(0, 0));
                    sts<uint2>(smem + P_AKTL, oz, make_uint2(0, 0));
                }
            };
            if (w == 2 || w == 3) {
                a_rk(w - 1);
            } else if (w >= 4 && w <= 6) {
                if (w == 6) a_rk(0);
                a_ak(w - 4);
            } else if (w == 7) {
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
        {
            // The row thread's own At values, read back for the key-major copy below
            // (cheaper than keeping them in registers through this phase).
            const int o = (t * PK + pairpos(j0)) * 2;
            const uint2 a01 = lds<uint2>(smem + P_AT, o), a23 = lds<uint2>(smem + P_AT, o + 16);
            at[0] = a01.x; at[1] = a01.y; at[2] = a23.x; at[3] = a23.y;
        }
        __syncthreads();
        if (w == 0) {
            // C(D10^T) = prod(C(T), C(D1^T)) = C(T^T D1^T): lane holds D10[lr][4 lq + r].
            const float4 x = lds<float4>(smem + P_D1T, (16 * lq + lr) * 16);
            store_blk(16, 0, prod(Tm, f32x4{x.x, x.y, x.z, x.w}));
        }
        // Key-major copy of At into the At / Bt area (read for the last time above).
        pair_col_store(smem + P_ATT, j0, t, at, psel);
        // The Rt values this wave adds to Q below, read now so that the Rt area is
        // free from the next barrier on (Bh^T goes there).
        uint2 rtq[2][2];   // [u][hi, lo]
        {
            const int kp = w >> 1, tb = w & 1;
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int orow = ((16 * tb + lr) * PK + pairpos(16 * (2 * kp + u) + 4 * lq)) * 2;
                rtq[u][0] = lds<uint2>(smem + P_RTH, orow);
                rtq[u][1] = lds<uint2>(smem + P_RTL, orow);
            }
        }
        __syncthreads();

        // ---------------- Q2: U = Dinv A_ak; W and Q for key pair kp, token block tb ----------------
        // Key-major copy of Bh into the Rt area (read for the last time above); read
        // in Q3, after this phase's barrier.
        pair_col_store(smem + P_BHT, j0, t, bhat, psel);
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
                st_rec(rec + kp * WS_KP + (BLK_W + tb) * WS_BLK + l * 16, to_f16x8(wt[0], wt[1]));
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
                const uint2 rh = rtq[u][0], rl = rtq[u][1];
                f32x4 acc = {lo_f32(rh.x) + lo_f32(rl.x), hi_f32(rh.x) + hi_f32(rl.x),
                             lo_f32(rh.y) + lo_f32(rl.y), hi_f32(rh.y) + hi_f32(rl.y)};
                acc = mfma32(cat(wh[0][u], wh[1][u]), Ar8, acc);
                acc = mfma32(cat(wl[0][u], wl[1][u]), Ar8, acc);
                qt[u] = acc;
            }
            st_rec(rec + kp * WS_KP + (BLK_Q + tb) * WS_BLK + l * 16, to_f16x8(qt[0], qt[1]));
        }
        __syncthreads();

        // ---------------- Q3: E = Kh + U^T Bh and Bh for key tile jt; P; d; bonus ----------------
        {
            const int kp = w >> 1, u = w & 1, jt = 2 * kp + u;
            const bf16x8 Bh8 = lds<bf16x8>(smem + P_BHT, opT(jt));
            {
                // Bh is bf16 here (the operand of E below); fp16 holds each value exactly
                // inside fp16's normal range.
                const uint4 b4 = __builtin_bit_cast(uint4, Bh8);
                st_rec(rec + kp * WS_KP + (BLK_BH + u) * WS_BLK + l * 16,
                    make_uint4(pack_f16(lo_f32(b4.x), hi_f32(b4.x)), pack_f16(lo_f32(b4.y), hi_f32(b4.y)),
                               pack_f16(lo_f32(b4.z), hi_f32(b4.z)), pack_f16(lo_f32(b4.w), hi_f32(b4.w))));
            }
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
            st_rec(rec + kp * WS_KP + (BLK_E + u) * WS_BLK + l * 16, to_f16x8(e[0], e[1]));
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
            st_rec(rec + WS_P + 0 * WS_BLK + l * 16, to_f16x8(pt[0], zero));
            st_rec(rec + WS_P + 1 * WS_BLK + l * 16, to_f16x8(pt[1], pt[2]));
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
    }
}


// Runs the chunks in windows of `win` chunks per (b, h): pass 1 then pass 2 for
// each window, the state carried from window to window in `carry` (state_out
// itself when given).  win >= the chunk count is the one-window form.
template <typename Tin, typename Ty, bool LOGW, bool EPI, bool KK>
hipError_t launch_t(const Params& p, void* ws, int win, float* carry, hipStream_t stream) {
    const int bh = p.B * p.H, nch = (p.T + L - 1) / L;
    const int nrec = win < nch ? win : nch;
    auto prep = prep128_kernel<Tin, LOGW, EPI, KK>;
    static bool attr_set = false;   // per template instance; idempotent if raced
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_PREP);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    float* s_carry = p.s1 ? p.s1 : carry;
    for (int cb = 0; cb < nch; cb += nrec) {
        const int nw = nch - cb < nrec ? nch - cb : nrec;
        const bool last = cb + nw == nch;
        // One pass-1 workgroup per item: the grid's work-items must fit in 32 bits (a
        // workspace for that many records would not fit in memory, so this does not
        // bind in practice).
        const int64_t items64 = int64_t(bh) * nw;
        if (items64 * NTHR_PREP > int64_t(0xffffffffu)) return hipErrorInvalidConfiguration;
        const int items = int(items64);
        PrepArgs pa{p.r, p.w, p.k, p.a, p.b, p.r_k, p.mask, static_cast<char*>(ws), p.T, p.H, p.H_kv,
                    cb, nw, nrec, items};
        hipLaunchKernelGGL(prep, dim3(items), dim3(NTHR_PREP), SMEM_PREP, stream, pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ScanArgs sa{p.v, cb == 0 ? p.s0 : s_carry, last ? p.s1 : s_carry, p.y, static_cast<const char*>(ws),
                    p.T, p.H, p.H_kv, bh, cb, cb + nw, nrec, p.y_scale};
        e = launch_scan128(sa, sizeof(Tin) == 4, sizeof(Ty) == 4, EPI, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename Tin, typename Ty, bool KK>
hipError_t dispatch_epi(const Params& p, void* ws, int win, float* carry, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_t<Tin, Ty, true, true, KK>(p, ws, win, carry, s)
                         : launch_t<Tin, Ty, true, false, KK>(p, ws, win, carry, s);
    return epi ? launch_t<Tin, Ty, false, true, KK>(p, ws, win, carry, s)
               : launch_t<Tin, Ty, false, false, KK>(p, ws, win, carry, s);
}

template <typename Tin, typename Ty>
hipError_t dispatch_modes(const Params& p, void* ws, int win, float* carry, hipStream_t s) {
    return p.ab_mode == WKV7_AB_FROM_K ? dispatch_epi<Tin, Ty, true>(p, ws, win, carry, s)
                                       : dispatch_epi<Tin, Ty, false>(p, ws, win, carry, s);
}

}  // namespace
}  // namespace tp128

using namespace tp128;

int64_t twopass128_workspace_bytes(int B, int H, int T) {
    return int64_t(B) * H * ((int64_t(T) + L - 1) / L) * WS_CHUNK;
}

int64_t twopass128_record_bytes() { return WS_CHUNK; }

// ---------------------------- allocation-free variant ----------------------------
//
// The scratch of wkv7_forward_noalloc: a file-scope device array, one copy per
// device, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it names a stand-in, not device memory): the device
// address is looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) char scratch[WKV7_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices] = {};

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

hipError_t noalloc_scratch_init(int device) {
    if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device]) return hipSuccess;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = static_cast<char*>(ptr);
    return hipSuccess;
}

int twopass128_noalloc_window(const Params& p) {
    const int64_t nch = (int64_t(p.T) + L - 1) / L;
    const int64_t carry = p.s1 ? 0 : round256(int64_t(p.B) * p.H * DK * DK * 4);
    const int64_t per_chunk = int64_t(p.B) * p.H * WS_CHUNK;
    if (per_chunk <= 0) return 0;
    const int64_t win = (WKV7_NOALLOC_SCRATCH_BYTES - carry) / per_chunk;
    return int(win < nch ? win : nch);
}

hipError_t launch_twopass128_noalloc(const Params& p, int device, hipStream_t stream) {
    char* base = (device >= 0 && device < kMaxScratchDevices) ? g_scratch_ptr[device] : nullptr;
    const int win = twopass128_noalloc_window(p);
    if (!base || win < 1) return hipErrorInvalidValue;
    // [state carry when state_out is null][records of one window]
    const int64_t carry = p.s1 ? 0 : round256(int64_t(p.B) * p.H * DK * DK * 4);
    return launch_twopass128(p, base + carry, win, p.s1 ? nullptr : reinterpret_cast<float*>(base), stream);
}

hipError_t launch_twopass128(const Params& p, void* ws, int win_chunks, float* carry, hipStream_t stream) {
    if (p.D != DK || p.chunk_len != L || win_chunks < 1) return hipErrorInvalidValue;
    if (int64_t(L) * p.H * DK * 4 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const int nch = (p.T + L - 1) / L;
    if (win_chunks < nch && !p.s1 && !carry) return hipErrorInvalidValue;
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<bf16_t, bf16_t>(p, ws, win_chunks, carry, stream)
                                      : dispatch_modes<bf16_t, float>(p, ws, win_chunks, carry, stream);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<float, bf16_t>(p, ws, win_chunks, carry, stream)
                                  : dispatch_modes<float, float>(p, ws, win_chunks, carry, stream);
}

}  // namespace wkv7
