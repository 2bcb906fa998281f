// Backward of the WKV-7 recurrence on gfx950: the gradients of
// L = <dy, y> + <dS_T, S_T> with respect to r, w, k, v, a, b, the initial
// state and the epilogue's r_k.
//
// No page gives these formulas.  They are the reverse-mode derivative of the
// chunk form the forward kernels use (unrolling S_t = S_{t-1}(diag(w_t) +
// a_t b_t^T) + v_t k_t^T over a chunk of L tokens from S0; wiki note "RWKV-7
// Goose", generalised delta rule).  With g_t the chunk-local cumulative
// log2-decay per key column, Rt = r 2^g, At = a 2^g_(t-1), Bt = b 2^-g,
// Kt = k 2^-g, d = 2^g_L and
//
//   A_ab = stril(At Bt^T), A_ak = stril(At Kt^T), A_rb = tril(Rt Bt^T), A_rk = tril(Rt Kt^T)
//   SA  = Dinv (At S0^T + A_ak V),   Dinv = (I - A_ab)^-1
//   Y   = Rt S0^T + A_rb SA + A_rk V
//   S_L = (S0 + SA^T Bt + V^T Kt) diag(d)
//
// the chunk's backward, given dY and U = dL/dS_L, is (dM = U diag(d))
//
//   dSA = Bt dM^T + A_rb^T dY,   dZ = Dinv^T dSA
//   dS0 = dM + dY^T Rt + dZ^T At                        (carried to the previous chunk)
//   dV  = Kt dM^T + A_rk^T dY + A_ak^T dZ
//   dA_rb = tril(dY SA^T), dA_rk = tril(dY V^T), dA_ab = stril(dZ SA^T), dA_ak = stril(dZ V^T)
//   dRt = dY S0 + dA_rb Bt + dA_rk Kt        dAt = dZ S0 + dA_ab Bt + dA_ak Kt
//   dBt = SA dM + dA_ab^T At + dA_rb^T Rt    dKt = V dM + dA_ak^T At + dA_rk^T Rt
//
// and dr = dRt 2^g, da = dAt 2^g_(t-1), db = dBt 2^-g, dk = dKt 2^-g.  The
// decay enters only through the 2^(+-g) factors and the final diag(d), so the
// gradient of each log-decay is a suffix sum within the chunk:
// dL/dlog w_s = sum_(t >= s) [Rt dRt + At_(t+1) dAt_(t+1) - Bt dBt - Kt dKt]_t
// + diag(S_L^T U) (at the chunk's last token).
//
// Every row of the state (value index) evolves on its own, so the value axis
// is processed in slices of 32 rows: the key-axis matrices of a chunk are
// built once and each slice adds its share to the key-axis gradients.
//
// Mapping: 512-thread workgroups, P per (b, h), each owning a group of the
// 32-row value slices (P grows while B H P <= 256, so that small B H still
// fills the chip).  A forward sweep over the chunks stores the group's rows of
// the state at every chunk boundary (fp32, in the workspace); the backward
// sweep walks the chunks in reverse with the group's rows of U = dL/dS in the
// workspace too, one slice at a time.  Rows of S, U, dS0 and columns of dV
// belong to one group; the key-axis gradients are sums over all slices, so
// groups 1 .. P - 1 write their shares to workspace slots that a reduce kernel
// adds to group 0's in group order.  All
// products run on v_mfma_f32_16x16x4f32 with fp32 operands staged in LDS
// (lane l: A[l & 15][l >> 4], B[l >> 4][l & 15], C[4 (l >> 4) + r][l & 15]).
// Masked tokens and tokens past the end are identity tokens (r, k, a, b, v,
// dy = 0, decay 1); their gradients are written as zero.
#include "wkv7_internal.h"
#include "wkv7_device.h"

namespace wkv7 {
namespace {

constexpr int BL = 32;        // chunk length
constexpr int BSL = 32;       // value rows per slice
constexpr int BNT = 512;      // threads per workgroup
constexpr int PL = BL + 1;    // LDS row pitch of [*][32] matrices (floats)

struct BwdArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;
    const float* r_k;
    const uint8_t* mask;
    const void* dy;
    const float* ds1;
    float *dr, *dw, *dk, *dv, *da, *db;   // dk, dv per query head: [B, T, H, D]
    float* ds0;
    float* drk;                            // [B, H, D] partial sums (EPI)
    float* ckpt;                           // [B H][nch + 1][D][D] states at the chunk boundaries
    float* ubuf;                           // [B H][D][D] dL/dS during the backward sweep
    float* dinv;                           // [P][B H][nch][BL][BL] (I - A_ab)^-1 of every chunk
    float* part;                           // [P - 1][5][B T H D] key-axis gradients of groups 1 ..
    int64_t nq;                            // B T H D
    int B, T, H, H_kv, nch;
    int split;                             // P: value-slice groups (workgroups) per (b, h)
    float y_scale;
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// This lane's position in a 16 x 16 tile: column i = lane & 15, row group q = lane >> 4.
// The kernel hides these values from the optimiser at the top of every chunk, so
// the LDS addresses built from them are recomputed per chunk instead of being
// kept in registers across the whole sweep.
struct LanePos {
    int i, q;
};

// This lane's operands of the k-step k .. k + 4 of a product with tiles at rows m0 / columns n0.
// TA: A is stored [k][m] (else [m][k]); TB: B is stored [n][k] (else [k][n]).
template <bool TA>
__device__ __forceinline__ float opA(const float* A, int lda, int m0, int k, LanePos lp) {
    return TA ? A[(k + lp.q) * lda + m0 + lp.i] : A[(m0 + lp.i) * lda + k + lp.q];
}
template <bool TB>
__device__ __forceinline__ float opB(const float* B, int ldb, int n0, int k, LanePos lp) {
    return TB ? B[(n0 + lp.i) * ldb + k + lp.q] : B[(k + lp.q) * ldb + n0 + lp.i];
}

// acc += op(A)[m0 .. m0 + 16, k0 .. k1) x op(B)[k0 .. k1, n0 .. n0 + 16) on LDS matrices.
// Every k-step unrolled, so that the operand reads of the whole product are in flight
// ahead of the accumulator chain (measured against 2 at a time: 0.95-0.97 against
// 1.01-1.02 ms per step at B8 T1024 H32 D64; unchanged, 24.5 ms, at B2 T16384 H32 D128).
template <bool TA, bool TB>
__device__ __forceinline__ f32x4 mm(const float* A, int lda, const float* B, int ldb, int m0, int n0,
                                    int k0, int k1, f32x4 acc, LanePos lp) {
    #pragma unroll
    for (int k = k0; k < k1; k += 4) acc = mfma4(opA<TA>(A, lda, m0, k, lp), opB<TB>(B, ldb, n0, k, lp), acc);
    return acc;
}

// Store a C tile to an LDS matrix [row][ld]; `keep(row, col)` masks elements to zero.
template <typename F>
__device__ __forceinline__ void st_tile(float* C, int ld, int m0, int n0, f32x4 acc, LanePos lp, F keep) {
    const int i = lp.i, q = lp.q;
    #pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = m0 + 4 * q + rr, col = n0 + i;
        C[row * ld + col] = keep(row, col) ? acc[rr] : 0.f;
    }
}

constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};

// Raw bits of one input element (a bf16 pattern zero-extended, or fp32 bits): loads
// issued ahead of their use stay unconverted, so nothing waits for them until then.
__device__ __forceinline__ uint32_t ld_raw(const bf16_t* p, int64_t i) { return uint32_t(p[i]); }
__device__ __forceinline__ uint32_t ld_raw(const float* p, int64_t i) { return __float_as_uint(p[i]); }
__device__ __forceinline__ float from_raw(uint32_t x, const bf16_t*) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float from_raw(uint32_t x, const float*) { return __uint_as_float(x); }

// N consecutive input elements starting at p (N * sizeof(T) a multiple of 8 bytes and
// p aligned to it) as raw 32-bit words: bf16 pairs packed, fp32 one per word.
template <int N, typename T>
__device__ __forceinline__ void ld_vec_raw(const T* p, uint32_t* o) {
    constexpr int NW = N * int(sizeof(T)) / 4;
    static_assert(NW % 2 == 0, "whole 8-byte loads");
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    if constexpr (NW % 4 == 0) {
        #pragma unroll
        for (int i = 0; i < NW; i += 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(q + i);
            o[i] = x.x; o[i + 1] = x.y; o[i + 2] = x.z; o[i + 3] = x.w;
        }
    } else {
        #pragma unroll
        for (int i = 0; i < NW; i += 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(q + i);
            o[i] = x.x; o[i + 1] = x.y;
        }
    }
}
// Element e of such a word array.
__device__ __forceinline__ float vec_elem(const uint32_t* o, int e, const bf16_t*) {
    const uint32_t x = o[e >> 1];
    return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
}
__device__ __forceinline__ float vec_elem(const uint32_t* o, int e, const float*) { return __uint_as_float(o[e]); }

template <int D, typename Tin, typename Tdy, bool LOGW, bool EPI>
__global__ __launch_bounds__(BNT) void bwd_kernel(BwdArgs g) {
    constexpr int PD = D + 1;            // LDS row pitch of [*][D] matrices
    constexpr int NS = D / BSL;          // value slices
    constexpr int TC = D / 16;           // column tiles of a [*][D] matrix
    constexpr int NU = TC / 4;           // tiles per wave of one slice: (2 row tiles x TC) / 8 waves
    constexpr int NA = (2 * TC) / 8;     // tiles per wave of one [32][D] matrix
    constexpr int UNI = (2 * BSL * PD > 4 * BL * PL) ? 2 * BSL * PD : 4 * BL * PL;
    constexpr int FU = D == 64 ? 2 : 1;   // unroll of the fused k-loops
    // At D = 128 a group's first slice of a chunk is fetched together with the chunk's
    // inputs (faster there: hxa07D runs one slice per group); at D = 64 each slice is
    // fetched at its start (faster there).
    constexpr bool PF0 = D == 128;
    static_assert(BSL == BL, "slice and chunk share the 32-wide LDS pitch");
    static_assert(BL * D <= 4 * BL * PL, "the w-derivative table fits VS .. DZS (ZS holds the suffix-sum partials)");

    extern __shared__ __attribute__((aligned(16))) float sm[];
    float* RT = sm;
    float* AT = RT + BL * PD;
    float* BT = AT + BL * PD;
    float* KT = BT + BL * PD;
    float* GG = KT + BL * PD;            // cumulative log2-decay g_t per key column
    float* AAB = GG + BL * PD;
    float* AAK = AAB + BL * PL;
    float* ARB = AAK + BL * PL;
    float* ARK = ARB + BL * PL;
    float* DINV = ARK + BL * PL;
    float* UN = DINV + BL * PL;          // per slice: S0 | dM;  then dA x 4;  then QP | QA
    float* S0S = UN;
    float* DMS = UN + BSL * PD;
    float* QP = UN;
    float* QA = UN + BL * PD;
    float* VS = UN + UNI;
    float* DYS = VS + BL * PL;
    float* SAS = DYS + BL * PL;
    float* DZS = SAS + BL * PL;
    float* ZS = DZS + BL * PL;
    float* DSAS = ZS + BL * PL;
    float* FAC = VS;                     // [BL][D] after the slices: d log w / d(w input)
    float* DD = DSAS + BL * PL;          // [D] diag(S_L^T U)
    float* DEC = DD + D;                 // [D] d = 2^g_L
    float* BETA = DEC + D;               // [BL] r k r_k per token
    float* DBETA = BETA + BL;            // [BL] dy . v per token
    float* DRK = DBETA + BL;             // [D] r_k gradient of this (b, h)

    int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    LanePos lp{lane & 15, lane >> 4};
    // Hide the thread's position from the optimiser (see LanePos).
    auto opaque_pos = [&]() { asm volatile("" : "+v"(tid), "+v"(lp.i), "+v"(lp.q)); };
    const int bh = blockIdx.x;
    // Value-slice group sg of P = g.split: slices [s_begin, s_end) of this (b, h).  The
    // rows of S, U, dS0 and the columns of dV split with no overlap; the key-axis
    // gradients are this group's share (group 0 writes the outputs, the others their
    // slots in g.part, summed afterwards).
    const int sg = blockIdx.y;
    const int s_begin = sg * (NS / g.split), s_end = s_begin + NS / g.split;
    const int e_begin = s_begin * BSL * D, e_end = s_end * BSL * D;   // this group's state elements
    const int64_t BH = int64_t(g.B) * g.H;
    float* const o_dr = sg == 0 ? g.dr : g.part + (int64_t(sg - 1) * 5 + 0) * g.nq;
    float* const o_da = sg == 0 ? g.da : g.part + (int64_t(sg - 1) * 5 + 1) * g.nq;
    float* const o_db = sg == 0 ? g.db : g.part + (int64_t(sg - 1) * 5 + 2) * g.nq;
    float* const o_dk = sg == 0 ? g.dk : g.part + (int64_t(sg - 1) * 5 + 3) * g.nq;
    float* const o_dw = sg == 0 ? g.dw : g.part + (int64_t(sg - 1) * 5 + 4) * g.nq;
    float* const dinv_g = g.dinv + (int64_t(sg) * BH + bh) * g.nch * BL * BL;
    const int H = g.H, T = g.T, H_kv = g.H_kv;
    const int bb = bh / H, h = bh - bb * H, hk = h / (H / H_kv);
    const Tin* rp = static_cast<const Tin*>(g.r);
    const Tin* wp = static_cast<const Tin*>(g.w);
    const Tin* kp = static_cast<const Tin*>(g.k);
    const Tin* vp = static_cast<const Tin*>(g.v);
    const Tin* ap = static_cast<const Tin*>(g.a);
    const Tin* bp = static_cast<const Tin*>(g.b);
    const Tdy* dyp = static_cast<const Tdy*>(g.dy);
    float* ck = g.ckpt + int64_t(bh) * (g.nch + 1) * D * D;

    auto qidx = [&](int t, int j) { return ((int64_t(bb) * T + t) * H + h) * D + j; };
    auto kvidx = [&](int t, int j) { return ((int64_t(bb) * T + t) * H_kv + hk) * D + j; };
    const uint8_t* mrow = g.mask ? g.mask + int64_t(bb) * T : nullptr;
    // Bit t of `vbits`: token c0 + t of the current chunk is kept (in range, not masked).
    uint32_t vbits = 0;
    auto set_chunk_bits = [&](int c0, uint32_t mbyte) {
        const int t = c0 + (lane & 31);
        const bool ok = t < T && mbyte != 0;
        vbits = uint32_t(__builtin_amdgcn_ballot_w64(ok && lane < BL));
    };
    auto valid = [&](int t_abs) { return ((vbits >> (t_abs & (BL - 1))) & 1u) != 0; };

    // Chunk c: g_t, the scaled key-axis operands and d.  With `with_r`, Rt and the
    // epilogue's r k r_k as well (the backward sweep), the stored Dinv of the chunk
    // and d log w / d(w input) per element (fac).  issue_chunk issues all of the
    // chunk's global loads (raw, into registers); load_chunk then consumes them.
    // Thread tid takes NE consecutive elements of one token row: t = tid / 16,
    // j0 = NE (tid mod 16), one vector load per input.  (Issuing the loads one
    // chunk ahead measured no faster: the issue cost about what the hidden latency
    // saved.)
    constexpr int NE = BL * D / BNT;      // elements of a [BL][D] matrix per thread
    constexpr int NW = NE * int(sizeof(Tin)) / 4;
    static_assert(D / NE == 16, "16 threads per token row");
    const int et = tid >> 4, ej0 = NE * (tid & 15);
    float fac[NE];
    uint32_t wr[NW], ar[NW], br[NW], kr[NW], rr_[NW], mraw;
    float2 dv2;
    auto issue_chunk = [&](int c, bool with_r) {
        const int c0 = c * BL;
        mraw = mrow ? uint32_t(mrow[min(c0 + (lane & 31), T - 1)]) : 1u;
        const int tt = min(c0 + et, T - 1);   // tokens past the end read the last one (unused)
        ld_vec_raw<NE>(wp + qidx(tt, ej0), wr);
        ld_vec_raw<NE>(ap + qidx(tt, ej0), ar);
        ld_vec_raw<NE>(bp + qidx(tt, ej0), br);
        ld_vec_raw<NE>(kp + kvidx(tt, ej0), kr);
        if (with_r) {
            ld_vec_raw<NE>(rp + qidx(tt, ej0), rr_);
            dv2 = *reinterpret_cast<const float2*>(dinv_g + int64_t(c) * BL * BL + 2 * tid);
        }
    };
    auto load_chunk = [&](int c, bool with_r) {
        const int c0 = c * BL;
        set_chunk_bits(c0, mraw);
        const int t = et, o0 = t * PD + ej0;
        const bool ok = valid(c0 + t);
        #pragma unroll
        for (int q = 0; q < NE; ++q) {
            const float wv = vec_elem(wr, q, wp);
            GG[o0 + q] = ok ? log2_decay(wv, LOGW) : 0.f;
            fac[q] = ok ? (LOGW ? -__builtin_amdgcn_exp2f(wv * kLog2e) : 1.f / wv) : 0.f;
        }
        if (with_r) {   // Dinv row 2 tid / 32, columns 2 tid mod 32 and the next
            DINV[(tid >> 4) * PL + 2 * (tid & 15)] = dv2.x;
            DINV[(tid >> 4) * PL + 2 * (tid & 15) + 1] = dv2.y;
        }
        __syncthreads();
        if (tid < D) {
            float col[BL];
            #pragma unroll
            for (int tq = 0; tq < BL; ++tq) col[tq] = GG[tq * PD + tid];
            float run = 0.f;
            #pragma unroll
            for (int tq = 0; tq < BL; ++tq) {
                run += col[tq];
                GG[tq * PD + tid] = run;
            }
            DEC[tid] = __builtin_amdgcn_exp2f(run);
        }
        __syncthreads();
        float rkk = 0.f;   // this thread's share of r . (k r_k) for token t
        #pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int o = o0 + q;
            const float gt = GG[o], gp = t > 0 ? GG[o - PD] : 0.f;
            const float ep = __builtin_amdgcn_exp2f(gt), em = __builtin_amdgcn_exp2f(-gt);
            const float kv = vec_elem(kr, q, kp);
            AT[o] = ok ? vec_elem(ar, q, ap) * __builtin_amdgcn_exp2f(gp) : 0.f;
            BT[o] = ok ? vec_elem(br, q, bp) * em : 0.f;
            KT[o] = ok ? kv * em : 0.f;
            if (with_r) {
                const float rv = vec_elem(rr_, q, rp);
                RT[o] = ok ? rv * ep : 0.f;
                if constexpr (EPI) rkk = fmaf(rv * kv, g.r_k[h * D + ej0 + q], rkk);
            }
        }
        if constexpr (EPI) {
            if (with_r) {   // the row's 16 threads are an aligned group of 16 lanes
                rkk = sum16(rkk);
                if ((tid & 15) == 0) BETA[t] = ok ? rkk : 0.f;
            }
        }
        __syncthreads();
    };

    // L x L matrices.  Forward sweep: A_ab, A_ak and Dinv = (I - A_ab)^-1 (wave 0),
    // stored for the backward sweep.  Backward sweep: A_ak, A_rb, A_rk (Dinv loaded).
    auto build_LL = [&](int c, bool bwd) {
        for (int n = w; n < (bwd ? 12 : 8); n += 8) {
            const int mat = (n >> 2) + (bwd ? 1 : 0), tile = n & 3, m0 = 16 * (tile >> 1), n0 = 16 * (tile & 1);
            const float* A = mat < 2 ? AT : RT;
            const float* B = (mat & 1) ? KT : BT;
            float* C = mat == 0 ? AAB : mat == 1 ? AAK : mat == 2 ? ARB : ARK;
            f32x4 acc = mm<false, true>(A, PD, B, PD, m0, n0, 0, D, kZero4, lp);
            if (mat < 2) st_tile(C, PL, m0, n0, acc, lp, [](int r, int c) { return c < r; });
            else st_tile(C, PL, m0, n0, acc, lp, [](int r, int c) { return c <= r; });
        }
        __syncthreads();
        if (bwd) return;
        if (w == 0) {
            // X = (I - A_ab)^-1 in 16 x 16 blocks.  The diagonal blocks by forward
            // substitution, both at once (lanes 0-15: columns of X11, lanes 16-31: of
            // X22): x_t = [t == col] + sum_(s<t) A_ab[t][s] x_s within the block.  Then
            // X21 = X22 A21 X11 on the matrix cores (the block of I - A_ab below the
            // diagonal is -A21); X12 = 0.
            if (lane < BL) {
                const int r0 = 16 * (lane >> 4), col = lane & 15;
                float x[16];
                #pragma unroll
                for (int t = 0; t < 16; ++t) x[t] = t == col ? 1.f : 0.f;
                #pragma unroll
                for (int s2 = 0; s2 < 16; ++s2) {
                    #pragma unroll
                    for (int t = s2 + 1; t < 16; ++t) x[t] = fmaf(AAB[(r0 + t) * PL + r0 + s2], x[s2], x[t]);
                }
                #pragma unroll
                for (int t = 0; t < 16; ++t) {
                    DINV[(r0 + t) * PL + r0 + col] = x[t];
                    if (r0 == 0) DINV[t * PL + 16 + col] = 0.f;   // X12 (by the X11 lanes)
                }
            }
            // One wave: its LDS accesses take effect in order, no barrier needed.
            const f32x4 tmp = mm<false, false>(AAB, PL, DINV, PL, 16, 0, 0, 16, kZero4, lp);   // A21 X11
            st_tile(DINV, PL, 16, 0, tmp, lp, [](int, int) { return true; });
            const f32x4 x21 = mm<false, false>(DINV, PL, DINV, PL, 16, 0, 16, 32, kZero4, lp);   // X22 (A21 X11)
            st_tile(DINV, PL, 16, 0, x21, lp, [](int, int) { return true; });
            if (lane < BL) {
                float* dg = dinv_g + int64_t(c) * BL * BL;
                #pragma unroll
                for (int t = 0; t < BL; ++t) dg[t * BL + lane] = DINV[t * PL + lane];
            }
        }
        __syncthreads();
    };

    // Tiles of one slice (32 rows x D) of a D x D matrix: this wave's u-th, at local
    // rows ml and columns n0 (tile n = w + 8 u of the slice's 2 x TC tiles).
    auto slice_tile = [&](int u, int& ml, int& n0) {
        const int n = w + 8 * u;
        ml = 16 * (n / TC);
        n0 = 16 * (n % TC);
    };
    float* ub = g.ubuf + int64_t(bh) * D * D;   // U = dL/dS of the backward sweep

    // ------------------------------- forward sweep: checkpoints -------------------------------
    for (int e = e_begin + tid; e < e_end; e += BNT) ck[e] = g.s0 ? g.s0[int64_t(bh) * D * D + e] : 0.f;
    __syncthreads();
    // A slice's rows of a D x D matrix and its [BL][32] value columns, element e = tid + BNT u.
    constexpr int NSE = BSL * D / BNT, NVE = BL * BSL / BNT;
    float ps0[NSE], puu[NSE], psl[NSE];   // one slice's loads, issued together
    uint32_t pvv[NVE], pdy[NVE];          // (raw: converted where used)
    auto fetch_slice = [&](int c, int s, bool bwd) {
        const int c0 = c * BL;
        const float* sc = ck + int64_t(c) * D * D + BSL * s * D;
        #pragma unroll
        for (int u = 0; u < NSE; ++u) {
            const int e = tid + BNT * u;
            ps0[u] = sc[e];
            if (bwd) {
                puu[u] = ub[BSL * s * D + e];
                psl[u] = sc[D * D + e];   // the next boundary: S_L of this chunk
            }
        }
        #pragma unroll
        for (int u = 0; u < NVE; ++u) {
            const int e = tid + BNT * u, t = e / BSL, i = e - t * BSL;
            const int tt = min(c0 + t, T - 1);
            pvv[u] = ld_raw(vp, kvidx(tt, BSL * s + i));
            if (bwd) pdy[u] = ld_raw(dyp, qidx(tt, BSL * s + i));
        }
    };
    for (int c = 0; c < g.nch; ++c) {
        opaque_pos();
        const int c0 = c * BL;
        float* sn = ck + int64_t(c + 1) * D * D;
        issue_chunk(c, false);
        if constexpr (PF0) fetch_slice(c, s_begin, false);   // in flight with the chunk's loads
        load_chunk(c, false);
        build_LL(c, false);
        #pragma unroll 1
        for (int s = s_begin; s < s_end; ++s) {
            if (!PF0 || s != s_begin) fetch_slice(c, s, false);
            #pragma unroll
            for (int u = 0; u < NSE; ++u) {
                const int e = tid + BNT * u;
                S0S[(e / D) * PD + (e % D)] = ps0[u];
            }
            #pragma unroll
            for (int u = 0; u < NVE; ++u) {
                const int e = tid + BNT * u, t = e / BSL, i = e - t * BSL;
                VS[t * PL + i] = valid(c0 + t) ? from_raw(pvv[u], vp) : 0.f;
            }
            __syncthreads();
            if (w < 4) {   // Z = At S0s^T + A_ak Vs
                const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);
                f32x4 acc = mm<false, true>(AT, PD, S0S, PD, m0, n0, 0, D, kZero4, lp);
                acc = mm<false, false>(AAK, PL, VS, PL, m0, n0, 0, BL, acc, lp);
                st_tile(ZS, PL, m0, n0, acc, lp, [](int, int) { return true; });
            }
            __syncthreads();
            if (w < 4) {   // SA = Dinv Z
                const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);
                f32x4 acc = mm<false, false>(DINV, PL, ZS, PL, m0, n0, 0, BL, kZero4, lp);
                st_tile(SAS, PL, m0, n0, acc, lp, [](int, int) { return true; });
            }
            __syncthreads();
            #pragma unroll
            for (int u = 0; u < NU; ++u) {   // S_next = (S + SA^T Bt + V^T Kt) diag(d)
                int ml, n0;
                slice_tile(u, ml, n0);
                f32x4 acc;
                #pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] = S0S[(ml + 4 * lp.q + rr) * PD + n0 + lp.i];
                acc = mm<true, false>(SAS, PL, BT, PD, ml, n0, 0, BL, acc, lp);
                acc = mm<true, false>(VS, PL, KT, PD, ml, n0, 0, BL, acc, lp);
                const float dc = DEC[n0 + lp.i];
                #pragma unroll
                for (int rr = 0; rr < 4; ++rr) sn[(BSL * s + ml + 4 * lp.q + rr) * D + n0 + lp.i] = acc[rr] * dc;
            }
            __syncthreads();
        }
    }

    // ------------------------------- backward sweep -------------------------------
    for (int e = e_begin + tid; e < e_end; e += BNT) ub[e] = g.ds1 ? g.ds1[int64_t(bh) * D * D + e] : 0.f;
    if (EPI && tid < D) DRK[tid] = 0.f;
    // r_k gradient: per-thread partials over all chunks (column j of tile w + 8 u is
    // fixed), added to DRK once at the end.
    float drkp[NA];
    #pragma unroll
    for (int u = 0; u < NA; ++u) drkp[u] = 0.f;
    __syncthreads();
    for (int c = g.nch - 1; c >= 0; --c) {
        opaque_pos();
        const int c0 = c * BL;
        // diag(S_L^T U) and dy . v: per-thread partials over the slices, reduced once per
        // chunk (LDS atomics on a few addresses would serialise).  A thread's column
        // j = tid mod D and its tokens t = (tid + BNT u) / 32 are the same in every slice.
        float ddp = 0.f, dbp[NVE];
        #pragma unroll
        for (int u = 0; u < NVE; ++u) dbp[u] = 0.f;
        issue_chunk(c, true);
        if constexpr (PF0) fetch_slice(c, s_begin, true);    // in flight with the chunk's loads
        load_chunk(c, true);
        build_LL(c, true);

        f32x4 accR[NA], accA[NA], accB[NA], accK[NA], accDA[2];
        #pragma unroll
        for (int u = 0; u < NA; ++u) accR[u] = accA[u] = accB[u] = accK[u] = kZero4;
        accDA[0] = accDA[1] = kZero4;
        // dA tiles of this wave: matrix w >> 1 (rb, rk, ab, ak), tiles 2 (w & 1) + {0, 1}.
        const int dmat = w >> 1;

        #pragma unroll 1
        for (int s = s_begin; s < s_end; ++s) {
            if (!PF0 || s != s_begin) fetch_slice(c, s, true);
            // S0 slice, dM = U diag(d), V and y_scale dy slices; diag(S_L^T U) and dy . v shares.
            #pragma unroll
            for (int u = 0; u < NSE; ++u) {
                const int e = tid + BNT * u, i = e / D, j = e - i * D;
                S0S[i * PD + j] = ps0[u];
                DMS[i * PD + j] = puu[u] * DEC[j];
                ddp = fmaf(psl[u], puu[u], ddp);
            }
            #pragma unroll
            for (int u = 0; u < NVE; ++u) {
                const int e = tid + BNT * u, t = e / BSL, i = e - t * BSL;
                const bool ok = valid(c0 + t);
                const float vv = ok ? from_raw(pvv[u], vp) : 0.f, dyv = ok ? from_raw(pdy[u], dyp) : 0.f;
                VS[t * PL + i] = vv;
                DYS[t * PL + i] = dyv * g.y_scale;
                if constexpr (EPI) dbp[u] = fmaf(dyv, vv, dbp[u]);
            }
            __syncthreads();
            if (w < 4) {   // Z = At S0s^T + A_ak Vs
                const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);
                f32x4 acc = mm<false, true>(AT, PD, S0S, PD, m0, n0, 0, D, kZero4, lp);
                acc = mm<false, false>(AAK, PL, VS, PL, m0, n0, 0, BL, acc, lp);
                st_tile(ZS, PL, m0, n0, acc, lp, [](int, int) { return true; });
            } else {       // dSA = Bt dM^T + A_rb^T dY
                const int m0 = 16 * ((w - 4) >> 1), n0 = 16 * (w & 1);
                f32x4 acc = mm<false, true>(BT, PD, DMS, PD, m0, n0, 0, D, kZero4, lp);
                acc = mm<true, false>(ARB, PL, DYS, PL, m0, n0, 0, BL, acc, lp);
                st_tile(DSAS, PL, m0, n0, acc, lp, [](int, int) { return true; });
            }
            __syncthreads();
            if (w < 4) {   // SA = Dinv Z
                const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);
                f32x4 acc = mm<false, false>(DINV, PL, ZS, PL, m0, n0, 0, BL, kZero4, lp);
                st_tile(SAS, PL, m0, n0, acc, lp, [](int, int) { return true; });
            } else {       // dZ = Dinv^T dSA
                const int m0 = 16 * ((w - 4) >> 1), n0 = 16 * (w & 1);
                f32x4 acc = mm<true, false>(DINV, PL, DSAS, PL, m0, n0, 0, BL, kZero4, lp);
                st_tile(DZS, PL, m0, n0, acc, lp, [](int, int) { return true; });
            }
            __syncthreads();
            // U <- dM + dY^T Rt + dZ^T At for this slice's rows (the two products in
            // independent chains, so that consecutive matrix-core ops do not wait on each other).
            #pragma unroll
            for (int u = 0; u < NU; ++u) {
                int ml, n0;
                slice_tile(u, ml, n0);
                f32x4 acc, acc2 = kZero4;
                #pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] = DMS[(ml + 4 * lp.q + rr) * PD + n0 + lp.i];
                #pragma unroll FU
                for (int k = 0; k < BL; k += 4) {
                    acc = mfma4(opA<true>(DYS, PL, ml, k, lp), opB<false>(RT, PD, n0, k, lp), acc);
                    acc2 = mfma4(opA<true>(DZS, PL, ml, k, lp), opB<false>(AT, PD, n0, k, lp), acc2);
                }
                #pragma unroll
                for (int rr = 0; rr < 4; ++rr) ub[(BSL * s + ml + 4 * lp.q + rr) * D + n0 + lp.i] = acc[rr] + acc2[rr];
            }
            // dV = Kt dM^T + A_rk^T dY + A_ak^T dZ (+ the epilogue's beta dy), this slice's columns.
            if (w < 4) {
                const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);
                f32x4 acc = kZero4, acc2 = kZero4;
                #pragma unroll FU
                for (int k = 0; k < D; k += 8) {
                    acc = mfma4(opA<false>(KT, PD, m0, k, lp), opB<true>(DMS, PD, n0, k, lp), acc);
                    acc2 = mfma4(opA<false>(KT, PD, m0, k + 4, lp), opB<true>(DMS, PD, n0, k + 4, lp), acc2);
                }
                #pragma unroll FU
                for (int k = 0; k < BL; k += 4) {
                    acc = mfma4(opA<true>(ARK, PL, m0, k, lp), opB<false>(DYS, PL, n0, k, lp), acc);
                    acc2 = mfma4(opA<true>(AAK, PL, m0, k, lp), opB<false>(DZS, PL, n0, k, lp), acc2);
                }
                #pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] += acc2[rr];
                #pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int t = m0 + 4 * lp.q + rr, i = BSL * s + n0 + lp.i;
                    if (c0 + t < T) {
                        float x = acc[rr];
                        if (!valid(c0 + t)) x = 0.f;
                        else if constexpr (EPI) x = fmaf(BETA[t], ld1(dyp, qidx(c0 + t, i)), x);
                        g.dv[qidx(c0 + t, i)] = x;
                    }
                }
            }
            // One k-loop over the slice rows for the dA shares (tril(dY SA^T), tril(dY V^T),
            // stril(dZ SA^T), stril(dZ V^T): matrix dmat, tiles at rows 16 (w & 1), columns 0
            // and 16) and for dRt += dY S0, dAt += dZ S0, dBt += SA dM, dKt += V dM, so the
            // matrix-core ops of a step are independent and share their operand reads.
            {
                const float* XA = dmat < 2 ? DYS : DZS;
                const float* XB = (dmat & 1) ? VS : SAS;
                const int ma = 16 * (w & 1);
                #pragma unroll FU
                for (int k = 0; k < BSL; k += 4) {
                    const float xa = opA<false>(XA, PL, ma, k, lp);
                    accDA[0] = mfma4(xa, opB<true>(XB, PL, 0, k, lp), accDA[0]);
                    accDA[1] = mfma4(xa, opB<true>(XB, PL, 16, k, lp), accDA[1]);
                    #pragma unroll
                    for (int u = 0; u < NA; ++u) {
                        const int n = w + 8 * u, m0 = 16 * (n / TC), n0 = 16 * (n % TC);
                        const float s0 = opB<false>(S0S, PD, n0, k, lp), dm = opB<false>(DMS, PD, n0, k, lp);
                        accR[u] = mfma4(opA<false>(DYS, PL, m0, k, lp), s0, accR[u]);
                        accA[u] = mfma4(opA<false>(DZS, PL, m0, k, lp), s0, accA[u]);
                        accB[u] = mfma4(opA<false>(SAS, PL, m0, k, lp), dm, accB[u]);
                        accK[u] = mfma4(opA<false>(VS, PL, m0, k, lp), dm, accK[u]);
                    }
                }
            }
            __syncthreads();
        }
        // The partials to the slice buffers ZS and DSAS (free until the next chunk).
        ZS[tid] = ddp;
        if constexpr (EPI) {
            #pragma unroll
            for (int u = 0; u < NVE; ++u) DSAS[tid + BNT * u] = dbp[u];
        }
        // dA matrices (masked) to LDS.
        {
            float* C = UN + dmat * BL * PL;
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tile = 2 * (w & 1) + u, m0 = 16 * (tile >> 1), n0 = 16 * (tile & 1);
                if (dmat < 2) st_tile(C, PL, m0, n0, accDA[u], lp, [](int r, int c) { return c <= r; });
                else st_tile(C, PL, m0, n0, accDA[u], lp, [](int r, int c) { return c < r; });
            }
        }
        __syncthreads();
        {
            // Reduce the per-thread partials: DD[j] over the threads of column j, DBETA[t]
            // over the 32 entries of token t (read in a rotated order to spread the banks).
            if (tid < D) {
                float sdd = 0.f;
                #pragma unroll
                for (int k = 0; k < BNT / D; ++k) sdd += ZS[tid + D * k];
                DD[tid] = sdd;
            }
            if constexpr (EPI) {
                if (tid >= D && tid < D + BL) {
                    const int t = tid - D;
                    float sb = 0.f;
                    #pragma unroll
                    for (int i = 0; i < BSL; ++i) sb += DSAS[t * BSL + ((i + t) & (BSL - 1))];
                    DBETA[t] = sb;
                }
            }
            const float* DRB = UN;
            const float* DRKm = UN + BL * PL;
            const float* DAB = UN + 2 * BL * PL;
            const float* DAK = UN + 3 * BL * PL;
            // dRt += dA_rb Bt + dA_rk Kt, dAt += dA_ab Bt + dA_ak Kt, dBt += dA_ab^T At +
            // dA_rb^T Rt, dKt += dA_ak^T At + dA_rk^T Rt.  At D = 64 in one k-loop with four
            // independent chains; at D = 128 the separate products measured faster.
            #pragma unroll
            for (int u = 0; u < NA; ++u) {
                const int n = w + 8 * u, m0 = 16 * (n / TC), n0 = 16 * (n % TC);
                if constexpr (D == 64) {
                    #pragma unroll 2
                    for (int k = 0; k < BL; k += 4) {
                        const float bt = opB<false>(BT, PD, n0, k, lp), kt = opB<false>(KT, PD, n0, k, lp);
                        const float at = opB<false>(AT, PD, n0, k, lp), rt = opB<false>(RT, PD, n0, k, lp);
                        accR[u] = mfma4(opA<false>(DRB, PL, m0, k, lp), bt, accR[u]);
                        accA[u] = mfma4(opA<false>(DAB, PL, m0, k, lp), bt, accA[u]);
                        accB[u] = mfma4(opA<true>(DAB, PL, m0, k, lp), at, accB[u]);
                        accK[u] = mfma4(opA<true>(DAK, PL, m0, k, lp), at, accK[u]);
                        accR[u] = mfma4(opA<false>(DRKm, PL, m0, k, lp), kt, accR[u]);
                        accA[u] = mfma4(opA<false>(DAK, PL, m0, k, lp), kt, accA[u]);
                        accB[u] = mfma4(opA<true>(DRB, PL, m0, k, lp), rt, accB[u]);
                        accK[u] = mfma4(opA<true>(DRKm, PL, m0, k, lp), rt, accK[u]);
                    }
                } else {
                    accR[u] = mm<false, false>(DRB, PL, BT, PD, m0, n0, 0, BL, accR[u], lp);
                    accR[u] = mm<false, false>(DRKm, PL, KT, PD, m0, n0, 0, BL, accR[u], lp);
                    accA[u] = mm<false, false>(DAB, PL, BT, PD, m0, n0, 0, BL, accA[u], lp);
                    accA[u] = mm<false, false>(DAK, PL, KT, PD, m0, n0, 0, BL, accA[u], lp);
                    accB[u] = mm<true, false>(DAB, PL, AT, PD, m0, n0, 0, BL, accB[u], lp);
                    accB[u] = mm<true, false>(DRB, PL, RT, PD, m0, n0, 0, BL, accB[u], lp);
                    accK[u] = mm<true, false>(DAK, PL, AT, PD, m0, n0, 0, BL, accK[u], lp);
                    accK[u] = mm<true, false>(DRKm, PL, RT, PD, m0, n0, 0, BL, accK[u], lp);
                }
            }
        }
        __syncthreads();
        // d log w / d(w input) of every kept token (0 for the others), for the suffix sums.
        #pragma unroll
        for (int q = 0; q < NE; ++q) FAC[et * D + ej0 + q] = fac[q];
        // Gradients of r, a, b, k; the log-decay suffix-sum terms.
        #pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int n = w + 8 * u, m0 = 16 * (n / TC), n0 = 16 * (n % TC);
            const int j = n0 + lp.i;
            #pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = m0 + 4 * lp.q + rr;
                const int o = t * PD + j;
                QP[o] = RT[o] * accR[u][rr] - BT[o] * accB[u][rr] - KT[o] * accK[u][rr];
                QA[o] = AT[o] * accA[u][rr];
                if (c0 + t < T) {
                    const bool ok = valid(c0 + t);
                    const float gt = GG[o], gp = t > 0 ? GG[o - PD] : 0.f;
                    float dr = accR[u][rr] * __builtin_amdgcn_exp2f(gt);
                    const float da = accA[u][rr] * __builtin_amdgcn_exp2f(gp);
                    const float db = accB[u][rr] * __builtin_amdgcn_exp2f(-gt);
                    float dk = accK[u][rr] * __builtin_amdgcn_exp2f(-gt);
                    if constexpr (EPI) {
                        if (ok) {
                            const float rv = ld1(rp, qidx(c0 + t, j)), kv = ld1(kp, kvidx(c0 + t, j));
                            const float rkj = g.r_k[h * D + j], dbt = DBETA[t];
                            dr = fmaf(dbt * kv, rkj, dr);
                            dk = fmaf(dbt * rv, rkj, dk);
                            drkp[u] = fmaf(dbt * rv, kv, drkp[u]);
                        }
                    }
                    const int64_t gi = qidx(c0 + t, j);
                    o_dr[gi] = ok ? dr : 0.f;
                    o_da[gi] = ok ? da : 0.f;
                    o_db[gi] = ok ? db : 0.f;
                    o_dk[gi] = ok ? dk : 0.f;
                }
            }
        }
        __syncthreads();
        {   // dL/dlog w: suffix sums within the chunk, carried to the w input.  Thread
            // (seg, j) takes tokens [SEG seg, SEG seg + SEG) of column j: the segment sums
            // go through LDS (ZS), then each thread adds the later segments' sums.
            constexpr int NSEG = BNT / D, SEG = BL / NSEG;
            const int j = tid % D, seg = tid / D, t0 = SEG * seg;
            float q[SEG], part = 0.f;
            #pragma unroll
            for (int t = 0; t < SEG; ++t) {
                const int tt = t0 + t;
                q[t] = QP[tt * PD + j] + (tt + 1 < BL ? QA[(tt + 1) * PD + j] : 0.f);
                part += q[t];
            }
            ZS[seg * D + j] = part;
            __syncthreads();
            float run = DD[j];
            for (int s2 = seg + 1; s2 < NSEG; ++s2) run += ZS[s2 * D + j];
            #pragma unroll
            for (int t = SEG - 1; t >= 0; --t) {
                run += q[t];
                const int tt = t0 + t;
                if (c0 + tt < T) o_dw[qidx(c0 + tt, j)] = run * FAC[tt * D + j];
            }
        }
        __syncthreads();
    }
    if (g.ds0) {
        for (int e = e_begin + tid; e < e_end; e += BNT) g.ds0[int64_t(bh) * D * D + e] = ub[e];
    }
    if constexpr (EPI) {
        #pragma unroll
        for (int u = 0; u < NA; ++u) atomicAdd(&DRK[16 * ((w + 8 * u) % TC) + lp.i], drkp[u]);
        __syncthreads();
        if (tid < D) g.drk[(int64_t(sg) * BH + bh) * D + tid] = DRK[tid];
    }
}

template <int D>
constexpr int bwd_smem_bytes() {
    constexpr int PD = D + 1;
    constexpr int UNI = (2 * BSL * PD > 4 * BL * PL) ? 2 * BSL * PD : 4 * BL * PL;
    return 4 * (5 * BL * PD + 5 * BL * PL + UNI + 6 * BL * PL + 2 * D + 2 * BL + D);
}
static_assert(bwd_smem_bytes<128>() <= 160 * 1024, "LDS budget at D = 128");

// dk, dv of the KV heads: sums over each group of query heads.  dr_k: sum over the batch.
__global__ __launch_bounds__(256) void group_sum_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                        int64_t n_out, int D, int H, int H_kv) {
    const int rep = H / H_kv;
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n_out; e += int64_t(gridDim.x) * 256) {
        const int64_t j = e % D, bthk = e / D;
        const int64_t hk = bthk % H_kv, bt = bthk / H_kv;
        float acc = 0.f;
        for (int u = 0; u < rep; ++u) acc += src[(bt * H + hk * rep + u) * D + j];
        dst[e] = acc;
    }
}
__global__ __launch_bounds__(256) void batch_sum_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                        int B, int HD) {
    for (int e = blockIdx.x * 256 + threadIdx.x; e < HD; e += gridDim.x * 256) {
        float acc = 0.f;
        for (int bb = 0; bb < B; ++bb) acc += src[int64_t(bb) * HD + e];
        dst[e] = acc;
    }
}

// Key-axis gradients of value-slice groups 1 .. P - 1 added to group 0's, in group order.
struct PartSum {
    float* out[5];   // dr, da, db, dk (per query head), dw
};
// Four elements per thread (nq is a multiple of 4, every array 16-byte aligned).
__global__ __launch_bounds__(256) void part_sum_kernel(PartSum o, const float* __restrict__ part, int64_t nq,
                                                       int P) {
    float4* dst = reinterpret_cast<float4*>(o.out[blockIdx.y]);
    const float4* src = reinterpret_cast<const float4*>(part);
    const int64_t n4 = nq / 4;
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n4; e += int64_t(gridDim.x) * 256) {
        float4 acc = dst[e];
        for (int sg = 1; sg < P; ++sg) {
            const float4 x = src[(int64_t(sg - 1) * 5 + blockIdx.y) * n4 + e];
            acc.x += x.x;
            acc.y += x.y;
            acc.z += x.z;
            acc.w += x.w;
        }
        dst[e] = acc;
    }
}

struct BwdLayout {
    int64_t ckpt, ubuf, dinv, dkq, dvq, drk, part, total;
    int split;
};

// Value-slice groups per (b, h): enough workgroups for the chip's 256 compute units
// when B H is small, at most one per 32-row slice, a power of two.
int bwd_split(const Params& p) {
    const int64_t bh = int64_t(p.B) * p.H;
    int P = 1;
    while (2 * P <= p.D / BSL && bh * 2 * P <= 256) P *= 2;
    return P;
}

BwdLayout bwd_layout(const Params& p) {
    auto al = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int nch = (p.T + BL - 1) / BL;
    BwdLayout o{};
    const int64_t bh = int64_t(p.B) * p.H;
    o.split = bwd_split(p);
    o.ckpt = 0;
    int64_t off = al(bh * (nch + 1) * p.D * p.D * 4);
    o.ubuf = off;
    off += al(bh * p.D * p.D * 4);
    o.dinv = off;
    off += al(o.split * bh * nch * BL * BL * 4);
    const bool grouped = p.H_kv != p.H;
    const int64_t nq = int64_t(p.B) * p.T * p.H * p.D;
    o.dkq = off;
    if (grouped) off += al(nq * 4);
    o.dvq = off;
    if (grouped) off += al(nq * 4);
    o.drk = off;
    if (p.r_k) off += al(o.split * bh * p.D * 4);
    o.part = off;
    off += al((o.split - 1) * 5 * nq * 4);
    o.total = off;
    return o;
}

template <int D, typename Tin, typename Tdy, bool LOGW, bool EPI>
hipError_t launch_bwd_t(const Params& p, const BwdIo& io, char* ws, hipStream_t stream) {
    const BwdLayout lay = bwd_layout(p);
    const bool grouped = p.H_kv != p.H;
    BwdArgs g{};
    g.r = p.r; g.w = p.w; g.k = p.k; g.v = p.v; g.a = p.a; g.b = p.b;
    g.s0 = p.s0; g.r_k = p.r_k; g.mask = p.mask; g.dy = io.dy; g.ds1 = io.ds1;
    g.dr = io.dr; g.dw = io.dw; g.da = io.da; g.db = io.db;
    g.dk = grouped ? reinterpret_cast<float*>(ws + lay.dkq) : io.dk;
    g.dv = grouped ? reinterpret_cast<float*>(ws + lay.dvq) : io.dv;
    g.ds0 = io.ds0;
    g.drk = p.r_k ? reinterpret_cast<float*>(ws + lay.drk) : nullptr;
    g.ckpt = reinterpret_cast<float*>(ws + lay.ckpt);
    g.ubuf = reinterpret_cast<float*>(ws + lay.ubuf);
    g.dinv = reinterpret_cast<float*>(ws + lay.dinv);
    g.part = reinterpret_cast<float*>(ws + lay.part);
    g.nq = int64_t(p.B) * p.T * p.H * D;
    g.B = p.B; g.T = p.T; g.H = p.H; g.H_kv = p.H_kv; g.nch = (p.T + BL - 1) / BL;
    g.split = lay.split;
    g.y_scale = p.y_scale;
    auto kern = bwd_kernel<D, Tin, Tdy, LOGW, EPI>;
    constexpr int smem = bwd_smem_bytes<D>();
    static bool attr_set = false;   // per template instance; idempotent if raced
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(p.B) * unsigned(p.H), unsigned(lay.split)), dim3(BNT), smem, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (lay.split > 1) {
        const PartSum o{{g.dr, g.da, g.db, g.dk, g.dw}};
        const int64_t blocks = (g.nq / 4 + 255) / 256;
        hipLaunchKernelGGL(part_sum_kernel, dim3(unsigned(blocks < 8192 ? blocks : 8192), 5), dim3(256), 0,
                           stream, o, g.part, g.nq, lay.split);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (grouped) {
        const int64_t n_out = int64_t(p.B) * p.T * p.H_kv * D;
        const int64_t blocks = (n_out + 255) / 256;
        const dim3 grid(unsigned(blocks < 65536 ? blocks : 65536));
        hipLaunchKernelGGL(group_sum_kernel, grid, dim3(256), 0, stream, g.dk, io.dk, n_out, D, p.H, p.H_kv);
        hipLaunchKernelGGL(group_sum_kernel, grid, dim3(256), 0, stream, g.dv, io.dv, n_out, D, p.H, p.H_kv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.r_k) {
        const int HD = p.H * D;
        hipLaunchKernelGGL(batch_sum_kernel, dim3(unsigned((HD + 255) / 256)), dim3(256), 0, stream,
                           g.drk, io.drk, p.B * lay.split, HD);
        e = hipGetLastError();
    }
    return e;
}

template <int D, typename Tin, typename Tdy>
hipError_t dispatch_modes(const Params& p, const BwdIo& io, char* ws, hipStream_t s) {
    const bool logw = p.w_mode == WKV7_W_LOGNEGLOG;
    const bool epi = p.r_k != nullptr;
    if (logw) return epi ? launch_bwd_t<D, Tin, Tdy, true, true>(p, io, ws, s) : launch_bwd_t<D, Tin, Tdy, true, false>(p, io, ws, s);
    return epi ? launch_bwd_t<D, Tin, Tdy, false, true>(p, io, ws, s) : launch_bwd_t<D, Tin, Tdy, false, false>(p, io, ws, s);
}

template <int D>
hipError_t dispatch_types(const Params& p, const BwdIo& io, char* ws, hipStream_t s) {
    if (p.in_dtype == WKV7_BF16)
        return p.y_dtype == WKV7_BF16 ? dispatch_modes<D, bf16_t, bf16_t>(p, io, ws, s) : dispatch_modes<D, bf16_t, float>(p, io, ws, s);
    return p.y_dtype == WKV7_BF16 ? dispatch_modes<D, float, bf16_t>(p, io, ws, s) : dispatch_modes<D, float, float>(p, io, ws, s);
}

}  // namespace

int64_t backward_workspace_bytes(const Params& p) {
    if (int64_t(p.B) * p.H == 0 || p.T == 0) return 0;
    return bwd_layout(p).total;
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256)
        dst[e] = src ? src[e] : 0.f;
}

hipError_t launch_backward(const Params& p, const BwdIo& io, void* ws, hipStream_t stream) {
    if (p.T == 0) {   // dS0 = dS_T, dr_k = 0
        const int64_t n = int64_t(p.B) * p.H * p.D * p.D;
        if (io.ds0 && n > 0) {
            const int64_t blocks = (n + 255) / 256;
            hipLaunchKernelGGL(fill_kernel, dim3(unsigned(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                               io.ds0, io.ds1, n);
        }
        if (p.r_k && p.H > 0)
            hipLaunchKernelGGL(fill_kernel, dim3(unsigned((p.H * p.D + 255) / 256)), dim3(256), 0, stream,
                               io.drk, static_cast<const float*>(nullptr), int64_t(p.H) * p.D);
        return hipGetLastError();
    }
    char* w = static_cast<char*>(ws);
    return p.D == 64 ? dispatch_types<64>(p, io, w, stream) : dispatch_types<128>(p, io, w, stream);
}

}  // namespace wkv7
