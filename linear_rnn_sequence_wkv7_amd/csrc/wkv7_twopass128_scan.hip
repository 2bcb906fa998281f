// Pass 2 of the D = 128 two-pass chunked WKV-7 forward: the chunk recurrence
//
//   Y   = Q S0^T + P V
//   S_L = S0 diag(d) + (S0 W^T) Bh + V^T E
//
// over the per-chunk operands that pass 1 (wkv7_twopass128.hip) leaves in the
// workspace (the chunk algebra and its rearrangement are described there; the
// update is the generalised delta rule of the wiki note "RWKV-7 Goose", the
// readout after the update as in the youngju.dev RWKV-7 article).
//
// Matrix cores in fp16 (v_mfma_f32_16x16x32_f16, fp32 accumulation): the
// record's W, Q, Bh and E, the state (fp32 in registers, rounded to fp16 as the
// operand of S W^T and Q S^T), the reduced X = S W^T and P are single fp16
// operands, and V is fp16 (exact for bf16 inputs of
// magnitude below 2^16 down to 2^-14; hi + lo for fp32 inputs).  fp16 carries
// 11 significant bits against bf16's 8, so a single fp16 operand rounds 8x
// finer than a single bf16 one; the values must stay inside fp16's range:
// state entries, v and the chunk operands below 65504 in magnitude (the
// one-pass kernels have bf16's range).  Every accumulator chain uses this one
// opcode.
//
// Four 256-thread workgroups per (b, h), each 32 value rows, ids 8 apart (one
// XCD under round-robin dispatch, so the four reads of each record meet in that
// XCD's L2).  Wave kp holds S for its 32 keys x 32 rows as four C tiles.
#include "wkv7_twopass128.h"

namespace wkv7 {
namespace tp128 {
namespace {

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

// LDS map of pass 2 (bytes): the four waves' partial X and Y tiles, the reduced X
// tiles as fp16 operands, and V^T of the slice (two chunk buffers).
constexpr int NTHR_SCAN = 256;
constexpr int S_PART = 0;                          // f32x4 [wave][tile 0..7][lane]
constexpr int S_XOH = S_PART + 4 * 8 * 64 * 16;    // fp16x4 [tile 0..3][lane]
constexpr int VS_BYTES = DV * PT * 2;
constexpr int S_VS = S_XOH + 4 * 64 * 8;           // fp16 [buffer][DV][PT] V^T hi
constexpr int S_VSL = S_VS + 2 * VS_BYTES;         // lo (fp32 inputs)
constexpr int SMEM_SCAN_BF16 = S_VSL;
constexpr int SMEM_SCAN_F32 = S_VSL + 2 * VS_BYTES;
static_assert(SMEM_SCAN_F32 <= 64 * 1024, "default dynamic LDS limit");

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

// Token-axis (pair-interleaved) store of one token's 4 values, rows row0 .. row0 + 3,
// packed in pairs in v, into a [row][PT] 16-bit matrix.  Lanes l and l ^ 1 hold
// tokens t and t ^ 1: the even lane writes rows row0, row0 + 1, the odd lane
// row0 + 2, row0 + 3, each a 32-bit pair of the two tokens (even token low).
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
    f16x8 W[2], Q[2], Bh[2], E[2], Ph;
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
    const int H = g.H, T = g.T, cb = g.cb, ce = g.ce;
    const int bb = bh / H, h = bh - bb * H, hk = h / (H / g.H_kv);
    const uint32_t stkv = uint32_t(g.H_kv) * DK * SI, sty = uint32_t(H) * DK * SY;
    const int64_t tok0 = int64_t(bb) * T;
    // Record of chunk c (cb <= c < ce) of this (b, h).
    const int64_t rec0 = int64_t(bh) * g.nrec - cb;
    auto rec_of = [&](int c) { return g.ws + (rec0 + c) * WS_CHUNK; };
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
    // The operands of the chunk after next are requested in three groups spread
    // over the chunk (when every wave of the chip issues them at once the memory
    // pipeline backs up and the issuing waves stall): W and Q (first needed), Bh
    // and E, then P, d and the bonus.  Two chunks ahead, a record that has left
    // the memory-side cache still arrives in time.
    auto load_wq = [&](int c, Ops& o) {
        const char* kb = rec_of(c) + kp * WS_KP + l * 16;
        #pragma unroll
        for (int i = 0; i < 2; ++i) {
            o.W[i] = *reinterpret_cast<const f16x8*>(kb + (BLK_W + i) * WS_BLK);
            o.Q[i] = *reinterpret_cast<const f16x8*>(kb + (BLK_Q + i) * WS_BLK);
        }
    };
    auto load_be = [&](int c, Ops& o) {
        const char* kb = rec_of(c) + kp * WS_KP + l * 16;
        #pragma unroll
        for (int i = 0; i < 2; ++i) {
            o.Bh[i] = *reinterpret_cast<const f16x8*>(kb + (BLK_BH + i) * WS_BLK);
            o.E[i] = *reinterpret_cast<const f16x8*>(kb + (BLK_E + i) * WS_BLK);
        }
    };
    auto load_p = [&](int c, Ops& o) {   // P, d and the bonus
        const char* rec = rec_of(c);
        o.Ph = *reinterpret_cast<const f16x8*>(rec + WS_P + ty * WS_BLK + l * 16);
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
            if constexpr (VSPLIT) split2h(vrow.get(e), vrow.get(e + 1), vh[e / 2], vl[e / 2]);
            else vh[e / 2] = pack_f16(vrow.get(e), vrow.get(e + 1));
        }
        pair_col_store4(smem + S_VS + buf * VS_BYTES, 4 * vg, vt, vh);
        if constexpr (VSPLIT) pair_col_store4(smem + S_VSL + buf * VS_BYTES, 4 * vg, vt, vl);
    };

    char* yp = static_cast<char*>(g.y);
    // One chunk: operands in `cur`, those of chunk c + 2 prefetched into `nxt`.  The
    // loop below rotates three operand sets, so no prefetched register is copied
    // (a copy would wait for the load); each load is waited for at its first use.
    auto chunk = [&](const int c, Ops& cur, Ops& nxt) {
        const int c0 = c * L, buf = (c - cb) & 1;
        // V rows of the next chunk first (their LDS store closes this iteration),
        // then W, Q of chunk c + 2.  The last iterations load the last chunk again
        // (unused): unconditional loads keep the compiler's wait counts exact.
        const int cn = min(c + 2, ce - 1);
        load_v(min(c + 1, ce - 1));
        load_wq(cn, nxt);
        asm volatile("" ::: "memory");
        // X and Y over this wave's 32 keys: X^T (t x i) = W S^T, Y (t x i) = Q S^T.
        f16x8 SBh[2];
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg) SBh[sg] = to_f16x8(ST[sg][0], ST[sg][1]);
        #pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            #pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                f32x4 xp = mfma16(cur.W[tb], SBh[sg], zero);
                f32x4 yq = mfma16(cur.Q[tb], SBh[sg], zero);
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
        f16x8 VB[2], VBl[2];
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            VB[sg] = lds<f16x8>(vs, ((16 * sg + lr) * PT + 8 * lq) * 2);
            if constexpr (VSPLIT) VBl[sg] = lds<f16x8>(smem + S_VSL + buf * VS_BYTES, ((16 * sg + lr) * PT + 8 * lq) * 2);
        }
        // S <- S diag(d) + V^T E (the X-independent part of the update).
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg)
            #pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 acc = ST[sg][u] * cur.d[u];
                acc = mfma16(cur.E[u], VB[sg], acc);
                if constexpr (VSPLIT) acc = mfma16(cur.E[u], VBl[sg], acc);
                ST[sg][u] = acc;
            }
        // Reduce X tile kp over the four key pairs -> fp16 operand tile.
        {
            f32x4 xs = lds<f32x4>(smem + S_PART, (kp * 64 + l) * 16);
            #pragma unroll
            for (int k2 = 1; k2 < 4; ++k2) xs += lds<f32x4>(smem + S_PART, ((k2 * 8 + kp) * 64 + l) * 16);
            sts<uint2>(smem + S_XOH, (kp * 64 + l) * 8, make_uint2(pack_f16(xs[0], xs[1]), pack_f16(xs[2], xs[3])));
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
            const f16x8 VBy = lds<f16x8>(vs, ov);
            ys = mfma16(cur.Ph, VBy, ys);
            if constexpr (VSPLIT) ys = mfma16(cur.Ph, lds<f16x8>(smem + S_VSL + buf * VS_BYTES, ov), ys);
            const int i_loc = 16 * sy + lr, tl0 = 16 * ty + 4 * lq;
            float vtr[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI) {
                const uint2 vr = lds<uint2>(vs, (i_loc * PT + pairpos(tl0)) * 2);
                vtr[0] = f16lo_f32(vr.x); vtr[1] = f16hi_f32(vr.x); vtr[2] = f16lo_f32(vr.y); vtr[3] = f16hi_f32(vr.y);
                if constexpr (VSPLIT) {
                    const uint2 vl = lds<uint2>(smem + S_VSL + buf * VS_BYTES, (i_loc * PT + pairpos(tl0)) * 2);
                    vtr[0] += f16lo_f32(vl.x); vtr[1] += f16hi_f32(vl.x);
                    vtr[2] += f16lo_f32(vl.y); vtr[3] += f16hi_f32(vl.y);
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
            const f16x8 xh = cat16(lds<uint2>(smem + S_XOH, (sg * 64 + l) * 8), lds<uint2>(smem + S_XOH, ((2 + sg) * 64 + l) * 8));
            #pragma unroll
            for (int u = 0; u < 2; ++u) ST[sg][u] = mfma16(cur.Bh[u], xh, ST[sg][u]);
        }
        // V^T of chunk c + 1 into the other buffer (last read during chunk c - 1); the
        // barrier after the next chunk's partial products publishes it.
        store_v(buf ^ 1);
    };
    Ops opa, opb, opc;
    load_v(cb);
    load_ops(cb, opa);
    load_ops(min(cb + 1, ce - 1), opb);
    store_v(0);
    // The first two operand sets complete here: their load order would otherwise
    // enter the compiler's wait counts of every loop iteration.
    #pragma unroll
    for (int i = 0; i < 2; ++i) {
        asm volatile("" : "+v"(opa.W[i]), "+v"(opa.Q[i]), "+v"(opa.Bh[i]), "+v"(opa.E[i]));
        asm volatile("" : "+v"(opa.d[i]));
        asm volatile("" : "+v"(opb.W[i]), "+v"(opb.Q[i]), "+v"(opb.Bh[i]), "+v"(opb.E[i]));
        asm volatile("" : "+v"(opb.d[i]));
    }
    asm volatile("" : "+v"(opa.Ph), "+v"(opa.bon));
    asm volatile("" : "+v"(opb.Ph), "+v"(opb.bon));
    // Three operand sets in rotation: chunk c uses its set and loads chunk c + 2's.
    int c = cb;
    for (; c + 2 < ce; c += 3) {
        chunk(c, opa, opc);
        chunk(c + 1, opb, opa);
        chunk(c + 2, opc, opb);
    }
    if (c < ce) chunk(c, opa, opc);
    if (c + 1 < ce) chunk(c + 1, opb, opa);

    if (g.s1) {
        #pragma unroll
        for (int sg = 0; sg < 2; ++sg)
            #pragma unroll
            for (int u = 0; u < 2; ++u)
                *reinterpret_cast<float4*>(g.s1 + sbase + int64_t(DV * q + 16 * sg + lr) * DK + 16 * (2 * kp + u) + 4 * lq) =
                    make_float4(ST[sg][u][0], ST[sg][u][1], ST[sg][u][2], ST[sg][u][3]);
    }
}

template <typename Tin, typename Ty, bool EPI>
hipError_t launch_t(const ScanArgs& g, hipStream_t stream) {
    constexpr int smem = sizeof(Tin) == 4 ? SMEM_SCAN_F32 : SMEM_SCAN_BF16;
    // 32 workgroups per group of 8 (b, h): 8 heads x 4 value slices.
    const unsigned groups = unsigned((g.BH + 7) / 8);
    hipLaunchKernelGGL((scan128_kernel<Tin, Ty, EPI>), dim3(groups * 32u), dim3(NTHR_SCAN), smem, stream, g);
    return hipGetLastError();
}

template <typename Tin, typename Ty>
hipError_t launch_epi(const ScanArgs& g, bool epi, hipStream_t s) {
    return epi ? launch_t<Tin, Ty, true>(g, s) : launch_t<Tin, Ty, false>(g, s);
}

}  // namespace

hipError_t launch_scan128(const ScanArgs& g, bool in_f32, bool y_f32, bool epi, hipStream_t stream) {
    if (in_f32) return y_f32 ? launch_epi<float, float>(g, epi, stream) : launch_epi<float, bf16_t>(g, epi, stream);
    return y_f32 ? launch_epi<bf16_t, float>(g, epi, stream) : launch_epi<bf16_t, bf16_t>(g, epi, stream);
}

}  // namespace tp128
}  // namespace wkv7
