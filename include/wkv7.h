/*
 * wkv7.h -- C ABI of libwkv7.so: the RWKV-7 "Goose" WKV recurrence on AMD
 * MI355X (gfx950).
 *
 * The operation (per batch b, head h; state S is D x D fp32, rows i index the
 * value, columns j the key):
 *
 *     S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T        (update)
 *     y_t = y_scale * (S_t r_t) + [r_k] (sum_j r_tj k_tj r_k[h,j]) v_t
 *
 * The update is the full state update of the generalised delta rule (wiki
 * note "RWKV-7 Goose: Expressive Dynamic State Evolution", section
 * "generalised delta rule"), with the kernel vectors a = -kappa_hat and
 * b = kappa_hat * alpha of the hxa07D article (zenn.dev "RWKV hxa07D
 * architecture explained", section 8: the kernel is called with -kk and
 * kk*a).  The readout uses the state after the update (youngju.dev RWKV-7
 * article, time-mix pseudocode).  y_scale and r_k are the hxa07D output
 * epilogue (same article, section 9); the log-decay input mode is its
 * section 3 and grouped KV heads its section 6.
 *
 * Kernel vectors from k (desc->ab_mode == WKV7_AB_FROM_K): the a input holds
 * the in-context rate alpha, b is not read, and per token and head the kernel
 * forms kk = k / max(|k|_2, 1e-12), a = -kk, b = kk * alpha and replaces k by
 * k * (1 - decay + alpha) in the update and in the r_k term, which is the
 * preparation the hxa07D forward listing does before its kernel call (same
 * article, section 8).
 *
 * Attention mask (desc->mask): the same listing hands its kernel an attention
 * mask.  A token whose mask byte is 0 leaves the state as it was and outputs
 * y = 0; the other tokens run as if the masked ones were not there.
 *
 * Layouts (row-major, contiguous, element strides implied by the sizes):
 *     r, w, a, b, y : [B, T, H, D]
 *     k, v          : [B, T, H_kv, D]      head h reads KV head h / (H / H_kv)
 *     state         : [B, H, D, D] fp32,  state[b][h][i][j] = S_ij
 *     r_k           : [H, D] fp32
 *     mask          : [B, T] bytes
 * Element types: r, w, k, v, a, b all have desc->in_dtype (fp32 or bf16);
 * y has desc->y_dtype; the state is always fp32.
 *
 * Ownership and memory: every pointer is DEVICE memory on the current HIP
 * device, owned by the caller.  The library never allocates, frees or keeps
 * a pointer after the call returns; the two-pass form of wkv7_forward_ws
 * works in a workspace the caller passes in.  All data pointers must be
 * 16-byte aligned.  state_in == state_out (in place) is allowed; y must not
 * overlap any input or the workspace.
 *
 * Streams: work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 * default stream) and the call returns without synchronising.  A fault in a
 * kernel surfaces at the caller's next synchronisation.  The library keeps no
 * mutable global state apart from a per-device architecture check done once,
 * so calls from several host threads are safe.
 *
 * Errors: functions return WKV7_OK (0) or a positive WKV7_E* code.  All
 * argument checks run before any HIP call, so a rejected call touches no
 * device.  wkv7_strerror() names a code; wkv7_last_error() gives a detail
 * message for the calling thread's most recent failure.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV7_ABI_VERSION 6

enum wkv7_status {
    WKV7_OK = 0,
    WKV7_EINVAL = 1,        /* null/misaligned pointer, negative size, H % H_kv != 0, bad enum */
    WKV7_EUNSUPPORTED = 2,  /* D not 64/128, unsupported mode/algorithm combination */
    WKV7_EDEVICE = 3,       /* current device is not gfx950, or a HIP device query failed */
    WKV7_ELAUNCH = 4,       /* a kernel launch reported an error */
    WKV7_ETIMEOUT = 5       /* a bounded device-side wait gave up (wkv4_wait_status) */
};

enum wkv7_dtype { WKV7_F32 = 0, WKV7_BF16 = 1 };

/* How the w input is read. */
enum wkv7_w_mode {
    WKV7_W_DECAY = 0,       /* w is the decay itself, in (0, 1] */
    WKV7_W_LOGNEGLOG = 1    /* w holds log(-log(decay)); decay = exp(-exp(w)) */
};

/* Where the kernel vectors a, b come from. */
enum wkv7_ab_mode {
    WKV7_AB_GIVEN = 0,      /* a and b are inputs */
    WKV7_AB_FROM_K = 1      /* a holds alpha, b is unused (may be NULL); a, b and the scaled k
                               are formed from k, alpha and the decay (see above).  Every
                               algorithm and the decode step support it. */
};

enum wkv7_algo {
    WKV7_ALGO_AUTO = 0,     /* library picks (see wkv7_resolve_algo) */
    WKV7_ALGO_SCAN = 1,     /* token-by-token scan, state in registers.  EUNSUPPORTED when a
                               token row is too wide for its 32-bit offsets (H * D * 68 >= 2^32,
                               about 6.3e7) or B * H workgroups (times 4 at D = 128) of 256
                               threads exceed 2^32 work-items */
    WKV7_ALGO_CHUNKED = 2,  /* chunk-parallel form on bf16 matrix cores, fp32 accumulation */
    WKV7_ALGO_TWO_PASS = 3  /* D = 128 only, wkv7_forward_ws only: the chunked form split in two
                               kernels, the state-independent matrices of every chunk first (in
                               parallel over chunks, into the workspace, as fp16), then the
                               recurrence on fp16 matrix cores (fp32 accumulation).  Range: the
                               state, v and the per-chunk matrices must stay below 65504 in
                               magnitude (fp16's largest finite value); past it y and the state
                               come out infinite or NaN.  The other algorithms keep bf16's range */
};

typedef struct wkv7_desc {
    int32_t B;          /* batch (sequences), >= 0 */
    int32_t T;          /* tokens per sequence, >= 0 (decode_step requires 1) */
    int32_t H;          /* heads, >= 0 */
    int32_t H_kv;       /* KV heads; H % H_kv == 0 (0 means H_kv = H) */
    int32_t D;          /* head size: 64 or 128 */
    int32_t in_dtype;   /* wkv7_dtype of r, w, k, v, a, b */
    int32_t y_dtype;    /* wkv7_dtype of y */
    int32_t w_mode;     /* wkv7_w_mode */
    int32_t algo;       /* wkv7_algo (forward only; decode_step ignores it) */
    int32_t chunk_len;  /* chunk length of ALGO_CHUNKED, fixed per head size: 64 at D = 64,
                           32 at D = 128; 0 selects it, other values are EUNSUPPORTED */
    float   y_scale;    /* multiplies S_t r_t; 1.0f for the plain readout */
    int32_t ab_mode;    /* wkv7_ab_mode */
    const float* r_k;   /* [H, D] fp32 device pointer, or NULL for no bonus term */
    const uint8_t* mask;/* [B, T] device bytes, 0 = masked token; NULL = no token masked.
                           No alignment needed.  Supported by every algorithm. */
} wkv7_desc;

/* Forward over T tokens for every (b, h).
 *   state_in  : initial state, or NULL for zeros.
 *   y         : output [B, T, H, D] of y_dtype (may be NULL only when B*T*H == 0).
 *   state_out : final state, or NULL to skip writing it.
 * T == 0 copies state_in (or zeros) to state_out and writes no y. */
int wkv7_forward(const wkv7_desc* desc,
                 const void* r, const void* w, const void* k, const void* v,
                 const void* a, const void* b,
                 const float* state_in, void* y, float* state_out,
                 void* stream);

/* wkv7_forward with a caller-provided device workspace for the two-pass form.
 *   workspace       : device memory, 16-byte aligned, at least
 *                     wkv7_workspace_bytes(desc) bytes; may be NULL when that is 0.
 *   workspace_bytes : its size.
 * The algorithm is WKV7_ALGO_TWO_PASS when desc->algo asks for it, and for
 * desc->algo == AUTO whenever wkv7_workspace_bytes(desc) > 0 (ab_mode
 * included); otherwise the call is wkv7_forward.  The workspace contents are scratch: not read before
 * they are written, undefined afterwards.  Calls that share a workspace must
 * be ordered (same stream).  EINVAL if the workspace is NULL, misaligned,
 * smaller than needed, or shares a byte with any array of the call (inputs,
 * y, state_in, state_out, mask, r_k). */
int wkv7_forward_ws(const wkv7_desc* desc,
                    const void* r, const void* w, const void* k, const void* v,
                    const void* a, const void* b,
                    const float* state_in, void* y, float* state_out,
                    void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of the device scratch that wkv7_forward_noalloc works in, per device. */
#define WKV7_NOALLOC_SCRATCH_BYTES (64LL << 20)

/* wkv7_forward_ws for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments (minus the workspace) and algorithm choice as
 * wkv7_forward_ws; calls no hipMalloc, hipFree or other allocating routine.
 *
 * The two-pass form keeps its per-chunk records, and the state carried between
 * windows when state_out is NULL, in a static device array of
 * WKV7_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends.  The chunks run in windows of as many 32-token chunks
 * per (b, h) as fit (B * H * 35584 bytes per chunk, after B * H * D * D * 4
 * bytes of state carry when state_out is NULL): pass 1 then pass 2 per
 * window, the state passed on through state_out (or the carry).  The results
 * are those of wkv7_forward_ws bit for bit.  EUNSUPPORTED when not even one
 * chunk per (b, h) fits.  Nothing in the scratch needs to start at zero (each
 * window's records and the carry are written before they are read).
 *
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents: calls that may overlap on one device (different streams,
 * several host threads) race, and the caller must order them.  The scratch's
 * device address is looked up once per device, on the first call that runs
 * the two-pass form with that device current. */
int wkv7_forward_noalloc(const wkv7_desc* desc,
                         const void* r, const void* w, const void* k, const void* v,
                         const void* a, const void* b,
                         const float* state_in, void* y, float* state_out,
                         void* stream);

/* Workspace bytes wkv7_forward_ws uses for this descriptor: for D = 128 with
 * algo AUTO and T >= the chunk length, or algo TWO_PASS and T >= 1, it is
 * B * H * ceil(T / 32) * 35584 (one 34.75 KiB record of operands per chunk);
 * 0 otherwise.  A negative wkv7_status if the descriptor is invalid.  Host
 * only: no HIP call. */
int64_t wkv7_workspace_bytes(const wkv7_desc* desc);

/* One decode token per sequence (desc->T must be 1): the recurrent (RNN)
 * mode of the model, in which each new token costs the same work and the
 * state is the only memory carried between tokens (104case.com translation of
 * the RWKV paper, part 2, "RNN-like sequential decoding"; youngju.dev RWKV-7
 * article, "inference mode").  The same operation as wkv7_forward with T = 1,
 * run by a kernel that streams the B*H states through HBM once (read
 * state_in, write state_out).  state_in may be NULL (zeros); state_out must
 * not be NULL; state_in == state_out (in place) is allowed. */
int wkv7_decode_step(const wkv7_desc* desc,
                     const void* r, const void* w, const void* k, const void* v,
                     const void* a, const void* b,
                     const float* state_in, void* y, float* state_out,
                     void* stream);

/* Backward of wkv7_forward: the gradients of L = <dy, y> + <dstate_out, state_out>
 * for the forward this descriptor describes (same inputs, same state_in).  No
 * page gives these formulas: they are the reverse-mode derivative of the update,
 * the readout and the epilogue (the update of the wiki note "RWKV-7 Goose",
 * generalised delta rule; readout and epilogue as in wkv7_forward).
 *   dy          : [B, T, H, D] of desc->y_dtype (required when B*T*H > 0).
 *   dstate_out  : [B, H, D, D] fp32 gradient of the final state, or NULL (zero).
 *   dr, dw, da, db : [B, T, H, D] fp32;  dk, dv : [B, T, H_kv, D] fp32 (summed over
 *                 each KV group).  dw is with respect to the w input in its own
 *                 mode (decay, or log(-log decay)).  Masked tokens get zeros.
 *   dstate_in   : [B, H, D, D] fp32 gradient of state_in, or NULL to skip it.
 *   dr_k        : [H, D] fp32, summed over the batch; required exactly when
 *                 desc->r_k is given.
 *   workspace   : device memory of at least wkv7_backward_workspace_bytes(desc)
 *                 bytes, 16-byte aligned (scratch: not read before it is written),
 *                 sharing no byte with any other array of the call (EINVAL).
 * desc->algo and desc->chunk_len are ignored; ab_mode FROM_K is EUNSUPPORTED.
 * Every pointer is device memory, 16-byte aligned, owned by the caller; outputs
 * must not overlap inputs or the workspace.  Runs one forward sweep that keeps
 * the state at every 32-token boundary in the workspace, then the backward. */
int wkv7_backward(const wkv7_desc* desc,
                  const void* r, const void* w, const void* k, const void* v,
                  const void* a, const void* b, const float* state_in,
                  const void* dy, const float* dstate_out,
                  float* dr, float* dw, float* dk, float* dv, float* da, float* db,
                  float* dstate_in, float* dr_k,
                  void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes of wkv7_backward.  With P the number of value-slice groups
 * per (b, h) (the largest power of two with P <= D / 32 and B H P <= 256; each
 * group is one workgroup), the parts are: B H (ceil(T / 32) + 1) D^2 4 for the
 * state checkpoints, B H D^2 4 for dL/dS, P B H ceil(T / 32) 32^2 4 for each
 * chunk's triangular inverse, 2 B T H D 4 for grouped KV heads (H_kv < H),
 * P B H D 4 with r_k, and (P - 1) 5 B T H D 4 for the key-axis gradients of
 * groups 1 .. P - 1; each rounded up to 256.  0 when B H T == 0.  A negative
 * wkv7_status if the descriptor is invalid.  Host only: no HIP call. */
int64_t wkv7_backward_workspace_bytes(const wkv7_desc* desc);

/* Which algorithm wkv7_forward would run for this descriptor (WKV7_ALGO_SCAN or
 * WKV7_ALGO_CHUNKED), or a negative wkv7_status if the descriptor is invalid.
 * AUTO picks the chunked form once T covers one chunk (T >= chunk length),
 * the scan otherwise.  An explicit
 * WKV7_ALGO_TWO_PASS is returned as is (wkv7_forward rejects it;
 * wkv7_forward_ws runs it).  Host only: no HIP call. */
int wkv7_resolve_algo(const wkv7_desc* desc);

/* Static name of a status code. */
const char* wkv7_strerror(int code);

/* Detail message of the calling thread's most recent failed call ("" if none). */
const char* wkv7_last_error(void);

/* WKV7_ABI_VERSION of the built library. */
int wkv7_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
