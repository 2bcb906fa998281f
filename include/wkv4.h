/*
 * wkv4.h -- C ABI of the RWKV-4 WKV operator in libwkv7.so (AMD MI355X, gfx950).
 *
 * Per batch b and channel c, over tokens t (SSM note "RWKV: state-space based
 * sequence model", time-mixing section, the WKV operator and its recurrent
 * form):
 *
 *     wkv_t = (a_{t-1} + e^{u + k_t} v_t) / (b_{t-1} + e^{u + k_t})
 *     a_t   = e^{-w} a_{t-1} + e^{k_t} v_t,     b_t = e^{-w} b_{t-1} + e^{k_t}
 *
 * i.e. wkv_t = (sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u+k_t} v_t) / (same with v = 1),
 * with a per-channel decay rate w and bonus u.  The receptance gate sigma(r)
 * of the time-mixing block is not part of the operator.
 *
 * Layouts (row-major, contiguous): k, v, y [B, T, C]; w, u [C] fp32.
 * State: [B, 3, C] fp32 holding (A, Bs, P) per channel with a = A e^P and
 * b = Bs e^P (a shared exponent keeps e^k from overflowing fp32); the zero
 * state is A = Bs = 0 and any P (state_in NULL means zero).
 *
 * Ownership, streams, errors: as in wkv7.h (caller-owned, 16-byte aligned
 * device pointers; work enqueued on `stream`; WKV7_* status codes with
 * wkv7_last_error() for details; all checks before any HIP call).
 */
#ifndef WKV4_H
#define WKV4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct wkv4_desc {
    int32_t B;          /* batch, >= 0 */
    int32_t T;          /* tokens, >= 0 */
    int32_t C;          /* channels, >= 0 */
    int32_t in_dtype;   /* wkv7_dtype of k, v */
    int32_t y_dtype;    /* wkv7_dtype of y */
    int32_t spin_limit; /* polls before a look-back wait gives up; 0 = the default bound (2^18), < 0 invalid */
} wkv4_desc;

/* Workspace bytes of wkv4_forward: 2 * B * ceil(T / 64) * 3 * C * 4 (each
 * 64-token chunk's local and inclusive states) rounded up to 256, plus 256 for
 * a ticket counter and the count of look-back waits that gave up; 0 when
 * B T C == 0; a negative wkv7_status if the descriptor is invalid.  Host only.
 * Calls that share a workspace must be ordered (same stream). */
int64_t wkv4_workspace_bytes(const wkv4_desc* desc);

/* y <- wkv over T tokens from state_in (or zero); state_out (may be NULL) gets
 * the state after the last token.  state_in == state_out is allowed.
 * workspace: at least wkv4_workspace_bytes(desc) bytes (may be NULL when 0),
 * sharing no byte with w, u, k, v, y or the states (EINVAL otherwise).
 * Each 64-token chunk waits for the state of the chunks before it, whose
 * workgroups started earlier.  A wait is bounded (desc->spin_limit polls): one
 * that gives up does not hang the device; it makes y of its channel NaN in its
 * chunk and in later chunks that take their incoming state from it (and the
 * final state, if the last chunk does), and it is counted in the workspace,
 * which wkv4_wait_status reads. */
int wkv4_forward(const wkv4_desc* desc, const float* w, const float* u,
                 const void* k, const void* v, const float* state_in,
                 void* y, float* state_out, void* workspace, int64_t workspace_bytes,
                 void* stream);

/* After wkv4_forward on `stream` with this descriptor and workspace: waits for
 * the stream, then reads how many look-back waits of that call gave up.
 * WKV7_OK if none did (or there was nothing to compute), WKV7_ETIMEOUT if any
 * did (wkv7_last_error() gives the count; y holds NaN where they gave up),
 * WKV7_EINVAL for a bad descriptor or a missing or too small workspace,
 * WKV7_EDEVICE if the stream or the copy fails.  The count is that of the
 * last wkv4_forward call that used the workspace. */
int wkv4_wait_status(const wkv4_desc* desc, const void* workspace, int64_t workspace_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WKV4_H */
