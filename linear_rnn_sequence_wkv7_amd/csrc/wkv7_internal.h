// Internal interface between the C-ABI entry points (wkv7_api.cpp) and the
// kernel launchers (wkv7_scan.hip, wkv7_chunked.hip, wkv7_chunked128.hip,
// wkv7_twopass128.hip, wkv7_twopass128_scan.hip, wkv7_decode.hip, wkv7_backward.hip,
// wkv4.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "../../include/wkv7.h"
#include "../../include/wkv4.h"

namespace wkv7 {

// Validated, resolved arguments of one call.  Sizes are those of wkv7_desc
// (H_kv already defaulted, chunk_len already defaulted).
struct Params {
    int B, T, H, H_kv, D;
    int in_dtype, y_dtype, w_mode, chunk_len;
    int ab_mode;              // wkv7_ab_mode
    float y_scale;
    const float* r_k;
    const uint8_t* mask;      // [B, T] or null
    const void *r, *w, *k, *v, *a, *b;
    const float* s0;   // may be null: zero initial state
    void* y;
    float* s1;         // may be null: final state not written
};

// Each launcher enqueues its kernel(s) on `stream` and returns the HIP status
// of the launch.  They assume Params passed validation in wkv7_api.cpp.
// Scan with D / 16 independent waves per (b, h) and DPP row sums; for T >= 1,
// rows (H * D) narrow enough for 32-bit offsets over a few tokens and grids
// within 2^32 work-items (scan_fits; checked by the entry points first).
bool scan_fits(const Params& p);
hipError_t launch_scan(const Params& p, hipStream_t stream);
hipError_t launch_chunked(const Params& p, hipStream_t stream);      // D = 64, L = 64
hipError_t launch_chunked128(const Params& p, hipStream_t stream);   // D = 128, L = 32
// Two-pass form at D = 128: per-chunk matrices into `ws`, then the recurrence.
// With win_chunks below the chunk count the chunks run in windows of that many
// per (b, h) (ws holds B H win_chunks records); the state passes from window to
// window through state_out, or through `carry` ([B, H, D, D] fp32) when state_out
// is null.
int64_t twopass128_workspace_bytes(int B, int H, int T);
int64_t twopass128_record_bytes();
hipError_t launch_twopass128(const Params& p, void* ws, int win_chunks, float* carry, hipStream_t stream);
// Allocation-free two-pass form: the records and the state carry live in the
// library's static device scratch (WKV7_NOALLOC_SCRATCH_BYTES per device).
// noalloc_scratch_init looks up the scratch's device address once per device
// (call it with that device current); the window is the chunks per (b, h) that
// fit (0: not even one).
hipError_t noalloc_scratch_init(int device);
int twopass128_noalloc_window(const Params& p);
hipError_t launch_twopass128_noalloc(const Params& p, int device, hipStream_t stream);
hipError_t launch_decode(const Params& p, hipStream_t stream);
// state_out <- state_in (or zeros) for T == 0.
hipError_t launch_state_copy(const Params& p, hipStream_t stream);

// Backward: the arrays beyond the forward's inputs.
struct BwdIo {
    const void* dy;        // [B, T, H, D] of y_dtype
    const float* ds1;      // dL/dS_T or null (zero)
    float *dr, *dw, *da, *db;   // [B, T, H, D]
    float *dk, *dv;        // [B, T, H_kv, D]
    float* ds0;            // dL/dS_0 or null (not written)
    float* drk;            // [H, D] when r_k is given
};
int64_t backward_workspace_bytes(const Params& p);

// RWKV-4 WKV (wkv4.hip).
struct Wkv4Params {
    int B, T, C, in_dtype, y_dtype;
    int spin_limit;   // polls before a look-back wait gives up (0: the default bound)
    const float *w, *u;
    const void *k, *v;
    void* y;
    const float* s0;
    float* s1;
    void* ws;
};
int64_t wkv4_workspace_bytes_internal(int B, int T, int C);
// Byte offset in the workspace of the int32 count of look-back waits that gave up.
int64_t wkv4_wait_counter_offset(int B, int T, int C);
hipError_t launch_wkv4(const Wkv4Params& p, hipStream_t stream);
hipError_t launch_backward(const Params& p, const BwdIo& io, void* ws, hipStream_t stream);

}  // namespace wkv7
