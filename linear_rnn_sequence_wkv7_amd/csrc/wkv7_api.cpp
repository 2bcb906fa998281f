// C-ABI entry points of libwkv7.so: argument validation (before any HIP
// call), a once-per-device architecture check, algorithm choice and dispatch
// to the kernel launchers.  See include/wkv7.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "wkv7_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A named device range [p, p + bytes) for the workspace overlap checks.
struct Span {
    const void* p;
    int64_t bytes;
    const char* name;
};

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + uint64_t(nb) && y < x + uint64_t(na);
}

// The workspace is written before it is read, so it must not share a byte with
// any array the call reads or writes.
int check_workspace_disjoint(const void* ws, int64_t need, const Span* spans, int n) {
    for (int i = 0; i < n; ++i)
        if (overlap(ws, need, spans[i].p, spans[i].bytes))
            return fail(WKV7_EINVAL, "workspace overlaps %s", spans[i].name);
    return WKV7_OK;
}

// Byte sizes of the arrays of one wkv7 call.
struct Sizes {
    int64_t q, kv, y, state, mask, rk;
};

Sizes sizes_of(const wkv7::Params& p) {
    const int64_t sin = p.in_dtype == WKV7_BF16 ? 2 : 4, sy = p.y_dtype == WKV7_BF16 ? 2 : 4;
    const int64_t bt = int64_t(p.B) * p.T;
    return {bt * p.H * p.D * sin, bt * p.H_kv * p.D * sin, bt * p.H * p.D * sy,
            int64_t(p.B) * p.H * p.D * p.D * 4, bt, int64_t(p.H) * p.D * 4};
}

// 0 = unchecked, 1 = gfx950, 2 = other architecture.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(WKV7_EDEVICE, "hipGetDevice failed");
    if (dev >= kMaxDevices) return fail(WKV7_EDEVICE, "device index %d out of range", dev);
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(WKV7_EDEVICE, "hipGetDeviceProperties failed on device %d", dev);
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
        if (st == 2)
            return fail(WKV7_EDEVICE, "device %d is %s; this library is built for gfx950 only",
                        dev, prop.gcnArchName);
    }
    if (st != 1) return fail(WKV7_EDEVICE, "device %d is not gfx950", dev);
    return WKV7_OK;
}

// Validate the descriptor and fill the size/mode fields of Params.
int check_desc(const wkv7_desc* d, wkv7::Params* p) {
    if (!d) return fail(WKV7_EINVAL, "desc is NULL");
    if (d->B < 0 || d->T < 0 || d->H < 0 || d->H_kv < 0)
        return fail(WKV7_EINVAL, "negative size (B=%d T=%d H=%d H_kv=%d)", d->B, d->T, d->H, d->H_kv);
    if (d->D <= 0) return fail(WKV7_EINVAL, "D must be positive (got %d)", d->D);
    if (d->D != 64 && d->D != 128) return fail(WKV7_EUNSUPPORTED, "D=%d; supported head sizes are 64 and 128", d->D);
    int H_kv = d->H_kv == 0 ? d->H : d->H_kv;
    if (d->H > 0 && (H_kv > d->H || d->H % H_kv != 0))
        return fail(WKV7_EINVAL, "H=%d is not a multiple of H_kv=%d", d->H, H_kv);
    if (d->in_dtype != WKV7_F32 && d->in_dtype != WKV7_BF16)
        return fail(WKV7_EINVAL, "in_dtype %d unknown", d->in_dtype);
    if (d->y_dtype != WKV7_F32 && d->y_dtype != WKV7_BF16)
        return fail(WKV7_EINVAL, "y_dtype %d unknown", d->y_dtype);
    if (d->w_mode != WKV7_W_DECAY && d->w_mode != WKV7_W_LOGNEGLOG)
        return fail(WKV7_EINVAL, "w_mode %d unknown", d->w_mode);
    if (d->algo < WKV7_ALGO_AUTO || d->algo > WKV7_ALGO_TWO_PASS)
        return fail(WKV7_EINVAL, "algo %d unknown", d->algo);
    if (d->ab_mode != WKV7_AB_GIVEN && d->ab_mode != WKV7_AB_FROM_K)
        return fail(WKV7_EINVAL, "ab_mode %d unknown", d->ab_mode);
    if (d->algo == WKV7_ALGO_TWO_PASS && d->D != 128)
        return fail(WKV7_EUNSUPPORTED, "the two-pass form needs D=128 (got %d)", d->D);
    // Each chunked kernel has one chunk length: 64 at D = 64, 32 at D = 128.
    const int L_native = d->D == 64 ? 64 : 32;
    int L = d->chunk_len == 0 ? L_native : d->chunk_len;
    if (L != L_native)
        return fail(WKV7_EUNSUPPORTED, "chunk_len=%d; supported at D=%d: %d (or 0)", d->chunk_len, d->D, L_native);
    if (!std::isfinite(d->y_scale)) return fail(WKV7_EINVAL, "y_scale is not finite");
    if (d->r_k && !aligned16(d->r_k)) return fail(WKV7_EINVAL, "r_k is not 16-byte aligned");
    // Grid and index limits: (b, h) pairs index a 1-D grid; element offsets are 64-bit.
    int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 30)) return fail(WKV7_EUNSUPPORTED, "B*H=%lld too large", (long long)bh);
    int64_t elems = bh * d->T * d->D;
    if (elems > (int64_t(1) << 46)) return fail(WKV7_EUNSUPPORTED, "B*T*H*D too large");
    p->B = d->B; p->T = d->T; p->H = d->H; p->H_kv = H_kv; p->D = d->D;
    p->in_dtype = d->in_dtype; p->y_dtype = d->y_dtype; p->w_mode = d->w_mode;
    p->chunk_len = L; p->ab_mode = d->ab_mode; p->y_scale = d->y_scale; p->r_k = d->r_k;
    p->mask = d->mask;
    return WKV7_OK;
}

int check_ptrs(const wkv7::Params& p, const void* const* in6, const void* y,
               const float* s0, const float* s1) {
    static const char* names[6] = {"r", "w", "k", "v", "a", "b"};
    bool has_tokens = int64_t(p.B) * p.T * p.H > 0;
    if (has_tokens) {
        // b is not read when the kernel vectors come from k.
        const int n_in = p.ab_mode == WKV7_AB_FROM_K ? 5 : 6;
        for (int i = 0; i < n_in; ++i) {
            if (!in6[i]) return fail(WKV7_EINVAL, "%s is NULL", names[i]);
            if (!aligned16(in6[i])) return fail(WKV7_EINVAL, "%s is not 16-byte aligned", names[i]);
        }
        if (!y) return fail(WKV7_EINVAL, "y is NULL");
        if (!aligned16(y)) return fail(WKV7_EINVAL, "y is not 16-byte aligned");
        for (int i = 0; i < 6; ++i)
            if (in6[i] == y) return fail(WKV7_EINVAL, "y aliases input %s", names[i]);
    }
    if (s0 && !aligned16(s0)) return fail(WKV7_EINVAL, "state_in is not 16-byte aligned");
    if (s1 && !aligned16(s1)) return fail(WKV7_EINVAL, "state_out is not 16-byte aligned");
    return WKV7_OK;
}

// AUTO: the chunked matrix-core form once a sequence spans at least one full
// chunk; with a workspace at D = 128 its two-pass variant.  The scan otherwise.
int resolve_algo(const wkv7::Params& p, int requested, bool with_workspace) {
    if (requested != WKV7_ALGO_AUTO) return requested;
    if (p.T < p.chunk_len) return WKV7_ALGO_SCAN;
    if (with_workspace && p.D == 128) return WKV7_ALGO_TWO_PASS;
    return WKV7_ALGO_CHUNKED;
}

int64_t workspace_bytes(const wkv7::Params& p, int algo) {
    if (algo != WKV7_ALGO_TWO_PASS || p.T == 0) return 0;
    return wkv7::twopass128_workspace_bytes(p.B, p.H, p.T);
}

int finish_launch(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(WKV7_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    e = hipGetLastError();
    if (e != hipSuccess) return fail(WKV7_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return WKV7_OK;
}

// How a forward call gets the two-pass form's workspace.
enum class WsMode { kNone, kCaller, kStatic };

int forward_impl(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                 const void* v, const void* a, const void* b, const float* state_in,
                 void* y, float* state_out, void* workspace, int64_t workspace_bytes_given,
                 WsMode ws_mode, void* stream) {
    g_last_error[0] = '\0';
    wkv7::Params p{};
    int rc = check_desc(desc, &p);
    if (rc) return rc;
    if (ws_mode == WsMode::kNone && desc->algo == WKV7_ALGO_TWO_PASS)
        return fail(WKV7_EINVAL, "algo TWO_PASS needs a workspace: call wkv7_forward_ws or wkv7_forward_noalloc");
    const void* in6[6] = {r, w, k, v, a, b};
    if ((rc = check_ptrs(p, in6, y, state_in, state_out))) return rc;
    const int algo = resolve_algo(p, desc->algo, ws_mode != WsMode::kNone);
    const bool has_work = int64_t(p.B) * p.H > 0 && p.T > 0;
    if (has_work && algo == WKV7_ALGO_SCAN && !wkv7::scan_fits(p))
        return fail(WKV7_EUNSUPPORTED, "scan: H*D=%lld or B*H=%lld too large (rows of 32-bit offsets, 2^32 work-items)",
                    (long long)(int64_t(p.H) * p.D), (long long)(int64_t(p.B) * p.H));
    const int64_t need = has_work ? workspace_bytes(p, algo) : 0;
    if (need > 0 && ws_mode == WsMode::kCaller) {
        if (!workspace) return fail(WKV7_EINVAL, "workspace is NULL (%lld bytes needed)", (long long)need);
        if (!aligned16(workspace)) return fail(WKV7_EINVAL, "workspace is not 16-byte aligned");
        if (workspace_bytes_given < need)
            return fail(WKV7_EINVAL, "workspace has %lld bytes, %lld needed",
                        (long long)workspace_bytes_given, (long long)need);
        if (workspace == y) return fail(WKV7_EINVAL, "y aliases the workspace");
        const Sizes z = sizes_of(p);
        const Span spans[11] = {{r, z.q, "r"}, {w, z.q, "w"}, {k, z.kv, "k"}, {v, z.kv, "v"}, {a, z.q, "a"},
                                {p.ab_mode == WKV7_AB_FROM_K ? nullptr : b, z.q, "b"}, {y, z.y, "y"},
                                {state_in, z.state, "state_in"}, {state_out, z.state, "state_out"},
                                {p.mask, z.mask, "mask"}, {p.r_k, z.rk, "r_k"}};
        if ((rc = check_workspace_disjoint(workspace, need, spans, 11))) return rc;
    }
    if (need > 0 && ws_mode == WsMode::kStatic) {
        p.s1 = state_out;   // the window size depends on whether the carry needs room
        if (wkv7::twopass128_noalloc_window(p) < 1)
            return fail(WKV7_EUNSUPPORTED,
                        "B*H=%lld needs %lld bytes of scratch for one chunk per (b, h)%s; the static scratch "
                        "holds %lld", (long long)(int64_t(p.B) * p.H),
                        (long long)(int64_t(p.B) * p.H * wkv7::twopass128_record_bytes()),
                        state_out ? "" : " plus the state carry", (long long)WKV7_NOALLOC_SCRATCH_BYTES);
    }
    p.r = r; p.w = w; p.k = k; p.v = v; p.a = a; p.b = b;
    p.s0 = state_in; p.y = y; p.s1 = state_out;
    if (int64_t(p.B) * p.H == 0) return WKV7_OK;
    if ((rc = check_device())) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.T == 0) {
        if (!state_out) return WKV7_OK;
        return finish_launch(wkv7::launch_state_copy(p, s), "state copy");
    }
    if (algo == WKV7_ALGO_TWO_PASS && ws_mode == WsMode::kStatic) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return fail(WKV7_EDEVICE, "hipGetDevice failed");
        const hipError_t e = wkv7::noalloc_scratch_init(dev);
        if (e != hipSuccess)
            return fail(WKV7_EDEVICE, "device address of the static scratch on device %d: %s", dev,
                        hipGetErrorString(e));
        return finish_launch(wkv7::launch_twopass128_noalloc(p, dev, s), "two-pass (D=128, static scratch)");
    }
    if (algo == WKV7_ALGO_TWO_PASS)
        return finish_launch(wkv7::launch_twopass128(p, workspace, (p.T + p.chunk_len - 1) / p.chunk_len, nullptr, s),
                             "two-pass (D=128)");
    if (algo == WKV7_ALGO_CHUNKED)
        return p.D == 64 ? finish_launch(wkv7::launch_chunked(p, s), "chunked")
                         : finish_launch(wkv7::launch_chunked128(p, s), "chunked (D=128)");
    return finish_launch(wkv7::launch_scan(p, s), "scan");
}

}  // namespace

extern "C" {

int wkv7_forward(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                 const void* v, const void* a, const void* b, const float* state_in,
                 void* y, float* state_out, void* stream) {
    return forward_impl(desc, r, w, k, v, a, b, state_in, y, state_out, nullptr, 0, WsMode::kNone, stream);
}

int wkv7_forward_ws(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                    const void* v, const void* a, const void* b, const float* state_in,
                    void* y, float* state_out, void* workspace, int64_t workspace_bytes_given,
                    void* stream) {
    return forward_impl(desc, r, w, k, v, a, b, state_in, y, state_out, workspace,
                        workspace_bytes_given, WsMode::kCaller, stream);
}

int wkv7_forward_noalloc(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                         const void* v, const void* a, const void* b, const float* state_in,
                         void* y, float* state_out, void* stream) {
    return forward_impl(desc, r, w, k, v, a, b, state_in, y, state_out, nullptr, 0, WsMode::kStatic, stream);
}

int64_t wkv7_workspace_bytes(const wkv7_desc* desc) {
    g_last_error[0] = '\0';
    wkv7::Params p{};
    int rc = check_desc(desc, &p);
    if (rc) return -rc;
    return workspace_bytes(p, resolve_algo(p, desc->algo, true));
}

int wkv7_decode_step(const wkv7_desc* desc, const void* r, const void* w, const void* k,
                     const void* v, const void* a, const void* b, const float* state_in,
                     void* y, float* state_out, void* stream) {
    g_last_error[0] = '\0';
    wkv7::Params p{};
    int rc = check_desc(desc, &p);
    if (rc) return rc;
    if (p.T != 1) return fail(WKV7_EINVAL, "decode_step needs T == 1 (got %d)", p.T);
    const void* in6[6] = {r, w, k, v, a, b};
    if ((rc = check_ptrs(p, in6, y, state_in, state_out))) return rc;
    if (int64_t(p.B) * p.H > 0 && !state_out) return fail(WKV7_EINVAL, "state_out is NULL");
    p.r = r; p.w = w; p.k = k; p.v = v; p.a = a; p.b = b;
    p.s0 = state_in; p.y = y; p.s1 = state_out;
    if (int64_t(p.B) * p.H == 0) return WKV7_OK;
    if ((rc = check_device())) return rc;
    return finish_launch(wkv7::launch_decode(p, reinterpret_cast<hipStream_t>(stream)), "decode");
}

int64_t wkv7_backward_workspace_bytes(const wkv7_desc* desc) {
    g_last_error[0] = '\0';
    wkv7::Params p{};
    int rc = check_desc(desc, &p);
    if (rc) return -rc;
    return wkv7::backward_workspace_bytes(p);
}

int wkv7_backward(const wkv7_desc* desc, const void* r, const void* w, const void* k, const void* v,
                  const void* a, const void* b, const float* state_in, const void* dy,
                  const float* dstate_out, float* dr, float* dw, float* dk, float* dv, float* da,
                  float* db, float* dstate_in, float* dr_k, void* workspace,
                  int64_t workspace_bytes_given, void* stream) {
    g_last_error[0] = '\0';
    wkv7::Params p{};
    int rc = check_desc(desc, &p);
    if (rc) return rc;
    if (p.ab_mode != WKV7_AB_GIVEN)
        return fail(WKV7_EUNSUPPORTED, "wkv7_backward takes the kernel vectors as inputs (ab_mode GIVEN)");
    const void* in6[6] = {r, w, k, v, a, b};
    if (int64_t(p.B) * p.T * p.H > 0 && !dy) return fail(WKV7_EINVAL, "dy is NULL");
    // dy plays the role of y in the input checks (aligned, not an input).
    if ((rc = check_ptrs(p, in6, dy, state_in, nullptr))) return rc;
    if (dstate_out && !aligned16(dstate_out)) return fail(WKV7_EINVAL, "dstate_out is not 16-byte aligned");
    const bool has_tokens = int64_t(p.B) * p.T * p.H > 0;
    float* outs[6] = {dr, dw, dk, dv, da, db};
    static const char* onames[6] = {"dr", "dw", "dk", "dv", "da", "db"};
    for (int i = 0; i < 6; ++i) {
        if (has_tokens && !outs[i]) return fail(WKV7_EINVAL, "%s is NULL", onames[i]);
        if (outs[i] && !aligned16(outs[i])) return fail(WKV7_EINVAL, "%s is not 16-byte aligned", onames[i]);
        for (int j = 0; j < 6; ++j)
            if (outs[i] && outs[i] == in6[j]) return fail(WKV7_EINVAL, "%s aliases input", onames[i]);
    }
    if (dstate_in && !aligned16(dstate_in)) return fail(WKV7_EINVAL, "dstate_in is not 16-byte aligned");
    if (p.r_k && p.H > 0 && !dr_k) return fail(WKV7_EINVAL, "dr_k is NULL but r_k is given");
    if (!p.r_k && dr_k) return fail(WKV7_EINVAL, "dr_k is given but r_k is NULL");
    if (dr_k && !aligned16(dr_k)) return fail(WKV7_EINVAL, "dr_k is not 16-byte aligned");
    const int64_t need = wkv7::backward_workspace_bytes(p);
    if (need > 0) {
        if (!workspace) return fail(WKV7_EINVAL, "workspace is NULL (%lld bytes needed)", (long long)need);
        if (!aligned16(workspace)) return fail(WKV7_EINVAL, "workspace is not 16-byte aligned");
        if (workspace_bytes_given < need)
            return fail(WKV7_EINVAL, "workspace has %lld bytes, %lld needed",
                        (long long)workspace_bytes_given, (long long)need);
        const Sizes z = sizes_of(p);
        const int64_t gq = z.y / (p.y_dtype == WKV7_BF16 ? 2 : 4) * 4;     // fp32 [B, T, H, D]
        const int64_t gkv = gq / p.H * p.H_kv;                              // fp32 [B, T, H_kv, D]
        const Span spans[19] = {{r, z.q, "r"}, {w, z.q, "w"}, {k, z.kv, "k"}, {v, z.kv, "v"}, {a, z.q, "a"},
                                {b, z.q, "b"}, {state_in, z.state, "state_in"}, {dy, z.y, "dy"},
                                {dstate_out, z.state, "dstate_out"}, {dr, gq, "dr"}, {dw, gq, "dw"},
                                {dk, gkv, "dk"}, {dv, gkv, "dv"}, {da, gq, "da"}, {db, gq, "db"},
                                {dstate_in, z.state, "dstate_in"}, {dr_k, z.rk, "dr_k"},
                                {p.mask, z.mask, "mask"}, {p.r_k, z.rk, "r_k"}};
        if ((rc = check_workspace_disjoint(workspace, need, spans, 19))) return rc;
    }
    p.r = r; p.w = w; p.k = k; p.v = v; p.a = a; p.b = b;
    p.s0 = state_in; p.y = nullptr; p.s1 = nullptr;
    if (int64_t(p.B) * p.H == 0) return WKV7_OK;
    if ((rc = check_device())) return rc;
    wkv7::BwdIo io{dy, dstate_out, dr, dw, da, db, dk, dv, dstate_in, dr_k};
    return finish_launch(wkv7::launch_backward(p, io, workspace, reinterpret_cast<hipStream_t>(stream)), "backward");
}

}  // extern "C"

namespace {

int check_wkv4(const wkv4_desc* d) {
    if (!d) return fail(WKV7_EINVAL, "desc is NULL");
    if (d->spin_limit < 0) return fail(WKV7_EINVAL, "desc->spin_limit must be >= 0 (got %d)", d->spin_limit);
    if (d->B < 0 || d->T < 0 || d->C < 0)
        return fail(WKV7_EINVAL, "negative size (B=%d T=%d C=%d)", d->B, d->T, d->C);
    if (d->in_dtype != WKV7_F32 && d->in_dtype != WKV7_BF16)
        return fail(WKV7_EINVAL, "in_dtype %d unknown", d->in_dtype);
    if (d->y_dtype != WKV7_F32 && d->y_dtype != WKV7_BF16)
        return fail(WKV7_EINVAL, "y_dtype %d unknown", d->y_dtype);
    if (int64_t(d->B) * d->T * d->C > (int64_t(1) << 46)) return fail(WKV7_EUNSUPPORTED, "B*T*C too large");
    if (d->B > 65535 || (int64_t(d->T) + 63) / 64 > 65535)
        return fail(WKV7_EUNSUPPORTED, "B=%d or T=%d beyond the grid limits", d->B, d->T);
    // Byte offsets inside one 64-token chunk are 32-bit.
    if (int64_t(d->C) * 64 * 4 >= (int64_t(1) << 31)) return fail(WKV7_EUNSUPPORTED, "C=%d too large", d->C);
    return WKV7_OK;
}

}  // namespace

extern "C" {

int64_t wkv4_workspace_bytes(const wkv4_desc* desc) {
    g_last_error[0] = '\0';
    int rc = check_wkv4(desc);
    if (rc) return -rc;
    return wkv7::wkv4_workspace_bytes_internal(desc->B, desc->T, desc->C);
}

int wkv4_forward(const wkv4_desc* desc, const float* w, const float* u, const void* k, const void* v,
                 const float* state_in, void* y, float* state_out, void* workspace,
                 int64_t workspace_bytes_given, void* stream) {
    g_last_error[0] = '\0';
    int rc = check_wkv4(desc);
    if (rc) return rc;
    const int64_t bc = int64_t(desc->B) * desc->C;
    const bool has_tokens = bc * desc->T > 0;
    if (bc > 0) {
        if (!w || !u) return fail(WKV7_EINVAL, "w or u is NULL");
        if (!aligned16(w) || !aligned16(u)) return fail(WKV7_EINVAL, "w or u is not 16-byte aligned");
    }
    if (has_tokens) {
        const void* ptrs[3] = {k, v, y};
        static const char* names[3] = {"k", "v", "y"};
        for (int i = 0; i < 3; ++i) {
            if (!ptrs[i]) return fail(WKV7_EINVAL, "%s is NULL", names[i]);
            if (!aligned16(ptrs[i])) return fail(WKV7_EINVAL, "%s is not 16-byte aligned", names[i]);
        }
        if (y == k || y == v) return fail(WKV7_EINVAL, "y aliases an input");
    }
    if (state_in && !aligned16(state_in)) return fail(WKV7_EINVAL, "state_in is not 16-byte aligned");
    if (state_out && !aligned16(state_out)) return fail(WKV7_EINVAL, "state_out is not 16-byte aligned");
    const int64_t need = has_tokens ? wkv7::wkv4_workspace_bytes_internal(desc->B, desc->T, desc->C) : 0;
    if (need > 0) {
        if (!workspace) return fail(WKV7_EINVAL, "workspace is NULL (%lld bytes needed)", (long long)need);
        if (!aligned16(workspace)) return fail(WKV7_EINVAL, "workspace is not 16-byte aligned");
        if (workspace_bytes_given < need)
            return fail(WKV7_EINVAL, "workspace has %lld bytes, %lld needed",
                        (long long)workspace_bytes_given, (long long)need);
        const int64_t btc = bc * desc->T;
        const int64_t sin = desc->in_dtype == WKV7_BF16 ? 2 : 4, sy = desc->y_dtype == WKV7_BF16 ? 2 : 4;
        const Span spans[7] = {{w, int64_t(desc->C) * 4, "w"}, {u, int64_t(desc->C) * 4, "u"},
                               {k, btc * sin, "k"}, {v, btc * sin, "v"}, {y, btc * sy, "y"},
                               {state_in, bc * 3 * 4, "state_in"}, {state_out, bc * 3 * 4, "state_out"}};
        if ((rc = check_workspace_disjoint(workspace, need, spans, 7))) return rc;
    }
    if (bc == 0) return WKV7_OK;
    if (!has_tokens && !state_out) return WKV7_OK;
    if ((rc = check_device())) return rc;
    wkv7::Wkv4Params p{desc->B, desc->T, desc->C, desc->in_dtype, desc->y_dtype, desc->spin_limit, w, u, k, v, y,
                       state_in, state_out, workspace};
    return finish_launch(wkv7::launch_wkv4(p, reinterpret_cast<hipStream_t>(stream)), "wkv4");
}

int wkv4_wait_status(const wkv4_desc* desc, const void* workspace, int64_t workspace_bytes_given, void* stream) {
    g_last_error[0] = '\0';
    int rc = check_wkv4(desc);
    if (rc) return rc;
    const bool has_tokens = int64_t(desc->B) * desc->T * desc->C > 0;
    const int64_t need = has_tokens ? wkv7::wkv4_workspace_bytes_internal(desc->B, desc->T, desc->C) : 0;
    if (need == 0) return WKV7_OK;
    if (!workspace) return fail(WKV7_EINVAL, "workspace is NULL (%lld bytes needed)", (long long)need);
    if (workspace_bytes_given < need)
        return fail(WKV7_EINVAL, "workspace has %lld bytes, %lld needed", (long long)workspace_bytes_given,
                    (long long)need);
    if ((rc = check_device())) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int32_t count = 0;
    const char* src = static_cast<const char*>(workspace) + wkv7::wkv4_wait_counter_offset(desc->B, desc->T, desc->C);
    hipError_t e = hipMemcpyAsync(&count, src, sizeof(count), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(WKV7_EDEVICE, "reading the wait count: %s", hipGetErrorString(e));
    if (count > 0)
        return fail(WKV7_ETIMEOUT, "%d look-back wait(s) gave up; y is NaN in their chunks", int(count));
    return WKV7_OK;
}

int wkv7_resolve_algo(const wkv7_desc* desc) {
    wkv7::Params p{};
    int rc = check_desc(desc, &p);
    if (rc) return -rc;
    return resolve_algo(p, desc->algo, false);
}

const char* wkv7_strerror(int code) {
    switch (code) {
        case WKV7_OK: return "ok";
        case WKV7_EINVAL: return "invalid argument";
        case WKV7_EUNSUPPORTED: return "unsupported configuration";
        case WKV7_EDEVICE: return "unsupported or unavailable device";
        case WKV7_ELAUNCH: return "kernel launch failed";
        case WKV7_ETIMEOUT: return "a bounded device-side wait gave up";
        default: return "unknown status";
    }
}

const char* wkv7_last_error(void) { return g_last_error; }

int wkv7_abi_version(void) { return WKV7_ABI_VERSION; }

}  // extern "C"
