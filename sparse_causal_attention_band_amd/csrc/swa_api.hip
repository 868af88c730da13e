// C ABI of the library: argument validation on the host, launch geometry,
// error reporting.  Declared in include/swa_attn.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <mutex>
#include <string>

#include "swa_attn.h"
#include "swa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return SWA_OK;
}

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

constexpr float kLog2e = 1.4426950408889634f;

int check_scale(const char* name, float scale) {
    if (!isfinite(scale) || scale == 0.f)
        return fail(SWA_ERR_INVALID_ARG, "%s: scale must be finite and non-zero (got %g)", name, (double)scale);
    return SWA_OK;
}

// Band forward shared by the causal entry points (right = 0) and the
// two-sided ones (stride = 0): row i reads keys max(0, i-window+1) ..
// min(N-1, i+right), plus the multiples of stride below the band.
// With q2/k2 (bf16 only, K/V arrays under 2 GiB per head): differential
// attention (A1 - lam A2) V in one pass of the 8-wave kernel.
int band_fwd(bool bf16, const char* name, const void* q, const void* k, const void* v, void* out, int B, int Hq,
             int Hkv, int N, int d, int window, int right, int stride, float scale, hipStream_t stream,
             const float* lam = nullptr, const int32_t* gidx = nullptr, int ng = 0, float* lse = nullptr,
             const void* q2 = nullptr, const void* k2 = nullptr) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1)
        return fail(SWA_ERR_INVALID_ARG, "%s: B, N, Hq, Hkv must be >= 1 (B=%d N=%d Hq=%d Hkv=%d)", name, B, N, Hq,
                    Hkv);
    if (Hq % Hkv != 0) return fail(SWA_ERR_INVALID_ARG, "%s: Hq (%d) must be a multiple of Hkv (%d)", name, Hq, Hkv);
    if (window < 1) return fail(SWA_ERR_INVALID_ARG, "%s: window must be >= 1 (got %d)", name, window);
    if (d != 64 && d != 128) return fail(SWA_ERR_UNSUPPORTED, "%s: head dim %d not built (64 or 128)", name, d);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(SWA_ERR_INVALID_ARG, "%s: q, k, v, out must be non-null and 16-byte aligned", name);
    const bool diff1 = q2 != nullptr || k2 != nullptr;
    if (diff1 && (!aligned16(q2) || !aligned16(k2)))
        return fail(SWA_ERR_INVALID_ARG, "%s: q2, k2 must be non-null and 16-byte aligned", name);
    if (int rc = check_scale(name, scale)) return rc;
    const long long es = bf16 ? 2 : 4;
    const long long qbytes = (long long)B * Hq * N * d * es;
    const long long kbytes = (long long)B * Hkv * N * d * es;
    auto overlap = [](const void* a, long long na, const void* b, long long nb) {
        const char* x = (const char*)a;
        const char* y = (const char*)b;
        return x < y + nb && y < x + na;
    };
    if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k, kbytes) || overlap(out, qbytes, v, kbytes))
        return fail(SWA_ERR_INVALID_ARG, "%s: out must not overlap q, k or v", name);
    if (lse != nullptr) {
        const long long lbytes = (long long)B * Hq * N * 4;
        if ((uintptr_t)lse & 3u) return fail(SWA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", name);
        if (overlap(lse, lbytes, out, qbytes) || overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
            overlap(lse, lbytes, v, kbytes))
            return fail(SWA_ERR_INVALID_ARG, "%s: lse must not overlap q, k, v or out", name);
    }
    const long long G = Hq / Hkv;
    const long long rows = (long long)N * d;
    if ((long long)B * Hq * rows > (1ll << 40)) return fail(SWA_ERR_UNSUPPORTED, "%s: tensor too large", name);

    swa::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.kring = nullptr;
    p.vring = nullptr;
    p.p0 = nullptr;
    p.q2 = q2;
    p.k2 = k2;
    p.lam = lam;
    p.lse = lse;
    p.gidx = gidx;
    p.ng = ng;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.W = window < N ? window : N;  // W >= N is full causal: identical work and bits
    p.wr = right < N ? right : N - 1;
    p.stride = stride > 0 ? stride : 0;
    p.c = fabsf(scale) * kLog2e;
    p.neg = scale < 0.f;
    p.G = (int)G;
    const int mode = diff1 ? swa::kDiff : ng > 0 ? swa::kGlobal : p.stride > 0 ? swa::kStrided : swa::kBand;
    // one-pass differential attention: 4 query blocks x 2 maps on 8 waves;
    // key split: 2 query blocks x 2 key halves on 4 waves
    p.ks = swa::key_split(bf16, mode, p.G) ? 1 : 0;
    const bool keylist = mode == swa::kStrided || (mode == swa::kGlobal && ng > swa::kMaxGlobal8);
    swa::set_wave_split(p, diff1 ? 4 : p.ks ? 2 : swa::waves_per_group(bf16, keylist, p.G, N, d), N);
    const long long total = (long long)B * Hkv * p.ngroups * p.nqb;
    if (total > 0x7fffffffll) return fail(SWA_ERR_UNSUPPORTED, "%s: grid too large", name);
    p.total = (int)total;
    p.nwg = p.HG * p.PB == 8 ? swa::persistent_workgroups(p.total) : p.total;  // persistent 8-wave kernel
    hipError_t e = swa::launch_band_fwd(bf16, d, mode, p, stream);
    if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
    return ok();
}

int attn_fwd(bool bf16, const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N,
             int d, int window, int stride, float scale, hipStream_t stream) {
    return band_fwd(bf16, bf16 ? "swa_attn_fwd" : "swa_attn_fwd_f32", q, k, v, out, B, Hq, Hkv, N, d, window, 0,
                    stride, scale, stream);
}

int attn_fwd_lse(bool bf16, const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                 int Hkv, int N, int d, int window, int stride, float scale, hipStream_t stream) {
    const char* name = bf16 ? "swa_attn_fwd_lse" : "swa_attn_fwd_lse_f32";
    if (lse == nullptr) return fail(SWA_ERR_INVALID_ARG, "%s: lse must be non-null", name);
    return band_fwd(bf16, name, q, k, v, out, B, Hq, Hkv, N, d, window, 0, stride, scale, stream, nullptr, nullptr, 0,
                    lse);
}

int two_sided_fwd(bool bf16, const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N,
                  int d, int left, int right, float scale, hipStream_t stream) {
    const char* name = bf16 ? "swa_attn_fwd_two_sided" : "swa_attn_fwd_two_sided_f32";
    if (left < 0 || right < 0)
        return fail(SWA_ERR_INVALID_ARG, "%s: left and right must be >= 0 (got %d, %d)", name, left, right);
    const int window = left < N ? left + 1 : (N > 0 ? N : 1);
    return band_fwd(bf16, name, q, k, v, out, B, Hq, Hkv, N, d, window, right, 0, scale, stream);
}

// Differential attention.  bf16 with windows under 512 and K/V arrays under
// 2 GiB per head: one pass of the 8-wave kernel, both maps over one tile
// stream (V staged once), the output rounded once.  Otherwise the first
// map's result is written to out, then a second launch subtracts lam[h]
// times its own result in its epilogue.  The one-pass workgroup holds four
// query blocks per map where a band launch holds eight, so it stages three
// tiles per step for half the rows: measured at 32/8 heads, d = 128,
// N = 16384, it is 5.6 % faster at W = 256 and 11-12 % slower from W = 1024
// on, where the second launch's fixed costs no longer dominate.
constexpr int kDiffOnePassMaxWindow = 511;
int diff_fwd(bool bf16, const void* q1, const void* k1, const void* q2, const void* k2, const void* v,
             const float* lam, void* out, int B, int Hq, int Hkv, int N, int d, int window, float scale,
             hipStream_t stream) {
    const char* name = bf16 ? "swa_diff_attn_fwd" : "swa_diff_attn_fwd_f32";
    if (lam == nullptr || ((uintptr_t)lam & 3u))
        return fail(SWA_ERR_INVALID_ARG, "%s: lam must be non-null, 4-byte aligned", name);
    if (B >= 1 && N >= 1 && Hq >= 1 && Hkv >= 1 && d >= 1) {
        const long long es = bf16 ? 2 : 4;
        const long long qbytes = (long long)B * Hq * N * d * es;
        const long long kbytes = (long long)B * Hkv * N * d * es;
        const char* o = (const char*)out;
        auto hits = [&](const void* a, long long na) {
            const char* x = (const char*)a;
            return x < o + qbytes && o < x + na;
        };
        if (hits(q2, qbytes) || hits(k2, kbytes) || hits(lam, (long long)Hq * 4))
            return fail(SWA_ERR_INVALID_ARG, "%s: out must not overlap q2, k2 or lam", name);
    }
    const bool one_pass = bf16 && d >= 1 && (long long)N * d * 2 < (1ll << 31) && window <= kDiffOnePassMaxWindow;
    if (one_pass)
        return band_fwd(bf16, name, q1, k1, v, out, B, Hq, Hkv, N, d, window, 0, 0, scale, stream, lam, nullptr, 0,
                        nullptr, q2, k2);
    if (int rc = band_fwd(bf16, name, q1, k1, v, out, B, Hq, Hkv, N, d, window, 0, 0, scale, stream)) return rc;
    return band_fwd(bf16, name, q2, k2, v, out, B, Hq, Hkv, N, d, window, 0, 0, scale, stream, lam);
}

size_t global_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int ng) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || ng < 1 || (long long)B * ng > 0x7fffffffll) return 0;
    return swa::decode_workspace_bytes(B * ng, Hq, Hkv, N, d);
}

// Local + global tokens: the band kernel with the global keys (every row
// reads the earlier global positions), then the global rows, which read
// every earlier key, recomputed by the split decode kernel in row mode
// over K/V as a linear cache of N slots; they overwrite the band result.
int global_fwd(bool bf16, const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N,
               int d, int window, const int32_t* gidx, int ng, float scale, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
    const char* name = bf16 ? "swa_attn_fwd_global" : "swa_attn_fwd_global_f32";
    if (ng < 0 || (N >= 1 && ng > N))
        return fail(SWA_ERR_INVALID_ARG, "%s: ng must be in 0..N (got %d)", name, ng);
    if (ng > 0) {
        if (gidx == nullptr || ((uintptr_t)gidx & 3u))
            return fail(SWA_ERR_INVALID_ARG, "%s: gidx must be non-null, 4-byte aligned", name);
        if (Hkv >= 1 && Hq % Hkv == 0) {
            const int G = Hq / Hkv;
            if (G != 1 && G != 2 && G != 4 && G != 8)
                return fail(SWA_ERR_UNSUPPORTED, "%s: Hq/Hkv = %d not built for global rows (1, 2, 4 or 8)", name, G);
        }
        if ((long long)B * ng > 65535 || Hkv > 65535)
            return fail(SWA_ERR_UNSUPPORTED, "%s: B * ng (%lld) too large", name, (long long)B * ng);
        const size_t need = global_workspace_bytes(B, Hq, Hkv, N, d, ng);
        if (need > 0 && !aligned16(workspace))
            return fail(SWA_ERR_INVALID_ARG, "%s: workspace must be non-null and 16-byte aligned", name);
        if (workspace_bytes < need)
            return fail(SWA_ERR_INVALID_ARG, "%s: workspace of %zu bytes is below the %zu needed", name,
                        workspace_bytes, need);
    }
    if (int rc = band_fwd(bf16, name, q, k, v, out, B, Hq, Hkv, N, d, window, 0, 0, scale, stream, nullptr,
                          ng > 0 ? gidx : nullptr, ng))
        return rc;
    if (ng == 0) return ok();
    swa::DecodeParams p{};
    p.q = q;
    p.kring = k;
    p.vring = v;
    p.pos = nullptr;
    p.out = out;
    p.B = B * ng;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.W = N;
    p.gidx = gidx;
    p.ng = ng;
    p.N = N;
    const swa::DecodeSplit plan = swa::decode_split_plan(p.B, Hkv, N);
    p.split_len = plan.split_len;
    p.nsplit = plan.nsplit;
    p.ws_acc = (float*)workspace;
    p.ws_ml = p.ws_acc + (size_t)p.B * Hq * p.nsplit * d;
    p.c = fabsf(scale) * kLog2e;
    p.neg = scale < 0.f;
    if ((long long)p.nsplit > 65535) return fail(SWA_ERR_UNSUPPORTED, "%s: grid too large", name);
    hipError_t e = swa::launch_decode(bf16, d, Hq / Hkv, p, stream);
    if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
    return ok();
}

int chunk_prefill(bool bf16, const void* q, const void* k, const void* v, const void* kring, const void* vring,
                  const int32_t* p0, void* out, int B, int Hq, int Hkv, int T, int d, int window, float scale,
                  hipStream_t stream, float* lse = nullptr, const char* name = nullptr) {
    if (name == nullptr) name = bf16 ? "swa_chunk_prefill" : "swa_chunk_prefill_f32";
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1)
        return fail(SWA_ERR_INVALID_ARG, "%s: B, T, Hq, Hkv must be >= 1 (B=%d T=%d Hq=%d Hkv=%d)", name, B, T, Hq,
                    Hkv);
    if (Hq % Hkv != 0) return fail(SWA_ERR_INVALID_ARG, "%s: Hq (%d) must be a multiple of Hkv (%d)", name, Hq, Hkv);
    if (window < 1) return fail(SWA_ERR_INVALID_ARG, "%s: window must be >= 1 (got %d)", name, window);
    if (d != 64 && d != 128) return fail(SWA_ERR_UNSUPPORTED, "%s: head dim %d not built (64 or 128)", name, d);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(kring) || !aligned16(vring))
        return fail(SWA_ERR_INVALID_ARG, "%s: q, k, v, kring, vring, out must be non-null and 16-byte aligned", name);
    if (p0 == nullptr || ((uintptr_t)p0 & 3u))
        return fail(SWA_ERR_INVALID_ARG, "%s: p0 must be non-null, 4-byte aligned", name);
    if (int rc = check_scale(name, scale)) return rc;
    if ((long long)T + window > 0x7fffffffll) return fail(SWA_ERR_UNSUPPORTED, "%s: T + window too large", name);
    if (lse != nullptr && ((uintptr_t)lse & 3u)) return fail(SWA_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", name);
    if (lse != nullptr) {
        const char* l0 = (const char*)lse;
        const long long lbytes = (long long)B * Hq * T * 4, obytes = (long long)B * Hq * T * d * (bf16 ? 2 : 4);
        const char* o0 = (const char*)out;
        if (l0 < o0 + obytes && o0 < l0 + lbytes)
            return fail(SWA_ERR_INVALID_ARG, "%s: lse must not overlap out", name);
    }
    const long long G = Hq / Hkv;
    swa::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.kring = kring;
    p.vring = vring;
    p.p0 = p0;
    p.lam = nullptr;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = T;
    p.W = window;  // the ring size; the kernel clamps the band to the keys it has
    p.wr = 0;
    p.stride = 0;
    p.c = fabsf(scale) * kLog2e;
    p.neg = scale < 0.f;
    p.G = (int)G;
    swa::set_wave_split(p, swa::waves_per_group(bf16, false, p.G, T > window ? T : window, d), T);
    const long long total = (long long)B * Hkv * p.ngroups * p.nqb;
    if (total > 0x7fffffffll) return fail(SWA_ERR_UNSUPPORTED, "%s: grid too large", name);
    p.total = (int)total;
    p.nwg = p.HG * p.PB == 8 ? swa::persistent_workgroups(p.total) : p.total;
    hipError_t e = swa::launch_band_fwd(bf16, d, swa::kChunk, p, stream);
    if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
    return ok();
}

int ring_append(bool bf16, const void* k, const void* v, const int32_t* p0, void* kring, void* vring, int B, int Hkv,
                int T, int d, int window, hipStream_t stream) {
    const char* name = bf16 ? "swa_ring_append" : "swa_ring_append_f32";
    if (B < 1 || T < 1 || Hkv < 1 || window < 1)
        return fail(SWA_ERR_INVALID_ARG, "%s: B, T, Hkv, window must be >= 1 (B=%d T=%d Hkv=%d window=%d)", name, B,
                    T, Hkv, window);
    if (d != 64 && d != 128) return fail(SWA_ERR_UNSUPPORTED, "%s: head dim %d not built (64 or 128)", name, d);
    if (!aligned16(k) || !aligned16(v) || !aligned16(kring) || !aligned16(vring))
        return fail(SWA_ERR_INVALID_ARG, "%s: k, v, kring, vring must be non-null and 16-byte aligned", name);
    if (p0 == nullptr || ((uintptr_t)p0 & 3u))
        return fail(SWA_ERR_INVALID_ARG, "%s: p0 must be non-null, 4-byte aligned", name);
    if (B > 65535 || Hkv > 65535) return fail(SWA_ERR_UNSUPPORTED, "%s: grid too large", name);
    hipError_t e = swa::launch_ring_append(bf16 ? 2 : 4, d, k, v, p0, kring, vring, B, Hkv, T, window, stream);
    if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
    return ok();
}

// Scratch of the allocation-free decode entry point: the split partials
// ([B, Hq, nsplit, d] sums, then [B, Hq, nsplit, 2] (max, sum)).  The split
// plan splits only below 256 (sequence, KV head) pairs, so pairs x splits
// stays under 512 (at most 255 x 2) and the partials under 8 heads per KV
// head x 510 x (128 + 2) floats.  Each GPU holds its own copy; host code never names the
// array itself (on the host the name is only a handle), it uses the device
// address looked up once per device.
constexpr size_t kNoAllocScratchBytes = SWA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there, with that device current); nullptr with an error on failure.
void* scratch_on_current_device(const char* name, int* rc) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = fail(SWA_ERR_HIP, "%s: hipGetDevice failed: %s", name, hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *rc = fail(SWA_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", name, dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            *rc = fail(SWA_ERR_HIP, "%s: scratch address lookup failed on device %d: %s", name, dev,
                       hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Decode step.  With use_scratch the workspace arguments are ignored and the
// split partials go to this device's copy of `scratch` (allocation-free
// entry point).
int decode(bool bf16, const void* q, const void* kring, const void* vring, const int32_t* pos, void* out, int B,
           int Hq, int Hkv, int d, float scale, void* workspace, size_t workspace_bytes, int window,
           hipStream_t stream, const char* name = nullptr, bool use_scratch = false) {
    if (name == nullptr) name = bf16 ? "swa_decode" : "swa_decode_f32";
    if (B < 1 || Hq < 1 || Hkv < 1)
        return fail(SWA_ERR_INVALID_ARG, "%s: B, Hq, Hkv must be >= 1 (B=%d Hq=%d Hkv=%d)", name, B, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(SWA_ERR_INVALID_ARG, "%s: Hq (%d) must be a multiple of Hkv (%d)", name, Hq, Hkv);
    if (window < 1) return fail(SWA_ERR_INVALID_ARG, "%s: window must be >= 1 (got %d)", name, window);
    if (d != 64 && d != 128) return fail(SWA_ERR_UNSUPPORTED, "%s: head dim %d not built (64 or 128)", name, d);
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(SWA_ERR_UNSUPPORTED, "%s: Hq/Hkv = %d not built (1, 2, 4 or 8)", name, G);
    if (!aligned16(q) || !aligned16(kring) || !aligned16(vring) || !aligned16(out))
        return fail(SWA_ERR_INVALID_ARG, "%s: q, kring, vring, out must be non-null and 16-byte aligned", name);
    if (pos == nullptr || ((uintptr_t)pos & 3u)) return fail(SWA_ERR_INVALID_ARG, "%s: pos must be non-null, 4-byte aligned", name);
    if (int rc = check_scale(name, scale)) return rc;
    const size_t need = swa::decode_workspace_bytes(B, Hq, Hkv, window, d);
    if (use_scratch) {
        if (need > kNoAllocScratchBytes)
            return fail(SWA_ERR_UNSUPPORTED, "%s: the split partials need %zu bytes, above the %zu-byte scratch",
                        name, need, kNoAllocScratchBytes);
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            int rc = SWA_OK;
            workspace = scratch_on_current_device(name, &rc);
            if (workspace == nullptr) return rc;
            workspace_bytes = kNoAllocScratchBytes;
        }
    }
    if (need > 0 && !aligned16(workspace))
        return fail(SWA_ERR_INVALID_ARG, "%s: workspace must be non-null and 16-byte aligned", name);
    if (workspace_bytes < need)
        return fail(SWA_ERR_INVALID_ARG, "%s: workspace of %zu bytes is below the %zu needed", name, workspace_bytes,
                    need);
    swa::DecodeParams p{};
    p.q = q;
    p.kring = kring;
    p.vring = vring;
    p.pos = pos;
    p.out = out;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.W = window;
    const swa::DecodeSplit plan = swa::decode_split_plan(B, Hkv, window);
    p.split_len = plan.split_len;
    p.nsplit = plan.nsplit;
    p.ws_acc = (float*)workspace;
    p.ws_ml = p.ws_acc + (size_t)B * Hq * p.nsplit * d;
    p.c = fabsf(scale) * kLog2e;
    p.neg = scale < 0.f;
    if ((long long)p.nsplit > 65535 || Hkv > 65535 || B > 65535)
        return fail(SWA_ERR_UNSUPPORTED, "%s: grid too large", name);
    hipError_t e = swa::launch_decode(bf16, d, G, p, stream);
    if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int swa_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N, int d,
                 int window, int stride, float scale, hipStream_t stream) {
    return attn_fwd(true, q, k, v, out, B, Hq, Hkv, N, d, window, stride, scale, stream);
}

int swa_attn_fwd_f32(const float* q, const float* k, const float* v, float* out, int B, int Hq, int Hkv, int N, int d,
                     int window, int stride, float scale, hipStream_t stream) {
    return attn_fwd(false, q, k, v, out, B, Hq, Hkv, N, d, window, stride, scale, stream);
}

int swa_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int N,
                     int d, int window, int stride, float scale, hipStream_t stream) {
    return attn_fwd_lse(true, q, k, v, out, lse, B, Hq, Hkv, N, d, window, stride, scale, stream);
}

int swa_attn_fwd_lse_f32(const float* q, const float* k, const float* v, float* out, float* lse, int B, int Hq,
                         int Hkv, int N, int d, int window, int stride, float scale, hipStream_t stream) {
    return attn_fwd_lse(false, q, k, v, out, lse, B, Hq, Hkv, N, d, window, stride, scale, stream);
}

int swa_decode(const void* q, const void* kring, const void* vring, const int32_t* pos, void* out, int B, int Hq,
               int Hkv, int d, float scale, void* workspace, size_t workspace_bytes, int window, hipStream_t stream) {
    return decode(true, q, kring, vring, pos, out, B, Hq, Hkv, d, scale, workspace, workspace_bytes, window, stream);
}

int swa_decode_f32(const float* q, const float* kring, const float* vring, const int32_t* pos, float* out, int B,
                   int Hq, int Hkv, int d, float scale, void* workspace, size_t workspace_bytes, int window,
                   hipStream_t stream) {
    return decode(false, q, kring, vring, pos, out, B, Hq, Hkv, d, scale, workspace, workspace_bytes, window, stream);
}

int swa_attn_fwd_two_sided(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N,
                           int d, int left, int right, float scale, hipStream_t stream) {
    return two_sided_fwd(true, q, k, v, out, B, Hq, Hkv, N, d, left, right, scale, stream);
}

int swa_attn_fwd_two_sided_f32(const float* q, const float* k, const float* v, float* out, int B, int Hq, int Hkv,
                               int N, int d, int left, int right, float scale, hipStream_t stream) {
    return two_sided_fwd(false, q, k, v, out, B, Hq, Hkv, N, d, left, right, scale, stream);
}

int swa_diff_attn_fwd(const void* q1, const void* k1, const void* q2, const void* k2, const void* v, const float* lam,
                      void* out, int B, int Hq, int Hkv, int N, int d, int window, float scale, hipStream_t stream) {
    return diff_fwd(true, q1, k1, q2, k2, v, lam, out, B, Hq, Hkv, N, d, window, scale, stream);
}

int swa_diff_attn_fwd_f32(const float* q1, const float* k1, const float* q2, const float* k2, const float* v,
                          const float* lam, float* out, int B, int Hq, int Hkv, int N, int d, int window, float scale,
                          hipStream_t stream) {
    return diff_fwd(false, q1, k1, q2, k2, v, lam, out, B, Hq, Hkv, N, d, window, scale, stream);
}

int swa_attn_fwd_global(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N, int d,
                        int window, const int32_t* gidx, int ng, float scale, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return global_fwd(true, q, k, v, out, B, Hq, Hkv, N, d, window, gidx, ng, scale, workspace, workspace_bytes,
                      stream);
}

int swa_attn_fwd_global_f32(const float* q, const float* k, const float* v, float* out, int B, int Hq, int Hkv, int N,
                            int d, int window, const int32_t* gidx, int ng, float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    return global_fwd(false, q, k, v, out, B, Hq, Hkv, N, d, window, gidx, ng, scale, workspace, workspace_bytes,
                      stream);
}

size_t swa_attn_fwd_global_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int ng) {
    return global_workspace_bytes(B, Hq, Hkv, N, d, ng);
}

int swa_chunk_prefill(const void* q, const void* k, const void* v, const void* kring, const void* vring,
                      const int32_t* p0, void* out, int B, int Hq, int Hkv, int T, int d, int window, float scale,
                      hipStream_t stream) {
    return chunk_prefill(true, q, k, v, kring, vring, p0, out, B, Hq, Hkv, T, d, window, scale, stream);
}

int swa_chunk_prefill_f32(const float* q, const float* k, const float* v, const float* kring, const float* vring,
                          const int32_t* p0, float* out, int B, int Hq, int Hkv, int T, int d, int window,
                          float scale, hipStream_t stream) {
    return chunk_prefill(false, q, k, v, kring, vring, p0, out, B, Hq, Hkv, T, d, window, scale, stream);
}

int swa_chunk_prefill_lse(const void* q, const void* k, const void* v, const void* kring, const void* vring,
                          const int32_t* p0, void* out, float* lse, int B, int Hq, int Hkv, int T, int d, int window,
                          float scale, hipStream_t stream) {
    if (lse == nullptr) return fail(SWA_ERR_INVALID_ARG, "swa_chunk_prefill_lse: lse must be non-null");
    return chunk_prefill(true, q, k, v, kring, vring, p0, out, B, Hq, Hkv, T, d, window, scale, stream, lse,
                         "swa_chunk_prefill_lse");
}

int swa_chunk_prefill_lse_f32(const float* q, const float* k, const float* v, const float* kring, const float* vring,
                              const int32_t* p0, float* out, float* lse, int B, int Hq, int Hkv, int T, int d,
                              int window, float scale, hipStream_t stream) {
    if (lse == nullptr) return fail(SWA_ERR_INVALID_ARG, "swa_chunk_prefill_lse_f32: lse must be non-null");
    return chunk_prefill(false, q, k, v, kring, vring, p0, out, B, Hq, Hkv, T, d, window, scale, stream, lse,
                         "swa_chunk_prefill_lse_f32");
}

int swa_ring_append(const void* k, const void* v, const int32_t* p0, void* kring, void* vring, int B, int Hkv, int T,
                    int d, int window, hipStream_t stream) {
    return ring_append(true, k, v, p0, kring, vring, B, Hkv, T, d, window, stream);
}

int swa_ring_append_f32(const float* k, const float* v, const int32_t* p0, float* kring, float* vring, int B, int Hkv,
                        int T, int d, int window, hipStream_t stream) {
    return ring_append(false, k, v, p0, kring, vring, B, Hkv, T, d, window, stream);
}

int swa_decode_noalloc(const void* q, const void* kring, const void* vring, const int32_t* pos, void* out, int B,
                       int Hq, int Hkv, int d, float scale, int window, hipStream_t stream) {
    return decode(true, q, kring, vring, pos, out, B, Hq, Hkv, d, scale, nullptr, 0, window, stream,
                  "swa_decode_noalloc", true);
}

size_t swa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int window) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || window < 1 || (d != 64 && d != 128)) return 0;
    return swa::decode_workspace_bytes(B, Hq, Hkv, window, d);
}

const char* swa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
