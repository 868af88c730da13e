// Rolling-window KV-cache decode step for CDNA4 (gfx950).
//
// One query token per sequence attends to the n = min(pos, W) valid slots of
// a W-slot ring that holds absolute position t in slot (t-1) % W (page
// "SWA：滑动窗口注意力与跨层信息传递", §4.2: a per-layer rolling cache of at
// most W rows; token-by-token inference reads only that cache).  The
// attention has no positional term, so the valid slots are reduced in slot
// order; which slots are valid is all that depends on pos.
//
// The step is bound by HBM bandwidth (about 4 flops per byte), so it is split
// along the slots ("split-K"): grid = (splits, KV heads, sequences), each
// workgroup streams up to 512 slots of one KV head in 64-slot tiles and
// serves all G query heads of that KV head, so every K/V byte is read from
// HBM once.  Per tile:
//   * K rows are copied HBM -> LDS with 16-byte coalesced loads (double
//     buffered); V rows go HBM -> registers in the layout the P*V step uses.
//   * scores: one (head, slot) pair per lane, a full-row dot product from LDS
//     (bf16 pairs through v_dot2, fp32 through fma);
//   * online softmax per head across the wave (log2 domain);
//   * P*V: lane = (16-byte column chunk, row group), fp32 accumulators.
// The workgroup writes (max, sum, weighted V) per head to the workspace; a
// second kernel merges the splits by log-sum-exp rescaling.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <type_traits>

#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTile = 64;

// XOR swizzle of 16-byte chunks by row: lane r reads row r, so the 8 lanes
// served together must hit 8 different chunk columns.
template <int RB>
__device__ __forceinline__ int kd_off(int row, int byte) {
    return row * RB + ((((byte >> 4) ^ (row & 7))) << 4) + (byte & 15);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Pair E of a bf16x8 value.  Taken with a vector shuffle: bit-casting a dword
// extracted from a u32x4 to bf16x2 mis-compiles (every pair becomes pair 0).
template <int E>
__device__ __forceinline__ bf16x2_t pair(bf16x8_t v) {
    return __builtin_shufflevector(v, v, 2 * E, 2 * E + 1);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
    using elem_t = typename std::conditional<BF, uint16_t, float>::type;
    constexpr int ES = (int)sizeof(elem_t);
    constexpr int RB = D * ES;          // bytes per ring row
    constexpr int CPR = RB / 16;        // 16-byte chunks per row
    constexpr int EPC = 16 / ES;        // elements per chunk
    constexpr int NCH = kTile * CPR / kThreads;   // K chunks per thread per tile
    constexpr int RG = kThreads / CPR;  // row groups of the P*V layout
    constexpr int RPT = kTile / RG;     // rows per thread per tile in P*V
    constexpr int HPW = (G + 3) / 4;    // heads per wave in the score phase
    static_assert(kTile * CPR % kThreads == 0 && kThreads % CPR == 0, "layout");

    __shared__ __attribute__((aligned(16))) char kl[2][kTile * RB];
    __shared__ __attribute__((aligned(16))) u32x4_t ql[G][CPR];      // query rows, raw
    __shared__ float pl[kTile][G];                                   // probabilities
    __shared__ float al[G];                                          // per-tile rescale

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int W = p.W;
    const int pb = p.pos[b];
    const int n = pb <= 0 ? 0 : min(pb, W);
    const int s0 = split * p.split_len;
    const int s1 = min(n, s0 + p.split_len);
    if (s0 >= s1) return;  // nothing valid here; the merge never reads this split

    const size_t ring = (size_t)(b * p.Hkv + kvh) * (size_t)W * D;
    const elem_t* kg = (const elem_t*)p.kring + ring;
    const elem_t* vg = (const elem_t*)p.vring + ring;
    const int h0 = kvh * G;  // first query head of this KV head

    // query rows -> LDS (sign of the scale folded in exactly)
    for (int u = tid; u < G * CPR; u += kThreads) {
        const int hh = u / CPR, ch = u % CPR;
        u32x4_t w = *(const u32x4_t*)((const char*)p.q + ((size_t)(b * p.Hq + h0 + hh) * D) * ES + ch * 16);
        if (p.neg) w ^= (BF ? 0x80008000u : 0x80000000u);
        ql[hh][ch] = w;
    }

    const int ntile = (s1 - s0 + kTile - 1) / kTile;
    u32x4_t kr[NCH], vr[RPT], vn[RPT];
    auto load_k = [&](int t) {
        const int base = s0 + t * kTile;
#pragma unroll
        for (int it = 0; it < NCH; ++it) {
            const int u = tid + kThreads * it;
            const int row = u / CPR, ch = u % CPR;
            u32x4_t w = {0u, 0u, 0u, 0u};
            if (base + row < s1) w = *(const u32x4_t*)((const char*)(kg + (size_t)(base + row) * D) + ch * 16);
            kr[it] = w;
        }
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int it = 0; it < NCH; ++it) {
            const int u = tid + kThreads * it;
            const int row = u / CPR, ch = u % CPR;
            *(u32x4_t*)(kl[buf] + kd_off<RB>(row, ch * 16)) = kr[it];
        }
    };
    const int dc = tid % CPR, rg = tid / CPR;
    auto load_v = [&](int t, u32x4_t* dst) {
        const int base = s0 + t * kTile;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int row = rg + RG * k;
            u32x4_t w = {0u, 0u, 0u, 0u};
            if (base + row < s1) w = *(const u32x4_t*)((const char*)(vg + (size_t)(base + row) * D) + dc * 16);
            dst[k] = w;
        }
    };

    float m_h[HPW], l_h[HPW];
#pragma unroll
    for (int k = 0; k < HPW; ++k) { m_h[k] = -INFINITY; l_h[k] = 0.f; }
    float acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;

    load_k(0);
    load_v(0, vr);
    store_k(0);
    __syncthreads();

    for (int t = 0; t < ntile; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntile) {
            load_k(t + 1);
            load_v(t + 1, vn);
        }
        // ---- scores and softmax: wave w owns heads w, w+4, ...
        const int base = s0 + t * kTile;
#pragma unroll
        for (int k = 0; k < HPW; ++k) {
            const int hh = wave + 4 * k;
            if (hh < G) {
                float dot = 0.f;
#pragma unroll
                for (int ch = 0; ch < CPR; ++ch) {
                    const u32x4_t kw = *(const u32x4_t*)(kl[buf] + kd_off<RB>(lane, ch * 16));
                    const u32x4_t qw = ql[hh][ch];
                    if constexpr (BF) {
                        const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kw);
                        const bf16x8_t q8 = __builtin_bit_cast(bf16x8_t, qw);
                        dot = __builtin_amdgcn_fdot2_f32_bf16(pair<0>(k8), pair<0>(q8), dot, false);
                        dot = __builtin_amdgcn_fdot2_f32_bf16(pair<1>(k8), pair<1>(q8), dot, false);
                        dot = __builtin_amdgcn_fdot2_f32_bf16(pair<2>(k8), pair<2>(q8), dot, false);
                        dot = __builtin_amdgcn_fdot2_f32_bf16(pair<3>(k8), pair<3>(q8), dot, false);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) dot = fmaf(__uint_as_float(kw[e]), __uint_as_float(qw[e]), dot);
                    }
                }
                const float s = (base + lane < s1) ? dot * p.c : -INFINITY;
                const float m_new = fmaxf(m_h[k], wave_max(s));
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_h[k] - m_use);
                const float e = __builtin_amdgcn_exp2f(s - m_use);
                m_h[k] = m_new;
                l_h[k] = l_h[k] * alpha + e;
                pl[lane][hh] = e;
                if (lane == 0) al[hh] = alpha;
            }
        }
        __syncthreads();
        // ---- P*V
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float a = al[hh];
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[hh][e] *= a;
        }
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int row = rg + RG * k;
            float vv[EPC];
            if constexpr (BF) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vv[2 * e] = bf_lo(vr[k][e]);
                    vv[2 * e + 1] = bf_hi(vr[k][e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e] = __uint_as_float(vr[k][e]);
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float pr = pl[row][hh];
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[hh][e] = fmaf(pr, vv[e], acc[hh][e]);
            }
        }
        if (t + 1 < ntile) {
            store_k(buf ^ 1);
#pragma unroll
            for (int k = 0; k < RPT; ++k) vr[k] = vn[k];
        }
        __syncthreads();
    }

    // ---- reduce the row groups: first inside the wave (lanes with the same
    // chunk), then across the 4 waves through LDS (reusing the K buffers).
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], o, 64);
    float* red = (float*)&kl[0][0];  // [4 waves][G][D] floats
    static_assert(4 * G * D * 4 <= 2 * kTile * RB, "reduction buffer");
    if (lane < CPR) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < EPC; ++e) red[(wave * G + hh) * D + lane * EPC + e] = acc[hh][e];
    }
    const size_t part = ((size_t)(b * p.Hq + h0) * p.nsplit + split);  // head hh adds hh * nsplit
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const int hh = wave + 4 * k;
        if (hh < G) {
            const float l = wave_sum(l_h[k]);
            if (lane == 0) {
                p.ws_ml[(part + (size_t)hh * p.nsplit) * 2 + 0] = m_h[k];
                p.ws_ml[(part + (size_t)hh * p.nsplit) * 2 + 1] = l;
            }
        }
    }
    __syncthreads();
    for (int u = tid; u < G * D; u += kThreads) {
        const int hh = u / D, d = u % D;
        const float s = red[(0 * G + hh) * D + d] + red[(1 * G + hh) * D + d] + red[(2 * G + hh) * D + d] +
                        red[(3 * G + hh) * D + d];
        p.ws_acc[(part + (size_t)hh * p.nsplit) * D + d] = s;
    }
}

// Merge the splits of one (sequence, query head): weights 2^(m_s - M).
template <bool BF, int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
    using elem_t = typename std::conditional<BF, uint16_t, float>::type;
    const int bh = blockIdx.x;
    const int b = bh / p.Hq;
    const int d = threadIdx.x;
    const int pb = p.pos[b];
    const int n = pb <= 0 ? 0 : min(pb, p.W);
    const int ns = (n + p.split_len - 1) / p.split_len;
    const float* ml = p.ws_ml + (size_t)bh * p.nsplit * 2;
    const float* ac = p.ws_acc + (size_t)bh * p.nsplit * D;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
        L = fmaf(ml[2 * s + 1], w, L);
        if (d < D) o = fmaf(ac[(size_t)s * D + d], w, o);
    }
    const float r = (ns > 0) ? o / L : 0.f;
    if (d < D) {
        elem_t* out = (elem_t*)p.out + (size_t)bh * D + d;
        if constexpr (BF) {
            const __bf16 x = (__bf16)r;
            *out = __builtin_bit_cast(uint16_t, x);
        } else {
            *out = r;
        }
    }
}

template <bool BF, int D, int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
    hipLaunchKernelGGL((decode_split_kernel<BF, D, G>), dim3(p.nsplit, p.Hkv, p.B), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<BF, D>), dim3(p.B * p.Hq), dim3(128), 0, s, p);
    return hipGetLastError();
}

template <bool BF, int D>
hipError_t launch_d(int G, const DecodeParams& p, hipStream_t s) {
    switch (G) {
        case 1: return launch_g<BF, D, 1>(p, s);
        case 2: return launch_g<BF, D, 2>(p, s);
        case 4: return launch_g<BF, D, 4>(p, s);
        default: return launch_g<BF, D, 8>(p, s);
    }
}

}  // namespace

hipError_t launch_decode(bool bf16, int d, int G, const DecodeParams& p, hipStream_t s) {
    if (bf16) return d == 128 ? launch_d<true, 128>(G, p, s) : launch_d<true, 64>(G, p, s);
    return d == 128 ? launch_d<false, 128>(G, p, s) : launch_d<false, 64>(G, p, s);
}

size_t decode_workspace_bytes(int B, int Hq, int W, int d) {
    const size_t nsplit = (size_t)(W + kDecodeSplit - 1) / kDecodeSplit;
    return (size_t)B * Hq * nsplit * ((size_t)d + 2) * sizeof(float);
}

}  // namespace swa
