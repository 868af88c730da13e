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
// along the slots ("split-K") only as far as needed to give every CU one
// workgroup: grid = (splits, KV heads, sequences), each workgroup streams
// its slots of one KV head in 64-slot tiles and serves all G query heads of
// that KV head, so every K/V byte is read from HBM once.  With one split
// (256 or more (sequence, KV head) pairs) the workgroup writes the output
// itself.  The kernel is a pure register stream:
//   * 16-byte chunks per lane, a ring row of d elements spread over CPR
//     consecutive lanes: a 256-byte bf16 row over 8 lanes with two chunks
//     each (chunks c and c + 8, so every load instruction reads whole
//     128-byte lines) where up to four query heads share the KV head, else
//     one chunk per lane; a 3-deep ring of tiles in registers so two more
//     tiles are in flight while one is consumed; the loads are non-temporal
//     (each byte is read once per step);
//   * scores: per-lane partial dot products (v_dot2 on bf16 pairs), summed
//     over the lanes of a row with DPP row permutes;
//   * each group of lanes sharing a row keeps its own online softmax (max,
//     sum, weighted V for its d-chunk) -- no barrier and no LDS in the loop;
//   * P*V: two rows at a time, bf16 V values of the two rows interleaved with
//     v_perm so one v_dot2 adds both rows' contribution (P rounded to bf16,
//     and the sum taken over the same rounded P);
//   * at the end the row groups are merged (log-sum-exp) through LDS, and the
//     workgroup writes (max, sum, weighted V) per head to the workspace.
// With several splits a second kernel merges them by log-sum-exp rescaling.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <type_traits>

#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kTile = 64;

// Pair E of a bf16x8 value.  Taken with a vector shuffle: bit-casting a dword
// extracted from a u32x4 to bf16x2 mis-compiles (every pair becomes pair 0).
template <int E>
__device__ __forceinline__ bf16x2_t pair(bf16x8_t v) {
    return __builtin_shufflevector(v, v, 2 * E, 2 * E + 1);
}

// Sum over the LANES consecutive lanes that hold one row (LANES = 8, 16 or 32).
template <int LANES>
__device__ __forceinline__ float row_sum(float x) {
    // xor 1 and xor 2 inside quads, then the 8- and 16-lane mirrors (all DPP)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
    if constexpr (LANES >= 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));
    if constexpr (LANES >= 32) x += __shfl_xor(x, 16, 64);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Where entry e reads its query rows and writes its output rows: element
// offset of head 0 and the stride between heads; its KV sequence and the
// number of positions it has (decode: pos[e]; row mode: row gidx + 1).
struct EntryRows {
    size_t row0, head_stride;
    int seq, pos;
};
template <bool GR, int D>
__device__ __forceinline__ EntryRows entry_rows(const DecodeParams& p, int e) {
    EntryRows r;
    if constexpr (GR) {
        const int b = e / p.ng;
        const int i = min(max(p.gidx[e % p.ng], 0), p.N - 1);
        r.seq = b;
        r.pos = i + 1;
        r.row0 = ((size_t)b * p.Hq * p.N + i) * D;
        r.head_stride = (size_t)p.N * D;
    } else {
        r.seq = e;
        r.pos = p.pos[e];
        r.row0 = (size_t)e * p.Hq * D;
        r.head_stride = D;
    }
    return r;
}

template <bool BF, int D, int G, bool GR>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeParams p) {
    using elem_t = typename std::conditional<BF, uint16_t, float>::type;
    constexpr int ES = (int)sizeof(elem_t);
    constexpr int RB = D * ES;          // bytes per ring row
    // 16-byte chunks per lane: two for bf16 rows of 128 with up to four heads
    // per KV head (a row over 8 lanes: half the cross-lane sums and
    // exponentials per lane), else one
    constexpr int CW = (BF && D == 128 && G <= 4) ? 2 : 1;
    constexpr int CPR = RB / (16 * CW);  // lanes per row
    constexpr int EPC = 16 / ES;        // elements per chunk
    constexpr int RG = kThreads / CPR;  // row groups per workgroup
    constexpr int RPT = kTile / RG;     // rows per lane per tile
    // tiles held in registers (fewer where the row and head count need the room)
    constexpr int PD = BF ? (G >= 8 ? 2 : 3) : (CPR >= 32 ? 1 : 2);
    static_assert(CPR == 8 || CPR == 16 || CPR == 32, "row width");
    static_assert(!BF || RPT % 2 == 0, "rows are paired for v_dot2");

    __shared__ float sm_ml[RG][G][2];
    __shared__ float sm_acc[RG][G][D];

    const int tid = threadIdx.x;
    const int dc = tid % CPR, rg = tid / CPR;
    const int split = blockIdx.x, kvh = blockIdx.y;
    const EntryRows er = entry_rows<GR, D>(p, blockIdx.z);
    const int b = er.seq;
    const int W = p.W;
    const int pb = er.pos;
    const int n = pb <= 0 ? 0 : min(pb, W);
    const int s0 = split * p.split_len;
    const int s1 = min(n, s0 + p.split_len);
    if (s0 >= s1) {
        // nothing valid here: the merge never reads this split; without a
        // merge (one split) this is a pos <= 0 row, which is all zeros
        if (p.nsplit == 1)
            for (int u = tid; u < G * D; u += kThreads)
                ((elem_t*)p.out)[er.row0 + (size_t)(kvh * G + u / D) * er.head_stride + u % D] = (elem_t)0;
        return;
    }

    const size_t ring = (size_t)(b * p.Hkv + kvh) * (size_t)W * D;
    const char* kg = (const char*)((const elem_t*)p.kring + ring) + dc * 16;
    const char* vg = (const char*)((const elem_t*)p.vring + ring) + dc * 16;
    const int h0 = kvh * G;

    // this lane's 16-byte chunks (dc, dc + CPR, ...) of every query row (sign
    // of the scale folded in)
    u32x4_t qc[G][CW];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            u32x4_t w = *(const u32x4_t*)((const char*)p.q + (er.row0 + (size_t)(h0 + hh) * er.head_stride) * ES +
                                          (dc + c * CPR) * 16);
            if (p.neg) w ^= (BF ? 0x80008000u : 0x80000000u);
            qc[hh][c] = w;
        }

    const int ntile = (s1 - s0 + kTile - 1) / kTile;
    u32x4_t kr[PD][RPT][CW], vr[PD][RPT][CW];
    auto load = [&](int t, u32x4_t (*kd)[CW], u32x4_t (*vd)[CW]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            // every lane loads (no branch: the compiler then counts the loads
            // in flight exactly and keeps the next tiles' loads outstanding
            // while this one is consumed); rows past the end read the last
            // valid row again, whose score is masked and whose P is 0
            const int slot = min(s0 + t * kTile + rg + RG * k, s1 - 1);
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                // read once per step: non-temporal loads stream past the caches
                kd[k][c] = __builtin_nontemporal_load((const u32x4_t*)(kg + (size_t)slot * RB + c * CPR * 16));
                vd[k][c] = __builtin_nontemporal_load((const u32x4_t*)(vg + (size_t)slot * RB + c * CPR * 16));
            }
        }
    };

    float m_h[G], l_h[G], acc[G][EPC * CW];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m_h[hh] = -INFINITY;
        l_h[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC * CW; ++e) acc[hh][e] = 0.f;
    }
    const float c = p.c;

    auto consume = [&](int t, const u32x4_t (*kd)[CW], const u32x4_t (*vd)[CW]) __attribute__((always_inline)) {
        // scores of this lane's RPT rows for every head (log2 domain)
        float sc[G][RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const bool valid = s0 + t * kTile + rg + RG * k < s1;
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float part = 0.f;
#pragma unroll
                for (int cw = 0; cw < CW; ++cw) {
                    if constexpr (BF) {
                        const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kd[k][cw]);
                        const bf16x8_t q8 = __builtin_bit_cast(bf16x8_t, qc[hh][cw]);
                        part = __builtin_amdgcn_fdot2_f32_bf16(pair<0>(k8), pair<0>(q8), part, false);
                        part = __builtin_amdgcn_fdot2_f32_bf16(pair<1>(k8), pair<1>(q8), part, false);
                        part = __builtin_amdgcn_fdot2_f32_bf16(pair<2>(k8), pair<2>(q8), part, false);
                        part = __builtin_amdgcn_fdot2_f32_bf16(pair<3>(k8), pair<3>(q8), part, false);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            part = fmaf(__uint_as_float(kd[k][cw][e]), __uint_as_float(qc[hh][cw][e]), part);
                    }
                }
                const float dot = row_sum<CPR>(part);
                sc[hh][k] = valid ? dot * c : -INFINITY;
            }
        }
        // online softmax per head for this row group; the reference max moves
        // only when it grows by more than 8 (log2 units), so most tiles skip
        // the rescale of acc (probabilities stay below 2^8)
        bool grow_any = false;
        float alpha[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float mx = sc[hh][0];
#pragma unroll
            for (int k = 1; k < RPT; ++k) mx = fmaxf(mx, sc[hh][k]);
            const float m_cand = fmaxf(m_h[hh], mx);
            const bool grow = m_cand > m_h[hh] + 8.f;
            alpha[hh] = grow ? __builtin_amdgcn_exp2f(m_h[hh] - m_cand) : 1.f;
            m_h[hh] = grow ? m_cand : m_h[hh];
            grow_any |= grow;
        }
        if (__builtin_amdgcn_ballot_w64(grow_any) != 0) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                l_h[hh] *= alpha[hh];
#pragma unroll
                for (int e = 0; e < EPC * CW; ++e) acc[hh][e] *= alpha[hh];
            }
        }
        if constexpr (BF) {
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int k = 0; k < RPT; k += 2) {
                // V values of rows k and k+1 interleaved per element
                uint32_t lo[CW][4], hi[CW][4];
#pragma unroll
                for (int cw = 0; cw < CW; ++cw)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[cw][e] = __builtin_amdgcn_perm(vd[k + 1][cw][e], vd[k][cw][e], 0x05040100u);
                        hi[cw][e] = __builtin_amdgcn_perm(vd[k + 1][cw][e], vd[k][cw][e], 0x07060302u);
                    }
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float mu = (m_h[hh] == -INFINITY) ? 0.f : m_h[hh];
                    const bf16x2_t pp = {(__bf16)__builtin_amdgcn_exp2f(sc[hh][k] - mu),
                                         (__bf16)__builtin_amdgcn_exp2f(sc[hh][k + 1] - mu)};
                    l_h[hh] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_h[hh], false);
#pragma unroll
                    for (int cw = 0; cw < CW; ++cw)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float& a0 = acc[hh][cw * EPC + 2 * e];
                            float& a1 = acc[hh][cw * EPC + 2 * e + 1];
                            a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo[cw][e]), pp, a0, false);
                            a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi[cw][e]), pp, a1, false);
                        }
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < RPT; ++k)
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float mu = (m_h[hh] == -INFINITY) ? 0.f : m_h[hh];
                    const float pr = __builtin_amdgcn_exp2f(sc[hh][k] - mu);
                    l_h[hh] += pr;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[hh][e] = fmaf(pr, __uint_as_float(vd[k][0][e]), acc[hh][e]);
                }
        }
    };

    // register ring: tiles t, t+1, ..., t+PD-1 are loaded before tile t is used
#pragma unroll
    for (int j = 0; j < PD; ++j) load(j, kr[j], vr[j]);
    // (no early exit inside a round: tiles past the end are all masked rows,
    // and a loop body without branches lets the compiler keep the loads of
    // the next tiles in flight across the round boundary)
    for (int t = 0; t < ntile; t += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            consume(t + j, kr[j], vr[j]);
            load(t + j + PD, kr[j], vr[j]);
        }
    }

    // ---- merge the row groups: per head M = max m, weights 2^(m - M)
    const int lane_in_row = dc;
    if (lane_in_row == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            sm_ml[rg][hh][0] = m_h[hh];
            sm_ml[rg][hh][1] = l_h[hh];
        }
    }
    __syncthreads();
    float wgt[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float M = -INFINITY;
#pragma unroll
        for (int r = 0; r < RG; ++r) M = fmaxf(M, sm_ml[r][hh][0]);
        wgt[hh] = (m_h[hh] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_h[hh] - M);
#pragma unroll
        for (int cw = 0; cw < CW; ++cw)
#pragma unroll
            for (int e = 0; e < EPC; ++e) sm_acc[rg][hh][(dc + cw * CPR) * EPC + e] = acc[hh][cw * EPC + e] * wgt[hh];
    }
    __syncthreads();
    if (p.nsplit == 1) {
        // the only split: normalise and write the output row directly
        for (int u = tid; u < G * D; u += kThreads) {
            const int hh = u / D, d = u % D;
            float M = -INFINITY;
            for (int r = 0; r < RG; ++r) M = fmaxf(M, sm_ml[r][hh][0]);
            float a = 0.f, L = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                a += sm_acc[r][hh][d];
                const float m = sm_ml[r][hh][0];
                if (m != -INFINITY) L += sm_ml[r][hh][1] * __builtin_amdgcn_exp2f(m - M);
            }
            elem_t* out = (elem_t*)p.out + er.row0 + (size_t)(h0 + hh) * er.head_stride + d;
            if constexpr (BF) {
                const __bf16 x = (__bf16)(a / L);
                *out = __builtin_bit_cast(uint16_t, x);
            } else {
                *out = a / L;
            }
        }
        return;
    }
    const size_t part = ((size_t)(blockIdx.z * p.Hq + h0) * p.nsplit + split);  // head hh adds hh * nsplit
    for (int u = tid; u < G * D; u += kThreads) {
        const int hh = u / D, d = u % D;
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) a += sm_acc[r][hh][d];
        p.ws_acc[(part + (size_t)hh * p.nsplit) * D + d] = a;
    }
    if (tid < G) {
        const int hh = tid;
        float M = -INFINITY;
        for (int r = 0; r < RG; ++r) M = fmaxf(M, sm_ml[r][hh][0]);
        float L = 0.f;
        for (int r = 0; r < RG; ++r) {
            const float m = sm_ml[r][hh][0];
            if (m != -INFINITY) L += sm_ml[r][hh][1] * __builtin_amdgcn_exp2f(m - M);
        }
        p.ws_ml[(part + (size_t)hh * p.nsplit) * 2 + 0] = M;
        p.ws_ml[(part + (size_t)hh * p.nsplit) * 2 + 1] = L;
    }
}

// Merge the splits of one (sequence, query head): weights 2^(m_s - M).
template <bool BF, int D, bool GR>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
    using elem_t = typename std::conditional<BF, uint16_t, float>::type;
    const int bh = blockIdx.x;
    const EntryRows er = entry_rows<GR, D>(p, bh / p.Hq);
    const int d = threadIdx.x;
    const int pb = er.pos;
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
        elem_t* out = (elem_t*)p.out + er.row0 + (size_t)(bh % p.Hq) * er.head_stride + d;
        if constexpr (BF) {
            const __bf16 x = (__bf16)r;
            *out = __builtin_bit_cast(uint16_t, x);
        } else {
            *out = r;
        }
    }
}

template <bool BF, int D, int G, bool GR>
hipError_t launch_gr(const DecodeParams& p, hipStream_t s) {
    hipLaunchKernelGGL((decode_split_kernel<BF, D, G, GR>), dim3(p.nsplit, p.Hkv, p.B), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<BF, D, GR>), dim3(p.B * p.Hq), dim3(128), 0, s, p);
    return hipGetLastError();
}

template <bool BF, int D, int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
    return p.gidx ? launch_gr<BF, D, G, true>(p, s) : launch_gr<BF, D, G, false>(p, s);
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

DecodeSplit decode_split_plan(int B, int Hkv, int W) {
    const long long pairs = (long long)B * Hkv;      // (sequence, KV head) pairs
    // one workgroup per CU: with fewer (sequence, KV head) pairs than CUs the
    // slots split until the pairs x splits workgroups fill them; more splits
    // (two or four workgroups per CU) measured slower on 4-32 sequences, the
    // extra partials and merge work outweighing the shorter streams
    const long long want = 256;
    const int tiles = (W + kTile - 1) / kTile;
    long long ns = pairs >= want ? 1 : (want + pairs - 1) / pairs;
    if (ns > tiles) ns = tiles;
    const int tiles_per_split = (int)((tiles + ns - 1) / ns);
    DecodeSplit sp;
    sp.split_len = tiles_per_split * kTile;
    sp.nsplit = (W + sp.split_len - 1) / sp.split_len;
    return sp;
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int W, int d) {
    const DecodeSplit sp = decode_split_plan(B, Hkv, W);
    if (sp.nsplit == 1) return 0;
    return (size_t)B * Hq * sp.nsplit * ((size_t)d + 2) * sizeof(float);
}

}  // namespace swa
