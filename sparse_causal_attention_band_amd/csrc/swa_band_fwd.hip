// Band-tiled causal sliding-window attention forward for CDNA4 (gfx950).
//
// What it computes: softmax(scale * Q K^T + M) V row by row, where row i may
// read key j iff j <= i and (i - j < W or (stride > 0 and j % stride == 0)).
// A third mode runs the same band over a chunk of new queries whose keys are
// the rolling-cache history followed by the chunk itself (chunked prefill).
// The band is the set N_W(i) of the page "SWA：滑动窗口注意力与跨层信息传递"
// (§3.1, window counting the current position), the strided keys are the
// "local + strided" mask of the page "注意力变体——滑动窗口、稀疏、差分"
// (构建它, 第 3 步).  The same pages note that the saving only exists if the
// out-of-window work is really skipped (SWA page §4.1; the attention-variants
// page, 稀疏 / 块注意力: never bring the zero entries on chip), so the kernel
// enumerates only key tiles that meet the band.
//
// Two kernels share the tile enumeration, layouts, masking and softmax: the
// 8-wave bf16 kernel at the end of this file (band, chunk and global-token
// modes with an even number of query heads per KV head, global lists of at
// most 64 positions, and one-pass differential attention) and the 4-wave
// kernel described here (fp32, the strided mode, longer global lists, one or
// an odd number of query heads per KV head, and K/V arrays of 2 GiB or more
// per head, which the 8-wave kernel's 32-bit byte offsets cannot address).
//
// Structure of the 4-wave kernel (one workgroup = 4 waves = 256 threads):
//  * A workgroup owns 4 blocks of 32 queries: HG query heads that share one
//    KV head times PB position blocks (HG * PB = 4).  Grouped heads therefore
//    read every K/V tile from LDS once per workgroup.  With the key split
//    (bf16 local + strided, odd head groups) it owns 2 blocks, and each
//    block's two waves take the two 32-key halves of every tile.
//  * Key tiles of 64 rows are visited from the diagonal tile down to the
//    lowest tile that meets the band; with stride > 0 a compact list of the
//    strided keys below the band follows (rows gathered at j = m * stride).
//    Each tile is copied HBM -> LDS directly (a 16-byte buffer load per
//    lane, coalesced), double-buffered, one barrier per tile.
//  * Per wave the score block is computed transposed, S^T = K Q^T, with the
//    32x32 matrix-core instruction (bf16: 32x32x16, fp32: 32x32x2).  In that
//    layout a lane owns one query and 32 of the tile's 64 keys; the other 32
//    sit in lane ^ 32, so the row max needs one cross-lane swap per tile and
//    the row sum none until the end.  K rows are fed in the order sigma()
//    below so the lane's probabilities are already the B operand of the
//    P*V product: O^T += V^T P^T, with V^T fragments read from LDS by the
//    gfx950 transpose read (bf16) or one dword per lane (fp32).
//  * Online softmax in the log2 domain; the mask is applied only on tiles
//    that are not entirely inside every row's band (edge tiles).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <float.h>
#include <atomic>
#include <type_traits>

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTileN = kKeysPerTile;  // 64 keys per tile
constexpr int kQw = kQueriesPerWave;  // 32 queries per wave

// Row of the 32-key block that lane x%32 feeds as the A operand of S^T = K Q^T.
// The 32x32 result row r of a lane in half g holds element i with
// r = 8*(i/4) + 4*g + i%4; swapping bits 2 and 3 makes the key behind element
// i equal to 16*(i/8) + 8*g + i%8, i.e. 8 consecutive keys per half and per
// 16-key chunk -- exactly the k-slots the P*V instruction expects.
__device__ __forceinline__ int sigma(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Global work id -> logical id so that consecutive logical ids (consecutive
// query tiles of one head) land on the same XCD: the dispatcher hands work
// group x to XCD x % 8, and each XCD has its own L2.
__device__ __forceinline__ int xcd_remap(int x, int total) {
    const int per = total >> 3, rem = total & 7;
    const int xcd = x & 7, idx = x >> 3;
    return xcd * per + min(xcd, rem) + idx;
}

// LDS tile layouts.  gfx950's LDS serves 256 bytes (64 banks) per cycle:
// 16 lanes of a 16-byte read, 32 lanes of an 8-byte read.
//  * K: rows in groups of 16, 16-byte chunks column-major inside a group:
//    position p, chunk c at ((p >> 4) * CPR + c) * 256 + (p & 15) * 16.
//    The 16 lanes served together read 16 consecutive positions of one chunk
//    column, 256 contiguous bytes.  Rows are stored in sigma order (position
//    p holds key row sigma(p)), so the lanes needing rows sigma(0..15) read
//    positions 0..15.  One 1 KiB copy block is 16 rows x 64 bytes of HBM.
//  * V: row-major with a 64-byte pad after each row (stride RB + 64).  An
//    8-byte transpose read by 32 lanes touches 4 consecutive rows x 64 bytes,
//    which the pad spreads over the 4 quarters of the banks.  Copy lanes that
//    fall on the pad are switched off.
// Every fragment address is then (per-lane base) + (compile-time offset).

__device__ __forceinline__ float partner_max(float x) {
    // permlane32_swap(x, x): lanes 0..31 receive (x[l], x[l+32]),
    // lanes 32..63 receive (x[l-32], x[l]); either way both copies.
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(p));
}

// Buffer resource over `rows` rows of `row_bytes` bytes (structured: a load
// names a row and a byte inside it; rows >= `rows` read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int row_bytes, int rows) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)row_bytes, rows, 0x00020000);
}

// MODE: kBand (window only), kStrided (window + multiples of the stride),
// kChunk (a chunk of new queries over the ring history plus the chunk).
// KS (key split): the workgroup holds two 32-query blocks, each served by a
// pair of waves that take the two 32-key halves of every tile with separate
// online softmaxes, merged by their log-sum-exp at the end.  A workgroup then
// spans 64 positions instead of 128, so with a short window each row walks
// fewer key tiles, and each wave holds one score block instead of two.
// With the split, d = 64 fits four workgroups per CU (120 registers); every
// other instantiation runs two (a cap of three spilled in the strided and
// global modes).
template <bool BF, int D, int MODE, bool KS = false>
__global__ __launch_bounds__(kThreads, KS && D == 64 ? 4 : 2) void
band_fwd_kernel(PrefillParams p) {
    constexpr bool STRIDED = MODE == kStrided;
    constexpr bool CHUNK = MODE == kChunk;
    constexpr bool GLOBAL = MODE == kGlobal;
    constexpr bool KEYLIST = STRIDED || GLOBAL;  // extra keys outside the window
    using elem_t = typename std::conditional<BF, uint16_t, float>::type;
    using frag_t = typename std::conditional<BF, bf16x8_t, float>::type;
    constexpr int RB = D * (int)sizeof(elem_t);      // bytes per K/V row
    constexpr int CPR = RB / 16;                     // 16-byte chunks per row
    constexpr int TILE_BYTES = kTileN * RB;          // K tile
    constexpr int RBV = RB + 64;                     // padded V row
    constexpr int VTILE_BYTES = kTileN * RBV;        // V tile
    constexpr int NCHV = VTILE_BYTES / (kThreads * 16);  // V copy blocks per wave
    constexpr int NCH = kTileN * CPR / kThreads;     // chunks per thread per tile
    constexpr int NDB = D / 32;                      // 32-row blocks of O^T
    constexpr int KSTEP = BF ? 16 : 2;               // contraction depth per instruction
    constexpr int NQF = D / KSTEP;
    constexpr int NKB = KS ? 1 : 2;                  // 32-key blocks of a tile per wave
    static_assert(NCH >= 1 && (kTileN * CPR) % kThreads == 0, "tile copy split");
    static_assert(VTILE_BYTES % (kThreads * 16) == 0, "V tile copy split");

    // Two K/V buffers as four distinct LDS objects: every access below names
    // its buffer statically (the tile loop is unrolled by two), so the
    // compiler can tell the in-flight copy of tile t+1 from the reads of tile
    // t and does not drain the copy before reading.
    __shared__ __attribute__((aligned(16))) char kb0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char vb0[VTILE_BYTES];
    __shared__ __attribute__((aligned(16))) char kb1[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char vb1[VTILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS copy targets stay scalar
    const int g = lane >> 5, l32 = lane & 31;
    const int half = KS ? (wave & 1) : 0;     // key half of every tile this wave takes
    const int blk = KS ? (wave >> 1) : wave;  // 32-query block of this wave

    // ---- which workgroup tile is this
    const int L = xcd_remap(blockIdx.x, p.total);
    const int qb = L % p.nqb;
    int rest = L / p.nqb;
    const int hg = rest % p.ngroups;
    rest /= p.ngroups;
    // sequences inner, KV heads outer: a contiguous range of logical blocks
    // (one XCD's) holds every sequence in equal parts, which balances the
    // XCDs when the sequences' lengths differ (chunked prefill)
    const int b = rest % p.B;
    const int kvh = rest / p.B;
    const int N = p.N;
    // Chunk mode (SWA page §4.3): the N queries are chunk rows that follow
    // `start` cached positions.  They are placed at the end of a virtual
    // sequence of NK = qoff + N keys whose first qoff = min(start, W-1) keys
    // are the history read from the ring (older positions are outside every
    // row's window) and whose last N keys are the chunk's own rows.  In the
    // other modes qoff = 0 and the virtual sequence is the input.
    int qoff = 0, hslot0 = 0;
    if constexpr (CHUNK) {
        // uniform per workgroup: scalar registers, so the copy offsets stay scalar
        const int start = __builtin_amdgcn_readfirstlane(max(p.p0[b], 0));
        qoff = min(start, p.W - 1);
        hslot0 = (start - qoff) % p.W;  // ring slot of the oldest history position used
    }
    const int NK = qoff + N;
    const int W = min(p.W, NK);  // a wider window reads the same keys
    const int BM = kQw * p.PB;
    const int q0 = qb * BM;
    const int h = kvh * p.G + hg * p.HG + (blk % p.HG);
    const int qw0 = q0 + kQw * (blk / p.HG);
    const int qi = qw0 + l32;        // query row in q / out
    const int qv = qoff + qi;        // its position in the virtual sequence
    const int qvw0 = qoff + qw0;

    const size_t kv_head = (size_t)(b * p.Hkv + kvh) * (size_t)N * D;
    const size_t q_head = (size_t)(b * p.Hq + h) * (size_t)N * D;
    const elem_t* kg = (const elem_t*)p.k + kv_head;
    const elem_t* vg = (const elem_t*)p.v + kv_head;
    const elem_t* qg = (const elem_t*)p.q + q_head;
    elem_t* og = (elem_t*)p.out + q_head;
    const size_t ring_head = (size_t)(b * p.Hkv + kvh) * (size_t)p.W * D;
    const elem_t* krg = CHUNK ? (const elem_t*)p.kring + ring_head : nullptr;
    const elem_t* vrg = CHUNK ? (const elem_t*)p.vring + ring_head : nullptr;

    // ---- key tiles of this workgroup: band tiles kt_hi .. kt_lo, then the
    // compact strided tiles (keys m*stride < kt_lo*64, read by every row).
    const int wr = p.wr;  // right radius of a two-sided band (0: causal)
    const int kt_hi = min(NK - 1, qoff + q0 + BM - 1 + wr) / kTileN;
    const int kt_lo = max(0, qoff + q0 - W + 1) / kTileN;
    const int nband = kt_hi - kt_lo + 1;
    // first entry of the sorted global list that is >= x (wave-uniform)
    auto global_lb = [&](int x) __attribute__((always_inline)) {
        int lo = 0, hi = p.ng;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (p.gidx[mid] < x)
                lo = mid + 1;
            else
                hi = mid;
        }
        return lo;
    };
    // extra keys below the lowest band tile, read by every row: multiples of
    // the stride, or the global positions there (a prefix of the sorted list)
    int M = 0, ncomp = 0;
    if (STRIDED) M = (kt_lo * kTileN + p.stride - 1) / p.stride;
    if (GLOBAL) M = global_lb(kt_lo * kTileN);
    if (KEYLIST) ncomp = (M + kTileN - 1) / kTileN;
    const int ntiles = nband + ncomp;

    const bool wave_live = qw0 < N;  // some row of this wave is a real query

    // ---- Q fragments (B operand of S^T = K Q^T), sign folded in
    frag_t qf[NQF];
    if constexpr (BF) {
        const uint32_t flip = p.neg ? 0x80008000u : 0u;
        // rows past N read row N-1 and are zeroed (never stored)
        const uint32_t keep = qi < N ? 0xffffffffu : 0u;
        const size_t qrow = (size_t)min(qi, N - 1) * D;
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
            u32x4_t w = *(const u32x4_t*)(qg + qrow + 16 * c + 8 * g);
            w = (w & keep) ^ flip;
            qf[c] = __builtin_bit_cast(bf16x8_t, w);
        }
    } else {
        const size_t qrow = (size_t)min(qi, N - 1) * D;
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
            const float x = qg[qrow + 2 * c + g];
            qf[c] = qi < N ? (p.neg ? -x : x) : 0.f;
        }
    }

    // ---- per-lane LDS bases of the fragment reads
    // K: position l32 (+32 per key half), chunk 2*cc + g (bf16) or cc/2 (fp32)
    // (key split: the wave's 32-key block is the tile's block `half`)
    const int k_lane = (BF ? ((((l32 >> 4) * CPR + g) << 8) + ((l32 & 15) << 4))
                           : ((((l32 >> 4) * CPR) << 8) + ((l32 & 15) << 4) + (g << 2))) +
                       ((half * 2 * CPR) << 8);
    // V (bf16 transpose read): row 8*g + (lane&15)/4 (+16*c2 + 4*rd),
    // element 16*((lane>>4)&1) + 4*(lane&3) (+32*db).  fp32: row 8*g, element l32.
    const int v_lane = (BF ? ((8 * g + ((lane & 15) >> 2)) * RBV + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2)
                           : (8 * g * RBV + l32 * 4)) +
                       32 * half * RBV;

    // ---- tile copy HBM -> LDS without registers: each wave's 16-byte
    // buffer load with the "lds" flag fills one contiguous 1 KiB block of LDS
    // (lane i writes bytes 16i..16i+15 of it), so the layout is applied by
    // choosing which 16-byte chunk of which row each lane fetches.  Rows past
    // the end are clamped to a valid row: those keys are always masked, and
    // the copy never leaves non-finite bits in LDS.  The resources address
    // (row, byte in row) of one (sequence, KV head) array; buffer loads,
    // unlike the global-segment form of the copy, are not FLAT instructions,
    // so the compiler can still wait for single LDS reads while copies fly.
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kg, RB, N);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vg, RB, N);
    const __amdgpu_buffer_rsrc_t rkr = CHUNK ? rows_rsrc(krg, RB, p.W) : rk;
    const __amdgpu_buffer_rsrc_t rvr = CHUNK ? rows_rsrc(vrg, RB, p.W) : rv;
    auto issue_tile = [&](int t, char* kl, char* vl, bool do_k, bool do_v) __attribute__((always_inline)) {
        // key row behind tile row r (virtual index in chunk mode)
        auto key_of = [&](int r) __attribute__((always_inline)) {
            if (!KEYLIST || t < nband) return min((kt_hi - t) * kTileN + r, NK - 1);
            const int m = min((t - nband) * kTileN + r, M - 1);
            if constexpr (GLOBAL) return min(max(p.gidx[m], 0), NK - 1);
            return m * p.stride;
        };
        // copy 16 bytes of key row j into LDS: from the input, or in chunk
        // mode from the ring for history keys (the two empty asm statements
        // differ, so the compiler cannot merge the two loads into one with a
        // per-lane resource)
        auto copy16 = [&](__amdgpu_buffer_rsrc_t in, __amdgpu_buffer_rsrc_t ring, int j, int byte, char* dst)
            __attribute__((always_inline)) {
            auto* l = (__attribute__((address_space(3))) void*)dst;
            if constexpr (CHUNK) {
                if (j < qoff) {
                    int slot = hslot0 + j;
                    slot -= slot >= p.W ? p.W : 0;
                    __builtin_amdgcn_struct_ptr_buffer_load_lds(ring, l, 16, slot, byte, 0, 0, 0);
                    asm volatile("; ring rows" ::: "memory");
                } else {
                    __builtin_amdgcn_struct_ptr_buffer_load_lds(in, l, 16, j - qoff, byte, 0, 0, 0);
                    asm volatile("; chunk rows" ::: "memory");
                }
            } else {
                __builtin_amdgcn_struct_ptr_buffer_load_lds(in, l, 16, j, byte, 0, 0, 0);
            }
        };
#pragma unroll
        for (int it = 0; it < NCH; ++it) {
            if (!do_k) break;
            const int blk = (wave * NCH + it) * 1024;  // wave-uniform LDS block
            const int P = blk + lane * 16;
            const int within = P % (CPR * 256);
            const int pos = (P / (CPR * 256)) * 16 + ((within >> 4) & 15);
            const int ch = within >> 8;
            copy16(rk, rkr, key_of(sigma(pos)), ch << 4, kl + blk);
        }
#pragma unroll
        for (int it = 0; it < NCHV; ++it) {
            if (!do_v) break;
            const int blk = (wave * NCHV + it) * 1024;
            const int P = blk + lane * 16;
            const int row = P / RBV, inrow = P % RBV;
            if (inrow < RB) copy16(rv, rvr, key_of(row), inrow, vl + blk);
        }
    };

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.c;

    // S^T of tile t from the K buffer kl (the lane feeds key row
    // kb*32 + sigma(l32), stored at position kb*32 + l32)
    auto scores = [&](const char* kl, f32x16_t* sc) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
#pragma unroll
            for (int cc = 0; cc < NQF; ++cc) {
                if constexpr (BF) {
                    const bf16x8_t a = *(const bf16x8_t*)(kl + k_lane + ((kb * 2 * CPR + 2 * cc) << 8));
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], sc[kb], 0, 0, 0);
                } else {
                    const float a =
                        *(const float*)(kl + k_lane + ((kb * 2 * CPR + (cc >> 1)) << 8) + ((cc & 1) << 3));
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[cc], sc[kb], 0, 0, 0);
                }
            }
        }
    };

    // mask tile t: only tiles not entirely inside every row of this wave's band
    auto mask_tile = [&](int t, f32x16_t* sc) __attribute__((always_inline)) {
        const bool band = !KEYLIST || t < nband;  // (band and chunk modes have no compact tiles)
        const int j0 = (kt_hi - t) * kTileN;
        const bool edge = band ? !(j0 + kTileN - 1 <= qvw0 + wr && j0 >= qvw0 + kQw - W && j0 + kTileN <= NK)
                               : ((t - nband + 1) * kTileN > M);
        if (edge) {
            // bit o of smask: key j0 + o is a multiple of the stride (or a
            // global position).  Strided tiles: o_first is the offset of the
            // first multiple at or after j0 (kTileN or more: none in the tile).
            uint64_t smask = 0;
            int o_first = kTileN;
            if (STRIDED && band) {
                const int r0 = j0 % p.stride;
                o_first = r0 == 0 ? 0 : p.stride - r0;
                for (int o = o_first; o < kTileN; o += p.stride) smask |= 1ull << o;
            }
            if (GLOBAL && band) {
                for (int e = global_lb(j0); e < p.ng && p.gidx[e] < j0 + kTileN; ++e) smask |= 1ull << (p.gidx[e] - j0);
            }
            // Element i of block kb holds key j0 + 8g + C with the constant
            // C = kb*32 + 16*(i/8) + i%8; with x = qv - j0 - 8g its distance is
            // x - C, so each test compares one per-tile bound with a constant
            // (the empty asm keeps the compiler from hoisting 32 per-lane key
            // offsets out of the tile loop instead).
            int lo, hi, nk;
            // (key split: the wave's keys start 32 * half into the tile)
            const int kofs = 8 * g + 32 * half;
            if (band) {
                const int x = qv - j0 - kofs;
                lo = x + wr;           // dist >= -wr  <=>  C <= lo
                hi = x - W;            // dist < W     <=>  C > hi
                nk = NK - j0 - kofs;   // key < NK     <=>  C < nk
            } else {
                lo = kTileN;
                hi = kTileN;
                nk = M - (t - nband) * kTileN - kofs;  // compact entry < M
            }
            asm volatile("" : "+v"(lo), "+v"(hi), "+v"(nk));
            const uint64_t sm = smask >> kofs;
            // which bounds this tile can violate (wave-uniform): most edge
            // tiles need one compare per element, not three
            const bool need_lo = j0 + kTileN - 1 > qvw0 + wr, need_nk = j0 + kTileN > NK;
            const bool need_hi = j0 < qvw0 + kQw - W;
            auto apply = [&](auto keep_of) __attribute__((always_inline)) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int C = kb * 32 + 16 * (i >> 3) + (i & 7);
                        sc[kb][i] = keep_of(C) ? sc[kb][i] : -INFINITY;
                    }
            };
            if (!band) {
                // compact tile: entries past the list end are clamped copies
                apply([&](int C) { return C < nk; });
            } else if (!need_hi && !need_nk) {
                // every key of the tile lies inside every row's window, so an
                // extra (strided or global) key changes nothing: causal bound only
                apply([&](int C) { return C <= lo; });
            } else if (!need_lo && !need_nk) {
                // every key is causal for every row: the window's lower
                // bound, or an extra key below it.  A stride of a tile or
                // more puts at most one multiple in the tile (at o_first), so
                // strided tiles compare with that one key, not a bit mask.
                if (STRIDED && p.stride >= kTileN) {
                    if (o_first >= kTileN) {
                        apply([&](int C) { return C > hi; });
                    } else {
                        int e = o_first - kofs;  // the multiple, as this lane's C
                        asm volatile("" : "+v"(e));
                        apply([&](int C) { return (C > hi) | (C == e); });
                    }
                } else if constexpr (KEYLIST) {
                    apply([&](int C) { return (C > hi) | (((sm >> C) & 1ull) != 0); });
                } else {
                    apply([&](int C) { return C > hi; });
                }
            } else {
                // non-short-circuit operators: a straight-line select, no
                // per-element divergent branches.  (Keys past the end exist
                // only as clamped copies of the last row; causal rows never
                // reach them.)
                apply([&](int C) {
                    return (C <= lo) & (C < nk) & ((C > hi) | (KEYLIST & (((sm >> C) & 1ull) != 0)));
                });
            }
        }
    };

    // online softmax of a masked score tile: first the row max and the
    // (rare) rescale of O, which ends in a branch; the exponentials follow in
    // softmax_pv, in the same basic block as the next tile's score MFMAs.
    float alpha = 1.f;
    auto softmax_head = [&](f32x16_t* sc) __attribute__((always_inline)) {
        // log2 domain; the lane pair (l, l^32) shares a query
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
        mx = partner_max(mx);
        // The reference max moves only when the tile max exceeds it by more
        // than 8 (log2 units): probabilities then stay below 2^8, which the
        // fp32 sums and the bf16 P operand carry without loss, and most tiles
        // skip the O / l rescale.  Lanes l and l^32 see the same max, so they
        // always take the same decision.
        const float m_cand = fmaxf(m_run, mx * c);
        const bool grow = m_cand > m_run + 8.f;  // false while both are -inf
        alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_cand) : 1.f;  // 0 on the first finite max
        m_run = grow ? m_cand : m_run;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
    };
    // exponentials, row sum, then O^T += V^T P^T from vl
    auto softmax_pv = [&](f32x16_t* sc, const char* vl) __attribute__((always_inline)) {
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;  // row with no allowed key yet
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], c, -m_use));

        // The row sum adds the same probabilities the product uses:
        // bf16-rounded ones (packed dot with (1, 1)), so the output is an
        // exact convex combination of V rows.
        float rs = 0.f;
        if constexpr (BF) {
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
            bf16x8_t pb[2 * NKB];
#pragma unroll
            for (int c2 = 0; c2 < 2 * NKB; ++c2) {
                // pairs are built as bf16x2 values and only whole vectors are
                // bit-cast: extracting a dword of a bf16x8 and bit-casting it
                // to bf16x2 mis-compiles (every pair reads element 0).
                u32x4_t pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16x2_t pr = {(__bf16)sc[c2 >> 1][8 * (c2 & 1) + 2 * e],
                                         (__bf16)sc[c2 >> 1][8 * (c2 & 1) + 2 * e + 1]};
                    rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
                    pw[e] = __builtin_bit_cast(uint32_t, pr);
                }
                pb[c2] = __builtin_bit_cast(bf16x8_t, pw);
            }
#pragma unroll
            for (int c2 = 0; c2 < 2 * NKB; ++c2)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    // rows 16*c2 + 8*g + 4*rd + (lane&15)/4 (+32*half), 4 elements at
                    // d = 32*db + 16*((lane>>4)&1) + 4*(lane&3)
                    const char* vp = vl + v_lane + 16 * c2 * RBV + 64 * db;
                    const i16x4_t lo = lds_read_tr16(vp);
                    const i16x4_t hi = lds_read_tr16(vp + 4 * RBV);
                    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
                    const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
                    const u32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a4), pb[c2],
                                                                      oacc[db], 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    rs += sc[kb][i];
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        // row kb*32 + 16*(i>>3) + 8*g + (i&7), d = 32*db + l32
                        const float a =
                            *(const float*)(vl + v_lane + (kb * 32 + 16 * (i >> 3) + (i & 7)) * RBV + 128 * db);
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sc[kb][i], oacc[db], 0, 0, 0);
                    }
                }
        }
        l_run = l_run * alpha + rs;
    };

    // Two-stage pipeline over the tile list: K runs one tile ahead of V.
    // Iteration t reads K(t+1) (scores of the next tile, whose matrix work
    // overlaps this tile's softmax) and V(t), while the copies of K(t+2) and
    // V(t+1) land in the buffers freed by iteration t-1.  Every wave walks the
    // whole tile list of its workgroup; tiles outside its own rows' band come
    // out fully masked.  A buffer is refilled only after the barrier that
    // closes the iteration which last read it.
    issue_tile(0, kb0, vb0, true, true);
    if (ntiles > 1) issue_tile(1, kb1, vb1, true, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16_t scur[NKB];
    scores(kb0, scur);
    mask_tile(0, scur);
    __syncthreads();

    auto step = [&](int t, const char* kn, const char* vc, char* ki, char* vi) __attribute__((always_inline)) {
        if (t + 2 < ntiles) issue_tile(t + 2, ki, vi, true, false);
        if (t + 1 < ntiles) issue_tile(t + 1, ki, vi, false, true);
        softmax_head(scur);
        f32x16_t snext[NKB];
        scores(kn, snext);  // past the last tile this reads stale data and is discarded
        softmax_pv(scur, vc);
        if (t + 1 < ntiles) mask_tile(t + 1, snext);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) scur[kb] = snext[kb];
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, kb1, vb0, kb0, vb1);
        if (t + 1 < ntiles) step(t + 1, kb0, vb1, kb1, vb0);
    }

    // ---- epilogue: O / l, lane holds d = 32*db + 8*quad + 4*g + 0..3
    // The exponentials were taken relative to m_fin (log2 units of scale*q.k).
    float lt = partner_sum(l_run);
    float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
    if constexpr (KS) {
        // The two waves of a block saw disjoint key halves: the second hands
        // its reference max, row sum and O to the first through LDS (the
        // loop's last barrier has freed the tile buffers), which rescales
        // both to the larger reference and adds them.
        float* xf = (float*)(blk == 0 ? vb0 : vb1);
        constexpr int NO = 16 * NDB;
        static_assert((NO + 2) * 64 * 4 <= VTILE_BYTES, "exchange fits a V buffer");
        // A half that met no allowed key has m_run = -inf and O = l = 0: it
        // takes weight 0 (not exp2 of its placeholder reference 0 minus the
        // other's max, which overflows when that max is very negative).
        if (half == 1) {
#pragma unroll
            for (int j = 0; j < NO; ++j) xf[j * 64 + lane] = oacc[j >> 4][j & 15];
            xf[NO * 64 + lane] = m_run;
            xf[(NO + 1) * 64 + lane] = lt;
        }
        __syncthreads();
        if (half == 1) return;
        const float m1 = xf[NO * 64 + lane], l1 = xf[(NO + 1) * 64 + lane];
        const float mx = fmaxf(m_run, m1);
        const float mm = mx == -INFINITY ? 0.f : mx;  // -inf: no allowed key in either half
        const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        lt = lt * a0 + l1 * a1;
#pragma unroll
        for (int j = 0; j < NO; ++j) oacc[j >> 4][j & 15] = oacc[j >> 4][j & 15] * a0 + xf[j * 64 + lane] * a1;
        m_fin = mm;
    }
    if (!wave_live || qi >= N) return;
    if (p.lse != nullptr && g == 0) {
        // ln of the row's softmax denominator
        p.lse[(size_t)(b * p.Hq + h) * N + qi] = (m_fin + __log2f(lt)) * 0.69314718055994531f;
    }
    if constexpr (BF) {
        if (p.lam == nullptr) {
            // plain bf16 output, 16 bytes per store: one swap between the two
            // lanes of a query (both active or both not) per pair of words
            // regroups quads 2qp and 2qp + 1 so that lane g holds
            // d = 32 db + 16 qp + 8 g + 0..7 (as in the 8-wave kernel)
            const float inv = 1.f / lt;
            auto pk = [&](int db, int quad, int k) __attribute__((always_inline)) {
                const bf16x2_t pr = {(__bf16)(oacc[db][4 * quad + 2 * k] * inv), (__bf16)(oacc[db][4 * quad + 2 * k + 1] * inv)};
                return __builtin_bit_cast(uint32_t, pr);
            };
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qp = 0; qp < 2; ++qp) {
                    u32x4_t w;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const auto r = __builtin_amdgcn_permlane32_swap(pk(db, 2 * qp, k), pk(db, 2 * qp + 1, k), false, false);
                        w[k] = r[0];
                        w[2 + k] = r[1];
                    }
                    *(u32x4_t*)(og + (size_t)qi * D + 32 * db + 16 * qp + 8 * g) = w;
                }
            return;
        }
    }
    // plain store (fp32), or (second map of differential attention) out -= lam * O/l
    const bool sub = p.lam != nullptr;
    const float inv = (sub ? -p.lam[h] : 1.f) / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int quad = 0; quad < 4; ++quad) {
            const int d0 = db * 32 + 8 * quad + 4 * g;
            float o0 = oacc[db][4 * quad + 0] * inv, o1 = oacc[db][4 * quad + 1] * inv;
            float o2 = oacc[db][4 * quad + 2] * inv, o3 = oacc[db][4 * quad + 3] * inv;
            if constexpr (BF) {
                typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                bf16x4_t* dst = (bf16x4_t*)(og + (size_t)qi * D + d0);
                if (sub) {
                    const bf16x4_t prev = *dst;
                    o0 += (float)prev[0];
                    o1 += (float)prev[1];
                    o2 += (float)prev[2];
                    o3 += (float)prev[3];
                }
                const bf16x4_t o = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
                *dst = o;
            } else {
                typedef float f32x4_t __attribute__((ext_vector_type(4)));
                f32x4_t* dst = (f32x4_t*)(og + (size_t)qi * D + d0);
                if (sub) {
                    const f32x4_t prev = *dst;
                    o0 += prev[0];
                    o1 += prev[1];
                    o2 += prev[2];
                    o3 += prev[3];
                }
                const f32x4_t o = {o0, o1, o2, o3};
                *dst = o;
            }
        }
}

// ---------------------------------------------------------------------------
// bf16 kernel: 8 waves per workgroup sharing one K/V tile stream, with three
// K and three V buffers so that every copy is issued two tiles before it is
// read.  The tile list, the K layout, masking and the online softmax are
// those of the 4-wave kernel above; the differences are:
//  * V is stored unpadded with its 64-byte quarters XOR-swizzled by row, so
//    that the four rows an 8-byte transpose read touches in one cycle fall
//    on four different bank quarters; a tile is then 8 KiB-aligned and every
//    wave copies the same number of 1 KiB blocks;
//  * step t reads K(t+1) (next scores) and V(t) (this tile's P*V), issues
//    K(t+3) and V(t+2), and waits only for the copies issued one step earlier;
//  * this tile's probabilities, its P*V product and the next tile's scores
//    form one straight-line block, 16 keys at a time, so that every matrix
//    instruction has vector work of the same wave beside it.  The scores run
//    one 16-key region ahead of P*V: the first region's score instructions
//    are issued beside the short softmax head, and the last region masks the
//    next score block and takes its row maximum beside this tile's last P*V
//    instructions, so no stretch of the step is vector work alone.  The K
//    fragments of a region are read from LDS two regions ahead, its V
//    fragments just before its instructions;
//  * the copies are buffer loads into LDS rather than global-segment loads:
//    the latter are FLAT instructions that may also address LDS, and with
//    one in flight the compiler's wait counting can no longer wait for a
//    single LDS read (every wait in the loop became a full drain);
//  * a block's steps run in three segments, masked, mask-free and masked,
//    so that the tiles inside every row's band go through a loop with no
//    mask code and no branch;
//  * the grid is persistent, one workgroup per CU running its blocks in
//    turn, and in band mode a block's last steps already copy the next
//    block's first tiles and stage its queries in LDS, and its last step
//    computes the next block's first score block;
//  * the output of each query is regrouped between its two lanes so that a
//    lane stores 16 consecutive bytes at a time.
constexpr int kThreads8 = 512;

// Raw buffer resource over [base, base + bytes): stride 0, bounds checked
// per access (out of range reads return zero).  bytes < 2^31 (checked on
// the host).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Logical block of workgroup w in its iteration `it` (-1: none left).  The
// blocks are split into 8 contiguous ranges, one per XCD (the dispatcher
// places workgroup w on XCD w % 8), as xcd_remap does for one block per
// workgroup; the nwg / 8 workgroups of an XCD take its blocks in rounds of
// nwg / 8 consecutive blocks, so the CUs of one XCD work on neighbouring
// query blocks (shared K/V tiles in its L2), and alternate direction between
// rounds (a snake), so the light blocks at the head of each sequence -- whose
// bands are cut short by position 0 -- spread evenly over the workgroups.
// nwg == total: one block per workgroup.  nwg < total: nwg is a multiple of 8.
__device__ __forceinline__ int persistent_block(int w, int it, int nwg, int total) {
    if (nwg >= total) return it == 0 ? xcd_remap(w, total) : -1;
    const int xcd = w & 7, slot = w >> 3, nslot = nwg >> 3;
    const int per = total >> 3, rem = total & 7;
    const int base = xcd * per + min(xcd, rem), cnt = per + (xcd < rem ? 1 : 0);
    const int idx = it * nslot + ((it & 1) ? nslot - 1 - slot : slot);
    return idx < cnt ? base + idx : -1;
}

// First entry of the sorted global-position list that is >= x (uniform
// arguments: scalar loads).
__device__ __forceinline__ int global_lower_bound(const int32_t* gidx, int ng, int x) {
    int lo = 0, hi = ng;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (gidx[mid] < x)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

__device__ __forceinline__ void lds_barrier() {
    // this wave's LDS reads done, then the workgroup barrier: no fence, so
    // the copies in flight are not drained
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads8, D == 64 ? 2 : 1) void band8_kernel(PrefillParams p) {
    constexpr bool CHUNK = MODE == kChunk;
    // Differential attention (A1 - lam A2) V in one pass: waves 0..3 run the
    // first map (q, k) and waves 4..7 the second (q2, k2) for the same four
    // 32-query blocks, over one tile stream that stages K1, K2 and the
    // shared V once per step; the epilogue combines the two normalised
    // results through LDS and rounds once.
    constexpr bool DIFF = MODE == kDiff;
    using elem_t = uint16_t;
    constexpr int RB = D * 2;                    // bytes per K/V row
    constexpr int CPR = RB / 16;                 // 16-byte chunks per row
    constexpr int TILE_BYTES = kTileN * RB;      // K or V tile
    constexpr int NBLK = TILE_BYTES / 8192;      // 1 KiB copy blocks per wave per tile
    constexpr int NDB = D / 32;                  // 32-row blocks of O^T
    constexpr int NQF = D / 16;                  // Q fragments
    static_assert(TILE_BYTES % 8192 == 0, "copy split");
    static_assert(NDB == NQF / 2, "one P*V instruction per score instruction");
    // Global tokens: the global positions below a block's band follow its band
    // tiles as one compact tile (the host routes lists of at most 64 positions
    // here), and inside the band they are extra keys of the edge tiles' masks.
    constexpr bool GLOBAL = MODE == kGlobal;
    static_assert(MODE == kBand || MODE == kChunk || MODE == kDiff || MODE == kGlobal,
                  "no strided keys: those take the 4-wave kernel");

    __shared__ __attribute__((aligned(16))) char kb0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char kb1[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char kb2[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char vb0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char vb1[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char vb2[TILE_BYTES];
    // the second map's K buffers (differential attention only)
    __shared__ __attribute__((aligned(16))) char kc0[DIFF ? TILE_BYTES : 16];
    __shared__ __attribute__((aligned(16))) char kc1[DIFF ? TILE_BYTES : 16];
    __shared__ __attribute__((aligned(16))) char kc2[DIFF ? TILE_BYTES : 16];
    // Band mode streams from one block into the next (see `pre` below): each
    // wave stages its 32 query rows of the next block in its region of these
    // (two waves per array), 16-byte chunk k of row r at (k * 32 + r) * 16.
    // Four arrays the size of a tile buffer, declared last, are placed after
    // the tile buffers, whose LDS reads then keep small address offsets.
    constexpr bool STREAM = MODE == kBand;
    constexpr int QST = STREAM ? 2 * kQw * RB : 16;
    __shared__ __attribute__((aligned(16))) char qs0[QST];
    __shared__ __attribute__((aligned(16))) char qs1[QST];
    __shared__ __attribute__((aligned(16))) char qs2[QST];
    __shared__ __attribute__((aligned(16))) char qs3[QST];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS copy targets stay scalar
    const int g = lane >> 5, l32 = lane & 31;
    const int map = DIFF ? (wave >> 2) : 0;   // which attention map this wave computes
    const int wv = DIFF ? (wave & 3) : wave;  // the wave's query block within its map

    // Persistent workgroups: the grid has p.nwg <= p.total workgroups and
    // each runs its logical blocks one after another (see persistent_block),
    // so a CU does not wait for a new workgroup to be dispatched between
    // blocks, and the code of the block loop stays in the instruction cache.
    // (the one-pass differential mode keeps one block per workgroup: the
    // block loop would push its registers past the budget)
    // A block's queries and its first tile's scores.  In band mode, blocks
    // after a workgroup's first get both from the previous block's last step
    // (the one whose score block would otherwise be discarded), so their
    // prologue only masks and takes the row maximum.
    bf16x8_t qf[NQF];
    f32x16_t scur[2];
    for (int iter = 0;; ++iter) {
        if (DIFF && iter > 0) break;
        const int L = DIFF ? xcd_remap(blockIdx.x, p.total) : persistent_block(blockIdx.x, iter, p.nwg, p.total);
        if (L < 0) break;
        // Band mode: the previous block's last steps already copied this
        // block's first K and V tiles into the buffers its prologue would fill
        // and staged its queries (its tile list is padded to a multiple of
        // three steps, so the buffer rotation continues unchanged), and its
        // last step loaded them and computed the first tile's scores, so the
        // prologue only masks that tile and has no barrier.  Other modes: the
        // previous block's waves are done with every LDS buffer (and every
        // copy has landed) before this block's prologue writes them.
        const bool pre = STREAM && iter > 0;
        if (iter > 0 && !pre) lds_barrier();
        const int qb = L % p.nqb;
        int rest = L / p.nqb;
        const int hg = rest % p.ngroups;
        rest /= p.ngroups;
        const int b = rest % p.B;  // sequences inner (see the 4-wave kernel)
        const int kvh = rest / p.B;
        const int N = p.N;
        // Chunk mode: the virtual key sequence is [placeholders | history |
        // chunk].  The qoff = min(start, W-1) history keys come from the ring
        // (older positions are outside every row's window); kmin < 64
        // placeholder keys before them put the chunk's first row at the start of
        // a 64-key tile, so that no tile mixes ring and chunk rows and every
        // tile's copy has a single source.  Placeholders are masked like keys
        // below the window.  Band mode: the sequence is the input (qbase = 0).
        int qoff = 0, hslot0 = 0, kmin = 0;
        if constexpr (CHUNK) {
            // uniform per workgroup: scalar registers, so the copy offsets stay scalar
            const int start = __builtin_amdgcn_readfirstlane(max(p.p0[b], 0));
            qoff = min(start, p.W - 1);
            hslot0 = (start - qoff) % p.W;  // ring slot of history entry 0
            kmin = (-qoff) & (kTileN - 1);
        }
        const int qbase = kmin + qoff;  // virtual position of query row 0
        const int NK = qbase + N;
        const int W = min(p.W, NK);
        const int BM = kQw * p.PB;
        const int q0 = qb * BM;
        const int h = kvh * p.G + hg * p.HG + (wv % p.HG);
        const int qw0 = q0 + kQw * (wv / p.HG);
        const int qi = qw0 + l32;
        const int qv = qbase + qi;
        const int qvw0 = qbase + qw0;

        const size_t kv_head = (size_t)(b * p.Hkv + kvh) * (size_t)N * D;
        const size_t q_head = (size_t)(b * p.Hq + h) * (size_t)N * D;
        const elem_t* kg = (const elem_t*)p.k + kv_head;
        const elem_t* k2g = DIFF ? (const elem_t*)p.k2 + kv_head : kg;
        const elem_t* vg = (const elem_t*)p.v + kv_head;
        const elem_t* qg = (const elem_t*)(map ? p.q2 : p.q) + q_head;
        elem_t* og = (elem_t*)p.out + q_head;
        const size_t ring_head = (size_t)(b * p.Hkv + kvh) * (size_t)p.W * D;
        const elem_t* krg = CHUNK ? (const elem_t*)p.kring + ring_head : nullptr;
        const elem_t* vrg = CHUNK ? (const elem_t*)p.vring + ring_head : nullptr;

        const int wr = p.wr;  // right radius of a two-sided band (0: causal)
        // every kernel argument the epilogue needs is in registers before the
        // tile loop: a scalar load still in flight there would force every LDS
        // wait in the loop to drain all outstanding reads
        const float* lam_ptr = p.lam;
        float* lse_ptr = p.lse;
        asm volatile("" ::"s"(lam_ptr), "s"(lse_ptr));
        const int kt_hi = min(NK - 1, qbase + q0 + BM - 1 + wr) / kTileN;
        const int kt_lo = max(0, qbase + q0 - W + 1) / kTileN;
        const int nband = kt_hi - kt_lo + 1;
        // global mode: M global positions lie below the band (entries 0..M-1
        // of the sorted list, the compact tile's rows)
        int M = 0;
        if constexpr (GLOBAL) M = global_lower_bound(p.gidx, p.ng, kt_lo * kTileN);
        const int ntiles = GLOBAL ? nband + (M > 0 ? 1 : 0) : nband;
        const bool wave_live = qw0 < N;
        // band mode: this workgroup's next block, whose first tiles and queries
        // are copied during this block's last steps (uniform scalars)
        const int Ln = STREAM ? persistent_block(blockIdx.x, iter + 1, p.nwg, p.total) : -1;
        const bool has_next = Ln >= 0;
        // its first tile, tile count, arrays and this wave's rows: set just
        // before the last masked segment, the only code that reads them (so
        // they take no registers in the loops before it)
        int kt_hi_n, n_n, qw0_n;
        const elem_t* kg_n;
        const elem_t* vg_n;
        const elem_t* qg_n;
        auto next_block = [&]() __attribute__((always_inline)) {
            const int Lx = max(Ln, 0);
            const int qb_n = Lx % p.nqb;
            int r_n = Lx / p.nqb;
            const int hg_n = r_n % p.ngroups;
            r_n /= p.ngroups;
            const int b_n = r_n % p.B, kvh_n = r_n / p.B;
            const int q0_n = qb_n * BM;
            kt_hi_n = min(NK - 1, q0_n + BM - 1 + wr) / kTileN;
            n_n = kt_hi_n - max(0, q0_n - W + 1) / kTileN + 1;
            const size_t kv_n = (size_t)(b_n * p.Hkv + kvh_n) * (size_t)N * D;
            kg_n = (const elem_t*)p.k + kv_n;
            vg_n = (const elem_t*)p.v + kv_n;
            qg_n = (const elem_t*)p.q + (size_t)(b_n * p.Hq + kvh_n * p.G + hg_n * p.HG + (wv % p.HG)) * (size_t)N * D;
            qw0_n = q0_n + kQw * (wv / p.HG);
        };
        // steps of this block: its tiles, then (with a next block) placeholder
        // steps that only copy, up to a multiple of three
        const int n3 = has_next ? (ntiles + 2) / 3 * 3 : ntiles;

        if (!pre) {
            const uint32_t flip = p.neg ? 0x80008000u : 0u;
            const uint32_t keep = qi < N ? 0xffffffffu : 0u;
            const size_t qrow = (size_t)min(qi, N - 1) * D;
#pragma unroll
            for (int c = 0; c < NQF; ++c) {
                u32x4_t w = *(const u32x4_t*)(qg + qrow + 16 * c + 8 * g);
                w = (w & keep) ^ flip;
                qf[c] = __builtin_bit_cast(bf16x8_t, w);
            }
        }

        // V swizzle: the 64-byte quarter q of row r is stored at quarter
        // q ^ vswz(r) (d=128: r mod 4; d=64: bit 1 of r)
        auto vswz = [](int r) __attribute__((always_inline)) {
            return D == 128 ? ((r & 3) << 6) : (((r >> 1) & 1) << 6);
        };
        const int k_lane = (((l32 >> 4) * CPR + g) << 8) + ((l32 & 15) << 4);
        // V transpose read: row 8*g + (lane&15)/4 (+16*c2, +4), bytes
        // 32*((lane>>4)&1) + 8*(lane&3) of quarter db (swizzled)
        const int v_row = 8 * g + ((lane & 15) >> 2);
        const int v_lane = v_row * RB + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
        const int vq = vswz(v_row);

        // copies: wave w fills 1 KiB blocks w, w+8, ... of the tile (lane i
        // writes bytes 16i..16i+15 of a block).  Per block the lane's source is
        // a fixed byte offset inside the tile's 64 rows (K: row sigma(pos),
        // chunk ch; V: the swizzled quarter), so a tile whose rows are 64
        // consecutive rows of one array costs one scalar base per tile (band
        // tiles and chunk tiles, the last key row bounding the resource).  Ring
        // tiles of chunk mode compute a slot per lane instead (the ring wraps).
        uint32_t koff[NBLK], voff[NBLK];  // row * RB + byte in row; row = off / RB
#pragma unroll
        for (int it = 0; it < NBLK; ++it) {
            const int P = (wave + 8 * it) * 1024 + lane * 16;
            const int within = P % (CPR * 256);
            const int pos = (P / (CPR * 256)) * 16 + ((within >> 4) & 15);
            koff[it] = (uint32_t)(sigma(pos) * RB + ((within >> 8) << 4));
            const int vr = P / RB;
            voff[it] = (uint32_t)(vr * RB + ((P % RB) ^ vswz(vr)));
        }
        // global mode: the same lane offsets for the compact tile, whose row r
        // is global position r of the list (rows past M repeat the last one and
        // are masked).  The list entries are loaded here and waited for at
        // once, so that no load of them is outstanding in the tile loop, whose
        // copy waits count copies only.
        uint32_t ckoff[NBLK], cvoff[NBLK];
        if constexpr (GLOBAL) {
#pragma unroll
            for (int it = 0; it < NBLK; ++it) {
                const int rk_ = (int)(koff[it] / RB), rv_ = (int)(voff[it] / RB);
                const int gk = M > 0 ? p.gidx[min(rk_, M - 1)] : 0;
                const int gv = M > 0 ? p.gidx[min(rv_, M - 1)] : 0;
                ckoff[it] = (uint32_t)(min(max(gk, 0), N - 1) * RB) + koff[it] % RB;
                cvoff[it] = (uint32_t)(min(max(gv, 0), N - 1) * RB) + voff[it] % RB;
                asm volatile("" ::"v"(ckoff[it]), "v"(cvoff[it]));
            }
        }
        // The copies are buffer loads straight into LDS (MUBUF "lds" form).  A
        // resource covers one (sequence, KV head) array; the byte offset of a
        // row is a lane offset, plus a scalar tile offset when the tile's 64 rows
        // are consecutive rows of one array.  (The global-segment form of the
        // same copy is a FLAT instruction that may touch LDS, which makes every
        // later LDS or memory wait in the loop drain completely.)
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg, (size_t)N * RB);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg, (size_t)N * RB);
        const __amdgpu_buffer_rsrc_t rkr = CHUNK ? make_rsrc(krg, (size_t)p.W * RB) : rk;
        const __amdgpu_buffer_rsrc_t rvr = CHUNK ? make_rsrc(vrg, (size_t)p.W * RB) : rv;
        auto issue_rows = [&](int t, char* dst, const elem_t* src, __amdgpu_buffer_rsrc_t rin,
                              __amdgpu_buffer_rsrc_t rring, const uint32_t* off, const uint32_t* coff)
            __attribute__((always_inline)) {
            if constexpr (GLOBAL) {
                // a band tile as in band mode, or the compact tile (t = nband):
                // per-lane rows of the whole array; source and offsets are
                // selected, not branched on, so every step issues the same copies
                const bool comp = t >= nband;
                const int j0 = (kt_hi - min(t, nband - 1)) * kTileN;
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(src + (size_t)j0 * D, (size_t)(NK - j0) * RB);
                const __amdgpu_buffer_rsrc_t r = comp ? rin : rb;
#pragma unroll
                for (int it = 0; it < NBLK; ++it)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        r, (__attribute__((address_space(3))) void*)(dst + (wave + 8 * it) * 1024), 16,
                        (int)(comp ? coff[it] : off[it]), 0, 0, 0);
                return;
            }
            if constexpr (!CHUNK) {
                // Band mode: one copy instruction per block whatever the tile (a
                // branch between a contiguous and a gathered copy leaves the
                // compiler's copy tracking unsure at the join, and it then drains
                // all copies before the next LDS read).  The resource starts at
                // the tile's first row and ends at the last key row, so the lane
                // offsets are loop invariant and rows past the end read as zero
                // (range-checked), which the mask and P = 0 make harmless.
                const int j0 = (kt_hi - t) * kTileN;
                const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)j0 * D, (size_t)(NK - j0) * RB);
#pragma unroll
                for (int it = 0; it < NBLK; ++it)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        r, (__attribute__((address_space(3))) void*)(dst + (wave + 8 * it) * 1024), 16, (int)off[it], 0, 0,
                        0);
                return;
            }
            // Chunk mode: a tile is all chunk rows (one scalar base into the
            // input, rows past the end read as zero) or all ring rows (history
            // and placeholder keys).  Ring rows take a slot per lane, wrapping at
            // the ring's end; placeholder rows read history entry 0, which
            // exists whenever there are placeholders, and are masked.  Source
            // and offsets are selected, not branched on, so every step issues
            // the same copies and the copy waits stay partial.
            const int j0 = (kt_hi - t) * kTileN;
            const bool ring = j0 < qbase;
            const int c0 = max(j0 - qbase, 0);
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(src + (size_t)c0 * D, (size_t)(N - c0) * RB);
            const __amdgpu_buffer_rsrc_t r = ring ? rring : rc;
            const int s0 = hslot0 + j0 - kmin;  // unwrapped slot of the tile's row 0
#pragma unroll
            for (int it = 0; it < NBLK; ++it) {
                const int row = (int)(off[it] / RB);
                const uint32_t byte = off[it] % RB;
                const uint32_t u = (uint32_t)max(s0 + row, hslot0);  // < 2W
                const uint32_t slot = min(u, u - (uint32_t)p.W);       // u or u - W
                const uint32_t o = ring ? slot * RB + byte : off[it];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    r, (__attribute__((address_space(3))) void*)(dst + (wave + 8 * it) * 1024), 16, (int)o, 0, 0, 0);
            }
        };
        // band mode: tile kt (absolute) of the K or V array `src`, as in issue_rows
        auto issue_band = [&](int kt, char* dst, const elem_t* src, const uint32_t* off) __attribute__((always_inline)) {
            const int j0 = kt * kTileN;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)j0 * D, (size_t)(NK - j0) * RB);
#pragma unroll
            for (int it = 0; it < NBLK; ++it)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    r, (__attribute__((address_space(3))) void*)(dst + (wave + 8 * it) * 1024), 16, (int)off[it], 0, 0, 0);
        };
        // copy stream position sp: the block's tile min(sp, n-1) (past the end
        // of its list the last tile again, into a buffer nobody reads), or in
        // band mode, from position n3 on, the next block's first tiles.  Only
        // the last masked segment and the copy-only steps reach position n3
        // (CROSS); there source and tile are selected, not branched on, so
        // every step issues the same copies.
        auto issue_k = [&](auto cross, int sp, char* kl, char* kl2) __attribute__((always_inline)) {
            if constexpr (STREAM && decltype(cross)::value) {
                const bool nx = has_next && sp >= n3;
                issue_band(nx ? kt_hi_n - min(sp - n3, n_n - 1) : kt_hi - min(sp, ntiles - 1), kl, nx ? kg_n : kg, koff);
            } else if constexpr (STREAM) {
                issue_band(kt_hi - min(sp, ntiles - 1), kl, kg, koff);
            } else {
                issue_rows(min(sp, ntiles - 1), kl, kg, rk, rkr, koff, ckoff);
                if constexpr (DIFF) issue_rows(min(sp, ntiles - 1), kl2, k2g, rk, rk, koff, ckoff);
            }
        };
        auto issue_v = [&](auto cross, int sp, char* vl) __attribute__((always_inline)) {
            if constexpr (STREAM && decltype(cross)::value) {
                const bool nx = has_next && sp >= n3;
                issue_band(nx ? kt_hi_n - min(sp - n3, n_n - 1) : kt_hi - min(sp, ntiles - 1), vl, nx ? vg_n : vg, voff);
            } else if constexpr (STREAM) {
                issue_band(kt_hi - min(sp, ntiles - 1), vl, vg, voff);
            } else {
                issue_rows(min(sp, ntiles - 1), vl, vg, rv, rvr, voff, cvoff);
            }
        };
        // band mode: this wave's 32 query rows of the next block into its qst
        // region (lane i of 1 KiB block b fetches chunk 2b + i/32 of row i%32;
        // the range check zeroes rows past the sequence)
        auto stage_q = [&]() __attribute__((always_inline)) {
            if constexpr (STREAM) {
                const __amdgpu_buffer_rsrc_t r =
                    make_rsrc(qg_n + (size_t)min(qw0_n, N) * D, (size_t)max(N - qw0_n, 0) * RB);
                char* qs = (wave < 4 ? (wave < 2 ? qs0 : qs1) : (wave < 6 ? qs2 : qs3)) + (wave & 1) * (kQw * RB);
#pragma unroll
                for (int b4 = 0; b4 < RB / 32; ++b4)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        r, (__attribute__((address_space(3))) void*)(qs + b4 * 1024), 16,
                        l32 * RB + ((2 * b4 + g) << 4), 0, 0, 0);
            }
        };
        // band mode: the next block's queries from the staging area into qf
        // (chunk 2c + g of row l32), at the last step of this block's list.
        // Rows past the sequence arrive as zeros (the staging copy's range
        // check), so only a negative scale needs a pass over the registers.
        auto load_next_q = [&]() __attribute__((always_inline)) {
            if constexpr (STREAM) {
                const char* qs = (wave < 4 ? (wave < 2 ? qs0 : qs1) : (wave < 6 ? qs2 : qs3)) + (wave & 1) * (kQw * RB);
#pragma unroll
                for (int c = 0; c < NQF; ++c) qf[c] = *(const bf16x8_t*)(qs + (((2 * c + g) * kQw + l32) << 4));
                if (p.neg) {
#pragma unroll
                    for (int c = 0; c < NQF; ++c)
                        qf[c] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, qf[c]) ^ 0x80008000u);
                }
            }
        };
        // Every step issues the same copies (past the end of the list the last
        // tile again, into a buffer nobody reads any more), so one fixed wait
        // count holds: the CPS*NBLK loads of the current step may stay in flight.
        constexpr int CPS = DIFF ? 3 : 2;  // tiles copied per step: K (K1 and K2) and V
        auto wait_older_copies = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0xF70 | (CPS * NBLK)); };

        f32x16_t oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
        // m_run starts at the lowest finite value rather than -inf: a row with
        // no allowed key yet then needs no special case (its scores are -inf,
        // exp2(-inf + FLT_MAX) = 0), and the first finite tile maximum always
        // grows it (alpha = exp2(-FLT_MAX - m) = 0)
        float m_run = -FLT_MAX, l_run = 0.f;
        const float c = p.c;
        float alpha = 1.f;

        auto scores = [&](const char* kl, f32x16_t* sc) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
#pragma unroll
                for (int cc = 0; cc < NQF; ++cc) {
                    const bf16x8_t a = *(const bf16x8_t*)(kl + k_lane + ((kb * 2 * CPR + 2 * cc) << 8));
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], sc[kb], 0, 0, 0);
                }
            }
        };
        auto mask_tile = [&](int t, f32x16_t* sc) __attribute__((always_inline)) {
            if constexpr (GLOBAL) {
                if (t >= nband) {
                    // the compact tile: element C of this lane holds entry
                    // 8g + C, valid below M
                    int nk = M - 8 * g;
                    asm volatile("" : "+v"(nk));
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int C = kb * 32 + 16 * (i >> 3) + (i & 7);
                            sc[kb][i] = C < nk ? sc[kb][i] : -INFINITY;
                        }
                    return;
                }
            }
            const int j0 = (kt_hi - t) * kTileN;
            const bool edge =
                !(j0 + kTileN - 1 <= qvw0 + wr && j0 >= qvw0 + kQw - W && j0 + kTileN <= NK && (!CHUNK || j0 >= kmin));
            if (edge) {
                // key of element i in block kb is j0 + 8g + C, C = kb*32 + 16*(i/8) + i%8;
                // with x = qv - j0 - 8g its distance is x - C, so each test is one
                // compare of a per-tile bound against a constant (the empty asm
                // keeps the compiler from turning them into 32 loop-invariant
                // per-lane constants)
                const int x = qv - j0 - 8 * g;
                int lo = x + wr;           // dist >= -wr  <=>  C <= lo
                int hi = x - W;            // dist < W     <=>  C > hi
                int nk = NK - j0 - 8 * g;  // key < NK     <=>  C < nk
                if constexpr (CHUNK) hi = max(hi, kmin - 1 - j0 - 8 * g);  // key >= kmin
                asm volatile("" : "+v"(lo), "+v"(hi), "+v"(nk));
                // which bounds this tile can violate (wave-uniform): most edge
                // tiles need one compare per element, not three
                const bool need_lo = j0 + kTileN - 1 > qvw0 + wr, need_nk = j0 + kTileN > NK;
                const bool need_hi = j0 < qvw0 + kQw - W || (CHUNK && j0 < kmin);
                auto apply = [&](auto keep_of) __attribute__((always_inline)) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int C = kb * 32 + 16 * (i >> 3) + (i & 7);
                            sc[kb][i] = keep_of(C) ? sc[kb][i] : -INFINITY;
                        }
                };
                // global mode: bit o of smask says key j0 + o is a global
                // position, allowed whatever the window (tiles inside every
                // row's window do not need it)
                auto global_bits = [&]() __attribute__((always_inline)) {
                    uint64_t smask = 0;
                    for (int e = global_lower_bound(p.gidx, p.ng, j0); e < p.ng && p.gidx[e] < j0 + kTileN; ++e)
                        smask |= 1ull << (p.gidx[e] - j0);
                    return smask >> (8 * g);
                };
                if (!need_hi && !need_nk) {
                    apply([&](int C) { return C <= lo; });
                } else if (!need_lo && !need_nk) {
                    if constexpr (GLOBAL) {
                        const uint64_t sm = global_bits();
                        apply([&](int C) { return (C > hi) | (((sm >> C) & 1ull) != 0); });
                    } else {
                        apply([&](int C) { return C > hi; });
                    }
                } else {
                    if constexpr (GLOBAL) {
                        const uint64_t sm = global_bits();
                        apply([&](int C) { return (C <= lo) & (C < nk) & ((C > hi) | (((sm >> C) & 1ull) != 0)); });
                    } else {
                        apply([&](int C) { return (C <= lo) & (C < nk) & (C > hi); });
                    }
                }
            }
        };
        auto tile_max = [&](const f32x16_t* sc) __attribute__((always_inline)) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
            return partner_max(mx);
        };
        auto softmax_head = [&](float mx) __attribute__((always_inline)) {
            const float m_cand = fmaxf(m_run, mx * c);
            const bool grow = m_cand > m_run + 8.f;
            alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_cand) : 1.f;
            m_run = grow ? m_cand : m_run;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            }
        };
        // Tile work of one step, in one straight-line block: DO_PV = this tile's
        // probabilities, row sum and P*V (from sc, vl); DO_S = the next tile's
        // scores (into sn, from kl).  16 keys at a time, so that every matrix
        // instruction has vector work of the same wave beside it.
        // K fragments of one 16-key region of the score block (the
        // contraction chunks cc = c2 * NQF/4 ..), loaded one region ahead
        struct KFrag {
            bf16x8_t a[NQF / 2];
        };
        auto load_k = [&](const char* kl, int c2, KFrag& f) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NQF / 2; ++i) {
                const int kb = i & 1, cc = c2 * (NQF / 4) + (i >> 1);
                f.a[i] = *(const bf16x8_t*)(kl + k_lane + ((kb * 2 * CPR + 2 * cc) << 8));
            }
        };
        // score instructions of one 16-key region (K fragments kf)
        auto s_region = [&](int c2, const KFrag& kf, f32x16_t* sn) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NQF / 2; ++i) {
                const int kb = i & 1, cc = c2 * (NQF / 4) + (i >> 1);
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.a[i], qf[cc], sn[kb], 0, 0, 0);
            }
        };
        auto tile_work = [&](auto do_pv, auto do_s, f32x16_t* sc, f32x16_t* sn, const char* kl, const char* vl,
                             KFrag& kf0, KFrag& kf1, auto finish_next) __attribute__((always_inline)) {
            constexpr bool DP = decltype(do_pv)::value, DS = decltype(do_s)::value;
            const float m_use = m_run;
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
            // one running row sum, started from the rescaled old one
            float rs = 0.f;
            if constexpr (DP) rs = l_run * alpha;
            bf16x8_t pb[4];
            auto probs = [&](int c2) __attribute__((always_inline)) {
                u32x4_t pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = __builtin_amdgcn_exp2f(fmaf(sc[c2 >> 1][8 * (c2 & 1) + 2 * e], c, -m_use));
                    const float x1 = __builtin_amdgcn_exp2f(fmaf(sc[c2 >> 1][8 * (c2 & 1) + 2 * e + 1], c, -m_use));
                    const bf16x2_t pr = {(__bf16)x0, (__bf16)x1};
                    rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
                    pw[e] = __builtin_bit_cast(uint32_t, pr);
                }
                pb[c2] = __builtin_bit_cast(bf16x8_t, pw);
                asm volatile("" : "+v"(rs));  // keep the dot chain beside its exponentials
            };
            // region c2: P*V of region c2 and the scores of region c2 + 1 (the
            // scores of region 0 were issued before the softmax head)
            auto mfmas = [&](int c2, const KFrag& kf) __attribute__((always_inline)) {
                u32x4_t vf[NDB];
                if constexpr (DP) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const char* vp = vl + v_lane + ((64 * db) ^ vq) + 16 * c2 * RB;
                        const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lds_read_tr16(vp));
                        const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, lds_read_tr16(vp + 4 * RB));
                        vf[db] = u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
                    }
                }
                if constexpr (DS) {
                    if (c2 < 2) load_k(kl, c2 + 2, (c2 & 1) ? kf1 : kf0);
                }
#pragma unroll
                for (int i = 0; i < NQF / 2; ++i) {
                    if constexpr (DS) {
                        if (c2 < 3) {
                            const int kb = i & 1, cc = (c2 + 1) * (NQF / 4) + (i >> 1);
                            sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.a[i], qf[cc], sn[kb], 0, 0, 0);
                        }
                    }
                    if constexpr (DP) {
                        const int db = i;
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[db]), pb[c2],
                                                                          oacc[db], 0, 0, 0);
                    }
                }
            };
            if constexpr (DP) probs(0);
            float mx_next = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2) {
                __builtin_amdgcn_sched_barrier(0);
                // the last region masks the next block (edge tiles) and takes its
                // row maximum beside this tile's last P*V instructions
                if (c2 == 3) mx_next = finish_next();
                mfmas(c2, (c2 & 1) ? kf0 : kf1);
                if constexpr (DP) {
                    if (c2 < 3) probs(c2 + 1);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (DP) l_run = rs;
            return mx_next;
        };

        const int n = ntiles;
        if (!pre) {
            {
                // V(0), the top tile, may end past the last key row; whether or
                // not a range-checked copy writes its zeros, those rows of vb0
                // must hold finite values (they meet P = 0), so the buffer starts
                // zeroed (the barrier below orders these writes before the
                // copies; later blocks find finite tile data there)
                const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int it = 0; it < TILE_BYTES / (kThreads8 * 16); ++it)
                    *(u32x4_t*)(vb0 + (it * kThreads8 + tid) * 16) = z;
            }
            // prologue: K(0), scores of tile 0; then K(1), V(0), K(2), V(1) in flight
            issue_k(std::false_type{}, 0, kb0, kc0);
            __builtin_amdgcn_s_waitcnt(0xF70);
            lds_barrier();
        }
        // (streamed: K(0), K(1) and V(0) landed before the previous block's
        // last barrier, K(2) and V(1) are in flight, and that block's last step
        // already computed tile 0's scores from K(0) with these queries)
        if (!pre) scores(map ? kc0 : kb0, scur);
        mask_tile(0, scur);
        float mx_cur = tile_max(scur);
        // tile 0's K reads are done before K(3) lands in kb0 (streamed: they
        // were done before the previous block's last barrier)
        if (!pre) lds_barrier();
        if (!pre) {
            issue_k(std::false_type{}, 1, kb1, kc1);
            issue_v(std::false_type{}, 0, vb0);
            issue_k(std::false_type{}, 2, kb2, kc2);
            issue_v(std::false_type{}, 1, vb1);
            wait_older_copies();
            lds_barrier();
        }

        // step t: scores of t+1 from kn, P*V of t from vc; K(t+3) -> ki, V(t+2) -> vi.
        // MASKED: tile t+1 may be an edge tile of this wave (the wave-uniform
        // test in mask_tile decides); otherwise it is known to be interior for
        // every wave and the step has no mask code at all.
        // kn2, ki2: the second map's K buffers (differential attention)
        // LASTPOS: the step may be the list's last position (a round's third
        // step of the last segment, as n3 is a multiple of three), whose score
        // block becomes the next block's first (tile 0 from K(0) in kb0, with
        // the next block's queries)
        auto step = [&](auto masked, auto cross, auto lastpos, int t, const char* kn1, const char* kn2, const char* vc,
                        char* ki, char* ki2, char* vi) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked)::value;
            if constexpr (STREAM && decltype(lastpos)::value) {
                if (has_next && t == n3 - 1) load_next_q();
            }
            issue_k(cross, t + 3, ki, ki2);
            issue_v(cross, t + 2, vi);
            const char* kn = map ? kn2 : kn1;  // this wave's K buffer
            // K fragments of the next tile's first two regions; its first
            // region's scores, then this tile's head (row maximum taken in the
            // previous step)
            KFrag kf0, kf1;
            load_k(kn, 0, kf0);
            load_k(kn, 1, kf1);
            f32x16_t snext[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) snext[kb][i] = 0.f;
            // past the last tile the score block reads stale data and is discarded
            s_region(0, kf0, snext);
            softmax_head(mx_cur);
            mx_cur = tile_work(std::true_type{}, std::true_type{}, scur, snext, kn, vc, kf0, kf1,
                               [&]() __attribute__((always_inline)) {
                                   if constexpr (MASKED) {
                                       if (t + 1 < n) mask_tile(t + 1, snext);
                                   }
                                   return tile_max(snext);
                               });
            scur[0] = snext[0];
            scur[1] = snext[1];
            wait_older_copies();
            lds_barrier();
        };
        // Tiles t_a .. t_b lie inside the band of every row of the workgroup
        // (interior for every wave: after the diagonal tiles of its lowest rows,
        // at or above the window start of its highest rows, whole, and in chunk
        // mode past the placeholder keys).  Step t masks tile t+1, so steps
        // [s1, s2), with t_a <= t+1 <= t_b, need no mask.  The steps run in three
        // segments -- masked, mask-free, masked -- each starting at a multiple
        // of three, so every segment rotates the static buffers the same way;
        // the mask-free segment is a whole number of three-step rounds, so its
        // loop body has no branch at all (at W = 4096 it holds all but ~4 of the
        // ~66 steps).
        const int lo_key = qbase + q0 + wr;                // last key of the lowest rows' band
        const int hi_key = qbase + q0 + kQw * p.PB - W;    // first key of the highest rows' band
        int t_a = max(max(kt_hi - ((lo_key - (kTileN - 1)) >> 6), kt_hi - ((NK - kTileN) >> 6)), 0);
        int t_b = min(kt_hi - ((hi_key + kTileN - 1) >> 6), n - 1);
        if constexpr (CHUNK) t_b = min(t_b, kt_hi - ((kmin + kTileN - 1) >> 6));
        int s1 = n3, s2 = n3;
        if (t_a <= t_b) {
            s1 = min((max(t_a - 1, 0) + 2) / 3 * 3, n3);
            s2 = s1 + max(0, t_b - s1) / 3 * 3;  // <= t_b < n; the last step's t+1 = s2 <= t_b
        }
        // with a next block the last masked segment is never empty (it issues
        // the query staging): s2 <= n3 - 3, both multiples of three
        if (STREAM && has_next) {
            s2 = min(s2, n3 - 3);
            s1 = min(s1, s2);
        }
        // (the last segment also stages the next block's queries, waited for
        // with its first step's older copies)
        auto run_masked = [&](int t0, int t1, auto last) __attribute__((always_inline)) {
            for (int t = t0; t < t1; t += 3) {
                // (already true here; stated so that the compiler's own copy
                // tracking does not lose it at the loop head)
                wait_older_copies();
                if constexpr (decltype(last)::value) {
                    if (t == t0 && has_next) stage_q();
                }
                step(std::true_type{}, last, std::false_type{}, t, kb1, kc1, vb0, kb0, kc0, vb2);
                if (t + 1 < t1) step(std::true_type{}, last, std::false_type{}, t + 1, kb2, kc2, vb1, kb1, kc1, vb0);
                if (t + 2 < t1) step(std::true_type{}, last, last, t + 2, kb0, kc0, vb2, kb2, kc2, vb1);
            }
        };
        run_masked(0, s1, std::false_type{});
        for (int t = s1; t < s2; t += 3) {
            wait_older_copies();
            step(std::false_type{}, std::false_type{}, std::false_type{}, t, kb1, kc1, vb0, kb0, kc0, vb2);
            step(std::false_type{}, std::false_type{}, std::false_type{}, t + 1, kb2, kc2, vb1, kb1, kc1, vb0);
            step(std::false_type{}, std::false_type{}, std::false_type{}, t + 2, kb0, kc0, vb2, kb2, kc2, vb1);
        }
        if constexpr (STREAM) next_block();
        run_masked(s2, n, std::true_type{});
        if constexpr (STREAM) {
            // steps n .. n3-1 (at most two, the last ones of a three-step round,
            // so their buffers are known): copies only, which bring the next
            // block's first tiles into the buffers its prologue would fill
            // (the list's last position computes the next block's tile 0
            // scores, as a tile step there would)
            auto copy_step = [&](auto last_pos, int t, char* ki, char* vi) __attribute__((always_inline)) {
                if constexpr (decltype(last_pos)::value) {
                    if (has_next) {
                        load_next_q();
                        scores(kb0, scur);
                    }
                }
                issue_k(std::true_type{}, t + 3, ki, ki);
                issue_v(std::true_type{}, t + 2, vi);
                wait_older_copies();
                lds_barrier();
            };
            if (n3 - n == 2) copy_step(std::false_type{}, n3 - 2, kb1, vb0);
            if (n3 - n >= 1) copy_step(std::true_type{}, n3 - 1, kb2, vb1);
        }
        // no copy may still be writing this workgroup's LDS when it ends (with
        // a next block, its first copies stay in flight)
        if (!has_next) __builtin_amdgcn_s_waitcnt(0xF70);

        const float lt = partner_sum(l_run);
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        f32x4_t ysub[NDB * 4];  // differential attention: lam * O2 / l2 of this block, in this lane's layout
        if constexpr (DIFF) {
            // Every wave has passed the last step's barrier and every copy has
            // landed, so the K buffers are free.  The second map's wave of query
            // block wv leaves lam * O2 / l2 in buffer wv (its 16-byte group r of
            // lane l at (r * 64 + l) * 16: each access is 1 KiB contiguous), and
            // the first map's wave of the same block, whose lanes hold the same
            // (row, column) elements, reads it back.
            char* xb = wv == 0 ? kb0 : wv == 1 ? kb1 : wv == 2 ? kb2 : kc0;
            if (map == 1) {
                const float s2 = lam_ptr[h] / lt;
#pragma unroll
                for (int r = 0; r < NDB * 4; ++r) {
                    const f32x4_t y = {oacc[r >> 2][4 * (r & 3) + 0] * s2, oacc[r >> 2][4 * (r & 3) + 1] * s2,
                                       oacc[r >> 2][4 * (r & 3) + 2] * s2, oacc[r >> 2][4 * (r & 3) + 3] * s2};
                    *(f32x4_t*)(xb + (r * 64 + lane) * 16) = y;
                }
            }
            lds_barrier();
            if (map == 1) continue;
#pragma unroll
            for (int r = 0; r < NDB * 4; ++r) ysub[r] = *(const f32x4_t*)(xb + (r * 64 + lane) * 16);
        }
        if (!wave_live || qi >= N) continue;
        if (lse_ptr != nullptr && g == 0)  // ln of the row's softmax denominator (see the 4-wave kernel)
            lse_ptr[(size_t)(b * p.Hq + h) * N + qi] = (m_run + __log2f(lt)) * 0.69314718055994531f;
        if constexpr (!DIFF) {
            if (lam_ptr == nullptr) {
                // Plain output, 16 bytes per lane and store: lane g of query l32
                // holds d = 32 db + 8 quad + 4 g + 0..3.  Rounded to bf16 pairs,
                // one cross-half swap per pair of words regroups quads 2qp and
                // 2qp + 1 so that lane g holds d = 32 db + 16 qp + 8 g + 0..7:
                // eight 16-byte stores per lane instead of sixteen 8-byte ones
                // (each store instruction touches the same 32 rows either way).
                const float inv = 1.f / lt;
                auto pk = [&](int db, int quad, int k) __attribute__((always_inline)) {
                    const bf16x2_t pr = {(__bf16)(oacc[db][4 * quad + 2 * k] * inv),
                                         (__bf16)(oacc[db][4 * quad + 2 * k + 1] * inv)};
                    return __builtin_bit_cast(uint32_t, pr);
                };
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int qp = 0; qp < 2; ++qp) {
                        u32x4_t w;
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            // lanes 0..31 keep quad 2qp and receive the other half's;
                            // lanes 32..63 receive quad 2qp + 1 and keep their own
                            const auto r = __builtin_amdgcn_permlane32_swap(pk(db, 2 * qp, k), pk(db, 2 * qp + 1, k),
                                                                            false, false);
                            w[k] = r[0];
                            w[2 + k] = r[1];
                        }
                        *(u32x4_t*)(og + (size_t)qi * D + 32 * db + 16 * qp + 8 * g) = w;
                    }
                continue;
            }
        }
        // second launch of the two-launch differential attention: out -= lam * O/l
        const bool sub = !DIFF && lam_ptr != nullptr;
        const float inv = (sub ? -lam_ptr[h] : 1.f) / lt;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int quad = 0; quad < 4; ++quad) {
                const int d0 = db * 32 + 8 * quad + 4 * g;
                typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                bf16x4_t* dst = (bf16x4_t*)(og + (size_t)qi * D + d0);
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = oacc[db][4 * quad + e] * inv;
                if constexpr (DIFF) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] -= ysub[db * 4 + quad][e];
                }
                if (sub) {
                    const bf16x4_t prev = *dst;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] += (float)prev[e];
                }
                const bf16x4_t ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
                *dst = ob;
            }
    }
}

template <bool BF, int D, int MODE>
hipError_t launch_one(const PrefillParams& p, hipStream_t s) {
    if constexpr (MODE == kDiff) {
        // one-pass differential attention: 8-wave kernel only (the host sends
        // other shapes to two band launches)
        if constexpr (BF) {
            hipLaunchKernelGGL((band8_kernel<D, kDiff>), dim3(p.nwg), dim3(kThreads8), 0, s, p);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        if constexpr (BF && (MODE == kBand || MODE == kChunk || MODE == kGlobal)) {
            // (the host picks 8 waves only where the 8-wave kernel applies,
            // including its 32-bit byte offsets into a K/V array and, for
            // global tokens, at most 64 positions)
            if (p.HG * p.PB == 8) {
                hipLaunchKernelGGL((band8_kernel<D, MODE>), dim3(p.nwg), dim3(kThreads8), 0, s, p);
                return hipGetLastError();
            }
        }
        if constexpr (BF && MODE == kStrided) {
            if (p.ks) {
                hipLaunchKernelGGL((band_fwd_kernel<BF, D, MODE, true>), dim3(p.total), dim3(kThreads), 0, s, p);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((band_fwd_kernel<BF, D, MODE>), dim3(p.total), dim3(kThreads), 0, s, p);
        return hipGetLastError();
    }
}

template <bool BF, int D>
hipError_t launch_mode(int mode, const PrefillParams& p, hipStream_t s) {
    if (mode == kStrided) return launch_one<BF, D, kStrided>(p, s);
    if (mode == kChunk) return launch_one<BF, D, kChunk>(p, s);
    if (mode == kGlobal) return launch_one<BF, D, kGlobal>(p, s);
    if (mode == kDiff) return launch_one<BF, D, kDiff>(p, s);
    return launch_one<BF, D, kBand>(p, s);
}

}  // namespace

int persistent_workgroups(int total) {
    // CUs of the current device, looked up once per device (a racing first
    // lookup on two threads stores the same value)
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return total;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) return total;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    n &= ~7;
    return total > n ? n : total;
}

hipError_t launch_band_fwd(bool bf16, int d, int mode, const PrefillParams& p, hipStream_t s) {
    if (bf16) return d == 128 ? launch_mode<true, 128>(mode, p, s) : launch_mode<true, 64>(mode, p, s);
    return d == 128 ? launch_mode<false, 128>(mode, p, s) : launch_mode<false, 64>(mode, p, s);
}

}  // namespace swa
