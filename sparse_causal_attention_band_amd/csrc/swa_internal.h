// Internal declarations shared by the kernel translation units and the C ABI
// layer.  Not installed; the public interface is include/swa_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

// ---------------------------------------------------------------- prefill
// kDiff: differential attention in one pass (bf16, 8-wave kernel): two
// query/key pairs over one V, the second map's waves beside the first's.
enum { kBand = 0, kStrided = 1, kChunk = 2, kGlobal = 3, kDiff = 4 };

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const void* kring;     // chunk mode: [B, Hkv, W, d] history ring
    const void* vring;
    const int32_t* p0;     // chunk mode: [B] positions already cached
    const void* q2;        // differential attention (kDiff): the second map's queries [B, Hq, N, d]
    const void* k2;        //   and keys [B, Hkv, N, d]; q / k are the first map's
    const float* lam;      // kDiff: out = A1 V - lam[h] A2 V; other modes, non-null: out -= lam[h] * result
    float* lse;            // non-null: [B, Hq, N] row log-sum-exp (natural log of the softmax denominator)
    const int32_t* gidx;   // global mode: sorted global positions [ng]
    int ng;
    int B, Hq, Hkv, N;
    int W;        // window (band modes: clamped to N; chunk mode: the ring size)
    int wr;       // two-sided band: keys up to i + wr are read too (0: causal)
    int stride;   // > 0 only for the strided instantiation
    float c;      // |scale| * log2(e): scores are kept in the log2 domain
    int neg;      // scale < 0: queries enter with flipped sign (exact)
    int G;        // Hq / Hkv
    int HG;       // query heads of one KV head that share a workgroup
    int PB;       // 32-query blocks per head in a workgroup (HG * PB = waves: 4 or 8;
                  // kDiff: 4, each block served by one wave per map)
    int nqb;      // query tiles per head
    int ngroups;  // G / HG
    int ks;       // 4-wave kernel, key split: HG * PB = 2 blocks, each on a pair of
                  // waves that take the two key halves of every tile
    int total;    // logical blocks (query tiles x head groups x sequences x KV heads,
                  // the first fastest)
    int nwg;      // workgroups in the grid: total, or (8-wave kernel) fewer persistent ones
};

// Persistent workgroups of the 8-wave kernel: one per CU (its LDS and
// registers allow one), a multiple of 8, at most `total`.
int persistent_workgroups(int total);

// Launch the band kernel for one (dtype, head dim, mode) combination.
hipError_t launch_band_fwd(bool bf16, int d, int mode, const PrefillParams& p, hipStream_t s);

// Copy a chunk's K/V rows into their ring slots (position t -> slot (t-1) % W).
hipError_t launch_ring_append(int elem_bytes, int d, const void* k, const void* v, const int32_t* p0, void* kring,
                              void* vring, int B, int Hkv, int T, int W, hipStream_t s);

// Rows of one workgroup tile, for host-side bookkeeping and tests.
constexpr int kQueriesPerWave = 32;
constexpr int kKeysPerTile = 64;

// Global positions the 8-wave kernel takes: the ones below a block's band
// form one compact tile.
constexpr int kMaxGlobal8 = 64;

// Waves per workgroup of the band kernels, which also picks the kernel (8
// waves: the 8-wave kernel, 4: the 4-wave one).  Every wave of a workgroup
// walks the key tiles of all its rows, so a workgroup should span few
// positions: bf16 band, chunk and global-token modes (at most kMaxGlobal8
// positions) with an even number of query heads per KV head run 8 waves
// (4 heads x 64 positions, or 2 heads x 128), and everything else (fp32,
// odd head groups, strided keys, longer global lists: `keylist`) 4 waves.
// The 8-wave kernel
// addresses a K/V array with 32-bit byte offsets: `rows` (the longest K/V
// array of one head, in rows of `d` bf16 values) must stay below 2 GiB.
inline int waves_per_group(bool bf16, bool keylist, int G, long long rows, int d) {
    const bool small = rows * d * 2 < (1ll << 31);
    return bf16 && !keylist && G % 2 == 0 && small ? 8 : 4;
}

// The bf16 local + strided forward with an odd number of query heads per KV
// head runs the 4-wave kernel with its key split: two 32-query blocks per
// workgroup (64 positions instead of 128), so each row walks fewer key tiles.
inline bool key_split(bool bf16, int mode, int G) {
    return bf16 && mode == kStrided && (G & 1);
}

// Split a workgroup's waves into HG query heads (of one KV head) times PB
// blocks of 32 positions: HG is the largest power of two <= waves dividing G.
inline void set_wave_split(PrefillParams& p, int waves, int rows) {
    int hg = 1;
    while (hg * 2 <= waves && p.G % (hg * 2) == 0) hg *= 2;
    p.HG = hg;
    p.PB = waves / hg;
    const int BM = kQueriesPerWave * p.PB;
    p.nqb = (rows + BM - 1) / BM;
    p.ngroups = p.G / hg;
}

// ---------------------------------------------------------------- decode
struct DecodeParams {
    const void* q;
    const void* kring;
    const void* vring;
    const int32_t* pos;
    void* out;
    float* ws_acc;   // [B, Hq, nsplit, d]  un-normalised weighted V sums
    float* ws_ml;    // [B, Hq, nsplit, 2]  (running max in log2 units, sum)
    int B, Hq, Hkv, W;
    int nsplit;      // ceil(W / split_len); 1 = the split kernel writes out itself
    // Row mode (global rows of the local + global pattern): entry e of the
    // B entries is sequence e / ng, row i = gidx[e % ng] of q/out laid out
    // [B/ng, Hq, N, d]; it reads keys 0..i of kring/vring = K/V [B/ng, Hkv, N, d]
    // (W = N).  nullptr: ordinary decode entries.
    const int32_t* gidx;
    int ng, N;
    int split_len;   // ring slots per split (multiple of the 64-slot tile)
    float c;         // |scale| * log2(e)
    int neg;
};

// Split plan: enough workgroups for one per CU (256 CUs), each split a whole
// number of 64-slot tiles.  One split means no workspace and no merge kernel.
struct DecodeSplit {
    int nsplit;
    int split_len;
};
DecodeSplit decode_split_plan(int B, int Hkv, int W);

hipError_t launch_decode(bool bf16, int d, int G, const DecodeParams& p, hipStream_t s);

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int W, int d);

}  // namespace swa
