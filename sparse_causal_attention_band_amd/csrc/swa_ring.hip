// Rolling-cache append: the rows of a new chunk go to their ring slots.
// Chunk row r of sequence b is absolute position p0[b] + r + 1 and lands in
// slot (p0[b] + r) % W (page "SWA：滑动窗口注意力与跨层信息传递", §4.2).  Only
// the last W rows of a chunk longer than the ring survive, so only those are
// copied (no two threads write one slot).  A plain 16-byte-per-lane copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void ring_append_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                          const int32_t* __restrict__ p0, char* __restrict__ kring,
                                                          char* __restrict__ vring, int Hkv, int T, int W, int RB) {
    const int b = blockIdx.z, kvh = blockIdx.y;
    const int cpr = RB >> 4;
    const int first = T > W ? T - W : 0;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const int r = first + (int)(idx / cpr);
    const int ch = (int)(idx % cpr);
    if (r >= T) return;
    const int start = max(p0[b], 0);
    const int slot = (int)(((long long)start + r) % W);
    const size_t head = (size_t)(b * Hkv + kvh);
    const size_t src = (head * T + r) * RB + ch * 16;
    const size_t dst = (head * W + slot) * RB + ch * 16;
    *(u32x4_t*)(kring + dst) = *(const u32x4_t*)(k + src);
    *(u32x4_t*)(vring + dst) = *(const u32x4_t*)(v + src);
}

}  // namespace

hipError_t launch_ring_append(int elem_bytes, int d, const void* k, const void* v, const int32_t* p0, void* kring,
                              void* vring, int B, int Hkv, int T, int W, hipStream_t s) {
    const int RB = d * elem_bytes;
    const long long rows = T < W ? T : W;
    const long long threads = rows * (RB / 16);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(ring_append_kernel, dim3(blocks, Hkv, B), dim3(256), 0, s, (const char*)k, (const char*)v, p0,
                       (char*)kring, (char*)vring, Hkv, T, W, RB);
    return hipGetLastError();
}

}  // namespace swa
