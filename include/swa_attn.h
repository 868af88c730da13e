/*
 * swa_attn.h -- C ABI of the MI355X (gfx950) sliding-window attention library.
 *
 * What is computed
 * ----------------
 * Causal sliding-window attention, softmax(scale * Q K^T + M) V, taken row by
 * row: query position i (0-based) reads key j iff
 *     j <= i  and  ( i - j < window   or   (stride > 0 and j % stride == 0) ).
 * The window counts the current position: with window W the band is
 * [max(0, i-W+1), i].  This is the set N_W(i) and mask M^SWA of the page
 * "SWA：滑动窗口注意力与跨层信息传递" (§3.1), written 0-based; the strided
 * part is the "local + strided" mask of the page
 * "注意力变体——滑动窗口、稀疏、差分" (构建它, 第 3 步), whose union with the
 * band is a set (a key is read once).  window >= N is full causal attention,
 * window == 1 returns V row for row.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises: each call validates its
 *    arguments on the host, enqueues its kernels on `stream` (NULL = the
 *    default stream) and returns.  Results are ready when the stream reaches
 *    that point.
 *  - Tensors are dense, row-major, with no padding between rows.
 *  - "bf16" is bfloat16 stored as 16-bit words.  Arithmetic is fp32 inside
 *    (scores, softmax and accumulators); the probabilities are rounded to
 *    bf16 (round to nearest even) for the P*V product on the bf16 matrix
 *    cores, the output is rounded once to bf16.  The *_f32 entry points do
 *    every step in fp32.
 *  - Grouped heads: query head h reads KV head h / (Hq / Hkv).
 *  - Return value: SWA_OK, or a negative code; on error nothing has been
 *    enqueued and swa_last_error() describes the problem.  No entry point
 *    aborts or throws.  Device-side data (decode `pos`) is not validated.
 *  - Outputs are deterministic: fixed reduction order, no float atomics.
 *  - Calls on different streams may run concurrently; a workspace must not be
 *    shared by calls that may overlap.
 *  - The header is plain C (C99 and later, or C++).  It includes the HIP
 *    runtime API header for hipStream_t, so a program compiled by a host
 *    compiler rather than hipcc defines __HIP_PLATFORM_AMD__, as for any HIP
 *    API use, and links libswa_attn.so.
 */
#ifndef SWA_ATTN_H
#define SWA_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifndef SWA_API
#define SWA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARG = -1, /* bad size, null or misaligned pointer, small workspace */
    SWA_ERR_UNSUPPORTED = -2, /* valid but not built: head dim other than 64/128, ... */
    SWA_ERR_HIP = -3          /* a HIP launch failed; message from hipGetErrorString */
};

/*
 * Prefill / whole-sequence forward, bf16 in, bf16 out.
 *   q, out : [B, Hq, N, d]     k, v : [B, Hkv, N, d]
 *   B, N >= 1; Hq % Hkv == 0; d in {64, 128}; window >= 1 (values >= N are
 *   treated as N: full causal, same bits); stride <= 0 disables the strided
 *   part; scale is any finite non-zero float (1/sqrt(d) for the usual
 *   attention).  Every pointer must be 16-byte aligned.  out must not alias
 *   q, k or v.
 * The band kernel visits only the (query tile, key tile) pairs that meet
 * the band (plus, when stride > 0, a compact tile list of the strided keys
 * below the band), so fully masked tiles are never loaded.
 */
SWA_API int swa_attn_fwd(const void* q, const void* k, const void* v, void* out,
                 int B, int Hq, int Hkv, int N, int d,
                 int window, int stride, float scale, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 matrix-core arithmetic. */
SWA_API int swa_attn_fwd_f32(const float* q, const float* k, const float* v, float* out,
                     int B, int Hq, int Hkv, int N, int d,
                     int window, int stride, float scale, hipStream_t stream);

/*
 * swa_attn_fwd plus the row log-sum-exp: lse[b][h][i] = ln of row i's softmax
 * denominator, ln sum over the allowed keys j of exp(scale * q_i . k_j) (the
 * row-wise softmax of the SWA page, §3.1), in fp32.  With it, results over
 * disjoint key sets merge exactly: o = (e1 o1 + e2 o2) / (e1 + e2) with
 * e_x = exp(lse_x - max(lse_1, lse_2)).
 *   lse : float [B, Hq, N] on the device, non-null, 4-byte aligned, not
 *         overlapping q, k, v or out.  Everything else as swa_attn_fwd; out
 *         is the same (bitwise) as swa_attn_fwd writes.
 */
SWA_API int swa_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Hq, int Hkv, int N, int d,
                     int window, int stride, float scale, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 matrix-core arithmetic. */
SWA_API int swa_attn_fwd_lse_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                     int B, int Hq, int Hkv, int N, int d,
                     int window, int stride, float scale, hipStream_t stream);

/*
 * One decode step per sequence over a rolling window-slot KV cache.
 * Absolute position t (1-based) lives in ring slot (t-1) % window, the rule
 * of the SWA page (§4.2); slot order is not time order, and since the
 * attention itself has no positional term the step reduces over the valid
 * slots in slot order.
 *   q, out       : [B, Hq, d]           (bf16)
 *   kring, vring : [B, Hkv, window, d]  (bf16)
 *   pos          : int32 [B] on the device: 1-based absolute position of each
 *                  query token, whose own K/V are already in the ring.  The
 *                  step reads n = min(pos, window) slots: all of them once
 *                  pos >= window, else slots 0 .. pos-1.  pos <= 0 gives an
 *                  all-zero output row.  Unread slots may hold anything,
 *                  NaN included.
 *   workspace    : device scratch of at least
 *                  swa_decode_workspace_bytes(B, Hq, Hkv, d, window) bytes,
 *                  16-byte aligned; its contents on entry do not matter.
 *                  When that size is 0 the pointer is not used (may be NULL).
 *   Hq / Hkv must be 1, 2, 4 or 8; d in {64, 128}; window >= 1.
 * One workgroup streams the K/V slots of one (sequence, KV head) pair from
 * HBM and serves its Hq/Hkv query heads.  With fewer than 256 such pairs the
 * slots are split so the GPU still gets one workgroup per CU: each split
 * writes (max, sum, weighted V) partials into the workspace and a second
 * kernel merges them by log-sum-exp; with 256 or more pairs there is one
 * kernel and no workspace.
 */
SWA_API int swa_decode(const void* q, const void* kring, const void* vring, const int32_t* pos,
               void* out, int B, int Hq, int Hkv, int d, float scale,
               void* workspace, size_t workspace_bytes, int window, hipStream_t stream);

/* Same contract with fp32 q, rings and out. */
SWA_API int swa_decode_f32(const float* q, const float* kring, const float* vring, const int32_t* pos,
                   float* out, int B, int Hq, int Hkv, int d, float scale,
                   void* workspace, size_t workspace_bytes, int window, hipStream_t stream);

/*
 * Two-sided (bidirectional) band, no causal cut: row i reads keys
 * i-left .. i+right (clipped to [0, N)).  The attention-variants page
 * (概念, 滑动窗口注意力) gives the bidirectional window [i - W/2, i + W/2];
 * the explainer page "滑动窗口注意力" (§3.1 band mask, §3.3 example) gives
 * [i - w, i + w] with a radius w; separate radii cover both.  right = 0
 * gives the same result as swa_attn_fwd with window = left + 1.
 *   q, out : [B, Hq, N, d]   k, v : [B, Hkv, N, d]   (as swa_attn_fwd)
 *   left, right >= 0 (values >= N act as N - 1); other arguments, layouts,
 *   ownership and errors as swa_attn_fwd.
 */
SWA_API int swa_attn_fwd_two_sided(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                                   int N, int d, int left, int right, float scale, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 matrix-core arithmetic. */
SWA_API int swa_attn_fwd_two_sided_f32(const float* q, const float* k, const float* v, float* out, int B, int Hq,
                                       int Hkv, int N, int d, int left, int right, float scale, hipStream_t stream);

/*
 * Differential sliding-window attention (attention-variants page, 概念 and
 * 第 4 步): out = (A1 - lam[h] * A2) V, where A1 and A2 are the causal
 * sliding-window softmax maps of (q1, k1) and (q2, k2) over the same band
 * and the same V, and lam holds one scalar per query head.
 *   q1, q2, out : [B, Hq, N, d]   k1, k2, v : [B, Hkv, N, d]
 *   lam : fp32 [Hq] on the device
 *   window, scale, d, alignment and errors as swa_attn_fwd.
 * bf16 with window < 512 (K/V arrays under 2 GiB per head): one pass of
 * the band kernel in which each workgroup runs both maps over one tile
 * stream -- the K tiles of both pairs and the shared V tile are staged once
 * per step -- and the result A1 V / l1 - lam * A2 V / l2 is formed in fp32
 * and rounded to bf16 once.  Otherwise (longer windows, where two launches
 * measure faster; fp32; larger arrays): two launches on `stream`, the first
 * writing A1 V to out and the second subtracting lam * A2 V in its epilogue
 * (in bf16, A1 V is then rounded once before the subtraction).  out must
 * not overlap any input.
 */
SWA_API int swa_diff_attn_fwd(const void* q1, const void* k1, const void* q2, const void* k2, const void* v,
                              const float* lam, void* out, int B, int Hq, int Hkv, int N, int d, int window,
                              float scale, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 matrix-core arithmetic. */
SWA_API int swa_diff_attn_fwd_f32(const float* q1, const float* k1, const float* q2, const float* k2,
                                  const float* v, const float* lam, float* out, int B, int Hq, int Hkv, int N, int d,
                                  int window, float scale, hipStream_t stream);

/*
 * Causal local window plus global tokens (attention-variants page, 稀疏 /
 * 块注意力, Longformer / BigBird; the interview page "Sliding Window
 * Attention 和 Sparse Attention 有什么区别", 其他 Sparse Attention 模式,
 * Global Token): a few global positions attend to every earlier position
 * and every later position attends to them; the rest keep the window.  Row
 * i reads key j iff j <= i and (i - j < window, or j is global, or i is
 * global).
 *   q, out : [B, Hq, N, d]   k, v : [B, Hkv, N, d]   (as swa_attn_fwd)
 *   gidx   : int32 [ng] on the device, sorted ascending, distinct, each in
 *            [0, N); the same positions for every sequence.  Not checked on
 *            the device: unsorted or repeated entries give wrong results
 *            (indices are clamped, so no out-of-bounds access).  ng = 0 is
 *            the plain band.
 *   workspace : device buffer of at least swa_attn_fwd_global_workspace_bytes
 *            (may be NULL when that is 0), overwritten.
 *   For ng > 0, Hq / Hkv must be 1, 2, 4 or 8 and B * ng <= 65535.
 * Two kernels on `stream`: the band kernel with the global keys, then the
 * split decode kernel over the global rows (their full causal rows, K/V
 * read as a linear cache), which overwrites those rows of out.
 */
SWA_API int swa_attn_fwd_global(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N,
                                int d, int window, const int32_t* gidx, int ng, float scale, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 arithmetic. */
SWA_API int swa_attn_fwd_global_f32(const float* q, const float* k, const float* v, float* out, int B, int Hq,
                                    int Hkv, int N, int d, int window, const int32_t* gidx, int ng, float scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes swa_attn_fwd_global(_f32) needs (0 when ng == 0 or the
 * global rows fit one split); 0 for invalid sizes. */
SWA_API size_t swa_attn_fwd_global_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int ng);

/*
 * Chunked prefill over the rolling cache (page "SWA：滑动窗口注意力与跨层信息传递",
 * §4.3): a chunk of T new tokens attends to the cached history plus its own
 * earlier rows, each row under its own band.  Chunk row r of sequence b is
 * absolute position i = p0[b] + r + 1 and reads positions max(1, i-W+1) .. i:
 * those up to p0[b] from the ring (position t in slot (t-1) % window), the
 * rest from the chunk.  Call it BEFORE swa_ring_append writes the chunk into
 * the ring: the append overwrites history that earlier rows of the chunk
 * still read.
 *   q, out       : [B, Hq, T, d]            k, v : [B, Hkv, T, d] (the chunk's K/V)
 *   kring, vring : [B, Hkv, window, d] holding positions up to p0[b]
 *   p0           : int32 [B] on the device, positions already cached (0 for
 *                  the first chunk; values < 0 are read as 0).  Slots the step
 *                  does not read may hold anything, NaN included.
 *   T >= 1, window >= 1, d in {64, 128}, Hq % Hkv == 0; 16-byte aligned
 *   pointers; scale finite and non-zero.  Same kernel as swa_attn_fwd (band
 *   mode over the history followed by the chunk).
 */
SWA_API int swa_chunk_prefill(const void* q, const void* k, const void* v, const void* kring, const void* vring,
                              const int32_t* p0, void* out, int B, int Hq, int Hkv, int T, int d, int window,
                              float scale, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 matrix-core arithmetic. */
SWA_API int swa_chunk_prefill_f32(const float* q, const float* k, const float* v, const float* kring,
                                  const float* vring, const int32_t* p0, float* out, int B, int Hq, int Hkv, int T,
                                  int d, int window, float scale, hipStream_t stream);

/*
 * swa_chunk_prefill plus the row log-sum-exp of each chunk row over the keys
 * it reads (history and chunk), as for swa_attn_fwd_lse.
 *   lse : float [B, Hq, T] on the device, non-null, 4-byte aligned, not
 *         overlapping out.  Everything else as swa_chunk_prefill.
 */
SWA_API int swa_chunk_prefill_lse(const void* q, const void* k, const void* v, const void* kring, const void* vring,
                                  const int32_t* p0, void* out, float* lse, int B, int Hq, int Hkv, int T, int d,
                                  int window, float scale, hipStream_t stream);

/* Same contract with fp32 tensors and fp32 matrix-core arithmetic. */
SWA_API int swa_chunk_prefill_lse_f32(const float* q, const float* k, const float* v, const float* kring,
                                      const float* vring, const int32_t* p0, float* out, float* lse, int B, int Hq,
                                      int Hkv, int T, int d, int window, float scale, hipStream_t stream);

/*
 * Rolling-cache append (SWA page §4.2): chunk row r of sequence b (absolute
 * position p0[b] + r + 1) is copied to slot (p0[b] + r) % window of kring and
 * vring; of a chunk longer than the ring only the last `window` rows are
 * written.  Bit-exact copy; afterwards the ring holds positions up to
 * p0[b] + T, ready for the next chunk or for swa_decode with pos = p0[b] + T
 * (+1 per later token).
 *   k, v : [B, Hkv, T, d]   kring, vring : [B, Hkv, window, d]   p0 : int32 [B]
 *   (device; < 0 read as 0).  16-byte aligned pointers, d in {64, 128}.
 */
SWA_API int swa_ring_append(const void* k, const void* v, const int32_t* p0, void* kring, void* vring, int B,
                            int Hkv, int T, int d, int window, hipStream_t stream);

/* Same for fp32 rings. */
SWA_API int swa_ring_append_f32(const float* k, const float* v, const int32_t* p0, float* kring, float* vring,
                                int B, int Hkv, int T, int d, int window, hipStream_t stream);

/* Workspace bytes swa_decode / swa_decode_f32 need (0 when the split plan
   for these sizes has one split, and for invalid sizes). */
SWA_API size_t swa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int window);

/*
 * swa_decode (bf16) without a caller-supplied workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * that must not call the allocator, harnesses that forbid it.  The split
 * partials go to a scratch array of SWA_DECODE_NOALLOC_SCRATCH_BYTES that the
 * library holds in each GPU's memory for the life of the process (one copy
 * per device, located once per device on the first call there).
 *   Arguments, layouts, results and errors as swa_decode, minus the
 *   workspace.  Every supported size fits (Hq / Hkv <= 8 and d <= 128 bound
 *   the split plan's partials below the scratch size); a size that would not
 *   is refused with SWA_ERR_UNSUPPORTED.  Nothing is allocated: no hipMalloc,
 *   no hipFree.  The scratch needs no clearing: every partial the merge reads
 *   is written earlier in the same call.
 *   All calls on one GPU share that GPU's scratch, which keeps the last call's
 *   partials: calls that may overlap on one GPU (different streams, or one
 *   stream and a graph replay) race and must be serialised by the caller.
 */
#define SWA_DECODE_NOALLOC_SCRATCH_BYTES 2129920
SWA_API int swa_decode_noalloc(const void* q, const void* kring, const void* vring, const int32_t* pos,
                               void* out, int B, int Hq, int Hkv, int d, float scale, int window,
                               hipStream_t stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
SWA_API const char* swa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SWA_ATTN_H */
