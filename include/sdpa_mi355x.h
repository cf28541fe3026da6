/*
 * sdpa_mi355x.h -- fused scaled-dot-product attention for AMD MI355X (gfx950).
 *
 * C linkage, plain pointers and sizes only.  The library computes, for every
 * query row, softmax(scale * Q K^T + mask) V without ever forming the
 * [heads, qL, kL] score matrix: the "fused" attention whose lack at
 * head_dim 256 makes long prefills run out of memory in lablup/mlxcel issue
 * #672 ("gemma-4 long-prompt prefill OOMs on CUDA because attention
 * materializes O(heads*L^2) scores instead of using flash SDPA", Summary and
 * Root cause), and which ml-explore/mlx PR #3293 ("fix: add head_dim=256 to
 * fused SDPA full attention kernel") and PR #3660 ("Fused SDPA
 * full-attention for head_dim=192/256") add to MLX for head_dim 192/256.
 * Its result equals the unfused matmul + softmax + matmul path (mlx PR
 * #3660, Microbenchmarks, where the fused and unfused outputs agree exactly;
 * mlx PR #3293, Benchmark) up to floating-point rounding.  Head dims: 64,
 * 80 and 128 (the dims MLX's fused kernel already took, per the routing
 * code in mlx PR #3293), 192 (which that PR's review discussion adds), 256
 * and 512, and through sdpa_forward_dv q/k of 192 with v of 256 (the
 * GLM4-MoE-Lite heads named in that same discussion).
 *
 * Tensor layout (all row-major and contiguous, as the (B, H, L, D) arrays of
 * the M3 Ultra test script in mlx PR #3293):
 *   q, out : [B, Hq,  qL, D]
 *   k, v   : [B, Hkv, kL, D]
 * Query head hq reads key/value head hq / (Hq / Hkv) (grouped-query heads,
 * e.g. n_q=16 over n_kv=8 in the mlx PR #3660 Microbenchmarks table).
 *
 * Query row i sits at absolute key position p = q_offset + i.  With causal
 * set, key j is visible from row i iff j <= p; with window w > 0 also
 * p - j < w (w keys including the row's own).  The masks are computed from
 * these indices; no [L, L] mask array exists (mlxcel issue #672, Suggested
 * fix direction 1: a causal flag instead of a materialized mask).
 * q_offset = kL - qL aligns the queries to the end of the key prefix: a
 * prefill chunk over a cached prefix (mlx PR #3660, End-to-end section) or
 * a verify block whose rows each attend their own trimmed prefix (lablup/
 * mlxcel issue #2160, "Gemma 4 MTP never engages on CUDA (GB10), verify
 * probe fails", Proposed Solution step 2).
 *
 * Calls with qL <= 4 (decode and verify) run a split-key path whose result
 * for a row is bit-identical to a qL = 1 call over that row's visible key
 * prefix, whatever qL is and whatever kL that prefix has (the byte-for-byte
 * verify-vs-decode requirement of mlxcel issue #2160, Acceptance Criteria).
 * The keys are split into chunks of a size that depends on neither: 1024
 * keys for sdpa_forward, and a size fixed by the cache's shape for
 * sdpa_forward_kv_view.
 *
 * Errors are returned as status codes; nothing is thrown across this
 * boundary, nothing aborts, nothing is printed.  The library allocates no
 * device memory; it keeps no mutable global state except a per-thread
 * message for the last failed call.  It is safe to call from several host
 * threads at once.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SDPA_OK 0
#define SDPA_INVALID_ARG 1          /* a pointer, size, flag or offset is out of range */
#define SDPA_UNSUPPORTED 2          /* head_dim not 64/80/128/192/256/512, or an unknown dtype */
#define SDPA_WORKSPACE_TOO_SMALL 3  /* workspace_bytes < sdpa_workspace_bytes(...) */
#define SDPA_HIP_ERROR 4            /* the kernel launch reported a HIP error */

/* Element types of q, k, v and out (all four share one). */
#define SDPA_FP16 0
#define SDPA_BF16 1

/*
 * Enqueue out = softmax(scale * q k^T + mask) v on `stream` and return
 * without waiting for it.
 *
 *   q, k, v   device pointers, layouts above, element type `dtype`; read only.
 *   out       device pointer, [B, Hq, qL, D]; written.  Must not overlap q/k/v.
 *   B, Hq, Hkv, qL, kL  sizes, all >= 1; Hq must be a multiple of Hkv.
 *   D         head dimension: 64, 80, 128, 192, 256 or 512 (else SDPA_UNSUPPORTED).
 *   scale     finite fp32 factor > 0 applied to q.k (1/sqrt(D) is the usual one).
 *   causal    0 or 1.
 *   window    0 (none) or >= 1; a window requires causal = 1.
 *   q_offset  absolute position of query row 0.  Ignored unless causal; with
 *             causal it must satisfy 0 <= q_offset <= kL - qL, so that every
 *             row sees at least one key.
 *   dtype     SDPA_FP16 or SDPA_BF16.
 *   workspace device scratch owned by the caller, at least
 *             sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D) bytes (may be NULL
 *             when that is 0).  Its contents on entry do not matter.
 *   stream    a hipStream_t, or NULL for the default stream.
 *
 * Arithmetic: fp16/bf16 products with fp32 accumulation; softmax state and
 * the output accumulator in fp32; the output rounded to `dtype` (nearest
 * even).  Every buffer must stay valid until the stream has passed this
 * call.  All arguments are checked on the host before anything is
 * enqueued; on a non-zero status nothing has been enqueued except for
 * SDPA_HIP_ERROR.
 */
int sdpa_forward(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                 int qL, int kL, int D, float scale, int causal, int window, int q_offset,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace sdpa_forward needs for this shape: a pure
 * function of its arguments (no device query), 0 when the call runs without
 * a key split.  It grows with B * Hq * qL * (kL / chunk) * D, never with
 * qL * kL.  Returns (size_t)-1 for sizes sdpa_forward would reject as
 * SDPA_INVALID_ARG or SDPA_UNSUPPORTED.
 */
size_t sdpa_workspace_bytes(int B, int Hq, int Hkv, int qL, int kL, int D);

/*
 * sdpa_forward over keys and values held in a KV cache: the decode and verify
 * calls of mlxcel issue #2160 run over such caches, including sliding-window
 * layers kept as a ring buffer with a cursor (Current Behavior, the 12B and
 * 31B geometries; Proposed Solution step 2) and "strided, sliced keys" (the
 * #1935 divergence class named under Current Behavior, 31B).
 *
 *   k, v         device pointers to caches [B, Hkv, kv_capacity, D] (row
 *                major, contiguous); read only.
 *   kL           live keys, 1 <= kL <= kv_capacity.
 *   kv_capacity  rows per head in the caches.
 *   ring_start   physical row of logical key 0, 0 <= ring_start < kv_capacity:
 *                logical key j is row (ring_start + j) % kv_capacity of its
 *                head.  0 for a cache filled from row 0; the ring's oldest
 *                row for a wrapped ring.  Rows outside the kL live keys are
 *                never read (they may hold anything, NaN included).
 *   Everything else, including positions, masks and q_offset, is as in
 *   sdpa_forward with key j meaning logical key j.
 *
 * The keys are accumulated in logical order, so a row's result depends on
 * the live keys' values in logical order and not on where in the cache they
 * sit.  With qL <= 4 the key chunks are sized from (B, Hkv, kv_capacity)
 * alone, so every call over one cache -- a verify block and the single-row
 * calls over each row's trimmed prefix -- uses the same chunk boundaries and
 * gives each row the same bytes.  The workspace is
 * sdpa_workspace_bytes_kv_view(...).  Status codes as sdpa_forward, plus
 * SDPA_INVALID_ARG for kv_capacity < kL or ring_start out of range.
 */
int sdpa_forward_kv_view(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                         int Hkv, int qL, int kL, int kv_capacity, int ring_start, int D,
                         float scale, int causal, int window, int q_offset, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of sdpa_forward_kv_view; (size_t)-1 for arguments it rejects. */
size_t sdpa_workspace_bytes_kv_view(int B, int Hq, int Hkv, int qL, int kL, int kv_capacity,
                                    int D);

/*
 * sdpa_forward with an additive mask array ("bias") added to the scaled
 * scores: s = scale * q.k + bias[b, hq, i, j], then the causal / window rules
 * and softmax as in sdpa_forward.  This is the array mask that lablup/mlxcel
 * issue #672 hands to SDPA and that cuDNN takes as a bias ("Root cause"),
 * and that CUDA's fused decode kernel rejects (mlxcel issue #2160, Current
 * Behavior, 12B).
 *
 *   bias     device pointer, element type `dtype`; row (b, hq, i) starts at
 *            element b * bias_stride_b + hq * bias_stride_h + i *
 *            bias_stride_q and holds kL contiguous keys.  A zero stride
 *            broadcasts that dimension.  Read only; must not overlap out.
 *            One batch's rows must lie within 2^30 elements
 *            (SDPA_UNSUPPORTED otherwise).  Entries are finite or -inf.
 *            No byte outside the rows the strides name is read, so the
 *            bias may end anywhere, a page boundary included.
 *   A key whose biased score is -inf is excluded like a masked key; a row
 *   with no finite biased score comes out as zeros.
 *   The workspace is sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D), and qL <= 4
 *   keeps the bit-exactness of sdpa_forward (1024-key chunks).
 */
int sdpa_forward_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      void* out, int B, int Hq, int Hkv, int qL, int kL, int D, float scale,
                      int causal, int window, int q_offset, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * sdpa_forward with a value head dim Dv that may differ from the query/key
 * head dim D: q and k are [B, Hq, qL, D] and [B, Hkv, kL, D], v is
 * [B, Hkv, kL, Dv] and out [B, Hq, qL, Dv].  Scores take the D-long dot
 * products; the output is the weighted sum of the Dv-long value rows.  The
 * pairs supported are D == Dv (any head dim sdpa_forward takes; the call is
 * then sdpa_forward) and D = 192 with Dv = 256, the Q=192/K=192/V=256 heads
 * that the review discussion of ml-explore/mlx PR #3293 says its
 * query_head_dim == value_head_dim gate keeps off the fused path.  Other
 * pairs: SDPA_UNSUPPORTED.  Everything else, qL <= 4 bit-exactness included,
 * is as in sdpa_forward; the workspace is sdpa_workspace_bytes_dv(...).
 */
int sdpa_forward_dv(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                    int qL, int kL, int D, int Dv, float scale, int causal, int window,
                    int q_offset, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of sdpa_forward_dv; (size_t)-1 for arguments it rejects. */
size_t sdpa_workspace_bytes_dv(int B, int Hq, int Hkv, int qL, int kL, int D, int Dv);

/*
 * sdpa_forward_kv_view over 4-bit K and V: the prefix KV cache that
 * ml-explore/mlx PR #3660 keeps 4-bit quantized at rest (End-to-end
 * section), read by decode / verify steps and by chunked prefill over that
 * prefix.  The pages give no format; the affine, group-64 form that
 * lablup/mlxcel issue #2160 names for its checkpoints is taken:
 *
 *   kq, vq   device pointers, [B, Hkv, kv_capacity, D / 8] 32-bit words.
 *            Element 8 w + n of a key or value row is the 4-bit code in bits
 *            4 n .. 4 n + 3 of word w of the row.
 *   ks, kb,  device pointers, [B, Hkv, kv_capacity, D / 64], element type
 *   vs, vb   `dtype`: the scale and the bias of each group of 64
 *            consecutive elements of a row.  Element d of a row is
 *            scale[d / 64] * code_d + bias[d / 64].
 *   kL, kv_capacity, ring_start   as in sdpa_forward_kv_view: kL live keys,
 *            logical key j in row (ring_start + j) % kv_capacity of its head.
 *   q, out   as in sdpa_forward.  None of the inputs may overlap out.
 *
 * The kernels stage the dequantized rows, Q and the softmax weights in fp16
 * whatever `dtype` is (fp16 keeps 11 significant bits to bf16's 8), and round
 * only the output to `dtype`.  A key element enters as scale * (code - 8),
 * exact in fp16 for a bf16 scale, and each key row's group constants bias +
 * 8 scale are applied to the query's group sums at near fp32 precision; a
 * value element is scale * code + bias rounded once to fp16.  Values, scales,
 * biases and Q must lie inside fp16's range.  Everything else is
 * sdpa_forward_kv_view's: masks, GQA, decode chunks sized from (B, Hkv,
 * kv_capacity) at absolute positions, and each verify row's bytes equal to
 * those of the single-row call over the same cache with its own trimmed
 * key count (qL <= 4).  D must be 256 and kv_capacity at most 33554432 rows
 * (2^25: one head's code words within 4 GiB), SDPA_UNSUPPORTED otherwise; the
 * workspace is sdpa_workspace_bytes_kv_view(B, Hq, Hkv, qL, kL,
 * kv_capacity, D).
 */
int sdpa_forward_q4kv(const void* q, const void* kq, const void* ks, const void* kb, const void* vq,
                      const void* vs, const void* vb, void* out, int B, int Hq, int Hkv, int qL, int kL,
                      int kv_capacity, int ring_start, int D, float scale, int causal, int window,
                      int q_offset, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and bytes out, without the workspace
 * arguments.  The key-split partials that sdpa_forward keeps in the caller's
 * workspace live instead in a scratch array of SDPA_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on, from the first call on that
 * GPU until the process ends (that first call also looks up the array's
 * device address).  No call allocates or frees anything.
 *
 * Calls whose sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D) exceeds
 * SDPA_NOALLOC_SCRATCH_BYTES return SDPA_WORKSPACE_TOO_SMALL before anything
 * is enqueued; other status codes as sdpa_forward.  Every call on one GPU
 * shares that GPU's array, and it keeps what the last call left there (a
 * call needs nothing cleared: it writes every partial it reads).  Calls that
 * may overlap on one GPU -- on different streams, or from several host
 * threads without ordering -- race on the array and must be serialised by
 * the caller; calls on one stream are ordered by it.
 */
#define SDPA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int sdpa_forward_noalloc(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                         int qL, int kL, int D, float scale, int causal, int window, int q_offset,
                         int dtype, void* stream);

/*
 * Message for the last non-zero status returned on the calling thread ("" if
 * none).  Failures are reported, never raised: the error-handling note of
 * lablup/mlxcel issue #2160 (Implementation Notes) asks that a failed check
 * fall back cleanly with its reason reported and without introducing any
 * crash, and this string is that reason.  The pointer stays valid until the thread's
 * next call into the library; the caller must not free it.
 */
const char* sdpa_last_error(void);

/*
 * Library version, major * 10000 + minor * 100 + patch.  A caller that
 * declines to use the library (the fail-closed path of the same
 * Implementation Notes) can compare it against the version it was built
 * for; it never fails.
 */
int sdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
