// C ABI of the attention library: argument checks, split planning, launch.
// The interface and its contract are documented in include/sdpa_mi355x.h.
#include "sdpa_mi355x.h"

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "sdpa_internal.h"

#define SDPA_API extern "C" __attribute__((visibility("default")))

namespace sdpa {

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks shared by every entry point and workspace query.  D is the
// head dim of q and k, Dv that of v and out: equal, one of 128, 192, 256 or
// 512, or the pair D = 192, Dv = 256.
int check_shape(int B, int Hq, int Hkv, int qL, int kL, int D, int Dv) {
  if (B < 1 || Hq < 1 || Hkv < 1 || qL < 1 || kL < 1)
    return fail(SDPA_INVALID_ARG, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d qL=%d kL=%d)", B, Hq,
                Hkv, qL, kL);
  if (Hq % Hkv != 0)
    return fail(SDPA_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (D != Dv && !(D == 192 && Dv == 256))
    return fail(SDPA_UNSUPPORTED, "head dims q/k %d with v %d are not supported (equal, or 192 with 256)", D, Dv);
  if (D != 64 && D != 80 && D != 128 && D != 192 && D != 256 && D != 512)
    return fail(SDPA_UNSUPPORTED, "head_dim %d is not supported (64, 80, 128, 192, 256 or 512)", D);
  // index arithmetic inside the kernels: packed rows per KV head and the
  // launch grid stay in 32-bit range; byte offsets are 64-bit
  const int64_t rows = (int64_t)(Hq / Hkv) * qL;
  const int64_t flat_rows = (int64_t)B * Hq * qL;
  if (rows > INT32_MAX / 2 || flat_rows > INT32_MAX / 2 ||
      (int64_t)B * Hkv * ceil_div(rows, block_rows(D)) > INT32_MAX / 2)
    return fail(SDPA_INVALID_ARG, "problem too large for one call");
  if ((int64_t)B * Hq * qL * Dv > INT64_MAX / 4 || (int64_t)B * Hkv * kL * Dv > INT64_MAX / 4)
    return fail(SDPA_INVALID_ARG, "element count overflows");
  return SDPA_OK;
}

size_t workspace_for(const SplitPlan& sp, int B, int Hq, int qL, int D) {
  if (!sp.partials) return 0;
  const size_t prow = (size_t)B * Hq * qL * (size_t)sp.nsplit;
  return prow * (size_t)D * sizeof(float) + prow * 2 * sizeof(float);
}

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

}  // namespace

SplitPlan plan_split(int B, int Hq, int Hkv, int qL, int kL, int D, int kv_capacity) {
  SplitPlan sp;
  if (qL <= kDecodeMaxRows) {
    // decode / verify: always the split path, with chunks at absolute key
    // positions.  A verify row must get the same chunks, and so the same
    // bits, as the single-row call over its own trimmed key prefix, whose kL
    // is smaller: the chunk may depend on neither qL nor kL.  Without a
    // cache capacity it is kDecodeChunk.  With one it is kDecodeChunk times
    // a power of two, the largest for which the (b, KV head) x chunk
    // workgroups of a full cache still fill one round of the CUs: a pure
    // function of (B, Hkv, capacity), which every call over that cache shares.
    int64_t chunk = kDecodeChunk;
    if (kv_capacity > 0) {
      const int64_t heads = (int64_t)B * Hkv;
      while (heads * ceil_div(kv_capacity, 2 * chunk) >= kPlannedCUs && 2 * chunk <= (int64_t)INT32_MAX / 2)
        chunk *= 2;
    }
    sp.split_len = (int)chunk;
    sp.nsplit = (int)ceil_div(kL, chunk);
    sp.partials = 1;
    (void)D;
    return sp;
  }
  // prefill: split the keys only when the row blocks alone cannot fill the
  // chip (one workgroup per CU at a time).  Among the split counts from the
  // smallest that fills one round upward, take the first whose last round
  // of workgroups is at least 90% full (else the fullest): fewer splits mean
  // less partial traffic for the combine.
  const int64_t rows = (int64_t)(Hq / Hkv) * qL;
  const int64_t wgs = (int64_t)B * Hkv * ceil_div(rows, block_rows(D));
  const int64_t cus = kPlannedCUs;
  const int64_t min_split_keys = 2048;
  sp.nsplit = 1;
  sp.split_len = (int)(ceil_div(kL, 1024) * 1024);
  sp.partials = 0;
  if (wgs < cus && kL >= 2 * min_split_keys) {
    const int64_t nmax = kL / min_split_keys;
    const int64_t nmin = ceil_div(cus, wgs);
    int64_t n = nmin;
    double best = 0.0;
    for (int64_t c = nmin; c <= 4 * nmin && c <= nmax; ++c) {
      const double fill = (double)(wgs * c) / (double)(ceil_div(wgs * c, cus) * cus);
      if (fill > best + 1e-9) {
        best = fill;
        n = c;
      }
      if (fill >= 0.9) break;
    }
    if (n > nmax) n = nmax;
    if (n > 1) {
      const int64_t len = ceil_div(ceil_div(kL, n), 1024) * 1024;
      sp.split_len = (int)len;
      sp.nsplit = (int)ceil_div(kL, len);
      sp.partials = sp.nsplit > 1;
    }
  }
  return sp;
}

}  // namespace sdpa

namespace sdpa {
namespace {

// KV-cache view checks (sdpa_forward_kv_view and its workspace query).
int check_view(int kL, int kv_capacity, int ring_start) {
  if (kv_capacity < kL)
    return fail(SDPA_INVALID_ARG, "kv_capacity (%d) must be >= kL (%d)", kv_capacity, kL);
  if (ring_start < 0 || ring_start >= kv_capacity)
    return fail(SDPA_INVALID_ARG, "ring_start must lie in [0, kv_capacity) = [0, %d) (got %d)",
                kv_capacity, ring_start);
  return SDPA_OK;
}

// Both forward entry points: K/V rows of a head are kv_cap apart, logical
// key j is physical row (ring_start + j) % kv_cap; chunk_cap is the cache
// capacity the decode chunks are sized from (0: none).
// 4-bit K/V of sdpa_forward_q4kv (k and v then point at the code words)
struct Q4Args {
  const void *ks, *kb, *vs, *vb;
};

int forward_impl(const void* q, const void* k, const void* v, const void* bias, int64_t bias_sb,
                 int64_t bias_sh, int64_t bias_sq, void* out, int B, int Hq, int Hkv, int qL, int kL,
                 int kv_cap, int ring_start, int chunk_cap, int D, int Dv, float scale, int causal,
                 int window, int q_offset, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream, const Q4Args* q4 = nullptr, bool launch = true) {
  if (!q || !k || !v || !out) return fail(SDPA_INVALID_ARG, "q, k, v and out must be non-null");
  int rc = check_shape(B, Hq, Hkv, qL, kv_cap, D, Dv);
  if (rc != SDPA_OK) return rc;
  if (dtype != SDPA_FP16 && dtype != SDPA_BF16)
    return fail(SDPA_UNSUPPORTED, "dtype %d is not supported (0 = fp16, 1 = bf16)", dtype);
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(SDPA_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1) return fail(SDPA_INVALID_ARG, "causal must be 0 or 1");
  if (window < 0) return fail(SDPA_INVALID_ARG, "window must be >= 0 (got %d)", window);
  if (window > 0 && !causal) return fail(SDPA_INVALID_ARG, "a sliding window requires causal=1");
  if (causal && (q_offset < 0 || q_offset > kL - qL))
    return fail(SDPA_INVALID_ARG,
                "causal q_offset must lie in [0, kL - qL] = [0, %d] so every row sees a key "
                "(got %d)",
                kL - qL, q_offset);
  const size_t qbytes = (size_t)B * Hq * qL * D * 2, obytes = (size_t)B * Hq * qL * Dv * 2;
  // 4-bit rows: D / 2 bytes of codes, and D / 64 scales and biases
  const size_t kbytes = (size_t)B * Hkv * kv_cap * (q4 ? D / 2 : D * 2);
  const size_t vbytes = (size_t)B * Hkv * kv_cap * (q4 ? Dv / 2 : Dv * 2);
  if (overlap(out, obytes, q, qbytes) || overlap(out, obytes, k, kbytes) ||
      overlap(out, obytes, v, vbytes))
    return fail(SDPA_INVALID_ARG, "out must not overlap q, k or v");
  if (q4) {
    const size_t gbytes = (size_t)B * Hkv * kv_cap * (D / 64) * 2;
    if (overlap(out, obytes, q4->ks, gbytes) || overlap(out, obytes, q4->kb, gbytes) ||
        overlap(out, obytes, q4->vs, gbytes) || overlap(out, obytes, q4->vb, gbytes))
      return fail(SDPA_INVALID_ARG, "out must not overlap the scales or biases");
  }

  const SplitPlan sp = plan_split(B, Hq, Hkv, qL, kL, D, chunk_cap);
  const size_t need = workspace_for(sp, B, Hq, qL, Dv);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SDPA_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (sp.nsplit > 65535) return fail(SDPA_INVALID_ARG, "too many key splits (%d)", sp.nsplit);
  if (!launch) return SDPA_OK;  // every check passed; nothing enqueued

  AttnParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = (uint16_t*)out;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.qL = qL;
  p.kL = kL;
  p.kv_cap = kv_cap;
  p.ring_start = ring_start;
  p.bias = (const uint16_t*)bias;
  p.kq4 = q4 ? (const uint32_t*)k : nullptr;
  p.vq4 = q4 ? (const uint32_t*)v : nullptr;
  p.ks4 = q4 ? (const uint16_t*)q4->ks : nullptr;
  p.kb4 = q4 ? (const uint16_t*)q4->kb : nullptr;
  p.vs4 = q4 ? (const uint16_t*)q4->vs : nullptr;
  p.vb4 = q4 ? (const uint16_t*)q4->vb : nullptr;
  p.bias_sb = bias_sb;
  p.bias_sh = bias_sh;
  p.bias_sq = bias_sq;
  p.causal = causal;
  p.window = window;
  p.q_offset = causal ? q_offset : 0;
  p.sl2 = scale * 1.4426950408889634f;
  p.inv_scale = 1.0f / scale;
  p.rows = p.G * qL;
  p.mblocks = (int)ceil_div(p.rows, block_rows(D));
  p.nsplit = sp.nsplit;
  p.split_len = sp.split_len;
  p.partials = sp.partials;
  if (sp.partials) {
    const size_t prow = (size_t)B * Hq * qL * (size_t)sp.nsplit;
    p.part_o = (float*)workspace;
    p.part_ml = (float*)((char*)workspace + prow * (size_t)Dv * sizeof(float));
  } else {
    p.part_o = nullptr;
    p.part_ml = nullptr;
  }
  // the rows of some tile wrap around the end of the cache rows only if the
  // live keys do
  const bool ring = (int64_t)ring_start + kL > kv_cap;
  // sliding-window prefill at head dim 256: a workgroup runs several row
  // blocks of its (batch, KV head) in one pipeline, S workgroups per head
  // (enough to fill the CUs once), workgroup w taking blocks w, w + S, ...
  // more than 8 heads (a multiple of 8) and no key split: each XCD takes
  // whole heads, one at a time (see the kernels' index mapping)
  p.xcd_heads = ((int64_t)B * Hkv > 8 && ((int64_t)B * Hkv) % 8 == 0 && sp.nsplit == 1) ? 1 : 0;
  p.pers_stride = 0;
  if (!q4 && !bias && !ring && D == 256 && Dv == 256 && window > 0 && !sp.partials) {
    const int64_t heads = (int64_t)B * Hkv;
    const int64_t S = ceil_div(kPlannedCUs, heads);
    if (S < p.mblocks) p.pers_stride = (int)S;
  }
  if (p.pers_stride > 0) p.xcd_heads = 0;  // the persistent grid maps its own way

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = !q4                        ? launch_attention(p, D, Dv, dtype, ring, s)
                 : qL <= kDecodeMaxRows      ? launch_attention_q4_decode(p, dtype, s)
                                             : launch_attention_q4(p, dtype, s);
  if (e == hipSuccess && sp.partials) e = launch_combine(p, Dv, dtype, s);
  if (e != hipSuccess) return fail(SDPA_HIP_ERROR, "kernel launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

}  // namespace

int forward_plain(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int qL,
                  int kL, int D, float scale, int causal, int window, int q_offset, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream, bool launch) {
  return forward_impl(q, k, v, nullptr, 0, 0, 0, out, B, Hq, Hkv, qL, kL, kL, 0, 0, D, D, scale, causal, window,
                      q_offset, dtype, workspace, workspace_bytes, stream, nullptr, launch);
}

}  // namespace sdpa

using namespace sdpa;

SDPA_API size_t sdpa_workspace_bytes(int B, int Hq, int Hkv, int qL, int kL, int D) {
  if (check_shape(B, Hq, Hkv, qL, kL, D, D) != SDPA_OK) return (size_t)-1;
  return workspace_for(plan_split(B, Hq, Hkv, qL, kL, D, 0), B, Hq, qL, D);
}

SDPA_API size_t sdpa_workspace_bytes_dv(int B, int Hq, int Hkv, int qL, int kL, int D, int Dv) {
  if (check_shape(B, Hq, Hkv, qL, kL, D, Dv) != SDPA_OK) return (size_t)-1;
  return workspace_for(plan_split(B, Hq, Hkv, qL, kL, D, 0), B, Hq, qL, Dv);
}

SDPA_API size_t sdpa_workspace_bytes_kv_view(int B, int Hq, int Hkv, int qL, int kL,
                                             int kv_capacity, int D) {
  if (check_shape(B, Hq, Hkv, qL, kL, D, D) != SDPA_OK || check_view(kL, kv_capacity, 0) != SDPA_OK ||
      check_shape(B, Hq, Hkv, qL, kv_capacity, D, D) != SDPA_OK)
    return (size_t)-1;
  return workspace_for(plan_split(B, Hq, Hkv, qL, kL, D, kv_capacity), B, Hq, qL, D);
}

SDPA_API const char* sdpa_last_error(void) { return g_last_error; }

SDPA_API int sdpa_version(void) { return 400; }

SDPA_API int sdpa_forward(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                          int Hkv, int qL, int kL, int D, float scale, int causal, int window,
                          int q_offset, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  clear_error();
  return forward_plain(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype, workspace,
                       workspace_bytes, stream, true);
}

SDPA_API int sdpa_forward_dv(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                             int Hkv, int qL, int kL, int D, int Dv, float scale, int causal,
                             int window, int q_offset, int dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  clear_error();
  return forward_impl(q, k, v, nullptr, 0, 0, 0, out, B, Hq, Hkv, qL, kL, kL, 0, 0, D, Dv, scale, causal,
                      window, q_offset, dtype, workspace, workspace_bytes, stream);
}

SDPA_API int sdpa_forward_bias(const void* q, const void* k, const void* v, const void* bias,
                               long long bias_stride_b, long long bias_stride_h,
                               long long bias_stride_q, void* out, int B, int Hq, int Hkv, int qL,
                               int kL, int D, float scale, int causal, int window, int q_offset,
                               int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int rc = check_shape(B, Hq, Hkv, qL, kL, D, D);
  if (rc != SDPA_OK) return rc;
  if (!bias) return fail(SDPA_INVALID_ARG, "bias must be non-null");
  if (bias_stride_b < 0 || bias_stride_h < 0 || bias_stride_q < 0)
    return fail(SDPA_INVALID_ARG, "bias strides must be >= 0");
  // the kernels address one batch's bias rows with 32-bit byte offsets
  const int64_t extent = (int64_t)(Hq - 1) * bias_stride_h + (int64_t)(qL - 1) * bias_stride_q + kL;
  if (bias_stride_h > (int64_t)1 << 30 || bias_stride_q > (int64_t)1 << 30 || extent > ((int64_t)1 << 30))
    return fail(SDPA_UNSUPPORTED, "one batch of the bias spans %lld elements (at most 2^30)", (long long)extent);
  const size_t qbytes = (size_t)B * Hq * qL * D * 2;
  const size_t bbytes = (size_t)(((int64_t)(B - 1) * bias_stride_b + extent) * 2);
  if (overlap(out, qbytes, bias, bbytes)) return fail(SDPA_INVALID_ARG, "out must not overlap the bias");
  return forward_impl(q, k, v, bias, bias_stride_b, bias_stride_h, bias_stride_q, out, B, Hq, Hkv, qL, kL,
                      kL, 0, 0, D, D, scale, causal, window, q_offset, dtype, workspace, workspace_bytes, stream);
}

SDPA_API int sdpa_forward_kv_view(const void* q, const void* k, const void* v, void* out, int B,
                                  int Hq, int Hkv, int qL, int kL, int kv_capacity, int ring_start,
                                  int D, float scale, int causal, int window, int q_offset,
                                  int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  clear_error();
  int rc = check_shape(B, Hq, Hkv, qL, kL, D, D);
  if (rc != SDPA_OK) return rc;
  rc = check_view(kL, kv_capacity, ring_start);
  if (rc != SDPA_OK) return rc;
  return forward_impl(q, k, v, nullptr, 0, 0, 0, out, B, Hq, Hkv, qL, kL, kv_capacity, ring_start,
                      kv_capacity, D, D, scale, causal, window, q_offset, dtype, workspace, workspace_bytes,
                      stream);
}

SDPA_API int sdpa_forward_q4kv(const void* q, const void* kq, const void* ks, const void* kb,
                               const void* vq, const void* vs, const void* vb, void* out, int B,
                               int Hq, int Hkv, int qL, int kL, int kv_capacity, int ring_start, int D,
                               float scale, int causal, int window, int q_offset, int dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int rc = check_shape(B, Hq, Hkv, qL, kL, D, D);
  if (rc != SDPA_OK) return rc;
  rc = check_view(kL, kv_capacity, ring_start);
  if (rc != SDPA_OK) return rc;
  if (D != 256) return fail(SDPA_UNSUPPORTED, "4-bit K/V: head dim %d is not supported (256 only)", D);
  // the kernel addresses a head's rows by 32-bit byte offsets from its first row
  if ((uint64_t)kv_capacity * (uint64_t)(D / 2) > (1ull << 32))
    return fail(SDPA_UNSUPPORTED, "4-bit K/V: kv_capacity %d exceeds %d rows (a head's code words must fit in 4 GiB)",
                kv_capacity, (int)((1ull << 32) / (uint64_t)(D / 2)));
  if (!ks || !kb || !vs || !vb) return fail(SDPA_INVALID_ARG, "scales and biases must be non-null");
  const Q4Args q4{ks, kb, vs, vb};
  return forward_impl(q, kq, vq, nullptr, 0, 0, 0, out, B, Hq, Hkv, qL, kL, kv_capacity, ring_start, kv_capacity,
                      D, D, scale, causal, window, q_offset, dtype, workspace, workspace_bytes, stream, &q4);
}
