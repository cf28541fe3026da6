// Internal declarations shared by the host dispatch and the kernel launchers.
// Not part of the public interface (that is include/sdpa_mi355x.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdpa {

// One workgroup of the attention kernel is 4 waves; a wave owns 32 query rows
// and D / d_split(D) of the head dimension.  At D = 512 two waves share each
// 32-row block (one per half of D), so a workgroup holds 64 rows.
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int d_split(int D) { return D == 512 ? 2 : 1; }
constexpr int block_rows(int D) { return kWaves / d_split(D) * kRowsPerWave; }

// Keys per LDS tile, by head dimension.
constexpr int tile_keys(int D) { return D == 512 ? 32 : 64; }

// Elements per K / V row in LDS: the head dims rounded up to 128, 256 or 512
// (a 192-wide row takes a 256-wide slot).
constexpr int lds_row(int dk, int dv) {
  return (dk > dv ? dk : dv) <= 128 ? 128 : (dk > dv ? dk : dv) <= 256 ? 256 : 512;
}

// Key chunk of the split path used by every call with qL <= kDecodeMaxRows
// when no KV-cache capacity is given.  With a capacity the chunk is this
// times a power of two chosen from (B, Hkv, capacity).  Either way chunk
// boundaries sit at absolute key positions and depend neither on qL nor on
// the number of live keys, so a row gets the same chunks, and the same bits,
// in a verify block and in a single-row call over its own key prefix.
constexpr int kDecodeChunk = 1024;
constexpr int kDecodeMaxRows = 4;

// Number of compute units the launch shapes are planned for (MI355X).
constexpr int kPlannedCUs = 256;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;      // direct output (nsplit == 1 and !partials)
  float* part_o;      // [rows_total, nsplit, Dv] unnormalised fp32 accumulators
  float* part_ml;     // [rows_total, nsplit, 2]: running max (log2 units), sum
  int B, Hq, Hkv, G, qL, kL;
  const uint16_t* bias;  // additive mask array or nullptr; keys contiguous within a row
  int64_t bias_sb, bias_sh, bias_sq;  // its batch, query-head and query-row strides (elements)
  // 4-bit K and V (the q4 instances; k and v are unused then): code words
  // [B, Hkv, kL, D / 8] (element 8 w + n in bits 4 n .. 4 n + 3 of word w),
  // per-64-element-group scales and biases [B, Hkv, kL, D / 64] in the dtype;
  // element d of a row is scale * code + bias
  const uint32_t* kq4;
  const uint16_t *ks4, *kb4;
  const uint32_t* vq4;
  const uint16_t *vs4, *vb4;
  int kv_cap;         // rows per KV head in k and v (head strides kv_cap * D, kv_cap * Dv), >= kL
  int ring_start;     // physical row of logical key 0; key j is row (ring_start + j) % kv_cap
  int causal, window, q_offset;
  float sl2;          // scale * log2(e)
  float inv_scale;    // 1 / scale: the kernels keep raw q.k scores, so a bias enters as bias / scale
  int rows;           // G * qL packed rows per (b, kv head)
  int mblocks;        // ceil(rows / block_rows(D))
  int nsplit;         // key splits
  int split_len;      // keys per split, a multiple of the tile width
  int partials;       // 1: write partials for the combine pass
  int pers_stride;    // > 0: S workgroups per (b, kv head), workgroup w running row
                      // blocks w, w + S, ... in one pipeline (head dim 256 only)
  int xcd_heads;      // 1: workgroup index -> (head, row block) so that each XCD runs
                      // whole heads one at a time (B * Hkv a multiple of 8, one split)
};

// Split plan for a shape: how many key splits, how long each, and whether
// the partial/combine path is used.  Pure function of the shape and of the
// KV-cache capacity (0: none given).
struct SplitPlan {
  int nsplit;
  int split_len;
  int partials;
};
SplitPlan plan_split(int B, int Hq, int Hkv, int qL, int kL, int D, int kv_capacity);

// D: head dim of q and k; Dv: of v and out (D, or 256 with D = 192).
// ring: some tile's keys wrap around the end of the cache rows; p.bias set:
// the instances that add the mask array (never together with ring, and
// neither with D != Dv)
hipError_t launch_attention(const AttnParams& p, int D, int Dv, int dtype, bool ring, hipStream_t stream);
// The 4-bit K/V instance (D = Dv = 256, no ring, no bias; p.kq4 ... set)
hipError_t launch_attention_q4(const AttnParams& p, int dtype, hipStream_t stream);
// The 4-bit decode/verify kernel (qL <= kDecodeMaxRows, D = Dv = 256, key
// splits with partials; p.kq4 ... set)
hipError_t launch_attention_q4_decode(const AttnParams& p, int dtype, hipStream_t stream);
hipError_t launch_combine(const AttnParams& p, int Dv, int dtype, hipStream_t stream);

// The calling thread's message for the last failed call: fail() formats it
// and returns `status`; clear_error() empties it.
int fail(int status, const char* fmt, ...);
void clear_error();

// sdpa_forward's argument checks and, when `launch` is set, its launches with
// the workspace given here.  With launch false it only checks (no HIP call).
int forward_plain(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int qL,
                  int kL, int D, float scale, int causal, int window, int q_offset, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream, bool launch);

}  // namespace sdpa
