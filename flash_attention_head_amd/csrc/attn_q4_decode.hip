// Decode and verify steps (at most kDecodeMaxRows query positions) over a
// 4-bit K/V cache, head dim 256, for gfx950 (MI355X).
//
// The cache rows are the 4-bit form in which ml-explore/mlx PR #3660 keeps
// its prefix KV cache at rest (End-to-end section): per key row, 32 code
// words of 8 codes (element 8 w + n in bits 4 n .. 4 n + 3 of word w) and
// one scale and one bias per 64-element group; element d is scale * code +
// bias.
//
// A workgroup takes one (batch, KV head, key chunk) and up to 16 packed
// query rows (row r: query position r / G of query head hk G + r % G).  The
// chunk's keys go in 32-key sub-tiles to the eight waves (two per SIMD) in
// turn, and each wave runs its own online softmax over its sub-tiles with
// 16x16x32 MFMAs:
//   S^T = K Q^T   A = the key codes, turned into fp16 operands in registers
//                 straight from the loaded words; B = Q, held in registers
//   O^T += V^T P^T  A = V^T, staged through the wave's own LDS buffer and read
//                 back transposed; B = the weights, straight from S's registers
// The waves never wait for each other until the end, where their eight
// (max, sum, output) states are merged in wave order into the chunk's
// partial for the combine pass.  Nothing a row computes depends on the other
// rows of the call, so a verify row gets the same bits as the single-row
// call over its own key prefix.
//
// From a code word to fp16 operands: OR-ing a code into the low mantissa
// bits of 1024.0 (0x6400) gives 1024 + code exactly, so with w's even
// nibbles masked in place (bits 0..3 and 16..19) one v_and_or forms two
// elements, and the odd nibbles (bits 4..7, 20..23) give 1024 + 16 code.
// Keys then take the centred value scale * (code - 8): exact in fp16 for a
// bf16 scale (8 significant bits times an integer of at most 3 bits), its
// odd nibbles 16 times that (the Q entries they meet are divided by 16,
// exactly).  Each key row's group constant bias + 8 scale reaches the scores
// through one more MFMA against the query's group sums, both split into
// fp16 high and low parts.  Values take fma(code, scale, bias) rounded once
// to fp16 (16 times that for the odd nibbles: the output columns they feed
// are divided by 16 at the end, exactly).
#include "sdpa_internal.h"

#include <math.h>

namespace sdpa {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

constexpr int kD = 256;                  // head dim
constexpr int kNW = 8;                   // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kNW;
constexpr int kSub = 32;                 // keys per sub-tile
constexpr int kVBuf = kSub * kD;         // one staged V sub-tile, fp16 elements
constexpr int kVBufs = kNW == 4 ? 2 : 1;  // staged V buffers per wave (LDS: 128 KiB in all)
constexpr int kOStride = kVBufs == 2 ? kD + 4 : kD;  // merge area row stride, floats (fits the wave's LDS)
constexpr int kMergeWords = 512 / kThreads;          // code words' columns per thread in the merge
constexpr float kRescaleLog2 = 8.f;      // lazy reference max, as in the 16-bit kernels
constexpr uint32_t kMagic = 0x64006400u;  // 1024.0 in both fp16 halves

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ f16x2_t h2(uint32_t x) { return __builtin_bit_cast(f16x2_t, x); }
__device__ __forceinline__ uint32_t u32(f16x2_t x) { return __builtin_bit_cast(uint32_t, x); }

// a 16-bit float of the input type, widened
template <int DT>
__device__ __forceinline__ float widen(uint32_t h) {
  if constexpr (DT == 1) return __builtin_bit_cast(float, (h & 0xffffu) << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}
// the same value as fp16 (exact for fp16 input; bf16 rounded to nearest even,
// exact inside fp16's range for the 8 significant bits of a bf16)
template <int DT>
__device__ __forceinline__ _Float16 to_half(uint32_t h) {
  if constexpr (DT == 1) return (_Float16)widen<1>(h);
  else return __builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}
__device__ __forceinline__ uint32_t pair(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// Values of lanes l and l ^ 16 (v_permlane16_swap) and of lanes l and l ^ 32
// (v_permlane32_swap): element 0 is the lower lane's, element 1 the upper's,
// in both lanes, so a + b has the same bits in both.
__device__ __forceinline__ float max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
__device__ __forceinline__ float sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
// the upper half's value (lanes 32..63) in the lower half
__device__ __forceinline__ float upper32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)r[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group, source
// lane a + 4 t (a, t in 0..3) names 4 consecutive 16-bit elements of row t of
// a 4-row block, and result lane j of the group receives column j of the
// block's four rows.
__device__ __forceinline__ uint2 read_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)p));
}

// (x & m) | c in one v_and_or_b32 (gfx9 VOP3 takes no literal, so the
// compiler splits the expression into two instructions with literals; here
// the mask sits in a scalar register and the constant in a vector register)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// MFMA operand of key code word w: entries (n0, n4), (n1, n5), (n2, n6),
// (n3, n7) of s (c_n - 8), the odd nibbles' pairs times 16.  s2: the scale
// in both halves.
__device__ __forceinline__ uint4 key_operand(uint32_t w, f16x2_t s2, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const f16x2_t lo = {(_Float16)-1032.f, (_Float16)-1032.f}, hi = {(_Float16)-1152.f, (_Float16)-1152.f};
  uint4 r;
  r.x = u32((h2(and_or(w, 0x000F000Fu, magic)) + lo) * s2);
  r.y = u32((h2(and_or(w, 0x00F000F0u, magic)) + hi) * s2);
  r.z = u32((h2(and_or(w8, 0x000F000Fu, magic)) + lo) * s2);
  r.w = u32((h2(and_or(w8, 0x00F000F0u, magic)) + hi) * s2);
  return r;
}
// Staged values of code word w, in the same entry order: fma(c, s, b)
// rounded once to fp16, the odd nibbles' pairs 16 times that (fma(16 c, s,
// 16 b)).  b16: 16 b in both halves.
__device__ __forceinline__ uint4 value_row(uint32_t w, f16x2_t s2, f16x2_t b2, f16x2_t b16, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const f16x2_t off = {(_Float16)-1024.f, (_Float16)-1024.f};
  uint4 r;
  r.x = u32(__builtin_elementwise_fma(h2(and_or(w, 0x000F000Fu, magic)) + off, s2, b2));
  r.y = u32(__builtin_elementwise_fma(h2(and_or(w, 0x00F000F0u, magic)) + off, s2, b16));
  r.z = u32(__builtin_elementwise_fma(h2(and_or(w8, 0x000F000Fu, magic)) + off, s2, b2));
  r.w = u32(__builtin_elementwise_fma(h2(and_or(w8, 0x00F000F0u, magic)) + off, s2, b16));
  return r;
}

// What one lane loads for one sub-tile.  Lane (r, q) = (lane % 16, lane /
// 16) takes key row r of each 16-key block b: code words 4 q .. 4 q + 3 and
// 16 + 4 q .. 16 + 4 q + 3 of K and of V (64-byte runs per four lanes), and
// the row's four scales and four biases of K and of V.
struct Loads {
  uint4 kw[2][2], vw[2][2];
  uint2 ks[2], kb[2], vs[2], vb[2];
};

template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kNW / 4, kNW / 4)))
void attn_q4_decode_kernel(AttnParams p) {
  // per wave its staged V sub-tile(s) (16 KiB each; at the end its merge
  // area), then the waves' (max, sum) per row
  __shared__ __attribute__((aligned(16))) uint16_t lds[kNW * kVBufs * kVBuf];
  __shared__ float ml_lds[kNW][16][2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r16 = lane & 15, lq = lane >> 4;
  // 0x64006400 in a vector register for v_and_or_b32 (the empty asm keeps
  // the compiler from folding it back into a literal)
  uint32_t magic = kMagic;
  asm volatile("" : "+v"(magic));

  const int nheads = p.B * p.Hkv;
  const int head = (int)(blockIdx.x % nheads), pass = (int)(blockIdx.x / nheads);
  const int split = blockIdx.y;
  const int b = head / p.Hkv, hkv = head % p.Hkv;

  // this workgroup's packed rows and the keys they see in this chunk
  const int row0 = pass * 16, rend = min(p.rows, row0 + 16);
  const int pos_first = p.q_offset + row0 / p.G, pos_last = p.q_offset + (rend - 1) / p.G;
  const int c_lo = split * p.split_len, c_hi = min(p.kL, c_lo + p.split_len);
  const int kbeg = max(c_lo, p.window > 0 ? pos_first - p.window + 1 : 0);
  const int kend = min(c_hi, p.causal ? pos_last + 1 : p.kL);
  if (kbeg >= kend) return;  // no row here sees this chunk (the combine skips it)
  // every key of a sub-tile in [vis_lo, vis_hi] is visible to every row
  const int vis_lo = p.window > 0 ? max(0, pos_last - p.window + 1) : 0;
  const int vis_hi = p.causal ? pos_first : p.kL - 1;

  // this lane's query row (the S and O columns it holds)
  const int my = row0 + r16;
  const bool valid = my < rend;
  const int qi = valid ? my / p.G : 0, hq = hkv * p.G + (valid ? my % p.G : 0);
  const int pos = p.q_offset + qi;
  const int key_lo = valid && p.window > 0 ? max(0, pos - p.window + 1) : 0;
  const int key_hi = valid && p.causal ? pos : p.kL - 1;

  // ---- Q: the B operands of the eight d steps -----------------------------
  // Step s takes code word W(s) = 4 q + s (s < 4) or 16 + 4 q + s - 4 of
  // every key row in the lanes of group q, so this lane's B entries of step s
  // are the query elements of that word, in the operand order (n0, n4, n1,
  // n5, n2, n6, n3, n7), the odd nibbles' ones divided by 16.
  uint4 qb[8];
  float qs_a = 0.f, qs_b = 0.f;  // sums of this lane's elements of groups q / 2 and 2 + q / 2
  {
    const uint16_t* qrow = p.q + ((size_t)(b * p.Hq + hq) * p.qL + qi) * kD;
    const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int word = s < 4 ? 4 * lq + s : 16 + 4 * lq + (s - 4);
      uint4 u = valid ? *(const uint4*)(qrow + 8 * word) : make_uint4(0, 0, 0, 0);
      _Float16 e[8];
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[2 * i] = to_half<DT>(uw[i]);
        e[2 * i + 1] = to_half<DT>(uw[i] >> 16);
      }
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a += (float)e[i];
      if (s < 4) qs_a += a;
      else qs_b += a;
      qb[s].x = pair(e[0], e[4]);
      qb[s].y = u32(h2(pair(e[1], e[5])) * sixteenth);
      qb[s].z = pair(e[2], e[6]);
      qb[s].w = u32(h2(pair(e[3], e[7])) * sixteenth);
    }
  }
  // Group-constant MFMA, B side: the query's group sums Q_g (lanes of groups
  // 0 and 1 hold Q_0 and Q_2 after the sum with their partner, groups 2 and 3
  // Q_1 and Q_3), split into fp16 high and low parts.  Lane group 0 holds
  // (Q_0..3 high, Q_0..3 low), group 1 (Q_0..3 high, 0 x 4), groups 2 and 3
  // zeros; against the key rows' (c_0..3 high, c_0..3 high | c_0..3 low, 0 x
  // 4 | 0) the product sums c_g (Q_g high + low) + c_g low Q_g high.
  uint4 qc;
  {
    const float qa = sum16(qs_a), qbs = sum16(qs_b);
    const float g[4] = {qa, upper32(qa), qbs, upper32(qbs)};
    _Float16 hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = (_Float16)g[i];
      lo[i] = (_Float16)(g[i] - (float)hi[i]);
    }
    const uint4 h4 = make_uint4(pair(hi[0], hi[1]), pair(hi[2], hi[3]), pair(lo[0], lo[1]), pair(lo[2], lo[3]));
    qc = lq == 0 ? h4 : lq == 1 ? make_uint4(h4.x, h4.y, 0u, 0u) : make_uint4(0, 0, 0, 0);
  }

  // ---- the wave's sub-tiles of this chunk: every kNW-th from the first -----
  // (sub-tile T to wave T mod kNW; chunks start at multiples of kNW sub-tiles)
  const int t_first = kbeg / kSub, t_last = (kend - 1) / kSub;
  const int tw0 = t_first + ((wave - t_first) % kNW + kNW) % kNW;
  const int nsub = tw0 <= t_last ? (t_last - tw0) / kNW + 1 : 0;
  auto sub_t = [&](int i) { return tw0 + kNW * min(i, nsub - 1); };

  // cache rows of the head; logical key j is row (ring_start + j) % kv_cap.
  // 32-bit byte offsets from the head's first row (the entry point bounds
  // kv_cap so that a head's code words stay below 4 GiB)
  const size_t head_row = (size_t)(b * p.Hkv + hkv) * (size_t)p.kv_cap;
  const char* const kq = (const char*)(p.kq4 + head_row * (kD / 8));
  const char* const vq = (const char*)(p.vq4 + head_row * (kD / 8));
  const char* const ksc = (const char*)(p.ks4 + head_row * (kD / 64));
  const char* const kbi = (const char*)(p.kb4 + head_row * (kD / 64));
  const char* const vsc = (const char*)(p.vs4 + head_row * (kD / 64));
  const char* const vbi = (const char*)(p.vb4 + head_row * (kD / 64));
  auto issue = [&](Loads& ld, int t) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // rows past kL repeat row kL - 1 (finite values; their keys are masked)
      const int key = min(t * kSub + 16 * blk + r16, p.kL - 1);
      int phys = p.ring_start + key;
      phys = phys >= p.kv_cap ? phys - p.kv_cap : phys;
      const uint32_t wo = (uint32_t)phys * (kD / 2) + 16u * (uint32_t)lq;
      const uint32_t go = (uint32_t)phys * (kD / 32);
      ld.kw[blk][0] = *(const uint4*)(kq + wo);
      ld.kw[blk][1] = *(const uint4*)(kq + wo + 64);
      ld.ks[blk] = *(const uint2*)(ksc + go);
      ld.kb[blk] = *(const uint2*)(kbi + go);
      ld.vw[blk][0] = *(const uint4*)(vq + wo);
      ld.vw[blk][1] = *(const uint4*)(vq + wo + 64);
      ld.vs[blk] = *(const uint2*)(vsc + go);
      ld.vb[blk] = *(const uint2*)(vbi + go);
    }
  };

  // staged V: key row k of the sub-tile (16 blk + r) at k * 256; code word W's
  // 8 values in chunk W ^ (k & 15) (16-byte chunks), in the operand entry
  // order.  The XOR spreads the writes (16 rows, 4 words) and the transposed
  // reads (16 rows, 2 chunks) over all 16 four-bank groups.
  uint16_t* const vbuf = lds + wave * kVBufs * kVBuf;
  const int g_a = lq >> 1, g_b = 2 + (lq >> 1);  // the groups of this lane's two runs of words
  auto stage_v = [&](const Loads& ld, uint16_t* vs) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint32_t sw[2] = {ld.vs[blk].x, ld.vs[blk].y}, bw[2] = {ld.vb[blk].x, ld.vb[blk].y};
      f16x2_t s2[2], b2[2], b16[2];
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const int g = run == 0 ? g_a : g_b;
        const _Float16 sv = to_half<DT>(sw[g >> 1] >> (16 * (g & 1)));
        const _Float16 bv = to_half<DT>(bw[g >> 1] >> (16 * (g & 1)));
        s2[run] = (f16x2_t){sv, sv};
        b2[run] = (f16x2_t){bv, bv};
        b16[run] = b2[run] * (f16x2_t){(_Float16)16.f, (_Float16)16.f};
      }
      const int k = 16 * blk + r16;
      uint16_t* rowp = vs + k * kD;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int run = s >> 2;
        const uint4 wv = ld.vw[blk][run];
        const uint32_t w = (s & 3) == 0 ? wv.x : (s & 3) == 1 ? wv.y : (s & 3) == 2 ? wv.z : wv.w;
        const int word = run == 0 ? 4 * lq + (s & 3) : 16 + 4 * lq + (s & 3);
        *(uint4*)(rowp + 8 * (word ^ (k & 15))) = value_row(w, s2[run], b2[run], b16[run], magic);
      }
    }
  };
  // V^T operand of output block db (staged columns 16 db .. 16 db + 15): for
  // lane group q, key rows 4 q .. 4 q + 3 and 16 + 4 q .. 16 + 4 q + 3, the
  // key order of the weights this lane holds
  const int tr_a = r16 & 3, tr_t = r16 >> 2;
  const int tr_row = 4 * lq + tr_t;  // + 16 for the second read (same row & 15)
  auto v_operand = [&](const uint16_t* vs, int db) {
    const int chunk = (2 * db + (tr_a >> 1)) ^ (tr_row & 15);
    const uint16_t* a = vs + tr_row * kD + 8 * chunk + 4 * (tr_a & 1);
    const uint2 x = read_tr(a), y = read_tr(a + 16 * kD);
    return make_uint4(x.x, x.y, y.x, y.y);
  };

  const uint32_t m_g0 = lq == 0 ? ~0u : 0u, m_g1 = lq == 1 ? ~0u : 0u;  // lane group 0, 1

  // ---- online softmax state of this lane's row over the wave's keys -------
  f32x4_t o[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;
  const float sl2 = p.sl2;

  auto compute = [&](const Loads& ld, int t, uint16_t* vs) {
    // scores: S^T blocks of keys 16 blk .. 16 blk + 15, lane (r, q) holding
    // keys 16 blk + 4 q .. + 3 of its row
    f32x4_t s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint32_t sw[2] = {ld.ks[blk].x, ld.ks[blk].y}, bw[2] = {ld.kb[blk].x, ld.kb[blk].y};
      // this key row's group constants bias + 8 scale (exact in fp32), for
      // the group-constant MFMA's A side
      _Float16 ch[4], cl[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float c = widen<DT>(bw[g >> 1] >> (16 * (g & 1))) + 8.f * widen<DT>(sw[g >> 1] >> (16 * (g & 1)));
        ch[g] = (_Float16)c;
        cl[g] = (_Float16)(c - (float)ch[g]);
      }
      // (lane masks rather than a select chain, which the compiler turns
      // into branches)
      const uint32_t h01 = pair(ch[0], ch[1]), h23 = pair(ch[2], ch[3]);
      const uint32_t l01 = pair(cl[0], cl[1]), l23 = pair(cl[2], cl[3]);
      const uint4 kc = make_uint4((h01 & m_g0) | (l01 & m_g1), (h23 & m_g0) | (l23 & m_g1), h01 & m_g0, h23 & m_g0);
      s[blk] = mfma16(kc, qc, (f32x4_t){0.f, 0.f, 0.f, 0.f});
      f16x2_t s2[2];
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const int g = run == 0 ? g_a : g_b;
        const _Float16 sv = to_half<DT>(sw[g >> 1] >> (16 * (g & 1)));
        s2[run] = (f16x2_t){sv, sv};
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const uint4 wv = ld.kw[blk][st >> 2];
        const uint32_t w = (st & 3) == 0 ? wv.x : (st & 3) == 1 ? wv.y : (st & 3) == 2 ? wv.z : wv.w;
        s[blk] = mfma16(key_operand(w, s2[st >> 2], magic), qb[st], s[blk]);
      }
    }
    stage_v(ld, vs);
    // the V^T operands of the first kVA output blocks, read now so that
    // their latency is hidden by the softmax (the same wave wrote them: LDS
    // operations of a wave complete in order); each later one is read kVA
    // MFMAs ahead
    constexpr int kVA = 4;
    uint4 va[kVA];
#pragma unroll
    for (int db = 0; db < kVA; ++db) va[db] = v_operand(vs, db);

    // mask (only sub-tiles some row cannot wholly see)
    const int k0 = t * kSub;
    if (!(k0 >= vis_lo && k0 + kSub - 1 <= vis_hi)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = k0 + 16 * blk + 4 * lq + v;
          s[blk][v] = (key >= key_lo && key <= key_hi) ? s[blk][v] : -INFINITY;
        }
    }
    // row max over the sub-tile -> lazy reference update
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max32(max16(mx));
    const bool upd = mx * sl2 > m_ref * sl2 + kRescaleLog2;
    const float alpha = upd ? ((m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_ref - mx) * sl2)) : 1.f;
    m_ref = upd ? mx : m_ref;
    if (__any(alpha != 1.f)) {  // x * 1 == x: most sub-tiles skip it
#pragma unroll
      for (int db = 0; db < 16; ++db) o[db] *= alpha;
      l_run *= alpha;
    }
    const float msc = (m_ref == -INFINITY) ? 0.f : m_ref * sl2;
    // weights, rounded to fp16 once; the row sum takes the rounded values
    _Float16 w[8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) w[4 * blk + v] = (_Float16)__builtin_amdgcn_exp2f(s[blk][v] * sl2 - msc);
    const uint4 pw = make_uint4(pair(w[0], w[1]), pair(w[2], w[3]), pair(w[4], w[5]), pair(w[6], w[7]));
    const f16x2_t one2 = {(_Float16)1.f, (_Float16)1.f};
    l_run = __builtin_amdgcn_fdot2(h2(pw.x), one2, l_run, false);
    l_run = __builtin_amdgcn_fdot2(h2(pw.y), one2, l_run, false);
    l_run = __builtin_amdgcn_fdot2(h2(pw.z), one2, l_run, false);
    l_run = __builtin_amdgcn_fdot2(h2(pw.w), one2, l_run, false);
    // O^T += V^T P^T: B entries 8 q + j are keys 4 q + j (j < 4) and 16 + 4
    // q + j - 4, the keys of the staged rows v_operand reads
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const uint4 cur = va[db % kVA];
      if (db + kVA < 16) va[db % kVA] = v_operand(vs, db + kVA);
      o[db] = mfma16(cur, pw, o[db]);
    }
  };

  // ---- the wave's sub-tiles, loads one ahead (no branch around a load) ----
  if (nsub > 0) {
    Loads la, lb;
    issue(la, sub_t(0));
    for (int i = 0; i < nsub; i += 2) {
      issue(lb, sub_t(i + 1));
      compute(la, tw0 + kNW * i, vbuf);
      issue(la, sub_t(i + 2));
      if (i + 1 < nsub) compute(lb, tw0 + kNW * (i + 1), vbuf + (kVBufs - 1) * kVBuf);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // ---- merge the waves' states in wave order ------------------------------
  const float lsum = sum32(sum16(l_run));  // the row's four lanes, same bits in each
  float* const om = (float*)vbuf;          // this wave's own LDS: rows of kOStride floats
#pragma unroll
  for (int db = 0; db < 16; ++db) *(f32x4_t*)(om + r16 * kOStride + 16 * db + 4 * lq) = o[db];
  if (lq == 0) {
    ml_lds[wave][r16][0] = m_ref;
    ml_lds[wave][r16][1] = lsum;
  }
  __syncthreads();

  // thread t: row t / (32 / kMergeWords), kMergeWords code words' output
  // columns from word kMergeWords (t % (32 / kMergeWords)) on
  const int mr = tid / (32 / kMergeWords), word0 = kMergeWords * (tid % (32 / kMergeWords));
  const int mrow = row0 + mr;
  if (mrow >= rend) return;
  float m_w[kNW], f[kNW];  // each wave's reference max, and its factor
  float mmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    m_w[w] = ml_lds[w][mr][0];
    mmax = fmaxf(mmax, m_w[w]);
  }
#pragma unroll
  for (int w = 0; w < kNW; ++w)
    f[w] = (m_w[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_w[w] - mmax) * sl2);
  float lt = f[0] * ml_lds[0][mr][1];
#pragma unroll
  for (int w = 1; w < kNW; ++w) lt = fmaf(f[w], ml_lds[w][mr][1], lt);
  const int mqi = mrow / p.G, mhq = hkv * p.G + mrow % p.G;
  const size_t prow = ((size_t)(b * p.Hq + mhq) * p.qL + mqi) * p.nsplit + split;
  float* const dst = p.part_o + prow * kD;
#pragma unroll
  for (int c = 0; c < kMergeWords; ++c) {
    const int word = word0 + c;
    float acc[8];
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float* ow = (const float*)(lds + w * kVBufs * kVBuf) + mr * kOStride + 8 * word;
      const float4 x = *(const float4*)ow, y = *(const float4*)(ow + 4);
      const float e[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = w == 0 ? f[0] * e[j] : fmaf(f[w], e[j], acc[j]);
    }
    // staged entry j holds element (j >> 1) + 4 (j & 1) of the word; the odd
    // nibbles' entries (j = 2, 3, 6, 7) were 16 times the value
    float out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) out[(j >> 1) + 4 * (j & 1)] = ((j >> 1) & 1) ? acc[j] * 0.0625f : acc[j];
    *(float4*)(dst + 8 * word) = make_float4(out[0], out[1], out[2], out[3]);
    *(float4*)(dst + 8 * word + 4) = make_float4(out[4], out[5], out[6], out[7]);
  }
  if (tid % (32 / kMergeWords) == 0) {
    p.part_ml[prow * 2 + 0] = (mmax == -INFINITY) ? -INFINITY : mmax * sl2;
    p.part_ml[prow * 2 + 1] = lt;
  }
}

}  // namespace

hipError_t launch_attention_q4_decode(const AttnParams& p, int dtype, hipStream_t stream) {
  const int passes = (p.rows + 15) / 16;
  const dim3 grid((unsigned)(p.B * p.Hkv * passes), (unsigned)p.nsplit, 1);
  if (dtype == 0) hipLaunchKernelGGL((attn_q4_decode_kernel<0>), grid, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((attn_q4_decode_kernel<1>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sdpa
